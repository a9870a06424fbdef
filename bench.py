"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

Headline workload (one decode step per layer call): B=16 sequences, H_q=32
query heads over H_kv=8 KV heads (GQA 4:1), head_dim 128, a 32K-token context
per sequence (the last 128 tokens in the FP16 window, the rest in 256-token
pages of 3-bit+QJL keys and 4-bit values, dense rotation), bf16 queries.  A
step appends one new token to every sequence (tq_append_page: the token
leaving the window is encoded into its page) and runs tq_decode_attn over
the whole context.  The context is prefilled so that the last timed step
decodes at exactly T = 32768.  Inputs are seeded synthetic data with the key
recipe of tq_inputs (heavy-tailed channels, RoPE) drawn on the GPU.

The JSON line carries, besides the step rate:
  roofline      the scan kernel (the one that streams the packed cache; with
                at most 4 query heads per KV head its last work-group of a
                head also combines the splits, so the tail is included):
                algorithmic bytes per launch / its duration.  The duration
                comes from HIP events the library records on the launch
                stream around each scan launch, over a replay of the timed
                steps (lengths and rings restored to where the timed region
                started, so the same tokens at the same context lengths);
                each event adds its own latency, so this fraction is a
                conservative one;
  decode_call   back-to-back tq_decode_attn calls at the final length
                between HIP events: prep + scan + finalize per call, against the
                bytes one call must read (pages and FP16 window);
  prefill       the first cache's bulk tq_append_page (HIP events);
  read_ceiling  the device's streaming-read rate (tq_read_probe, 1 GiB);
  workloads     the two other decode workloads (below), same fields;
  encode        tq_encode of 4M fp16 vectors at 2, 3 and 4 bits, dense and
                randomized-Hadamard rotations, keys with QJL and values;
  cpu_baseline  the float64 oracle on a bounded slice of the headline
                workload, on the host cores.

Other decode workloads (--workload selects one of them alone):
  long    B=1, H_q=64, H_kv=8, T=131,072, keys 2-bit+QJL, values 2-bit,
          Hadamard rotation.  One layer's cache is 97 MB, less than the
          256 MB last-level cache, so three replicas of it take turns (step i
          appends to and decodes replica i mod 3) and every decode reads its
          pages from HBM.
  layers  36 layers, each its own cache: B=64 sequences with lengths drawn
          uniformly from 1,024..16,384 tokens, H_q=16, H_kv=2, keys
          3-bit+QJL, values 4-bit, dense rotation.  A step appends one token
          and decodes, layer after layer.
"""

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# decode workloads: sequences, heads, context (a range: lengths drawn per
# sequence), formats, cache replicas taking turns, layers
WORKLOADS = {
    "batch": dict(B=16, Hq=32, Hkv=8, T=32768, kbits=3, vbits=4, rotation="dense", replicas=1, layers=1),
    "long": dict(B=1, Hq=64, Hkv=8, T=131072, kbits=2, vbits=2, rotation="hadamard", replicas=3, layers=1),
    "layers": dict(B=64, Hq=16, Hkv=2, T=(1024, 16384), kbits=3, vbits=4, rotation="dense", replicas=1, layers=36),
}
METRIC = "decode-attn compressed-KV tokens/s & HBM GB/s vs peak; encode vectors/s"
DTYPE = "fp32 accumulate; fp16 MFMA operands (query side split hi+lo, ~22 bits)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-encode", action="store_true", help="skip the tq_encode legs")
    ap.add_argument("--no-extra", action="store_true", help="skip the other decode workloads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=None,
                    help="time this decode workload alone (default: the headline line with all legs)")
    ap.add_argument("--T", type=int, default=None, help="context length (batch and long workloads)")
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--valu-scan", action="store_true", help="time the vector-ALU scan kernel instead")
    ap.add_argument("--pages-per-split", type=int, default=0, help="decode split size (0: the library's choice)")
    ap.add_argument("--key-bits", type=int, default=None)
    ap.add_argument("--value-bits", type=int, default=None)
    ap.add_argument("--key-mixed", action="store_true", help="keys at key_bits + 1/2 (mixed-channel rate)")
    ap.add_argument("--value-mixed", action="store_true", help="values at value_bits + 1/2")
    ap.add_argument("--key-norm-u8", action="store_true", help="key norms as u8 log-norm codes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    return ap.parse_args()


def host_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_baseline(T, W, P, G, Hkv, B, min_seconds, kbits=3, vbits=4, kmix=0, vmix=0, kn8=0, rotation="dense"):
    """The oracle's decode (dequantise + float64 softmax attention) on one
    (sequence, KV head) slice of a layer call: G query heads over a T-token
    context.  Repeated until min_seconds of CPU work.  A layer call is B x Hkv
    such slices, so the rate in the workload's unit (sequence tokens attended
    per second) is calls * T / (time * Hkv)."""
    from threadpoolctl import threadpool_info
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import attention as att
    from oracle_cache import Setup, fill
    import tq_inputs
    s = Setup(Hq=G, Hkv=1, key_bits=kbits, key_qjl=1, value_bits=vbits, P=P, W=W, key_mixed=bool(kmix),
              value_mixed=bool(vmix), key_norm_u8=bool(kn8), rotation=rotation)
    cache = s.cache(1, T)
    fill(s, cache, [T])
    q = tq_inputs.queries(3, (1, G, 128))
    calls, t0 = 0, time.perf_counter()
    while True:
        att.attention_plain(cache, q, 1 / np.sqrt(128))
        calls += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    model, cores = host_info()
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": calls * T / Hkv / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "blas_threads": blas,
            "sample": f"{calls} oracle decode call(s) of one (sequence, KV head) slice ({G} query heads, "
                      f"T={T}) of the {B} x {Hkv}-slice layer call, {el:.1f} s; tokens/s = calls x T / "
                      f"(seconds x {Hkv} KV heads)"}


SCAN_SOURCES = ["decode_mfma.hip", "decode_finalize.h", "decode_common.h", "device_common.h", "tq_internal.h",
                "decode.hip"]


def scan_traffic():
    """HBM bytes per scan launch from the committed rocprofv3 counter summary
    (profiles/decode_scan_traffic.json), when it was taken on the current
    kernel source; None otherwise."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode_scan_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in SCAN_SOURCES:
        h.update(open(os.path.join(ROOT, "kv_cache_vector_tq_amd", "csrc", f), "rb").read())
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return rec.get("hbm_bytes_per_launch")


def encode_legs(tqa, tq_inputs, reps=10):
    """tq_encode of 4M fp16 vectors (4,096 sequences x 1,024 positions of the
    key recipe, and as many N(0,1) values) at 2, 3 and 4 bits, dense and
    Hadamard rotations; keys with the QJL sketch.  HIP-event time per call.
    Dense rotation: algorithmic flops 4 d^2 per key, 2 d^2 per value; MFMA
    flops as executed (fp16 passes: rotation 2, QJL projection 3)."""
    import torch
    n, d = 4096 * 1024, 128
    k, v = tq_inputs.torch_kv(5, 4096, 1, 1024, d, "cuda")
    k, v = k.view(n, d), v.view(n, d)
    codes = torch.empty((n, 64), dtype=torch.uint8, device="cuda")
    norms = torch.empty(n, dtype=torch.float32, device="cuda")
    signs = torch.empty((n, 16), dtype=torch.uint8, device="cuda")
    rnorms = torch.empty(n, dtype=torch.float32, device="cuda")
    out = {"workload": "tq_encode of 4,194,304 fp16 vectors d=128 (4,096 x 1,024 positions) into flat records"}
    for rotation in ("dense", "hadamard"):
        for bits in (2, 3, 4):
            params = tqa.make_params(key_bits=bits, key_qjl=1, value_bits=bits,
                                     rotation=tqa.TQ_ROT_DENSE if rotation == "dense" else tqa.TQ_ROT_HADAMARD)
            rd = tq_inputs.rotation_draws(0, d) if rotation == "dense" else tq_inputs.hadamard_draws(0, d)
            ctx = tqa.Context(params, rd, tq_inputs.qjl_draws(0, d))
            for name, kind, x, qjl in ((f"{rotation}_keys_{bits}bit_qjl", tqa.TQ_KIND_KEY, k, True),
                                       (f"{rotation}_values_{bits}bit", tqa.TQ_KIND_VALUE, v, False)):
                def call():
                    tqa.tq_encode(ctx, kind, x, codes, norms, signs if qjl else None, rnorms if qjl else None)
                call()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    call()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                rec_bytes = 16 * bits + 4 + (16 + 4 if qjl else 0)
                hbm = (n * d * 2 + n * rec_bytes) / (ms / 1e3) / 1e9
                r = {"ms": ms, "vectors_per_s": n / (ms / 1e3), "hbm_gbps": hbm, "hbm_frac": hbm / HBM_PEAK_GBPS}
                if rotation == "dense":
                    r["algorithmic_tflops"] = (4 if qjl else 2) * d * d * n / (ms / 1e3) / 1e12
                    r["mfma_tflops_executed"] = (5 if qjl else 2) * 2 * d * d * n / (ms / 1e3) / 1e12
                out[name] = r
            ctx.close()
    del codes, norms, signs, rnorms
    # the same vectors written into 256-token pages by one bulk tq_append_page
    # (4,096 sequences x 1,024 tokens, no FP16 window): keys 3-bit + QJL and
    # values 4-bit, dense rotation
    params = tqa.make_params(key_bits=3, key_qjl=1, value_bits=4, page_tokens=256, window=0)
    ctx = tqa.Context(params, tq_inputs.rotation_draws(0, d), tq_inputs.qjl_draws(0, d))
    pb = tqa.tq_page_bytes(params)
    npg = 4096 * 4
    pool = torch.zeros(npg * pb, dtype=torch.uint8, device="cuda")
    bt = torch.arange(npg, dtype=torch.int32, device="cuda").view(4096, 4)
    sl = torch.zeros(4096, dtype=torch.int32, device="cuda")
    kp, vp = k.view(4096, 1, 1024, d), v.view(4096, 1, 1024, d)
    times = []
    for _ in range(3):
        sl.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        tqa.tq_append_page(ctx, pool, bt, sl, kp, vp, None, None, num_pages=npg)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = min(times)
    out["pages_dense_k3qjl_v4"] = {"ms": ms, "vectors_per_s": 2 * n / (ms / 1e3),
                                   "hbm_gbps": (2 * n * d * 2 + n * (72 + 68)) / (ms / 1e3) / 1e9,
                                   "what": "tq_append_page of 4,096 sequences x 1,024 tokens (keys and values, "
                                           "8,388,608 vectors) into 256-token pages, W=0; fastest of 3"}
    ctx.close()
    del k, v, kp, vp, pool
    return out


def decode_workload(tqa, tq_inputs, wname, args, fmt_over=None):
    """Prefill, warm up, time args.steps decode steps of one workload; then
    replay the timed steps with scan events; then time back-to-back decode
    calls at the final lengths.  Returns the JSON fields of the workload."""
    import torch
    dev = "cuda"
    wl = WORKLOADS[wname]
    fo = fmt_over or {}
    B = fo.get("B", wl["B"])
    Hq, Hkv, d, P, W = wl["Hq"], wl["Hkv"], 128, 256, 128
    G = Hq // Hkv
    R, L = wl["replicas"], wl["layers"]
    ncache = R * L
    kbits, vbits = fo.get("kbits", wl["kbits"]), fo.get("vbits", wl["vbits"])
    kmix, vmix, kn8 = fo.get("kmix", 0), fo.get("vmix", 0), fo.get("kn8", 0)
    rotation = wl["rotation"]
    if isinstance(wl["T"], tuple):
        Tf = tq_inputs.ragged_lengths(0, B, *wl["T"]).astype(np.int64)
    else:
        Tf = np.full(B, fo.get("T", wl["T"]), dtype=np.int64)
    ntimed = args.warmup + args.steps

    def appends(c, n):  # appends cache c receives in steps 0 .. n-1
        return len(range(c % R, n, R)) if R > 1 else n
    params = tqa.make_params(key_bits=kbits, key_qjl=1, value_bits=vbits,
                             rotation=tqa.TQ_ROT_DENSE if rotation == "dense" else tqa.TQ_ROT_HADAMARD,
                             num_q_heads=Hq, num_kv_heads=Hkv, page_tokens=P, window=W, seed=0,
                             flags=tqa.TQ_FLAG_VALU_SCAN if fo.get("valu") else 0, key_mixed=kmix, value_mixed=vmix,
                             key_norm_u8=kn8)
    rdraws = tq_inputs.rotation_draws(0, d) if rotation == "dense" else tq_inputs.hadamard_draws(0, d)
    ctx = tqa.Context(params, rdraws, tq_inputs.qjl_draws(0, d))
    pb = tqa.tq_page_bytes(params)
    max_pages = -(-(int(Tf.max()) - W) // P)
    npages = B * max_pages
    caches = []
    prefill = None
    for c in range(ncache):
        pool = torch.zeros(npages * pb, dtype=torch.uint8, device=dev)
        # pages of a sequence are scattered over the pool
        perm = torch.from_numpy(np.random.default_rng(1 + c).permutation(npages).astype(np.int32))
        cache = dict(pool=pool, block_table=perm.reshape(B, max_pages).to(dev),
                     seq_lens=torch.zeros(B, dtype=torch.int32, device=dev),
                     k_win=torch.zeros((B, Hkv, W, d), dtype=torch.float16, device=dev))
        cache["v_win"] = torch.zeros_like(cache["k_win"])
        # prefill so that the cache's last timed append ends at the target lengths
        lens0 = Tf - appends(c, ntimed)
        T0 = int(lens0.max())
        k, v = tq_inputs.torch_kv(0, B, Hkv, T0, d, dev, layer=c % L)
        counts = None if np.all(lens0 == T0) else torch.from_numpy(lens0.astype(np.int32)).to(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        tqa.tq_append_page(ctx, pool, cache["block_table"], cache["seq_lens"], k, v, cache["k_win"], cache["v_win"],
                           new_counts=counts, num_pages=npages)
        e1.record()
        if c == 0:  # the bulk prefill of the first cache: every token leaving the window is encoded
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            nvec = 2 * Hkv * int(np.maximum(lens0 - W, 0).sum())
            prefill = {"ms": ms, "vectors": nvec, "vectors_per_s": nvec / (ms / 1e3),
                       "what": "one tq_append_page of the whole prompt (keys and values of every KV head; "
                               "HIP events), the cache's first prefill"}
        del k, v
        cache["lens"] = lens0.copy()
        caches.append(cache)
    k_new, v_new = tq_inputs.torch_kv(0, B, Hkv, ntimed, d, dev, layer=L, start=int(Tf.max()))
    ksteps = [k_new[:, :, i:i + 1].contiguous() for i in range(ntimed)]
    vsteps = [v_new[:, :, i:i + 1].contiguous() for i in range(ntimed)]
    del k_new, v_new
    qsteps = [tq_inputs.torch_queries(0, (B, Hq, d), dev, torch.bfloat16, step=i) for i in range(ntimed)]
    pps = fo.get("pps", 0)
    ws = torch.empty(tqa.tq_decode_workspace_bytes(ctx, B, max_pages, pps), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    sm = 1.0 / np.sqrt(d)
    torch.cuda.synchronize()
    assert tqa.tq_get_status(ctx) == 0

    def step_caches(i):
        return [caches[i % R]] if R > 1 else caches

    def decode(c, i):
        tqa.tq_decode_attn(ctx, qsteps[i], c["pool"], c["block_table"], c["seq_lens"], c["k_win"], c["v_win"],
                           out, ws, sm, pages_per_split=pps, num_pages=npages)

    def step(i):
        for c in step_caches(i):
            tqa.tq_append_page(ctx, c["pool"], c["block_table"], c["seq_lens"], ksteps[i], vsteps[i], c["k_win"],
                               c["v_win"], num_pages=npages)
            decode(c, i)

    # context lengths each decode call attends (host bookkeeping of the appends)
    attended = []
    for i in range(ntimed):
        lens_i = []
        for c in step_caches(i):
            c["lens"] = c["lens"] + 1
            lens_i.append(c["lens"].copy())
        attended.append(lens_i)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # where the timed region starts: lengths and rings, restored for the replay
    snap = [(c["seq_lens"].clone(), c["k_win"].clone(), c["v_win"].clone()) for c in caches]
    # timed region: the steps as a caller runs them
    t0 = time.perf_counter()
    for i in range(args.warmup, ntimed):
        step(i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    final = [c["seq_lens"].clone() for c in caches]
    # replay of the timed steps with HIP events around each scan launch
    for c, (sl, kw, vw) in zip(caches, snap):
        c["seq_lens"].copy_(sl)
        c["k_win"].copy_(kw)
        c["v_win"].copy_(vw)
    torch.cuda.synchronize()
    nprof = sum(len(step_caches(i)) for i in range(args.warmup, ntimed))
    tqa.tq_profile_begin(ctx, nprof)
    for i in range(args.warmup, ntimed):
        step(i)
    torch.cuda.synchronize()
    scan_ms, ncalls = tqa.tq_profile_end(ctx)
    for c, f in zip(caches, final):
        assert torch.equal(c["seq_lens"], f), "the replay did not end at the timed region's lengths"
    # back-to-back decode calls at the final lengths (no appends): prep + scan
    # (+ finalize), between two events on the stream the calls are launched on
    ncall = max(args.steps, 10)
    torch.cuda.synchronize()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record()
    for j in range(ncall):
        for c in step_caches(ntimed - 1 - (j % R)):
            decode(c, ntimed - 1)
    e3.record()
    torch.cuda.synchronize()
    el_call = e2.elapsed_time(e3) / 1e3 / (ncall * (L if R == 1 else 1))
    status = tqa.tq_get_status(ctx)
    if status != 0 or not torch.isfinite(out).all():
        raise SystemExit(f"bench: bad status {status} or non-finite output")
    for c in caches:
        assert np.array_equal(c["seq_lens"].cpu().numpy(), c["lens"]), "sequence lengths drifted from the bookkeeping"
    timed = range(args.warmup, ntimed)
    tokens = sum(int(x.sum()) for i in timed for x in attended[i])
    # key codes + signs + norm + rnorm, value codes + norm (a mixed rate adds d/16 code bytes)
    # (a u8 log-norm key norm takes 1 byte instead of 4)
    per_tok_head = (16 * kbits + 8 * kmix + 16 + 4 + (1 if kn8 else 4)) + (16 * vbits + 8 * vmix + 4)

    def comp_bytes(lens):  # compressed bytes one scan launch reads
        return Hkv * int(np.maximum(lens - W, 0).sum()) * per_tok_head
    win_bytes = B * Hkv * W * d * 2 * 2
    prof_bytes = [comp_bytes(x) for i in timed for x in attended[i]]
    scan_s = scan_ms / 1e3 / max(ncalls, 1)
    achieved = (sum(prof_bytes) / len(prof_bytes)) / scan_s / 1e9
    ms_step = el / args.steps * 1e3
    call_bytes = comp_bytes(attended[ntimed - 1][-1]) + win_bytes
    lo_T, hi_T = int(min(x.max() for i in timed for x in attended[i])), int(Tf.max())
    fmt = (f"keys {kbits + 0.5 * kmix:g}-bit+QJL{' with u8 log-norms' if kn8 else ''}, values "
           f"{vbits + 0.5 * vmix:g}-bit, {rotation} rotation, bf16 queries")
    if wname == "batch":
        desc = (f"decode step (append 1 token + decode attention), B={B}, Hq={Hq}, Hkv={Hkv}, d={d}, "
                f"T={int(Tf[0])} (last step), W={W} fp16 window, P={P}, {fmt}")
    elif wname == "long":
        desc = (f"long-context decode step (append 1 token + decode attention), B={B}, Hq={Hq}, Hkv={Hkv}, d={d}, "
                f"T={int(Tf[0])} (last step), W={W}, P={P}, {fmt}; {R} cache replicas take turns so that "
                f"each decode reads from HBM")
    else:
        desc = (f"{L}-layer decode step (per layer: append 1 token + decode attention), B={B} sequences, "
                f"lengths U{{{wl['T'][0]}..{wl['T'][1]}}} (mean {Tf.mean():.0f} at the last step), Hq={Hq}, "
                f"Hkv={Hkv}, d={d}, W={W}, P={P}, {fmt}")
    res = {
        "value": tokens / el, "unit": "tokens/s", "ms_per_step": ms_step,
        "config": {"workload": desc, "batch": B, "seq_len": int(Tf.max()), "parallelism": "none (1 GPU)"},
        "hbm_gbps_step": (sum(comp_bytes(x) for i in timed for x in attended[i]) / args.steps
                          + len(step_caches(0)) * win_bytes) / (ms_step / 1e3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "scan_kernel (VALU)" if fo.get("valu") else (
                         "scan_mfma_kernel (with at most 4 query heads per KV head its last work-group per "
                         "KV head also combines the splits and the window)"),
                     "algorithmic_bytes_per_launch": sum(prof_bytes) / len(prof_bytes),
                     "launch_us": scan_s * 1e6,
                     "launches": f"{ncalls} scan launches by HIP events, a replay of the timed steps "
                                 f"(longest context {lo_T}..{hi_T})"},
        "decode_call": {"us": el_call * 1e6, "bytes": call_bytes,
                        "gbps": call_bytes / el_call / 1e9, "frac": call_bytes / el_call / 1e9 / HBM_PEAK_GBPS,
                        "what": f"tq_decode_attn (prep + scan + finalize) at longest context {hi_T}, mean of "
                                f"{ncall} back-to-back calls between HIP events; bytes = packed pages + FP16 window"},
    }
    res["prefill"] = prefill
    if L > 1:
        res["layer_calls_per_s"] = L * args.steps / el
    del caches, ksteps, vsteps, ws, out
    ctx.close()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus above 1 is not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "launches": 3}))
        return
    import kv_cache_vector_tq_amd as tqa
    import tq_inputs
    if not os.path.exists(tqa.LIB_PATH):
        raise SystemExit(f"{tqa.LIB_PATH} is missing: build the library first (python -m kv_cache_vector_tq_amd.build)")
    wname = args.workload or "batch"
    headline = args.workload is None
    fo = {}
    for key, val in (("kbits", args.key_bits), ("vbits", args.value_bits), ("B", args.batch), ("T", args.T)):
        if val is not None:
            fo[key] = val
    fo.update(kmix=int(args.key_mixed), vmix=int(args.value_mixed), kn8=int(args.key_norm_u8),
              valu=bool(args.valu_scan), pps=args.pages_per_split)
    default_fmt = not any(k in fo for k in ("kbits", "vbits", "B", "T")) and not (
        args.key_mixed or args.value_mixed or args.key_norm_u8 or args.valu_scan or args.pages_per_split)
    w = decode_workload(tqa, tq_inputs, wname, args, fo)
    res = {"metric": METRIC, "value": w.pop("value"), "unit": w.pop("unit"), "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": w.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE,
           "data": "synthetic"}
    res.update(w)
    if wname == "batch" and default_fmt:
        # the committed counter record covers the headline workload and formats only
        res["roofline"]["traffic"] = scan_traffic()
    # measured ceiling: a plain coalesced streaming read of 1 GiB (beyond the
    # 256 MB last-level cache), fastest of 5 launches
    rbuf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    rbuf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    read_gbps = rbuf.numel() / (tqa.tq_read_probe(rbuf, sink, reps=5) / 1e3) / 1e9
    del rbuf
    res["read_ceiling"] = {"GBps": read_gbps, "bytes": 1 << 30, "kernel": "tq_read_probe (coalesced 16-byte loads)",
                           "frac_of_peak": read_gbps / HBM_PEAK_GBPS}
    res["roofline"]["frac_of_read_ceiling"] = res["roofline"]["achieved"] / read_gbps
    if headline and default_fmt and not args.no_extra:
        extra = {}
        for other in ("long", "layers"):
            ow = decode_workload(tqa, tq_inputs, other, args)
            extra[other] = ow
        res["workloads"] = extra
    if headline and default_fmt and not args.no_encode:
        res["encode"] = encode_legs(tqa, tq_inputs)
    if not args.no_cpu_baseline:
        wl = WORKLOADS[wname]
        res["cpu_baseline"] = cpu_baseline(int(res["config"]["seq_len"]), 128, 256, wl["Hq"] // wl["Hkv"], wl["Hkv"],
                                           res["config"]["batch"], args.cpu_seconds,
                                           fo.get("kbits", wl["kbits"]), fo.get("vbits", wl["vbits"]),
                                           fo["kmix"], fo["vmix"], fo["kn8"], wl["rotation"])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
