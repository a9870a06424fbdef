"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

Workload (one decode step per layer call): B=16 sequences, H_q=32 query heads
over H_kv=8 KV heads (GQA 4:1), head_dim 128, a 32K-token context per
sequence (the last 128 tokens in the FP16 window, the rest in 256-token
pages of 3-bit+QJL keys and 4-bit values, dense rotation), bf16 queries.
A step appends one new token to every sequence (tq_append_page: the token
leaving the window is encoded into its page) and runs tq_decode_attn over
the whole context.  The context is prefilled so that the last timed step
decodes at exactly T = 32768.  Inputs are seeded synthetic data with the
key recipe of tq_inputs (heavy-tailed channels, RoPE) drawn on the GPU.

Prints one JSON line: tokens/s (sum of context lengths attended per second),
the step time, the scan kernel's roofline (algorithmic bytes per launch /
its HIP-event time vs the 8 TB/s HBM peak, and vs the device's measured
streaming-read rate) and a CPU baseline (the float64 oracle on a bounded
sample of the same workload).  The scan's HIP events are recorded over a
second run of as many steps right after the timed ones: each event record
adds a few microseconds of queue time, which the timed steps do not carry.

Two more decode workloads are available with --workload (the default is
"batch", the workload above):
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-encode", action="store_true", help="skip the tq_encode leg")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="batch")
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


def cpu_baseline(T, W, P, G, Hkv, min_seconds, kbits=3, vbits=4, kmix=0, vmix=0, kn8=0, rotation="dense"):
    """The oracle's decode (dequantise + float64 softmax attention) on one
    sequence and one KV head (G query heads) at context T, repeated until
    min_seconds of CPU work; converted to sequence-tokens/s at H_kv heads."""
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
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": calls * T / Hkv / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} oracle decode call(s) of 1 sequence x 1 KV head ({G} query heads) at T={T}, "
                      f"{el:.1f} s; rate scaled to {Hkv} KV heads"}


SCAN_SOURCES = ["decode_mfma.hip", "decode_common.h", "device_common.h", "tq_internal.h"]


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


def encode_leg(tqa, tq_inputs, ctx, params, reps=10):
    """tq_encode of 4M fp16 vectors (4,096 sequences x 1,024 positions of the
    key recipe, and as many N(0,1) values) with the decode workload's formats:
    keys 3-bit + QJL, values 4-bit, dense rotation.  HIP-event time per call;
    MFMA work as executed (rotation in two fp16 passes, QJL projection in
    three) and as the two d x d products count it (4 d^2 flop per key)."""
    import torch
    n, d = 4096 * 1024, 128
    k, v = tq_inputs.torch_kv(5, 4096, 1, 1024, d, "cuda")
    k, v = k.view(n, d), v.view(n, d)
    codes = torch.empty((n, 64), dtype=torch.uint8, device="cuda")
    norms = torch.empty(n, dtype=torch.float32, device="cuda")
    signs = torch.empty((n, 16), dtype=torch.uint8, device="cuda")
    rnorms = torch.empty(n, dtype=torch.float32, device="cuda")
    out = {}
    for name, kind, x, qjl in (("keys_3bit_qjl", tqa.TQ_KIND_KEY, k, True), ("values_4bit", tqa.TQ_KIND_VALUE, v, False)):
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
        algo = (4 if qjl else 2) * d * d * n
        executed = (5 if qjl else 2) * 2 * d * d * n
        in_bytes = n * d * 2
        out_bytes = n * ((48 + 16 + 8) if qjl else (64 + 4))
        out[name] = {"ms": ms, "vectors_per_s": n / (ms / 1e3), "algorithmic_tflops": algo / (ms / 1e3) / 1e12,
                     "mfma_tflops_executed": executed / (ms / 1e3) / 1e12,
                     "hbm_gbps": (in_bytes + out_bytes) / (ms / 1e3) / 1e9}
    out["workload"] = "tq_encode of 4,194,304 fp16 vectors d=128 (4,096 x 1,024 positions), dense rotation"
    del k, v, codes, norms, signs, rnorms
    return out


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
        from kv_cache_vector_tq_amd import build
        build.build()
    dev = "cuda"
    wl = WORKLOADS[args.workload]
    default_run = args.workload == "batch"
    B = args.batch if args.batch is not None else wl["B"]
    Hq, Hkv, d, P, W = wl["Hq"], wl["Hkv"], 128, 256, 128
    G = Hq // Hkv
    R, L = wl["replicas"], wl["layers"]
    ncache = R * L
    kbits = args.key_bits if args.key_bits is not None else wl["kbits"]
    vbits = args.value_bits if args.value_bits is not None else wl["vbits"]
    kmix, vmix = int(args.key_mixed), int(args.value_mixed)
    kn8 = int(args.key_norm_u8)
    rotation = wl["rotation"]
    # target length of each sequence at the last step (a drawn length per
    # sequence for a range)
    if isinstance(wl["T"], tuple):
        Tf = tq_inputs.ragged_lengths(0, B, *wl["T"]).astype(np.int64)
    else:
        Tf = np.full(B, args.T if args.T is not None else wl["T"], dtype=np.int64)
    # warm-up steps, then the timed steps, then as many steps again with HIP
    # events around each scan launch (the roofline's kernel time; each event
    # record adds queue time, so they are not timed).  Step i appends one
    # token to, and decodes, every layer's cache, or replica i mod R.
    nsteps = args.warmup + 2 * args.steps
    ntimed = args.warmup + args.steps

    def appends(c, n):  # appends cache c receives in steps 0 .. n-1
        return len(range(c % R, n, R)) if R > 1 else n
    params = tqa.make_params(key_bits=kbits, key_qjl=1, value_bits=vbits,
                             rotation=tqa.TQ_ROT_DENSE if rotation == "dense" else tqa.TQ_ROT_HADAMARD,
                             num_q_heads=Hq, num_kv_heads=Hkv, page_tokens=P, window=W, seed=0,
                             flags=tqa.TQ_FLAG_VALU_SCAN if args.valu_scan else 0, key_mixed=kmix, value_mixed=vmix,
                             key_norm_u8=kn8)
    rdraws = tq_inputs.rotation_draws(0, d) if rotation == "dense" else tq_inputs.hadamard_draws(0, d)
    ctx = tqa.Context(params, rdraws, tq_inputs.qjl_draws(0, d))
    pb = tqa.tq_page_bytes(params)
    # lengths reach Tf at the last timed step; the evented steps go past it
    max_pages = -(-(int(Tf.max()) + max(appends(c, nsteps) - appends(c, ntimed) for c in range(ncache)) - W) // P)
    npages = B * max_pages
    caches = []
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
        tqa.tq_append_page(ctx, pool, cache["block_table"], cache["seq_lens"], k, v, cache["k_win"], cache["v_win"],
                           new_counts=counts, num_pages=npages)
        del k, v
        cache["lens"] = lens0.copy()
        caches.append(cache)
    # new tokens and queries of the steps (the same for every layer's cache)
    k_new, v_new = tq_inputs.torch_kv(0, B, Hkv, nsteps, d, dev, layer=L, start=int(Tf.max()))
    ksteps = [k_new[:, :, i:i + 1].contiguous() for i in range(nsteps)]
    vsteps = [v_new[:, :, i:i + 1].contiguous() for i in range(nsteps)]
    del k_new, v_new
    qsteps = [tq_inputs.torch_queries(0, (B, Hq, d), dev, torch.bfloat16, step=i) for i in range(nsteps)]
    pps = args.pages_per_split
    ws = torch.empty(tqa.tq_decode_workspace_bytes(ctx, B, max_pages, pps), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    sm = 1.0 / np.sqrt(d)
    torch.cuda.synchronize()
    assert tqa.tq_get_status(ctx) == 0

    def step_caches(i):
        return [caches[i % R]] if R > 1 else caches

    def step(i):
        for c in step_caches(i):
            tqa.tq_append_page(ctx, c["pool"], c["block_table"], c["seq_lens"], ksteps[i], vsteps[i], c["k_win"],
                               c["v_win"], num_pages=npages)
            tqa.tq_decode_attn(ctx, qsteps[i], c["pool"], c["block_table"], c["seq_lens"], c["k_win"], c["v_win"],
                               out, ws, sm, pages_per_split=pps, num_pages=npages)

    # context lengths each decode call attends (host bookkeeping of the appends)
    attended = []
    for i in range(nsteps):
        lens_i = []
        for c in step_caches(i):
            c["lens"] = c["lens"] + 1
            lens_i.append(c["lens"].copy())
        attended.append(lens_i)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: the steps as a caller runs them
    t0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        step(i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    # the scan kernel's time: HIP events recorded by the library on the launch
    # stream around each scan launch of the next steps
    nprof = sum(len(step_caches(i)) for i in range(args.warmup + args.steps, nsteps))
    tqa.tq_profile_begin(ctx, nprof)
    t1 = time.perf_counter()
    for i in range(args.warmup + args.steps, nsteps):
        step(i)
    torch.cuda.synchronize()
    el_prof = time.perf_counter() - t1
    scan_ms, ncalls = tqa.tq_profile_end(ctx)
    status = tqa.tq_get_status(ctx)
    if status != 0 or not torch.isfinite(out).all():
        raise SystemExit(f"bench: bad status {status} or non-finite output")
    for c in caches:
        assert np.array_equal(c["seq_lens"].cpu().numpy(), c["lens"]), "sequence lengths drifted from the bookkeeping"
    timed = range(args.warmup, args.warmup + args.steps)
    tokens = sum(int(x.sum()) for i in timed for x in attended[i])
    # key codes + signs + norm + rnorm, value codes + norm (a mixed rate adds d/16 code bytes)
    # (a u8 log-norm key norm takes 1 byte instead of 4)
    per_tok_head = (16 * kbits + 8 * kmix + 16 + 4 + (1 if kn8 else 4)) + (16 * vbits + 8 * vmix + 4)

    def comp_bytes(lens):  # compressed bytes one scan launch reads
        return Hkv * int(np.maximum(lens - W, 0).sum()) * per_tok_head

    prof_bytes = [comp_bytes(x) for i in range(args.warmup + args.steps, nsteps) for x in attended[i]]
    win_bytes = B * Hkv * W * d * 2 * 2
    scan_s = scan_ms / 1e3 / max(ncalls, 1)
    achieved = (sum(prof_bytes) / len(prof_bytes)) / scan_s / 1e9
    ms_step = el / args.steps * 1e3
    fmt = (f"keys {kbits + 0.5 * kmix:g}-bit+QJL{' with u8 log-norms' if kn8 else ''}, values "
           f"{vbits + 0.5 * vmix:g}-bit, {rotation} rotation, bf16 queries")
    if args.workload == "batch":
        desc = (f"decode step (append 1 token + decode attention), B={B}, Hq={Hq}, Hkv={Hkv}, d={d}, "
                f"T={int(Tf[0])} (last step), W={W} fp16 window, P={P}, {fmt}")
    elif args.workload == "long":
        desc = (f"long-context decode step (append 1 token + decode attention), B={B}, Hq={Hq}, Hkv={Hkv}, d={d}, "
                f"T={int(Tf[0])} (last step), W={W}, P={P}, {fmt}; {R} cache replicas take turns so that "
                f"each decode reads from HBM")
    else:
        desc = (f"{L}-layer decode step (per layer: append 1 token + decode attention), B={B} sequences, "
                f"lengths U{{{wl['T'][0]}..{wl['T'][1]}}} (mean {Tf.mean():.0f} at the last step), Hq={Hq}, "
                f"Hkv={Hkv}, d={d}, W={W}, P={P}, {fmt}")
    res = {
        "metric": METRIC, "value": tokens / el, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": desc, "batch": B, "seq_len": int(Tf.max()), "parallelism": "none (1 GPU)"},
        "hbm_gbps_step": (sum(comp_bytes(x) for i in timed for x in attended[i]) / args.steps
                          + len(step_caches(0)) * win_bytes) / (ms_step / 1e3) / 1e9,
        "scan_us": scan_s * 1e6,
        "ms_per_step_with_scan_events": el_prof / args.steps * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     # the committed counter record covers the default workload and formats only
                     "traffic": scan_traffic() if default_run and (kbits, vbits, kmix, vmix, kn8) == (3, 4, 0, 0, 0)
                     else None,
                     "kernel": "scan_kernel (VALU)" if args.valu_scan else "scan_mfma_kernel",
                     "algorithmic_bytes_per_launch": sum(prof_bytes) / len(prof_bytes)},
    }
    if L > 1:
        res["layer_calls_per_s"] = L * args.steps / el
    del caches, ksteps, vsteps, ws
    # measured ceiling: a plain coalesced streaming read of 1 GiB (beyond the
    # 256 MB last-level cache), fastest of 5 launches
    rbuf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    rbuf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    read_gbps = rbuf.numel() / (tqa.tq_read_probe(rbuf, sink, reps=5) / 1e3) / 1e9
    del rbuf
    res["read_ceiling"] = {"GBps": read_gbps, "bytes": 1 << 30, "kernel": "tq_read_probe (coalesced 16-byte loads)",
                           "frac_of_peak": read_gbps / HBM_PEAK_GBPS}
    res["roofline"]["frac_of_read_ceiling"] = achieved / read_gbps
    # the encode leg measures the default formats (3-bit+QJL keys, 4-bit values)
    if default_run and not args.no_encode and (kbits, vbits, kmix, vmix, kn8) == (3, 4, 0, 0, 0):
        res["encode"] = encode_leg(tqa, tq_inputs, ctx, params)
    if not args.no_cpu_baseline:
        # one sequence at the workload's longest context
        res["cpu_baseline"] = cpu_baseline(int(Tf.max()), W, P, G, Hkv, args.cpu_seconds, kbits, vbits, kmix, vmix,
                                           kn8, rotation)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
