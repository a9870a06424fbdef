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
METRIC = "decode-attn compressed-KV tokens/s & HBM GB/s vs peak; encode vectors/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-encode", action="store_true", help="skip the tq_encode leg")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--T", type=int, default=32768)
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--valu-scan", action="store_true", help="time the vector-ALU scan kernel instead")
    ap.add_argument("--key-bits", type=int, default=3)
    ap.add_argument("--value-bits", type=int, default=4)
    ap.add_argument("--key-mixed", action="store_true", help="keys at key_bits + 1/2 (mixed-channel rate)")
    ap.add_argument("--value-mixed", action="store_true", help="values at value_bits + 1/2")
    ap.add_argument("--key-norm-u8", action="store_true", help="key norms as u8 log-norm codes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    return ap.parse_args()


def cpu_baseline(T, W, P, G, Hkv, min_seconds, kbits=3, vbits=4, kmix=0, vmix=0, kn8=0):
    """The oracle's decode (dequantise + float64 softmax attention) on one
    sequence and one KV head (G query heads) at context T, repeated until
    min_seconds of CPU work; converted to sequence-tokens/s at H_kv heads."""
    from threadpoolctl import threadpool_info
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import attention as att
    from oracle_cache import Setup, fill
    import tq_inputs
    s = Setup(Hq=G, Hkv=1, key_bits=kbits, key_qjl=1, value_bits=vbits, P=P, W=W, key_mixed=bool(kmix),
              value_mixed=bool(vmix), key_norm_u8=bool(kn8))
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
    B, Hq, Hkv, d, P, W = args.batch, 32, 8, 128, 256, 128
    G = Hq // Hkv
    Tf = args.T
    # warm-up steps, then the timed steps (the last at T = Tf), then as many
    # steps again with HIP events around each scan launch (the roofline's
    # kernel time; each event record adds queue time, so they are not timed)
    nsteps = args.warmup + 2 * args.steps
    T0 = Tf - args.warmup - args.steps
    Tend = T0 + nsteps
    kbits, vbits, kmix, vmix = args.key_bits, args.value_bits, int(args.key_mixed), int(args.value_mixed)
    kn8 = int(args.key_norm_u8)
    params = tqa.make_params(key_bits=kbits, key_qjl=1, value_bits=vbits, rotation=tqa.TQ_ROT_DENSE, num_q_heads=Hq,
                             num_kv_heads=Hkv, page_tokens=P, window=W, seed=0,
                             flags=tqa.TQ_FLAG_VALU_SCAN if args.valu_scan else 0, key_mixed=kmix, value_mixed=vmix,
                             key_norm_u8=kn8)
    ctx = tqa.Context(params, tq_inputs.rotation_draws(0, d), tq_inputs.qjl_draws(0, d))
    pb = tqa.tq_page_bytes(params)
    max_pages = -(-(Tend - W) // P)
    npages = B * max_pages
    pool = torch.zeros(npages * pb, dtype=torch.uint8, device=dev)
    # pages of a sequence are scattered over the pool
    perm = torch.from_numpy(np.random.default_rng(1).permutation(npages).astype(np.int32))
    block_table = perm.reshape(B, max_pages).to(dev)
    seq_lens = torch.zeros(B, dtype=torch.int32, device=dev)
    k_win = torch.zeros((B, Hkv, W, d), dtype=torch.float16, device=dev)
    v_win = torch.zeros_like(k_win)
    k_all, v_all = tq_inputs.torch_kv(0, B, Hkv, Tend, d, dev)
    kpre = k_all[:, :, :T0].contiguous()
    vpre = v_all[:, :, :T0].contiguous()
    tqa.tq_append_page(ctx, pool, block_table, seq_lens, kpre, vpre, k_win, v_win, num_pages=npages)
    del kpre, vpre
    ksteps = [k_all[:, :, T0 + i:T0 + i + 1].contiguous() for i in range(nsteps)]
    vsteps = [v_all[:, :, T0 + i:T0 + i + 1].contiguous() for i in range(nsteps)]
    del k_all, v_all
    qsteps = [tq_inputs.torch_queries(0, (B, Hq, d), dev, torch.bfloat16, step=i) for i in range(nsteps)]
    ws = torch.empty(tqa.tq_decode_workspace_bytes(ctx, B, max_pages), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    sm = 1.0 / np.sqrt(d)
    torch.cuda.synchronize()
    assert tqa.tq_get_status(ctx) == 0

    def step(i):
        tqa.tq_append_page(ctx, pool, block_table, seq_lens, ksteps[i], vsteps[i], k_win, v_win, num_pages=npages)
        tqa.tq_decode_attn(ctx, qsteps[i], pool, block_table, seq_lens, k_win, v_win, out, ws, sm, num_pages=npages)

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
    tqa.tq_profile_begin(ctx, args.steps)
    t1 = time.perf_counter()
    for i in range(args.warmup + args.steps, nsteps):
        step(i)
    torch.cuda.synchronize()
    el_prof = time.perf_counter() - t1
    scan_ms, ncalls = tqa.tq_profile_end(ctx)
    status = tqa.tq_get_status(ctx)
    if status != 0 or not torch.isfinite(out).all():
        raise SystemExit(f"bench: bad status {status} or non-finite output")
    # tokens attended in the timed steps: after step i the length is T0 + i + 1
    lens = [T0 + i + 1 for i in range(args.warmup, args.warmup + args.steps)]
    lens_prof = [T0 + i + 1 for i in range(args.warmup + args.steps, nsteps)]
    tokens = B * sum(lens)
    # key codes + signs + norm + rnorm, value codes + norm (a mixed rate adds d/16 code bytes)
    # (a u8 log-norm key norm takes 1 byte instead of 4)
    per_tok_head = (16 * kbits + 8 * kmix + 16 + 4 + (1 if kn8 else 4)) + (16 * vbits + 8 * vmix + 4)
    comp_bytes = [B * Hkv * (T - W) * per_tok_head for T in lens_prof]
    win_bytes = B * Hkv * W * d * 2 * 2
    scan_s = scan_ms / 1e3 / max(ncalls, 1)
    achieved = (sum(comp_bytes) / len(comp_bytes)) / scan_s / 1e9
    ms_step = el / args.steps * 1e3
    res = {
        "metric": METRIC, "value": tokens / el, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"decode step (append 1 token + decode attention), B={B}, Hq={Hq}, Hkv={Hkv}, "
                               f"d={d}, T={Tf} (last step), W={W} fp16 window, P={P}, keys "
                               f"{kbits + 0.5 * kmix:g}-bit+QJL{' with u8 log-norms' if kn8 else ''}, values "
                               f"{vbits + 0.5 * vmix:g}-bit, dense rotation, bf16 queries",
                   "batch": B, "seq_len": Tf, "parallelism": "none (1 GPU)"},
        "hbm_gbps_step": (sum(B * Hkv * (T - W) * per_tok_head for T in lens) / len(lens) + win_bytes)
                         / (ms_step / 1e3) / 1e9,
        "scan_us": scan_s * 1e6,
        "ms_per_step_with_scan_events": el_prof / args.steps * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     # the committed counter record covers the default formats only
                     "traffic": scan_traffic() if (kbits, vbits, kmix, vmix, kn8) == (3, 4, 0, 0, 0) else None,
                     "kernel": "scan_kernel (VALU)" if args.valu_scan else "scan_mfma_kernel",
                     "algorithmic_bytes_per_launch": sum(comp_bytes) / len(comp_bytes)},
    }
    del pool, k_win, v_win, ksteps, vsteps, ws
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
    if not args.no_encode and (kbits, vbits, kmix, vmix, kn8) == (3, 4, 0, 0, 0):
        res["encode"] = encode_leg(tqa, tq_inputs, ctx, params)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(Tf, W, P, G, Hkv, args.cpu_seconds, kbits, vbits, kmix, vmix, kn8)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
