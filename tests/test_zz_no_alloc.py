"""tq_decode_attn_noalloc (the allocation-free decode: the workspace lives
in the library's static device scratch) against tq_decode_attn with a
caller workspace: bit-identical outputs on two calls in a row, the second
with a smaller batch and shorter contexts (under the deterministic schedule;
the default one, whose sums group differently from call to call, within
1e-5 of max|o|), and the size limit reported as TQ_ERR_WORKSPACE."""

import numpy as np
import pytest
import torch

import kv_cache_vector_tq_amd as tqa
import tq_inputs
from gpu_helpers import assert_out_close, context_for, run_decode, upload_cache
from oracle import attention as att
from oracle_cache import Setup, fill

pytestmark = pytest.mark.gpu


def _noalloc(ctx, q, dev, pps=0):
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    tqa.tq_decode_attn_noalloc(ctx, q, dev["pool"], dev["block_table"], dev["seq_lens"], dev["k_win"], dev["v_win"],
                               out, 1 / np.sqrt(128), pages_per_split=pps, num_pages=dev["num_pages"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_matches_workspace_decode():
    print("case noalloc two calls", flush=True)
    s = Setup(Hq=8, Hkv=2, W=32, P=64)
    # first call: 6 sequences up to 3000 tokens; second: 2 sequences up to 700
    for lens, seed in (([3000, 1200, 64, 33, 0, 2500], 21), ([700, 90], 22)):
        cache = s.cache(len(lens), max(lens))
        fill(s, cache, lens)
        ctx = context_for(s, tqa.TQ_FLAG_DETERMINISTIC)
        dev = upload_cache(cache)
        q = tq_inputs.queries(seed, (len(lens), s.Hq, 128))
        qt = torch.from_numpy(q.astype(np.float32)).cuda()
        want, _ = run_decode(ctx, qt, dev, 1 / np.sqrt(128))
        got = _noalloc(ctx, qt, dev)
        assert np.array_equal(got, want), lens
        ctx_b = context_for(s)
        got_b = _noalloc(ctx_b, qt, dev)
        assert np.max(np.abs(got_b - want)) <= 1e-5 * np.max(np.abs(want)), lens
        ref, _ = att.attention_plain(cache, q.astype(np.float32).astype(np.float64), 1 / np.sqrt(128))
        for b in range(len(lens)):
            for g in range(s.Hq):
                if lens[b]:
                    assert_out_close(got[b, g], ref[b, g], 1e-3, (b, g))
        assert tqa.tq_get_status(ctx) == 0


def test_noalloc_rejects_workspace_beyond_the_scratch():
    s = Setup(Hq=8, Hkv=2, W=16, P=32)
    ctx = context_for(s)
    B, max_pages = 4096, 4096
    assert tqa.tq_decode_workspace_bytes(ctx, B, max_pages, 1) > tqa.TQ_NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    bt = torch.zeros((B, max_pages), dtype=torch.int32, device="cuda")
    with pytest.raises(tqa.TQError) as e:
        tqa.tq_decode_attn_noalloc(ctx, torch.zeros((B, 8, 128), device="cuda"), dummy, bt,
                                   torch.zeros(B, dtype=torch.int32, device="cuda"),
                                   torch.zeros((B, 2, 16, 128), dtype=torch.float16, device="cuda"),
                                   torch.zeros((B, 2, 16, 128), dtype=torch.float16, device="cuda"),
                                   torch.zeros((B, 8, 128), device="cuda"), 0.1, pages_per_split=1, num_pages=0)
    assert e.value.code == tqa.TQ_ERR_WORKSPACE
