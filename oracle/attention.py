"""Decode attention over the paged compressed cache (test oracle only).

Plain definition ("TurboQuant Family Design Study", section "Why keys and
values need different treatment"): logits l_t = q.k_t / sqrt(d) (sm_scale),
p = softmax(l), o = sum_t p_t v_t.  Compressed tokens use the dequantised
k_hat, v_hat; the last min(T, W) tokens use their FP16 values (section
"Packed format and complete bit accounting", recommended first mode).  With
GQA, query head g reads kv head g // (Hq / Hkv) (contiguous grouping; the
pages only define GQA as Hkv < Hq).

``attention_compressed`` is the second route, the compressed-domain formula
("TurboQuant Family Design Study", sections "Placement relative to RoPE and
attention" (q.k = (Tq).(Tk)) and "CPU and WASM kernel design"; "aither-kvcache"
README, "Zero-buffer fused attention"): rotate the query once, score each
token as n_t <q_rot, c[idx_t]> + sqrt(pi/2)/d ||r_t|| <S q_rot, 2 sigma_t - 1>,
accumulate n^V_t c_V[idx^V_t] in the rotated basis, rotate back once, and add
the exactly scored window.  In exact arithmetic both routes agree.
"""

import numpy as np

from . import codec


def _softmax_out(logits, values):
    m = np.max(logits)
    w = np.exp(logits - m)
    return (w @ values) / np.sum(w), w


def attention_plain(cache, q, sm_scale, pairs=None):
    """Returns (out [B, Hq, d], logits list per (b, g) in token order).

    ``pairs``: optional list of (b, kv head) to evaluate (the others are left
    at zero / None), for sampled checks of large caches."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    H = cache.lay.H
    G = Hq // H
    out = np.zeros((B, Hq, d))
    logits = [[None] * Hq for _ in range(B)]
    want = None if pairs is None else set((int(b), int(h)) for b, h in pairs)
    for b in range(B):
        for h in range(H):
            if want is not None and (b, h) not in want:
                continue
            ks, vs = [], []
            comp = cache.compressed(b, h)
            if comp is not None:
                krec, vn, vidx = comp
                ks.append(codec.dequantize(krec.codes, krec.norms, cache.rot, cache.kcb,
                                           krec.signs, krec.rnorms, cache.S, cache.qjl_coef))
                vs.append(cache.rot.inverse(vn.astype(np.float64)[:, None] * cache.vcb.values(vidx)))
            _, kw, vw = cache.window_tokens(b, h)
            ks.append(kw)
            vs.append(vw)
            K = np.concatenate(ks)
            V = np.concatenate(vs)
            for g in range(h * G, (h + 1) * G):
                if K.shape[0] == 0:
                    logits[b][g] = np.zeros(0)
                    continue
                l = (K @ q[b, g]) * sm_scale
                out[b, g], _ = _softmax_out(l, V)
                logits[b][g] = l
    return out, logits


def attention_compressed(cache, q, sm_scale):
    """Compressed-domain route; same return convention as ``attention_plain``."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    lay = cache.lay
    H, D = lay.H, lay.D
    G = Hq // H
    alpha = cache.qjl_coef
    out = np.zeros((B, Hq, d))
    logits = [[None] * Hq for _ in range(B)]
    for b in range(B):
        for h in range(H):
            comp = cache.compressed(b, h)
            _, kw, vw = cache.window_tokens(b, h)
            for g in range(h * G, (h + 1) * G):
                qg = q[b, g]
                q_rot = cache.rot.forward(qg[None, :])[0]
                parts = []
                if comp is not None:
                    krec, vn, vidx = comp
                    kidx = cache.kcb.unpack(krec.codes, D)
                    s = krec.norms.astype(np.float64) * (cache.kcb.values(kidx) @ q_rot)
                    if lay.qjl:
                        p = cache.S @ q_rot
                        pm = 2.0 * codec.unpack_bits(krec.signs, 1, D) - 1.0
                        s = s + alpha * krec.rnorms.astype(np.float64) * (pm @ p)
                    parts.append(s * sm_scale)
                parts.append((kw @ qg) * sm_scale)
                l = np.concatenate(parts)
                if l.size == 0:
                    logits[b][g] = l
                    continue
                m = np.max(l)
                w = np.exp(l - m)
                nc = 0 if comp is None else comp[0].norms.shape[0]
                acc_rot = np.zeros(D)
                if nc:
                    acc_rot = (w[:nc] * vn.astype(np.float64)) @ cache.vcb.values(vidx)
                acc_win = w[nc:] @ vw
                out[b, g] = (cache.rot.inverse(acc_rot[None, :])[0] + acc_win) / np.sum(w)
                logits[b][g] = l
    return out, logits
