"""Byte and bit accounting (test oracle only).

* FP KV bytes per token = 2 L H_kv d s ("TurboQuant Family Design Study",
  section "Capacity model").
* Payload with a recent FP16 window ("Capacity model", the M(T) formula):
  L H_kv d ( max(T-W,0) (bK+bV)/8 + min(T,W) * 4 ), excluding page and scratch.
* All-in bits per channel b_nominal + (b_norm + b_aux)/d + 64*8/(P H_kv d)
  (section "Packed format and complete bit accounting").
* Memory compression factor 4 / ((bK+bV)/8) (section "Final recommendation
  and expected gains").
* Per-vector record: d*b/8 code bytes + a 4-byte f32 norm ("aither-kvcache"
  README, "Compression Ratios"); keys with QJL add d/8 sign bytes and a 4-byte
  residual norm (the sign sketch of "TurboQuant on a 16GB MacBook"; its
  residual norm storage is this build's reading).
"""


def fp_bytes_per_token(layers, kv_heads, head_dim, bytes_per_scalar):
    return 2 * layers * kv_heads * head_dim * bytes_per_scalar


def payload_bytes_windowed(layers, kv_heads, head_dim, T, W, key_bits, value_bits):
    comp = max(T - W, 0)
    win = min(T, W)
    return layers * kv_heads * head_dim * (comp * (key_bits + value_bits) / 8 + win * 4)


def all_in_bpc(b_nominal, b_norm, b_aux, head_dim, page_tokens, kv_heads, header_bytes=64):
    return b_nominal + (b_norm + b_aux) / head_dim + header_bytes * 8 / (page_tokens * kv_heads * head_dim)


def memory_compression(key_bits, value_bits):
    return 4.0 / ((key_bits + value_bits) / 8.0)


def record_bytes(head_dim, bits, qjl=False, norm_bytes=4):
    """Bytes per stored vector: codes + f32 norm (+ d/8 signs + f32 residual norm)."""
    b = head_dim * bits // 8 + norm_bytes
    if qjl:
        b += head_dim // 8 + 4
    return b


def compressed_token_head_bytes(head_dim, key_bits, key_qjl, value_bits):
    """Key record + value record bytes for one token of one kv head."""
    return record_bytes(head_dim, key_bits, key_qjl) + record_bytes(head_dim, value_bits, False)


def decode_algorithmic_bytes(seq_lens, kv_heads, head_dim, key_bits, key_qjl, value_bits, window):
    """Bytes one decode call must read from the cache: the compressed records of
    every token older than the window plus the FP16 window K and V."""
    per = compressed_token_head_bytes(head_dim, key_bits, key_qjl, value_bits)
    total = 0
    for T in seq_lens:
        comp = max(int(T) - window, 0)
        win = min(int(T), window)
        total += kv_heads * (comp * per + win * head_dim * 2 * 2)
    return total
