"""Paged compressed KV cache with an FP16 recent-token window (test oracle only).

Follows the page design of "TurboQuant Family Design Study", section "Packed
format and complete bit accounting" (fixed-token pages, token-major append,
head-major inner layout, a 64-byte header, body order: key norms, key codes,
key residual signs, value norms, value codes, 16-byte alignment) and the
recent FP16 window of the same page's recommended first mode (last W tokens
of K and V kept in FP16); the capacity formula in "Capacity model" counts the
window inside T, so a sequence of T tokens has max(T - W, 0) compressed
tokens.  Append order and fixed-page growth follow "Paging, lifecycle, and
cache identity".

Byte layout (the pages leave field order and sizes open; this is the layout
the library implements, stated here independently of its source):

  page_bytes = roundup(256 + H_kv * head_bytes, 256)
  header, bytes [0, 64):
     0 u32 magic 0x564B5154 ("TQKV")     4 u16 format version (1)
     6 u16 head_dim                        8 u8 key_bits   9 u8 key QJL (0 none,
                                           1 Gaussian S, 2 orthogonal S)
    10 u8 value_bits                      11 u8 rotation (0 dense, 1 hadamard)
    12 u16 num_kv_heads                   14 u16 page_tokens
    16 u32 valid tokens in this page      20 u32 codebook version (1)
    24 u64 seed                           32 u32 page index within its sequence
    36 u8 key norm format (0 float32, 1 u8 log-norm)
    37..63 zero; bytes [64, 256) zero
  body, head h at 256 + h * head_bytes, streams in this order:
    key norms   f32 [P], or u8 [P] log-norm codes (``oracle.lognorm``)
    key rnorms  f32 [P]                (QJL only)
    key codes   u8  [P][D*bK/8]        token-major, LSB-first per token
    key signs   u8  [P][D/8]           (QJL only) bit j = sigma_j
    value norms f32 [P]
    value codes u32 [P/32][bV][D]      for each 32-token group and coordinate j
                the bV words w=0..bV-1 (word w at index [group][w][j]) form a
                32*bV-bit little-endian string; token i of the group has its
                code at bits [i*bV, (i+1)*bV).
  D is the transform size, the next power of two >= head_dim d (records of a
  head size that is not a power of two hold all D transform coordinates, see
  ``oracle.rotation``); the header stores d.
  Mixed-channel rates b + 1/2 (``oracle.mixed``): the header bits byte holds
  b + 16; a key record holds (D/2) b + (D/2)(b+1) bits (low-rate coordinates
  first); a value group holds a low-rate block u32 [bV][D/2] followed by a
  high-rate block u32 [bV+1][D/2], coordinates of each half in ascending
  order, each coordinate's words forming its 32-token string as above.
  FP16 ring: k_win, v_win [B, H_kv, W, d]; token at position t lives in slot
  t mod W while it is one of the last W tokens.
"""

import numpy as np

from . import codec
from .rotation import transform_dim

MAGIC = 0x564B5154
FORMAT_VERSION = 1
CODEBOOK_VERSION = 1
HEADER_BYTES = 64
BODY_OFFSET = 256
V_GROUP = 32


class Layout:
    def __init__(self, head_dim, key_bits, key_qjl, value_bits, num_kv_heads, page_tokens, key_mixed=False,
                 value_mixed=False, key_norm_u8=False):
        d, P = transform_dim(head_dim), page_tokens
        if P % V_GROUP:
            raise ValueError("page_tokens must be a multiple of 32")
        self.d, self.D = head_dim, d
        self.bK, self.qjl, self.bV, self.H, self.P = key_bits, int(key_qjl), value_bits, num_kv_heads, P
        self.kmix, self.vmix = bool(key_mixed), bool(value_mixed)
        self.kn8 = bool(key_norm_u8)
        # code bytes of one key record and of one token's value codes
        self.k_rec = d * key_bits // 8 + (d // 16 if self.kmix else 0)
        self.v_rec = d * value_bits // 8 + (d // 16 if self.vmix else 0)
        off = 0
        self.k_norm = off; off += (1 if self.kn8 else 4) * P
        if self.qjl:
            self.k_rnorm = off; off += 4 * P
        self.k_codes = off; off += P * self.k_rec
        if self.qjl:
            self.k_signs = off; off += P * d // 8
        self.v_norm = off; off += 4 * P
        self.v_codes = off; off += P * self.v_rec
        self.head_bytes = off
        self.page_bytes = -(-(BODY_OFFSET + num_kv_heads * off) // 256) * 256
        # value group words: coordinate j's word w sits at v_base[j] + w * v_stride
        self.v_width = np.full(d, value_bits, dtype=np.int64)
        if self.vmix:
            hi = (np.arange(d) % 8) >= 4
            rank = np.zeros(d, dtype=np.int64)
            rank[~hi] = np.arange(d // 2)
            rank[hi] = np.arange(d // 2)
            self.v_width[hi] = value_bits + 1
            self.v_base = np.where(hi, value_bits * (d // 2) + rank, rank)
            self.v_stride = d // 2
        else:
            self.v_base = np.arange(d, dtype=np.int64)
            self.v_stride = d
        self.v_group_words = V_GROUP * self.v_rec // 4

    def head_base(self, h):
        return BODY_OFFSET + h * self.head_bytes


def write_header(page: np.ndarray, lay: Layout, rotation_kind: int, seed: int, valid: int, page_index: int):
    hdr = np.zeros(HEADER_BYTES, dtype=np.uint8)
    hv = hdr.view(np.uint32)
    hv[0] = MAGIC
    hdr[4:6] = np.frombuffer(np.uint16(FORMAT_VERSION).tobytes(), np.uint8)
    hdr[6:8] = np.frombuffer(np.uint16(lay.d).tobytes(), np.uint8)
    hdr[8], hdr[9], hdr[10], hdr[11] = lay.bK + 16 * lay.kmix, lay.qjl, lay.bV + 16 * lay.vmix, rotation_kind
    hdr[12:14] = np.frombuffer(np.uint16(lay.H).tobytes(), np.uint8)
    hdr[14:16] = np.frombuffer(np.uint16(lay.P).tobytes(), np.uint8)
    hv[4] = valid
    hv[5] = CODEBOOK_VERSION
    hdr[24:32] = np.frombuffer(np.uint64(seed).tobytes(), np.uint8)
    hv[8] = page_index
    hdr[36] = 1 if lay.kn8 else 0
    page[:HEADER_BYTES] = hdr


def _f32(page, off, n):
    return page[off:off + 4 * n].view(np.float32)


def write_key_records(page, lay: Layout, h, slots, rec: codec.Encoded):
    """Store key records (flat ``codec.Encoded``) at the given token slots."""
    base = lay.head_base(h)
    cb = lay.k_rec
    if lay.kn8:
        page[base + lay.k_norm: base + lay.k_norm + lay.P][slots] = rec.norm_codes
    else:
        _f32(page, base + lay.k_norm, lay.P)[slots] = rec.norms
    codes = page[base + lay.k_codes: base + lay.k_codes + lay.P * cb].reshape(lay.P, cb)
    codes[slots] = rec.codes
    if lay.qjl:
        _f32(page, base + lay.k_rnorm, lay.P)[slots] = rec.rnorms
        sb = lay.D // 8
        signs = page[base + lay.k_signs: base + lay.k_signs + lay.P * sb].reshape(lay.P, sb)
        signs[slots] = rec.signs


def _v_words(page, lay, h):
    """Value code words of head h: u32 [P/32, words per group]."""
    base = lay.head_base(h) + lay.v_codes
    n = lay.P * lay.v_rec
    return page[base: base + n].view(np.uint32).reshape(lay.P // V_GROUP, lay.v_group_words)


def write_value_records(page, lay: Layout, h, slots, value_cb, rec: codec.Encoded):
    """Store value records at the given slots, re-packing codes group-interleaved."""
    base = lay.head_base(h)
    _f32(page, base + lay.v_norm, lay.P)[slots] = rec.norms
    words = _v_words(page, lay, h)
    idx = value_cb.unpack(rec.codes, lay.D)
    for s, code_row in zip(np.asarray(slots), idx):
        g, i = divmod(int(s), V_GROUP)
        for wd in np.unique(lay.v_width):
            js = np.nonzero(lay.v_width == wd)[0]
            for k in range(int(wd)):
                w, pos = divmod(i * int(wd) + k, 32)
                at = lay.v_base[js] + w * lay.v_stride
                val = ((code_row[js] >> k) & 1).astype(np.uint32) << np.uint32(pos)
                words[g, at] = (words[g, at] & ~np.uint32(1 << pos)) | val


def read_key_records(page, lay: Layout, h, n):
    base = lay.head_base(h)
    cb = lay.k_rec
    if lay.kn8:
        from . import lognorm
        nc = page[base + lay.k_norm: base + lay.k_norm + n].copy()
        norms = lognorm.decode(nc).astype(np.float32)
    else:
        nc = None
        norms = _f32(page, base + lay.k_norm, lay.P)[:n].copy()
    codes = page[base + lay.k_codes: base + lay.k_codes + lay.P * cb].reshape(lay.P, cb)[:n].copy()
    signs = rnorms = None
    if lay.qjl:
        rnorms = _f32(page, base + lay.k_rnorm, lay.P)[:n].copy()
        sb = lay.D // 8
        signs = page[base + lay.k_signs: base + lay.k_signs + lay.P * sb].reshape(lay.P, sb)[:n].copy()
    return codec.Encoded(codes, norms, signs, rnorms, norm_codes=nc)


def read_value_idx(page, lay: Layout, h, n):
    """Value norms [n] and code indices [n, D] of the first n slots."""
    base = lay.head_base(h)
    norms = _f32(page, base + lay.v_norm, lay.P)[:n].copy()
    words = _v_words(page, lay, h).astype(np.int64)
    idx = np.zeros((lay.P, lay.D), dtype=np.int64)
    for s in range(n):
        g, i = divmod(s, V_GROUP)
        code = np.zeros(lay.D, dtype=np.int64)
        for k in range(int(lay.v_width.max())):
            live = k < lay.v_width
            w, pos = np.divmod(i * lay.v_width + k, 32)
            at = np.where(live, lay.v_base + w * lay.v_stride, 0)
            code |= np.where(live, (words[g, at] >> pos) & 1, 0) << k
        idx[s] = code
    return norms, idx[:n]


class PagedCache:
    """Host model of the cache for one layer: page pool, block table, ring, lengths.

    ``append`` is the plain sequential definition: for each new token at
    position t of a sequence, if t >= W the ring slot t mod W holds the token
    at position t - W, which is encoded into page (t - W) // P, slot
    (t - W) mod P; then the new token (rounded to FP16) is written into slot
    t mod W.  With W = 0 every token is encoded straight into its page.
    Compressed tokens are encoded from their FP16 values.
    """

    def __init__(self, lay: Layout, rotation, key_cb, value_cb, qjl_S, window, num_pages, batch,
                 max_pages, rotation_kind=0, seed=0, qjl_coef=None):
        self.lay, self.rot, self.kcb, self.vcb, self.S = lay, rotation, key_cb, value_cb, qjl_S
        self.qjl_coef = codec.qjl_scale(lay.D) if qjl_coef is None else qjl_coef
        self.W = window
        self.pool = np.zeros((num_pages, lay.page_bytes), dtype=np.uint8)
        self.block_table = np.full((batch, max_pages), -1, dtype=np.int32)
        self.seq_lens = np.zeros(batch, dtype=np.int32)
        self.k_win = np.zeros((batch, lay.H, window, lay.d), dtype=np.float16)
        self.v_win = np.zeros_like(self.k_win)
        self.rotation_kind, self.seed = rotation_kind, seed

    def append(self, k_new, v_new, counts=None):
        """k_new, v_new: [B, H, n, d] (any float type, rounded to FP16)."""
        k16 = np.asarray(k_new).astype(np.float16)
        v16 = np.asarray(v_new).astype(np.float16)
        B, H, n, d = k16.shape
        lay, P, W = self.lay, self.lay.P, self.W
        for b in range(B):
            cnt = n if counts is None else int(counts[b])
            T0 = int(self.seq_lens[b])
            for h in range(H):
                enc_pos, enc_k, enc_v = [], [], []
                for j in range(cnt):
                    t = T0 + j
                    if W == 0:
                        enc_pos.append(t)
                        enc_k.append(k16[b, h, j].astype(np.float64))
                        enc_v.append(v16[b, h, j].astype(np.float64))
                        continue
                    if t >= W:
                        slot = t % W
                        enc_pos.append(t - W)
                        enc_k.append(self.k_win[b, h, slot].astype(np.float64))
                        enc_v.append(self.v_win[b, h, slot].astype(np.float64))
                    self.k_win[b, h, t % W] = k16[b, h, j]
                    self.v_win[b, h, t % W] = v16[b, h, j]
                if enc_pos:
                    self._store(b, h, np.array(enc_pos), np.array(enc_k), np.array(enc_v))
            self.seq_lens[b] = T0 + cnt
            self._headers(b, T0, T0 + cnt)

    def _store(self, b, h, pos, kx, vx):
        lay = self.lay
        krec = codec.encode(kx, self.rot, self.kcb, self.S if lay.qjl else None, norm_u8=lay.kn8)
        vrec = codec.encode(vx, self.rot, self.vcb, None)
        for pg in np.unique(pos // lay.P):
            sel = np.nonzero(pos // lay.P == pg)[0]
            pid = int(self.block_table[b, pg])
            if pid < 0:
                raise ValueError("no page reserved")
            page = self.pool[pid]
            slots = pos[sel] % lay.P
            sub = lambda r: codec.Encoded(r.codes[sel], r.norms[sel],
                                          None if r.signs is None else r.signs[sel],
                                          None if r.rnorms is None else r.rnorms[sel],
                                          norm_codes=None if r.norm_codes is None else r.norm_codes[sel])
            write_key_records(page, lay, h, slots, sub(krec))
            write_value_records(page, lay, h, slots, self.vcb, sub(vrec))

    def _headers(self, b, T0, T1):
        lay, W = self.lay, self.W
        c0, c1 = max(T0 - W, 0), max(T1 - W, 0)
        if c1 <= c0:
            return
        for pg in range(c0 // lay.P, (c1 - 1) // lay.P + 1):
            valid = min(lay.P, c1 - pg * lay.P)
            write_header(self.pool[int(self.block_table[b, pg])], lay, self.rotation_kind, self.seed, valid, pg)

    def compressed(self, b, h):
        """Dequantise-ready records of every compressed token of (b, h), in order."""
        lay = self.lay
        C = max(int(self.seq_lens[b]) - self.W, 0)
        krecs, vn, vidx = [], [], []
        for pg in range(-(-C // lay.P)):
            n = min(lay.P, C - pg * lay.P)
            page = self.pool[int(self.block_table[b, pg])]
            krecs.append(read_key_records(page, lay, h, n))
            a, i = read_value_idx(page, lay, h, n)
            vn.append(a)
            vidx.append(i)
        if not krecs:
            return None
        cat = lambda xs: None if xs[0] is None else np.concatenate(xs)
        k = codec.Encoded(cat([r.codes for r in krecs]), cat([r.norms for r in krecs]),
                          cat([r.signs for r in krecs]), cat([r.rnorms for r in krecs]),
                          norm_codes=cat([r.norm_codes for r in krecs]))
        return k, np.concatenate(vn), np.concatenate(vidx)

    def window_tokens(self, b, h):
        """(positions, k, v) of the FP16 window tokens of (b, h) as float64."""
        T = int(self.seq_lens[b])
        pos = np.arange(max(T - self.W, 0), T)
        if self.W == 0:
            z = np.zeros((0, self.lay.d))
            return pos, z, z
        slots = pos % self.W
        return pos, self.k_win[b, h, slots].astype(np.float64), self.v_win[b, h, slots].astype(np.float64)
