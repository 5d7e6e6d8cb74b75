"""Whole-tensor encode/decode and the blob layout, contiguous and paged.

The pages (the abstract of *Beyond Compression Ratio: High-Throughput KV
Compression for Disaggregated LLM Serving* and the episode notes of
*FastKVComp: checking whether high-throughput KV compression pays off*)
describe compressing the KV cache before it crosses the prefill-to-decode
link and decoding it on the other side; they define no byte format.  The
layout used here, for a KV tensor [L, 2, T, H, D] (2 = K then V) with b_K
and b_V bits per code and group size G:

  codes section  for l in 0..L-1, for kv in (K, V): the code slab of T*H
                 rows in (t, h) order, each row D*b_kv/8 bytes of packed
                 codes, stored in tiles of 64 rows (see ``tile_codes``),
                 then zero bytes up to a multiple of 256
  meta section   for l in 0..L-1, for kv in (K, V): the meta slab of T*H*D/G
                 entries of 4 bytes in (t, h, group) order, fp16 scale
                 (bytes 0-1) then fp16 zero (bytes 2-3), little endian, then
                 zero bytes up to a multiple of 256

Every slab therefore starts on a 256-byte boundary, and so does every full
tile of 64 rows inside it (64 code rows are a multiple of 1 KiB, 64 rows of
meta a multiple of 256 bytes).  When T*H*D*b/8 and T*H*D/G*4 are multiples
of 256 there is no padding between slabs.

Paged input: a pool [L, 2, num_blocks, block_size, H, D] and, per request
r, a row of a block table naming the physical block of each logical block
of ``block_size`` tokens, and a length seq_len[r].  Request r is encoded as
the contiguous tensor of its first seq_len[r] tokens; its blob sits at
offsets[r], the prefix sum of the earlier requests' blob sizes (each a
multiple of 256).  Table entries past ceil(seq_len / block_size) and the
slots of the last block past seq_len are ignored, and decode writes only
the first seq_len[r] tokens of each request.
"""

from dataclasses import dataclass

import numpy as np

from .rounding import storage_to_f64, f64_to_storage
from .signs import sign_vector
from .rht import rotate, unrotate
from .quant import group_meta, quantize, pack_codes, unpack_codes, dequantize


def _align256(n: int) -> int:
    return (n + 255) // 256 * 256


TILE_ROWS = 64   # rows of one code tile
PIECE = 16       # bytes of one piece of a code row

# Order of the code bytes inside a slab (this library's own reading; the pages
# fix no byte format).  Rows are cut into tiles of TILE_ROWS consecutive rows
# (the last tile may be shorter, n rows); tile k starts at byte
# k * TILE_ROWS * RB of the slab.  Inside a tile each row's RB bytes are cut
# into RB / PIECE pieces of PIECE bytes, and piece c of the tile's row i sits
# at byte (c * n + i) * PIECE of the tile: all rows' piece 0, then all rows'
# piece 1, and so on.  The tiles take rows * RB bytes, the slab's padding
# follows them.


def tile_codes(rows: np.ndarray) -> np.ndarray:
    """[R, RB] packed code rows -> the slab's R * RB bytes in tiled order."""
    rows = np.asarray(rows, dtype=np.uint8)
    R, RB = rows.shape
    if RB % PIECE:
        raise ValueError("row bytes must be a multiple of the piece size")
    out = np.empty(R * RB, dtype=np.uint8)
    for t0 in range(0, R, TILE_ROWS):
        n = min(TILE_ROWS, R - t0)
        pieces = rows[t0:t0 + n].reshape(n, RB // PIECE, PIECE)     # [row, piece, byte]
        out[t0 * RB:(t0 + n) * RB] = pieces.transpose(1, 0, 2).reshape(-1)
    return out


def untile_codes(data: np.ndarray, R: int, RB: int) -> np.ndarray:
    """Inverse of :func:`tile_codes`: R * RB slab bytes -> [R, RB] rows."""
    data = np.asarray(data, dtype=np.uint8)[:R * RB]
    rows = np.empty((R, RB), dtype=np.uint8)
    for t0 in range(0, R, TILE_ROWS):
        n = min(TILE_ROWS, R - t0)
        pieces = data[t0 * RB:(t0 + n) * RB].reshape(RB // PIECE, n, PIECE)   # [piece, row, byte]
        rows[t0:t0 + n] = pieces.transpose(1, 0, 2).reshape(n, RB)
    return rows


def code_offsets(rows_idx, R: int, RB: int) -> np.ndarray:
    """Byte offsets inside a slab of the RB code bytes of each row in rows_idx ([k, RB])."""
    r = np.asarray(rows_idx, dtype=np.int64)[:, None]
    t0 = r // TILE_ROWS * TILE_ROWS
    n = np.minimum(TILE_ROWS, R - t0)
    j = np.arange(RB, dtype=np.int64)[None, :]
    return t0 * RB + ((j // PIECE) * n + (r - t0)) * PIECE + j % PIECE


@dataclass(frozen=True)
class BlobLayout:
    layers: int
    tokens: int
    kv_heads: int
    head_dim: int
    bits_k: int
    bits_v: int
    group: int

    @property
    def rows(self) -> int:
        return self.tokens * self.kv_heads

    def row_bytes(self, kv: int) -> int:
        return self.head_dim * (self.bits_k if kv == 0 else self.bits_v) // 8

    @property
    def groups(self) -> int:
        return self.head_dim // self.group

    def code_slab_bytes(self, kv: int) -> int:
        """Bytes of one (layer, K/V) code slab, padding included."""
        return _align256(self.rows * self.row_bytes(kv))

    @property
    def meta_slab_bytes(self) -> int:
        """Bytes of one (layer, K/V) meta slab, padding included."""
        return _align256(self.rows * self.groups * 4)

    @property
    def meta_offset(self) -> int:
        return self.layers * (self.code_slab_bytes(0) + self.code_slab_bytes(1))

    @property
    def total(self) -> int:
        return self.meta_offset + 2 * self.layers * self.meta_slab_bytes

    def codes_slab(self, l: int, kv: int) -> int:
        """Byte offset of the (layer, K/V) code slab."""
        return l * (self.code_slab_bytes(0) + self.code_slab_bytes(1)) + kv * self.code_slab_bytes(0)

    def meta_slab(self, l: int, kv: int) -> int:
        """Byte offset of the (layer, K/V) meta slab."""
        return self.meta_offset + (l * 2 + kv) * self.meta_slab_bytes

    def padding(self):
        """The zero-filled byte ranges [start, end) of the blob, in order."""
        out = []
        for l in range(self.layers):
            for kv in range(2):
                c = self.codes_slab(l, kv)
                out.append((c + self.rows * self.row_bytes(kv), c + self.code_slab_bytes(kv)))
        for l in range(self.layers):
            for kv in range(2):
                m = self.meta_slab(l, kv)
                out.append((m + self.rows * self.groups * 4, m + self.meta_slab_bytes))
        return [(a, b) for a, b in out if b > a]


def blob_layout(layers, tokens, kv_heads, head_dim, bits_k, bits_v, group) -> BlobLayout:
    if head_dim < 2 or head_dim & (head_dim - 1):
        raise ValueError("head_dim must be a power of two")
    for b in (bits_k, bits_v):
        if b not in (2, 4, 8):
            raise ValueError("bits must be 2, 4 or 8")
    if group <= 0 or head_dim % group:
        raise ValueError("group must divide head_dim")
    return BlobLayout(layers, tokens, kv_heads, head_dim, bits_k, bits_v, group)


@dataclass
class EncodeTrace:
    """Intermediate values of one oracle encode (indexed [L, 2, T, H, ...])."""
    y: np.ndarray       # rotated values y = H (s * x) / sqrt(D), float64 [L,2,T,H,D]
    t: np.ndarray       # pre-rounding code values (y - zero) / scale, float64 [L,2,T,H,D]
    q: np.ndarray       # codes, uint8 [L,2,T,H,D]
    scale: np.ndarray   # float16 [L,2,T,H,D/G]
    zero: np.ndarray    # float16 [L,2,T,H,D/G]


def encode(x_bits: np.ndarray, dtype: str, bits_k: int, bits_v: int, group: int, seed: int):
    """Encode a [L, 2, T, H, D] tensor given as uint16 storage of ``dtype``.

    Returns (blob uint8 array, EncodeTrace).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    L, two, T, H, D = x_bits.shape
    if two != 2:
        raise ValueError("second axis must be K/V")
    lay = blob_layout(L, T, H, D, bits_k, bits_v, group)
    s = sign_vector(seed, D)
    x = storage_to_f64(x_bits, dtype)
    y = rotate(x, s)
    blob = np.zeros(lay.total, dtype=np.uint8)
    G = group
    t_all = np.zeros_like(y)
    q_all = np.zeros(y.shape, dtype=np.uint8)
    sc_all = np.zeros((L, 2, T, H, D // G), dtype=np.float16)
    ze_all = np.zeros_like(sc_all)
    for l in range(L):
        for kv in range(2):
            b = bits_k if kv == 0 else bits_v
            yl = y[l, kv].reshape(T * H, D)
            scale, zero = group_meta(yl, G, b)
            q, t = quantize(yl, scale, zero, G, b)
            packed = tile_codes(pack_codes(q, b))
            off = lay.codes_slab(l, kv)
            blob[off:off + packed.size] = packed
            meta = np.stack([scale.view(np.uint16), zero.view(np.uint16)], axis=-1)
            mbytes = meta.astype("<u2").view(np.uint8).reshape(-1)
            moff = lay.meta_slab(l, kv)
            blob[moff:moff + mbytes.size] = mbytes
            t_all[l, kv] = t.reshape(T, H, D)
            q_all[l, kv] = q.reshape(T, H, D)
            sc_all[l, kv] = scale.reshape(T, H, D // G)
            ze_all[l, kv] = zero.reshape(T, H, D // G)
    return blob, EncodeTrace(y=y, t=t_all, q=q_all, scale=sc_all, zero=ze_all)


def decode(blob: np.ndarray, shape, dtype: str, bits_k: int, bits_v: int, group: int, seed: int):
    """Decode a blob back to a [L, 2, T, H, D] tensor.

    Returns (uint16 storage of ``dtype`` rounded to nearest even, float64
    values before that rounding).
    """
    L, two, T, H, D = shape
    lay = blob_layout(L, T, H, D, bits_k, bits_v, group)
    blob = np.asarray(blob, dtype=np.uint8)
    if blob.size < lay.total:
        raise ValueError("blob smaller than the layout requires")
    s = sign_vector(seed, D)
    G = group
    xhat = np.zeros((L, 2, T, H, D), dtype=np.float64)
    for l in range(L):
        for kv in range(2):
            b = bits_k if kv == 0 else bits_v
            rb = lay.row_bytes(kv)
            off = lay.codes_slab(l, kv)
            packed = untile_codes(blob[off:off + T * H * rb], T * H, rb)
            q = unpack_codes(packed, b, D)
            moff = lay.meta_slab(l, kv)
            m = blob[moff:moff + T * H * (D // G) * 4].view("<u2").reshape(T * H, D // G, 2)
            scale = m[..., 0].astype(np.uint16).view(np.float16)
            zero = m[..., 1].astype(np.uint16).view(np.float16)
            yhat = dequantize(q, scale, zero, G)
            xhat[l, kv] = unrotate(yhat, s).reshape(T, H, D)
    return f64_to_storage(xhat, dtype), xhat


def paged_layout(seq_lens, layers, kv_heads, head_dim, bits_k, bits_v, group):
    """Per-request blob offsets (int64 array) and the total size in bytes."""
    offsets = []
    total = 0
    for n in seq_lens:
        if n < 0:
            raise ValueError("negative sequence length")
        offsets.append(total)
        total += blob_layout(layers, int(n), kv_heads, head_dim, bits_k, bits_v, group).total
    return np.array(offsets, dtype=np.int64), total


def gather_request(pool: np.ndarray, table_row, seq_len: int) -> np.ndarray:
    """Tokens 0..seq_len-1 of one request from a [L,2,NB,BS,H,D] pool."""
    L, two, NB, BS, H, D = pool.shape
    out = np.zeros((L, 2, seq_len, H, D), dtype=pool.dtype)
    for t in range(seq_len):
        blk = int(table_row[t // BS])
        if not 0 <= blk < NB:
            raise IndexError("block table entry outside the pool")
        out[:, :, t] = pool[:, :, blk, t % BS]
    return out


def encode_paged(pool_bits, block_table, seq_lens, dtype, bits_k, bits_v, group, seed):
    """Encode every request of a paged pool; returns (blob, offsets, traces)."""
    L, two, NB, BS, H, D = pool_bits.shape
    offsets, total = paged_layout(seq_lens, L, H, D, bits_k, bits_v, group)
    blob = np.zeros(total, dtype=np.uint8)
    traces = []
    for r, n in enumerate(seq_lens):
        x = gather_request(pool_bits, block_table[r], int(n))
        b, tr = encode(x, dtype, bits_k, bits_v, group, seed)
        blob[offsets[r]:offsets[r] + b.size] = b
        traces.append(tr)
    return blob, offsets, traces


def decode_paged(blob, pool_bits, block_table, seq_lens, dtype, bits_k, bits_v, group, seed):
    """Decode every request into a copy of ``pool_bits`` (other slots kept)."""
    L, two, NB, BS, H, D = pool_bits.shape
    offsets, total = paged_layout(seq_lens, L, H, D, bits_k, bits_v, group)
    out = np.array(pool_bits, dtype=np.uint16, copy=True)
    for r, n in enumerate(seq_lens):
        n = int(n)
        lay = blob_layout(L, n, H, D, bits_k, bits_v, group)
        sub = np.asarray(blob)[offsets[r]:offsets[r] + lay.total]
        xb, _ = decode(sub, (L, 2, n, H, D), dtype, bits_k, bits_v, group, seed)
        for t in range(n):
            out[:, :, int(block_table[r][t // BS]), t % BS] = xb[:, :, t]
    return out
