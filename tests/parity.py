"""GPU-vs-oracle comparison helpers (test infrastructure).

The four parity criteria, on identical seeded inputs:
  (1) rotated values: |y_gpu - y_ref| <= 1e-5 * max(|y_ref|, rms of y_ref's vector);
  (2) meta: fp16 scale / zero within 1 ulp (distance of ordered bit patterns);
  (3) codes: bit-exact except where the pre-rounding value t, recomputed by
      the oracle (binary32 decision arithmetic) from its rotated values and
      the GPU's own stored meta, lies within 1e-5 of a rounding boundary
      k + 1/2 (mismatches are counted and reported);
  (4) decode: relative RMS of GPU decode vs the oracle's decode (rounded to
      the storage dtype) <= 1e-3 per (layer, K/V) slice.
"""

from dataclasses import dataclass, field

import numpy as np

import oracle

ROT_RTOL = 1e-5
BOUNDARY = 1e-5
DECODE_RRMS = 1e-3


def ordered16(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def check_rotation(y_gpu, y_ref):
    """Criterion (1); returns the worst |dy| / allowed ratio."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64).reshape(-1, y_ref.shape[-1])
    y_ref = np.asarray(y_ref, dtype=np.float64).reshape(-1, y_ref.shape[-1])
    rms = np.sqrt(np.mean(y_ref ** 2, axis=1, keepdims=True))
    allowed = ROT_RTOL * np.maximum(np.abs(y_ref), rms)
    err = np.abs(y_gpu - y_ref)
    bad = err > allowed
    assert not bad.any(), "rotation: %d elements outside 1e-5 relative (worst %.3g)" % (
        bad.sum(), (err / np.maximum(allowed, 1e-300)).max())
    return float((err / np.maximum(allowed, 1e-300)).max())


@dataclass
class CodeReport:
    vectors: int = 0
    groups: int = 0
    meta_diff_groups: int = 0       # (i) groups whose meta differs by one ulp
    code_mismatches: int = 0        # (ii) elements whose codes differ
    worst_boundary_distance: float = 0.0   # (iii) max |t - (k + 1/2)| among (ii)
    notes: list = field(default_factory=list)

    def merge(self, o):
        self.vectors += o.vectors
        self.groups += o.groups
        self.meta_diff_groups += o.meta_diff_groups
        self.code_mismatches += o.code_mismatches
        self.worst_boundary_distance = max(self.worst_boundary_distance, o.worst_boundary_distance)
        return self


def check_rows(x_bits, dtype, bits, group, seed, codes_gpu, meta_gpu, boundary=BOUNDARY):
    """Criteria (2) and (3) for N vectors of one code width.

    x_bits: uint16 [N, D] storage; codes_gpu: uint8 [N, D*bits/8];
    meta_gpu: uint16 [N, D/group, 2] (scale, zero) bit patterns.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    N, D = x_bits.shape
    s = oracle.sign_vector(seed, D)
    u = oracle.rotate_raw(oracle.storage_to_f64(x_bits, dtype), s)
    scale, zero = oracle.group_meta(u, group, bits)
    q_ref, _ = oracle.quantize(u, scale, zero, group, bits)
    sg = np.asarray(meta_gpu[..., 0], dtype=np.uint16)
    zg = np.asarray(meta_gpu[..., 1], dtype=np.uint16)
    ds = np.abs(ordered16(sg) - ordered16(scale.view(np.uint16)))
    dz = np.abs(ordered16(zg) - ordered16(zero.view(np.uint16)))
    assert ds.max(initial=0) <= 1 and dz.max(initial=0) <= 1, \
        "meta differs by more than one fp16 ulp (scale %d, zero %d)" % (ds.max(), dz.max())
    rep = CodeReport(vectors=N, groups=ds.size, meta_diff_groups=int(((ds > 0) | (dz > 0)).sum()))
    q_gpu = oracle.unpack_codes(np.asarray(codes_gpu, dtype=np.uint8), bits, D)
    # pre-rounding value from the oracle's rotated values and the GPU's own
    # stored meta, in the oracle's binary32 decision arithmetic
    t = oracle.code_values(u, sg.view(np.float16), zg.view(np.float16), group)
    q_exp = np.rint(np.clip(t, 0, 2 ** bits - 1))
    dist = np.abs(t - (np.floor(t) + 0.5))
    near = dist < boundary
    neighbor = (q_gpu == np.floor(t)) | (q_gpu == np.floor(t) + 1)
    bad = (q_gpu != q_exp) & ~(near & neighbor)
    assert not bad.any(), "%d codes differ away from a rounding boundary (t=%s, gpu=%s)" % (
        bad.sum(), t[bad][:4], q_gpu[bad][:4])
    mism = q_gpu != q_ref
    rep.code_mismatches = int(mism.sum())
    flips = q_gpu != q_exp
    if flips.any():
        rep.worst_boundary_distance = float(dist[flips].max())
    return rep


def check_decode(x_gpu_bits, x_ref_bits, dtype, axis_slices=None):
    """Criterion (4): relative RMS per slice (leading axes) and overall."""
    g = oracle.storage_to_f64(np.asarray(x_gpu_bits, dtype=np.uint16), dtype)
    r = oracle.storage_to_f64(np.asarray(x_ref_bits, dtype=np.uint16), dtype)
    lead = g.shape[:2] if axis_slices is None else axis_slices
    g2 = g.reshape(int(np.prod(lead)), -1)
    r2 = r.reshape(int(np.prod(lead)), -1)
    num = np.sqrt(np.sum((g2 - r2) ** 2, axis=1))
    den = np.sqrt(np.sum(r2 ** 2, axis=1))
    rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    assert rel.max(initial=0) <= DECODE_RRMS, "decode relative RMS %.3g > 1e-3" % rel.max()
    return float(rel.max(initial=0))


def blob_rows(blob, lay, l, kv, rows_idx):
    """(codes [n, RB], meta [n, NG, 2]) of rows `rows_idx` of slab (l, kv) in a host blob."""
    rb = lay.row_bytes(kv)
    ng = lay.groups
    c0 = lay.codes_slab(l, kv)
    m0 = lay.meta_slab(l, kv)
    idx = np.asarray(rows_idx, dtype=np.int64)
    codes = blob[c0 + oracle.code_offsets(idx, lay.rows, rb)]
    meta = blob[m0:m0 + lay.rows * ng * 4].view("<u2").reshape(lay.rows, ng, 2)[idx]
    return codes, meta


def check_blob(x_bits, blob_gpu, dtype, bits_k, bits_v, group, seed):
    """Whole-blob comparison of a small contiguous encode: (2), (3) and the padding."""
    L, _, T, H, D = x_bits.shape
    lay = oracle.blob_layout(L, T, H, D, bits_k, bits_v, group)
    blob_gpu = np.asarray(blob_gpu, dtype=np.uint8)
    assert blob_gpu.size >= lay.total
    rep = CodeReport()
    for l in range(L):
        for kv in range(2):
            b = bits_k if kv == 0 else bits_v
            codes, meta = blob_rows(blob_gpu, lay, l, kv, np.arange(T * H))
            rep.merge(check_rows(x_bits[l, kv].reshape(-1, D), dtype, b, group, seed, codes, meta))
    for a, b in lay.padding():
        assert not blob_gpu[a:b].any(), "padding [%d, %d) not zero" % (a, b)
    return rep
