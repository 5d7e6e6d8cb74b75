"""GPU-vs-oracle comparison helpers (test infrastructure).

The four parity criteria, on identical seeded inputs, against the oracle's
plain definition of the method (``oracle/``):
  (1) rotated values: |y_gpu - y_ref| <= 1e-5 * max(|y_ref|, rms of y_ref's vector);
  (2) meta: fp16 scale / zero within 1 ulp of the oracle's
      (RD16(min y), RU16((max y - zero) / (2^b - 1))), as a distance of
      ordered bit patterns.  The scale is defined from the zero, so where the
      GPU's zero is the neighbouring fp16 value, its scale is compared with
      RU16((max y - zero_gpu) / (2^b - 1)) as well (in a group with a tiny
      range far from 0, one ulp of the zero is many ulps of the scale);
  (3) codes: equal to the code nearest to y among the levels of the GPU's own
      stored meta -- round-half-even of the exact t = (y - zero) / scale,
      computed in float64 from the oracle's y -- except where that t lies
      within a band of a rounding boundary k + 1/2, where either neighbour is
      accepted; such flips are counted and the largest boundary distance
      among them is reported.  The band is the stated 1e-5 for every code
      width (at 8 bits, where t reaches 255 and binary32 cannot resolve 1e-5,
      the kernels decide the codes near a tie again in float64).  Degenerate
      groups (a huge offset and a tiny range) are judged against the GPU's own
      rotated values, with a per-element band derived from eight binary32
      roundings of |y| and |zero| in units of the scale (``band_fp32``);
  (4) decode: relative RMS of GPU decode vs the oracle's decode (rounded to
      the storage dtype) <= 1e-3 per (layer, K/V) slice, where the oracle
      decodes its own encode with the differences that (2) and (3) allow
      replaced by the GPU's (the groups whose meta differs take the GPU's meta
      and codes, the counted flips take the GPU's code).
"""

from dataclasses import dataclass

import numpy as np

import oracle

ROT_RTOL = 1e-5
BOUNDARY = 1e-5
DECODE_RRMS = 1e-3


def band_for(bits):
    return BOUNDARY


def band_fp32(y, zero, scale, G, bits):
    """Per-element band for degenerate groups: 1e-5 plus 2^-21 (eight binary32
    roundings) of (|y| + |zero| + (2^b - 1) scale) in units of the scale."""
    yg = np.abs(np.asarray(y, dtype=np.float64)).reshape(y.shape[:-1] + (-1, G))
    z = np.abs(zero.astype(np.float64))[..., None]
    s = scale.astype(np.float64)[..., None]
    qmax = 2 ** bits - 1
    band = BOUNDARY + 2.0 ** -21 * (yg + z + qmax * s) / np.where(s > 0, s, 1.0)
    return band.reshape(y.shape)


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
    codes: int = 0
    meta_diff_groups: int = 0        # (i) groups whose meta differs by one ulp
    code_mismatches: int = 0         # (ii) elements whose codes differ from the oracle's own
    boundary_flips: int = 0          # codes differing from the nearest level of the GPU's meta
    worst_boundary_distance: float = 0.0   # (iii) max |t - (k + 1/2)| among the flips
    flips_beyond_1e5: int = 0        # flips farther than 1e-5 from their boundary (8-bit only)

    def merge(self, o):
        for f in ("vectors", "groups", "codes", "meta_diff_groups", "code_mismatches", "boundary_flips",
                  "flips_beyond_1e5"):
            setattr(self, f, getattr(self, f) + getattr(o, f))
        self.worst_boundary_distance = max(self.worst_boundary_distance, o.worst_boundary_distance)
        return self

    def as_dict(self):
        return dict(self.__dict__)


@dataclass
class RowsResult:
    report: CodeReport
    codes: np.ndarray     # the oracle's codes with the allowed differences taken from the GPU, uint8 [N, D]
    scale: np.ndarray     # the oracle's meta with the allowed differences taken from the GPU, float16
    zero: np.ndarray


def check_rows(x_bits, dtype, bits, group, seed, codes_gpu, meta_gpu, band=None, y=None):
    """Criteria (2) and (3) for N vectors of one code width.

    x_bits: uint16 [N, D] storage; codes_gpu: uint8 [N, D*bits/8];
    meta_gpu: uint16 [N, D/group, 2] (scale, zero) bit patterns.
    band: None for ``band_for(bits)``, a float, an array shaped like the
    codes, or "fp32" for ``band_fp32`` of the GPU's meta.  A code is accepted
    when it is the nearest level, or when |q - t| <= 1/2 + band (t clipped to
    the code range).  y: the rotated values to judge the meta and codes
    against; by default the oracle's, y = H (s * x) / sqrt(D).  Returns a
    RowsResult.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    N, D = x_bits.shape
    if y is None:
        y = oracle.rotate(oracle.storage_to_f64(x_bits, dtype), oracle.sign_vector(seed, D))
    y = np.asarray(y, dtype=np.float64).reshape(N, D)
    scale, zero = oracle.group_meta(y, group, bits)
    q_ref, _ = oracle.quantize(y, scale, zero, group, bits)
    sg = np.asarray(meta_gpu[..., 0], dtype=np.uint16)
    zg = np.asarray(meta_gpu[..., 1], dtype=np.uint16)
    dz = np.abs(ordered16(zg) - ordered16(zero.view(np.uint16)))
    ds = np.abs(ordered16(sg) - ordered16(scale.view(np.uint16)))
    if (dz > 0).any():   # the scale that belongs to the GPU's own zero
        mx = y.reshape(N, -1, group).max(axis=-1)
        zgf = zg.view(np.float16).astype(np.float64)
        with np.errstate(over="ignore"):
            s_zg = oracle.ru16(np.maximum(mx - zgf, 0.0) / float(2 ** bits - 1))
        ds = np.minimum(ds, np.abs(ordered16(sg) - ordered16(s_zg.view(np.uint16))))
    assert ds.max(initial=0) <= 1 and dz.max(initial=0) <= 1, \
        "meta differs by more than one fp16 ulp (scale %d, zero %d)" % (ds.max(), dz.max())
    meta_diff = (ds > 0) | (dz > 0)
    rep = CodeReport(vectors=N, groups=ds.size, codes=N * D, meta_diff_groups=int(meta_diff.sum()))
    q_gpu = oracle.unpack_codes(np.asarray(codes_gpu, dtype=np.uint8), bits, D)
    # the exact t of the oracle's y against the GPU's own stored meta
    s_g, z_g = sg.view(np.float16), zg.view(np.float16)
    t = oracle.code_values(y, s_g, z_g, group)
    q_exp = oracle.nearest_codes(t, bits)
    if band is None:
        band = band_for(bits)
    elif isinstance(band, str):
        assert band == "fp32", band
        band = band_fp32(y, z_g, s_g, group, bits)
    t_c = np.clip(t, 0.0, float(2 ** bits - 1))
    # a flip's excess over one half: its distance from the boundary between
    # the GPU's code and the nearest one (for a neighbouring code)
    excess = np.abs(q_gpu - t_c) - 0.5
    flips = q_gpu != q_exp
    bad = flips & (excess > band)
    assert not bad.any(), "%d codes differ away from a rounding boundary (t=%s, gpu=%s)" % (
        bad.sum(), t[bad][:4], q_gpu[bad][:4])
    rep.code_mismatches = int((q_gpu != q_ref).sum())
    rep.boundary_flips = int(flips.sum())
    if flips.any():
        rep.worst_boundary_distance = float(excess[flips].max())
        rep.flips_beyond_1e5 = int((flips & (excess >= BOUNDARY)).sum())
    # the oracle's encode with the allowed differences replaced by the GPU's
    group_of = np.repeat(meta_diff, group, axis=-1)
    q_sub = np.where(group_of | flips, q_gpu, q_ref).astype(np.uint8)
    s_sub = np.where(meta_diff, s_g, scale).astype(np.float16)
    z_sub = np.where(meta_diff, z_g, zero).astype(np.float16)
    return RowsResult(rep, q_sub, s_sub, z_sub)


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


def decode_rows_ref(res: RowsResult, dtype, group, seed):
    """The oracle's decode (storage bits [N, D]) of a RowsResult's substituted encode."""
    D = res.codes.shape[-1]
    yhat = oracle.dequantize(res.codes, res.scale, res.zero, group)
    return oracle.f64_to_storage(oracle.unrotate(yhat, oracle.sign_vector(seed, D)), dtype)


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


@dataclass
class BlobResult:
    report: CodeReport
    blob: np.ndarray        # the oracle's blob of the substituted encode (criterion 4's reference)
    reference: np.ndarray   # the oracle's decode of that blob, uint16 [L, 2, T, H, D]


def check_blob(x_bits, blob_gpu, dtype, bits_k, bits_v, group, seed, band=None):
    """Whole-blob comparison of a small contiguous encode: (2), (3) and the
    padding; returns a BlobResult whose ``reference`` is the decode that
    criterion (4) compares the GPU's decode with."""
    L, _, T, H, D = x_bits.shape
    lay = oracle.blob_layout(L, T, H, D, bits_k, bits_v, group)
    blob_gpu = np.asarray(blob_gpu, dtype=np.uint8)
    assert blob_gpu.size >= lay.total
    rep = CodeReport()
    ref = np.zeros(x_bits.shape, dtype=np.uint16)
    sub = np.zeros(lay.total, dtype=np.uint8)
    for l in range(L):
        for kv in range(2):
            b = bits_k if kv == 0 else bits_v
            codes, meta = blob_rows(blob_gpu, lay, l, kv, np.arange(T * H))
            r = check_rows(x_bits[l, kv].reshape(-1, D), dtype, b, group, seed, codes, meta, band)
            rep.merge(r.report)
            ref[l, kv] = decode_rows_ref(r, dtype, group, seed).reshape(T, H, D)
            packed = oracle.tile_codes(oracle.pack_codes(r.codes, b))
            c0 = lay.codes_slab(l, kv)
            sub[c0:c0 + packed.size] = packed
            m = np.stack([r.scale.view(np.uint16), r.zero.view(np.uint16)], axis=-1).astype("<u2")
            m0 = lay.meta_slab(l, kv)
            sub[m0:m0 + m.size * 2] = m.view(np.uint8).reshape(-1)
    for a, b in lay.padding():
        assert not blob_gpu[a:b].any(), "padding [%d, %d) not zero" % (a, b)
    return BlobResult(rep, sub, ref)
