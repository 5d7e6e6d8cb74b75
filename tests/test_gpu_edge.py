"""GPU parity on the method's own edge cases, element by element against the
oracle: all-zero vectors and constant groups (scale 0), degenerate groups (a
huge offset with a tiny range, where binary32 decisions can push t past the
code range and the kernel's clamp keeps the code in its bits), and the 8-bit
boundary window on a large sample."""
import sys

import numpy as np
import pytest
import torch

import oracle
import parity
from kernel_models import butterfly_model
import gpu_util
import kv_cache_compression_kvc_amd as kvc
from kv_cache_compression_kvc_amd import inputs, presets

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _tensor(rows_k, rows_v, dtype):
    """[1, 2, T, 1, D] tensor from two float64 [T, D] arrays (values exact in dtype)."""
    x = torch.from_numpy(np.stack([rows_k, rows_v])[None, :, :, None, :]).to(TORCH[dtype])
    assert np.array_equal(x.double().numpy()[0, :, :, 0], np.stack([rows_k, rows_v])), "inputs not exact"
    return x


def _encode_check(x, bits, G, seed, band=None):
    xb = inputs.as_u16(x)
    dtype = "bf16" if x.dtype == torch.bfloat16 else "fp16"
    total, _ = kvc.encoded_size(1, x.shape[2], 1, x.shape[4], bits, bits, G, dtype)
    whole, out = gpu_util.guarded(total, DEV)
    kvc.encode(x.to(DEV), bits, bits, G, seed=seed, out=out)
    xd = kvc.decode(out, x.shape, dtype, bits, bits, G, seed=seed)
    torch.cuda.synchronize()
    assert gpu_util.canaries_intact(whole)
    blob = out.cpu().numpy()
    res = parity.check_blob(xb, blob, dtype, bits, bits, G, seed, band=band)
    rr = parity.check_decode(inputs.as_u16(xd), res.reference, dtype)
    return blob, res, rr


CONST = [(D, dt, b, G) for D in (64, 128) for dt in ("bf16", "fp16") for b in (2, 4, 8)
         for G in (32, D)]


@pytest.mark.parametrize("D,dtype,bits,G", CONST)
def test_zero_and_constant_groups(D, dtype, bits, G):
    """All-zero vectors, and at head_dim 64 (1/sqrt(D) = 1/8) vectors whose
    rotated groups are constant fp16 values: scale 0 and every code 0,
    decoding exactly; ordinary rows share the tiles."""
    rng = np.random.default_rng(D + bits + G)
    seed = 4
    rows = [np.zeros(D) for _ in range(5)]
    const_rows = list(range(5))
    if D == 64:
        # c e_k with k a multiple of G: y_i = c s_k (-1)^popcount(i & k) / 8,
        # one value per group; c e_0 + d e_G: two values, one per group half
        s = oracle.sign_vector(seed, D)
        for c in (3.0, -0.5, 12.0, 0.25):
            for k in range(0, D, G):
                r = np.zeros(D)
                r[k] = c
                rows.append(r)
                const_rows.append(len(rows) - 1)
        if G < D:
            r = np.zeros(D)
            r[0], r[G] = 6.0, 2.0
            rows.append(r)
            const_rows.append(len(rows) - 1)
        assert len(s) == D
    while len(rows) < 70:   # past one tile of 64 rows
        rows.append(oracle.storage_to_f64(oracle.f64_to_storage(rng.normal(size=D), dtype), dtype))
    rk = np.array(rows)
    rv = rk[::-1].copy()
    x = _tensor(rk, rv, dtype)
    _say("constant groups", D, dtype, bits, G)
    blob, res, rr = _encode_check(x, bits, G, seed)
    _say("  ", res.report, "decode rrms %.3g" % rr)
    lay = oracle.blob_layout(1, len(rows), 1, D, bits, bits, G)
    for kv, idx in ((0, const_rows), (1, [len(rows) - 1 - i for i in const_rows])):
        codes, meta = parity.blob_rows(blob, lay, 0, kv, np.array(idx))
        assert np.all(meta[..., 0] == 0), "constant groups must store scale 0"
        assert not codes.any(), "constant groups must store codes 0"
    # constant groups decode exactly: the decoded rows equal the inputs
    xd = kvc.decode(torch.from_numpy(blob).to(DEV), x.shape, dtype, bits, bits, G, seed=seed)
    got = inputs.as_u16(xd)[0, 0, const_rows, 0]
    assert np.array_equal(oracle.storage_to_f64(got, dtype), rk[const_rows])


def _degenerate_candidates(D, G, dtype, n, rng):
    """One large channel k, a multiple of G (so that every rotated value of a
    group sits near the same +-c / sqrt(D): the sign (-1)^popcount(i & k) is
    constant over a group), and small perturbations on a few others (a tiny
    range per group)."""
    r = np.zeros((n, D))
    r[np.arange(n), rng.integers(0, D // G, n) * G] = rng.choice([1000.0, -700.0, 2048.0, -4096.0, 16384.0], n)
    for _ in range(3):
        r[np.arange(n), rng.integers(0, D, n)] += rng.integers(1, 16, n) * 2.0 ** -rng.integers(8, 19, n)
    return oracle.storage_to_f64(oracle.f64_to_storage(r, dtype), dtype)


def _f32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def _fma_f32(a, b, c):
    """Binary32 fused multiply-add of binary32 values: a*b is exact in float64,
    the sum is rounded once to binary32 (a float64 sum that lands exactly on a
    binary32 midpoint is resolved by the sign of its rounding error)."""
    p = a * b
    s = p + c
    e = (p - (s - (s - p))) + (c - (s - p))          # TwoSum: s + e == p + c exactly
    r = _f32(s)
    lo = np.nextafter(r.astype(np.float32), np.float32(-np.inf)).astype(np.float64)
    hi = np.nextafter(r.astype(np.float32), np.float32(np.inf)).astype(np.float64)
    mid_lo, mid_hi = (r + lo) / 2, (r + hi) / 2
    r = np.where((s == mid_lo) & (e < 0), lo, r)
    r = np.where((s == mid_hi) & (e > 0), hi, r)
    return r


def kernel_decision_model(u, D, G, bits):
    """White-box binary32 model of the encode kernel's meta and code decision
    from its unnormalized rotated values u (binary32 values as float64, [N, D]):
    zero = RD16(mn * rs), scale = RU16((mx * rs - zero) / (2^b - 1)),
    inv = 1 / scale, A = inv * rs, Bz = -zero * inv (each rounded once),
    t = fma(u, A, Bz), clamped to 2^b - 1 when fma(mx, A, Bz) >= 2^b - 1/2,
    then rounded half to even and saturated to [0, 255].  Returns (codes,
    scale, zero, t before the clamp, which groups took the clamp)."""
    assert D == 64, "the model takes rs = 1/8 exactly"
    rs, qmax = 0.125, float(2 ** bits - 1)
    ug = u.reshape(len(u), D // G, G)
    mn, mx = ug.min(-1), ug.max(-1)
    zero = oracle.rd16(_f32(mn * rs))
    zf = zero.astype(np.float64)
    scale = oracle.ru16(_f32(_f32(_f32(mx * rs) - zf) / qmax))
    sf = scale.astype(np.float64)
    inv = np.where(sf > 0, _f32(1.0 / np.where(sf > 0, sf, 1.0)), 0.0)
    A, Bz = _f32(inv * rs), _f32(-zf * inv)
    t = _fma_f32(ug, A[..., None], Bz[..., None])
    clamp = ~(_fma_f32(mx, A, Bz) < qmax + 0.5)
    tq = np.where(clamp[..., None], np.minimum(t, qmax), t)
    q = np.clip(np.rint(tq), 0, 255).astype(np.uint8)
    return q.reshape(u.shape), scale, zero, t.reshape(u.shape), clamp


def _degenerate_rows(D, dtype, bits, G, seed, n, rng, want_hot=16):
    """n degenerate rows, up to want_hot of them with a group whose minimum
    sits just above an fp16 grid point: there the stored zero is that point,
    the scale is tiny, and |y| / scale is large enough that binary32
    decisions can move t by more than one half (band above 1/2).  At
    head_dim 64 those rows are picked where the kernel's decision (modelled
    on binary32-rounded exact sums) takes the clamp."""
    hot, plain = [], []
    s = oracle.sign_vector(seed, D)
    for _ in range(60):
        c = _degenerate_candidates(D, G, dtype, 4096, rng)
        y = oracle.rotate(c, s)
        sc, ze = oracle.group_meta(y, G, bits)
        if D == 64:
            over = kernel_decision_model(_f32(oracle.rotate_raw(c, s)), D, G, bits)[4].any(axis=1)
        else:
            over = (parity.band_fp32(y, ze, sc, G, bits) > 0.5).any(axis=1)
        hot.extend(c[over])
        plain.extend(c[~over][: n])
        if len(hot) >= want_hot:
            break
    hot = hot[:want_hot]
    rows = np.array(hot + plain[: n - len(hot)])
    return rows[rng.permutation(len(rows))]


@pytest.mark.parametrize("D,dtype,bits", [(D, dt, b) for D in (64, 128) for dt in ("bf16", "fp16")
                                          for b in (2, 4, 8)])
def test_degenerate_groups(D, dtype, bits):
    """Huge offset, tiny range.  Here a group's range is comparable with the
    binary32 rounding of its rotated values (within criterion (1), checked
    first), so the meta and codes are judged against the definition applied
    to the GPU's own rotated values: zero = RD16(min y), scale =
    RU16((max y - zero) / (2^b - 1)) within one fp16 ulp, codes the nearest
    level of the GPU's meta under a band derived from binary32 decisions
    (parity.band_fp32), which exceeds one half on some elements, so t can
    leave the code range there.  At head_dim 64 the kernel's own binary32
    decision is also modelled on the GPU's transform output (exact there:
    1/sqrt(64) = 1/8), and codes and meta must equal the model's to the bit,
    including groups where the clamp to 2^b - 1 acts -- so the clamp branch
    runs and keeps every code within its bits.  8-bit contiguous encodes
    rotate with the in-register butterfly, not the matrix cores of
    kvc_debug_rotate: there the GPU's own rotated values are those of the
    butterfly (butterfly_model, held to criterion (1) as well)."""
    rng = np.random.default_rng(17 * D + bits)
    G, seed = 32, 9
    rk = _degenerate_rows(D, dtype, bits, G, seed, 640, rng)
    rv = _degenerate_rows(D, dtype, bits, G, seed, 640, rng)
    n = len(rk)
    x = _tensor(rk, rv, dtype)
    xb = inputs.as_u16(x)
    xg = x.to(DEV)
    y_ref = oracle.rotate(np.concatenate([rk, rv]), oracle.sign_vector(seed, D))
    y_gpu = kvc.debug_rotate(xg, seed=seed).cpu().numpy().astype(np.float64).reshape(-1, D)
    rot = parity.check_rotation(y_gpu, y_ref)
    if bits == 8:
        rs = np.float32(1.0 / np.sqrt(D))
        y_gpu = (butterfly_model(np.concatenate([rk, rv]), seed, D).astype(np.float32) * rs).astype(np.float64)
        rot = max(rot, parity.check_rotation(y_gpu, y_ref))
    total, _ = kvc.encoded_size(1, n, 1, D, bits, bits, G, dtype)
    whole, out = gpu_util.guarded(total, DEV)
    kvc.encode(xg, bits, bits, G, seed=seed, out=out)
    xd = kvc.decode(out, x.shape, dtype, bits, bits, G, seed=seed)
    torch.cuda.synchronize()
    assert gpu_util.canaries_intact(whole)
    blob = out.cpu().numpy()
    scale, zero = oracle.group_meta(y_gpu, G, bits)
    band = parity.band_fp32(y_gpu, zero, scale, G, bits)
    _say("degenerate groups", D, dtype, bits, "rotation worst/allowed %.3f;" % rot,
         "elements with band > 1/2:", int((band > 0.5).sum()))
    lay = oracle.blob_layout(1, n, 1, D, bits, bits, G)
    rep = parity.CodeReport()
    ref = np.zeros((2 * n, D), dtype=np.uint16)
    for kv in (0, 1):
        codes, meta = parity.blob_rows(blob, lay, 0, kv, np.arange(n))
        rows = slice(kv * n, (kv + 1) * n)
        res = parity.check_rows(xb[0, kv, :, 0], dtype, bits, G, seed, codes, meta, band="fp32", y=y_gpu[rows])
        rep.merge(res.report)
        ref[rows] = parity.decode_rows_ref(res, dtype, G, seed)
    rr = parity.check_decode(inputs.as_u16(xd)[0, :, :, 0].reshape(-1, D), ref, dtype, axis_slices=(2,))
    _say("  ", rep, "decode rrms %.3g" % rr)
    if bits == 8:   # the kernel decides 8-bit codes near a tie again in float64: every code is the
        # nearest level of the exact t (the oracle's y, the GPU's meta), up to 1e-5 of a tie
        exact = 0
        for kv in (0, 1):
            codes, meta = parity.blob_rows(blob, lay, 0, kv, np.arange(n))
            rows = slice(kv * n, (kv + 1) * n)
            s_g, z_g = meta[..., 0].view(np.float16), meta[..., 1].view(np.float16)
            t = oracle.code_values(y_ref[rows], s_g, z_g, G)
            q_gpu = oracle.unpack_codes(codes, bits, D)
            q_exp = oracle.nearest_codes(t, bits)
            excess = np.abs(q_gpu - np.clip(t, 0.0, 255.0)) - 0.5
            # both sides hold y to float64 rounding, which |y| / scale magnifies in these groups
            s64 = s_g.astype(np.float64)
            yz = (np.abs(y_ref[rows]).reshape(n, -1, G) + np.abs(z_g.astype(np.float64))[..., None]) \
                / np.where(s64 > 0, s64, 1.0)[..., None]
            band = parity.BOUNDARY + 2.0 ** -50 * yz.reshape(n, D)
            bad = (q_gpu != q_exp) & (excess > band)
            assert not bad.any(), "%d 8-bit codes are not the nearest level of the exact t" % bad.sum()
            exact += int((q_gpu == q_exp).sum())
        _say("   8-bit codes equal to the nearest level of the exact t: %d of %d" % (exact, 2 * n * D))
    if D != 64:
        return
    q_m, s_m, z_m, t_m, clamp = kernel_decision_model(y_gpu * 8.0, D, G, bits)
    clamped = clamp[..., None] & (t_m.reshape(len(y_gpu), -1, G) > 2 ** bits - 0.5)
    _say("   groups taking the clamp: %d, elements past the code range: %d" % (int(clamp.sum()), int(clamped.sum())))
    if bits == 4:   # the searched data reaches the clamp at 4 bits (2-bit codes keep a wider
        # margin, and 8-bit codes saturate in the conversion anyway)
        assert clamped.any(), "the data never takes the clamp"
    for kv in (0, 1):
        codes, meta = parity.blob_rows(blob, lay, 0, kv, np.arange(n))
        rows = slice(kv * n, (kv + 1) * n)
        assert np.array_equal(meta[..., 0], s_m[rows].view(np.uint16)), "scale differs from the model"
        assert np.array_equal(meta[..., 1], z_m[rows].view(np.uint16)), "zero differs from the model"
        if bits < 8:   # 8-bit codes near a tie are decided again in float64 (checked above)
            assert np.array_equal(oracle.unpack_codes(codes, bits, D), q_m[rows]), "codes differ from the model"


@pytest.mark.parametrize("bits,G", [(4, 128), (4, 32), (8, 128), (8, 32)])
def test_boundary_window_large_sample(bits, G):
    """4M codes of 8B-shaped data per case: codes flip only within 1e-5 of a
    boundary, at 8 bits too (t up to 255, where the kernel decides the codes
    near a tie again in float64)."""
    p = presets.preset("llama3_8b_4k").with_(name="window-%d-%d" % (bits, G), layers=1, tokens=2048,
                                              bits_k=bits, bits_v=bits, group=G)
    x = inputs.make_kv(p)
    _say("boundary window", bits, G)
    _, res, rr = _encode_check_multihead(x, p)
    r = res.report
    _say("   %d codes: flips %d (worst excess %.3g, beyond 1e-5: %d), meta groups differing %d; decode rrms %.3g"
         % (r.codes, r.boundary_flips, r.worst_boundary_distance, r.flips_beyond_1e5, r.meta_diff_groups, rr))
    assert r.flips_beyond_1e5 == 0


def _encode_check_multihead(x, p):
    xb = inputs.as_u16(x)
    blob = kvc.encode(x.to(DEV), p.bits_k, p.bits_v, p.group, seed=p.seed)
    xd = kvc.decode(blob, x.shape, p.dtype, p.bits_k, p.bits_v, p.group, seed=p.seed)
    torch.cuda.synchronize()
    res = parity.check_blob(xb, blob.cpu().numpy(), p.dtype, p.bits_k, p.bits_v, p.group, p.seed)
    rr = parity.check_decode(inputs.as_u16(xd), res.reference, p.dtype)
    return blob, res, rr


@pytest.mark.parametrize("D,dtype,name", [(128, "bf16", "llama3_8b_4k"), (128, "bf16", "llama3_70b_16k"),
                                          (64, "fp16", "llama3_8b_4k")])
def test_transform_error_within_the_8bit_bound(D, dtype, name):
    """The 8-bit encode re-decides every code whose binary32 t lies within a
    bound of a tie; the bound's main term takes each of the D - 1 fp32
    additions behind an element of u = H (s * x) to err by at most 2^-23 of
    sum |x_j|.  On the matrix-core transform of real-shaped data (the rotate
    hook runs the encode's own transform, then rounds u / sqrt(D) once more),
    every element's error against the exact float64 rotation stays within
    2 D 2^-24 sum|x_j| / sqrt(D) + 2^-24 |y|."""
    p = presets.preset(name).with_(name="bound-%s-%d" % (name, D), layers=2, tokens=4096, head_dim=D, dtype=dtype)
    x = inputs.make_kv(p)
    xb = inputs.as_u16(x).reshape(-1, D)
    y_gpu = kvc.debug_rotate(x.to(DEV), seed=p.seed).cpu().numpy().astype(np.float64).reshape(-1, D)
    x64 = oracle.storage_to_f64(xb, dtype)
    y_ref = oracle.rotate(x64, oracle.sign_vector(p.seed, D))
    w = 2.0 ** -24
    S = np.abs(x64).sum(axis=1, keepdims=True)
    bound = 2 * D * w * S / np.sqrt(D) + w * np.abs(y_ref)
    err = np.abs(y_gpu - y_ref)
    ratio = float((err / bound).max())
    _say("   %s D=%d %s: %d elements, worst error / bound %.4f" % (name, D, dtype, err.size, ratio))
    assert ratio <= 1.0
