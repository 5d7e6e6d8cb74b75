"""The parity checker itself, on the CPU: blobs written by the oracle stand in
for GPU output, with mistakes planted on the CPU side."""
import numpy as np
import pytest

import oracle
import parity
from kv_cache_compression_kvc_amd import inputs, presets


def _case(bits=4, G=64, T=512):
    p = presets.preset("llama3_8b_4k").with_(name="parity-rules", layers=1, tokens=T, kv_heads=8,
                                              bits_k=bits, bits_v=bits, group=G, seed=3)
    xb = inputs.as_u16(inputs.make_kv(p))
    blob, tr = oracle.encode(xb, p.dtype, bits, bits, G, p.seed)
    return p, xb, blob, tr


def _code_byte(lay, l, kv, row, elem, bits, D):
    """Byte offset in the blob of code `elem` of `row`, and its bit shift."""
    per_byte = 8 // bits
    off = lay.codes_slab(l, kv) + oracle.code_offsets([row], lay.rows, lay.row_bytes(kv))[0][elem // per_byte]
    return off, bits * (elem % per_byte)


def test_oracle_blob_passes_with_nothing_counted():
    p, xb, blob, _ = _case()
    res = parity.check_blob(xb, blob, p.dtype, p.bits_k, p.bits_v, p.group, p.seed)
    r = res.report
    assert r.boundary_flips == 0 and r.code_mismatches == 0 and r.meta_diff_groups == 0
    assert np.array_equal(res.blob, blob)
    ref, _ = oracle.decode(blob, xb.shape, p.dtype, p.bits_k, p.bits_v, p.group, p.seed)
    assert np.array_equal(res.reference, ref)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_flip_near_a_boundary_is_counted_far_one_fails(bits):
    p, xb, blob, tr = _case(bits=bits)
    D = p.head_dim
    lay = oracle.blob_layout(1, p.tokens, p.kv_heads, D, bits, bits, p.group)
    t = tr.t[0, 0].reshape(-1, D)
    dist = np.abs(t - (np.floor(t) + 0.5))
    # the element nearest to a boundary (well inside 1e-5 on this many codes)
    row, elem = np.unravel_index(np.argmin(dist), dist.shape)
    assert dist[row, elem] < 1e-5
    q = int(tr.q[0, 0].reshape(-1, D)[row, elem])
    other = q + 1 if t[row, elem] > q else q - 1
    off, sh = _code_byte(lay, 0, 0, row, elem, bits, D)
    near = blob.copy()
    near[off] = (near[off] & ~(((1 << bits) - 1) << sh)) | (other << sh)
    res = parity.check_blob(xb, near, p.dtype, bits, bits, p.group, p.seed)
    assert res.report.boundary_flips == 1 and res.report.worst_boundary_distance < 1e-5
    assert np.array_equal(res.blob, near)        # the flip is substituted into the reference
    # an element far from any boundary: the same kind of change must fail
    row, elem = np.unravel_index(np.argmax(np.where((t > 1) & (t < 2 ** bits - 2), dist, 0)), dist.shape)
    assert dist[row, elem] > 0.05
    q = int(tr.q[0, 0].reshape(-1, D)[row, elem])
    off, sh = _code_byte(lay, 0, 0, row, elem, bits, D)
    far = blob.copy()
    far[off] = (far[off] & ~(((1 << bits) - 1) << sh)) | ((q + 1) << sh)
    with pytest.raises(AssertionError, match="away from a rounding boundary"):
        parity.check_blob(xb, far, p.dtype, bits, bits, p.group, p.seed)


def test_meta_one_ulp_accepted_two_ulps_fail():
    p, xb, blob, tr = _case()
    D, G = p.head_dim, p.group
    lay = oracle.blob_layout(1, p.tokens, p.kv_heads, D, p.bits_k, p.bits_v, G)
    m0 = lay.meta_slab(0, 1)
    for step, ok in ((1, True), (2, False)):
        b = blob.copy()
        meta = b[m0:m0 + 4].view("<u2")
        meta[0] += step                          # scale of group 0 of row 0 of V, step ulps up
        # the codes of that group re-quantized with the changed meta
        y = tr.y[0, 1].reshape(-1, D)[:1, :G]
        s = meta[:1].view(np.float16).reshape(1, 1)
        z = meta[1:2].view(np.float16).reshape(1, 1)
        q, _ = oracle.quantize(y, s, z, G, p.bits_v)
        row = tr.q[0, 1].reshape(-1, D)[:1].copy()
        row[0, :G] = q[0]
        packed = oracle.pack_codes(row, p.bits_v)[0]
        offs = lay.codes_slab(0, 1) + oracle.code_offsets([0], lay.rows, lay.row_bytes(1))[0]
        b[offs] = packed
        if ok:
            res = parity.check_blob(xb, b, p.dtype, p.bits_k, p.bits_v, G, p.seed)
            assert res.report.meta_diff_groups == 1
            assert np.array_equal(res.blob, b)
        else:
            with pytest.raises(AssertionError, match="meta differs"):
                parity.check_blob(xb, b, p.dtype, p.bits_k, p.bits_v, G, p.seed)


def test_decode_rule_per_slice():
    p, xb, blob, _ = _case()
    ref, _ = oracle.decode(blob, xb.shape, p.dtype, p.bits_k, p.bits_v, p.group, p.seed)
    assert parity.check_decode(ref, ref, p.dtype) == 0.0
    x = oracle.storage_to_f64(ref, p.dtype)
    noisy = oracle.f64_to_storage(x * (1 + 3e-3), p.dtype)
    with pytest.raises(AssertionError, match="relative RMS"):
        parity.check_decode(noisy, ref, p.dtype)


def test_zero_one_ulp_down_takes_the_scale_of_that_zero():
    """A tiny-range group far from 0: with the zero one fp16 step lower, the
    scale that belongs to it is many fp16 steps larger; it is accepted, an
    unrelated scale is not."""
    D, G, bits = 64, 32, 4
    x = np.zeros((1, 2, 1, 1, D))
    x[0, :, 0, 0, 0] = 1000.0
    x[0, :, 0, 0, 5] = 2.0 ** -10
    xb = oracle.f64_to_storage(x, "fp16")
    blob, tr = oracle.encode(xb, "fp16", bits, bits, G, 0)
    lay = oracle.blob_layout(1, 1, 1, D, bits, bits, G)
    y = tr.y[0, 0, 0, 0]
    m0 = lay.meta_slab(0, 0)
    z = tr.zero[0, 0, 0, 0, 0]
    z_dn = np.nextafter(z, np.float16(-np.inf))
    s_dn = oracle.ru16((y[:G].max() - float(z_dn)) / (2 ** bits - 1))
    assert abs(int(s_dn.view(np.uint16)) - int(tr.scale[0, 0, 0, 0, 0].view(np.uint16))) > 1
    for s_new, ok in ((s_dn, True), (np.float16(float(s_dn) * 3), False)):
        b = blob.copy()
        meta = b[m0:m0 + 4].view("<u2")
        meta[0] = np.asarray(s_new, dtype=np.float16).view(np.uint16)
        meta[1] = z_dn.view(np.uint16)
        q, _ = oracle.quantize(y[None, :G], np.array([[s_new]], dtype=np.float16),
                               np.array([[z_dn]], dtype=np.float16), G, bits)
        row = tr.q[0, 0, 0, 0].copy()
        row[:G] = q[0]
        offs = lay.codes_slab(0, 0) + oracle.code_offsets([0], 1, lay.row_bytes(0))[0]
        b[offs] = oracle.pack_codes(row[None], bits)[0]
        if ok:
            assert parity.check_blob(xb, b, "fp16", bits, bits, G, 0).report.meta_diff_groups == 1
        else:
            with pytest.raises(AssertionError, match="meta differs"):
                parity.check_blob(xb, b, "fp16", bits, bits, G, 0)
