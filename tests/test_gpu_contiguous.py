"""GPU parity of the contiguous encode / decode against the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
import parity
import gpu_util
import kv_cache_compression_kvc_amd as kvc
from kv_cache_compression_kvc_amd import inputs, presets

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _small(D, dtype, bk, bv, G, L=2, T=37, H=3, seed=11):
    return presets.preset("llama3_8b_4k").with_(
        name="small-%d-%s-%d%d-%d" % (D, dtype, bk, bv, G), layers=L, tokens=T, kv_heads=H,
        head_dim=D, dtype=dtype, bits_k=bk, bits_v=bv, group=G, seed=seed)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


GRID = [(D, dt, bk, bv, G)
        for D in (64, 128) for dt in ("bf16", "fp16")
        for bk, bv in [(2, 2), (4, 4), (8, 8), (2, 4), (4, 8)]
        for G in (32, 64, 128) if G <= D]


@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (64, "fp16"), (128, "bf16"), (128, "fp16")])
def test_rotation_matches_oracle(D, dtype):
    p = _small(D, dtype, 4, 4, 32, T=53)
    x = inputs.make_kv(p)
    _say("rotate", D, dtype)
    y = kvc.debug_rotate(x.to(DEV), seed=p.seed).cpu().numpy()
    yref = oracle.rotate(oracle.storage_to_f64(inputs.as_u16(x), dtype), oracle.sign_vector(p.seed, D))
    parity.check_rotation(y, yref)


@pytest.mark.parametrize("D,dtype,bk,bv,G", GRID)
def test_encode_decode_small(D, dtype, bk, bv, G):
    p = _small(D, dtype, bk, bv, G)
    x = inputs.make_kv(p)
    xb = inputs.as_u16(x)
    total, _ = kvc.encoded_size(p.layers, p.tokens, p.kv_heads, D, bk, bv, G, dtype)
    whole, out = gpu_util.guarded(total, DEV)
    _say("encode", p.name)
    kvc.encode(x.to(DEV), bk, bv, G, seed=p.seed, out=out)
    torch.cuda.synchronize()
    assert gpu_util.canaries_intact(whole)
    blob = out.cpu().numpy()
    res = parity.check_blob(xb, blob, dtype, bk, bv, G, p.seed)
    _say("  codes vs oracle:", res.report)
    # decode of the GPU blob, checked against the oracle's decode of its own
    # encode (criterion 4, the allowed differences substituted) and of the
    # GPU's blob (decoupled from the encode)
    _say("decode", p.name)
    dwhole, draw = gpu_util.guarded(x.numel() * 2, DEV)
    xd = draw.view(x.dtype).view(x.shape)
    kvc.decode(out, x.shape, dtype, bk, bv, G, seed=p.seed, out=xd)
    torch.cuda.synchronize()
    assert gpu_util.canaries_intact(dwhole), "decode wrote outside its output"
    xd_b = inputs.as_u16(xd)
    parity.check_decode(xd_b, res.reference, dtype)
    ref_same, _ = oracle.decode(blob, x.shape, dtype, bk, bv, G, p.seed)
    parity.check_decode(xd_b, ref_same, dtype)
    oblob, _ = oracle.encode(xb, dtype, bk, bv, G, p.seed)
    ref_own, _ = oracle.decode(oblob, x.shape, dtype, bk, bv, G, p.seed)
    # GPU decode of the oracle's blob
    xo = kvc.decode(torch.from_numpy(oblob).to(DEV), x.shape, dtype, bk, bv, G, seed=p.seed)
    parity.check_decode(inputs.as_u16(xo), ref_own, dtype)


def test_tiny_workload_all_criteria():
    p = presets.preset("tiny")
    x = inputs.make_kv(p)
    xb = inputs.as_u16(x)
    xg = x.to(DEV)
    _say("tiny: rotate / encode / decode")
    y = kvc.debug_rotate(xg, seed=p.seed).cpu().numpy()
    yref = oracle.rotate(oracle.storage_to_f64(xb, p.dtype), oracle.sign_vector(p.seed, p.head_dim))
    worst = parity.check_rotation(y, yref)
    blob = kvc.encode(xg, p.bits_k, p.bits_v, p.group, seed=p.seed)
    res = parity.check_blob(xb, blob.cpu().numpy(), p.dtype, p.bits_k, p.bits_v, p.group, p.seed)
    xd = kvc.decode(blob, x.shape, p.dtype, p.bits_k, p.bits_v, p.group, seed=p.seed)
    rr = parity.check_decode(inputs.as_u16(xd), res.reference, p.dtype)
    # the oracle's own decode, nothing substituted: over the whole tensor
    oblob, _ = oracle.encode(xb, p.dtype, p.bits_k, p.bits_v, p.group, p.seed)
    ref, _ = oracle.decode(oblob, x.shape, p.dtype, p.bits_k, p.bits_v, p.group, p.seed)
    r_all = parity.check_decode(inputs.as_u16(xd), ref, p.dtype, axis_slices=(1,))
    _say("  rotation worst/allowed %.3g; %s; decode rrms %.3g (unsubstituted %.3g)" % (worst, res.report, rr, r_all))


@pytest.mark.parametrize("L,T,H", [(1, 1, 1), (1, 64, 1), (3, 1, 5), (1, 65, 1), (2, 0, 8), (0, 16, 8)])
def test_edge_shapes(L, T, H):
    p = _small(128, "bf16", 4, 2, 64, L=L, T=T, H=H)
    x = inputs.make_kv(p).to(DEV)
    _say("edge", L, T, H)
    blob = kvc.encode(x, 4, 2, 64, seed=p.seed)
    dwhole, draw = gpu_util.guarded(x.numel() * 2, DEV)
    xd = draw.view(x.dtype).view(x.shape)
    kvc.decode(blob, x.shape, "bf16", 4, 2, 64, seed=p.seed, out=xd)
    torch.cuda.synchronize()
    assert gpu_util.canaries_intact(dwhole), "decode wrote outside its output"
    if x.numel() == 0:
        assert blob.numel() == 0 or not blob.cpu().numpy().any()
        return
    xb = inputs.as_u16(x)
    res = parity.check_blob(xb, blob.cpu().numpy(), "bf16", 4, 2, 64, p.seed)
    parity.check_decode(inputs.as_u16(xd), res.reference, "bf16")


def test_host_validation_rejects_before_launch():
    x = torch.zeros((1, 2, 4, 1, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(kvc.KvcError, match="KVC_EBITS"):
        kvc.encode(x, 3, 4, 32)
    with pytest.raises(kvc.KvcError, match="KVC_EGROUP"):
        kvc.encode(x, 4, 4, 48)
    small = torch.zeros(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(kvc.KvcError, match="KVC_ENOSPC"):
        kvc.encode(x, 4, 4, 32, out=small)
    mis = torch.zeros(4096 + 8, dtype=torch.uint8, device=DEV)[8:]
    with pytest.raises(kvc.KvcError, match="KVC_EALIGN"):
        kvc.encode(x, 4, 4, 32, out=mis)
    x64 = torch.zeros((1, 2, 4, 1, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(kvc.KvcError, match="KVC_ESHAPE"):
        kvc.encode(x64, 4, 4, 32)


def test_side_stream_and_seeds():
    p = _small(128, "bf16", 4, 4, 128, T=40, H=2, seed=2 ** 64 - 1)
    x = inputs.make_kv(p)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        xg = x.to(DEV, non_blocking=False)
        blob = kvc.encode(xg, 4, 4, 128, seed=p.seed, stream=s)
    s.synchronize()
    parity.check_blob(inputs.as_u16(x), blob.cpu().numpy(), "bf16", 4, 4, 128, p.seed)


def test_probe_stream_stays_in_bounds():
    """The same-mix yardstick reads and writes only the sizes it is given, at
    any ratio, with any grid."""
    src = torch.randint(0, 255, (1 << 22,), dtype=torch.uint8, device=DEV)
    for rb, wb, wpc in ((1 << 22, 1 << 20, 4), (1 << 20, 1 << 22, 8), (1 << 22, 0, 16), (0, 1 << 21, 8),
                        (1024 * 37, 1024 * 5, 1), (1024 * 5, 1024 * 37, 32)):
        whole, dst = gpu_util.guarded(max(wb, 1024) + 4096, DEV)
        dst.fill_(0x5A)
        kvc.probe_stream(src, rb, dst, wb, waves_per_cu=wpc)
        torch.cuda.synchronize()
        assert gpu_util.canaries_intact(whole), (rb, wb)
        assert bool((dst[wb:] == 0x5A).all()), (rb, wb)
    with pytest.raises(kvc.KvcError, match="KVC_EALIGN"):
        kvc.probe_stream(src, 1000, src, 0)
    with pytest.raises(kvc.KvcError, match="KVC_EINVAL"):
        kvc.probe_stream(src, 1024, src, 0, waves_per_cu=33)


def test_probe_stream_runs_stays_in_bounds():
    """The run-at-once yardstick reads and writes only the sizes it is given,
    at any ratio and run length, including a last partial run, with any grid."""
    src = torch.randint(0, 255, (1 << 22,), dtype=torch.uint8, device=DEV)
    for rb, wb, run, wpc in ((1 << 22, 1 << 20, 16, 4), (1 << 20, 1 << 22, 16, 8), (1 << 22, 0, 16, 2),
                             (0, 1 << 21, 8, 8), (1024 * 37, 1024 * 5, 16, 1), (1024 * 5, 1024 * 37, 16, 32),
                             (1024 * 37, 1024 * 37, 4, 3), (1024 * 3, 1024 * 2, 16, 4)):
        whole, dst = gpu_util.guarded(max(wb, 1024) + 4096, DEV)
        dst.fill_(0x5A)
        kvc.probe_stream_runs(src, rb, dst, wb, run_kib=run, waves_per_cu=wpc)
        torch.cuda.synchronize()
        assert gpu_util.canaries_intact(whole), (rb, wb, run)
        assert bool((dst[wb:] == 0x5A).all()), (rb, wb, run)
        if wb:
            assert not bool((dst[:wb] == 0x5A).all()), (rb, wb, run)
    with pytest.raises(kvc.KvcError, match="KVC_EALIGN"):
        kvc.probe_stream_runs(src, 1000, src, 0)
    with pytest.raises(kvc.KvcError, match="KVC_EINVAL"):
        kvc.probe_stream_runs(src, 1024, src, 0, run_kib=5)
    with pytest.raises(kvc.KvcError, match="KVC_EINVAL"):
        kvc.probe_stream_runs(src, 1024, src, 0, waves_per_cu=0)


def test_probe_blocks_stays_in_bounds():
    """The block gather / scatter yardstick touches only the listed blocks
    (entries outside the region are skipped) and the first stream_bytes of
    its stream, in both directions."""
    bb, nblk = 4096, 12
    region_whole, region = gpu_util.guarded(bb * nblk, DEV)
    seq_whole, seq = gpu_util.guarded(64 * 1024 + 4096, DEV)
    blocks = torch.tensor([3, 0, 11, -1, 7, 12, 3, 100000], dtype=torch.int32, device=DEV)
    listed = {0, 3, 7, 11}
    for scatter in (0, 1):
        region.fill_(0x5A)
        seq.fill_(0x5A)
        kvc.probe_blocks(region, bb, blocks, seq, 64 * 1024, scatter, waves_per_cu=2)
        torch.cuda.synchronize()
        assert gpu_util.canaries_intact(region_whole) and gpu_util.canaries_intact(seq_whole), scatter
        r = region.view(nblk, bb).cpu()
        for b in range(nblk):
            untouched = bool((r[b] == 0x5A).all())
            assert untouched == (not scatter or b not in listed), (scatter, b)
        assert bool((seq[64 * 1024:] == 0x5A).all())
        if not scatter:
            assert not bool((seq[:64 * 1024] == 0x5A).all())
    with pytest.raises(kvc.KvcError, match="KVC_EALIGN"):
        kvc.probe_blocks(region, 1000, blocks, seq, 1024, 0)
    with pytest.raises(kvc.KvcError, match="KVC_EINVAL"):
        kvc.probe_blocks(region, bb, blocks, seq, 1024, 2)


def test_probe_copy():
    a = torch.randint(0, 255, (1 << 24,), dtype=torch.uint8, device=DEV)
    b = torch.zeros_like(a)
    kvc.probe_copy(a, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# full-size workloads: the presets, the 8B-4k byte count at head_dim 64 in
# fp16, and a 70B-shaped cache whose blob is larger than 4 GiB
FULL = {
    "llama3_8b_4k": ("llama3_8b_4k", {}),
    "llama3_8b_32k": ("llama3_8b_32k", {}),
    "llama3_70b_16k": ("llama3_70b_16k", {}),
    "llama3_8b_4k_d64_fp16": ("llama3_8b_4k", dict(head_dim=64, tokens=8192, group=64, dtype="fp16")),
    # a blob past 4 GiB (6.6 GB of 8-bit codes): 64-bit code and meta offsets
    "llama3_70b_40k_8bit": ("llama3_70b_16k", dict(tokens=40000, bits_k=8, bits_v=8)),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled(name):
    base, over = FULL[name]
    p = presets.preset(base).with_(name=name, **over)
    rng = np.random.default_rng(7)
    _say("full size", name, "generate")
    x = inputs.make_kv(p, device=DEV)
    total, _ = kvc.encoded_size(p.layers, p.tokens, p.kv_heads, p.head_dim, p.bits_k, p.bits_v,
                                p.group, p.dtype)
    whole, out = gpu_util.guarded(total, DEV)
    _say("full size", name, "encode")
    kvc.encode(x, p.bits_k, p.bits_v, p.group, seed=p.seed, out=out)
    torch.cuda.synchronize()
    assert gpu_util.canaries_intact(whole)
    idx = gpu_util.sample_vectors(p, rng)
    # criterion (1) on the sampled vectors of the full-size transform
    D = p.head_dim
    _say("full size", name, "rotate")
    y = kvc.debug_rotate(x, seed=p.seed)
    gi = torch.from_numpy(idx).to(DEV)
    ys = y.view(-1, D)[gi].cpu().numpy()
    del y
    torch.cuda.empty_cache()
    xs = inputs.as_u16(x.view(-1, D)[gi])
    yref = oracle.rotate(oracle.storage_to_f64(xs, p.dtype), oracle.sign_vector(p.seed, D))
    _say("  sampled rotation worst/allowed: %.3f over %d vectors" % (parity.check_rotation(ys, yref), len(idx)))
    rep, reference = gpu_util.check_sampled_encode(p, x, out, idx)
    _say("  sampled codes vs oracle:", rep)
    _say("full size", name, "decode")
    xd = kvc.decode(out, x.shape, p.dtype, p.bits_k, p.bits_v, p.group, seed=p.seed)
    torch.cuda.synchronize()
    ratio = gpu_util.decode_error_bound_ok(p, x, xd, out)
    _say("  worst ||x - xhat|| / bound over all vectors: %.4f" % ratio)
    assert ratio <= 1.0
    # criterion (4) on the sampled vectors: the GPU decode against the oracle's
    # decode of its own encode (allowed differences substituted)
    got_all = inputs.as_u16(xd.view(-1, D)[torch.from_numpy(idx).to(DEV)])
    rr = parity.check_decode(got_all, reference, p.dtype, axis_slices=(1,))
    _say("  sampled decode vs the oracle's decode: rrms %.3g over %d vectors" % (rr, len(idx)))
    # and against the oracle's decode of the GPU's codes (decoupled from the encode)
    rows = p.tokens * p.kv_heads
    lay = oracle.blob_layout(p.layers, p.tokens, p.kv_heads, D, p.bits_k, p.bits_v, p.group)
    sub = idx[:400]
    got = inputs.as_u16(xd.view(-1, D)[torch.from_numpy(sub).to(DEV)])
    refs = []
    for v in sub:
        s, r = divmod(int(v), rows)
        l, kv = divmod(s, 2)
        b = p.bits_k if kv == 0 else p.bits_v
        ci = lay.codes_slab(l, kv) + oracle.code_offsets([r], rows, lay.row_bytes(kv))[0]
        m0 = lay.meta_slab(l, kv) + r * lay.groups * 4
        codes = out[torch.from_numpy(ci).to(out.device)].cpu().numpy()
        meta = out[m0:m0 + lay.groups * 4].cpu().numpy().view("<u2").reshape(lay.groups, 2)
        q = oracle.unpack_codes(codes[None], b, D)
        yhat = oracle.dequantize(q, meta[None, :, 0].view(np.float16), meta[None, :, 1].view(np.float16), p.group)
        refs.append(oracle.f64_to_storage(oracle.unrotate(yhat, oracle.sign_vector(p.seed, D)), p.dtype)[0])
    parity.check_decode(got, np.stack(refs), p.dtype, axis_slices=(1,))
    del x, xd, whole, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_subnormal_and_tiny_inputs(dtype):
    """Subnormal storage values go through the matrix-core transform exactly like
    ordinary ones (criterion 1 on rows made only of them), and encode to valid blobs."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    g = torch.Generator().manual_seed(0)
    tiny = torch.finfo(tdt).tiny
    x = torch.zeros(1, 2, 64, 1, 128, dtype=tdt)
    x[0, 0, :32] = (torch.randn(32, 1, 128, generator=g) * tiny * 0.25).to(tdt)
    x[0, 0, 32:] = (torch.randn(32, 1, 128, generator=g) * tiny * 4).to(tdt)
    x[0, 1] = torch.randn(64, 1, 128, generator=g).to(tdt)
    xb = inputs.as_u16(x)
    _say("subnormal inputs", dtype)
    y = kvc.debug_rotate(x.to(DEV), seed=1).cpu().numpy()
    yref = oracle.rotate(oracle.storage_to_f64(xb, dtype), oracle.sign_vector(1, 128))
    parity.check_rotation(y, yref)
    blob = kvc.encode(x.to(DEV), 4, 4, 128, seed=1)
    parity.check_blob(xb, blob.cpu().numpy(), dtype, 4, 4, 128, 1)


def _tokens_for(D, bk, bv, G, H, target):
    """Tokens giving a one-layer blob of about `target` bytes, 3 past a multiple of 64."""
    per_token = H * (D * bk // 8 + D * bv // 8 + 8 * D // G)
    return (target // per_token) // 64 * 64 + 3


# Where the contiguous decode takes the butterfly variant (kDecodeLarge): at
# head_dim 64 past 192 MiB of blob, at head_dim 128 for 4-bit codes with
# G = 128 past 512 MiB.  Every such (head_dim, bits, group), plus K 2-bit /
# V 4-bit at G = 128, where only the V launch takes the butterfly.
# (head_dim, bits_k, bits_v, group, MiB of one layer's blob, line in MiB)
LARGE_GRID = [(64, b, b, G, 120, 192) for b in (2, 4, 8) for G in (32, 64)]
LARGE_GRID += [(128, 4, 4, 128, 300, 512), (128, 2, 4, 128, 300, 512)]
# from 384 MiB of blob the matrix-core decode runs three waves per CU instead
# of one per SIMD: a two-layer blob past that line against each layer alone
LARGE_GRID += [(128, 2, 2, 32, 250, 384), (128, 8, 4, 64, 250, 384)]


@pytest.mark.slow
@pytest.mark.parametrize("D,bk,bv,G,layer_mib,line_mib", LARGE_GRID)
def test_large_blob_decode_matches_per_layer(D, bk, bv, G, layer_mib, line_mib):
    """Two layers whose blob is past the line decode with another launch
    shape (the butterfly variant at one wave per SIMD, or the matrix cores at
    three waves per CU); each layer alone, below the line, decodes on the
    matrix cores at one wave per SIMD.  Both must give the same bits; the
    slabs end in a partial tile (8 heads, tokens 3 past a multiple of 64)."""
    dtype = "bf16" if G != 64 else "fp16"
    T = _tokens_for(D, bk, bv, G, 8, layer_mib << 20)
    p = _small(D, dtype, bk, bv, G, L=2, T=T, H=8)
    _say("large blob", D, bk, bv, G, dtype, T)
    x = inputs.make_kv(p, device=DEV)
    total, _ = kvc.encoded_size(2, T, 8, D, bk, bv, G, dtype)
    one, _ = kvc.encoded_size(1, T, 8, D, bk, bv, G, dtype)
    assert total > line_mib << 20 and one < line_mib << 20
    xd = kvc.decode(kvc.encode(x, bk, bv, G, seed=p.seed), x.shape, dtype, bk, bv, G, seed=p.seed)
    for l in range(2):
        xl = x[l:l + 1].contiguous()
        dl = kvc.decode(kvc.encode(xl, bk, bv, G, seed=p.seed), xl.shape, dtype, bk, bv, G, seed=p.seed)
        assert torch.equal(dl.view(torch.int16), xd[l:l + 1].view(torch.int16)), "layer %d" % l
    torch.cuda.synchronize()
    del x, xd
    torch.cuda.empty_cache()
