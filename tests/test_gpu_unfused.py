"""GPU parity of the separate-kernel comparator (kvc_encode_unfused /
kvc_decode_unfused): its blob is bit-identical to the fused matrix-core
encode's (the default transform except at 8 bits), its decode agrees with the fused decode within the decode criterion (the two
round in different places: the comparator dequantizes and then runs the
whole inverse transform, the fused decode transforms the integer codes
within their groups first), and both meet the oracle criteria on their own."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import parity
import gpu_util
import kv_cache_compression_kvc_amd as kvc
from kv_cache_compression_kvc_amd import _lib, inputs, presets

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _small(D, dtype, bk, bv, G, L=2, T=37, H=3, seed=7):
    return presets.preset("llama3_8b_4k").with_(
        name="uf-%d-%s-%d%d-%d" % (D, dtype, bk, bv, G), layers=L, tokens=T, kv_heads=H,
        head_dim=D, dtype=dtype, bits_k=bk, bits_v=bv, group=G, seed=seed)


GRID = [(D, dt, bk, bv, G)
        for D in (64, 128) for dt in ("bf16", "fp16")
        for bk, bv in [(2, 2), (4, 4), (8, 8), (4, 2)]
        for G in (32, 64, 128) if G <= D]


def _decodes_agree(dec_a, dec_b):
    """Relative RMS per (layer, K/V) slice within the decode criterion, on the GPU."""
    if dec_a.numel() == 0:
        return
    a = dec_a.double().flatten(2)
    b = dec_b.double().flatten(2)
    num = (a - b).norm(dim=2)
    den = b.norm(dim=2)
    rel = torch.where(den > 0, num / den.clamp_min(1e-300), num)
    assert float(rel.max()) <= parity.DECODE_RRMS, "fused and separate-kernel decodes differ by %.3g" % float(rel.max())


def _both(p, x):
    """(fused blob, unfused blob, fused decode, unfused decode) of x on the GPU."""
    D = p.head_dim
    total, _ = kvc.encoded_size(p.layers, p.tokens, p.kv_heads, D, p.bits_k, p.bits_v, p.group, p.dtype)
    ws_bytes = kvc.unfused_workspace_size(p.layers, p.tokens, p.kv_heads, D, p.bits_k, p.bits_v, p.group, p.dtype)
    ws_whole, ws = gpu_util.guarded(ws_bytes, DEV)
    whole, out_u = gpu_util.guarded(total, DEV)
    # the comparator mirrors the matrix-core encode (its first stage is that
    # transform), which 8-bit encodes take only when asked
    out_f = kvc.encode(x, p.bits_k, p.bits_v, p.group, seed=p.seed, transform="matrix")
    kvc.encode_unfused(x, p.bits_k, p.bits_v, p.group, seed=p.seed, out=out_u, workspace=ws)
    torch.cuda.synchronize()
    assert gpu_util.canaries_intact(whole) and gpu_util.canaries_intact(ws_whole)
    dec_f = kvc.decode(out_f, x.shape, p.dtype, p.bits_k, p.bits_v, p.group, seed=p.seed)
    dec_u = kvc.decode_unfused(out_u, x.shape, p.dtype, p.bits_k, p.bits_v, p.group, seed=p.seed, workspace=ws)
    torch.cuda.synchronize()
    assert gpu_util.canaries_intact(ws_whole)
    return out_f, out_u, dec_f, dec_u


@pytest.mark.parametrize("D,dtype,bk,bv,G", GRID)
def test_unfused_equals_fused_and_oracle(D, dtype, bk, bv, G):
    p = _small(D, dtype, bk, bv, G)
    x = inputs.make_kv(p)
    _say("unfused", p.name)
    out_f, out_u, dec_f, dec_u = _both(p, x.to(DEV))
    assert torch.equal(out_f, out_u), "unfused blob differs from the fused blob"
    _decodes_agree(dec_u, dec_f)
    xb = inputs.as_u16(x)
    res = parity.check_blob(xb, out_u.cpu().numpy(), dtype, bk, bv, G, p.seed)
    parity.check_decode(inputs.as_u16(dec_u), res.reference, dtype)


@pytest.mark.parametrize("L,T,H", [(1, 1, 1), (3, 1, 5), (1, 65, 1), (2, 33, 3), (2, 0, 8), (0, 16, 8)])
def test_unfused_edge_shapes(L, T, H):
    p = _small(128, "bf16", 2, 4, 64, L=L, T=T, H=H)
    x = inputs.make_kv(p).to(DEV)
    _say("unfused edge", L, T, H)
    out_f, out_u, dec_f, dec_u = _both(p, x)
    assert torch.equal(out_f, out_u)
    _decodes_agree(dec_u, dec_f)


def test_unfused_workspace_validation():
    lib = _lib.lib()
    x = torch.zeros((1, 2, 8, 2, 128), dtype=torch.bfloat16, device=DEV)
    need = kvc.unfused_workspace_size(1, 8, 2, 128, 4, 4, 32)
    assert need == 2 * 8 * 2 * 128 * 5          # 4096 code bytes (256-aligned), then fp32
    with pytest.raises(kvc.KvcError, match="KVC_ENOSPC"):
        kvc.encode_unfused(x, 4, 4, 32, workspace=torch.zeros(need - 1, dtype=torch.uint8, device=DEV))
    with pytest.raises(kvc.KvcError, match="KVC_EALIGN"):
        kvc.encode_unfused(x, 4, 4, 32, workspace=torch.zeros(need + 16, dtype=torch.uint8, device=DEV)[4:])
    out = torch.zeros(8192, dtype=torch.uint8, device=DEV)
    d = _lib.KvcDesc(1, 8, 2, 128, 0, 4, 4, 32, 0)
    assert lib.kvc_encode_unfused(ctypes.byref(d), x.data_ptr(), out.data_ptr(), out.numel(), None, 0, None) == -1
    assert lib.kvc_decode_unfused(ctypes.byref(d), out.data_ptr(), out.numel(), x.data_ptr(), None, 0, None) == -1


@pytest.mark.slow
@pytest.mark.parametrize("name", ["llama3_8b_4k", "llama3_8b_32k"])
def test_unfused_full_size_equals_fused(name):
    p = presets.preset(name)
    _say("unfused full size: generate", p.name)
    x = inputs.make_kv(p, device=DEV)
    out_f, out_u, dec_f, dec_u = _both(p, x)
    assert torch.equal(out_f, out_u)
    _decodes_agree(dec_u, dec_f)
    del x, out_f, out_u, dec_f, dec_u
    torch.cuda.empty_cache()


# (head_dim, dtype, bits, group, tokens, heads, line in MiB): blobs past the
# size where the decode takes the butterfly variant (head_dim 64: 192 MiB;
# head_dim 128, 4-bit, G = 128: 512 MiB), whose slabs end in a partial tile
# (rows per slab 2000015 = 15 mod 64, 1000015 = 15)
LARGE_RAGGED = [(128, "bf16", 4, 128, 400003, 5, 512), (64, "fp16", 8, 32, 200003, 5, 192)]


@pytest.mark.slow
@pytest.mark.parametrize("D,dtype,b,G,T,H,line_mib", LARGE_RAGGED)
def test_large_ragged_blob_both_decodes(D, dtype, b, G, T, H, line_mib):
    """A blob past the line (decoded by the butterfly variant, one wave per
    SIMD, stores overlapped) whose slabs end in a partial tile.  Each layer
    encoded on its own gives a blob below the line, decoded by the
    matrix-core variant; the two decodes must agree to the bit, the encode
    must match the separate-kernel comparator's blob, and nothing may be
    written outside the decode output."""
    p = _small(D, dtype, b, b, G, L=2, T=T, H=H)
    _say("large ragged: generate", D, dtype)
    x = inputs.make_kv(p, device=DEV)
    total, _ = kvc.encoded_size(p.layers, p.tokens, p.kv_heads, D, b, b, G, dtype)
    assert total > line_mib << 20
    out_f, out_u, dec_f, dec_u = _both(p, x)
    assert torch.equal(out_f, out_u)
    _decodes_agree(dec_u, dec_f)
    dwhole, draw = gpu_util.guarded(x.numel() * 2, DEV)
    xd = draw.view(x.dtype).view(x.shape)
    kvc.decode(out_f, x.shape, dtype, b, b, G, seed=p.seed, out=xd)
    torch.cuda.synchronize()
    assert gpu_util.canaries_intact(dwhole)
    assert torch.equal(xd.view(torch.int16), dec_f.view(torch.int16))
    for l in range(p.layers):
        xl = x[l:l + 1].contiguous()
        tl, _ = kvc.encoded_size(1, p.tokens, p.kv_heads, D, b, b, G, dtype)
        assert tl < line_mib << 20
        bl = kvc.encode(xl, b, b, G, seed=p.seed, transform="matrix")
        dl = kvc.decode(bl, xl.shape, dtype, b, b, G, seed=p.seed)
        torch.cuda.synchronize()
        _say("  layer %d: per-layer decode vs whole decode" % l)
        assert torch.equal(dl.view(torch.int16), dec_f[l:l + 1].view(torch.int16))
    del x, out_f, out_u, dec_f, dec_u, dwhole, draw, xd
    torch.cuda.empty_cache()
