"""The no-allocation encode entry point against the existing one: the
separate-kernel encode with its workspace in the library's static device
array must write the same blob, bit for bit, as the same encode with a
caller-owned workspace -- on two calls in a row, the second smaller, so the
array is reused with the first call's contents still in it."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import parity
import kv_cache_compression_kvc_amd as kvc
from kv_cache_compression_kvc_amd import _lib, inputs, presets

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _noalloc(x, p, out):
    """kvc_encode_unfused_noalloc straight through the C ABI."""
    L, _, T, H, D = x.shape
    d = _lib.KvcDesc(L, T, H, D, _lib.DTYPE[p.dtype], p.bits_k, p.bits_v, p.group, p.seed)
    st = _lib.lib().kvc_encode_unfused_noalloc(ctypes.byref(d), ctypes.c_void_p(x.data_ptr()),
                                               ctypes.c_void_p(out.data_ptr()), out.numel(),
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def _reference(x, p):
    """The same encode through kvc_encode_unfused with a caller-owned workspace."""
    return kvc.encode_unfused(x, p.bits_k, p.bits_v, p.group, seed=p.seed)


CALLS = [  # (layers, tokens, heads, head_dim, dtype, bits_k, bits_v, group): large, then smaller
    [(4, 1000, 8, 128, "bf16", 4, 2, 64), (1, 37, 3, 128, "bf16", 4, 2, 64)],
    [(2, 2048, 8, 64, "fp16", 8, 8, 32), (1, 65, 2, 64, "fp16", 2, 4, 64)],
]


@pytest.mark.parametrize("calls", CALLS)
def test_noalloc_equals_workspace_encode_twice(calls):
    for k, (L, T, H, D, dt, bk, bv, G) in enumerate(calls):
        p = presets.preset("llama3_8b_4k").with_(name="noalloc-%d" % k, layers=L, tokens=T, kv_heads=H,
                                                  head_dim=D, dtype=dt, bits_k=bk, bits_v=bv, group=G, seed=7 + k)
        x = inputs.make_kv(p, device=DEV)
        need = kvc.unfused_workspace_size(L, T, H, D, bk, bv, G, dt)
        assert need <= _lib.NOALLOC_WORKSPACE_BYTES
        total, _ = kvc.encoded_size(L, T, H, D, bk, bv, G, dt)
        _say("noalloc call", k, (L, T, H, D, dt, bk, bv, G), "workspace", need)
        out = torch.full((total,), 0xA5, dtype=torch.uint8, device=DEV)
        assert _noalloc(x, p, out) == 0
        ref = _reference(x, p)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "no-allocation blob differs from the workspace encode"
        # and the blob is the method's: criteria (2) and (3) against the oracle
        if k == len(calls) - 1:
            parity.check_blob(inputs.as_u16(x), out.cpu().numpy(), dt, bk, bv, G, p.seed)


def test_noalloc_refuses_a_shape_past_its_array():
    # 2 x 6.8M elements: 5 bytes each is more than the static workspace
    L, T, H, D = 1, 26624, 2, 128
    need = kvc.unfused_workspace_size(L, T, H, D, 4, 4, 64, "bf16")
    assert need > _lib.NOALLOC_WORKSPACE_BYTES
    p = presets.preset("llama3_8b_4k").with_(name="noalloc-big", layers=L, tokens=T, kv_heads=H,
                                              head_dim=D, bits_k=4, bits_v=4, group=64)
    x = torch.zeros((L, 2, T, H, D), dtype=torch.bfloat16, device=DEV)
    total, _ = kvc.encoded_size(L, T, H, D, 4, 4, 64, "bf16")
    out = torch.zeros(total, dtype=torch.uint8, device=DEV)
    assert _noalloc(x, p, out) == -7          # KVC_ENOSPC, nothing enqueued
    torch.cuda.synchronize()
    assert not out.any()
    with pytest.raises(kvc.KvcError, match="KVC_ENOSPC"):
        kvc.encode_unfused_noalloc(x, 4, 4, 64, out=out)
