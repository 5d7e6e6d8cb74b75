"""Fused KV-cache encode / decode for AMD MI355X (gfx950).

Python face of the C ABI in ``include/kvc.h``: every function here only
marshals torch tensors (device memory) and the current torch stream into a
call of ``libkvc.so``; all of the encode / decode runs in the HIP kernels.
There is no CPU fallback: the calls raise if the library is not built.

Encode (per head_dim vector of a [layers, 2, tokens, kv_heads, head_dim]
bf16 / fp16 tensor): seeded +/-1 sign flip, orthonormal Walsh-Hadamard
transform, per-group fp16 min/max meta, round-half-even 2/4/8-bit codes,
LSB-first packing -- the randomized Hadamard transform and low-bit
quantization stages that the episode notes of "FastKVComp: checking
whether high-throughput KV compression pays off" describe, fused in one
pass as the abstract of "Beyond Compression Ratio: High-Throughput KV
Compression for Disaggregated LLM Serving" states.  Decode is the inverse.
"""

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import KvcDesc, KvcPaged, KvcError, DTYPE

__all__ = [
    "KvcError", "DTYPE", "abi_version", "encoded_size", "sign_mask", "encode", "decode",
    "paged_layout", "paged_order", "encode_paged", "decode_paged", "debug_rotate", "probe_copy", "probe_stream", "probe_stream_runs", "probe_blocks",
    "unfused_workspace_size", "encode_unfused", "decode_unfused", "encode_unfused_noalloc",
    "chunked_size", "encode_send", "receive_decode",
]

_TORCH_TO_NAME = {torch.bfloat16: "bf16", torch.float16: "fp16"}
_NAME_TO_TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _desc(layers, tokens, kv_heads, head_dim, dtype, bits_k, bits_v, group, seed=0):
    return KvcDesc(int(layers), int(tokens), int(kv_heads), int(head_dim), DTYPE[dtype],
                   int(bits_k), int(bits_v), int(group), int(seed) & ((1 << 64) - 1))


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else ctypes.c_void_p(0)


def _nbytes(t):
    return t.numel() * t.element_size()


def _dtype_name(t):
    if t.dtype not in _TORCH_TO_NAME:
        raise ValueError("KV tensors must be bfloat16 or float16, not %s" % t.dtype)
    return _TORCH_TO_NAME[t.dtype]


def _torch_dtype(name):
    if name not in _NAME_TO_TORCH:
        raise ValueError("dtype must be 'bf16' or 'fp16', not %r" % (name,))
    return _NAME_TO_TORCH[name]


def _kv_shape(shape, what):
    """(L, T, H, D) of a [L, 2, T, H, D] shape; axis 1 holds K and V."""
    shape = tuple(int(n) for n in shape)
    if len(shape) != 5 or shape[1] != 2:
        raise ValueError("%s must have shape [L, 2, T, H, D], got %s" % (what, list(shape)))
    return shape[0], shape[2], shape[3], shape[4]


def _check_out(out, shape, dtype):
    """A caller's output tensor must be exactly what the kernels write: the C
    calls take no output size, so a smaller tensor would be written past its
    end."""
    if out is not None and (tuple(out.shape) != tuple(shape) or out.dtype != dtype):
        raise ValueError("out must be a %s tensor of shape %s, got %s of shape %s"
                         % (dtype, list(shape), out.dtype, list(out.shape)))


def _check_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def abi_version():
    return _lib.lib().kvc_abi_version()


def encoded_size(layers, tokens, kv_heads, head_dim, bits_k, bits_v, group, dtype="bf16"):
    """(total bytes, byte offset of the meta section) of a blob."""
    lib = _lib.lib()
    total, meta = ctypes.c_uint64(), ctypes.c_uint64()
    d = _desc(layers, tokens, kv_heads, head_dim, dtype, bits_k, bits_v, group)
    _lib.check(lib.kvc_encoded_size(ctypes.byref(d), int(tokens), ctypes.byref(total), ctypes.byref(meta)))
    return total.value, meta.value


def sign_mask(seed, head_dim):
    """Integer whose bit j is set iff sign j of the transform is -1."""
    lib = _lib.lib()
    words = (ctypes.c_uint64 * ((head_dim + 63) // 64))()
    _lib.check(lib.kvc_sign_mask(int(seed) & ((1 << 64) - 1), int(head_dim), words))
    return sum(int(w) << (64 * i) for i, w in enumerate(words))


def _opts(transform, events):
    """kvc_launch_opts for the *_with calls, or None when neither is given.
    ``events``: (start, stop) hipEvent_t handles (ints or c_void_p; either may be None)."""
    if transform is None and events is None:
        return None
    if transform is not None and transform not in _lib.TRANSFORM:
        raise ValueError("transform must be one of %s" % sorted(_lib.TRANSFORM))
    start, stop = events if events is not None else (None, None)
    val = lambda e: e.value if isinstance(e, ctypes.c_void_p) else e
    return _lib.KvcLaunchOpts(_lib.TRANSFORM[transform or "auto"], 0, val(start), val(stop))


def encode(kv, bits_k, bits_v, group, seed=0, out=None, stream=None, transform=None, events=None):
    """Encode a contiguous [L, 2, T, H, D] GPU tensor; returns the uint8 blob.
    ``transform`` ("auto", "matrix" or "butterfly") or ``events`` (start,
    stop hipEvent_t handles for the kernels' own times) call kvc_encode_with."""
    L, T, H, D = _kv_shape(kv.shape, "kv")
    dt = _dtype_name(kv)
    _check_cuda(kv, out)
    total, _ = encoded_size(L, T, H, D, bits_k, bits_v, group, dt)
    if out is None:
        out = torch.empty(total, dtype=torch.uint8, device=kv.device)
    d = _desc(L, T, H, D, dt, bits_k, bits_v, group, seed)
    o = _opts(transform, events)
    if o is None:
        _lib.check(_lib.lib().kvc_encode(ctypes.byref(d), _ptr(kv), _ptr(out), _nbytes(out), _stream(stream)))
    else:
        _lib.check(_lib.lib().kvc_encode_with(ctypes.byref(d), _ptr(kv), _ptr(out), _nbytes(out),
                                              ctypes.byref(o), _stream(stream)))
    return out


def decode(blob, shape, dtype, bits_k, bits_v, group, seed=0, out=None, stream=None, transform=None, events=None):
    """Decode a blob into a [L, 2, T, H, D] GPU tensor of ``dtype``.
    ``transform`` / ``events`` as for :func:`encode` (kvc_decode_with)."""
    L, T, H, D = _kv_shape(shape, "shape")
    _check_out(out, shape, _torch_dtype(dtype))
    _check_cuda(blob, out)
    if out is None:
        out = torch.empty(tuple(shape), dtype=_torch_dtype(dtype), device=blob.device)
    d = _desc(L, T, H, D, dtype, bits_k, bits_v, group, seed)
    o = _opts(transform, events)
    if o is None:
        _lib.check(_lib.lib().kvc_decode(ctypes.byref(d), _ptr(blob), _nbytes(blob), _ptr(out), _stream(stream)))
    else:
        _lib.check(_lib.lib().kvc_decode_with(ctypes.byref(d), _ptr(blob), _nbytes(blob), _ptr(out),
                                              ctypes.byref(o), _stream(stream)))
    return out


def unfused_workspace_size(layers, tokens, kv_heads, head_dim, bits_k, bits_v, group, dtype="bf16"):
    """Device workspace bytes of the separate-kernel comparator for this shape."""
    n = ctypes.c_uint64()
    d = _desc(layers, tokens, kv_heads, head_dim, dtype, bits_k, bits_v, group)
    _lib.check(_lib.lib().kvc_unfused_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def _workspace(ws, nbytes, device):
    if ws is None:
        ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    _check_cuda(ws)
    return ws


def encode_unfused(kv, bits_k, bits_v, group, seed=0, out=None, workspace=None, stream=None):
    """Comparator: :func:`encode` computed by separate kernels through ``workspace``."""
    L, T, H, D = _kv_shape(kv.shape, "kv")
    dt = _dtype_name(kv)
    _check_cuda(kv, out)
    total, _ = encoded_size(L, T, H, D, bits_k, bits_v, group, dt)
    if out is None:
        out = torch.empty(total, dtype=torch.uint8, device=kv.device)
    ws = _workspace(workspace, unfused_workspace_size(L, T, H, D, bits_k, bits_v, group, dt), kv.device)
    d = _desc(L, T, H, D, dt, bits_k, bits_v, group, seed)
    _lib.check(_lib.lib().kvc_encode_unfused(ctypes.byref(d), _ptr(kv), _ptr(out), _nbytes(out), _ptr(ws),
                                             _nbytes(ws), _stream(stream)))
    return out


def encode_unfused_noalloc(kv, bits_k, bits_v, group, seed=0, out=None, stream=None):
    """Comparator encode whose workspace is the library's static device array
    (allocates nothing in the call itself; ``out`` must then be given by
    callers that cannot allocate).  Calls that overlap on one device race."""
    L, T, H, D = _kv_shape(kv.shape, "kv")
    dt = _dtype_name(kv)
    _check_cuda(kv, out)
    if out is None:
        total, _ = encoded_size(L, T, H, D, bits_k, bits_v, group, dt)
        out = torch.empty(total, dtype=torch.uint8, device=kv.device)
    d = _desc(L, T, H, D, dt, bits_k, bits_v, group, seed)
    _lib.check(_lib.lib().kvc_encode_unfused_noalloc(ctypes.byref(d), _ptr(kv), _ptr(out), _nbytes(out),
                                                     _stream(stream)))
    return out


def decode_unfused(blob, shape, dtype, bits_k, bits_v, group, seed=0, out=None, workspace=None, stream=None):
    """Comparator: :func:`decode` computed by separate kernels through ``workspace``."""
    L, T, H, D = _kv_shape(shape, "shape")
    _check_out(out, shape, _torch_dtype(dtype))
    _check_cuda(blob, out)
    if out is None:
        out = torch.empty(tuple(shape), dtype=_torch_dtype(dtype), device=blob.device)
    ws = _workspace(workspace, unfused_workspace_size(L, T, H, D, bits_k, bits_v, group, dtype), blob.device)
    d = _desc(L, T, H, D, dtype, bits_k, bits_v, group, seed)
    _lib.check(_lib.lib().kvc_decode_unfused(ctypes.byref(d), _ptr(blob), _nbytes(blob), _ptr(out), _ptr(ws),
                                             _nbytes(ws), _stream(stream)))
    return out


def chunked_size(layers, tokens, kv_heads, head_dim, bits_k, bits_v, group, chunk_layers, dtype="bf16"):
    """(total bytes, stride between chunk starts) of a chunked blob."""
    total, stride = ctypes.c_uint64(), ctypes.c_uint64()
    d = _desc(layers, tokens, kv_heads, head_dim, dtype, bits_k, bits_v, group)
    _lib.check(_lib.lib().kvc_chunked_size(ctypes.byref(d), int(chunk_layers), ctypes.byref(total),
                                           ctypes.byref(stride)))
    return total.value, stride.value


def encode_send(kv, bits_k, bits_v, group, chunk_layers, dst, seed=0, out=None, compute_stream=None,
                copy_stream=None):
    """Encode layer chunks on ``compute_stream`` and copy each finished chunk
    into ``dst`` (a pinned host or device tensor) on ``copy_stream``."""
    L, T, H, D = _kv_shape(kv.shape, "kv")
    dt = _dtype_name(kv)
    _check_cuda(kv, out)
    if not dst.is_contiguous():
        raise ValueError("dst must be contiguous")
    total, _ = chunked_size(L, T, H, D, bits_k, bits_v, group, chunk_layers, dt)
    if out is None:
        out = torch.empty(total, dtype=torch.uint8, device=kv.device)
    d = _desc(L, T, H, D, dt, bits_k, bits_v, group, seed)
    _lib.check(_lib.lib().kvc_encode_send(ctypes.byref(d), _ptr(kv), _ptr(out), _nbytes(out), int(chunk_layers),
                                          _ptr(dst), _nbytes(dst), _stream(compute_stream),
                                          _stream(copy_stream)))
    return out


def receive_decode(src, shape, dtype, bits_k, bits_v, group, chunk_layers, seed=0, staging=None, out=None,
                   compute_stream=None, copy_stream=None):
    """Copy layer chunks of ``src`` (a pinned host or device tensor) into
    ``staging`` on ``copy_stream`` and decode each on ``compute_stream``
    into ``out``."""
    L, T, H, D = _kv_shape(shape, "shape")
    _check_out(out, shape, _torch_dtype(dtype))
    _check_cuda(staging, out)
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    total, _ = chunked_size(L, T, H, D, bits_k, bits_v, group, chunk_layers, dtype)
    if staging is None:
        device = src.device if src.is_cuda else torch.device("cuda", torch.cuda.current_device())
        staging = torch.empty(max(total, 1), dtype=torch.uint8, device=device)
    if out is None:
        out = torch.empty(tuple(shape), dtype=_torch_dtype(dtype), device=staging.device)
    d = _desc(L, T, H, D, dtype, bits_k, bits_v, group, seed)
    _lib.check(_lib.lib().kvc_receive_decode(ctypes.byref(d), _ptr(src), _nbytes(src), _ptr(staging),
                                             _nbytes(staging), int(chunk_layers), _ptr(out),
                                             _stream(compute_stream), _stream(copy_stream)))
    return out


def paged_layout(seq_lens, layers, kv_heads, head_dim, bits_k, bits_v, group, dtype="bf16"):
    """(offsets int64 numpy array, total bytes) of the per-request blobs."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    offs = np.zeros(len(lens), dtype=np.int64)
    total = ctypes.c_uint64()
    d = _desc(layers, 0, kv_heads, head_dim, dtype, bits_k, bits_v, group)
    _lib.check(_lib.lib().kvc_paged_layout(
        ctypes.byref(d), lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(lens),
        offs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ctypes.byref(total)))
    return offs, total.value


PAGED_ITEM = np.dtype([("block", "<i4"), ("block_index", "<i4"), ("req", "<i4"), ("len", "<i4"),
                       ("offset", "<i8"), ("reserved", "<i8")])


def paged_order(block_table, seq_lens, offsets, block_size, num_blocks, lib=None):
    """Host prologue of the pool-order paged calls: the (request, block) items
    of the call sorted by pool block, as a numpy array of PAGED_ITEM (upload
    its bytes, e.g. ``torch.from_numpy(items.view(np.uint8))``, and pass them
    as ``order=``)."""
    lib = lib or _lib.lib()
    table = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    if table.ndim != 2 or lens.shape != (table.shape[0],) or offs.shape != lens.shape:
        raise ValueError("block_table must be [R, max_blocks] with one length and offset per row")
    R, MB = table.shape
    P32, P64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    n = ctypes.c_int64()
    args = (table.ctypes.data_as(P32), R, MB, lens.ctypes.data_as(P32), offs.ctypes.data_as(P64), int(block_size),
            int(num_blocks))
    _lib.check(lib.kvc_paged_order(*args, None, ctypes.byref(n)))
    items = np.zeros(n.value, dtype=PAGED_ITEM)
    if n.value:
        _lib.check(lib.kvc_paged_order(*args, ctypes.c_void_p(items.ctypes.data), ctypes.byref(n)))
    return items


def _pool_shape(pool):
    """(L, NB, BS, H, D) of a [L, 2, NB, BS, H, D] pool."""
    if pool.dim() != 6 or pool.shape[1] != 2:
        raise ValueError("pool must have shape [L, 2, NB, BS, H, D], got %s" % list(pool.shape))
    L, _, NB, BS, H, D = pool.shape
    return L, NB, BS, H, D


def _paged(pool, block_table, seq_lens, out_offsets, err_flag, order=None):
    """The kernels read seq_lens[r], out_offsets[r] and the first max_blocks
    entries of row r of block_table for every r < R, and write err_flag[0]:
    the arrays must hold that much.  ``order``: an optional device tensor
    holding PAGED_ITEM entries (a whole number of 32-byte items)."""
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or out_offsets.dtype != torch.int64:
        raise ValueError("block_table / seq_lens must be int32 and out_offsets int64")
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_reqs, max_blocks]")
    R, MB = block_table.shape
    if tuple(seq_lens.shape) != (R,) or tuple(out_offsets.shape) != (R,):
        raise ValueError("seq_lens and out_offsets must hold one entry per block_table row (%d)" % R)
    if err_flag is not None and (err_flag.dtype != torch.int32 or err_flag.numel() < 1):
        raise ValueError("err_flag must be an int32 tensor of at least one element")
    _check_cuda(block_table, seq_lens, out_offsets, err_flag, order)
    n_order = 0
    if order is not None:
        if _nbytes(order) % PAGED_ITEM.itemsize:
            raise ValueError("order must hold whole %d-byte items" % PAGED_ITEM.itemsize)
        n_order = _nbytes(order) // PAGED_ITEM.itemsize
    return KvcPaged(pool.shape[2], pool.shape[3], R, MB, 0, _ptr(block_table).value,
                    _ptr(seq_lens).value, _ptr(out_offsets).value,
                    _ptr(err_flag).value if err_flag is not None else None,
                    _ptr(order).value if n_order else None, n_order)


def encode_paged(pool, block_table, seq_lens, out_offsets, total, bits_k, bits_v, group, seed=0,
                 out=None, err_flag=None, stream=None, order=None, transform=None, events=None):
    """Encode every request of a [L, 2, NB, BS, H, D] pool into one blob buffer
    (in pool order when ``order`` holds the call's :func:`paged_order` items).
    ``transform`` / ``events`` as for :func:`encode` (kvc_encode_paged_with)."""
    L, NB, BS, H, D = _pool_shape(pool)
    dt = _dtype_name(pool)
    pg = _paged(pool, block_table, seq_lens, out_offsets, err_flag, order)
    _check_cuda(pool, out)
    if out is None:
        out = torch.empty(int(total), dtype=torch.uint8, device=pool.device)
    d = _desc(L, 0, H, D, dt, bits_k, bits_v, group, seed)
    o = _opts(transform, events)
    if o is None:
        _lib.check(_lib.lib().kvc_encode_paged(ctypes.byref(d), _ptr(pool), ctypes.byref(pg), _ptr(out),
                                               _nbytes(out), _stream(stream)))
    else:
        _lib.check(_lib.lib().kvc_encode_paged_with(ctypes.byref(d), _ptr(pool), ctypes.byref(pg), _ptr(out),
                                                    _nbytes(out), ctypes.byref(o), _stream(stream)))
    return out


def decode_paged(blob, pool, block_table, seq_lens, out_offsets, bits_k, bits_v, group, seed=0,
                 err_flag=None, stream=None, order=None, transform=None, events=None):
    """Decode every request's blob back into the pool slots of its block table
    (in pool order when ``order`` holds the call's :func:`paged_order` items).
    ``transform`` / ``events`` as for :func:`encode` (kvc_decode_paged_with)."""
    L, NB, BS, H, D = _pool_shape(pool)
    dt = _dtype_name(pool)
    pg = _paged(pool, block_table, seq_lens, out_offsets, err_flag, order)
    _check_cuda(blob, pool)
    d = _desc(L, 0, H, D, dt, bits_k, bits_v, group, seed)
    o = _opts(transform, events)
    if o is None:
        _lib.check(_lib.lib().kvc_decode_paged(ctypes.byref(d), _ptr(blob), _nbytes(blob), ctypes.byref(pg),
                                               _ptr(pool), _stream(stream)))
    else:
        _lib.check(_lib.lib().kvc_decode_paged_with(ctypes.byref(d), _ptr(blob), _nbytes(blob), ctypes.byref(pg),
                                                    _ptr(pool), ctypes.byref(o), _stream(stream)))
    return pool


def debug_rotate(kv, seed=0, out=None, stream=None):
    """Rotated values y = H (s * x) / sqrt(D) of the encode path, fp32."""
    L, T, H, D = _kv_shape(kv.shape, "kv")
    dt = _dtype_name(kv)
    _check_out(out, kv.shape, torch.float32)
    _check_cuda(kv, out)
    if out is None:
        out = torch.empty(tuple(kv.shape), dtype=torch.float32, device=kv.device)
    d = _desc(L, T, H, D, dt, 4, 4, 32, seed)
    _lib.check(_lib.lib().kvc_debug_rotate(ctypes.byref(d), _ptr(kv), _ptr(out), _stream(stream)))
    return out


def probe_copy(src, dst, stream=None):
    """Streaming device copy of src into dst (same byte size)."""
    _check_cuda(src, dst)
    nbytes = _nbytes(src)
    if _nbytes(dst) < nbytes:
        raise ValueError("destination too small")
    _lib.check(_lib.lib().kvc_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))
    return dst


def probe_blocks(region, block_bytes, blocks, seq, stream_bytes, scatter, waves_per_cu=8, stream=None):
    """Block gather / scatter yardstick (kvc_probe_blocks): ``region`` holds
    whole blocks of ``block_bytes``; ``blocks`` is a device int32 tensor of
    block indices moved in list order against ``stream_bytes`` of ``seq``."""
    _check_cuda(region, seq, blocks)
    if blocks.dtype != torch.int32 or blocks.dim() != 1:
        raise ValueError("blocks must be a 1-D int32 tensor")
    if stream_bytes > _nbytes(seq):
        raise ValueError("stream_bytes exceeds seq")
    region_blocks = _nbytes(region) // int(block_bytes)
    _lib.check(_lib.lib().kvc_probe_blocks(_ptr(region), region_blocks, int(block_bytes), _ptr(blocks),
                                           blocks.numel(), _ptr(seq), int(stream_bytes), int(scatter),
                                           int(waves_per_cu), _stream(stream)))
    return region if scatter else seq


def probe_stream(src, read_bytes, dst, write_bytes, waves_per_cu=8, stream=None):
    """Streaming yardstick: read ``read_bytes`` of ``src`` and write
    ``write_bytes`` of ``dst`` (multiples of 1024, within the tensors)."""
    _check_cuda(src, dst)
    if read_bytes > _nbytes(src) or write_bytes > _nbytes(dst):
        raise ValueError("probe sizes exceed the tensors")
    _lib.check(_lib.lib().kvc_probe_stream(_ptr(src), int(read_bytes), _ptr(dst), int(write_bytes),
                                           int(waves_per_cu), _stream(stream)))
    return dst


def probe_stream_runs(src, read_bytes, dst, write_bytes, run_kib=16, waves_per_cu=4, stream=None):
    """Streaming yardstick with each run of ``run_kib`` KiB of the larger
    stream issued at once: read ``read_bytes`` of ``src`` and write
    ``write_bytes`` of ``dst`` (multiples of 1024, within the tensors)."""
    _check_cuda(src, dst)
    if read_bytes > _nbytes(src) or write_bytes > _nbytes(dst):
        raise ValueError("probe sizes exceed the tensors")
    _lib.check(_lib.lib().kvc_probe_stream_runs(_ptr(src), int(read_bytes), _ptr(dst), int(write_bytes),
                                                int(run_kib), int(waves_per_cu), _stream(stream)))
    return dst
