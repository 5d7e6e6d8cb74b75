"""The binding's argument checks.  The C calls take no size for a decode's
output tensor or for the paged arrays, so the binding must refuse shapes
the kernels would read or write past; every check here fires before any
library call, so these run on CPU tensors."""
import pytest
import torch

import kv_cache_compression_kvc_amd as kvc

SHAPE = (2, 2, 8, 1, 64)


def _blob():
    return torch.zeros(4096, dtype=torch.uint8)


@pytest.mark.parametrize("shape", [(2, 1, 8, 1, 64), (2, 3, 8, 1, 64), (2, 8, 1, 64), (1, 2, 2, 8, 1, 64)])
def test_decode_refuses_a_shape_without_k_and_v(shape):
    with pytest.raises(ValueError, match=r"\[L, 2, T, H, D\]"):
        kvc.decode(_blob(), shape, "bf16", 4, 4, 64)
    with pytest.raises(ValueError, match=r"\[L, 2, T, H, D\]"):
        kvc.decode_unfused(_blob(), shape, "bf16", 4, 4, 64)
    with pytest.raises(ValueError, match=r"\[L, 2, T, H, D\]"):
        kvc.receive_decode(_blob(), shape, "bf16", 4, 4, 64, 1)


@pytest.mark.parametrize("out", [torch.empty((1, 2, 8, 1, 64), dtype=torch.bfloat16),   # one layer short
                                 torch.empty(SHAPE, dtype=torch.float16),               # other dtype
                                 torch.empty(2 * 2 * 8 * 64, dtype=torch.bfloat16)])    # flat
def test_decode_refuses_an_output_tensor_of_another_shape_or_dtype(out):
    with pytest.raises(ValueError, match="out must be"):
        kvc.decode(_blob(), SHAPE, "bf16", 4, 4, 64, out=out)
    with pytest.raises(ValueError, match="out must be"):
        kvc.decode_unfused(_blob(), SHAPE, "bf16", 4, 4, 64, out=out)
    with pytest.raises(ValueError, match="out must be"):
        kvc.receive_decode(_blob(), SHAPE, "bf16", 4, 4, 64, 1, out=out)


def test_dtype_names_and_tensor_dtypes_are_checked():
    with pytest.raises(ValueError, match="dtype must be"):
        kvc.decode(_blob(), SHAPE, "fp32", 4, 4, 64)
    with pytest.raises(ValueError, match="bfloat16 or float16"):
        kvc.encode(torch.zeros(SHAPE, dtype=torch.float32), 4, 4, 64)
    with pytest.raises(ValueError, match="bfloat16 or float16"):
        kvc.debug_rotate(torch.zeros(SHAPE, dtype=torch.float32))


def test_encode_side_refuses_a_tensor_without_k_and_v():
    x = torch.zeros((2, 1, 8, 1, 64), dtype=torch.bfloat16)
    for call in (lambda: kvc.encode(x, 4, 4, 64),
                 lambda: kvc.encode_unfused(x, 4, 4, 64),
                 lambda: kvc.encode_send(x, 4, 4, 64, 1, _blob()),
                 lambda: kvc.debug_rotate(x)):
        with pytest.raises(ValueError, match=r"\[L, 2, T, H, D\]"):
            call()


def test_debug_rotate_output_must_be_fp32_of_the_input_shape():
    x = torch.zeros(SHAPE, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out must be"):
        kvc.debug_rotate(x, out=torch.empty(SHAPE, dtype=torch.bfloat16))


def _paged_args(R=3, MB=4):
    return (torch.zeros((R, MB), dtype=torch.int32), torch.zeros(R, dtype=torch.int32),
            torch.zeros(R, dtype=torch.int64))


def test_paged_calls_check_the_pool_and_the_request_arrays():
    pool = torch.zeros((2, 2, 5, 16, 1, 64), dtype=torch.bfloat16)
    bt, sl, of = _paged_args()
    with pytest.raises(ValueError, match="pool must have shape"):
        kvc.encode_paged(pool[:, :1], bt, sl, of, 4096, 4, 4, 64)
    with pytest.raises(ValueError, match="pool must have shape"):
        kvc.decode_paged(_blob(), pool[0], bt, sl, of, 4, 4, 64)
    with pytest.raises(ValueError, match="one entry per block_table row"):
        kvc.encode_paged(pool, bt, sl[:2], of, 4096, 4, 4, 64)
    with pytest.raises(ValueError, match="one entry per block_table row"):
        kvc.decode_paged(_blob(), pool, bt, sl, torch.zeros(4, dtype=torch.int64), 4, 4, 64)
    with pytest.raises(ValueError, match=r"\[num_reqs, max_blocks\]"):
        kvc.encode_paged(pool, bt.reshape(-1), sl, of, 4096, 4, 4, 64)
    with pytest.raises(ValueError, match="int32 and out_offsets int64"):
        kvc.encode_paged(pool, bt, sl.long(), of, 4096, 4, 4, 64)
    with pytest.raises(ValueError, match="err_flag"):
        kvc.encode_paged(pool, bt, sl, of, 4096, 4, 4, 64, err_flag=torch.zeros(1, dtype=torch.int64))
    with pytest.raises(ValueError, match="err_flag"):
        kvc.encode_paged(pool, bt, sl, of, 4096, 4, 4, 64, err_flag=torch.zeros(0, dtype=torch.int32))


def test_well_formed_cpu_tensors_still_stop_at_the_device_check():
    """Past the shape checks, host tensors are refused before the library runs."""
    with pytest.raises(ValueError, match="live on the GPU"):
        kvc.decode(_blob(), SHAPE, "bf16", 4, 4, 64, out=torch.empty(SHAPE, dtype=torch.bfloat16))
    pool = torch.zeros((2, 2, 5, 16, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="live on the GPU"):
        kvc.encode_paged(pool, *_paged_args(), 4096, 4, 4, 64)
