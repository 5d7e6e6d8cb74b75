"""The oracle's pins catch plausible mistakes: each case below plants one
mistake in the oracle (on the CPU, by patching the function that holds the
step), runs the pins of test_oracle_*.py, and requires that at least one of
them fails.  A pin suite that let any of these through would not be pinning
the step it covers."""
import numpy as np
import pytest

import oracle
from oracle import blob as o_blob
from oracle import quant as o_quant
from oracle import rht as o_rht
from oracle import rounding as o_round
from oracle import scalar as o_scalar
from oracle import signs as o_signs

import test_oracle_blob as T_blob
import test_oracle_quant as T_quant
import test_oracle_rht as T_rht
import test_oracle_rounding as T_round
import test_oracle_signs as T_signs

MODULES = [oracle, o_signs, o_rht, o_quant, o_blob, o_round, o_scalar]

# fast pins first; each case stops at the first one that fails
BATTERY = [
    (T_signs.test_splitmix64_published_vectors, ()),
    (T_signs.test_signs_follow_bit63_and_are_counter_based, ()),
    (T_rht.test_hadamard_orthogonal_and_equals_scipy, (8,)),
    (T_rht.test_worked_examples, ()),
    (T_rht.test_closed_forms, (8,)),
    (T_rht.test_norm_preservation_and_round_trip, (64,)),
    (T_quant.test_packing_worked_examples, ()),
    (T_quant.test_error_bound_and_code_range, (4, 32)),
    (T_quant.test_exact_grid_groups_round_trip, (4,)),
    (T_quant.test_exact_ties_go_to_the_even_code, (4,)),
    (T_quant.test_brute_force_4x8, (4, 8, 0)),
    (T_quant.test_codes_match_exact_brute_force, (4,)),
    (T_blob.test_code_tiles_by_hand, ()),
    (T_blob.test_decode_inverts_encode_up_to_quantization, ("bf16",)),
    (T_round.test_rne_bf16_matches_torch_float32_conversion, ()),
    (T_blob.test_tiny_preset_matches_scalar_twin, ()),
    (T_blob.test_paged_equals_contiguous_per_request, ()),
    (T_round.test_directed_rounding_matches_exhaustive_search, ()),
]


def _first_failing():
    """(pin, exception type name) of the first pin that fails, or None."""
    for fn, args in BATTERY:
        try:
            fn(*args)
        except Exception as e:  # an assertion of the pin, or the step raising on its own check
            return fn.__name__, type(e).__name__
    return None


def _everywhere(mp, name, fn):
    """Replace `name` in every oracle module that holds it."""
    hit = [m for m in MODULES if hasattr(m, name)]
    assert hit, name
    for m in hit:
        mp.setattr(m, name, fn)


_hadamard, _rotate_raw, _dequantize = o_rht.hadamard, o_rht.rotate_raw, o_quant.dequantize
_blob_layout = o_blob.blob_layout
_splitmix = o_signs.splitmix64_outputs


def m_gamma(mp):          # a wrong SplitMix64 increment
    mp.setattr(o_signs, "_GAMMA", o_signs._GAMMA ^ 2)


def m_sign_bit(mp):       # the sign taken from bit 62 instead of bit 63
    def sv(seed, D):
        return np.array([-1.0 if (z >> 62) & 1 else 1.0 for z in _splitmix(seed, D)])
    _everywhere(mp, "sign_vector", sv)


def m_hadamard_rows(mp):  # two rows of H exchanged (still orthogonal)
    def h(D):
        H = _hadamard(D).copy()
        if D >= 4:
            H[[1, 2]] = H[[2, 1]]
        return H
    _everywhere(mp, "hadamard", h)


def m_no_norm(mp):        # the 1/sqrt(D) dropped from the forward transform
    _everywhere(mp, "rotate", lambda x, s: _rotate_raw(x, s))


def m_inverse_sign(mp):   # the sign not applied by the inverse transform
    def unrot(y, s):
        y = np.asarray(y, dtype=np.float64)
        return (y @ _hadamard(y.shape[-1])) / np.sqrt(y.shape[-1])
    _everywhere(mp, "unrotate", unrot)


def m_zero_nearest(mp):   # the zero rounded to nearest instead of down
    mp.setattr(o_quant, "rd16", lambda x: o_round.to_fp16(o_round.round_binary(x, "fp16", "rne")))


def m_scale_levels(mp):   # the range divided by 2^b instead of 2^b - 1
    def gm(y, G, bits):
        y = np.asarray(y, dtype=np.float64)
        yg = y.reshape(y.shape[:-1] + (y.shape[-1] // G, G))
        zero = o_round.rd16(yg.min(axis=-1) + 0.0)
        scale = o_round.ru16((yg.max(axis=-1) - zero.astype(np.float64)) / float(2 ** bits))
        return scale, zero
    _everywhere(mp, "group_meta", gm)


def m_ties_up(mp):        # ties rounded up instead of to even
    _everywhere(mp, "nearest_codes",
                lambda t, bits: np.clip(np.floor(np.asarray(t) + 0.5), 0, 2 ** bits - 1).astype(np.uint8))


def m_msb_first(mp):      # codes packed from the most significant bits (consistently both ways)
    def pk(q, bits):
        q = np.asarray(q, dtype=np.uint8)
        n = 8 // bits
        qb = q.reshape(q.shape[:-1] + (q.shape[-1] // n, n)).astype(np.uint16)
        out = np.zeros(qb.shape[:-1], dtype=np.uint16)
        for k in range(n):
            out |= qb[..., k] << (bits * (n - 1 - k))
        return out.astype(np.uint8)

    def upk(p, bits, D):
        p = np.asarray(p, dtype=np.uint8)
        n = 8 // bits
        parts = [(p >> (bits * (n - 1 - k))) & ((1 << bits) - 1) for k in range(n)]
        return np.stack(parts, axis=-1).reshape(p.shape[:-1] + (D,)).astype(np.uint8)
    _everywhere(mp, "pack_codes", pk)
    _everywhere(mp, "unpack_codes", upk)


def m_no_zero(mp):        # the decode drops the zero term
    _everywhere(mp, "dequantize", lambda q, s, z, G: _dequantize(q, s, np.zeros_like(np.asarray(z)), G))


def m_untiled(mp):        # code rows laid out row after row instead of in tiles
    _everywhere(mp, "tile_codes", lambda rows: np.asarray(rows, dtype=np.uint8).reshape(-1))


def m_bf16_truncate(mp):  # bf16 by truncation instead of round to nearest even
    def rb(x):
        f = np.asarray(x, dtype=np.float64).astype(np.float32)
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    _everywhere(mp, "rne_bf16", rb)


def m_sign_after(mp):     # the sign applied after the transform instead of before
    def rot(x, s):
        x = np.asarray(x, dtype=np.float64)
        return ((x @ _hadamard(x.shape[-1])) * s) / np.sqrt(x.shape[-1])
    _everywhere(mp, "rotate", rot)


def m_strided_groups(mp):  # groups taken with a stride instead of as consecutive coordinates
    def groups(a, G):
        D = a.shape[-1]
        return np.swapaxes(a.reshape(a.shape[:-1] + (G, D // G)), -1, -2)
    mp.setattr(o_quant, "_groups", groups)


def m_block_slot(mp):      # the slots of a block read in reverse order
    def gather(pool, table_row, seq_len):
        L, two, NB, BS, H, D = pool.shape
        out = np.zeros((L, 2, seq_len, H, D), dtype=pool.dtype)
        for t in range(seq_len):
            out[:, :, t] = pool[:, :, int(table_row[t // BS]), BS - 1 - t % BS]
        return out
    _everywhere(mp, "gather_request", gather)


def m_inclusive_offsets(mp):  # each request's offset taken after its own blob instead of before
    def layout(seq_lens, layers, kv_heads, head_dim, bits_k, bits_v, group):
        offsets, total = [], 0
        for n in seq_lens:
            total += _blob_layout(layers, int(n), kv_heads, head_dim, bits_k, bits_v, group).total
            offsets.append(total)
        return np.array(offsets, dtype=np.int64), total + (offsets[-1] if offsets else 0)
    _everywhere(mp, "paged_layout", layout)


MUTATIONS = [m_gamma, m_sign_bit, m_hadamard_rows, m_no_norm, m_inverse_sign, m_sign_after, m_zero_nearest,
             m_scale_levels, m_strided_groups, m_ties_up, m_msb_first, m_no_zero, m_untiled, m_bf16_truncate,
             m_block_slot, m_inclusive_offsets]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m.__name__ for m in MUTATIONS])
def test_planted_mistake_is_caught(mutation, monkeypatch):
    with monkeypatch.context() as mp:
        mutation(mp)
        caught = _first_failing()
    print(mutation.__name__, "caught by", caught)
    assert caught is not None, "no pin caught %s" % mutation.__name__
    assert caught[1] == "AssertionError", "%s raised %s in %s rather than failing a pin" % (
        mutation.__name__, caught[1], caught[0])
