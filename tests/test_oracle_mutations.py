"""The pins are sharp: plausible mistakes planted in the oracle (on the CPU,
through monkeypatching) make at least one pin fail."""

import numpy as np
import pytest

from oracle import nm_oracle as O
from tests import test_oracle_pins as P


def _select_tie_high(keys, N, M):
    R, K = keys.shape
    g = keys.reshape(R, K // M, M)
    rank = np.zeros(g.shape, np.int64)
    for p in range(M):
        for q in range(M):
            if q != p:
                rank[:, :, p] += g[:, :, q] > g[:, :, p]
                if q > p:                                   # mistake: higher index wins ties
                    rank[:, :, p] += g[:, :, q] == g[:, :, p]
    return (rank < N).astype(np.uint8).reshape(R, K)


def _select_no_ties(keys, N, M):
    R, K = keys.shape
    g = keys.reshape(R, K // M, M)
    rank = np.zeros(g.shape, np.int64)
    for p in range(M):
        for q in range(M):
            if q != p:
                rank[:, :, p] += g[:, :, q] > g[:, :, p]   # mistake: equality term dropped
    return (rank < N).astype(np.uint8).reshape(R, K)


_orig_pack = O.pack_positions
_orig_unpack = O.unpack_positions_flat
_orig_l1 = O.venom_column_l1
_orig_relu = O.relu_raw
_orig_decompress = O.decompress_nm
_orig_reprune = O.reprune_t
_orig_prune = O.prune_nm


def _pack_msb_first(pos, M, nbytes):
    b = O.meta_bits(M)
    swapped = np.zeros_like(pos)
    for t in range(b):                                      # mistake: bits of a field reversed
        swapped |= ((pos >> t) & 1) << (b - 1 - t)
    return _orig_pack(swapped, M, nbytes)


def _unpack_msb_first(meta, F, M):
    pos = _orig_unpack(meta, F, M)
    b = O.meta_bits(M)
    out = np.zeros_like(pos)
    for t in range(b):
        out |= ((pos >> t) & 1) << (b - 1 - t)
    return out


def _l1_max(x, V, M):
    R, K = x.shape
    return np.abs(x).reshape(R // V, V, K).max(axis=1)     # mistake: max instead of sum


def _l1_signed(x, V, M):
    R, K = x.shape
    return x.reshape(R // V, V, K).sum(axis=1)             # mistake: |.| dropped


def _relu_keeps_negzero(raw, dtype):
    x = O.decode(raw, dtype)
    out = raw.copy()
    out[x < 0] = 0                                          # mistake: -0.0 survives
    return out


def _decompress_negzero(values, meta, R, K, N, M):
    out = _orig_decompress(values, meta, R, K, N, M)
    fill = np.float32(-0.0) if out.dtype == np.float32 else np.uint16(0x8000)
    pos = O.unpack_positions(meta, R, K, N, M)
    keep = np.zeros((R, K // M, M), bool)
    np.put_along_axis(keep, pos, True, axis=2)
    out = out.copy()
    out[~keep.reshape(R, K)] = fill                         # mistake: -0.0 fill
    return out


def _reprune_no_transpose(values, meta, R, K, dtype):
    ws = _orig_decompress(values, meta, R, K, 2, 4)
    vt, mt, _ = O.compress_nm(ws, _orig_prune(ws, dtype, 2, 4), 2, 4)   # mistake: no transpose
    return vt, mt


def _prune_signed(raw, dtype, N, M):
    return O.nm_select(O.decode(raw, dtype), N, M)          # mistake: signed key, not magnitude


_orig_encode = O.encode_bf16


def _encode_half_up(x):
    x = np.asarray(x, np.float64)
    f, e = np.frexp(x)
    step_exp = np.maximum(e - 8, -133)
    y = np.floor(np.abs(np.ldexp(x, -step_exp)) + 0.5) * np.sign(x) * np.ldexp(1.0, step_exp)   # mistake: ties up
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _encode_truncate(x):
    return (np.asarray(x, np.float64).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)  # mistake: chops


_orig_spmm = O.spmm_nm


def _lowrank_dropped(values, meta, R, K, B_raw, U_raw, Vt_raw, dtype):
    T = O.decode(Vt_raw, dtype) @ O.decode(B_raw, dtype)
    return _orig_spmm(values, meta, R, K, B_raw, dtype), T        # mistake: adapter term left out


def _lowrank_minus(values, meta, R, K, B_raw, U_raw, Vt_raw, dtype):
    T = O.decode(Vt_raw, dtype) @ O.decode(B_raw, dtype)
    return _orig_spmm(values, meta, R, K, B_raw, dtype) - O.decode(U_raw, dtype) @ T, T   # mistake: sign


def _lowrank_rows_reversed(values, meta, R, K, B_raw, U_raw, Vt_raw, dtype):
    T = O.decode(Vt_raw, dtype) @ O.decode(B_raw, dtype)
    return _orig_spmm(values, meta, R, K, B_raw, dtype) + O.decode(U_raw, dtype)[::-1] @ T, T  # mistake: U rows


def _lowrank_k_reversed(values, meta, R, K, B_raw, U_raw, Vt_raw, dtype):
    T = O.decode(Vt_raw, dtype)[:, ::-1] @ O.decode(B_raw, dtype)   # mistake: Vt index order
    return _orig_spmm(values, meta, R, K, B_raw, dtype) + O.decode(U_raw, dtype) @ T, T


def _general_slot_shift(values, meta, R, K, N, M, B_raw, dtype):
    pos = O.unpack_positions(meta, R, K, N, M)
    v = O.decode(values, dtype).reshape(R, K // M, N)
    A = np.zeros((R, K // M, M))
    np.put_along_axis(A, pos, np.roll(v, 1, axis=2), axis=2)   # mistake: values paired with the wrong slot
    return A.reshape(R, K) @ O.decode(B_raw, dtype)


_orig_kept = O.venom_kept_columns


def _kept_no_colsel(meta, colsel, T, F, V, M):
    G = F // M
    pos = O.unpack_positions(meta, T, G * 4, 2, 4)
    return (np.arange(G)[None, :, None] * M + pos).reshape(T, G * 2)   # mistake: j_s used as the column


def _kept_block_of_next_row(meta, colsel, T, F, V, M):
    return _orig_kept(meta, np.roll(colsel, -1, axis=0), T, F, V, M)    # mistake: wrong V-block's choice


def _sddmm_venom_gate_inverted(dY_raw, Wd_raw, h_values, h_meta, h_colsel, T, F, V, M, dtype, relu):
    full = O.decode(dY_raw, dtype) @ O.decode(Wd_raw, dtype).T
    out = np.take_along_axis(full, _orig_kept(h_meta, h_colsel, T, F, V, M), axis=1)
    return np.where(O.decode(h_values, dtype) <= 0, out, 0.0) if relu else out   # mistake: gate inverted


def _spmm_venom_tn_tokens_shifted(h_values, h_meta, h_colsel, T, F, V, M, dY_raw, dtype):
    H = O.decode(O.decompress_venom(h_values, h_meta, h_colsel, T, F, V, M), dtype)
    return H.T @ np.roll(O.decode(dY_raw, dtype), 1, axis=0)   # mistake: dY rows paired with the wrong tokens


MUTATIONS = [
    ("nm_select", _select_tie_high, [lambda: P.test_nm_select_exhaustive_m4(2, "f32")]),
    ("nm_select", _select_no_ties, [lambda: P.test_prune_compress_invariants(2, 4, "bf16")]),
    ("prune_nm", _prune_signed, [lambda: P.test_golden_nm24()]),
    ("pack_positions", _pack_msb_first, [lambda: P.test_golden_nm28_bit_stream()]),
    ("unpack_positions_flat", _unpack_msb_first, [lambda: P.test_golden_reprune_t()]),
    ("venom_column_l1", _l1_max, [lambda: P.test_venom_brute(2, 8)]),
    ("venom_column_l1", _l1_signed, [lambda: P.test_venom_brute(3, 8)]),
    ("relu_raw", _relu_keeps_negzero, [lambda: P.test_relu_venom()]),
    ("decompress_nm", _decompress_negzero, [lambda: P.test_prune_compress_invariants(2, 4, "f32")]),
    ("reprune_t", _reprune_no_transpose, [lambda: P.test_golden_reprune_t()]),
    ("encode_bf16", _encode_half_up, [lambda: P.test_encode_bf16_known_values(),
                                      lambda: P.test_encode_bf16_is_nearest_ties_even_brute()]),
    ("encode_bf16", _encode_truncate, [lambda: P.test_encode_bf16_known_values(),
                                       lambda: P.test_encode_bf16_matches_fp32_bit_rounding()]),
    ("spmm_nm_lowrank", _lowrank_dropped, [lambda: P.test_spmm_lowrank_exact_integers()]),
    ("spmm_nm_lowrank", _lowrank_minus, [lambda: P.test_spmm_lowrank_is_the_adapted_weight_times_b()]),
    ("spmm_nm_lowrank", _lowrank_rows_reversed, [lambda: P.test_spmm_lowrank_exact_integers(),
                                                 lambda: P.test_spmm_lowrank_special_cases()]),
    ("spmm_nm_lowrank", _lowrank_k_reversed, [lambda: P.test_spmm_lowrank_exact_integers()]),
    ("spmm_nm_general", _general_slot_shift, [lambda: P.test_spmm_general_gather_loop_and_exact_integers(2, 8)]),
    ("venom_kept_columns", _kept_no_colsel, [lambda: P.test_sddmm_venom_loop_and_exact_integers(False),
                                             lambda: P.test_venom_backward_adjoint_identities(4, 8)]),
    ("venom_kept_columns", _kept_block_of_next_row, [lambda: P.test_sddmm_venom_loop_and_exact_integers(False),
                                                     lambda: P.test_venom_backward_adjoint_identities(4, 8)]),
    ("sddmm_venom", _sddmm_venom_gate_inverted, [lambda: P.test_sddmm_venom_loop_and_exact_integers(True),
                                                 lambda: P.test_sddmm_venom_relu_gate()]),
    ("spmm_venom_tn", _spmm_venom_tn_tokens_shifted, [lambda: P.test_spmm_venom_tn_loop_and_exact_integers(),
                                                lambda: P.test_venom_backward_adjoint_identities(2, 4)]),
]


@pytest.mark.parametrize("name,fn,pins", MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn, pins):
    monkeypatch.setattr(O, name, fn)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()


def test_spmm_transposed_operand_is_caught(monkeypatch):
    def spmm_bt(values, meta, R, K, B_raw, dtype):
        A = O.decode(_orig_decompress(values, meta, R, K, 2, 4), dtype)
        B = O.decode(B_raw, dtype)
        return A @ B[::-1]                                  # mistake: B rows reversed
    monkeypatch.setattr(O, "spmm_nm", spmm_bt)
    with pytest.raises(AssertionError):
        P.test_spmm_gather_loop_equals_dgemm("f32")
    with pytest.raises(AssertionError):
        P.test_golden_nm24()
