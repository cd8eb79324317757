"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case swaps one oracle function for a copy with a plausible mistake (wrong tie rule,
wrong grid, wrong divisor, dropped term, swapped sign or index, transposed operand) and
checks that at least one pin test fails.  Mistakes are planted only in the oracle, on the
CPU.
"""
import numpy as np
import pytest

from oracle import nvfp4_oracle as O
from tests import test_oracle_codec as C
from tests import test_oracle_klt as K
from tests import test_oracle_mse_scale as M
from tests import test_oracle_transforms as T


def _ties_to_odd(a, unit, grid):
    a = np.asarray(a, dtype=np.float64)
    unit = np.broadcast_to(np.asarray(unit, dtype=np.float64), a.shape)
    mids = (grid[:-1] + grid[1:]) / 2.0
    idx = np.zeros(a.shape, dtype=np.int64)
    for k, mk in enumerate(mids):
        thr = mk * unit
        idx += (a > thr) | ((a == thr) & ((k + 1) % 2 == 1))
    return idx


def _quantize_absmax_to_4(y32, g):
    return ORIG_Q(np.asarray(y32, np.float32) * np.float32(1.5), g)


def _quantize_swapped_nibbles(y32, g):
    codes, scales = ORIG_Q(y32, g)
    return ((codes >> 4) | (codes << 4)).astype(np.uint8), scales


def _butterfly_wrong_sign(y):
    y = np.array(y, dtype=np.float32, copy=True)
    n = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < n:
        v = y.reshape(lead + (n // (2 * h), 2, h))
        a, b = v[..., 0, :], v[..., 1, :]
        y = np.stack([(a + b).astype(np.float32), (b - a).astype(np.float32)], -2).reshape(lead + (n,))
        h *= 2
    return y


def _key_transform_times_s(x, r, flags):
    rr = None if r is None else (np.float32(1) / np.asarray(r, np.float32)).astype(np.float32)
    return ORIG_KT(x, rr, flags)


def _calibrate_keep_pos0(k_win, v_win, exclude_pos0=True, k_flags=O.FLAG_SMOOTH):
    return ORIG_CAL(k_win, v_win, exclude_pos0=False, k_flags=k_flags)


def _attention_wrong_group(qp, k_hat, v_hat, seq_lens, sm_scale):
    qp = np.asarray(qp, np.float64)
    B, Hq, D = qp.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        K = np.asarray(k_hat[b])[:n]
        V = np.asarray(v_hat[b])[:n]
        Hkv = K.shape[1]
        for hq in range(Hq):
            h = hq % Hkv                      # interleaved instead of grouped mapping
            e = sm_scale * (K[:, h] @ qp[b, hq])
            p = np.exp(e - e.max())
            out[b, hq] = (p / p.sum()) @ V[:, h]
    return out


def _causal_sees_one_less(qp, k_hat, v_hat, seq_lens, sm_scale):
    """Off-by-one mask: position p attends to keys 0..p-1 (p = 0 then sees key 0)."""
    qp = np.asarray(qp, np.float64)
    B, Tq, Hq, D = qp.shape
    out = np.zeros((B, Tq, Hq, D))
    for b in range(B):
        n = int(seq_lens[b])
        K = np.asarray(k_hat[b], np.float64)
        V = np.asarray(v_hat[b], np.float64)
        grp = Hq // K.shape[1]
        for i in range(Tq):
            p = n - Tq + i
            if p < 0:
                continue
            last = max(p, 1)
            for hq in range(Hq):
                e = sm_scale * (K[:last, hq // grp] @ qp[b, i, hq])
                w = np.exp(e - e.max())
                out[b, i, hq] = (w / w.sum()) @ V[:last, hq // grp]
    return out


def _causal_wrong_offset(qp, k_hat, v_hat, seq_lens, sm_scale):
    """Queries placed at positions 0..Tq-1 instead of n-Tq..n-1."""
    qp = np.asarray(qp, np.float64)
    Tq = qp.shape[1]
    return ORIG_CA(qp, k_hat, v_hat, [min(int(n), Tq) for n in seq_lens], sm_scale)


def _mse_sse_drops_flushed(absy, c, g64):
    """Leaves out the elements that round to zero (their error |y|^2)."""
    c = np.asarray(c, dtype=np.int64)
    sigma = O.E4M3_GRID[c]
    unit = (sigma * g64)[:, None] * np.ones_like(absy)
    mag = O.rne_grid_index(absy, unit, O.E2M1_MAG_GRID)
    mag = np.where((sigma == 0.0)[:, None], 0, mag)
    d = np.where(mag > 0, absy - O.E2M1_MAG_GRID[mag] * unit, 0.0)
    return (d * d).sum(-1)


def _mse_pick_ties_to_last(cand, err):
    """Ties go to the last candidate column (the largest code) instead of the absmax code."""
    cols = [k for k in range(cand.shape[0]) if cand[k] >= 0]
    return min(cols, key=lambda k: (err[k], -k))


def _mse_ties_to_last(y32, g):
    """The whole search with ties to the largest code, fp64 ties included."""
    absy = np.abs(np.asarray(y32, np.float32).astype(np.float64)).reshape(-1, O.BLOCK)
    g64 = np.float64(np.float32(g))
    A = absy.max(-1)
    cand = O.mse_candidates(A, g64, O.absmax_scale_codes(A, g64))
    best = np.array([cand[i, _mse_pick_ties_to_last(cand[i], O.mse_block_sse_exact(absy[i], cand[i], g64))]
                     for i in range(cand.shape[0])])
    return best.reshape(np.asarray(y32).shape[:-1] + (O.N_BLOCKS,))


ORIG_CANDIDATES = O.mse_candidates


def _mse_candidates_without_absmax(A, g64, s0):
    """The candidates are the run only (the absmax-to-6 code only when it lies in the run, or
    when the run is empty)."""
    run = ORIG_CANDIDATES(A, g64, np.full_like(s0, -1))[:, 1:]
    cand = np.full((A.shape[0], 1 + run.shape[1]), -1, dtype=np.int64)
    cand[:, 1:] = run
    empty = (run < 0).all(axis=1)
    cand[empty, 0] = s0[empty]
    return cand


def _klt_variant(k_win, r, k_flags, exclude_pos0=True, centred=True, descending=True, sign=1.0):
    y = O.key_transform(np.asarray(k_win, np.float32), None if r is None else r[None, None], k_flags & O.FLAG_SMOOTH)
    y = y[:, 1:] if exclude_pos0 else y
    hkv = y.shape[2]
    X = y.astype(np.float64).reshape(-1, hkv, 128)
    B = np.zeros((hkv, 128, 128), np.float32)
    L = np.zeros((hkv, 128))
    for h in range(hkv):
        D = X[:, h] - X[:, h].mean(0) if centred else X[:, h]
        lam, V = np.linalg.eigh(D.T @ D / D.shape[0])
        order = np.argsort(-lam if descending else lam, kind="stable")
        lam, V = lam[order], V[:, order]
        for i in range(128):
            a = np.abs(V[:, i])
            j = int(np.argmax(a >= (1 - 1e-6) * a.max()))
            if sign * V[j, i] < 0:
                V[:, i] = -V[:, i]
        B[h], L[h] = V.astype(np.float32), lam
    return B, L


def _klt_uncentred(k_win, r, k_flags, exclude_pos0=True):
    return _klt_variant(k_win, r, k_flags, exclude_pos0, centred=False)


def _klt_ascending(k_win, r, k_flags, exclude_pos0=True):
    return _klt_variant(k_win, r, k_flags, exclude_pos0, descending=False)


def _klt_largest_negative(k_win, r, k_flags, exclude_pos0=True):
    return _klt_variant(k_win, r, k_flags, exclude_pos0, sign=-1.0)


def _rotate_transposed(y, basis):
    return ORIG_ROT(y, np.swapaxes(np.asarray(basis), 1, 2))


def _rotate_two_roundings(y, basis):
    return K._two_roundings(np.asarray(y, dtype=np.float32), np.asarray(basis, dtype=np.float32))


def _query_basis_not_transposed(q, s, flags, basis=None):
    if flags & O.FLAG_KLT:
        basis = np.swapaxes(np.asarray(basis), -1, -2)
    return ORIG_QT(q, s, flags, basis)


def _dequant_drop_g(codes, scales, g):
    return ORIG_DQ(codes, scales, 1.0)


ORIG_Q = O.quantize_rows
ORIG_KT = O.key_transform
ORIG_CAL = O.calibrate
ORIG_DQ = O.dequantize
ORIG_CA = O.causal_attention
ORIG_ROT = O.rotate_fp32
ORIG_QT = O.query_transform

CASES = [
    ("rne_grid_index", _ties_to_odd, [C.test_e4m3_block_scale_vs_fraction_brute_force,
                                      C.test_e2m1_constructed_ties_and_midpoints]),
    ("E2M1_MAG_GRID", np.array([0, .5, 1, 1.5, 2, 3, 4, 5.0]), [C.test_e2m1_table_matches_hand_enumeration_and_max6]),
    ("quantize_rows", _quantize_absmax_to_4, [C.test_quantize_rows_vs_fraction_brute_force_random_rows]),
    ("quantize_rows", _quantize_swapped_nibbles, [C.test_quantize_rows_vs_fraction_brute_force_random_rows]),
    ("hadamard_butterfly_fp32", _butterfly_wrong_sign, [T.test_butterfly_unit_vectors_equal_dense_columns]),
    ("key_transform", _key_transform_times_s, [T.test_smoothing_preserves_scores_up_to_rounding]),
    ("calibrate", _calibrate_keep_pos0, [T.test_calibrate_excludes_position0_and_rounds_exactly]),
    ("attention", _attention_wrong_group, [T.test_attention_matches_torch_sdpa_fp64]),
    ("dequantize", _dequant_drop_g, [C.test_dequantize_exact_and_roundtrip_error_bound]),
    ("causal_attention", _causal_sees_one_less, [T.test_causal_attention_matches_torch_sdpa_fp64,
                                                 T.test_causal_attention_special_cases]),
    ("causal_attention", _causal_wrong_offset, [T.test_causal_attention_matches_torch_sdpa_fp64]),
    ("mse_block_sse", _mse_sse_drops_flushed, [M.test_mse_scale_vs_fraction_brute_force_random_blocks]),
    ("MSE_RATIO_HI", 6.0, [M.test_mse_scale_vs_fraction_brute_force_random_blocks,
                           M.test_mse_candidates_are_one_run_near_the_absmax_code]),
    ("MSE_RATIO_LO", 1.5, [M.test_mse_scale_vs_fraction_brute_force_random_blocks,
                           M.test_mse_candidates_are_one_run_near_the_absmax_code]),
    ("mse_scale_codes", _mse_ties_to_last, [M.test_mse_worked_example_with_tie]),
    ("mse_candidates", _mse_candidates_without_absmax, [M.test_mse_scale_vs_fraction_brute_force_random_blocks,
                                                        M.test_mse_special_cases]),
    ("klt_basis", _klt_uncentred, [K.test_klt_basis_closed_form_hadamard_columns]),
    ("klt_basis", _klt_ascending, [K.test_klt_basis_closed_form_hadamard_columns]),
    ("klt_basis", _klt_largest_negative, [K.test_klt_basis_closed_form_hadamard_columns,
                                          K.test_diagonal_covariance_gives_an_exact_permutation]),
    ("rotate_fp32", _rotate_transposed, [K.test_rotation_order_vs_exact_rationals]),
    ("rotate_fp32", _rotate_two_roundings, [K.test_rotation_order_vs_exact_rationals]),
    ("query_transform", _query_basis_not_transposed,
     [lambda: K.test_klt_keeps_scores_and_g_is_over_rotated_keys(O.FLAG_KLT)]),
]


@pytest.mark.parametrize("name,mutant,pins", CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(O, name, mutant)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"planted mistake in {name} not caught"
