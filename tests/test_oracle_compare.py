"""Pins of the acceptance checks that judge every GPU result (oracle/compare.py).

The Top-K check enforces the index-set tolerance: the set of positions must equal the
oracle's except at positions whose fp32 score lies within 1e-6 relative of the oracle's K-th
score, with exactly K_eff distinct positions in [0, V) followed by -1 (the index list that
the fused indexer outputs: "Day0 Adaptation and Sparse Attention Optimization for
Long-Sequence LLM Inference", section 4).  The reference row used here is written by hand,
with its ranking, K-th score and band fixed by construction rather than computed by the
oracle, and each plausible wrong answer must be rejected while the right ones pass.

The attention check bounds max |O - O_ref| and, when asked, the log-sum-exp; its LSE branch
treats equal infinities as equal and everything else (opposite infinities, NaN, a gap above
the bound) as a mismatch.
"""
import numpy as np
import pytest

import oracle
from oracle.indexer import IndexerResult

# Hand-built row: V = 12 positions, K = 5.
#   rank: pos 3 (9.0), pos 7 (8.0), pos 0 (7.0), pos 10 (6.0), pos 5 (5.0): K-th score 5.0
#   band |S - 5| <= 5e-6: positions 5 and 9 (both 5.0; the lower position, 5, wins the tie)
#   and 2 (4.999996, just below the K-th score, not selected).
_S =np.array([7.0, 1.0, 4.999996, 9.0, 0.5, 5.0, 2.0, 8.0, 3.0, 5.0, 6.0, 0.0],
              dtype=np.float32)
_SEL = np.array([3, 7, 0, 10, 5])               # rank order; position 9 ties with 5 and loses
_BAND = np.zeros(12, dtype=bool)
_BAND[[2, 5, 9]] = True                          # |S - 5| <= 5e-6 exactly these


def _ref(K=5):
    idx = np.full(K, -1, dtype=np.int64)
    idx[:5] = _SEL
    return IndexerResult(t=0, k_eff=5, idx=idx, S32=_S.copy(), kth=np.float32(5.0), band=_BAND)


def test_hand_built_row_is_consistent_with_its_definition():
    # the hand ranking and band agree with the plain definitions written out here
    order = sorted(range(12), key=lambda s: (-float(_S[s]), s))
    assert order[:5] == _SEL.tolist()
    band = np.abs(_S.astype(np.float64) - 5.0) <= 1e-6 * 5.0
    assert np.array_equal(band, _BAND)


def _check(row, strict=False, K=5):
    return oracle.check_topk_row(np.array(row, dtype=np.int64), _ref(K), strict=strict)


def test_exact_set_in_any_order_passes():
    for row in ([3, 7, 0, 10, 5], [0, 3, 5, 7, 10], [10, 5, 7, 3, 0]):
        c = _check(row, strict=True)
        assert c.ok and c.n_in_band_diff == 0 and c.n_outside_band == 0, c.msgs


def test_exact_set_with_minus_one_tail_passes():
    c = _check([0, 3, 5, 7, 10, -1, -1], K=7)
    assert c.ok, c.msgs


def test_out_of_band_swap_fails():
    # position 10 (score 6.0) replaced by position 8 (score 3.0): both far from the band
    c = _check([3, 7, 0, 8, 5])
    assert not c.ok and c.n_outside_band == 2


def test_one_sided_out_of_band_difference_fails():
    # position 5 (in band) replaced by position 1 (score 1.0, out of band)
    c = _check([3, 7, 0, 10, 1])
    assert not c.ok and c.n_outside_band == 1


def test_duplicate_position_fails():
    c = _check([3, 7, 0, 10, 10])
    assert not c.ok
    assert any("duplicate" in m for m in c.msgs)


def test_position_at_or_above_V_fails():
    assert not _check([3, 7, 0, 10, 12]).ok
    assert not _check([3, 7, 0, 10, 1 << 20]).ok


def test_negative_position_inside_K_eff_fails():
    assert not _check([3, 7, 0, 10, -1]).ok
    assert not _check([3, 7, -5, 10, 5]).ok


def test_non_minus_one_tail_fails():
    c = _check([3, 7, 0, 10, 5, 9, -1], K=7)
    assert not c.ok
    assert any("past K_eff" in m for m in c.msgs)
    assert not _check([3, 7, 0, 10, 5, -1, 0], K=7).ok


def test_in_band_swap_passes_unless_strict():
    # position 5 (the K-th, 5.0) replaced by position 9 (also 5.0) or 2 (4.999996): both in band
    for other in (9, 2):
        c = _check([3, 7, 0, 10, other])
        assert c.ok and c.n_in_band_diff == 2 and c.n_outside_band == 0, c.msgs
        s = _check([3, 7, 0, 10, other], strict=True)
        assert not s.ok and any("strict" in m for m in s.msgs)


def test_check_topk_collects_per_query_failures():
    r0 = _ref()
    r1 = _ref()
    r1.t = 1
    got = np.array([[3, 7, 0, 10, 5], [3, 7, 0, 8, 5]], dtype=np.int64)
    c = oracle.check_topk(got, [r0, r1])
    assert not c.ok and all(m.startswith("query 1") for m in c.msgs)
    assert oracle.check_topk(got[:1], [r0]).ok


# ------------------------------------------------------------------ attention check
def _attn(lse, lse_ref, tol=1e-4):
    O = np.zeros((2, 3))
    return oracle.check_attention(O, O.copy(), 2e-2, np.array(lse, dtype=np.float64),
                                  np.array(lse_ref, dtype=np.float64), tol)


def test_lse_equal_infinities_pass():
    c = _attn([-np.inf, 1.0], [-np.inf, 1.0])
    assert c.ok and c.lse_max_abs == 0.0
    assert _attn([np.inf], [np.inf]).ok


def test_lse_opposite_infinities_fail():
    assert not _attn([np.inf, 1.0], [-np.inf, 1.0]).ok
    assert not _attn([-np.inf], [np.inf]).ok


def test_lse_infinity_against_finite_fails():
    assert not _attn([-np.inf], [3.0]).ok
    assert not _attn([3.0], [-np.inf]).ok


def test_lse_nan_fails():
    assert not _attn([np.nan, 1.0], [0.5, 1.0]).ok
    assert not _attn([0.5], [np.nan]).ok


def test_lse_gap_above_bound_fails_and_below_passes():
    assert not _attn([1.0 + 2e-4], [1.0]).ok
    assert _attn([1.0 + 5e-5], [1.0]).ok


def test_output_bound_and_nan_output():
    O_ref = np.ones((2, 4))
    assert oracle.check_attention(O_ref + 1e-2, O_ref, 2e-2).ok
    assert not oracle.check_attention(O_ref + 3e-2, O_ref, 2e-2).ok
    bad = O_ref.copy()
    bad[1, 2] = np.nan
    c = oracle.check_attention(bad, O_ref, 2e-2)
    assert not c.ok and c.worst == (1, 2)
