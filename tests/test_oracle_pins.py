"""Pins for the fp64 CPU oracle: each test fixes the oracle against something
other than itself -- the tutorial's worked example, closed forms, exact rational
results, invariants, special cases and brute force in independent Python code.

Sources:
  [P1] Golden et al., "Is Flash Attention Stable?" (translated page), sec. II-A:
       the attention definition; sec. IV-A: the fp64 "golden value".
  [P3] yadro-code tutorial "How FlashAttention reduces GPU memory traffic":
       safe softmax, online merge, self-checking program, closing exercise.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E = math.e


def load_example():
    with open(os.path.join(GOLDEN, "tutorial_worked_example.json")) as f:
        return json.load(f)


def close(a, b, rel=1e-12, abs_=1e-12):
    return all(math.isclose(x, y, rel_tol=rel, abs_tol=abs_) for x, y in zip(a, b))


# ---------------------------------------------------------------- brute force
def brute_attention(q, k, v, scale, causal=False, mask=None):
    """Independent pure-Python attention for tiny inputs (lists of lists).

    Builds the full score matrix, then each row's softmax with math.fsum; no
    code in common with the C oracle.  Returns (o, lse) as nested lists.
    """
    B, H, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    O = [[[[0.0] * d for _ in range(N)] for _ in range(H)] for _ in range(B)]
    LSE = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            S = [[scale * math.fsum(q[b][h][i][c] * k[b][h][j][c] for c in range(d))
                  for j in range(N)] for i in range(N)]
            for i in range(N):
                cols = [j for j in range(N)
                        if (not causal or j <= i) and (mask is None or mask[b][j] == 0)]
                if not cols:
                    O[b][h][i] = [0.0] * d
                    LSE[b][h][i] = -math.inf
                    continue
                top = max(S[i][j] for j in cols)
                w = {j: math.exp(S[i][j] - top) for j in cols}
                tot = math.fsum(w.values())
                O[b][h][i] = [math.fsum(w[j] * v[b][h][j][c] for j in cols) / tot for c in range(d)]
                LSE[b][h][i] = top + math.log(tot)
    return O, LSE


# ------------------------------------------------- P1: the tutorial's example
def test_worked_example_blocked_equals_unblocked_every_prefix_and_width():
    """[P3] self-checking program: every causal prefix, widths 1, 2, 3, 8."""
    ex = load_example()
    s, vals = ex["scores"], ex["values"]
    for visible in range(1, len(s) + 1):
        ref, ref_lse = oracle.row_softmax(s[:visible], vals[:visible])
        for width in ex["widths"]:
            for order in (0, 1):
                got, got_lse = oracle.row_blocked(s[:visible], vals[:visible], width, order)
                assert close(got, ref, ex["rel_tol"], ex["abs_tol"]), (visible, width, order)
                assert math.isclose(got_lse, ref_lse, rel_tol=1e-15, abs_tol=1e-12)


def test_worked_example_closed_forms():
    """[P3] example, first two prefixes in closed form; all prefixes against
    brute force in stdlib Python.  Scores near 1000 would overflow exp() if the
    maximum were not subtracted (the tutorial's safe-softmax paragraph)."""
    ex = load_example()
    s, vals = ex["scores"], ex["values"]
    out1, lse1 = oracle.row_softmax(s[:1], vals[:1])
    assert list(out1) == [2.0, -1.0] and lse1 == 1000.0          # one visible key: v0 exactly
    out2, lse2 = oracle.row_softmax(s[:2], vals[:2])
    assert close(out2, [2 / (1 + E), (3 * E - 1) / (1 + E)], 1e-14, 1e-14)
    assert math.isclose(lse2, 1001 + math.log1p(math.exp(-1)), rel_tol=1e-15)
    for visible in range(1, 6):
        w = [math.exp(x - 1004.0) for x in s[:visible]]
        tot = math.fsum(w)
        want = [math.fsum(wi * vals[j][c] for j, wi in enumerate(w)) / tot for c in range(2)]
        got, lse = oracle.row_softmax(s[:visible], vals[:visible])
        assert close(got, want, 1e-13, 1e-13)
        assert math.isclose(lse, 1004.0 + math.log(tot), rel_tol=1e-15)


# -------------------------------------------- P2: averaging block softmaxes
def test_averaging_block_softmaxes_is_wrong():
    """[P3] the wrong merge: averaging per-block results gives exactly 0.5; the
    whole row gives 1/(1 + e^-100) > 0.999, lse = 100 + ln 2 + ln(1 + e^-100)."""
    ex = load_example()["averaging_example"]
    s, vals = ex["scores"], ex["values"]
    whole, lse = oracle.row_softmax(s, vals)
    parts = [oracle.row_softmax([s[j] for j in blk], [vals[j] for j in blk])[0][0] for blk in ex["blocks"]]
    wrong = (parts[0] + parts[1]) / 2
    assert whole[0] > ex["whole_greater_than"]
    assert wrong == ex["wrong_average_equals"]
    assert math.isclose(whole[0], 1 / (1 + math.exp(-100)), rel_tol=1e-15)
    assert math.isclose(lse, 100 + math.log(2) + math.log1p(math.exp(-100)), rel_tol=1e-15)
    for width in (1, 2, 3, 4):
        got, got_lse = oracle.row_blocked(s, vals, width)
        assert math.isclose(got[0], whole[0], rel_tol=1e-15) and math.isclose(got_lse, lse, rel_tol=1e-15)


# ------------------------------------------------ P3: the rescale mutation
def test_dropping_the_rescale_is_caught():
    """[P3] closing exercise: with the rescale removed, the shortest failing row
    is two scores with a rising maximum, e.g. [0, 1] with values [0], [1] at
    width 1: the correct value is e/(1+e), the mutant gives 1/2."""
    good, _ = oracle.row_blocked([0.0, 1.0], [[0.0], [1.0]], 1, rescale=True)
    bad, _ = oracle.row_blocked([0.0, 1.0], [[0.0], [1.0]], 1, rescale=False)
    assert math.isclose(good[0], E / (1 + E), rel_tol=1e-15)
    assert bad[0] == 0.5
    # a falling maximum never needs the rescale, so the mutant agrees there
    good2, _ = oracle.row_blocked([1.0, 0.0], [[0.0], [1.0]], 1, rescale=True)
    bad2, _ = oracle.row_blocked([1.0, 0.0], [[0.0], [1.0]], 1, rescale=False)
    assert good2[0] == bad2[0]
    # a single block (width >= n) never rescales either
    one, _ = oracle.row_blocked([0.0, 1.0], [[0.0], [1.0]], 2, rescale=False)
    assert math.isclose(one[0], E / (1 + E), rel_tol=1e-15)
    # visited in descending block order the same row has a falling maximum, so
    # the mutant is right there: this also shows `order` really reverses blocks
    desc, _ = oracle.row_blocked([0.0, 1.0], [[0.0], [1.0]], 1, order=1, rescale=False)
    assert math.isclose(desc[0], E / (1 + E), rel_tol=1e-15)


def test_descending_tile_order_is_a_different_fold():
    """Tensor level: both tile orders agree to 1e-12 yet are not bitwise equal
    on random data, so the order switch changes the fold and nothing else."""
    rng = np.random.default_rng([7, 3])
    q, k, v = (rng.standard_normal((1, 2, 64, 8)) for _ in range(3))
    a, la = oracle.attn_blocked(q, k, v, 0.5, 4, 0)
    b, lb = oracle.attn_blocked(q, k, v, 0.5, 4, 1)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    assert not np.array_equal(a, b)


# ------------------------------------------------------ P4, P5: invariants
def test_block_order_permutation_and_shift_invariance():
    """[P3] exercise: reordering the blocks keeps the result within rounding;
    [P3] safe softmax: shifting every score by c keeps the output, adds c to lse."""
    rng = np.random.default_rng([7, 1])
    for n in (1, 2, 5, 17, 64):
        s = rng.standard_normal(n) * 3
        vals = rng.standard_normal((n, 3))
        ref, ref_lse = oracle.row_softmax(s, vals)
        for width in (1, 2, 3, 8, 100):
            for order in (0, 1):
                got, got_lse = oracle.row_blocked(s, vals, width, order)
                assert close(got, ref) and math.isclose(got_lse, ref_lse, rel_tol=1e-13, abs_tol=1e-13)
        shifted, sh_lse = oracle.row_softmax(s + 1000.0, vals)
        assert close(shifted, ref, 1e-12, 1e-12)
        assert math.isclose(sh_lse, ref_lse + 1000.0, rel_tol=1e-14)


# -------------------------------------------- exact rational pin (log weights)
def test_log_weight_scores_give_the_exact_rational_average():
    """Closed form: if s_j = ln(w_j) + c with integer weights w_j, softmax(s) = w / sum(w)
    exactly, so the output is the rational sum w_j v_j / sum w_j (computed with
    fractions.Fraction) and lse = c + ln(sum w)."""
    rng = np.random.default_rng([7, 2])
    for n in (1, 3, 9, 40):
        w = [int(x) for x in rng.integers(1, 50, n)]
        vals = [[int(x) for x in row] for row in rng.integers(-9, 10, (n, 2))]
        c = -37.5
        s = [math.log(x) + c for x in w]
        tot = sum(w)
        want = [float(sum(Fraction(w[j] * vals[j][col]) for j in range(n)) / tot) for col in range(2)]
        got, lse = oracle.row_softmax(s, vals)
        assert close(got, want, 1e-13, 1e-13)
        assert math.isclose(lse, c + math.log(tot), rel_tol=1e-14)
        for width in (1, 4):
            gb, lb = oracle.row_blocked(s, vals, width, 1)
            assert close(gb, want, 1e-13, 1e-13)


# --------------------------------------------------- tensor-level brute force
def small_int_problem(seed, B, H, N, d):
    rng = np.random.default_rng([11, seed])
    q = rng.integers(-3, 4, (B, H, N, d)).astype(np.float64)
    k = rng.integers(-3, 4, (B, H, N, d)).astype(np.float64)
    v = rng.integers(-5, 6, (B, H, N, d)).astype(np.float64)
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("use_mask", [False, True])
def test_tensor_oracle_matches_brute_force(causal, use_mask):
    """[P1] sec. II-A definition on tiny tensors (N <= 8, d <= 4, small integers)
    against independent stdlib Python; Q and K differ, so a transposed product,
    a dropped scale, a wrong value row or a misplaced mask all fail."""
    for seed, (B, H, N, d) in enumerate([(1, 1, 1, 1), (2, 2, 5, 3), (1, 3, 8, 4), (2, 1, 7, 2)]):
        q, k, v = small_int_problem(seed, B, H, N, d)
        mask = None
        if use_mask:
            mask = (np.random.default_rng([12, seed]).random((B, N)) < 0.3).astype(np.uint8)
            mask[0, 0] = 1
        scale = 0.5
        o, lse = oracle.attn(q, k, v, scale, causal, mask)
        bo, blse = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, causal,
                                   None if mask is None else mask.tolist())
        np.testing.assert_allclose(o, np.array(bo), rtol=1e-13, atol=1e-13)
        bl = np.array(blse)
        assert np.array_equal(np.isinf(lse), np.isinf(bl))
        np.testing.assert_allclose(lse[np.isfinite(bl)], bl[np.isfinite(bl)], rtol=1e-14, atol=1e-13)
        for bc in (1, 2, 3, 8):
            for order in (0, 1):
                ob, lb = oracle.attn_blocked(q, k, v, scale, bc, order, causal, mask)
                np.testing.assert_allclose(ob, o, rtol=1e-12, atol=1e-12)
                assert np.array_equal(np.isinf(lb), np.isinf(lse))


def test_lse_against_fsum():
    """lse = ln sum_j exp(s_j) for moderate scores, summed directly with math.fsum."""
    rng = np.random.default_rng([13, 0])
    q = rng.standard_normal((1, 2, 9, 4))
    k = rng.standard_normal((1, 2, 9, 4))
    v = rng.standard_normal((1, 2, 9, 4))
    _, lse = oracle.attn(q, k, v, 0.7)
    for h in range(2):
        for i in range(9):
            s = [0.7 * math.fsum(q[0, h, i, c] * k[0, h, j, c] for c in range(4)) for j in range(9)]
            assert math.isclose(lse[0, h, i], math.log(math.fsum(math.exp(x) for x in s)), rel_tol=1e-14)


# ------------------------------------------------------- special cases
def test_equal_scores_give_the_mean_of_v():
    """Q = 0 makes every score equal, so the output is the plain mean of the
    visible value rows (exact rational mean via Fraction)."""
    rng = np.random.default_rng([14, 0])
    B, H, N, d = 1, 2, 6, 3
    q = np.zeros((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.integers(-9, 10, (B, H, N, d)).astype(np.float64)
    o, lse = oracle.attn(q, k, v, 0.125, causal=True)
    for h in range(H):
        for i in range(N):
            want = [float(sum(Fraction(v[0, h, j, c]) for j in range(i + 1)) / (i + 1)) for c in range(d)]
            np.testing.assert_allclose(o[0, h, i], want, rtol=1e-15, atol=1e-15)
            assert math.isclose(lse[0, h, i], math.log(i + 1), rel_tol=1e-15, abs_tol=1e-15)


def test_single_visible_key_returns_its_value_bitwise():
    """[P3] a single visible position: causal row 0, and N = 1, return v_0 exactly."""
    rng = np.random.default_rng([15, 0])
    q, k, v = (rng.standard_normal((2, 3, 5, 4)) for _ in range(3))
    o, lse = oracle.attn(q, k, v, 0.3, causal=True)
    assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :])
    s0 = 0.3 * np.einsum("bhc,bhc->bh", q[:, :, 0], k[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], s0, rtol=1e-15, atol=1e-15)
    o1, _ = oracle.attn(q[:, :, :1], k[:, :, :1], v[:, :, :1], 0.3)
    assert np.array_equal(o1, v[:, :, :1])


def test_fully_masked_rows_are_zero_and_minus_inf():
    """A row with nothing visible outputs +0.0 and lse = -inf (bit patterns), and
    no NaN appears anywhere; the blocked forms agree, in both orders."""
    rng = np.random.default_rng([16, 0])
    q, k, v = (rng.standard_normal((3, 2, 6, 4)) for _ in range(3))
    mask = np.zeros((3, 6), np.uint8)
    mask[1, :] = 1          # whole sequence padded
    mask[2, 0] = 1          # with causal: only query row 0 of batch 2 sees nothing
    for fn in (lambda: oracle.attn(q, k, v, 0.5, True, mask),
               lambda: oracle.attn_blocked(q, k, v, 0.5, 2, 0, True, mask),
               lambda: oracle.attn_blocked(q, k, v, 0.5, 2, 1, True, mask),
               lambda: oracle.attn_blocked(q, k, v, 0.5, 4, 1, True, mask, kv_outer=True)):
        o, lse = fn()
        assert not np.isnan(o).any() and not np.isnan(lse).any()
        zero_rows = [(1, h, i) for h in range(2) for i in range(6)] + [(2, h, 0) for h in range(2)]
        for (b, h, i) in zero_rows:
            assert o[b, h, i].view(np.uint64).tolist() == [0] * 4      # +0.0 exactly
            assert lse[b, h, i] == -np.inf
        assert np.isfinite(lse[0]).all() and np.isfinite(lse[2, :, 1:]).all()


def test_sentinel_trap_scores_far_below_minus_50000():
    """[P1 page, FlashInfer note] a finite mask sentinel of -50,000 is wrong when
    valid scores are smaller.  Valid scores here sit near -60,000 (log weights
    shifted), masked keys must get no weight at all: exact rational result."""
    w = [3, 1, 4, 1, 5]
    masked = [1, 0, 1, 0, 0, 1, 0, 0]      # 8 keys, 5 visible
    N, d = len(masked), 2
    vis_idx = [j for j in range(N) if not masked[j]]
    q = np.zeros((1, 1, N, d)); k = np.zeros((1, 1, N, d)); v = np.zeros((1, 1, N, d))
    q[0, 0, :, 0] = 1.0
    rng = np.random.default_rng([17, 0])
    v[0, 0] = rng.integers(-9, 10, (N, d))
    for t, j in enumerate(vis_idx):
        k[0, 0, j, 0] = math.log(w[t]) - 60000.0
    for j in range(N):
        if masked[j]:
            k[0, 0, j, 0] = -50000.0 + 7.0        # would dominate under a -50,000 sentinel
    mask = np.array([masked], np.uint8)
    o, lse = oracle.attn(q, k, v, 1.0, False, mask)
    tot = sum(w)
    for c in range(d):
        want = float(sum(Fraction(w[t]) * Fraction(v[0, 0, j, c]) for t, j in enumerate(vis_idx)) / tot)
        np.testing.assert_allclose(o[0, 0, :, c], want, rtol=1e-10, atol=1e-10)


def test_constant_value_rows_and_linearity():
    """V = 1 gives O = 1 on every row with a visible key (convex combination);
    O(aV + b) = a O(V) + b."""
    rng = np.random.default_rng([18, 0])
    q, k, v = (rng.standard_normal((2, 2, 9, 5)) for _ in range(3))
    o1, _ = oracle.attn(q, k, np.ones_like(v), 0.4, causal=True)
    np.testing.assert_allclose(o1, 1.0, rtol=0, atol=4e-16)
    o, _ = oracle.attn(q, k, v, 0.4, causal=True)
    o2, _ = oracle.attn(q, k, 2.5 * v - 1.25, 0.4, causal=True)
    np.testing.assert_allclose(o2, 2.5 * o - 1.25, rtol=1e-12, atol=1e-12)


def test_joint_key_value_permutation_leaves_output_unchanged():
    """Without causal mask or padding, permuting the key rows and the value rows
    together leaves every output row unchanged."""
    rng = np.random.default_rng([19, 0])
    q, k, v = (rng.standard_normal((1, 2, 11, 4)) for _ in range(3))
    perm = rng.permutation(11)
    o, lse = oracle.attn(q, k, v, 0.6)
    op, lsep = oracle.attn(q, k[:, :, perm], v[:, :, perm], 0.6)
    np.testing.assert_allclose(op, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lsep, lse, rtol=1e-14, atol=1e-14)


def test_causal_row_equals_unmasked_attention_over_its_prefix():
    """[P3] program comment: the causal mask is the prefix 0..i of row i."""
    rng = np.random.default_rng([20, 0])
    q, k, v = (rng.standard_normal((1, 2, 10, 3)) for _ in range(3))
    o, lse = oracle.attn(q, k, v, 0.8, causal=True)
    for i in range(10):
        op, lp = oracle.attn(q[:, :, :i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.8)
        np.testing.assert_allclose(o[:, :, i], op[:, :, i], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], lp[:, :, i], rtol=1e-14, atol=1e-14)


def test_loop_nest_swap_is_bitwise_neutral_in_fp64():
    """Key-tile-outer and query-row-outer nests apply the same operations to each
    row, so their fp64 outputs are bitwise equal (for either tile order)."""
    rng = np.random.default_rng([21, 0])
    q, k, v = (rng.standard_normal((2, 2, 13, 4)) for _ in range(3))
    mask = np.zeros((2, 13), np.uint8); mask[1, 9:] = 1
    for bc in (1, 4, 5, 16):
        for order in (0, 1):
            a = oracle.attn_blocked(q, k, v, 0.5, bc, order, True, mask)
            b = oracle.attn_blocked(q, k, v, 0.5, bc, order, True, mask, kv_outer=True)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rows_subset_matches_full_tensor():
    """The selected-rows entry point gives bitwise the same rows as the full call."""
    rng = np.random.default_rng([22, 0])
    q, k, v = (rng.standard_normal((2, 3, 17, 8)) for _ in range(3))
    mask = np.zeros((2, 17), np.uint8); mask[0, 12:] = 1
    o, lse = oracle.attn(q, k, v, 0.35, True, mask)
    rows = np.array([0, 5, 16, 17, 40, 101])
    orows, lrows = oracle.attn_rows(q, k, v, 0.35, rows, True, mask)
    assert np.array_equal(orows, o.reshape(-1, 8)[rows])
    assert np.array_equal(lrows, lse.reshape(-1)[rows])


def test_bad_arguments_are_rejected():
    with pytest.raises(ValueError):
        oracle.row_blocked([1.0], [[1.0]], 0)
    with pytest.raises(ValueError):
        oracle.attn_rows(np.zeros((1, 1, 2, 2)), np.zeros((1, 1, 2, 2)), np.zeros((1, 1, 2, 2)), 1.0, [4])


# ------------------------------------------------- query block against a key cache
def brute_attention_kv(q, k, v, scale, causal=False, mask=None):
    """Independent pure-Python attention of Nq query rows against Nk keys, the
    causal prefix aligned to the end of the keys (row i sees j <= Nk - Nq + i)."""
    B, H, Nq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Nk = len(k[0][0])
    O, LSE = [], []
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                cols = [j for j in range(Nk) if (not causal or j <= Nk - Nq + i) and (mask is None or mask[b][j] == 0)]
                if not cols:
                    O.append([0.0] * d); LSE.append(-math.inf)
                    continue
                s = {j: scale * math.fsum(q[b][h][i][c] * k[b][h][j][c] for c in range(d)) for j in cols}
                top = max(s.values())
                w = {j: math.exp(s[j] - top) for j in cols}
                tot = math.fsum(w.values())
                O.append([math.fsum(w[j] * v[b][h][j][c] for j in cols) / tot for c in range(d)])
                LSE.append(top + math.log(tot))
    return np.array(O).reshape(B, H, Nq, d), np.array(LSE).reshape(B, H, Nq)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("use_mask", [False, True])
def test_key_cache_oracle_matches_brute_force(causal, use_mask):
    """[P3] prompt vs cache-decoding shapes: Nq != Nk on small integer inputs,
    against independent stdlib Python."""
    for seed, (B, H, Nq, Nk, d) in enumerate([(1, 1, 1, 1, 1), (2, 2, 1, 9, 3), (1, 3, 4, 11, 4), (2, 1, 6, 6, 2)]):
        rng = np.random.default_rng([40, seed])
        q = rng.integers(-3, 4, (B, H, Nq, d)).astype(np.float64)
        k = rng.integers(-3, 4, (B, H, Nk, d)).astype(np.float64)
        v = rng.integers(-5, 6, (B, H, Nk, d)).astype(np.float64)
        mask = None
        if use_mask:
            mask = (rng.random((B, Nk)) < 0.3).astype(np.uint8)
            mask[0, :] = 1 if Nk == 1 else mask[0, :]
        o, lse = oracle.attn_kv(q, k, v, 0.5, causal, mask)
        bo, bl = brute_attention_kv(q.tolist(), k.tolist(), v.tolist(), 0.5, causal,
                                    None if mask is None else mask.tolist())
        np.testing.assert_allclose(o, bo, rtol=1e-13, atol=1e-13)
        assert np.array_equal(np.isinf(lse), np.isinf(bl))
        np.testing.assert_allclose(lse[np.isfinite(bl)], bl[np.isfinite(bl)], rtol=1e-14, atol=1e-13)


def test_cache_decoding_equals_the_tail_of_causal_self_attention():
    """Causal self-attention over a whole sequence and the last Nq rows decoded
    against the full key cache are the same rows ([P3] causal prefix)."""
    rng = np.random.default_rng([41, 0])
    q = rng.standard_normal((2, 2, 40, 8))
    k = rng.standard_normal((2, 2, 40, 8))
    v = rng.standard_normal((2, 2, 40, 8))
    o, lse = oracle.attn(q, k, v, 0.4, True)
    for nq in (1, 3, 40):
        od, ld = oracle.attn_kv(q[:, :, -nq:], k, v, 0.4, True)
        np.testing.assert_allclose(od, o[:, :, -nq:], rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(ld, lse[:, :, -nq:], rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------- gradient
def test_gradient_matches_central_differences():
    """dL/dq, dL/dk, dL/dv of L = sum(dO * O) against central differences of the
    oracle's own forward (fp64, step 1e-6): independent of the gradient formula."""
    rng = np.random.default_rng([42, 0])
    for causal, use_mask in ((False, False), (True, False), (False, True)):
        B, H, N, d = 1, 2, 6, 3
        q, k, v, g = (rng.standard_normal((B, H, N, d)) for _ in range(4))
        mask = None
        if use_mask:
            mask = np.zeros((B, N), np.uint8); mask[0, [1, 4]] = 1
        dq, dk, dv = oracle.attn_bwd(q, k, v, g, 0.6, causal, mask)
        h = 1e-6
        for x, dx in ((q, dq), (k, dk), (v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + h
                op, _ = oracle.attn(q, k, v, 0.6, causal, mask)
                x[idx] = old - h
                om, _ = oracle.attn(q, k, v, 0.6, causal, mask)
                x[idx] = old
                num[idx] = np.sum(g * (op - om)) / (2 * h)
            np.testing.assert_allclose(dx, num, rtol=1e-6, atol=1e-8)


def test_gradient_sum_rules():
    """Rows of P sum to one and rows of dS to zero, so sum_j dV_j = sum_i dO_i
    and (non-causal, unmasked) sum_j dK_j = 0; a fully masked row contributes nothing."""
    rng = np.random.default_rng([43, 0])
    q, k, v, g = (rng.standard_normal((2, 2, 17, 5)) for _ in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, g, 0.4)
    np.testing.assert_allclose(dv.sum(axis=2), g.sum(axis=2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    mask = np.zeros((2, 17), np.uint8); mask[1, :] = 1
    dq, dk, dv = oracle.attn_bwd(q, k, v, g, 0.4, False, mask)
    assert np.all(dq[1] == 0) and np.all(dk[1] == 0) and np.all(dv[1] == 0)


# ------------------------------------------------------- block-sparse visibility
def test_block_mask_matches_brute_force():
    """Block-sparse reading: pair (i, j) visible iff causal/padding allow it and
    its block is on; against the brute-force definition with the equivalent
    element mask built in Python."""
    rng = np.random.default_rng([44, 0])
    B, H, N, d, bs = 2, 2, 11, 3, 4
    q, k, v = (rng.integers(-3, 4, (B, H, N, d)).astype(np.float64) for _ in range(3))
    nb = (N + bs - 1) // bs
    bm = (rng.random((B, H, nb, nb)) < 0.6).astype(np.uint8)
    bm[0, 0, 1, :] = 0                                  # a whole row block off
    for causal in (False, True):
        o, lse = oracle.attn_blockmask(q, k, v, 0.5, bm, bs, causal)
        for b in range(B):
            for h in range(H):
                for i in range(N):
                    cols = [j for j in range(N) if (not causal or j <= i) and bm[b, h, i // bs, j // bs]]
                    if not cols:
                        assert np.all(o[b, h, i] == 0) and lse[b, h, i] == -math.inf
                        continue
                    s = {j: 0.5 * math.fsum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) for j in cols}
                    top = max(s.values())
                    w = {j: math.exp(s[j] - top) for j in cols}
                    tot = math.fsum(w.values())
                    ref = [math.fsum(w[j] * v[b, h, j, c] for j in cols) / tot for c in range(d)]
                    np.testing.assert_allclose(o[b, h, i], ref, rtol=1e-13, atol=1e-13)
                    assert math.isclose(lse[b, h, i], top + math.log(tot), rel_tol=1e-14, abs_tol=1e-13)


def test_all_blocks_on_is_the_dense_definition():
    rng = np.random.default_rng([45, 0])
    q, k, v = (rng.standard_normal((1, 2, 150, 8)) for _ in range(3))
    bm = np.ones((1, 2, 3, 3), np.uint8)
    for causal in (False, True):
        o, l = oracle.attn_blockmask(q, k, v, 0.3, bm, 64, causal)
        od, ld = oracle.attn(q, k, v, 0.3, causal)
        assert np.array_equal(o, od) and np.array_equal(l, ld)
