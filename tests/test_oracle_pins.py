"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own formulas: exact rational
arithmetic (fractions.Fraction), brute-force enumeration, closed forms,
identities of the review's equations, values worked by hand and stored under
tests/golden/ with their citation, and special cases that reduce to a textbook
routine.  None of these tests touches the GPU or the product library.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import svdq_oracle as O
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# exact nearest-even rounding onto a binary floating-point grid (Fractions)
# ---------------------------------------------------------------------------

def _round_to_grid(x: Fraction, sig_bits: int, emin: int, emax_finite: Fraction):
    """Nearest value with `sig_bits` significant bits (ties to even mantissa).

    emin: exponent of the smallest normal binade; below it the spacing is fixed
    (subnormals).  Returns a Fraction, or +-inf if beyond the largest finite.
    """
    if x == 0:
        return Fraction(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - (sig_bits - 1))
    t = a / q
    fl = t.numerator // t.denominator
    rem = t - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * q
    if v > emax_finite:
        return sgn * math.inf
    return sgn * v


BF16_MAX = Fraction(2) ** 127 * (2 - Fraction(1, 2 ** 7))
FP16_MAX = Fraction(65504)


def _bf16_exact(x):
    return _round_to_grid(Fraction(x), 8, -126, BF16_MAX)


def _fp16_exact(x):
    return _round_to_grid(Fraction(x), 11, -14, FP16_MAX)


# ---------------------------------------------------------------------------
# rounding primitives
# ---------------------------------------------------------------------------

def test_bf16_from_f32_constructed_ties():
    one = 1.0
    cases = [
        (one + 2 ** -8, 1.0),                     # tie -> even (1.0)
        (one + 3 * 2 ** -8, one + 2 ** -6),       # tie -> even (mantissa 2)
        (-(one + 2 ** -8), -1.0),
        (one + 2 ** -8 + 2 ** -20, one + 2 ** -7),  # just above the tie
        (3.0, 3.0),
    ]
    got = O.bf16_from_f32(np.array([c[0] for c in cases], np.float32))
    assert list(got) == [c[1] for c in cases]


def test_bf16_from_f32_matches_exact_rational_rounding():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-30, 30, 4000))).astype(np.float32)
    got = O.bf16_from_f32(x)
    for xi, gi in zip(x, got):
        assert Fraction(float(gi)) == _bf16_exact(float(xi))


def test_bf16_from_f64_single_rounding_matches_exact():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000) * np.exp(rng.uniform(-40, 40, 3000))
    # plus values that are exactly bf16 ties in float64 but not representable in float32
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -40, -(1 + 2 ** -8 - 2 ** -45)])
    x = np.concatenate([x, ties])
    got = O.bf16_from_f64(x)
    for xi, gi in zip(x, got):
        assert Fraction(float(gi)) == _bf16_exact(float(xi)), xi


def test_fp16_from_f32_sat_matches_exact_and_saturates():
    rng = np.random.default_rng(3)
    x = np.abs(rng.standard_normal(3000) * np.exp(rng.uniform(-18, 12, 3000))).astype(np.float32)
    got = O.fp16_from_f32_sat(x)
    for xi, gi in zip(x, got):
        e = _fp16_exact(float(xi))
        e = FP16_MAX if e == math.inf else e
        assert Fraction(float(gi)) == e
    spec = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -25, 3 * 2 ** -25, 65519.0, 65520.0, 1e9],
                    np.float32)
    assert list(O.fp16_from_f32_sat(spec)) == [1.0, 1 + 2 ** -9, 0.0, 2 ** -23, 65504.0, 65504.0,
                                                65504.0]


# ---------------------------------------------------------------------------
# quantizer, Eq.(1)
# ---------------------------------------------------------------------------

def _brute_codes(group_vals, s):
    """argmin over the 15 symmetric codes of |v - s*c|, ties to the even code."""
    out = []
    s = Fraction(float(s))
    for v in group_vals:
        v = Fraction(float(v))
        if s == 0:
            out.append(0)
            continue
        best = None
        for c in range(-7, 8):
            d = abs(v - s * c)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        out.append(best[1])
    return out


def test_quantizer_brute_force_on_bf16_groups():
    rng = np.random.default_rng(4)
    x = workloads.random_bf16_bits(rng, (6, 128), 3.0)
    xv = workloads.bf16_bits_to_f32(x)
    xv[0, :64] = 0.0                       # an all-zero group
    xv[1, 5] = 90.0                        # an outlier
    codes, scales = O.quantize_groups(xv)
    for i in range(xv.shape[0]):
        for g in range(2):
            grp = xv[i, 64 * g:64 * (g + 1)]
            amax = Fraction(float(np.max(np.abs(grp))))
            # s = fp16(fl32(amax/7)): the float32 quotient is the exact quotient rounded
            s_expect = _fp16_exact(float(_round_to_grid(amax / 7, 24, -126, Fraction(2) ** 128)))
            assert Fraction(float(scales[i, g])) == s_expect
            assert list(codes[i, 64 * g:64 * (g + 1)]) == _brute_codes(grp, scales[i, g])


def test_quantizer_constructed_ties_round_to_even():
    # a group whose amax is 7 gets s = 1; v = 2.5 is an exact tie -> 2, 3.5 -> 4, -2.5 -> -2
    grp = np.zeros(64, np.float32)
    grp[:6] = [7.0, 2.5, 3.5, -2.5, 0.5, 1.5]
    codes, s = O.quantize_groups(grp[None, :])
    assert s[0, 0] == 1.0
    assert list(codes[0, :6]) == [7, 2, 4, -2, 0, 2]


def test_quantizer_worked_example_fig2():
    gold = _golden("fig2_worked_example.json")
    for case in gold["cases"]:
        grp = np.full(64, case["pad_to_group_with"], np.float32)
        grp[:len(case["values"])] = case["values"]
        codes, s = O.quantize_groups(grp[None, :])
        assert float(s[0, 0]) == case["expected_scale"]
        assert list(codes[0, :len(case["values"])]) == case["expected_codes"]


def test_quantizer_code_range_zero_underflow_saturation():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((50, 256)) * np.exp(rng.uniform(-5, 5, (50, 1)))).astype(np.float32)
    codes, s = O.quantize_groups(v)
    assert codes.min() >= -7 and codes.max() <= 7
    # the element that sets amax gets |code| 7 (s = fp16(amax/7) is within 2^-11 of amax/7)
    g = v.reshape(50, 4, 64)
    idx = np.argmax(np.abs(g), axis=-1)
    cg = codes.reshape(50, 4, 64)
    assert np.all(np.abs(np.take_along_axis(cg, idx[..., None], -1)) == 7)
    # underflowing group: scale 0, codes 0
    tiny = np.full((1, 64), 1e-9, np.float32)
    c, s0 = O.quantize_groups(tiny)
    assert s0[0, 0] == 0 and np.all(c == 0)
    # saturating group: s = 65504, codes clamp to +-7
    big = np.zeros((1, 64), np.float32)
    big[0, :3] = [1e6, -1e6, 65504.0 * 3]
    c, sb = O.quantize_groups(big)
    assert sb[0, 0] == 65504.0 and list(c[0, :3]) == [7, -7, 3]


def test_quantizer_eq9_bound_per_group():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((40, 64 * 8)).astype(np.float32)
    v[:, 7] *= 40
    codes, s = O.quantize_groups(v)
    deq = O.dequantize_groups(codes, s)
    err = (v.astype(np.float64) - deq).reshape(40, 8, 64)
    vv = v.reshape(40, 8, 64)
    for i in range(40):
        for g in range(8):
            # fp16 rounding of the scale can enlarge the step by at most 2^-11
            assert np.linalg.norm(err[i, g]) <= O.eq9_group_bound(vv[i, g]) * (1 + 2 ** -10)
            assert np.max(np.abs(err[i, g])) <= 0.5 * s[i, g] * (1 + 1e-12)


# ---------------------------------------------------------------------------
# smoothing, Eq.(3)-(4)
# ---------------------------------------------------------------------------

def test_smoothing_lambda_hand_values():
    gold = _golden("smoothing_lambda_examples.json")
    a = np.array(gold["act_amax"], np.float32)
    wmax = np.array(gold["w_row_amax"])
    w = np.zeros((4, 3), np.float32)
    w[:, 1] = -wmax                        # row maxima carried by a negative entry
    for case in gold["cases"]:
        lam, lam32, inv32 = O.smoothing_lambda(a, w, case["alpha"])
        np.testing.assert_allclose(lam, case["lambda"], rtol=1e-15)
        assert np.all(lam32 == np.float32(case["lambda"]))
        assert np.all(inv32 == (1.0 / np.array(case["lambda"])).astype(np.float32))


def test_smoothing_closed_form_and_invariance_eq3():
    inp = workloads.make_inputs("tiny")
    x, w = inp["x"], inp["w"]
    a = O.act_amax(x)
    assert np.all(a == np.max(np.abs(x), axis=0))
    lam, lam32, inv32 = O.smoothing_lambda(a, w, 0.5)
    wmax = np.max(np.abs(w.astype(np.float64)), axis=1)
    np.testing.assert_allclose(lam, np.sqrt(a / wmax), rtol=1e-14)
    # Eq.(3): X D^-1 D W = X W exactly in exact arithmetic
    xs = x.astype(np.float64) / lam32.astype(np.float64)[None, :]
    wt = O.smooth_weight(w, lam32)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    assert np.linalg.norm(xs @ wt - ref) / np.linalg.norm(ref) < 1e-13
    # smoothing flattens the activation outlier channels (the point of sec. 3.1)
    xt = O.smooth_activation(x, inv32)
    amax_t = O.act_amax(xt)
    assert amax_t.max() / np.median(amax_t) < a.max() / np.median(a)


def test_smooth_activation_null_is_identity_on_bf16():
    inp = workloads.make_inputs("tiny")
    assert np.array_equal(O.smooth_activation(inp["x"], None), inp["x"])


# ---------------------------------------------------------------------------
# SVD and residual, Eq.(10)
# ---------------------------------------------------------------------------

def test_truncated_svd_tail_energy_eq10_and_optimality():
    rng = np.random.default_rng(7)
    wt = rng.standard_normal((96, 160))
    wt[3] *= 20
    r = 8
    l1, l2, sig = O.truncated_svd(wt, r)
    res = wt - l1 @ l2
    tail = np.sum(sig[r:] ** 2)
    assert abs(np.linalg.norm(res) ** 2 - tail) / tail < 1e-10
    # Eckart-Young: no other rank-r candidate does better
    for _ in range(5):
        a = rng.standard_normal((96, r))
        # best approximation in the column span of a (projection), still rank r
        q, _ = np.linalg.qr(a)
        assert np.linalg.norm(wt - q @ (q.T @ wt)) ** 2 >= tail
    # independent routine: scipy's ARPACK truncated SVD gives the same top values
    from scipy.sparse.linalg import svds
    s2 = np.sort(svds(wt, k=r, random_state=0)[1])[::-1]
    np.testing.assert_allclose(sig[:r], s2, rtol=1e-9)
    # exact low-rank input: residual vanishes
    lr = rng.standard_normal((96, r)) @ rng.standard_normal((r, 160))
    l1, l2, _ = O.truncated_svd(lr, r)
    assert np.linalg.norm(lr - l1 @ l2) < 1e-10 * np.linalg.norm(lr)


def test_prepare_weights_decomposition_exact_with_stored_factors():
    inp = workloads.make_inputs("tiny")
    a = O.act_amax(inp["x"])
    lay = O.prepare_weights(inp["w"], a, 16)
    # factors are bf16 values
    assert np.array_equal(O.bf16_from_f32(lay["l1"]), lay["l1"])
    assert np.array_equal(O.bf16_from_f32(lay["l2"]), lay["l2"])
    # W~ = L1 L2 + R with the stored factors (reading R8)
    recon = lay["l1"].astype(np.float64) @ lay["l2"].astype(np.float64) + lay["r64"]
    assert np.linalg.norm(recon - lay["wt"]) <= 1e-14 * np.linalg.norm(lay["wt"])
    # residual energy is close to the optimal tail (bf16 factors add a little)
    tail = np.sum(lay["sigma"][16:] ** 2)
    assert np.linalg.norm(lay["r64"]) ** 2 <= tail * 1.01
    # the protected branch removed the dominant directions
    assert np.max(np.abs(lay["r64"])) < 0.5 * np.max(np.abs(lay["wt"]))


# ---------------------------------------------------------------------------
# main branch: per-group integer sums and Eq.(7)
# ---------------------------------------------------------------------------

def test_group_isums_brute_force_loops():
    rng = np.random.default_rng(8)
    qx = rng.integers(-7, 8, (3, 128)).astype(np.int8)
    qw = rng.integers(-7, 8, (128, 4)).astype(np.int8)
    isum = O.group_isums(qx, qw)
    for i in range(3):
        for j in range(4):
            for g in range(2):
                s = 0
                for k in range(64 * g, 64 * g + 64):
                    s += int(qx[i, k]) * int(qw[k, j])
                assert isum[i, j, g] == s
    assert np.abs(isum).max() <= 64 * 49


def test_gemm_main_equals_scaled_group_sums():
    rng = np.random.default_rng(9)
    qx = rng.integers(-7, 8, (5, 192)).astype(np.int8)
    qw = rng.integers(-7, 8, (192, 6)).astype(np.int8)
    sx = O.fp16_from_f32_sat(rng.uniform(0.01, 2, (5, 3)).astype(np.float32))
    sw = O.fp16_from_f32_sat(rng.uniform(0.01, 2, (3, 6)).astype(np.float32))
    isum = O.group_isums(qx, qw)
    y = O.gemm_main(qx, sx, qw, sw)
    for i in range(5):
        for j in range(6):
            ref = sum(Fraction(float(sx[i, g])) * Fraction(float(sw[g, j])) * int(isum[i, j, g])
                      for g in range(3))
            assert abs(Fraction(y[i, j]) - ref) <= abs(ref) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


def test_linear_integer_inputs_make_quantization_exact():
    # every group of X and W holds +-7 and integers in [-7, 7]: scales are 1 and
    # Q is the identity, so rank-0 Y equals X W exactly
    rng = np.random.default_rng(10)
    x = rng.integers(-7, 8, (8, 128)).astype(np.float32)
    w = rng.integers(-7, 8, (128, 12)).astype(np.float32)
    x[:, ::64] = 7
    w[::64, :] = -7
    lay = O.prepare_weights(w, None, 0)
    assert np.all(lay["sw"] == 1.0)
    out = O.linear(x, lay)
    assert np.all(out["sx"] == 1.0)
    assert np.array_equal(out["y"], x.astype(np.float64) @ w.astype(np.float64))


def test_linear_rank0_is_plain_group_quantized_gemm():
    inp = workloads.make_inputs("tiny")
    lay = O.prepare_weights(inp["w"], None, 0)
    out = O.linear(inp["x"], lay)
    qx, sx = O.quantize_groups(inp["x"])
    qw_t, sw_t = O.quantize_groups(np.ascontiguousarray(inp["w"].T))
    ref = O.dequantize_groups(qx, sx) @ O.dequantize_groups(qw_t, sw_t).T
    np.testing.assert_allclose(out["y"], ref, rtol=1e-13, atol=1e-12)


def test_linear_full_rank_leaves_only_rounding_residual():
    rng = np.random.default_rng(11)
    x = workloads.bf16_bits_to_f32(workloads.random_bf16_bits(rng, (16, 64)))
    w = (rng.standard_normal((64, 48)) / 8).astype(np.float32)
    a = O.act_amax(x)
    lay = O.prepare_weights(w, a, 48)
    # R is only the bf16 rounding of the factors
    assert np.linalg.norm(lay["r64"]) < 1e-2 * np.linalg.norm(lay["wt"])
    y = O.linear(x, lay)["y"]
    ref = x.astype(np.float64) @ w.astype(np.float64)
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 1e-2


def test_linear_rows_equals_slice():
    inp = workloads.make_inputs("tiny")
    lay = O.prepare_weights(inp["w"], O.act_amax(inp["x"]), 16)
    full = O.linear(inp["x"], lay)["y"]
    rows = np.array([0, 5, 63])
    cols = np.array([1, 100, 255])
    sub = O.linear_rows(inp["x"][rows], lay, cols)
    np.testing.assert_allclose(sub, full[np.ix_(rows, cols)], rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# LoRA, Eq.(13)
# ---------------------------------------------------------------------------

def test_append_lora_matches_adapter_product():
    rng = np.random.default_rng(12)
    inp = workloads.make_inputs("tiny")
    x, w = inp["x"], inp["w"]
    a = O.act_amax(x)
    lay = O.prepare_weights(w, a, 16)
    A = (rng.standard_normal((256, 4)) * 0.3).astype(np.float32)
    B = (rng.standard_normal((4, 256)) * 0.3).astype(np.float32)
    l1p, l2p = O.append_lora(lay["l1"], lay["l2"], lay["lam32"], A, B, 0.5)
    assert l1p.shape == (256, 20) and l2p.shape == (20, 256)
    assert np.array_equal(l1p[:, :16], lay["l1"]) and np.array_equal(l2p[:16], lay["l2"])
    lay2 = dict(lay, l1=l1p, l2=l2p)
    dy = O.linear(x, lay2)["y"] - O.linear(x, lay)["y"]
    ref = 0.5 * (x.astype(np.float64) @ A.astype(np.float64)) @ B.astype(np.float64)
    assert np.linalg.norm(dy - ref) / np.linalg.norm(ref) < 1e-2


# ---------------------------------------------------------------------------
# error analysis, Eq.(5)-(6), and the direction of the pages' claims
# ---------------------------------------------------------------------------

def test_eq5_identity_and_eq6_bound():
    inp = workloads.make_inputs("tiny")
    x = inp["x"].astype(np.float64)
    w = inp["w"].astype(np.float64)
    qx, sx = O.quantize_groups(inp["x"])
    qw, sw = O.quantize_weight_residual(inp["w"])
    xq = O.dequantize_groups(qx, sx)
    wq = O.dequantize_groups(np.ascontiguousarray(qw.T), np.ascontiguousarray(sw.T)).T
    lhs = x @ w - xq @ wq
    rhs = x @ (w - wq) + (x - xq) @ wq
    assert np.linalg.norm(lhs - rhs) <= 1e-12 * np.linalg.norm(lhs)
    assert np.linalg.norm(lhs) <= O.prop41_bound(x, w, xq, wq)


@pytest.mark.parametrize("cfg_name", ["tiny"])
def test_svdquant_reduces_output_error_direction(cfg_name):
    inp = workloads.make_inputs(cfg_name)
    x, w = inp["x"], inp["w"]
    a = O.act_amax(x)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    lay = O.prepare_weights(w, a, 16)
    e_svdq = np.linalg.norm(O.linear(x, lay)["y"] - ref)
    e_smooth = np.linalg.norm(O.smoothed_w4a4_no_branch(x, w, a) - ref)
    e_naive = np.linalg.norm(O.naive_w4a4(x, w) - ref)
    e_fix = np.linalg.norm(O.lowrank_fix_of_quant_error(x, w, a, 16) - ref)
    assert e_svdq < e_smooth < e_naive
    assert e_svdq < e_fix


# ---------------------------------------------------------------------------
# accounting, Eq.(11)-(12)
# ---------------------------------------------------------------------------

def test_accounting_matches_printed_example():
    gold = _golden("accounting_eq11_eq12.json")
    m, n, r = gold["m"], gold["n"], gold["rank"]
    assert O.mac_ratio(m, n, r) == gold["mac_ratio"]
    assert O.storage_ratio(m, n, r) == gold["storage_ratio"]
    assert round(1 / O.storage_ratio(m, n, r), 2) == gold["compression_approx"]


# ---------------------------------------------------------------------------
# candidate search and refinement of Algorithm 1 steps 6-8 (readings R16, R17)
# ---------------------------------------------------------------------------

def _refine_case(m=128, n=96, b=48, seed=21):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, m))
    x[:, rng.choice(m, 3, replace=False)] *= 30
    x32 = workloads.bf16_bits_to_f32(workloads.bf16_bits_of(x.astype(np.float32)))
    w = (rng.standard_normal((m, n)) / np.sqrt(m)).astype(np.float32)
    return x32, w


def test_layer_output_error_zero_when_quantization_is_exact():
    """Integer activations and weights whose groups each reach 7 quantize
    exactly (scale 1); without smoothing and with rank 0 the layer output is
    X W, so the error is 0; scaling W by 2 in one column makes it computable by
    hand."""
    rng = np.random.default_rng(2)
    m, n, b = 128, 16, 8
    x = rng.integers(-7, 8, (b, m)).astype(np.float32)
    x[:, ::64] = 7
    w = rng.integers(-7, 8, (m, n)).astype(np.float32)
    w[::64, :] = 7
    lay = O.prepare_weights(w, None, 0)
    assert O.layer_output_error(x, w, lay) == 0.0
    # a layer built for W, scored against 2 W: Y = X W, reference 2 X W -> error 1/2
    assert abs(O.layer_output_error(x, 2 * w, lay) - 0.5) < 1e-15


def test_refine_reduces_to_prepare_weights():
    x32, w = _refine_case()
    a = O.act_amax(x32)
    got = O.refine_weights(w, a, x32, 16, alphas=(0.5,), iters=0)
    ref = O.prepare_weights(w, a, 16)
    for k in ("qw", "sw", "l1", "l2", "lam32", "inv32"):
        assert np.array_equal(got[k], ref[k]), k
    assert got["iteration"] == 0 and got["candidates"] == [(0.5, 0, got["rel_err"])]


def test_refine_keeps_the_lowest_scoring_candidate():
    """The kept candidate has the lowest score of all candidates (first of equals),
    each score re-evaluated here from a layer built independently."""
    x32, w = _refine_case()
    a = O.act_amax(x32)
    alphas = (0.3, 0.5, 0.7)
    got = O.refine_weights(w, a, x32, 16, alphas=alphas, iters=2)
    scores = []
    for al in alphas:
        # the C ABI takes the strengths as float: the oracle rounds them the same way
        lay = O.prepare_weights(w, a, 16, alpha=float(np.float32(al)))
        for it in range(3):
            scores.append(O.layer_output_error(x32, w, lay))
            lay = O.refit_factors(lay)
    assert [c[2] for c in got["candidates"]] == scores
    k = int(np.argmin(scores))
    assert got["rel_err"] == scores[k]
    assert (got["alpha"], got["iteration"]) == (float(np.float32(alphas[k // 3])), k % 3)
    assert got["rel_err"] <= scores[1 * 3 + 0]      # never worse than alpha = 0.5, no refinement


def test_refit_factors_is_the_best_rank1_fit_by_power_iteration():
    """Step 6 at rank 1: the refitted factor product is the top singular pair
    of W~ - Q(R), here found independently by power iteration (then rounded to
    bf16 like the stored factors)."""
    x32, w = _refine_case(m=64, n=40)
    lay = O.prepare_weights(w, O.act_amax(x32), 1)
    target = lay["wt"] - O.dequantize_weight_residual(lay["qw"], lay["sw"])
    v = np.ones(target.shape[1])
    for _ in range(500):
        v = target.T @ (target @ v)
        v /= np.linalg.norm(v)
    u = target @ v                       # = sigma_1 u_1
    best = np.outer(u, v)
    new = O.refit_factors(lay)
    prod = new["l1"].astype(np.float64) @ new["l2"].astype(np.float64)
    assert np.linalg.norm(prod - best) <= 1e-2 * np.linalg.norm(best)   # bf16 factors: ~2^-9 each
    # and the residual is formed from the new stored factors
    assert np.array_equal(new["r64"], lay["wt"] - prod)


# ---------------------------------------------------------------------------
# the 8-bit setting (reading R19)
# ---------------------------------------------------------------------------

def test_quantize_rows8_brute_force():
    """Each code is the argmin over -127..127 of |v - s q| (ties to even), with
    s the exact-rational nearest fp16 of fl32(amax / 127)."""
    rng = np.random.default_rng(8)
    v = O.bf16_from_f32((rng.standard_normal((6, 96)) * rng.uniform(0.01, 50, (6, 1))).astype(np.float32))
    v[0, :4] = [12.5, -12.5, 0.0, 127.0]
    q, s = O.quantize_rows8(v)
    for i in range(v.shape[0]):
        amax = Fraction(float(np.max(np.abs(v[i]))))
        s_f32 = _round_to_grid(amax / 127, 24, -126, Fraction(2) ** 128)
        s_exact = _round_to_grid(s_f32, 11, -14, Fraction(65504))
        assert Fraction(float(s[i])) == s_exact
        for k in range(v.shape[1]):
            quot = _round_to_grid(Fraction(float(v[i, k])) / s_exact, 24, -126, Fraction(2) ** 128)
            best = min(range(-127, 128), key=lambda c: (abs(quot - c), c % 2))
            assert q[i, k] == best


def test_w8a8_linear_integer_inputs_are_exact_and_rank0_is_plain_int8_gemm():
    rng = np.random.default_rng(9)
    # integers with each row / column reaching 127: scales are 1 and Q is exact
    x = rng.integers(-127, 128, (6, 128)).astype(np.float32)
    x[:, 0] = 127
    w = rng.integers(-127, 128, (128, 10)).astype(np.float32)
    w[0, :] = -127
    lay = O.prepare_weights_w8a8(w, None, 0)
    out = O.linear_w8a8(x, lay)
    assert np.all(out["sx"] == 1) and np.all(lay["sw"] == 1)
    assert np.array_equal(out["y"], x.astype(np.float64) @ w.astype(np.float64))
    # rank 0 on general inputs: dequantized per-token x per-channel product
    inp = workloads.make_inputs("tiny")
    lay = O.prepare_weights_w8a8(inp["w"], None, 0)
    out = O.linear_w8a8(inp["x"], lay)
    qx, sx = O.quantize_rows8(inp["x"])
    qw_t, sw = O.quantize_rows8(np.ascontiguousarray(inp["w"].T))
    ref = (qx * sx[:, None].astype(np.float64)) @ (qw_t * sw[:, None].astype(np.float64)).T
    np.testing.assert_allclose(out["y"], ref, rtol=1e-13, atol=1e-12)


def test_w8a8_error_below_w4a4_on_an_outlier_layer():
    """Direction only (the pages give no margin): eight bits per value leave a
    smaller output error than four on the same synthetic outlier layer."""
    inp = workloads.make_inputs("tiny")
    x, w = inp["x"], inp["w"]
    a = O.act_amax(x)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    e8 = np.linalg.norm(O.linear_w8a8(x, O.prepare_weights_w8a8(w, a, 16))["y"] - ref)
    e4 = np.linalg.norm(O.linear(x, O.prepare_weights(w, a, 16))["y"] - ref)
    assert e8 < e4


# ---------------------------------------------------------------------------
# the NVFP4 setting (reading R20)
# ---------------------------------------------------------------------------

def _e4m3_by_rationals(x: Fraction) -> Fraction:
    """4 significant bits, smallest normal binade 2^-6, saturation at 448."""
    v = _round_to_grid(x, 4, -6, Fraction(448))
    return Fraction(448) if v == math.inf else v


def test_e4m3_round_matches_rational_rounding_and_bit_patterns():
    # every finite non-negative E4M3 value decodes, encodes and rounds to itself
    vals = O.e4m3_from_bits(np.arange(0x7F))
    assert vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6 and vals[0x7E] == 448.0
    assert np.array_equal(O.e4m3_bits(vals), np.arange(0x7F, dtype=np.uint8))
    assert np.array_equal(O.e4m3_round(vals), vals)
    # midpoints (ties), their neighbours, random magnitudes and values past the range
    mids = (vals[1:] + vals[:-1]) / 2
    rng = np.random.default_rng(20)
    xs = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                         np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), 3000)), [0.0, 449.0, 1e6]])
    xs = xs.astype(np.float32).astype(np.float64)
    got = O.e4m3_round(xs)
    for x, g in zip(xs, got):
        assert Fraction(float(g)) == _e4m3_by_rationals(Fraction(float(x))), x


def _e2m1_by_thresholds(y: float) -> int:
    """Independent form of the E2M1 rounding: count the midpoints below |y|;
    a quotient exactly on a midpoint goes to the even code (up at 0.75, 1.75,
    3.5; down at 0.25, 1.25, 2.5, 5)."""
    a = abs(y)
    up_on_tie = {0.75, 1.75, 3.5}
    idx = sum(1 for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0) if a > t or (a == t and t in up_on_tie))
    return idx + (8 if math.copysign(1.0, y) < 0 else 0)


def test_e2m1_codes_match_threshold_form_on_every_bf16_and_the_ties():
    bits = np.arange(0x10000, dtype=np.uint32)
    ys = (bits << 16).view(np.float32)
    ys = ys[np.isfinite(ys) & (np.abs(ys) <= 16)]
    extra = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    ys = np.concatenate([ys, extra, -extra, np.nextafter(extra, np.float32(0)), np.nextafter(extra, np.float32(9))])
    got = O.e2m1_codes(ys)
    want = np.array([_e2m1_by_thresholds(float(y)) for y in ys])
    assert np.array_equal(got, want)
    assert np.array_equal(O.e2m1_values(np.arange(16)),
                          [0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])


def test_fp4_block_quantizer_hand_example():
    """Two blocks worked by hand at t = 1.
    Block 0: amax 6 -> fl32(6/6) = 1 -> sb = 1, S = 1; the codes are the grid
    roundings of the values themselves.
    Block 1: amax 0.9 -> fl32(0.9/6) = 0.15 (fl32) lies in [2^-3, 2^-2), E4M3
    quantum 2^-6: 0.15 / 2^-6 = 9.6 -> 10 -> sb = 0.15625; 0.9 / S = 5.76 -> 6."""
    b0 = [6, -3, 1.3, 0.2, 0.26, -0.75, 2.5, 5, 0, -0.0, 1.75, 3.5, -5.5, 0.25, 1.25, -6]
    b1 = [0.9, -0.1, 0.2, 0.0] + [0.05] * 12
    v = np.array([b0 + b1], np.float32)
    codes, sb = O.quantize_fp4_blocks(v, 1.0)
    assert sb.tolist() == [[1.0, 0.15625]]
    want0 = [7, 13, 3, 0, 1, 10, 4, 6, 0, 8, 4, 6, 15, 0, 2, 15]
    # block 1: 0.9/S = 5.76 -> 6 (7); -0.1/S = -0.64 -> -0.5 (9); 0.2/S = 1.28 -> 1.5 (3);
    # 0 -> 0; 0.05/S = 0.32 -> 0.5 (1)
    want1 = [7, 9, 3, 0] + [1] * 12
    assert codes[0].tolist() == want0 + want1
    # a zero block and a block whose scale underflows E4M3 give code 0 everywhere
    z = np.zeros((1, 32), np.float32)
    z[0, 16:] = 1e-6
    cz, sz = O.quantize_fp4_blocks(z, 1.0)
    assert sz.tolist() == [[0.0, 0.0]] and not cz.any()


def test_fp4_codes_within_half_a_grid_step():
    """|v/S - value(code)| is at most half the grid spacing at |v/S| (0.25 below
    2, 0.5 below 4, 1 above), or the overshoot past 6 when sb rounded down."""
    rng = np.random.default_rng(21)
    v = (rng.standard_normal((40, 64)) * np.exp(rng.uniform(-8, 4, (40, 1)))).astype(np.float32)
    t = O.fp4_tensor_scale(np.max(np.abs(v)))
    codes, sb = O.quantize_fp4_blocks(v, t)
    S = np.repeat(sb * t, 16, axis=-1)
    ok = S > 0
    y = np.abs(v.astype(np.float64)[ok] / S[ok])
    err = np.abs(y - np.abs(O.e2m1_values(codes[ok])))
    half = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    assert np.all(err <= np.maximum(half, y - 6.0) + 1e-12)
    # E4M3 rounding moves the block scale by at most half a quantum: 2^-4
    # relative for normal scales, 2^-10 t absolute for subnormal ones
    amax_b = np.max(np.abs(v.reshape(40, 4, 16)), -1).astype(np.float64)
    assert np.all(np.abs(sb * t - amax_b / 6) <= np.maximum(amax_b / 6 * 2 ** -4, 2 ** -10 * t) * (1 + 1e-6))


def test_fp4_linear_exact_when_blocks_sit_on_the_grid():
    """Rank 0, no smoothing; every 16-block of X and of each column of W holds
    grid values times one power of two and reaches 6 * 2^k, so every block
    scale is 2^k / t exactly and Q loses nothing: Y = X W exactly."""
    rng = np.random.default_rng(22)
    def grid_blocks(rows, K):
        v = O.E2M1_VALUES[rng.integers(0, 8, (rows, K))] * rng.choice([-1.0, 1.0], (rows, K))
        v[:, ::16] = 6.0
        return v * np.repeat(2.0 ** rng.integers(-3, 4, (rows, K // 16)), 16, axis=1)
    x = grid_blocks(5, 64).astype(np.float32)
    w = grid_blocks(24, 64).T.astype(np.float32)          # blocks along the input channels
    lay = O.prepare_weights_fp4(w, None, 0)
    assert lay["t_x"] == 1.0
    out = O.linear_fp4(x, lay)
    assert np.array_equal(out["y"], x.astype(np.float64) @ w.astype(np.float64))


def test_fp4_tensor_scale_places_block_scales_in_range():
    for amax in [1e-6, 0.01, 1.0, 2688.0, 2689.0, 1e6]:
        t = O.fp4_tensor_scale(amax)
        assert math.frexp(t)[0] == 0.5                     # a power of two
        assert amax / (6 * t) <= 448.0 < 2 * amax / (6 * t)


def test_fp4_error_below_int4_on_an_outlier_layer():
    """Direction only (the pages report better similarity for NVFP4 than INT4,
    sec. 8 / Table 1, without a margin that transfers to synthetic layers)."""
    inp = workloads.make_inputs("tiny")
    x, w = inp["x"], inp["w"]
    a = O.act_amax(x)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    ef = np.linalg.norm(O.linear_fp4(x, O.prepare_weights_fp4(w, a, 16))["y"] - ref)
    e4 = np.linalg.norm(O.linear(x, O.prepare_weights(w, a, 16))["y"] - ref)
    assert ef < e4
