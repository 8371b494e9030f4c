"""Exhaustive host proof of the activation kernels' division-free quantizer
(INT4 codes, maximum 7, and the 8-bit setting's codes, maximum 127).

The activation kernel never divides by the group scale s: it forms
rc = fl32(1/s), p = fl32(v rc), the exact remainder e = fma(-p, s, v) and one
correction q1 = fma(e, rc, p), clamps with med3 and rounds by adding 1.5*2^23.
The definition (SVDQuant technical review, sec. 2.2 Eq.(1), with the readings
ties-to-even, codes in [-7, 7], fp16 scale s = fp16(fl32(amax / 7)) saturated
at 65504, code 0 when s = 0) divides.  ``tests/native/quant_exhaustive.c``
enumerates every pair the kernel can meet -- every positive finite bf16 group
maximum A with its scale s(A), and every bf16 v with |v| <= A, both signs
(1.07e9 pairs) -- and requires identical codes.  A planted mistake (the
correction step dropped) must be caught.

The scale table s(A) is built here with numpy's float32 -> float16 cast
(round-to-nearest-even) and checked against the oracle's own group quantizer.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import svdq_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "quant_exhaustive.c")


def _scale_table(q):
    a = (np.arange(32768, dtype=np.uint32) << np.uint32(16)).view(np.float32)
    fin = np.isfinite(a)
    with np.errstate(all="ignore"):
        s = np.minimum(a / np.float32(q), np.float32(65504.0)).astype(np.float32).astype(np.float16)
    s[~fin] = 0
    return a, fin, s


@pytest.mark.parametrize("q", [7, 127])
def test_scale_table_matches_oracle(q):
    a, fin, s = _scale_table(q)
    pos = fin & (a >= 0)
    amax = a[pos]
    # one group (row) per A: the maximum itself followed by zeros
    groups = np.zeros((amax.size, 64), np.float32)
    groups[:, 0] = amax
    _, sc = O.quantize_groups(groups) if q == 7 else O.quantize_rows8(groups)
    sc = sc[:, 0] if sc.ndim == 2 else sc
    assert np.array_equal(sc, s[pos].astype(np.float32))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    d = tmp_path_factory.mktemp("qe")
    exe = str(d / "quant_exhaustive")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                           "-o", exe, SRC, "-lm"])
    tabs = {}
    for q in (7, 127):
        tabs[q] = str(d / f"tab{q}.bin")
        _scale_table(q)[2].view(np.uint16).tofile(tabs[q])
    return exe, tabs


@pytest.mark.parametrize("q", [7, 127])
def test_division_free_quantizer_exhaustive(checker, q):
    exe, tabs = checker
    r = subprocess.run([exe, tabs[q], str(q)], capture_output=True, text=True, timeout=600)
    pairs, bad, ties, nans = map(int, r.stdout.split())
    assert pairs == 1065402238          # sum over A of 2 (A + 1), A = 1 .. 0x7F7F
    assert ties > 0                     # exact .5 quotients are exercised
    assert bad == 0 and nans == 0 and r.returncode == 0


def test_checker_catches_missing_correction(checker):
    exe, tabs = checker
    r = subprocess.run([exe, tabs[7], "7", "nocorr"], capture_output=True, text=True, timeout=600)
    pairs, bad, ties, nans = map(int, r.stdout.split())
    assert bad > 0 and r.returncode == 1


# ---------------------------------------------------------------------------
# the NVFP4 setting: division-free quotient against v / S for every E4M3
# block scale, tensor-scale exponent and bf16 value
# ---------------------------------------------------------------------------

FP4_SRC = os.path.join(HERE, "native", "fp4_quotient_exhaustive.c")


@pytest.fixture(scope="module")
def fp4_checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("fp4q") / "fp4_quotient_exhaustive")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                           "-o", exe, FP4_SRC, "-lm"])
    return exe


def test_fp4_division_free_quotient_exhaustive(fp4_checker):
    r = subprocess.run([fp4_checker], capture_output=True, text=True, timeout=600)
    pairs, bad, _ = map(int, r.stdout.split())
    assert pairs == 126 * 41 * (65536 - 256)   # finite bf16 patterns, 126 scales, 41 exponents
    assert bad == 0 and r.returncode == 0


def test_fp4_checker_catches_missing_correction(fp4_checker):
    r = subprocess.run([fp4_checker, "nocorr"], capture_output=True, text=True, timeout=600)
    _, bad, _ = map(int, r.stdout.split())
    assert bad > 0 and r.returncode == 1


def test_fp4_checker_code_rule_matches_oracle():
    """The checker's threshold-form E2M1 rounding and E4M3 decoding are those of
    the oracle (the checker is C; this ties the two together on all inputs)."""
    vals = O.e4m3_from_bits(np.arange(1, 0x7F))
    assert vals.min() == 2.0 ** -9 and vals.max() == 448.0 and len(set(vals.tolist())) == 126
