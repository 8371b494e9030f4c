"""CPU tests of the C-ABI library: it loads, exports every declared symbol, its
host preparation matches the oracle, and every validation error is raised on
the host before any HIP call.  No test here launches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

import workloads
from oracle import svdq_oracle as O
from tests import layout as LY

S = pytest.importorskip("w4a4_rank_corrected_amd")
from w4a4_rank_corrected_amd import _binding as B  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_or_skip():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libsvdq.so not built")
    return B.lib()


def test_exports_every_symbol_declared_in_header():
    L = _lib_or_skip()
    hdr = open(os.path.join(ROOT, "include", "svdq.h")).read()
    names = set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(svdq_\w+)\s*\(", hdr, re.M))
    assert len(names) >= 12
    for nm in names:
        assert hasattr(L, nm), nm
    assert {s[0] for s in B.SIGNATURES} == names
    assert L.svdq_abi_version() == 106


# Host logic of the GEMM schedule (the planner runs on the host; without a GPU
# the library plans for 256 CUs, the MI355X count).  Every setting runs three
# workgroups per CU, so a round is 768 tiles.  After full rounds, a last round
# of R tiles is split into k = min(768 // R, 8, G // 8) pieces per tile when
# k >= 3; when all T tiles fit in one round, into k = min(768 // T, 16, G // 8)
# pieces when k >= 2.  NVFP4 tiles are never split.  INT4 tiles are 128 x 64
# instead of 128 x 128 when the wide tiles would not fill one round.
SCHEDULES = [
    # (b, n, m, setting, tiles, grid, split workgroups, split tiles, workgroups per CU)
    (4608, 9216, 3072, "int4", 2592, 2592, 0, 0, 3),      # last round 288 tiles: halves are not used
    (4096, 4608, 1152, "int4", 1152, 1152, 0, 0, 3),      # last round half full: one tile per workgroup
    (4608, 3072, 12288, "int4", 864, 1536, 768, 96, 3),   # last round 96 tiles: 8 pieces of 24 groups
    (4608, 3072, 12288, "w8a8", 864, 1536, 768, 96, 3),   # the 8-bit setting plans like INT4
    (4608, 9216, 3072, "w8a8", 2592, 2592, 0, 0, 3),
    (4608, 5760, 3072, "w8a8", 1620, 2040, 504, 84, 3),   # 768 // 84 = 9 pieces, capped at G // 8 = 6
    (4608, 9216, 3072, "fp4", 2592, 2592, 0, 0, 3),
    (4608, 3072, 12288, "fp4", 864, 864, 0, 0, 3),        # NVFP4: never split
    (256, 21504, 3072, "fp4", 336, 336, 0, 0, 3),
    (256, 21504, 3072, "int4", 672, 672, 0, 0, 3),        # 336 wide tiles: 672 narrow ones, one per workgroup
    (256, 3072, 15360, "int4", 96, 768, 768, 96, 3),      # 96 narrow tiles: 8 pieces of 30 groups
    (256, 3072, 15360, "w8a8", 48, 768, 768, 48, 3),
    (4992, 5120, 1536, "int4", 1560, 1608, 72, 24, 3),    # 24 tiles left: 32 pieces, capped at G // 8 = 3
    (4608, 5376, 3072, "int4", 1512, 1512, 0, 0, 3),      # last round 744 tiles: no split
    (4608, 3072, 1024, "int4", 864, 864, 0, 0, 3),        # G = 16: at most 2 pieces after full rounds
    (256, 3072, 1024, "int4", 96, 192, 192, 96, 3),       # one round, G = 16: 2 pieces of 8 groups
    (256, 256, 64, "int4", 8, 8, 0, 0, 3),                # one group (narrow tiles)
    (0, 256, 256, "int4", 0, 0, 0, 0, 3),
]


@pytest.mark.parametrize("b,n,m,setting,tiles,grid,skw,skt,wpc", SCHEDULES)
def test_gemm_schedule(b, n, m, setting, tiles, grid, skw, skt, wpc):
    _lib_or_skip()
    if S.svdq_gemm_schedule(128, 128, 64, "w8a8")["grid"] != 1:
        pytest.skip("unexpected device")
    got = S.svdq_gemm_schedule(b, n, m, setting)
    assert got == {"tiles": tiles, "grid": grid, "split_workgroups": skw, "split_tiles": skt,
                   "workgroups_per_cu": wpc}


def test_gemm_schedule_rejects_bad_arguments():
    L = _lib_or_skip()
    info = (ctypes.c_int * 5)(-5, -5, -5, -5, -5)
    assert L.svdq_gemm_schedule(64, 64, 64, 0, None) == 1
    assert L.svdq_gemm_schedule(64, 64, 64, 3, info) == 1
    assert L.svdq_gemm_schedule(-1, 64, 64, 0, info) == 1
    assert L.svdq_gemm_schedule(64, 0, 64, 0, info) == 1
    for m in (0, 100, 1 << 23):
        assert L.svdq_gemm_schedule(64, 64, m, 0, info) != 0
    assert L.svdq_gemm_schedule(64, 64, 2 * 131072, 1, info) != 0   # above the 8-bit limit
    assert list(info) == [-5] * 5                            # untouched on error
    assert L.svdq_gemm_schedule(64, 64, 2 * 131072, 0, info) == 0


def test_status_strings():
    L = _lib_or_skip()
    for st in range(0, 9):
        assert L.svdq_status_string(st)
    assert L.svdq_status_string(99) == b"unknown status"


# ---------------------------------------------------------------------------
# host preparation vs oracle
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny():
    inp = workloads.make_inputs("tiny")
    a = O.act_amax(inp["x"])
    return inp, a, O.prepare_weights(inp["w"], a, 16)


def test_prepare_lambda_bit_exact(tiny):
    _lib_or_skip()
    inp, a, ref = tiny
    p = S.svdq_prepare_weights(inp["w"], a, 16)
    assert np.array_equal(p["lambda"], ref["lam32"])
    assert np.array_equal(p["smooth_inv"], ref["inv32"])


def test_prepare_svd_near_optimal_and_decomposition_exact(tiny):
    _lib_or_skip()
    inp, a, ref = tiny
    p = S.svdq_prepare_weights(inp["w"], a, 16, want_residual=True)
    l1 = LY.bf16_bits_to_f32(p["l1"]).T.astype(np.float64)   # [m][r]
    l2 = LY.bf16_bits_to_f32(p["l2"]).T.astype(np.float64)   # [r][n]
    wt = ref["wt"]
    r_lib = wt - l1 @ l2
    # the stored residual is exactly W~ - L1 L2 (up to its fp32 rounding)
    assert np.linalg.norm(r_lib - p["residual"]) <= 2 ** -23 * np.linalg.norm(r_lib)
    # truncated-SVD optimality (Eq.10): tail energy within 1e-3 of the oracle's
    assert np.linalg.norm(r_lib) ** 2 <= (1 + 1e-3) * np.linalg.norm(ref["r64"]) ** 2
    # the quantized residual is the library's own quantization of that residual
    qw2, ws2 = S.svdq_quantize_residual(p["residual"])
    assert np.array_equal(qw2, p["qw"]) and np.array_equal(ws2, p["wscale"])


@pytest.mark.parametrize("name", ["pixart_fc1", "flux_qkv"])
def test_prepare_svd_near_optimal_full_size(name):
    """The library's SVD on the PixArt- and FLUX-shaped synthetic layers, whose
    smoothed weights have a flat Marchenko-Pastur-like bulk (sigma_r and
    sigma_{r+1} nearly equal, so the rank-r subspace is ill-determined and the
    factors are judged by optimality, Eq.(10)): the residual's energy within
    1e-3 of the oracle's (ARPACK factors, rounded to bf16 the same way), the
    energy the branch removes at least (1 - 1e-3) of the top-r singular values'
    energy, the decomposition exact, and the codes and scales the oracle's
    quantization of the library's residual."""
    _lib_or_skip()
    inp = workloads.make_inputs(name)
    c = inp["cfg"]
    a = O.act_amax(inp["x"])
    p = S.svdq_prepare_weights(inp["w"], a, c.rank, want_residual=True)
    ref = O.prepare_weights(inp["w"], a, c.rank, svd="arpack")
    assert np.array_equal(p["lambda"], ref["lam32"]) and np.array_equal(p["smooth_inv"], ref["inv32"])
    l1 = LY.bf16_bits_to_f32(p["l1"]).T.astype(np.float64)
    l2 = LY.bf16_bits_to_f32(p["l2"]).T.astype(np.float64)
    wt = ref["wt"]
    low = l1 @ l2
    assert np.linalg.norm(wt - (low + p["residual"])) <= 1e-6 * np.linalg.norm(wt)
    tail = np.linalg.norm(wt - low) ** 2
    assert tail <= (1 + 1e-3) * np.linalg.norm(ref["r64"]) ** 2
    assert np.linalg.norm(wt) ** 2 - tail >= (1 - 1e-3) * np.sum(ref["sigma"][:c.rank] ** 2)
    codes, sw = O.quantize_weight_residual(p["residual"])
    assert np.array_equal(LY.unpack_codes(p["qw"]), np.ascontiguousarray(codes.T))
    assert np.array_equal(p["wscale"], LY.f32_to_fp16_bits(sw))


def test_prepare_svd_exact_when_the_space_is_whole():
    """Small layers (the Krylov space covers the short side) get the exact
    truncated SVD.  With a spectrum with clear gaps the singular vectors are
    unique up to sign, and both sides fix the sign the same way (largest entry
    of each L1 column positive), so the library's bf16 factors equal the bf16
    rounding of LAPACK's factors (the oracle's), wide and tall, up to full rank."""
    _lib_or_skip()
    rng = np.random.default_rng(8)
    for (m, n, r) in [(192, 256, 12), (256, 128, 20), (64, 64, 64), (128, 320, 1)]:
        U, _ = np.linalg.qr(rng.standard_normal((m, min(m, n))))
        V, _ = np.linalg.qr(rng.standard_normal((n, min(m, n))))
        sig = np.exp(-np.arange(min(m, n)) / 6.0)
        w = ((U * sig) @ V.T).astype(np.float32)
        p = S.svdq_prepare_weights(w, None, r, want_residual=True)
        ref = O.prepare_weights(w, None, r)
        assert np.array_equal(p["l1"], LY.f32_to_bf16_bits(ref["l1"]).T), (m, n, r)
        assert np.array_equal(p["l2"], LY.f32_to_bf16_bits(ref["l2"]).T), (m, n, r)


def test_svd_no_convergence_is_reported():
    """With the eigen-solver's iteration limit forced to 0 (the test hook),
    every preparation entry point returns SVDQ_ERR_NO_CONVERGENCE with its
    message and leaves the outputs untouched; rank 0 needs no SVD and still
    succeeds; restoring the limit restores the result bit for bit."""
    L = _lib_or_skip()
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((128, 96)) / 11).astype(np.float32)
    a = np.abs(rng.standard_normal(128)).astype(np.float32) + 0.5
    good = S.svdq_prepare_weights(w, a, 8)
    prev = L.svdq_test_set_svd_iteration_limit(0)
    try:
        assert prev == 60
        calls = [lambda: S.svdq_prepare_weights(w, a, 8),
                 lambda: S.svdq_w8a8_prepare_weights(w, a, 8),
                 lambda: S.svdq_fp4_prepare_weights(w, a, 8),
                 lambda: S.svdq_prepare_weights_refined(
                     w, a, workloads.random_bf16_bits(rng, (16, 128)), 8, alphas=(0.5,), iters=1)]
        for call in calls:
            with pytest.raises(B.SvdqError) as ei:
                call()
            assert ei.value.status == B.SVDQ_ERR_NO_CONVERGENCE
            assert "did not converge" in str(ei.value)
        S.svdq_prepare_weights(w, a, 0)  # no SVD at rank 0
        # outputs untouched on the error path
        qw = np.full((2, 96, 32), 0xAB, np.uint8)
        st = L.svdq_prepare_weights(B._ptr(w), B._ptr(a), 128, 96, 8, 64, 0.5, B._ptr(qw),
                                    B._ptr(np.zeros((2, 96), np.uint16)), B._ptr(np.zeros((8, 128), np.uint16)),
                                    B._ptr(np.zeros((96, 8), np.uint16)), B._ptr(np.zeros(128, np.float32)),
                                    B._ptr(np.zeros(128, np.float32)), None)
        assert st == B.SVDQ_ERR_NO_CONVERGENCE and np.all(qw == 0xAB)
    finally:
        assert L.svdq_test_set_svd_iteration_limit(-1) == 0
    again = S.svdq_prepare_weights(w, a, 8)
    for key in ("qw", "wscale", "l1", "l2", "lambda", "smooth_inv"):
        assert np.array_equal(again[key], good[key]), key


def test_quantize_residual_bit_exact_given_same_R(tiny):
    _lib_or_skip()
    _, _, ref = tiny
    qw, ws = S.svdq_quantize_residual(ref["r32"])
    assert np.array_equal(LY.unpack_codes(qw), np.ascontiguousarray(ref["qw"].T))
    assert np.array_equal(ws, LY.f32_to_fp16_bits(ref["sw"]))


def test_quantize_residual_adversarial_groups():
    _lib_or_skip()
    rng = np.random.default_rng(3)
    R = (rng.standard_normal((256, 40)) * np.exp(rng.uniform(-6, 6, (1, 40)))).astype(np.float32)
    R[:64, 0] = 0.0                                   # all-zero group
    R[64:128, 1] = 1e-9                               # underflowing scale
    R[128:192, 2] = np.tile([7.0, 2.5, 3.5, -2.5, 0.5, 1.5, -7.0, 0.0], 8)  # exact ties
    R[192:, 3] = 1e6                                  # saturating scale
    R[0, 4] = -3e5
    qw, ws = S.svdq_quantize_residual(R)
    codes, sw = O.quantize_weight_residual(R)
    assert np.array_equal(LY.unpack_codes(qw), np.ascontiguousarray(codes.T))
    assert np.array_equal(ws, LY.f32_to_fp16_bits(sw))


def test_prepare_rank0_and_no_smoothing():
    _lib_or_skip()
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((128, 48)) / 11).astype(np.float32)
    p = S.svdq_prepare_weights(w, None, 0, want_residual=True)
    assert np.all(p["lambda"] == 1) and np.all(p["smooth_inv"] == 1)
    assert np.array_equal(p["residual"], w)
    ref = O.prepare_weights(w, None, 0)
    assert np.array_equal(LY.unpack_codes(p["qw"]), np.ascontiguousarray(ref["qw"].T))


def test_prepare_full_rank_residual_small():
    _lib_or_skip()
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 40)) / 8).astype(np.float32)
    p = S.svdq_prepare_weights(w, None, 40, want_residual=True)
    assert np.linalg.norm(p["residual"]) < 1e-2 * np.linalg.norm(w)


def test_append_lora_matches_oracle_bits(tiny):
    _lib_or_skip()
    inp, a, ref = tiny
    rng = np.random.default_rng(6)
    A = (rng.standard_normal((256, 4)) * 0.14).astype(np.float32)
    Bm = (rng.standard_normal((4, 256)) * 0.14).astype(np.float32)
    host = LY.oracle_layer_to_host_abi(ref)
    l1o, l2o = S.svdq_append_lora(host["l1"], host["l2"], 256, 256, 16, ref["lam32"], A, Bm, 0.5)
    e1, e2 = O.append_lora(ref["l1"], ref["l2"], ref["lam32"], A, Bm, np.float32(0.5))
    assert np.array_equal(l1o, LY.f32_to_bf16_bits(e1).T)
    assert np.array_equal(l2o, LY.f32_to_bf16_bits(e2).T)
    # rank-0 base: the adapter alone
    l1z, l2z = S.svdq_append_lora(None, None, 256, 256, 0, None, A, Bm, 1.0)
    e1, e2 = O.append_lora(np.zeros((256, 0), np.float32), np.zeros((0, 256), np.float32), None, A, Bm, 1.0)
    assert np.array_equal(l1z, LY.f32_to_bf16_bits(e1).T) and np.array_equal(l2z, LY.f32_to_bf16_bits(e2).T)


def test_host_bf16_rounding_matches_oracle_on_ties():
    """The library's fp64->bf16 rounding (used for factors) against the oracle's."""
    _lib_or_skip()
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -40,
                     3.0e38, 3.4e38, 1e-40, -2.5e-39, 0.0], np.float64)
    # route through append_lora with lambda = 1 and A = the values (fp32-exact ones only)
    v32 = vals.astype(np.float32)
    A = v32.reshape(-1, 1)
    m = len(vals)
    l1o, _ = S.svdq_append_lora(None, None, m, 1, 0, None, A, np.ones((1, 1), np.float32), 1.0)
    assert np.array_equal(l1o[0], LY.f32_to_bf16_bits(O.bf16_from_f64(v32.astype(np.float64))))


# ---------------------------------------------------------------------------
# validation errors: raised on the host, nothing launched, outputs untouched
# ---------------------------------------------------------------------------

FAKE = 1 << 20  # a 16-byte aligned non-null address that is never dereferenced


def _layer(**kw):
    d = dict(m=128, n=64, rank=8, group=64, smooth_inv=None, qw=FAKE, wscale=FAKE, l1=FAKE, l2=FAKE,
             bias=None)
    d.update(kw)
    return B.svdq_layer(d["m"], d["n"], d["rank"], d["group"], d["smooth_inv"], d["qw"], d["wscale"],
                        d["l1"], d["l2"], d["bias"])


@pytest.mark.parametrize("kw,code", [
    (dict(group=32), B.SVDQ_ERR_UNSUPPORTED),
    (dict(m=100), B.SVDQ_ERR_UNSUPPORTED),
    (dict(n=0), B.SVDQ_ERR_INVALID_ARG),
    (dict(rank=300), B.SVDQ_ERR_UNSUPPORTED),
    (dict(rank=-1), B.SVDQ_ERR_UNSUPPORTED),
    (dict(qw=None), B.SVDQ_ERR_INVALID_ARG),
    (dict(qw=FAKE + 4), B.SVDQ_ERR_ALIGNMENT),
    (dict(l2=None), B.SVDQ_ERR_INVALID_ARG),
    (dict(l1=None), B.SVDQ_ERR_INVALID_ARG),
    (dict(n=B.SVDQ_MAX_DIM + 1), B.SVDQ_ERR_UNSUPPORTED),
    (dict(m=B.SVDQ_MAX_DIM + 64), B.SVDQ_ERR_UNSUPPORTED),
])
def test_linear_validation_errors(kw, code):
    L = _lib_or_skip()
    lay = _layer(**kw)
    st = L.svdq_linear(FAKE, ctypes.byref(lay), 16, FAKE, B.SVDQ_OUT_BF16, FAKE, 1 << 30, None)
    assert st == code, L.svdq_last_error()
    assert L.svdq_last_error()


def test_linear_workspace_and_dtype_errors():
    L = _lib_or_skip()
    lay = _layer()
    need = L.svdq_linear_workspace_size(16, 128, 64, 8, 64)
    assert need > 0
    assert L.svdq_linear(FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE, need - 1, None) == B.SVDQ_ERR_WORKSPACE
    assert L.svdq_linear(FAKE, ctypes.byref(lay), 16, FAKE, 0, None, need, None) == B.SVDQ_ERR_WORKSPACE
    assert L.svdq_linear(FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE + 16, need, None) == B.SVDQ_ERR_ALIGNMENT
    assert L.svdq_linear(FAKE, ctypes.byref(lay), 16, FAKE, 7, FAKE, need, None) == B.SVDQ_ERR_INVALID_ARG
    assert L.svdq_linear(FAKE + 2, ctypes.byref(lay), 16, FAKE, 0, FAKE, need, None) == B.SVDQ_ERR_ALIGNMENT
    assert L.svdq_linear(None, ctypes.byref(lay), 16, FAKE, 0, FAKE, need, None) == B.SVDQ_ERR_INVALID_ARG
    assert L.svdq_linear(FAKE, None, 16, FAKE, 0, FAKE, need, None) == B.SVDQ_ERR_INVALID_ARG
    assert L.svdq_linear(FAKE, ctypes.byref(lay), -1, FAKE, 0, FAKE, need, None) == B.SVDQ_ERR_INVALID_ARG
    assert L.svdq_linear(FAKE, ctypes.byref(lay), B.SVDQ_MAX_DIM + 1, FAKE, 0, FAKE, need, None) == \
        B.SVDQ_ERR_UNSUPPORTED
    # empty batch: valid, nothing to do, no workspace needed
    assert L.svdq_linear(FAKE, ctypes.byref(lay), 0, None, 0, None, 0, None) == B.SVDQ_OK


def test_linear_unfused_validation_errors():
    L = _lib_or_skip()
    lay = _layer()
    need = L.svdq_linear_unfused_workspace_size(16, 128, 64, 8, 64)
    assert need > L.svdq_linear_workspace_size(16, 128, 64, 8, 64)   # the second b x n output
    assert L.svdq_linear_unfused_workspace_size(16, 128, 64, 0, 64) == L.svdq_linear_workspace_size(16, 128, 64, 0, 64)
    f = L.svdq_linear_unfused
    assert f(FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE, need - 1, None) == B.SVDQ_ERR_WORKSPACE
    assert f(FAKE, ctypes.byref(lay), 16, FAKE + 8, 0, FAKE, need, None) == B.SVDQ_ERR_ALIGNMENT
    assert f(FAKE, ctypes.byref(_layer(group=32)), 16, FAKE, 0, FAKE, need, None) == B.SVDQ_ERR_UNSUPPORTED
    assert f(None, ctypes.byref(lay), 16, FAKE, 0, FAKE, need, None) == B.SVDQ_ERR_INVALID_ARG
    assert f(FAKE, ctypes.byref(lay), 0, None, 0, None, 0, None) == B.SVDQ_OK


def test_act_and_gemm_validation_errors():
    L = _lib_or_skip()
    f = L.svdq_quantize_act_lowrank_down
    assert f(FAKE, 16, 128, 8, 32, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.SVDQ_ERR_UNSUPPORTED
    assert f(FAKE, 16, 96, 8, 64, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.SVDQ_ERR_UNSUPPORTED
    assert f(FAKE, 16, 128, 8, 64, None, None, FAKE, FAKE, FAKE, None, 0, None) == B.SVDQ_ERR_INVALID_ARG
    assert f(FAKE, 16, 128, 8, 64, None, FAKE, FAKE, FAKE, None, None, 0, None) == B.SVDQ_ERR_INVALID_ARG
    assert f(FAKE + 8, 16, 128, 8, 64, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.SVDQ_ERR_ALIGNMENT
    assert f(FAKE, 16, 128, 0, 64, FAKE + 4, None, FAKE, FAKE, None, None, 0, None) == B.SVDQ_ERR_ALIGNMENT
    assert f(FAKE, 0, 128, 8, 64, None, None, None, None, None, None, 0, None) == B.SVDQ_OK
    # a shape that splits the channel groups needs a workspace
    need = L.svdq_act_workspace_size(64, 4096, 32)
    assert need > 0
    assert f(FAKE, 64, 4096, 32, 64, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.SVDQ_ERR_WORKSPACE
    g = L.svdq_gemm_w4a4_lowrank_up
    lay = _layer()
    W = 1 << 30
    assert g(FAKE, FAKE, None, ctypes.byref(lay), 16, FAKE, 0, FAKE, W, None) == B.SVDQ_ERR_INVALID_ARG
    assert g(None, FAKE, FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE, W, None) == B.SVDQ_ERR_INVALID_ARG
    assert g(FAKE + 1, FAKE, FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE, W, None) == B.SVDQ_ERR_ALIGNMENT
    assert g(FAKE, FAKE, FAKE, ctypes.byref(lay), 16, FAKE + 2, 1, FAKE, W, None) == B.SVDQ_ERR_ALIGNMENT
    # two channel groups can never be split: no GEMM workspace; 32 groups can
    assert L.svdq_gemm_workspace_size(16, 64, 128) == 0
    lay = _layer(m=2048)
    gneed = L.svdq_gemm_workspace_size(16, 64, 2048)
    assert gneed > 0
    assert g(FAKE, FAKE, FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE, gneed - 1, None) == B.SVDQ_ERR_WORKSPACE
    assert g(FAKE, FAKE, FAKE, ctypes.byref(lay), 16, FAKE, 0, None, gneed, None) == B.SVDQ_ERR_WORKSPACE
    assert g(FAKE, FAKE, FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE + 8, gneed, None) == B.SVDQ_ERR_ALIGNMENT
    c = L.svdq_calibrate_act_amax
    assert c(FAKE, 16, 100, FAKE, 0, None) == B.SVDQ_ERR_UNSUPPORTED
    assert c(FAKE, 16, 128, None, 0, None) == B.SVDQ_ERR_INVALID_ARG


def test_prepare_validation_errors():
    _lib_or_skip()
    w = np.ones((128, 32), np.float32)
    with pytest.raises(B.SvdqError) as e:
        S.svdq_prepare_weights(w, None, 64)              # rank > min(m, n)
    assert e.value.status == B.SVDQ_ERR_INVALID_ARG
    w2 = w.copy()
    w2[3, 4] = np.nan
    with pytest.raises(B.SvdqError) as e:
        S.svdq_prepare_weights(w2, None, 4)
    assert e.value.status == B.SVDQ_ERR_NONFINITE
    with pytest.raises(B.SvdqError) as e:
        S.svdq_prepare_weights(w, -np.ones(128, np.float32), 4)
    assert e.value.status == B.SVDQ_ERR_INVALID_ARG
    with pytest.raises(B.SvdqError) as e:
        S.svdq_prepare_weights(w, None, 4, alpha=1.5)
    assert e.value.status == B.SVDQ_ERR_INVALID_ARG
    with pytest.raises(B.SvdqError) as e:
        S.svdq_prepare_weights(np.ones((100, 32), np.float32), None, 4)
    assert e.value.status == B.SVDQ_ERR_UNSUPPORTED
    with pytest.raises(B.SvdqError) as e:
        S.svdq_append_lora(None, None, 128, 32, 250, None, np.ones((128, 8), np.float32),
                           np.ones((8, 32), np.float32), 1.0)
    assert e.value.status == B.SVDQ_ERR_UNSUPPORTED


def test_workspace_sizes_cover_layout():
    L = _lib_or_skip()
    for (b, m, n, r) in [(1, 64, 8, 0), (37, 256, 200, 16), (4608, 3072, 9216, 32), (256, 15360, 3072, 48)]:
        w = L.svdq_linear_workspace_size(b, m, n, r, 64)
        G = m // 64
        gw = L.svdq_gemm_workspace_size(b, n, m)
        assert w >= G * b * 32 + G * b * 2 + b * r * 4 + gw
        assert w % 256 == 0 and gw % 256 == 0
    assert L.svdq_linear_workspace_size(16, 100, 8, 8, 64) == 0
    assert L.svdq_gemm_workspace_size(16, 8, 100) == 0


# ---------------------------------------------------------------------------
# preparation with candidate search and refinement (Algorithm 1 steps 6-8)
# ---------------------------------------------------------------------------

def _refine_inputs(m=256, n=192, b=64, seed=31):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, m))
    x[:, rng.choice(m, 4, replace=False)] *= 40
    xbits = workloads.bf16_bits_of(x.astype(np.float32))
    w = (rng.standard_normal((m, n)) / np.sqrt(m)).astype(np.float32)
    w[rng.choice(m, 4, replace=False)] *= 8
    return xbits, LY.bf16_bits_to_f32(xbits), w


def test_refined_single_candidate_equals_prepare_weights():
    _lib_or_skip()
    xbits, x, w = _refine_inputs()
    a = O.act_amax(x)
    got = S.svdq_prepare_weights_refined(w, a, xbits, 16, alphas=(0.5,), iters=0)
    ref = S.svdq_prepare_weights(w, a, 16)
    for k in ("qw", "wscale", "l1", "l2", "lambda", "smooth_inv"):
        assert np.array_equal(got[k], ref[k]), k
    assert got["alpha"] == 0.5 and got["iteration"] == 0


def test_refined_reported_error_matches_oracle_evaluation():
    """The library scores candidates with its own fp64 host evaluation of the
    quantized layer; the oracle's evaluation of the returned layer agrees."""
    _lib_or_skip()
    xbits, x, w = _refine_inputs()
    got = S.svdq_prepare_weights_refined(w, O.act_amax(x), xbits, 16, alphas=(0.4, 0.6), iters=1)
    lay = LY.host_abi_to_oracle_layer(got)
    err = O.layer_output_error(x, w, lay)
    assert abs(got["rel_err"] - err) <= 1e-9 * err


def test_refined_search_beats_baseline_and_tracks_oracle():
    _lib_or_skip()
    xbits, x, w = _refine_inputs()
    a = O.act_amax(x)
    alphas = (0.3, 0.4, 0.5, 0.6, 0.7)
    got = S.svdq_prepare_weights_refined(w, a, xbits, 16, alphas=alphas, iters=2)
    base = S.svdq_prepare_weights_refined(w, a, xbits, 16, alphas=(0.5,), iters=0)
    assert got["rel_err"] <= base["rel_err"]
    ora = O.refine_weights(w, a, x, 16, alphas=alphas, iters=2)
    # different SVD algorithms (randomized vs LAPACK): the best scores agree closely
    assert abs(got["rel_err"] - ora["rel_err"]) <= 0.05 * ora["rel_err"]


def test_refined_validation_errors():
    _lib_or_skip()
    xbits, x, w = _refine_inputs(m=128, n=64, b=8)
    with pytest.raises(B.SvdqError) as e:
        S.svdq_prepare_weights_refined(w, None, xbits, 8, alphas=(1.5,))
    assert e.value.status == B.SVDQ_ERR_INVALID_ARG
    with pytest.raises(B.SvdqError) as e:
        S.svdq_prepare_weights_refined(w, None, xbits, 8, iters=17)
    assert e.value.status == B.SVDQ_ERR_INVALID_ARG
    with pytest.raises(B.SvdqError) as e:
        S.svdq_prepare_weights_refined(w, None, np.zeros((0, 128), np.uint16), 8)
    assert e.value.status == B.SVDQ_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# the 8-bit setting: host preparation and validation
# ---------------------------------------------------------------------------

def _codes8_by_column(qw):
    """[m/64][n][64] int8 records -> codes [n][m]."""
    G, n, _ = qw.shape
    return np.ascontiguousarray(qw.transpose(1, 0, 2).reshape(n, G * 64)).astype(np.int16)


def test_w8a8_prepare_shares_steps_2_to_4_and_quantizes_per_column(tiny):
    _lib_or_skip()
    inp, a, _ = tiny
    p4 = S.svdq_prepare_weights(inp["w"], a, 16, want_residual=True)
    p8 = S.svdq_w8a8_prepare_weights(inp["w"], a, 16, want_residual=True)
    for k in ("lambda", "smooth_inv", "l1", "l2", "residual"):
        assert np.array_equal(p4[k], p8[k]), k
    codes, sw = O.quantize_rows8(np.ascontiguousarray(p8["residual"].T))
    assert np.array_equal(_codes8_by_column(p8["qw"]), codes)
    assert np.array_equal(p8["wscale"], LY.f32_to_fp16_bits(sw))


def test_w8a8_quantizer_adversarial_columns():
    _lib_or_skip()
    rng = np.random.default_rng(8)
    R = (rng.standard_normal((256, 40)) * np.exp(rng.uniform(-6, 6, (1, 40)))).astype(np.float32)
    R[:, 0] = 0.0                                     # all-zero column
    R[:, 1] = 1e-9                                    # underflowing scale
    R[:, 2] = np.tile([127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -127.0, 0.0], 32)  # exact ties
    R[:, 3] = 1e8                                     # saturating scale
    R[0, 4] = -3e5
    p = S.svdq_w8a8_prepare_weights(R, None, 0, want_residual=True)   # rank 0, lambda = 1: R = W
    assert np.array_equal(p["residual"], R)
    codes, sw = O.quantize_rows8(np.ascontiguousarray(R.T))
    assert np.array_equal(_codes8_by_column(p["qw"]), codes)
    assert np.array_equal(p["wscale"], LY.f32_to_fp16_bits(sw))
    assert codes[2].tolist()[:8] == [127, 2, 4, -2, 0, 2, -127, 0]


def _layer8(**kw):
    d = dict(m=128, n=64, rank=8, smooth_inv=None, qw=FAKE, wscale=FAKE, l1=FAKE, l2=FAKE, bias=None)
    d.update(kw)
    return B.svdq_w8a8_layer(d["m"], d["n"], d["rank"], d["smooth_inv"], d["qw"], d["wscale"], d["l1"],
                             d["l2"], d["bias"])


@pytest.mark.parametrize("kw,code", [
    (dict(m=100), B.SVDQ_ERR_UNSUPPORTED),
    (dict(m=B.SVDQ_W8A8_MAX_M + 64), B.SVDQ_ERR_UNSUPPORTED),
    (dict(n=0), B.SVDQ_ERR_INVALID_ARG),
    (dict(rank=300), B.SVDQ_ERR_UNSUPPORTED),
    (dict(qw=None), B.SVDQ_ERR_INVALID_ARG),
    (dict(qw=FAKE + 8), B.SVDQ_ERR_ALIGNMENT),
    (dict(wscale=FAKE + 1), B.SVDQ_ERR_ALIGNMENT),
    (dict(l2=None), B.SVDQ_ERR_INVALID_ARG),
    (dict(l1=None), B.SVDQ_ERR_INVALID_ARG),
])
def test_w8a8_linear_validation_errors(kw, code):
    L = _lib_or_skip()
    lay = _layer8(**kw)
    st = L.svdq_w8a8_linear(FAKE, ctypes.byref(lay), 16, FAKE, B.SVDQ_OUT_BF16, FAKE, 1 << 30, None)
    assert st == code, L.svdq_last_error()
    assert L.svdq_last_error()


def test_w8a8_act_gemm_workspace_validation():
    L = _lib_or_skip()
    lay = _layer8()
    need = L.svdq_w8a8_linear_workspace_size(16, 128, 64, 8)
    assert need > 0 and need % 256 == 0
    f = L.svdq_w8a8_linear
    assert f(FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE, need - 1, None) == B.SVDQ_ERR_WORKSPACE
    assert f(FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE + 16, need, None) == B.SVDQ_ERR_ALIGNMENT
    assert f(FAKE, ctypes.byref(lay), 16, FAKE, 5, FAKE, need, None) == B.SVDQ_ERR_INVALID_ARG
    assert f(FAKE, ctypes.byref(lay), 0, None, 0, None, 0, None) == B.SVDQ_OK
    a = L.svdq_w8a8_quantize_act_lowrank_down
    assert a(FAKE, 16, 96, 8, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.SVDQ_ERR_UNSUPPORTED
    assert a(FAKE, 16, B.SVDQ_W8A8_MAX_M + 64, 0, None, None, FAKE, FAKE, None, None, 0, None) == \
        B.SVDQ_ERR_UNSUPPORTED
    assert a(FAKE, 16, 128, 8, None, None, FAKE, FAKE, FAKE, None, 0, None) == B.SVDQ_ERR_INVALID_ARG
    assert a(FAKE, 16, 128, 0, None, None, FAKE + 8, FAKE, None, None, 0, None) == B.SVDQ_ERR_ALIGNMENT
    assert a(FAKE, 16, 128, 0, None, None, FAKE, FAKE + 1, None, None, 0, None) == B.SVDQ_ERR_ALIGNMENT
    assert a(FAKE, 0, 128, 8, None, None, None, None, None, None, 0, None) == B.SVDQ_OK
    assert L.svdq_w8a8_act_workspace_size(64, 4096, 32) == L.svdq_act_workspace_size(64, 4096, 32) > 0
    assert a(FAKE, 64, 4096, 32, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.SVDQ_ERR_WORKSPACE
    g = L.svdq_w8a8_gemm_lowrank_up
    assert L.svdq_w8a8_gemm_workspace_size(16, 64, 128) == 0   # two groups: never split
    lay = _layer8(m=2048)
    gneed = L.svdq_w8a8_gemm_workspace_size(16, 64, 2048)
    assert gneed == L.svdq_gemm_workspace_size(16, 64, 2048) > 0
    assert g(FAKE, FAKE, None, ctypes.byref(lay), 16, FAKE, 0, FAKE, gneed, None) == B.SVDQ_ERR_INVALID_ARG
    assert g(FAKE + 4, FAKE, FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE, gneed, None) == B.SVDQ_ERR_ALIGNMENT
    assert g(FAKE, FAKE, FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE, gneed - 1, None) == B.SVDQ_ERR_WORKSPACE
    for (b, m, n, r) in [(1, 64, 8, 0), (37, 256, 200, 16), (4096, 3072, 9216, 16)]:
        w = L.svdq_w8a8_linear_workspace_size(b, m, n, r)
        assert w >= m * b + 2 * b + b * r * 4 + L.svdq_w8a8_gemm_workspace_size(b, n, m)
    assert L.svdq_w8a8_linear_workspace_size(16, B.SVDQ_W8A8_MAX_M + 64, 8, 8) == 0


def test_w8a8_prepare_validation_errors():
    _lib_or_skip()
    with pytest.raises(B.SvdqError) as e:
        S.svdq_w8a8_prepare_weights(np.ones((128, 32), np.float32), None, 64)
    assert e.value.status == B.SVDQ_ERR_INVALID_ARG
    with pytest.raises(B.SvdqError) as e:
        S.svdq_w8a8_prepare_weights(np.ones((128, 32), np.float32), None, 4, alpha=-0.1)
    assert e.value.status == B.SVDQ_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# the NVFP4 setting: host preparation and validation
# ---------------------------------------------------------------------------

def test_fp4_prepare_shares_steps_2_to_4_and_matches_oracle_quantizer(tiny):
    _lib_or_skip()
    inp, a, _ = tiny
    p4 = S.svdq_prepare_weights(inp["w"], a, 16, want_residual=True)
    pf = S.svdq_fp4_prepare_weights(inp["w"], a, 16, want_residual=True)
    for k in ("lambda", "smooth_inv", "l1", "l2", "residual"):
        assert np.array_equal(p4[k], pf[k]), k
    ref = O.prepare_weights_fp4(inp["w"], a, 16)
    assert pf["t_x"] == ref["t_x"]
    assert pf["t_w"] == O.fp4_tensor_scale(np.max(np.abs(pf["residual"])))
    codes, sb = O.quantize_fp4_blocks(np.ascontiguousarray(pf["residual"].T), pf["t_w"])
    assert np.array_equal(LY.unpack_fp4_codes(pf["qw"]), codes)
    assert np.array_equal(LY.unpack_fp4_scales(pf["wscale"]), O.e4m3_bits(sb))


def test_fp4_quantizer_adversarial_columns():
    _lib_or_skip()
    rng = np.random.default_rng(23)
    R = (rng.standard_normal((256, 40)) * np.exp(rng.uniform(-6, 6, (1, 40)))).astype(np.float32)
    R[:, 0] = 0.0                                                   # all-zero column
    R[:16, 1] = 1e-12                                               # a block whose scale underflows
    R[:, 2] = np.tile([6.0, 0.25, 0.75, -1.25, 1.75, 2.5, 3.5, 5.0, -0.0, 4.0, 3.0, 1.5, -0.5, 2.0, 1.0, 0.1], 16)
    R[:, 3] *= 1e6                                                  # a huge column
    p = S.svdq_fp4_prepare_weights(R, None, 0, want_residual=True)  # rank 0, lambda = 1: R = W
    assert np.array_equal(p["residual"], R) and p["t_x"] == 1.0
    t_w = O.fp4_tensor_scale(np.max(np.abs(R)))
    assert p["t_w"] == t_w
    codes, sb = O.quantize_fp4_blocks(np.ascontiguousarray(R.T), t_w)
    assert np.array_equal(LY.unpack_fp4_codes(p["qw"]), codes)
    assert np.array_equal(LY.unpack_fp4_scales(p["wscale"]), O.e4m3_bits(sb))


def _layer_fp4(**kw):
    d = dict(m=128, n=64, rank=8, t_x=1.0, t_w=0.5, smooth_inv=None, qw=FAKE, wscale=FAKE, l1=FAKE, l2=FAKE,
             bias=None)
    d.update(kw)
    return B.svdq_fp4_layer(d["m"], d["n"], d["rank"], d["t_x"], d["t_w"], d["smooth_inv"], d["qw"], d["wscale"],
                            d["l1"], d["l2"], d["bias"])


@pytest.mark.parametrize("kw,code", [
    (dict(m=100), B.SVDQ_ERR_UNSUPPORTED),
    (dict(n=0), B.SVDQ_ERR_INVALID_ARG),
    (dict(rank=300), B.SVDQ_ERR_UNSUPPORTED),
    (dict(t_x=0.75), B.SVDQ_ERR_INVALID_ARG),       # not a power of two
    (dict(t_w=0.0), B.SVDQ_ERR_INVALID_ARG),
    (dict(t_w=2.0 ** 70), B.SVDQ_ERR_INVALID_ARG),
    (dict(t_x=float("nan")), B.SVDQ_ERR_INVALID_ARG),
    (dict(qw=None), B.SVDQ_ERR_INVALID_ARG),
    (dict(qw=FAKE + 8), B.SVDQ_ERR_ALIGNMENT),
    (dict(wscale=FAKE + 1), B.SVDQ_ERR_ALIGNMENT),
    (dict(l2=None), B.SVDQ_ERR_INVALID_ARG),
    (dict(l1=None), B.SVDQ_ERR_INVALID_ARG),
])
def test_fp4_linear_validation_errors(kw, code):
    L = _lib_or_skip()
    lay = _layer_fp4(**kw)
    st = L.svdq_fp4_linear(FAKE, ctypes.byref(lay), 16, FAKE, B.SVDQ_OUT_BF16, FAKE, 1 << 30, None)
    assert st == code, L.svdq_last_error()
    assert L.svdq_last_error()


def test_fp4_act_gemm_workspace_validation():
    L = _lib_or_skip()
    lay = _layer_fp4()
    need = L.svdq_fp4_linear_workspace_size(16, 128, 64, 8)
    assert need > 0 and need % 256 == 0
    f = L.svdq_fp4_linear
    assert f(FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE, need - 1, None) == B.SVDQ_ERR_WORKSPACE
    assert f(FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE + 16, need, None) == B.SVDQ_ERR_ALIGNMENT
    assert f(FAKE, ctypes.byref(lay), 0, None, 0, None, 0, None) == B.SVDQ_OK
    a = L.svdq_fp4_quantize_act_lowrank_down
    assert a(FAKE, 16, 96, 8, None, FAKE, 1.0, FAKE, FAKE, FAKE, None, 0, None) == B.SVDQ_ERR_UNSUPPORTED
    assert a(FAKE, 16, 128, 8, None, FAKE, 3.0, FAKE, FAKE, FAKE, None, 0, None) == B.SVDQ_ERR_INVALID_ARG
    assert a(FAKE, 16, 128, 8, None, None, 1.0, FAKE, FAKE, FAKE, None, 0, None) == B.SVDQ_ERR_INVALID_ARG
    assert a(FAKE, 16, 128, 0, None, None, 1.0, FAKE + 8, FAKE, None, None, 0, None) == B.SVDQ_ERR_ALIGNMENT
    assert a(FAKE, 0, 128, 8, None, None, 1.0, None, None, None, None, 0, None) == B.SVDQ_OK
    assert L.svdq_fp4_act_workspace_size(64, 4096, 32) == L.svdq_act_workspace_size(64, 4096, 32) > 0
    assert a(FAKE, 64, 4096, 32, None, FAKE, 1.0, FAKE, FAKE, FAKE, None, 0, None) == B.SVDQ_ERR_WORKSPACE
    g = L.svdq_fp4_gemm_lowrank_up
    assert L.svdq_fp4_gemm_workspace_size(16, 64, 128) == 0    # two groups: never split
    lay = _layer_fp4(m=2048)
    gneed = L.svdq_fp4_gemm_workspace_size(16, 64, 2048)
    assert gneed == L.svdq_gemm_workspace_size(16, 64, 2048) > 0
    assert g(FAKE, FAKE, None, ctypes.byref(lay), 16, FAKE, 0, FAKE, gneed, None) == B.SVDQ_ERR_INVALID_ARG
    assert g(FAKE + 4, FAKE, FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE, gneed, None) == B.SVDQ_ERR_ALIGNMENT
    assert g(FAKE, FAKE, FAKE, ctypes.byref(lay), 16, FAKE, 0, FAKE, gneed - 1, None) == B.SVDQ_ERR_WORKSPACE
    for (b, m, n, r) in [(1, 64, 8, 0), (37, 256, 200, 16), (4608, 3072, 9216, 32)]:
        w = L.svdq_fp4_linear_workspace_size(b, m, n, r)
        assert w >= m * b // 2 + m * b // 16 + b * r * 4 + L.svdq_fp4_gemm_workspace_size(b, n, m)


def test_fp4_prepare_validation_errors():
    _lib_or_skip()
    with pytest.raises(B.SvdqError) as e:
        S.svdq_fp4_prepare_weights(np.ones((128, 32), np.float32), None, 64)
    assert e.value.status == B.SVDQ_ERR_INVALID_ARG
    with pytest.raises(B.SvdqError) as e:
        S.svdq_fp4_prepare_weights(np.ones((96, 32), np.float32), None, 4)
    assert e.value.status == B.SVDQ_ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# the Python binding checks every device tensor before a call reaches the
# library (a host tensor, a wrong dtype or shape would be read or written out
# of bounds by a kernel)
# ---------------------------------------------------------------------------

class _FakeGpuTensor:
    """Stands in for a GPU tensor (device, dtype, shape) on a machine without one."""

    def __init__(self, shape, dtype, device="cuda:0", contiguous=True):
        import torch
        self.shape, self.dtype, self.device = tuple(shape), dtype, torch.device(device)
        self.is_cuda, self._c = True, contiguous

    def is_contiguous(self):
        return self._c

    def dim(self):
        return len(self.shape)


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    import types
    x = torch.zeros((16, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.svdq_linear(x, None)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.svdq_linear_unfused(x, None)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.svdq_w8a8_linear(x, None)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.svdq_fp4_linear(x, None)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.svdq_calibrate_act_amax(x)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.svdq_quantize_act_lowrank_down(x, None, None, 0)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.svdq_w8a8_quantize_act_lowrank_down(x, None, None, 0)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.svdq_fp4_quantize_act_lowrank_down(x, None, None, 0, 1.0)
    lay = types.SimpleNamespace(m=128, n=64, rank=0)
    qx = torch.zeros((2, 16, 32), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.svdq_gemm_w4a4_lowrank_up(qx, None, None, lay)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.svdq_fp4_gemm_lowrank_up(qx, None, None, lay)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.svdq_w8a8_gemm_lowrank_up(qx.view(torch.int8), None, None, lay)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.DeviceLayer.from_tensors(128, 64, 0, qx, None)


def test_binding_checks_dtype_shape_and_output_type():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match="out_dtype"):
        B._out_code(torch.float16)
    assert B._out_code(None) == B.SVDQ_OUT_BF16
    assert B._out_code(torch.bfloat16) == B.SVDQ_OUT_BF16
    assert B._out_code(torch.float32) == B.SVDQ_OUT_F32
    dev = torch.device("cuda:0")
    # a preallocated output must match the requested dtype and [b][n]
    with pytest.raises(ValueError, match="dtype"):
        B._output(_FakeGpuTensor((16, 64), torch.bfloat16), 16, 64, torch.float32, dev)
    with pytest.raises(ValueError, match="shape"):
        B._output(_FakeGpuTensor((16, 32), torch.float32), 16, 64, torch.float32, dev)
    y = _FakeGpuTensor((16, 64), torch.float32)
    assert B._output(y, 16, 64, torch.float32, dev) == (y, B.SVDQ_OUT_F32)
    with pytest.raises(ValueError, match="contiguous"):
        B._output(_FakeGpuTensor((16, 64), torch.float32, contiguous=False), 16, 64, torch.float32, dev)
    with pytest.raises(ValueError, match="expected cuda:0"):
        B._output(_FakeGpuTensor((16, 64), torch.float32, device="cuda:1"), 16, 64, torch.float32, dev)
    # activations are bf16 matrices
    with pytest.raises(ValueError, match="dtype"):
        B._input(_FakeGpuTensor((16, 128), torch.float32))
    with pytest.raises(ValueError, match="2-D"):
        B._input(_FakeGpuTensor((2, 16, 128), torch.bfloat16))
    assert tuple(B._input(_FakeGpuTensor((16, 128), torch.bfloat16))) == (16, 128)
    # GEMM inputs follow the layer: [m/64][b][record] codes, per-group scales, z [b][rank]
    import types
    lay = types.SimpleNamespace(m=128, n=64, rank=8, qw=_FakeGpuTensor((2, 64, 32), torch.uint8))
    qx = _FakeGpuTensor((2, 16, 32), torch.uint8)
    asc = _FakeGpuTensor((2, 16), torch.float16)
    z = _FakeGpuTensor((16, 8), torch.float32)
    assert B._gemm_operands(qx, asc, z, lay, None, True, 32, torch.uint8, torch.float16) == 16
    with pytest.raises(ValueError, match="qx has shape"):
        B._gemm_operands(qx, asc, z, lay, 8, True, 32, torch.uint8, torch.float16)
    with pytest.raises(ValueError, match="qx has shape"):
        B._gemm_operands(_FakeGpuTensor((3, 16, 32), torch.uint8), asc, z, lay, None, True, 32, torch.uint8,
                         torch.float16)
    with pytest.raises(ValueError, match="ascale has shape"):
        B._gemm_operands(qx, _FakeGpuTensor((2, 15), torch.float16), z, lay, None, True, 32, torch.uint8,
                         torch.float16)
    with pytest.raises(ValueError, match="z has shape"):
        B._gemm_operands(qx, asc, _FakeGpuTensor((16, 4), torch.float32), lay, None, True, 32, torch.uint8,
                         torch.float16)
    with pytest.raises(ValueError, match="ascale has dtype"):
        B._gemm_operands(qx, _FakeGpuTensor((2, 16), torch.float32), z, lay, None, True, 32, torch.uint8,
                         torch.float16)
    # the 8-bit setting: one scale per token; NVFP4: four E4M3 bytes per row and group
    assert B._gemm_operands(_FakeGpuTensor((2, 16, 64), torch.int8), _FakeGpuTensor((16,), torch.float16), z, lay,
                            None, False, 64, torch.int8, torch.float16) == 16
    assert B._gemm_operands(qx, _FakeGpuTensor((2, 16, 4), torch.uint8), z, lay, None, True, 32, torch.uint8,
                            torch.uint8, (4,)) == 16
    # host arrays and tensors must be contiguous (a ValueError, not an assert)
    with pytest.raises(ValueError, match="contiguous"):
        B._ptr(np.zeros((4, 4), np.float32)[:, ::2])


# ---------------------------------------------------------------------------
# stored layer files (Algorithm 1 step 9: keep the prepared layer)
# ---------------------------------------------------------------------------

LAYER_KEYS = ("lambda", "smooth_inv", "qw", "wscale", "l1", "l2")


def _prepared(rank=16, lora=0):
    inp = workloads.make_inputs("tiny")
    host = S.svdq_prepare_weights(inp["w"], O.act_amax(inp["x"]), rank)
    if lora:
        rng = np.random.default_rng(12)
        A = (rng.standard_normal((256, lora)) * 0.14).astype(np.float32)
        Bm = (rng.standard_normal((lora, 256)) * 0.14).astype(np.float32)
        l1, l2 = S.svdq_append_lora(host["l1"], host["l2"], 256, 256, rank, host["lambda"], A, Bm, 1.0)
        host = dict(host, l1=l1, l2=l2, rank=rank + lora)
    return host


@pytest.mark.parametrize("rank,lora,with_bias", [(16, 0, False), (16, 8, True), (0, 0, True)])
def test_layer_file_round_trip(tmp_path, rank, lora, with_bias):
    _lib_or_skip()
    host = _prepared(rank, lora)
    bias = workloads.bf16_bits_of(np.linspace(-1, 1, 256).astype(np.float32)) if with_bias else None
    path = str(tmp_path / "layer.svdq")
    S.svdq_save_layer(path, host, alpha=0.5, bias=bias)
    back = S.svdq_load_layer(path)
    assert (back["m"], back["n"], back["rank"], back["alpha"]) == (256, 256, rank + lora, 0.5)
    for key in LAYER_KEYS:
        assert np.array_equal(back[key], host[key] if back["rank"] or key not in ("l1", "l2")
                              else np.zeros_like(back[key])), key
    if with_bias:
        assert np.array_equal(back["bias"], bias)
    else:
        assert back["bias"] is None
    assert os.path.getsize(path) == 64 + 4 * 256 * 2 + 4 * 256 * 32 + 2 * 4 * 256 + \
        2 * (rank + lora) * 512 + (512 if with_bias else 0)


def test_layer_file_rejects_damaged_files(tmp_path):
    """Corrupted, truncated, extended, foreign and missing files give
    SVDQ_ERR_IO and leave the caller's buffers untouched."""
    L = _lib_or_skip()
    host = _prepared()
    good = str(tmp_path / "good.svdq")
    S.svdq_save_layer(good, host)
    raw = open(good, "rb").read()

    def variant(name, data):
        p = str(tmp_path / name)
        with open(p, "wb") as f:
            f.write(data)
        return p

    flipped = bytearray(raw)
    flipped[64 + 1000] ^= 0x10                        # one payload bit
    header = bytearray(raw)
    header[0:8] = b"NOTALAYR"
    version = bytearray(raw)
    version[8] = 2
    dims = bytearray(raw)
    dims[16:20] = (320).to_bytes(4, "little")         # m no longer matches the payload size
    cases = {"corrupt": variant("c.svdq", bytes(flipped)), "truncated": variant("t.svdq", raw[:-10]),
             "extended": variant("e.svdq", raw + b"\0"), "magic": variant("m.svdq", bytes(header)),
             "version": variant("v.svdq", bytes(version)), "dims": variant("d.svdq", bytes(dims)),
             "short": variant("s.svdq", raw[:40]), "missing": str(tmp_path / "none.svdq")}
    for what, path in cases.items():
        with pytest.raises(B.SvdqError) as ei:
            S.svdq_load_layer(path)
        assert ei.value.status == B.SVDQ_ERR_IO, what
    # buffers untouched when the checksum fails
    lam = np.full(256, 7.0, np.float32)
    qw = np.full((4, 256, 32), 0x5A, np.uint8)
    st = L.svdq_load_layer(os.fsencode(cases["corrupt"]), B._ptr(lam), B._ptr(np.zeros(256, np.float32)),
                           B._ptr(qw), B._ptr(np.zeros((4, 256), np.uint16)), B._ptr(np.zeros((16, 256), np.uint16)),
                           B._ptr(np.zeros((256, 16), np.uint16)), None)
    assert st == B.SVDQ_ERR_IO and b"checksum" in L.svdq_last_error()
    assert np.all(lam == 7.0) and np.all(qw == 0x5A)


def test_layer_file_argument_errors(tmp_path):
    L = _lib_or_skip()
    host = _prepared()
    path = str(tmp_path / "x.svdq")
    assert L.svdq_save_layer(None, None) == B.SVDQ_ERR_INVALID_ARG
    with pytest.raises(ValueError, match="shape"):
        S.svdq_save_layer(path, dict(host, qw=host["qw"][:, :-1]))
    with pytest.raises(B.SvdqError) as ei:
        S.svdq_save_layer(str(tmp_path / "no_dir" / "x.svdq"), host)
    assert ei.value.status == B.SVDQ_ERR_IO
    S.svdq_save_layer(path, host)
    m = ctypes.c_int32()
    assert L.svdq_load_layer_info(os.fsencode(path), ctypes.byref(m), None, None, None, None) == \
        B.SVDQ_ERR_INVALID_ARG
    # l1 / l2 are required for a rank-16 file
    st = L.svdq_load_layer(os.fsencode(path), B._ptr(np.zeros(256, np.float32)), B._ptr(np.zeros(256, np.float32)),
                           B._ptr(np.zeros((4, 256, 32), np.uint8)), B._ptr(np.zeros((4, 256), np.uint16)),
                           None, None, None)
    assert st == B.SVDQ_ERR_INVALID_ARG
