"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars (from the layer's contract):
  * INT4 codes, fp16 scales, calibration maxima: bit-exact.
  * per-group integer sums: exact (checked through fp32 outputs that carry them
    exactly).
  * Z: ||Z - Z_ref||_F / ||Z_ref||_F <= 1e-4 (fp32 MFMA accumulation vs fp64).
  * Y: ||Y - Y_ref||_F / ||Y_ref||_F <= 2e-3 for fp32 and bf16 outputs.
Inputs are seeded synthetic tensors; layers are prepared by the oracle, so no
oracle input or expected value comes from the product.
"""
import sys

import numpy as np
import pytest

import workloads
from oracle import svdq_oracle as O
from tests import layout as LY

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

Y_TOL = 2e-3
Z_TOL = 1e-4


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a4_rank_corrected_amd as S
    S.lib()  # raises if the library is missing: no fallback
    return S


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def device_layer(S, lay, bias_bits=None, smoothing=True):
    host = LY.oracle_layer_to_host_abi(lay)
    return S.DeviceLayer(host, bias=bias_bits, smoothing=smoothing and lay.get("inv32") is not None)


def y_to_np(y):
    if y.dtype == torch.bfloat16:
        return LY.bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16))
    return y.cpu().numpy()


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------

def adversarial_x(rng, b, m):
    """bf16 activations exercising ties, zero / underflowing / saturating groups."""
    x = rng.standard_normal((b, m)).astype(np.float32)
    G = m // 64
    for i in range(b):
        g = i % G
        kind = i % 7
        seg = slice(64 * g, 64 * g + 64)
        if kind == 0:
            x[i, seg] = rng.integers(-7, 8, 64)
            x[i, 64 * g] = 7.0                           # s = 1: exact integer codes
        elif kind == 1:
            x[i, seg] = rng.integers(-7, 8, 64) + 0.5    # many exact .5 ties
            x[i, 64 * g] = 7.0
        elif kind == 2:
            x[i, seg] = 0.0                              # all-zero group
        elif kind == 3:
            x[i, seg] *= 1e-30                           # fp16 scale underflows to 0
        elif kind == 4:
            x[i, seg] *= 1e7                             # scale saturates at 65504
        elif kind == 5:
            x[i, seg] = rng.integers(-14, 15, 64) * 0.25  # ties against s = 0.5
            x[i, 64 * g] = 3.5
        elif kind == 6:
            x[i, seg] *= 2.0 ** -133                     # bf16 subnormals
    return workloads.bf16_bits_of(x)


# ---------------------------------------------------------------------------
# calibration statistic
# ---------------------------------------------------------------------------

def test_calibrate_amax_bit_exact(S):
    rng = np.random.default_rng(0)
    for (b, m) in [(64, 256), (37, 192), (1, 64), (300, 1024)]:
        _say(f"calibrate b={b} m={m}")
        xb = workloads.random_bf16_bits(rng, (b, m), 3.0)
        xd = dev_bf16(xb)
        am = S.svdq_calibrate_act_amax(xd)
        torch.cuda.synchronize()
        assert np.array_equal(am.cpu().numpy(), O.act_amax(LY.bf16_bits_to_f32(xb)))
        # accumulate a second batch
        xb2 = workloads.random_bf16_bits(rng, (b, m), 5.0)
        S.svdq_calibrate_act_amax(dev_bf16(xb2), am, accumulate=True)
        torch.cuda.synchronize()
        both = np.concatenate([LY.bf16_bits_to_f32(xb), LY.bf16_bits_to_f32(xb2)])
        assert np.array_equal(am.cpu().numpy(), O.act_amax(both))


# ---------------------------------------------------------------------------
# fused activation quantization + down-projection
# ---------------------------------------------------------------------------

ACT_CASES = [
    # (b, m, rank, smoothing, adversarial)
    (64, 256, 16, True, False),
    (37, 192, 20, True, False),
    (1, 64, 8, False, False),
    (17, 128, 0, True, False),
    (200, 512, 48, True, True),
    (33, 320, 33, False, True),
    (16, 4096, 32, True, False),     # many groups per split
    (5, 64, 256, True, False),       # maximum rank
    (3000, 12288, 48, True, False),  # several LDS chunks per split, odd chunk size
    (1024, 6144, 200, True, False),  # rank > 128: one group per chunk
    (2000, 6144, 72, False, False),  # 8 blocks of Z, two groups per chunk
    (4100, 640, 40, True, False),    # wide kernel: 16-row strips (ragged last), 10 groups over 8 waves
    (4096, 1536, 0, False, True),    # wide kernel, codes only, 3 groups per wave
]


@pytest.mark.parametrize("b,m,rank,smooth,adv", ACT_CASES)
def test_act_quant_down_parity(S, b, m, rank, smooth, adv):
    _say(f"act_quant_down b={b} m={m} rank={rank} smooth={smooth} adv={adv}")
    rng = np.random.default_rng(b * 1000 + m + rank)
    xb = adversarial_x(rng, b, m) if adv else workloads.random_bf16_bits(rng, (b, m), 2.0)
    x = LY.bf16_bits_to_f32(xb)
    inv = None
    if smooth:
        inv = (1.0 / np.exp(rng.uniform(-2, 2, m))).astype(np.float32)
    l1 = O.bf16_from_f32((rng.standard_normal((m, rank)) / np.sqrt(m)).astype(np.float32))
    xt, qx, sx = O.quantize_activation(x, inv)
    z_ref = O.lowrank_down(xt, l1)
    qd, asd, zd = S.svdq_quantize_act_lowrank_down(
        dev_bf16(xb), None if inv is None else dev_f32(inv),
        dev_bf16(np.ascontiguousarray(LY.f32_to_bf16_bits(l1).T)) if rank else None, rank)
    torch.cuda.synchronize()
    assert np.array_equal(LY.unpack_codes(qd.cpu().numpy()), qx)
    assert np.array_equal(asd.cpu().numpy().view(np.uint16), LY.f32_to_fp16_bits(sx.T))
    if rank:
        assert rel(zd.cpu().numpy(), z_ref) <= Z_TOL


def test_z_split_reduction_same_bits_on_both_paths(S):
    """Few rows and many channel groups: Z is summed over 64 splits (chunks of
    every 16th split, then the chunks in order).  The 16-byte reduction kernel
    (z 16-byte aligned) and the one-element kernel (z only 4-byte aligned) must
    give the same bits, within the oracle's bar."""
    b, m, rank = 64, 12288, 24
    need = S.svdq_act_workspace_size(b, m, rank)
    assert need >= 17 * b * rank * 4      # more than 16 splits: the chunked order matters
    rng = np.random.default_rng(77)
    xb = workloads.random_bf16_bits(rng, (b, m), 2.0)
    x = LY.bf16_bits_to_f32(xb)
    l1 = O.bf16_from_f32((rng.standard_normal((m, rank)) / np.sqrt(m)).astype(np.float32))
    xd = dev_bf16(xb)
    l1d = dev_bf16(np.ascontiguousarray(LY.f32_to_bf16_bits(l1).T))
    _say(f"z split reduction b={b} m={m} rank={rank}")
    _, _, za = S.svdq_quantize_act_lowrank_down(xd, None, l1d, rank)
    store = torch.empty(b * rank + 1, dtype=torch.float32, device="cuda")
    zm = store[1:].view(b, rank)          # 4-byte aligned, not 16
    assert zm.data_ptr() % 16 != 0
    S.svdq_quantize_act_lowrank_down(xd, None, l1d, rank, z=zm)
    torch.cuda.synchronize()
    assert torch.equal(za, zm)
    xt, _, _ = O.quantize_activation(x, None)
    assert rel(za.cpu().numpy(), O.lowrank_down(xt, l1)) <= Z_TOL


# ---------------------------------------------------------------------------
# fused W4A4 GEMM + up-projection
# ---------------------------------------------------------------------------

def test_act_workspace_garbage_and_reuse(S):
    """Split partial sums of Z live in the caller's workspace: random initial
    contents, two shapes in turn on one workspace, and a repeated call must all
    give the oracle's codes and the same Z."""
    shapes = [(300, 2048, 24), (90, 4096, 40)]
    need = max(S.svdq_act_workspace_size(b, m, r) for b, m, r in shapes)
    assert need > 0
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda")
    runs = {}
    for rep in range(2):
        for (b, m, rank) in shapes:
            _say(f"act workspace reuse rep={rep} b={b} m={m} rank={rank}")
            xb = workloads.random_bf16_bits(np.random.default_rng(b + m), (b, m), 2.0)
            x = LY.bf16_bits_to_f32(xb)
            l1 = O.bf16_from_f32((np.random.default_rng(rank).standard_normal((m, rank)) / np.sqrt(m))
                                 .astype(np.float32))
            xt, qx, sx = O.quantize_activation(x, None)
            qd, asd, zd = S.svdq_quantize_act_lowrank_down(
                dev_bf16(xb), None, dev_bf16(np.ascontiguousarray(LY.f32_to_bf16_bits(l1).T)), rank,
                workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(LY.unpack_codes(qd.cpu().numpy()), qx)
            zc = zd.cpu().numpy()
            assert rel(zc, O.lowrank_down(xt, l1)) <= Z_TOL
            if rep == 0:
                runs[(b, m)] = zc
            else:
                assert np.array_equal(runs[(b, m)], zc)


def _oracle_layer(rng, m, n, rank, x32):
    w = (rng.standard_normal((m, n)) / np.sqrt(m)).astype(np.float32)
    w[rng.choice(m, max(1, m // 64), replace=False)] *= 8
    return O.prepare_weights(w, O.act_amax(x32), rank)


GEMM_CASES = [
    # (b, m, n, rank, bias)
    (64, 256, 256, 16, False),
    (37, 192, 100, 20, True),     # ragged b, n (n % 4 != 0), rank not a multiple of 8
    (130, 128, 260, 0, True),     # rank 0 = plain W4A4
    (1, 64, 7, 3, False),
    (256, 512, 384, 48, True),
    (256, 4096, 256, 16, True),   # split-K: each tile split over 8 workgroups
    (300, 2368, 200, 24, False),  # split-K: uneven splits, ragged edges
]


@pytest.mark.parametrize("b,m,n,rank,bias", GEMM_CASES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_up_parity(S, b, m, n, rank, bias, out):
    _say(f"gemm_up b={b} m={m} n={n} rank={rank} bias={bias} out={out}")
    rng = np.random.default_rng(b + m + n + rank)
    xb = workloads.random_bf16_bits(rng, (b, m), 1.5)
    x = LY.bf16_bits_to_f32(xb)
    lay = _oracle_layer(rng, m, n, rank, x)
    bias_v = O.bf16_from_f32(rng.standard_normal(n).astype(np.float32)) if bias else None
    xt, qx, sx = O.quantize_activation(x, lay["inv32"])
    z = O.lowrank_down(xt, lay["l1"])
    y_ref = O.gemm_main(qx, sx, lay["qw"], lay["sw"])
    if rank:
        y_ref = y_ref + O.lowrank_up(z.astype(np.float32).astype(np.float64), lay["l2"])
    if bias:
        y_ref = y_ref + bias_v[None, :]
    dl = device_layer(S, lay, LY.f32_to_bf16_bits(bias_v) if bias else None)
    qd = torch.from_numpy(LY.pack_codes(qx)).cuda()
    asd = torch.from_numpy(LY.f32_to_fp16_bits(np.ascontiguousarray(sx.T)).view(np.int16)).cuda().view(torch.float16)
    zd = dev_f32(z) if rank else None
    y = S.svdq_gemm_w4a4_lowrank_up(qd, asd, zd, dl, b, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    yn = y_to_np(y)
    err = rel(yn, y_ref)
    _say(f"  rel err {err:.3e}")
    assert err <= (1e-5 if out == "f32" else Y_TOL)
    if out == "bf16":
        # only rare one-ulp flips against the correctly rounded reference
        yr = O.bf16_from_f64(y_ref)
        assert np.mean(yn != yr) < 0.01


def test_gemm_exact_group_sums(S):
    """All scales 1, rank 0, fp32 output: Y = sum_g isum exactly; isolating one
    group at a time (other groups' activation scales 0) yields each isum."""
    rng = np.random.default_rng(7)
    b, m, n = 50, 256, 72
    G = m // 64
    qx = rng.integers(-7, 8, (b, m)).astype(np.int8)
    qw = rng.integers(-7, 8, (m, n)).astype(np.int8)
    qx[:3] = 7
    qw[:, :2] = -7                                      # extreme sums 64*49
    isum = O.group_isums(qx, qw)
    host = {"m": m, "n": n, "rank": 0, "qw": LY.pack_codes(np.ascontiguousarray(qw.T)),
            "wscale": LY.f32_to_fp16_bits(np.ones((G, n), np.float32)),
            "l1": np.zeros((0, m), np.uint16), "l2": np.zeros((n, 0), np.uint16),
            "smooth_inv": np.ones(m, np.float32)}
    dl = S.DeviceLayer(host, smoothing=False)
    qd = torch.from_numpy(LY.pack_codes(qx)).cuda()
    ones = np.ones((G, b), np.float32)
    for g in [None] + list(range(G)):
        sc = ones.copy()
        if g is not None:
            sc[:] = 0.0
            sc[g] = 1.0
        asd = torch.from_numpy(LY.f32_to_fp16_bits(sc).view(np.int16)).cuda().view(torch.float16)
        y = S.svdq_gemm_w4a4_lowrank_up(qd, asd, None, dl, b, torch.float32)
        torch.cuda.synchronize()
        expect = isum.sum(axis=2) if g is None else isum[:, :, g]
        assert np.array_equal(y.cpu().numpy(), expect.astype(np.float32)), f"group {g}"


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

LINEAR_CASES = [
    ("tiny", None),
    ("tiny_ragged", None),
    ("tiny_lora", None),
]


def _linear_case(name):
    rng = np.random.default_rng(11)
    if name.startswith("tiny"):
        inp = workloads.make_inputs("tiny")
        xb, x, w = inp["x_bits"], inp["x"], inp["w"]
        if name == "tiny_ragged":
            xb, x, w = xb[:45], x[:45], w[:, :200]
        lay = O.prepare_weights(w, O.act_amax(x), 16)
        if name == "tiny_lora":
            A = (rng.standard_normal((w.shape[0], 16)) * np.sqrt(0.02)).astype(np.float32)
            Bm = (rng.standard_normal((16, w.shape[1])) * np.sqrt(0.02)).astype(np.float32)
            l1p, l2p = O.append_lora(lay["l1"], lay["l2"], lay["lam32"], A, Bm, 1.0)
            lay = dict(lay, l1=l1p, l2=l2p)
        return xb, x, lay


@pytest.mark.parametrize("name", [c[0] for c in LINEAR_CASES])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_linear_parity(S, name, out):
    _say(f"linear {name} out={out}")
    xb, x, lay = _linear_case(name)
    rng = np.random.default_rng(5)
    n = lay["qw"].shape[1]
    bias_v = O.bf16_from_f32(rng.standard_normal(n).astype(np.float32) * 0.1)
    ref = O.linear(x, lay, bias=bias_v)
    dl = device_layer(S, lay, LY.f32_to_bf16_bits(bias_v))
    y = S.svdq_linear(dev_bf16(xb), dl, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    err = rel(y_to_np(y), ref["y"])
    _say(f"  rel err {err:.3e}")
    assert err <= Y_TOL
    if out == "f32":
        assert err <= 1e-4


def _random_shape(k):
    rng = np.random.default_rng(1000 + k)
    b = int(rng.integers(1, 600))
    m = 64 * int(rng.integers(1, 41))
    n = int(rng.integers(1, 600))
    rank = int(rng.integers(0, min(64, m, n) + 1))
    return rng, b, m, n, rank, bool(rng.integers(0, 2))


@pytest.mark.parametrize("k", range(16))
def test_linear_random_shapes(S, k):
    """Seeded random layers (ragged b and n, any group count and rank up to
    64, with and without bias) on whatever schedule the planner picks: fp32
    output within 1e-4 of the oracle, and repeat calls bit-identical."""
    rng, b, m, n, rank, with_bias = _random_shape(k)
    _say(f"random layer {k}: b={b} m={m} n={n} rank={rank} bias={with_bias} "
         f"schedule={S.svdq_gemm_schedule(b, n, m)}")
    xb = workloads.random_bf16_bits(rng, (b, m), 1.5)
    x = LY.bf16_bits_to_f32(xb)
    lay = _oracle_layer(rng, m, n, rank, x)
    bias_v = O.bf16_from_f32(rng.standard_normal(n).astype(np.float32) * 0.1) if with_bias else None
    ref = O.linear(x, lay, bias=bias_v)["y"]
    dl = device_layer(S, lay, None if bias_v is None else LY.f32_to_bf16_bits(bias_v))
    xd = dev_bf16(xb)
    ys = [S.svdq_linear(xd, dl, torch.float32) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    err = rel(ys[0].cpu().numpy(), ref)
    _say(f"  rel err {err:.3e}")
    assert err <= 1e-4


def test_linear_equals_standalone_kernels_bitwise(S):
    """svdq_linear = act kernel then GEMM kernel; Z partials are summed in the
    same order in both routes, so the outputs agree bit for bit."""
    xb, x, lay = _linear_case("tiny_lora")
    dl = device_layer(S, lay)
    xd = dev_bf16(xb)
    y1 = S.svdq_linear(xd, dl, torch.float32)
    qd, asd, zd = S.svdq_quantize_act_lowrank_down(xd, dl.smooth_inv, dl.l1, dl.rank)
    y2 = S.svdq_gemm_w4a4_lowrank_up(qd, asd, zd, dl, xd.shape[0], torch.float32)
    y3 = S.svdq_linear(xd, dl, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y1, y3)  # deterministic across calls


@pytest.mark.parametrize("b,m,n", [(256, 4096, 256), (300, 2368, 200), (512, 3072, 1024)])
def test_splitk_deterministic_and_match_oracle(S, b, m, n):
    """Shapes whose tiles are split over several workgroups (partial sums
    published and added in a fixed order): repeated runs are bit-identical and
    match the oracle."""
    _say(f"split-K b={b} m={m} n={n}")
    rng = np.random.default_rng(b + m + n)
    xb = workloads.random_bf16_bits(rng, (b, m), 1.5)
    x = LY.bf16_bits_to_f32(xb)
    lay = _oracle_layer(rng, m, n, 16, x)
    ref = O.linear(x, lay)["y"]
    dl = device_layer(S, lay)
    xd = dev_bf16(xb)
    ys = [S.svdq_linear(xd, dl, torch.float32) for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])
    err = rel(ys[0].cpu().numpy(), ref)
    _say(f"  rel err {err:.3e}")
    assert err <= 1e-4


def test_splitk_workspace_garbage_and_alternating_shapes(S):
    """Split-K partial slots live in the caller's workspace: random initial
    bytes (whatever a previous launch or process could leave), two split
    shapes alternating on one workspace, and repeats must all give the same
    bits and the oracle's Y."""
    shapes = [(256, 4096, 256), (300, 2368, 520)]
    need = max(S.svdq_linear_workspace_size(b, m, n, 16) for b, m, n in shapes)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda")
    cases = []
    for (b, m, n) in shapes:
        sch = S.svdq_gemm_schedule(b, n, m)
        assert sch["split_workgroups"] > 0, sch
        rng = np.random.default_rng(b * 7 + n)
        xb = workloads.random_bf16_bits(rng, (b, m), 1.5)
        x = LY.bf16_bits_to_f32(xb)
        lay = _oracle_layer(rng, m, n, 16, x)
        cases.append((dev_bf16(xb), device_layer(S, lay), O.linear(x, lay)["y"]))
    first = {}
    for rep in range(3):
        for k, (xd, dl, ref) in enumerate(cases):
            _say(f"split-K workspace reuse rep={rep} shape={shapes[k]}")
            y = S.svdq_linear(xd, dl, torch.float32, workspace=ws)
            torch.cuda.synchronize()
            if rep == 0:
                first[k] = y
                assert rel(y.cpu().numpy(), ref) <= 1e-4
            else:
                assert torch.equal(y, first[k])
        if rep == 0:  # scribble over the workspace between rounds
            ws.random_(0, 256)


# The INT4 GEMM has three schedules: one tile per workgroup, every tile split
# into pieces (under half a round of tiles), or a split last round after full
# rounds of whole tiles.  Each case finds the smallest b x n (m = 1536) that the
# library schedules that way on this device.
SCHEDULE_KINDS = {
    "one_tile": lambda s: s["split_workgroups"] == 0,
    "split": lambda s: 0 < s["split_workgroups"] == s["grid"],
    "hybrid": lambda s: 0 < s["split_workgroups"] < s["grid"],
}


def _shape_for(S, kind, m=1536):
    best = None
    for tm in range(1, 48):
        for tn in range(1, 64):
            if best is not None and tm * tn >= best[0]:
                break
            if SCHEDULE_KINDS[kind](S.svdq_gemm_schedule(128 * tm, 128 * tn, m)):
                best = (tm * tn, tm, tn)
    assert best is not None, f"no {kind} schedule for this device"
    return 128 * best[1] - 37, 128 * best[2] - 5, m   # ragged rows and columns, same tiles


@pytest.mark.parametrize("kind", list(SCHEDULE_KINDS))
def test_schedule_kinds_match_oracle(S, kind):
    """Every schedule the planner can choose: bit-identical repeats, and rows
    spread over the whole output (every tile row) against the oracle."""
    b, n, m = _shape_for(S, kind)
    sch = S.svdq_gemm_schedule(b, n, m)
    assert SCHEDULE_KINDS[kind](sch)
    _say(f"schedule {kind}: b={b} m={m} n={n}: {sch}")
    rng = np.random.default_rng(11)
    xb = workloads.random_bf16_bits(rng, (b, m), 1.5)
    x = LY.bf16_bits_to_f32(xb)
    lay = _oracle_layer(rng, m, n, 32, x)
    dl = device_layer(S, lay)
    xd = dev_bf16(xb)
    ys = [S.svdq_linear(xd, dl, torch.float32) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    rows = np.unique(np.concatenate([np.arange(0, b, max(1, b // 48)), [b - 1]]))
    err = rel(ys[0].cpu().numpy()[rows], O.linear_rows(x[rows], lay))
    _say(f"  sampled rows {len(rows)}: rel err {err:.3e}")
    assert err <= 1e-4


# The unfused path rounds the W4A4 product to bf16 in y, the up-projection to
# bf16 in its own b x n output, and their sum to bf16 again: two roundings of
# full-size values where the fused path has one.  One round-to-nearest-even to
# bf16 costs about 1.66e-3 relative Frobenius error on these Gaussian-like
# outputs, and independent roundings add in quadrature, so the unfused path
# sits near sqrt(2) * 1.66e-3 = 2.35e-3 (2.36e-3 measured on the tiny layer) and
# cannot meet the fused layer's 2e-3.  Its bf16 bar is that figure with 25 %
# margin; fp32 output (one rounding of each part, no bf16) keeps 1e-4.
UNFUSED_BF16_TOL = 3e-3


@pytest.mark.parametrize("name", [c[0] for c in LINEAR_CASES])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_linear_unfused_parity(S, name, out):
    """Without the fusion (separate down- and up-projection kernels, a second
    b x n output and an addition) the layer is the same up to rounding."""
    _say(f"linear unfused {name} out={out}")
    xb, x, lay = _linear_case(name)
    rng = np.random.default_rng(5)
    n = lay["qw"].shape[1]
    bias_v = O.bf16_from_f32(rng.standard_normal(n).astype(np.float32) * 0.1)
    ref = O.linear(x, lay, bias=bias_v)
    dl = device_layer(S, lay, LY.f32_to_bf16_bits(bias_v))
    y = S.svdq_linear_unfused(dev_bf16(xb), dl, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    err = rel(y_to_np(y), ref["y"])
    _say(f"  rel err {err:.3e}")
    assert err <= (1e-4 if out == "f32" else UNFUSED_BF16_TOL)


@pytest.mark.parametrize("b,m,n,rank", [(300, 2368, 200, 16), (130, 4096, 96, 48)])
def test_linear_unfused_split_shapes(S, b, m, n, rank):
    """Shapes whose channel groups are split for the down-projection."""
    _say(f"linear unfused b={b} m={m} n={n} rank={rank}")
    rng = np.random.default_rng(b + rank)
    xb = workloads.random_bf16_bits(rng, (b, m), 1.5)
    x = LY.bf16_bits_to_f32(xb)
    lay = _oracle_layer(rng, m, n, rank, x)
    ref = O.linear(x, lay)["y"]
    dl = device_layer(S, lay)
    xd = dev_bf16(xb)
    yu = S.svdq_linear_unfused(xd, dl, torch.float32)
    yf = S.svdq_linear(xd, dl, torch.float32)
    torch.cuda.synchronize()
    assert rel(yu.cpu().numpy(), ref) <= 1e-4
    assert rel(yu.cpu().numpy(), yf.cpu().numpy()) <= 1e-5


def test_linear_unfused_rank0_is_the_fused_path(S):
    """At rank 0 both routes launch the same two kernels: identical bits."""
    rng = np.random.default_rng(3)
    xb = workloads.random_bf16_bits(rng, (77, 512), 1.5)
    x = LY.bf16_bits_to_f32(xb)
    lay = _oracle_layer(rng, 512, 136, 0, x)
    dl = device_layer(S, lay)
    xd = dev_bf16(xb)
    yu = S.svdq_linear_unfused(xd, dl, torch.bfloat16)
    yf = S.svdq_linear(xd, dl, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(yu, yf)


def test_linear_empty_batch(S):
    xb, x, lay = _linear_case("tiny")
    dl = device_layer(S, lay)
    for f in (S.svdq_linear, S.svdq_linear_unfused):
        y = f(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"), dl)
        torch.cuda.synchronize()
        assert y.shape == (0, 256)


def test_binding_rejects_mismatched_tensors(S):
    """Tensors whose device, dtype or shape do not match the layer raise before
    any launch (a kernel would otherwise read or write out of bounds)."""
    xb, x, lay = _linear_case("tiny")
    dl = device_layer(S, lay)
    xd = dev_bf16(xb)
    b, m = xd.shape
    y_ok = S.svdq_linear(xd, dl, torch.float32)
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="out_dtype"):
        S.svdq_linear(xd, dl, torch.float16)
    with pytest.raises(ValueError, match="dtype"):
        S.svdq_linear(xd, dl, torch.float32, y=torch.empty((b, dl.n), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="shape"):
        S.svdq_linear(xd, dl, torch.float32, y=torch.empty((b, dl.n - 1), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="dtype"):
        S.svdq_linear(xd.float(), dl)
    with pytest.raises(ValueError, match="channels"):
        S.svdq_linear(xd[:, :m - 64].contiguous(), dl)
    with pytest.raises(ValueError, match="GPU tensor"):
        S.svdq_linear(xd.cpu(), dl)
    qx, asc, z = S.svdq_quantize_act_lowrank_down(xd, dl.smooth_inv, dl.l1, dl.rank)
    with pytest.raises(ValueError, match="qx has shape"):
        S.svdq_gemm_w4a4_lowrank_up(qx, asc, z, dl, b - 1)
    with pytest.raises(ValueError, match="z has shape"):
        S.svdq_gemm_w4a4_lowrank_up(qx, asc, z[:, :1].contiguous(), dl)
    with pytest.raises(ValueError, match="qx has shape"):
        S.svdq_quantize_act_lowrank_down(xd, dl.smooth_inv, dl.l1, dl.rank, qx=qx[:, 1:].contiguous())
    # the valid calls still agree after the rejected ones
    y2 = S.svdq_gemm_w4a4_lowrank_up(qx, asc, z, dl, None, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y2, y_ok)


# ---------------------------------------------------------------------------
# full-size layers, sampled rows (the configurations the benchmark times)
# ---------------------------------------------------------------------------

FULL = ["pixart_fc1", "flux_qkv", "flux_fc2", "flux_single_fc", "flux_single_out",
        "flux_single_fc_b256", "flux_single_out_b256"]


@pytest.mark.parametrize("cfg", FULL)
def test_full_size_sampled(S, cfg):
    _say(f"full-size {cfg}: generating inputs and oracle layer")
    inp = workloads.make_inputs(cfg)
    c = inp["cfg"]
    x, xb = inp["x"], inp["x_bits"]
    b = x.shape[0]
    lay = O.prepare_weights(inp["w"], O.act_amax(x), c.rank, svd="arpack")
    if c.lora_rank:
        l1p, l2p = O.append_lora(lay["l1"], lay["l2"], lay["lam32"], inp["lora_a"], inp["lora_b"],
                                 inp["lora_scale"])
        lay = dict(lay, l1=l1p, l2=l2p)
    del inp
    dl = device_layer(S, lay)
    xd = dev_bf16(xb)
    _say(f"full-size {cfg}: running svdq_linear b={b} m={c.m} n={c.n} rank={lay['l1'].shape[1]}")
    y = S.svdq_linear(xd, dl, torch.bfloat16)
    qd, asd, zd = S.svdq_quantize_act_lowrank_down(xd, dl.smooth_inv, dl.l1, dl.rank)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, b, max(1, b // 40)), [b - 1]]))
    y_ref = O.linear_rows(x[rows], lay)
    err = rel(y_to_np(y)[rows], y_ref)
    _say(f"  sampled rows {len(rows)}: rel err {err:.3e}")
    assert err <= Y_TOL
    xt, qx, sx = O.quantize_activation(x[rows], lay["inv32"])
    qx_dev = LY.unpack_codes(qd[:, torch.from_numpy(rows).cuda(), :].cpu().numpy())
    assert np.array_equal(qx_dev, qx)
    assert np.array_equal(asd[:, torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16),
                          LY.f32_to_fp16_bits(np.ascontiguousarray(sx.T)))
    assert rel(zd.cpu().numpy()[rows], O.lowrank_down(xt, lay["l1"])) <= Z_TOL
