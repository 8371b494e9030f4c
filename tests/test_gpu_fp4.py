"""GPU parity of the NVFP4 setting (FP4 E2M1 codes with FP8 E4M3 scales per
16 channels and power-of-two tensor scales, plus the low-rank branch) against
the CPU oracle, through the C ABI.

Bars: codes and block-scale bytes bit-exact; the GEMM's products exact (checked
with unit and power-of-two scales, where every sum is exact in fp32); Z within
1e-4 and bit-identical to the INT4 path's Z (the same kernel); Y within 1e-5
(fp32 output of the GEMM alone), 1e-4 (fp32 output of the whole layer) or 2e-3
(bf16).  Layers are prepared by the oracle, so no expected value comes from the
product.
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


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def y_to_np(y):
    if y.dtype == torch.bfloat16:
        return LY.bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16))
    return y.cpu().numpy()


def device_layer_fp4(S, lay, bias_bits=None):
    return S.DeviceLayerFp4(LY.oracle_fp4_to_host_abi(lay, O.e4m3_bits), bias=bias_bits,
                            smoothing=lay.get("inv32") is not None)


def adversarial_blocks(rng, b, m):
    """bf16 rows whose 16-channel blocks exercise E2M1 ties, zero and
    underflowing blocks, large and subnormal magnitudes."""
    x = rng.standard_normal((b, m)).astype(np.float32)
    grid_ties = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5,
                          -5.0, -0.0], np.float32)
    for i in range(b):
        for blk in range(m // 16):
            kind = (i + blk) % 6
            seg = slice(16 * blk, 16 * blk + 16)
            if kind == 0:
                x[i, seg] = grid_ties * 2.0 ** rng.integers(-4, 4)   # amax 6*2^k: S = 2^k, exact ties
            elif kind == 1:
                x[i, seg] = 0.0
            elif kind == 2:
                x[i, seg] *= 1e-30                                  # block scale underflows
            elif kind == 3:
                x[i, seg] *= 3e4                                    # large block
            elif kind == 4:
                x[i, seg] *= 2.0 ** -133                            # bf16 subnormals
    return workloads.bf16_bits_of(x)


# ---------------------------------------------------------------------------
# NVFP4 activation quantization + down-projection
# ---------------------------------------------------------------------------

ACT_CASES = [
    # (b, m, rank, smoothing, adversarial, tensor-scale shift: t_x = auto * 2^shift)
    (64, 256, 16, True, False, 0),
    (37, 192, 0, False, False, 0),
    (1, 64, 8, True, False, 0),
    (200, 512, 16, True, True, 0),
    (33, 1024, 24, False, True, 0),
    (19, 4096, 32, True, False, 0),      # split Z
    (300, 12288, 48, True, False, 0),    # several LDS chunks per split
    (5, 64, 256, True, False, 0),        # maximum rank
    (64, 512, 16, True, False, -6),      # t_x too small: block scales saturate at 448
    (64, 512, 16, True, False, 20),      # t_x too large: block scales underflow
    (4100, 640, 40, True, False, 0),     # wide kernel (16-row strips, waves over the groups)
]


@pytest.mark.parametrize("b,m,rank,smooth,adv,shift", ACT_CASES)
def test_fp4_act_parity(S, b, m, rank, smooth, adv, shift):
    _say(f"fp4 act b={b} m={m} rank={rank} smooth={smooth} adv={adv} shift={shift}")
    rng = np.random.default_rng(b * 1000 + m + rank + shift)
    xb = adversarial_blocks(rng, b, m) if adv else workloads.random_bf16_bits(rng, (b, m), 2.0)
    x = LY.bf16_bits_to_f32(xb)
    inv = (1.0 / np.exp(rng.uniform(-2, 2, m))).astype(np.float32) if smooth else None
    l1 = O.bf16_from_f32((rng.standard_normal((m, rank)) / np.sqrt(m)).astype(np.float32))
    xt0 = O.smooth_activation(x, inv)
    t_x = O.fp4_tensor_scale(np.max(np.abs(xt0))) * 2.0 ** shift
    xt, qx, sbx = O.quantize_activation_fp4(x, inv, t_x)
    xd = dev_bf16(xb)
    invd = None if inv is None else dev_f32(inv)
    l1d = dev_bf16(np.ascontiguousarray(LY.f32_to_bf16_bits(l1).T)) if rank else None
    qd, asd, zd = S.svdq_fp4_quantize_act_lowrank_down(xd, invd, l1d, rank, t_x)
    torch.cuda.synchronize()
    assert np.array_equal(LY.unpack_fp4_codes(qd.cpu().numpy()), qx)
    assert np.array_equal(LY.unpack_fp4_scales(asd.cpu().numpy()), O.e4m3_bits(sbx))
    if shift == -6:
        assert np.any(sbx == 448.0)
    if rank:
        assert rel(zd.cpu().numpy(), O.lowrank_down(xt, l1)) <= Z_TOL
        _, _, z4 = S.svdq_quantize_act_lowrank_down(xd, invd, l1d, rank)
        torch.cuda.synchronize()
        assert torch.equal(zd, z4)


# ---------------------------------------------------------------------------
# NVFP4 GEMM + up-projection
# ---------------------------------------------------------------------------

def _oracle_layer_fp4(rng, m, n, rank, x32):
    w = (rng.standard_normal((m, n)) / np.sqrt(m)).astype(np.float32)
    w[rng.choice(m, max(1, m // 64), replace=False)] *= 8
    return O.prepare_weights_fp4(w, O.act_amax(x32), rank)


GEMM_CASES = [
    # (b, m, n, rank, bias)
    (64, 256, 256, 16, False),
    (37, 192, 100, 20, True),
    (130, 128, 260, 0, True),
    (1, 64, 7, 3, False),
    (256, 512, 384, 48, True),
    (256, 4096, 256, 16, True),   # 64 groups per tile (NVFP4 tiles are never split)
    (300, 2368, 200, 24, False),  # 37 groups, ragged edges
]


@pytest.mark.parametrize("b,m,n,rank,bias", GEMM_CASES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fp4_gemm_parity(S, b, m, n, rank, bias, out):
    _say(f"fp4 gemm b={b} m={m} n={n} rank={rank} bias={bias} out={out}")
    rng = np.random.default_rng(b + m + n + rank)
    xb = workloads.random_bf16_bits(rng, (b, m), 1.5)
    x = LY.bf16_bits_to_f32(xb)
    lay = _oracle_layer_fp4(rng, m, n, rank, x)
    bias_v = O.bf16_from_f32(rng.standard_normal(n).astype(np.float32)) if bias else None
    ref = O.linear_fp4(x, lay, bias=bias_v)
    z32 = ref["z"].astype(np.float32)
    xhat = O.dequantize_fp4_blocks(ref["qx"], ref["sbx"])
    what = O.dequantize_fp4_blocks(lay["qw"].T, lay["sbw"].T).T
    y_ref = (lay["t_x"] * lay["t_w"]) * (xhat @ what)
    if rank:
        y_ref = y_ref + O.lowrank_up(z32.astype(np.float64), lay["l2"])
    if bias:
        y_ref = y_ref + bias_v[None, :]
    dl = device_layer_fp4(S, lay, LY.f32_to_bf16_bits(bias_v) if bias else None)
    qd = dev_u8(LY.pack_fp4_codes(ref["qx"]))
    asd = dev_u8(LY.pack_fp4_scales(O.e4m3_bits(ref["sbx"])))
    y = S.svdq_fp4_gemm_lowrank_up(qd, asd, dev_f32(z32) if rank else None, dl, b,
                                   torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    yn = y_to_np(y)
    err = rel(yn, y_ref)
    _say(f"  rel err {err:.3e}")
    if out == "f32":
        assert err <= 1e-5
    else:
        # every element within one bf16 ulp of the correctly rounded reference;
        # the Frobenius bar and the flip rate need enough elements to average
        # the rounding (a single bf16 rounding can cost up to 2^-8 relative)
        yr = O.bf16_from_f64(y_ref).astype(np.float64)
        ulp = np.ldexp(1.0, np.frexp(np.where(yr != 0, yr, 1.0))[1] - 8)
        assert np.all(np.abs(yn - yr) <= ulp)
        if yn.size >= 256:
            assert err <= Y_TOL
            assert np.mean(yn != yr) < 0.01


@pytest.mark.parametrize("b,m,n", [(50, 256, 72), (256, 4096, 256), (300, 2368, 200)])
def test_fp4_gemm_exact_products(S, b, m, n):
    """Rank 0, fp32 output, tensor scales 1, block scales 2^k for k in [-2, 2]:
    every product and partial sum is a multiple of 2^-6 below 2^17, so the
    fp32 result is exact and equals the oracle's bit for bit, on one-tile and
    K-long shapes (NVFP4 tiles are never split)."""
    _say(f"fp4 gemm exact b={b} m={m} n={n}")
    rng = np.random.default_rng(b + m + n)
    qx = rng.integers(0, 16, (b, m)).astype(np.uint8)
    qw = rng.integers(0, 16, (n, m)).astype(np.uint8)          # per output column
    sbx = 2.0 ** rng.integers(-2, 3, (b, m // 16))
    sbw = 2.0 ** rng.integers(-2, 3, (n, m // 16))
    xhat = O.dequantize_fp4_blocks(qx, sbx)
    what = O.dequantize_fp4_blocks(qw, sbw)
    y_ref = xhat @ what.T
    assert np.all(np.abs(y_ref) < 2 ** 17)
    host = {"m": m, "n": n, "rank": 0, "t_x": 1.0, "t_w": 1.0, "qw": LY.pack_fp4_codes(qw),
            "wscale": LY.pack_fp4_scales(O.e4m3_bits(sbw)), "l1": np.zeros((0, m), np.uint16),
            "l2": np.zeros((n, 0), np.uint16), "smooth_inv": np.ones(m, np.float32)}
    dl = S.DeviceLayerFp4(host, smoothing=False)
    qd = dev_u8(LY.pack_fp4_codes(qx))
    asd = dev_u8(LY.pack_fp4_scales(O.e4m3_bits(sbx)))
    ys = [S.svdq_fp4_gemm_lowrank_up(qd, asd, None, dl, b, torch.float32) for _ in range(2)]
    torch.cuda.synchronize()
    assert np.array_equal(ys[0].cpu().numpy(), y_ref.astype(np.float32))
    assert torch.equal(ys[0], ys[1])


@pytest.mark.parametrize("m", [256, 4096])
def test_fp4_gemm_every_block_scale(S, m):
    """Every nonzero E4M3 block scale (codes 1..126, subnormals included) on
    both operands: row i of X and column j of W use one scale each, so every
    partial sum is s_i s_j (at most 8 significant bits) times a multiple of 1/4
    below 2^14, exact in fp32, and the result equals the oracle's bit for bit.
    m = 256 (all codes) runs one tile per workgroup; m = 4096 (codes of
    magnitude <= 1, to keep the sums below 2^14) runs 64 groups per
    tile."""
    b, n = 126, 130
    _say(f"fp4 gemm every block scale m={m}")
    rng = np.random.default_rng(m)
    pool = np.arange(16, dtype=np.uint8) if m <= 256 else np.array([0, 1, 2, 8, 9, 10], np.uint8)
    qx = rng.choice(pool, (b, m))
    qw = rng.choice(pool, (n, m))
    cx, cw = O.e2m1_values(qx), O.e2m1_values(qw)
    assert (np.abs(cx) @ np.abs(cw).T).max() < 2 ** 14
    codes_x = (np.arange(b) % 126 + 1).astype(np.uint8)
    codes_w = (np.arange(n) % 126 + 1).astype(np.uint8)
    sbx = np.repeat(O.e4m3_from_bits(codes_x)[:, None], m // 16, axis=1)
    sbw = np.repeat(O.e4m3_from_bits(codes_w)[:, None], m // 16, axis=1)
    y_ref = O.dequantize_fp4_blocks(qx, sbx) @ O.dequantize_fp4_blocks(qw, sbw).T
    host = {"m": m, "n": n, "rank": 0, "t_x": 1.0, "t_w": 1.0, "qw": LY.pack_fp4_codes(qw),
            "wscale": LY.pack_fp4_scales(O.e4m3_bits(sbw)), "l1": np.zeros((0, m), np.uint16),
            "l2": np.zeros((n, 0), np.uint16), "smooth_inv": np.ones(m, np.float32)}
    dl = S.DeviceLayerFp4(host, smoothing=False)
    y = S.svdq_fp4_gemm_lowrank_up(dev_u8(LY.pack_fp4_codes(qx)), dev_u8(LY.pack_fp4_scales(O.e4m3_bits(sbx))),
                                   None, dl, b, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y_ref.astype(np.float32))


# ---------------------------------------------------------------------------
# whole NVFP4 layer
# ---------------------------------------------------------------------------

def _linear_case(name):
    rng = np.random.default_rng(11)
    inp = workloads.make_inputs("tiny")
    xb, x, w = inp["x_bits"], inp["x"], inp["w"]
    if name == "tiny_ragged":
        xb, x, w = xb[:45], x[:45], w[:, :200]
    rank = 0 if name == "tiny_rank0" else 16
    lay = O.prepare_weights_fp4(w, O.act_amax(x), rank)
    if name == "tiny_lora":
        A = (rng.standard_normal((w.shape[0], 16)) * np.sqrt(0.02)).astype(np.float32)
        Bm = (rng.standard_normal((16, w.shape[1])) * np.sqrt(0.02)).astype(np.float32)
        l1p, l2p = O.append_lora(lay["l1"], lay["l2"], lay["lam32"], A, Bm, 1.0)
        lay = dict(lay, l1=l1p, l2=l2p)
    return xb, x, lay


@pytest.mark.parametrize("name", ["tiny", "tiny_ragged", "tiny_lora", "tiny_rank0"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fp4_linear_parity(S, name, out):
    _say(f"fp4 linear {name} out={out}")
    xb, x, lay = _linear_case(name)
    rng = np.random.default_rng(5)
    n = lay["qw"].shape[1]
    bias_v = O.bf16_from_f32(rng.standard_normal(n).astype(np.float32) * 0.1)
    ref = O.linear_fp4(x, lay, bias=bias_v)
    dl = device_layer_fp4(S, lay, LY.f32_to_bf16_bits(bias_v))
    y = S.svdq_fp4_linear(dev_bf16(xb), dl, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    err = rel(y_to_np(y), ref["y"])
    _say(f"  rel err {err:.3e}")
    assert err <= (1e-4 if out == "f32" else Y_TOL)


def test_fp4_linear_equals_standalone_kernels_bitwise(S):
    xb, x, lay = _linear_case("tiny_lora")
    dl = device_layer_fp4(S, lay)
    xd = dev_bf16(xb)
    y1 = S.svdq_fp4_linear(xd, dl, torch.float32)
    qd, asd, zd = S.svdq_fp4_quantize_act_lowrank_down(xd, dl.smooth_inv, dl.l1, dl.rank, dl.t_x)
    y2 = S.svdq_fp4_gemm_lowrank_up(qd, asd, zd, dl, xd.shape[0], torch.float32)
    y3 = S.svdq_fp4_linear(xd, dl, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)


def test_fp4_linear_empty_batch(S):
    xb, x, lay = _linear_case("tiny")
    dl = device_layer_fp4(S, lay)
    y = S.svdq_fp4_linear(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"), dl)
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


def test_fp4_linear_full_size_sampled(S):
    """The FLUX.1 attention-QKV layer at its full size (b = 4608 tokens,
    m = 3072, n = 9216) with the rank-32 branch, checked on sampled rows."""
    _say("fp4 linear full-size flux_qkv: generating inputs and oracle layer")
    inp = workloads.make_inputs("flux_qkv")
    x, xb = inp["x"], inp["x_bits"]
    b = x.shape[0]
    lay = O.prepare_weights_fp4(inp["w"], O.act_amax(x), 32, svd="arpack")
    del inp
    dl = device_layer_fp4(S, lay)
    xd = dev_bf16(xb)
    _say(f"fp4 linear full-size flux_qkv: running b={b}")
    y = S.svdq_fp4_linear(xd, dl, torch.bfloat16)
    qd, asd, zd = S.svdq_fp4_quantize_act_lowrank_down(xd, dl.smooth_inv, dl.l1, dl.rank, dl.t_x)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, b, max(1, b // 40)), [b - 1]]))
    ref = O.linear_fp4(x[rows], lay)
    err = rel(y_to_np(y)[rows], ref["y"])
    _say(f"  sampled rows {len(rows)}: rel err {err:.3e}")
    assert err <= Y_TOL
    ridx = torch.from_numpy(rows).cuda()
    assert np.array_equal(LY.unpack_fp4_codes(qd[:, ridx, :].cpu().numpy()), ref["qx"])
    assert np.array_equal(LY.unpack_fp4_scales(asd[:, ridx, :].cpu().numpy()), O.e4m3_bits(ref["sbx"]))
    assert rel(zd.cpu().numpy()[rows], ref["z"]) <= Z_TOL


# ---------------------------------------------------------------------------
# seeded random layers on whatever schedule the planner picks
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("k", range(8))
def test_fp4_linear_random_shapes(S, k):
    """Seeded random NVFP4 layers (ragged b and n, any group count and rank up to
    64, with and without bias): fp32 output within 1e-4 of the oracle, and
    repeat calls bit-identical."""
    rng = np.random.default_rng(3000 + k)
    b, m, n = int(rng.integers(1, 600)), 64 * int(rng.integers(1, 41)), int(rng.integers(1, 600))
    rank = int(rng.integers(0, min(64, m, n) + 1))
    with_bias = bool(rng.integers(0, 2))
    _say(f"random NVFP4 layer {k}: b={b} m={m} n={n} rank={rank} bias={with_bias} "
         f"schedule={S.svdq_gemm_schedule(b, n, m, 'fp4')}")
    xb = workloads.random_bf16_bits(rng, (b, m), 1.5)
    x = LY.bf16_bits_to_f32(xb)
    w = (rng.standard_normal((m, n)) / np.sqrt(m)).astype(np.float32)
    w[rng.choice(m, max(1, m // 64), replace=False)] *= 8
    lay = O.prepare_weights_fp4(w, O.act_amax(x), rank)
    bias_v = O.bf16_from_f32(rng.standard_normal(n).astype(np.float32) * 0.1) if with_bias else None
    ref = O.linear_fp4(x, lay, bias=bias_v)["y"]
    dl = device_layer_fp4(S, lay, None if bias_v is None else LY.f32_to_bf16_bits(bias_v))
    xd = dev_bf16(xb)
    ys = [S.svdq_fp4_linear(xd, dl, torch.float32) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    err = rel(ys[0].cpu().numpy(), ref)
    _say(f"  rel err {err:.3e}")
    assert err <= 1e-4
