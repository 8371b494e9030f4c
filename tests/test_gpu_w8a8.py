"""GPU parity of the 8-bit setting (per-token / per-channel INT8 with the
low-rank branch) against the CPU oracle, through the C ABI.

Bars: INT8 codes and fp16 scales bit-exact; integer products exact (checked
through fp32 outputs that carry them exactly); Z within 1e-4 and bit-identical
to the INT4 path's Z (the same kernel); Y within 1e-5 (fp32 output of the GEMM
alone), 1e-4 (fp32 output of the whole layer) or 2e-3 (bf16).  Layers are
prepared by the oracle, so no expected value comes from the product.
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


def dev_f16_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.float16)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def y_to_np(y):
    if y.dtype == torch.bfloat16:
        return LY.bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16))
    return y.cpu().numpy()


def device_layer8(S, lay, bias_bits=None):
    return S.DeviceLayer8(LY.oracle_w8a8_to_host_abi(lay), bias=bias_bits,
                          smoothing=lay.get("inv32") is not None)


def adversarial_rows(rng, b, m):
    """bf16 rows exercising ties, zero / underflowing / saturating rows and subnormals."""
    x = rng.standard_normal((b, m)).astype(np.float32)
    for i in range(b):
        kind = i % 7
        if kind == 0:
            x[i] = rng.integers(-127, 128, m)
            x[i, 0] = 127.0                      # s = 1: exact integer codes
        elif kind == 1:
            x[i] = rng.integers(-127, 127, m) + 0.5   # exact .5 ties
            x[i, 0] = 127.0
        elif kind == 2:
            x[i] = 0.0                           # all-zero row
        elif kind == 3:
            x[i] *= 1e-30                        # fp16 scale underflows to 0
        elif kind == 4:
            x[i] *= 1e9                          # scale saturates at 65504
        elif kind == 5:
            x[i] = rng.integers(-254, 255, m) * 0.25   # ties against s = 0.5
            x[i, 0] = 63.5
        elif kind == 6:
            x[i] *= 2.0 ** -133                  # bf16 subnormals
    return workloads.bf16_bits_of(x)


# ---------------------------------------------------------------------------
# per-token activation quantization + down-projection
# ---------------------------------------------------------------------------

ACT8_CASES = [
    # (b, m, rank, smoothing, adversarial)
    (64, 256, 16, True, False),
    (37, 192, 0, False, False),
    (1, 64, 8, True, False),
    (200, 512, 16, True, True),
    (33, 1024, 24, False, True),     # 2 pieces per lane
    (19, 4096, 16, True, False),     # 8 pieces per lane, split Z
    (7, 12288, 16, True, True),      # 24 pieces per lane
    (5, 16384, 16, True, False),     # row read twice (beyond the register budget)
    (3, 131072, 0, True, False),     # largest m
    (4100, 640, 24, True, False),    # Z by the wide kernel (16-row strips, waves over the groups)
]


@pytest.mark.parametrize("b,m,rank,smooth,adv", ACT8_CASES)
def test_act8_parity(S, b, m, rank, smooth, adv):
    _say(f"act8 b={b} m={m} rank={rank} smooth={smooth} adv={adv}")
    rng = np.random.default_rng(b * 1000 + m + rank)
    xb = adversarial_rows(rng, b, m) if adv else workloads.random_bf16_bits(rng, (b, m), 2.0)
    x = LY.bf16_bits_to_f32(xb)
    inv = (1.0 / np.exp(rng.uniform(-2, 2, m))).astype(np.float32) if smooth else None
    l1 = O.bf16_from_f32((rng.standard_normal((m, rank)) / np.sqrt(m)).astype(np.float32))
    xt, qx, sx = O.quantize_activation_w8a8(x, inv)
    xd = dev_bf16(xb)
    invd = None if inv is None else dev_f32(inv)
    l1d = dev_bf16(np.ascontiguousarray(LY.f32_to_bf16_bits(l1).T)) if rank else None
    qd, asd, zd = S.svdq_w8a8_quantize_act_lowrank_down(xd, invd, l1d, rank)
    torch.cuda.synchronize()
    assert np.array_equal(LY.unpack_codes8(qd.cpu().numpy()), qx)
    assert np.array_equal(asd.cpu().numpy().view(np.uint16), LY.f32_to_fp16_bits(sx))
    if rank:
        assert rel(zd.cpu().numpy(), O.lowrank_down(xt, l1)) <= Z_TOL
        # the same down-projection kernel and summation order as the INT4 path
        _, _, z4 = S.svdq_quantize_act_lowrank_down(xd, invd, l1d, rank)
        torch.cuda.synchronize()
        assert torch.equal(zd, z4)


# ---------------------------------------------------------------------------
# 8-bit GEMM + up-projection
# ---------------------------------------------------------------------------

def _oracle_layer8(rng, m, n, rank, x32):
    w = (rng.standard_normal((m, n)) / np.sqrt(m)).astype(np.float32)
    w[rng.choice(m, max(1, m // 64), replace=False)] *= 8
    return O.prepare_weights_w8a8(w, O.act_amax(x32), rank)


GEMM8_CASES = [
    # (b, m, n, rank, bias)
    (64, 256, 256, 16, False),
    (37, 192, 100, 20, True),     # ragged b, n, rank not a multiple of 8
    (130, 128, 260, 0, True),     # rank 0 = plain W8A8
    (1, 64, 7, 3, False),
    (256, 512, 384, 48, True),
    (256, 4096, 256, 16, True),   # split-K: int32 partials
    (300, 2368, 200, 24, False),  # split-K: uneven splits, ragged edges
]


@pytest.mark.parametrize("b,m,n,rank,bias", GEMM8_CASES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm8_parity(S, b, m, n, rank, bias, out):
    _say(f"gemm8 b={b} m={m} n={n} rank={rank} bias={bias} out={out}")
    rng = np.random.default_rng(b + m + n + rank)
    xb = workloads.random_bf16_bits(rng, (b, m), 1.5)
    x = LY.bf16_bits_to_f32(xb)
    lay = _oracle_layer8(rng, m, n, rank, x)
    bias_v = O.bf16_from_f32(rng.standard_normal(n).astype(np.float32)) if bias else None
    ref = O.linear_w8a8(x, lay, bias=bias_v)
    # the kernel consumes the fp32 Z it is given: the reference takes the same Z
    z32 = ref["z"].astype(np.float32)
    y_ref = ref["sx"][:, None].astype(np.float64) * ref["isum"] * lay["sw"][None, :].astype(np.float64)
    if rank:
        y_ref = y_ref + O.lowrank_up(z32.astype(np.float64), lay["l2"])
    if bias:
        y_ref = y_ref + bias_v[None, :]
    dl = device_layer8(S, lay, LY.f32_to_bf16_bits(bias_v) if bias else None)
    qd = torch.from_numpy(LY.pack_codes8(ref["qx"])).cuda()
    asd = dev_f16_bits(LY.f32_to_fp16_bits(ref["sx"]))
    y = S.svdq_w8a8_gemm_lowrank_up(qd, asd, dev_f32(z32) if rank else None, dl, b,
                                    torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    yn = y_to_np(y)
    err = rel(yn, y_ref)
    _say(f"  rel err {err:.3e}")
    assert err <= (1e-5 if out == "f32" else Y_TOL)
    if out == "bf16":
        assert np.mean(yn != O.bf16_from_f64(y_ref)) < 0.01


@pytest.mark.parametrize("b,m,n", [(50, 256, 72), (256, 4096, 256), (300, 2368, 200)])
def test_gemm8_exact_integer_sums(S, b, m, n):
    """Unit scales, rank 0, fp32 output: Y = qx qw exactly (|sum| < 2^24), on
    one-tile and split-K schedules (int32 partials)."""
    _say(f"gemm8 exact sums b={b} m={m} n={n}")
    rng = np.random.default_rng(b + m)
    qx = rng.integers(-127, 128, (b, m)).astype(np.int16)
    qw = rng.integers(-127, 128, (m, n)).astype(np.int16)
    if m <= 512:
        qx[:3] = 127
        qw[:, :2] = -127                                    # extreme sums -127^2 m
    isum = qx.astype(np.int64) @ qw.astype(np.int64)
    assert np.abs(isum).max() < 2 ** 24
    host = {"m": m, "n": n, "rank": 0, "qw": LY.pack_codes8(np.ascontiguousarray(qw.T)),
            "wscale": LY.f32_to_fp16_bits(np.ones(n, np.float32)),
            "l1": np.zeros((0, m), np.uint16), "l2": np.zeros((n, 0), np.uint16),
            "smooth_inv": np.ones(m, np.float32)}
    dl = S.DeviceLayer8(host, smoothing=False)
    qd = torch.from_numpy(LY.pack_codes8(qx)).cuda()
    asd = dev_f16_bits(LY.f32_to_fp16_bits(np.ones(b, np.float32)))
    ys = [S.svdq_w8a8_gemm_lowrank_up(qd, asd, None, dl, b, torch.float32) for _ in range(2)]
    torch.cuda.synchronize()
    assert np.array_equal(ys[0].cpu().numpy(), isum.astype(np.float32))
    assert torch.equal(ys[0], ys[1])


# ---------------------------------------------------------------------------
# whole 8-bit layer
# ---------------------------------------------------------------------------

def _linear8_case(name):
    rng = np.random.default_rng(11)
    inp = workloads.make_inputs("tiny")
    xb, x, w = inp["x_bits"], inp["x"], inp["w"]
    if name == "tiny_ragged":
        xb, x, w = xb[:45], x[:45], w[:, :200]
    lay = O.prepare_weights_w8a8(w, O.act_amax(x), 16)
    if name == "tiny_lora":
        A = (rng.standard_normal((w.shape[0], 16)) * np.sqrt(0.02)).astype(np.float32)
        Bm = (rng.standard_normal((16, w.shape[1])) * np.sqrt(0.02)).astype(np.float32)
        l1p, l2p = O.append_lora(lay["l1"], lay["l2"], lay["lam32"], A, Bm, 1.0)
        lay = dict(lay, l1=l1p, l2=l2p)
    if name == "tiny_rank0":
        lay = O.prepare_weights_w8a8(w, O.act_amax(x), 0)
    return xb, x, lay


@pytest.mark.parametrize("name", ["tiny", "tiny_ragged", "tiny_lora", "tiny_rank0"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_linear8_parity(S, name, out):
    _say(f"linear8 {name} out={out}")
    xb, x, lay = _linear8_case(name)
    rng = np.random.default_rng(5)
    n = lay["qw"].shape[1]
    bias_v = O.bf16_from_f32(rng.standard_normal(n).astype(np.float32) * 0.1)
    ref = O.linear_w8a8(x, lay, bias=bias_v)
    dl = device_layer8(S, lay, LY.f32_to_bf16_bits(bias_v))
    y = S.svdq_w8a8_linear(dev_bf16(xb), dl, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    err = rel(y_to_np(y), ref["y"])
    _say(f"  rel err {err:.3e}")
    assert err <= (1e-4 if out == "f32" else Y_TOL)


def test_linear8_equals_standalone_kernels_bitwise(S):
    xb, x, lay = _linear8_case("tiny_lora")
    dl = device_layer8(S, lay)
    xd = dev_bf16(xb)
    y1 = S.svdq_w8a8_linear(xd, dl, torch.float32)
    qd, asd, zd = S.svdq_w8a8_quantize_act_lowrank_down(xd, dl.smooth_inv, dl.l1, dl.rank)
    y2 = S.svdq_w8a8_gemm_lowrank_up(qd, asd, zd, dl, xd.shape[0], torch.float32)
    y3 = S.svdq_w8a8_linear(xd, dl, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)


def test_linear8_empty_batch(S):
    xb, x, lay = _linear8_case("tiny")
    dl = device_layer8(S, lay)
    y = S.svdq_w8a8_linear(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"), dl)
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


def test_linear8_full_size_sampled(S):
    """The FLUX.1 attention-QKV layer at its full size (b = 4608 tokens, m =
    3072, n = 9216) with the rank-16 branch, checked on sampled rows."""
    _say("linear8 full-size flux_qkv: generating inputs and oracle layer")
    inp = workloads.make_inputs("flux_qkv")
    x, xb = inp["x"], inp["x_bits"]
    b = x.shape[0]
    lay = O.prepare_weights_w8a8(inp["w"], O.act_amax(x), 16, svd="arpack")
    del inp
    dl = device_layer8(S, lay)
    xd = dev_bf16(xb)
    _say(f"linear8 full-size flux_qkv: running b={b}")
    y = S.svdq_w8a8_linear(xd, dl, torch.bfloat16)
    qd, asd, zd = S.svdq_w8a8_quantize_act_lowrank_down(xd, dl.smooth_inv, dl.l1, dl.rank)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, b, max(1, b // 40)), [b - 1]]))
    ref = O.linear_w8a8(x[rows], lay)
    err = rel(y_to_np(y)[rows], ref["y"])
    _say(f"  sampled rows {len(rows)}: rel err {err:.3e}")
    assert err <= Y_TOL
    ridx = torch.from_numpy(rows).cuda()
    assert np.array_equal(LY.unpack_codes8(qd[:, ridx, :].cpu().numpy()), ref["qx"])
    assert np.array_equal(asd[ridx].cpu().numpy().view(np.uint16), LY.f32_to_fp16_bits(ref["sx"]))
    assert rel(zd.cpu().numpy()[rows], ref["z"]) <= Z_TOL


# ---------------------------------------------------------------------------
# seeded random layers on whatever schedule the planner picks
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("k", range(8))
def test_linear8_random_shapes(S, k):
    """Seeded random 8-bit layers (ragged b and n, any group count and rank up to
    64, with and without bias): fp32 output within 1e-4 of the oracle, and
    repeat calls bit-identical."""
    rng = np.random.default_rng(2000 + k)
    b, m, n = int(rng.integers(1, 600)), 64 * int(rng.integers(1, 41)), int(rng.integers(1, 600))
    rank = int(rng.integers(0, min(64, m, n) + 1))
    with_bias = bool(rng.integers(0, 2))
    _say(f"random 8-bit layer {k}: b={b} m={m} n={n} rank={rank} bias={with_bias} "
         f"schedule={S.svdq_gemm_schedule(b, n, m, 'w8a8')}")
    xb = workloads.random_bf16_bits(rng, (b, m), 1.5)
    x = LY.bf16_bits_to_f32(xb)
    w = (rng.standard_normal((m, n)) / np.sqrt(m)).astype(np.float32)
    w[rng.choice(m, max(1, m // 64), replace=False)] *= 8
    lay = O.prepare_weights_w8a8(w, O.act_amax(x), rank)
    bias_v = O.bf16_from_f32(rng.standard_normal(n).astype(np.float32) * 0.1) if with_bias else None
    ref = O.linear_w8a8(x, lay, bias=bias_v)["y"]
    dl = device_layer8(S, lay, None if bias_v is None else LY.f32_to_bf16_bits(bias_v))
    xd = dev_bf16(xb)
    ys = [S.svdq_w8a8_linear(xd, dl, torch.float32) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    err = rel(ys[0].cpu().numpy(), ref)
    _say(f"  rel err {err:.3e}")
    assert err <= 1e-4
