"""Full-size layers prepared by the LIBRARY (not the oracle), run on the GPU.

The other GPU parity tests feed the kernels layers the oracle prepared.  Here
the library's own host preparation (smoothing of Eq.(4), its truncated SVD of
Eq.(10), the residual and its INT4 quantization, Algorithm 1 steps 2-5 of the
SVDQuant review) builds the FLUX-shaped layers the benchmark times, and each
step is pinned against the oracle at that size:

  * lambda and 1/lambda bit-exact (the GPU calibration statistic first, also
    bit-exact);
  * the decomposition exact: ||W~ - (L1 L2 + R)||_F / ||W~||_F <= 1e-6 with the
    stored bf16 factors and the fp32 residual;
  * the SVD near-optimal (Eq.(10)): ||W~ - L1 L2||_F^2 <= (1 + 1e-3) times the
    oracle's (ARPACK factors rounded to bf16 the same way), and the energy the
    branch removes from the residual, ||W~||_F^2 - ||W~ - L1 L2||_F^2, at least
    (1 - 1e-3) sum_{i<=r} sigma_i^2 (ARPACK's singular values).  The raw
    ||L1 L2||_F^2 is not a usable pin: rounding a few dominant entries of the
    factors to bf16 moves it by about 1e-3 either way, while the removed energy
    stays within 1e-5 of the optimum;
  * codes and scales of the residual bit-exact against the oracle's quantizer
    applied to the library's own residual;
  * the LoRA-widened factors (sec. 7 Eq.(13)) bit-exact against the oracle;
  * then the whole layer through svdq_linear against the oracle's linear on
    that same layer, on sampled rows: bf16 output <= 2e-3, fp32 <= 1e-4;
  * the layer written to a layer file and read back (Algorithm 1 step 9)
    gives the same Y bit for bit.

Inputs are the seeded FLUX-shaped synthetic layers (workloads.py); every
expected value comes from the oracle.
"""
import sys

import numpy as np
import pytest

import workloads
from oracle import svdq_oracle as O
from tests import layout as LY

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a4_rank_corrected_amd as S
    S.lib()
    return S


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / np.linalg.norm(b)


@pytest.mark.parametrize("cfg", ["flux_qkv", "flux_single_fc"])
def test_library_prepared_full_size_layer(S, cfg, tmp_path):
    inp = workloads.make_inputs(cfg)
    c = inp["cfg"]
    x, xb, w = inp["x"], inp["x_bits"], inp["w"]
    b, m, n, r = x.shape[0], c.m, c.n, c.rank
    xd = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda().view(torch.bfloat16)

    _say(f"{cfg}: calibration statistic on the GPU, library preparation (b={b} m={m} n={n} rank {r})")
    amax = S.svdq_calibrate_act_amax(xd).cpu().numpy()
    assert np.array_equal(amax, O.act_amax(x))
    host = S.svdq_prepare_weights(w, amax, r, want_residual=True)

    _, lam32, inv32 = O.smoothing_lambda(amax, w)
    assert np.array_equal(host["lambda"], lam32)
    assert np.array_equal(host["smooth_inv"], inv32)

    wt = O.smooth_weight(w, lam32)
    l1 = LY.bf16_bits_to_f32(host["l1"]).T.astype(np.float64)   # [m][r]
    l2 = LY.bf16_bits_to_f32(host["l2"]).T.astype(np.float64)   # [r][n]
    low = l1 @ l2
    wt_norm = np.linalg.norm(wt)
    assert np.linalg.norm(wt - (low + host["residual"])) <= 1e-6 * wt_norm

    _say(f"{cfg}: oracle preparation (ARPACK SVD) for the optimality pins")
    ref = O.prepare_weights(w, amax, r, svd="arpack")
    tail_lib = np.linalg.norm(wt - low) ** 2
    tail_ref = np.linalg.norm(ref["r64"]) ** 2
    removed = wt_norm ** 2 - tail_lib
    optimum = float(np.sum(ref["sigma"][:r] ** 2))
    _say(f"{cfg}: tail energy ratio {tail_lib / tail_ref:.7f}, removed energy ratio {removed / optimum:.7f}")
    assert tail_lib <= (1 + 1e-3) * tail_ref
    assert removed >= (1 - 1e-3) * optimum
    del ref

    codes, sw = O.quantize_weight_residual(host["residual"])
    assert np.array_equal(LY.unpack_codes(host["qw"]), np.ascontiguousarray(codes.T))
    assert np.array_equal(host["wscale"], LY.f32_to_fp16_bits(sw))
    del codes, sw

    lay = LY.host_abi_to_oracle_layer(host)
    if c.lora_rank:
        l1w, l2w = S.svdq_append_lora(host["l1"], host["l2"], m, n, r, host["lambda"], inp["lora_a"],
                                      inp["lora_b"], inp["lora_scale"])
        e1, e2 = O.append_lora(lay["l1"], lay["l2"], lay["lam32"], inp["lora_a"], inp["lora_b"],
                               inp["lora_scale"])
        assert np.array_equal(l1w, LY.f32_to_bf16_bits(e1).T)
        assert np.array_equal(l2w, LY.f32_to_bf16_bits(e2).T)
        host = dict(host, l1=l1w, l2=l2w, rank=r + c.lora_rank)
        lay = dict(lay, l1=e1, l2=e2)
    host.pop("residual")
    del inp, w, wt, low

    dl = S.DeviceLayer(host)
    _say(f"{cfg}: svdq_linear on the library-prepared layer (rank {dl.rank})")
    y16 = S.svdq_linear(xd, dl, torch.bfloat16)
    y32 = S.svdq_linear(xd, dl, torch.float32)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, b, max(1, b // 40)), [b - 1]]))
    y_ref = O.linear_rows(x[rows], lay)
    ridx = torch.from_numpy(rows).cuda()
    e16 = rel(LY.bf16_bits_to_f32(y16[ridx].view(torch.int16).cpu().numpy().view(np.uint16)), y_ref)
    e32 = rel(y32[ridx].cpu().numpy(), y_ref)
    _say(f"{cfg}: sampled rows {len(rows)}: rel err bf16 {e16:.3e}, fp32 {e32:.3e}")
    assert e16 <= 2e-3
    assert e32 <= 1e-4

    path = str(tmp_path / f"{cfg}.svdq")
    S.svdq_save_layer(path, host, alpha=0.5)
    back = S.svdq_load_layer(path)
    y16b = S.svdq_linear(xd, S.DeviceLayer(back), torch.bfloat16)
    torch.cuda.synchronize()
    _say(f"{cfg}: layer file round trip, {len(open(path, 'rb').read()) >> 20} MiB")
    assert torch.equal(y16b, y16)
