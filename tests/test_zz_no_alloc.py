"""The allocation-free entry point svdq_linear_noalloc (device scratch held by
the library) against svdq_linear with a caller workspace, through the C ABI.

Both run the same kernels on the same plan, so the outputs must agree bit for
bit; each is also held to the layer's bar against the oracle (fp32 output
within 1e-4, codes and scales checked elsewhere).  Two calls in a row share the
scratch, the second with a smaller input, so stale contents of the first call
must not leak into the second.  A layer whose workspace exceeds the scratch is
refused on the host before any launch.
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


def _layer(S, rng, m, n, rank, x32):
    w = (rng.standard_normal((m, n)) / np.sqrt(m)).astype(np.float32)
    w[rng.choice(m, max(1, m // 64), replace=False)] *= 8
    lay = O.prepare_weights(w, O.act_amax(x32), rank)
    return lay, S.DeviceLayer(LY.oracle_layer_to_host_abi(lay))


def _rel(a, b):
    return np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b)


# (b, m, n, rank): a split-K shape (partial sums in the scratch, added by the reduction kernel),
# then a smaller one-tile shape on the same scratch
CASES = [(300, 2368, 520, 24), (45, 512, 200, 16)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_noalloc_matches_linear_two_calls(S, out):
    dt = torch.float32 if out == "f32" else torch.bfloat16
    for k, (b, m, n, rank) in enumerate(CASES):
        _say(f"noalloc call {k}: b={b} m={m} n={n} rank={rank} out={out} "
             f"schedule={S.svdq_gemm_schedule(b, n, m)}")
        rng = np.random.default_rng(100 + k)
        xb = workloads.random_bf16_bits(rng, (b, m), 1.5)
        x = LY.bf16_bits_to_f32(xb)
        lay, dl = _layer(S, rng, m, n, rank, x)
        xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        y_ref = S.svdq_linear(xd, dl, dt)
        y = torch.full((b, n), float("nan"), dtype=dt, device="cuda")
        S.svdq_linear_noalloc(xd, dl, dt, y=y)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
        yn = y.float().cpu().numpy()
        err = _rel(yn, O.linear(x, lay)["y"])
        _say(f"  bit-identical to svdq_linear; rel err vs oracle {err:.3e}")
        assert err <= (1e-4 if out == "f32" else 2e-3)


def test_noalloc_refuses_layers_above_the_scratch(S):
    """A batch whose workspace exceeds the scratch fails on the host with
    SVDQ_ERR_WORKSPACE and leaves y untouched."""
    cap = S.svdq_linear_noalloc_max_workspace()
    assert cap == 128 << 20
    m, n, rank = 4096, 64, 8
    b = 1
    while S.svdq_linear_workspace_size(b, m, n, rank) <= cap:
        b *= 2
    rng = np.random.default_rng(5)
    x32 = LY.bf16_bits_to_f32(workloads.random_bf16_bits(rng, (4, m), 1.0))
    _, dl = _layer(S, rng, m, n, rank, x32)
    xd = torch.zeros((b, m), dtype=torch.bfloat16, device="cuda")
    y = torch.full((b, n), 7.0, dtype=torch.float32, device="cuda")
    from w4a4_rank_corrected_amd import _binding as B
    with pytest.raises(B.SvdqError) as ei:
        S.svdq_linear_noalloc(xd, dl, torch.float32, y=y)
    assert ei.value.status == B.SVDQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))
