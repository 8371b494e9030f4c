"""Replays of a captured HIP graph of the layer (all three settings).

A split-K launch is two kernels: the GEMM stores each piece's partial sums in
the caller's workspace and a reduction kernel adds them; a captured graph
replays both, and each replay overwrites every slot it reads.  Each replay runs
on new inputs copied in eagerly (with synchronizations between replays) and
must equal, bit for bit, the eager call on the same inputs.
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


def _inputs(b, m, n, rank, seed):
    rng = np.random.default_rng(seed)
    xs = [workloads.random_bf16_bits(rng, (b, m), 1.5) for _ in range(4)]
    w = (rng.standard_normal((m, n)) / np.sqrt(m)).astype(np.float32)
    return xs, w, O.act_amax(LY.bf16_bits_to_f32(xs[0]))


def _layer(S, fmt, w, a, rank):
    if fmt == "int4":
        lay = O.prepare_weights(w, a, rank)
        return S.DeviceLayer(LY.oracle_layer_to_host_abi(lay)), S.svdq_linear, S.svdq_linear_workspace_size
    if fmt == "w8a8":
        lay = O.prepare_weights_w8a8(w, a, rank)
        return (S.DeviceLayer8(LY.oracle_w8a8_to_host_abi(lay)), S.svdq_w8a8_linear,
                lambda b, m, n, r: S.svdq_w8a8_linear_workspace_size(b, m, n, r))
    lay = O.prepare_weights_fp4(w, a, rank)
    return (S.DeviceLayerFp4(LY.oracle_fp4_to_host_abi(lay, O.e4m3_bits)), S.svdq_fp4_linear,
            lambda b, m, n, r: S.svdq_fp4_linear_workspace_size(b, m, n, r))


@pytest.mark.parametrize("fmt", ["int4", "w8a8", "fp4"])
@pytest.mark.parametrize("b,m,n", [(256, 4096, 256), (300, 2368, 200), (130, 512, 260)])
def test_graph_replays_match_eager(S, fmt, b, m, n):
    _say(f"graph replay {fmt} b={b} m={m} n={n}")
    rank = 16
    xs, w, a = _inputs(b, m, n, rank, b + m + n)
    dl, linear, ws_size = _layer(S, fmt, w, a, rank)
    dev = torch.device("cuda")
    ws = torch.empty(max(ws_size(b, m, n, rank), 1), dtype=torch.uint8, device=dev)
    x_static = torch.empty((b, m), dtype=torch.bfloat16, device=dev)
    y_static = torch.empty((b, n), dtype=torch.float32, device=dev)
    to_dev = lambda bits: torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    # eager references (also warms the library up before capture)
    refs = []
    for xb in xs:
        refs.append(linear(to_dev(xb), dl, torch.float32, workspace=ws))
    torch.cuda.synchronize()
    x_static.copy_(to_dev(xs[0]))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        linear(x_static, dl, torch.float32, y=y_static, workspace=ws)
    torch.cuda.synchronize()
    for k in [1, 2, 3, 0, 2]:
        x_static.copy_(to_dev(xs[k]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_static, refs[k]), f"replay with input {k}"
        # eager work on the same workspace between replays
        yk = linear(to_dev(xs[(k + 1) % 4]), dl, torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(yk, refs[(k + 1) % 4])
