"""HIP graph capture of the whole layer: the library enqueues only kernels
(no memset or copy nodes), and the blocks that hand values to each other
through the workspace's slots return them to zero within the launch, so a
captured forward can be replayed any number of times.  Every replay, with
eager calls on the same workspace and host synchronisations in between, must
equal the eager result bit for bit."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_expert_ffn_moe_amd as moe  # noqa: E402
from gpu_util import DevLayer, to_host  # noqa: E402


@pytest.mark.parametrize("over", [
    dict(T=1),               # one token: front kernel + VALU GEMV with the h exchange
    dict(T=1, fused=True),   # one token: front kernel + the fused expert kernel (epoch-tagged words)
    dict(T=3, fmt="fp8"),    # front kernel + VALU GEMV (FP8), 3 tokens
    dict(T=6),               # mid-size router with act_quant, permute, grouped GEMM, combine
    dict(T=40),              # mid-size router with act_quant, permute, grouped GEMM, combine
])
def test_graph_replays_equal_the_eager_forward(over):
    over = dict(over)
    fused = over.pop("fused", False)
    moe.moe_debug_set_decode_fused(1 if fused else 0)
    try:
        _replays(over)
    finally:
        moe.moe_debug_set_decode_fused(0)


def _replays(over):
    L = synth.make_layer("tiny_t8", **over)
    D = DevLayer(L)
    T, H, k = L.wl.T, L.wl.H, L.wl.k
    print("graph replay", over, flush=True)

    def fwd(out):
        moe.dsv4_moe_forward(D.w, D.wr, D.x, T, k, None, None, out, moe.MOE_DT_F32, D.ws,
                             D.ws_bytes)

    out_e = torch.empty((T, H), dtype=torch.float32, device="cuda:0")
    out_g = torch.empty_like(out_e)
    fwd(out_e)
    ref = to_host(out_e)
    assert np.isfinite(ref).all()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
        fwd(out_g)
    for rep in range(4):
        out_g.fill_(-1.0)
        g.replay()
        got = to_host(out_g)
        assert np.array_equal(got, ref), f"replay {rep}"
        out_e.fill_(-2.0)
        fwd(out_e)
        assert np.array_equal(to_host(out_e), ref), f"eager after replay {rep}"
    assert moe.moe_device_status(D.ws) == 0
