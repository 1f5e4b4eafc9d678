"""The allocation-free whole-layer call (dsv4_moe_forward_noalloc) against
dsv4_moe_forward on a caller-owned workspace, through the C ABI.  Both run
the same kernels in the same order, so their outputs must be equal bit for
bit.  Calls follow each other on the one static array: a 32-token batch
(grouped GEMM path), then smaller ones -- one token on the VALU path and 5
tokens on the mid-size router -- and the first batch again."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_expert_ffn_moe_amd as moe  # noqa: E402
from gpu_util import DevLayer, to_host  # noqa: E402
from oracle import Oracle, Weights  # noqa: E402


def _both(D, x, T, ids=None, rw=None, out_dtype=moe.MOE_DT_F32):
    dt = torch.float32 if out_dtype == moe.MOE_DT_F32 else torch.uint16
    a = torch.full((T, D.wl.H), -3.0, device="cuda:0").to(dt)
    b = torch.full((T, D.wl.H), -5.0, device="cuda:0").to(dt)
    moe.dsv4_moe_forward_noalloc(D.w, D.wr, x, T, D.wl.k, ids, rw, a, out_dtype)
    moe.dsv4_moe_forward(D.w, D.wr, x, T, D.wl.k, ids, rw, b, out_dtype, D.ws, D.ws_bytes)
    return to_host(a), to_host(b)


def test_noalloc_forward_equals_workspace_forward():
    L = synth.make_layer("verify_t32")             # drawn routing, 32 tokens
    D = DevLayer(L)
    print("noalloc: 32 tokens, drawn routing", flush=True)
    a, b = _both(D, D.x, 32, D.ids, D.rw)
    assert np.isfinite(a).all() and np.array_equal(a, b)
    ref = Oracle().forward(Weights.from_layer(L), L.wr, L.x, 6, ids=L.ids, w=L.w, tokens=[0, 31])
    rel = np.linalg.norm(a[[0, 31]] - ref) / np.linalg.norm(ref)
    assert rel <= 2e-3, rel
    print("noalloc: 1 token, router on x", flush=True)
    a1, b1 = _both(D, D.x[:1], 1)
    assert np.isfinite(a1).all() and np.array_equal(a1, b1)
    print("noalloc: 5 tokens, router on x, bf16 out", flush=True)
    a5, b5 = _both(D, D.x[:5], 5, out_dtype=moe.MOE_DT_BF16)
    assert np.array_equal(a5, b5)
    print("noalloc: 32 tokens again", flush=True)
    a2, b2 = _both(D, D.x, 32, D.ids, D.rw)
    assert np.array_equal(a2, a)
    assert moe.moe_device_status(D.ws) == 0


def test_noalloc_refuses_calls_beyond_its_array():
    L = synth.make_layer("tiny_t8")
    D = DevLayer(L, max_tokens=1)
    w4k = moe.make_weights(moe.MOE_W_FP4_E2M1_UE8M0_K32, 256, 4096, 2048, *[D.t[n] for n in (
        "gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")])
    big = 4096
    assert moe.moe_workspace_bytes(w4k, big, 6) > moe.MOE_NOALLOC_SCRATCH_BYTES
    out = torch.empty((1, 4096), dtype=torch.float32, device="cuda:0")
    with pytest.raises(moe.MoeError) as ei:
        moe.dsv4_moe_forward_noalloc(w4k, D.wr, D.x, big, 6, None, None, out, moe.MOE_DT_F32)
    assert ei.value.status == moe.MOE_ENOTSUP
