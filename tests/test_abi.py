"""CPU tests of the C-ABI boundary: the library loads, exports every entry
point that include/moe.h declares, sizes its workspace, and rejects bad
arguments on the host before any HIP call is made (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

moe = pytest.importorskip("bit_expert_ffn_moe_amd")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s+\**\s*([a-z_0-9]+)\s*\(", src, re.M)
    return sorted(set(names))


def test_header_declares_the_documented_entry_points():
    names = _declared()
    for n in ["moe_route", "act_quant_fp8", "moe_permute", "moe_expert_ffn", "moe_combine",
              "dsv4_moe_forward", "moe_workspace_bytes", "moe_workspace_init",
              "moe_status_string", "moe_device_status", "moe_debug_intermediates"]:
        assert n in names, n


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIBRARY_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in _declared():
        assert n in exported, n
        assert hasattr(moe._lib, n)
    assert set(moe.EXPORTED) == set(_declared())


def test_library_links_no_oracle_code():
    out = subprocess.run(["nm", "-D", moe.LIBRARY_PATH], check=True, capture_output=True,
                         text=True).stdout
    assert "orc_" not in out
    deps = subprocess.run(["ldd", moe.LIBRARY_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in deps


def _w(fmt=1, E=256, H=4096, I=2048, ptr=0x10000):
    return moe.moe_weights(fmt, E, H, I, ptr, ptr, ptr, ptr, ptr, ptr)


def test_workspace_bytes_monotone_and_sized():
    w = _w()
    b1 = moe.moe_workspace_bytes(w, 1, 6)
    b32 = moe.moe_workspace_bytes(w, 32, 6)
    b8k = moe.moe_workspace_bytes(w, 8192, 6)
    assert 0 < b1 < b32 < b8k
    R = 8192 * 7
    assert b8k >= R * 4096 * 4 + R * 2048 + 8192 * 4096   # y rows + hq + xq at least
    assert moe.moe_workspace_bytes(_w(fmt=7), 1, 6) == 0
    assert moe.moe_workspace_bytes(w, 0, 6) == 0
    assert moe.moe_workspace_bytes(w, 1, 300) == 0


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert moe.moe_status_string(s)
    assert "unknown" in moe.moe_status_string(42)


@pytest.mark.parametrize("case,expect", [
    ("null_x", moe.MOE_EINVAL),
    ("bad_k", moe.MOE_EINVAL),
    ("k_over_16", moe.MOE_ENOTSUP),
    ("h_not_128", moe.MOE_EINVAL),
    ("misaligned", moe.MOE_EALIGN),
    ("small_ws", moe.MOE_EWORKSPACE),
    ("ws_misaligned", moe.MOE_EALIGN),
])
def test_route_rejects_bad_arguments_on_host(case, expect):
    p, ws = 0x100000, 0x200000
    args = dict(x=p, wr=p, T=4, H=4096, E=256, k=6, ids=p, w=p, ws=ws, wsb=1 << 30)
    if case == "null_x":
        args["x"] = None
    elif case == "bad_k":
        args["k"] = 0
    elif case == "k_over_16":
        args["k"] = 17
    elif case == "h_not_128":
        args["H"] = 4000
    elif case == "misaligned":
        args["ids"] = p + 4
    elif case == "small_ws":
        args["wsb"] = 100
    elif case == "ws_misaligned":
        args["ws"] = ws + 16
    rc = moe.raw_call("moe_route", args["x"], args["wr"], args["T"], args["H"], args["E"],
                      args["k"], args["ids"], args["w"], args["ws"], args["wsb"], None)
    assert rc == expect


def test_forward_rejects_bad_arguments_on_host():
    p, ws = 0x100000, 0x200000
    w = _w(ptr=p)
    big = 1 << 40
    f = moe._lib.dsv4_moe_forward
    # routing ids without weights
    assert f(ctypes.byref(w), p, p, 4, 6, p, None, p, 2, ws, big, None) == moe.MOE_EINVAL
    # unknown out dtype
    assert f(ctypes.byref(w), p, p, 4, 6, None, None, p, 9, ws, big, None) == moe.MOE_EINVAL
    # unknown weight format
    w2 = _w(fmt=3, ptr=p)
    assert f(ctypes.byref(w2), p, p, 4, 6, None, None, p, 2, ws, big, None) == moe.MOE_ENOTSUP
    # misaligned weight pointer
    w3 = _w(ptr=p + 8)
    assert f(ctypes.byref(w3), p, p, 4, 6, None, None, p, 2, ws, big, None) == moe.MOE_EALIGN
    # too-small workspace
    assert f(ctypes.byref(w), p, p, 4, 6, None, None, p, 2, ws, 1024, None) == moe.MOE_EWORKSPACE
    # expert count over the limit, intermediate not a multiple of 128
    assert f(ctypes.byref(_w(E=300, ptr=p)), p, p, 4, 6, None, None, p, 2, ws, big,
             None) == moe.MOE_ENOTSUP
    assert f(ctypes.byref(_w(I=2000, ptr=p)), p, p, 4, 6, None, None, p, 2, ws, big,
             None) == moe.MOE_EINVAL


def test_act_quant_rejects_bad_arguments_on_host():
    p = 0x100000
    f = moe._lib.act_quant_fp8
    assert f(p, 1, 4, 100, p, p, None) == moe.MOE_EINVAL       # cols % 128
    assert f(p, 5, 4, 128, p, p, None) == moe.MOE_EINVAL       # dtype
    assert f(p, 1, -1, 128, p, p, None) == moe.MOE_EINVAL      # rows
    assert f(p + 2, 1, 4, 128, p, p, None) == moe.MOE_EALIGN
    assert f(None, 1, 4, 128, p, p, None) == moe.MOE_EINVAL


def test_permute_and_combine_reject_bad_arguments_on_host():
    p, ws = 0x100000, 0x200000
    assert moe._lib.moe_permute(p, 4, 7, 6, p, p, p, ws, 1 << 30, None) == moe.MOE_EINVAL  # k > E
    assert moe._lib.moe_permute(p, 4, 2, 6, p, p, p, ws, 8, None) == moe.MOE_EWORKSPACE
    assert moe._lib.moe_combine(p, p, p, 4, 2, 4096, p, 3, None) == moe.MOE_EINVAL
    assert moe._lib.moe_combine(p, p, p, 4, 2, 4097, p, 2, None) == moe.MOE_EINVAL


def test_python_binding_raises_on_error_status():
    with pytest.raises(moe.MoeError) as ei:
        moe.act_quant_fp8(0x100000, 1, 4, 100, 0x100000, 0x100000, stream=0)
    assert ei.value.status == moe.MOE_EINVAL


def test_empty_batch_is_accepted_without_a_device():
    """T = 0 (rows = 0): the other arguments are still checked, then MOE_OK
    with nothing enqueued -- so the answer needs no GPU; T < 0 is invalid."""
    p, ws, big = 0x100000, 0x200000, 1 << 30
    w = _w(ptr=p)
    L = moe._lib
    wb = ctypes.byref(w)
    assert L.moe_route(p, p, 0, 4096, 256, 6, p, p, ws, big, None) == moe.MOE_OK
    assert L.act_quant_fp8(p, moe.MOE_DT_BF16, 0, 4096, p, p, None) == moe.MOE_OK
    assert L.moe_permute(p, 0, 6, 256, p, p, p, ws, big, None) == moe.MOE_OK
    assert L.moe_expert_ffn(wb, p, p, 0, 6, p, p, p, ws, big, None) == moe.MOE_OK
    assert L.moe_expert_gate_up(wb, p, p, 0, 6, p, p, ws, big, None) == moe.MOE_OK
    assert L.moe_expert_down(wb, 0, 6, p, p, p, p, p, moe.MOE_DT_F32, ws, big,
                             None) == moe.MOE_OK
    assert L.moe_combine(p, p, p, 0, 6, 4096, p, moe.MOE_DT_F32, None) == moe.MOE_OK
    assert L.dsv4_moe_forward(wb, p, p, 0, 6, None, None, p, moe.MOE_DT_F32, ws, big,
                              None) == moe.MOE_OK
    # the other arguments are still validated for an empty batch
    assert L.moe_route(None, p, 0, 4096, 256, 6, p, p, ws, big, None) == moe.MOE_EINVAL
    assert L.moe_route(p, p, 0, 4096, 256, 6, p + 4, p, ws, big, None) == moe.MOE_EALIGN
    assert L.act_quant_fp8(p, moe.MOE_DT_BF16, 0, 100, p, p, None) == moe.MOE_EINVAL
    assert L.dsv4_moe_forward(wb, p, p, 0, 17, None, None, p, moe.MOE_DT_F32, ws, big,
                              None) == moe.MOE_ENOTSUP
    # negative sizes are not
    assert L.moe_route(p, p, -1, 4096, 256, 6, p, p, ws, big, None) == moe.MOE_EINVAL
    assert L.act_quant_fp8(p, moe.MOE_DT_BF16, -1, 4096, p, p, None) == moe.MOE_EINVAL
    assert L.moe_combine(p, p, p, -1, 6, 4096, p, moe.MOE_DT_F32, None) == moe.MOE_EINVAL
    assert L.dsv4_moe_forward(wb, p, p, -1, 6, None, None, p, moe.MOE_DT_F32, ws, big,
                              None) == moe.MOE_EINVAL
    # no intermediates for an empty batch
    h = ctypes.c_void_p()
    assert L.moe_debug_intermediates(wb, 0, 6, ws, big, ctypes.byref(h), None,
                                     None) == moe.MOE_EINVAL


def test_token_count_limit():
    """At most 2^18 tokens per call (32-bit row offsets of x in the kernels):
    one more is refused on the host with MOE_ENOTSUP."""
    p, ws, big = 0x100000, 0x200000, 1 << 45
    w = _w(ptr=p)
    wb = ctypes.byref(w)
    L = moe._lib
    assert moe.moe_workspace_bytes(w, 1 << 18, 6) > 0
    assert moe.moe_workspace_bytes(w, (1 << 18) + 1, 6) == 0
    assert L.dsv4_moe_forward(wb, p, p, (1 << 18) + 1, 6, None, None, p, moe.MOE_DT_F32, ws,
                              big, None) == moe.MOE_ENOTSUP
    assert L.moe_route(p, p, (1 << 18) + 1, 4096, 256, 6, p, p, ws, big, None) == moe.MOE_ENOTSUP
    assert L.moe_permute(p, (1 << 18) + 1, 6, 256, p, p, p, ws, big, None) == moe.MOE_ENOTSUP
    assert L.moe_combine(p, p, p, (1 << 18) + 1, 6, 4096, p, moe.MOE_DT_F32,
                         None) == moe.MOE_ENOTSUP


def test_debug_h_sink_arguments():
    L = moe._lib
    assert L.moe_debug_store_h(None, 16) == moe.MOE_EINVAL
    assert L.moe_debug_store_h(0x100000, 0) == moe.MOE_EINVAL
    assert L.moe_debug_store_h(0x100004, 16) == moe.MOE_EALIGN
    assert L.moe_debug_store_h(0x100000, 16) == moe.MOE_OK
    assert L.moe_debug_store_h(None, 0) == moe.MOE_OK


def test_debug_decode_path_switch_and_kernel_ids():
    L = moe._lib
    for bad in (-1, 2, 7):
        assert L.moe_debug_set_decode_fused(bad) == moe.MOE_EINVAL
    assert L.moe_debug_set_decode_fused(1) == moe.MOE_OK
    assert L.moe_debug_set_decode_fused(0) == moe.MOE_OK
    # every kernel id of the timing hook is accepted (clearing), others refused
    for k in (moe.MOE_KERNEL_GEMV_GATE_UP, moe.MOE_KERNEL_GEMM_GATE_UP, moe.MOE_KERNEL_GEMV_DOWN,
              moe.MOE_KERNEL_GEMM_DOWN, moe.MOE_KERNEL_DECODE_FFN):
        assert L.moe_debug_time_kernel(k, None, None) == moe.MOE_OK
    assert L.moe_debug_time_kernel(0, None, None) == moe.MOE_EINVAL
    assert L.moe_debug_time_kernel(moe.MOE_KERNEL_DECODE_FFN + 1, None, None) == moe.MOE_EINVAL
    assert L.moe_debug_time_kernel(moe.MOE_KERNEL_DECODE_FFN, 0x10, None) == moe.MOE_EINVAL


def test_noalloc_forward_checks_arguments_and_size_on_host():
    """The allocation-free forward validates like dsv4_moe_forward and
    refuses a call whose workspace need exceeds its static array, before
    touching a device."""
    p = 0x100000
    w = _w(ptr=p)
    wb = ctypes.byref(w)
    L = moe._lib
    f = L.dsv4_moe_forward_noalloc
    assert moe.moe_workspace_bytes(w, 4096, 6) > moe.MOE_NOALLOC_SCRATCH_BYTES
    assert f(wb, p, p, 4096, 6, None, None, p, moe.MOE_DT_F32, None) == moe.MOE_ENOTSUP
    assert f(wb, p, p, 0, 6, None, None, p, moe.MOE_DT_F32, None) == moe.MOE_OK
    assert f(wb, p, p, 1, 6, None, None, None, moe.MOE_DT_F32, None) == moe.MOE_EINVAL
    assert f(wb, p, p, 1, 6, None, None, p, 7, None) == moe.MOE_EINVAL
    assert f(wb, p, p, 1, 6, p, None, p, moe.MOE_DT_F32, None) == moe.MOE_EINVAL
    assert f(wb, p, p + 2, 1, 6, None, None, p, moe.MOE_DT_F32, None) == moe.MOE_EALIGN
    assert f(wb, p, p, 1, 17, None, None, p, moe.MOE_DT_F32, None) == moe.MOE_ENOTSUP


def test_host_experts_call_checks_arguments_on_host():
    """The host-resident-experts call refuses malformed caches and calls
    whose experts cannot all be cached at once, before touching a device."""
    import numpy as np
    p = 0x100000
    host_w = _w(E=32, ptr=p)
    slot_w = _w(E=8, ptr=p)
    cache = moe.ExpertCache(32, 8)
    f = moe._lib.moe_forward_host_experts
    C = ctypes.byref(cache.c)
    args = lambda T, k, cw=slot_w: (ctypes.byref(host_w), ctypes.byref(cw), C, p, p, T, k, p,
                                    moe.MOE_DT_F32, p, 1 << 30, p, 1 << 20, p, None, None)
    assert f(*args(2, 6)) == moe.MOE_ENOTSUP            # 12 experts may not fit in 8 slots
    assert f(*args(1, 6, _w(E=9, ptr=p))) == moe.MOE_EINVAL   # slots != cache.n_slots
    assert f(*args(0, 6)) == moe.MOE_OK                 # empty batch
    assert cache.c.calls == 0
    assert moe.moe_host_experts_workspace_bytes(host_w, 4, 6) > \
        moe.moe_workspace_bytes(host_w, 4, 6)
    assert moe.moe_host_experts_scratch_bytes(32, 4, 6) >= 2 * 4 * 6 * 4 + 2 * 33
    assert np.all(cache.slot_of == -1)


def _route_ws_need(T, H, E, k=6):
    """Smallest workspace moe_route accepts (the check precedes any HIP call:
    below it the call returns MOE_EWORKSPACE, from it on another status)."""
    p, ws = 0x100000, 0x200000

    def rc(b):
        return moe.raw_call("moe_route", p, p, T, H, E, k, p, p, ws, b, None)
    lo, hi = 0, 1 << 34
    assert rc(hi) != moe.MOE_EWORKSPACE
    while lo + 1 < hi:
        mid = (lo + hi) // 2
        if rc(mid) == moe.MOE_EWORKSPACE:
            lo = mid
        else:
            hi = mid
    return hi


@pytest.mark.parametrize("H,E", [(4096, 256), (384, 200), (8192, 100)])
def test_route_workspace_holds_the_transposed_router_from_256_tokens(H, E):
    """From 256 tokens on the router copies its matrix transposed into the
    workspace ([E][H] bf16) besides the group sums, so the router section
    grows by at least E*H*2 bytes from 255 to 256 tokens; below that it grows
    by the group sums of one token only."""
    n254, n255, n256 = (_route_ws_need(T, H, E) for T in (254, 255, 256))
    groups = (H // 64 + 3) // 4
    assert n255 - n254 <= groups * E * 4 + 256
    assert n256 - n255 >= E * H * 2
    assert moe.moe_workspace_bytes(_w(E=E, H=H), 256, 6) >= n256
