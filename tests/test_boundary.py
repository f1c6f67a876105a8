"""The C-ABI boundary on the CPU: symbols, sizes and argument validation.

Every call here is rejected by host-side validation (or is a T = 0 no-op)
before any HIP call, so these run without a GPU.  The fake pointers are never
dereferenced; no call in this file may pass validation with them.
"""
import ctypes
import os
import re

import pytest

from quantized_moe_amd import lib, synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = lib.lib()
    names = _declared_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(L, name), name
    for required in ["moe_route_topk", "moe_expert_ffn_decode", "moe_expert_ffn_prefill", "moe_layer_forward"]:
        assert required in names


def test_abi_and_status_strings():
    assert lib.abi_version() == lib.MOE_ABI_VERSION
    L = lib.lib()
    for code, name in [(0, b"MOE_OK"), (-1, b"MOE_ERR_INVALID_ARG"), (-2, b"MOE_ERR_UNSUPPORTED"),
                       (-3, b"MOE_ERR_WORKSPACE"), (-4, b"MOE_ERR_HIP")]:
        assert L.moe_status_string(code) == name


@pytest.mark.parametrize("fmt,E,rows,K", [(1, 384, 2048, 4096), (2, 384, 4096, 2048), (3, 1, 2048, 4096),
                                          (2, 8, 512, 256), (4, 384, 2048, 4096), (5, 384, 4096, 2048),
                                          (6, 384, 2048, 4096), (7, 384, 4096, 2048), (6, 3, 5, 64), (7, 2, 3, 128)])
def test_matrix_bytes_matches_format_sizes(fmt, E, rows, K):
    assert lib.matrix_bytes(fmt, E, rows, K) == synth.matrix_bytes(fmt, E, rows, K)


def test_matrix_bytes_of_the_decode_layer():
    # 2,162,688 B per IQ2 matrix, 2,752,512 B per Q2K matrix, 8,912,896 per Q8 matrix
    assert lib.matrix_bytes(1, 1, 2048, 4096) == 2162688
    assert lib.matrix_bytes(2, 1, 4096, 2048) == 2752512
    assert lib.matrix_bytes(3, 1, 2048, 4096) == 8912896
    assert lib.matrix_bytes(4, 1, 2048, 4096) == 4718592   # Q4K: 144 B per 256 weights
    assert lib.matrix_bytes(5, 1, 2048, 4096) == 4456448   # MXFP4: 17 B per 32 weights
    assert lib.matrix_bytes(6, 1, 2048, 4096) == 1576960   # VQ12: 2 + 768 B per row of 4096
    assert lib.matrix_bytes(7, 1, 2048, 4096) == 1708032   # VQ13: 2 + 768 + 64 B per row of 4096
    with pytest.raises(lib.MoeError):
        lib.matrix_bytes(6, 1, 16, 32)                     # VQ rows: K a multiple of 64


def _layer(**over):
    fields = dict(abi_version=lib.MOE_ABI_VERSION, n_experts=384, d_model=4096, d_ff=2048, top_k=6,
                  fmt_gate_up=1, fmt_down=2, layout=lib.MOE_LAYOUT_DEVICE, w_gate=256, w_up=512, w_down=768,
                  iq2_grid=1024, w_router=1280, has_shared=1, fmt_shared=3, s_gate=1536, s_up=1792, s_down=2048)
    fields.update(over)
    return lib.MoeLayer(**fields)


def _ffn_decode(layer, T=1, x=4096, idx=4352, wt=4608, y=4864, ws=5120, ws_bytes=0):
    L = lib.lib()
    return L.moe_expert_ffn_decode(ctypes.byref(layer), x, lib.MOE_F32, T, idx, wt, y, ws, ws_bytes, None)


def _forward(layer, T=1, x=4096, y=4864, ws=5120, ws_bytes=0, path=0, dtype=0):
    L = lib.lib()
    return L.moe_layer_forward(ctypes.byref(layer), x, dtype, T, y, None, None, path, ws, ws_bytes, None)


@pytest.mark.parametrize("over,code", [
    (dict(abi_version=1), lib.MOE_ERR_UNSUPPORTED),      # the layout before router_bias / down_gain
    (dict(abi_version=2), lib.MOE_ERR_UNSUPPORTED),      # the layout before vq_codebook / vq_codes
    (dict(abi_version=99), lib.MOE_ERR_UNSUPPORTED),
    (dict(layout=lib.MOE_LAYOUT_CANONICAL), lib.MOE_ERR_UNSUPPORTED),
    (dict(layout=7), lib.MOE_ERR_UNSUPPORTED),
    (dict(fmt_gate_up=9), lib.MOE_ERR_UNSUPPORTED),
    (dict(fmt_down=0), lib.MOE_ERR_UNSUPPORTED),
    (dict(fmt_shared=4), lib.MOE_ERR_UNSUPPORTED),        # Q4K_L: routed experts only
    (dict(fmt_shared=5), lib.MOE_ERR_UNSUPPORTED),        # MXFP4_L: routed experts only
    (dict(fmt_shared=6), lib.MOE_ERR_UNSUPPORTED),        # VQ: routed experts only
    (dict(fmt_shared=7), lib.MOE_ERR_UNSUPPORTED),
    (dict(fmt_gate_up=8), lib.MOE_ERR_UNSUPPORTED),
    (dict(fmt_gate_up=6, vq_codebook=0x8000, vq_codes=4096), lib.MOE_ERR_UNSUPPORTED),  # VQ gate/up, Q2K down
    (dict(fmt_gate_up=6, fmt_down=6, vq_codes=4096), lib.MOE_ERR_INVALID_ARG),           # no codebook
    (dict(fmt_gate_up=6, fmt_down=6, vq_codebook=0x8008, vq_codes=4096), lib.MOE_ERR_INVALID_ARG),  # misaligned
    (dict(fmt_gate_up=6, fmt_down=6, vq_codebook=0x8000, vq_codes=1000), lib.MOE_ERR_INVALID_ARG),
    (dict(fmt_gate_up=7, fmt_down=6, vq_codebook=0x8000, vq_codes=4096), lib.MOE_ERR_INVALID_ARG),  # 13 bits: 8192
    (dict(n_experts=0), lib.MOE_ERR_INVALID_ARG),
    (dict(n_experts=1025), lib.MOE_ERR_INVALID_ARG),
    (dict(d_model=4000), lib.MOE_ERR_INVALID_ARG),
    (dict(d_model=128), lib.MOE_ERR_INVALID_ARG),
    (dict(d_ff=16384), lib.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), lib.MOE_ERR_INVALID_ARG),
    (dict(top_k=17), lib.MOE_ERR_INVALID_ARG),
    (dict(n_experts=4, top_k=5), lib.MOE_ERR_INVALID_ARG),
    (dict(w_gate=0), lib.MOE_ERR_INVALID_ARG),
    (dict(w_down=0x1008), lib.MOE_ERR_INVALID_ARG),       # misaligned
    (dict(iq2_grid=0), lib.MOE_ERR_INVALID_ARG),          # IQ2 in use needs the grid
    (dict(s_up=0), lib.MOE_ERR_INVALID_ARG),
    (dict(has_shared=2), lib.MOE_ERR_INVALID_ARG),
    (dict(router_bias=0x1002), lib.MOE_ERR_INVALID_ARG),  # misaligned
    (dict(down_gain=0x1008), lib.MOE_ERR_INVALID_ARG),    # not 16-byte aligned
])
def test_layer_validation(over, code):
    assert _ffn_decode(_layer(**over)) == code
    assert lib.last_error() != ""


def test_grid_not_needed_without_iq2_and_shared_optional():
    layer = _layer(fmt_gate_up=2, iq2_grid=0, has_shared=0, s_gate=0, s_up=0, s_down=0)
    # gets past layer validation; fails on the (deliberately) empty workspace
    assert _ffn_decode(layer) == lib.MOE_ERR_WORKSPACE


def test_vq_layers_pass_validation():
    for gu, dn, n in [(6, 6, 4096), (6, 6, 8192), (7, 6, 8192), (6, 7, 8192), (7, 7, 8192)]:
        layer = _layer(fmt_gate_up=gu, fmt_down=dn, vq_codebook=0x8000, vq_codes=n, iq2_grid=0)
        assert _ffn_decode(layer) == lib.MOE_ERR_WORKSPACE, (gu, dn, n)  # past validation
    # the codebook is not read by block formats
    assert _ffn_decode(_layer(vq_codebook=0x8008, vq_codes=5)) == lib.MOE_ERR_WORKSPACE


def test_bias_and_gains_are_optional():
    layer = _layer(router_bias=0x3000, down_gain=0x4000)
    assert _ffn_decode(layer) == lib.MOE_ERR_WORKSPACE                  # past validation
    assert _route_bias_misaligned() == lib.MOE_ERR_INVALID_ARG


def _route_bias_misaligned():
    return lib.lib().moe_route_topk(256, 0x1002, 384, 4096, 512, 0, 1, 6, 768, 1024, 1280, 1 << 20, None)


def test_router_needed_only_by_the_whole_layer():
    layer = _layer(w_router=0)
    assert _ffn_decode(layer) == lib.MOE_ERR_WORKSPACE
    assert _forward(layer) == lib.MOE_ERR_INVALID_ARG


def test_T_limits_and_noop():
    layer = _layer()
    assert _ffn_decode(layer, T=-1) == lib.MOE_ERR_INVALID_ARG
    assert _ffn_decode(layer, T=9) == lib.MOE_ERR_INVALID_ARG            # decode path holds T <= 8
    assert _forward(layer, T=9, path=lib.MOE_PATH_DECODE) == lib.MOE_ERR_INVALID_ARG
    assert _forward(layer, T=65537) == lib.MOE_ERR_INVALID_ARG
    assert _forward(layer, T=0, x=0, y=0, ws=0) == lib.MOE_OK            # T = 0: nothing to do
    assert _forward(layer, path=5) == lib.MOE_ERR_INVALID_ARG
    assert _forward(layer, dtype=2) == lib.MOE_ERR_UNSUPPORTED


def test_workspace_too_small_is_rejected_before_launch():
    layer = _layer()
    assert _forward(layer, T=1, ws_bytes=16) == lib.MOE_ERR_WORKSPACE
    assert _forward(layer, T=1024, ws_bytes=1 << 20) == lib.MOE_ERR_WORKSPACE
    assert "need" in lib.last_error()


def test_prefill_offset_limit_is_checked_before_any_launch():
    """The prefill path addresses H [T*k][f] fp16 with 32-bit offsets: T =
    65536, k = 6, f = 4096 is inside the documented size limits but its H
    needs 3 GiB.  The call must fail on the host, as an invalid argument,
    before the router, top-k or bucketing kernels are enqueued (the fake
    pointers would fault if anything were)."""
    layer = _layer(d_ff=4096)
    ws = 1 << 62  # a workspace "large enough": the size check must come first
    assert _forward(layer, T=65536, ws_bytes=ws) == lib.MOE_ERR_INVALID_ARG
    assert "2^31" in lib.last_error()
    L = lib.lib()
    rc = L.moe_expert_ffn_prefill(ctypes.byref(layer), 4096, lib.MOE_BF16, 65536, 4352, 4608, 4864, None, 5120,
                                  ws, None)
    assert rc == lib.MOE_ERR_INVALID_ARG
    # x16 [T][d] alone: T = 65536, d = 8192 is 1 GiB (fits); with k = 16, f = 2048 H is 4 GiB
    assert _forward(_layer(d_model=8192, top_k=16, d_ff=2048), T=65536, ws_bytes=ws) == lib.MOE_ERR_INVALID_ARG


def test_prepare_weights_validation():
    """moe_prepare_weights validates the canonical layer and every
    destination before its first launch; the fake pointers are never used."""
    L = lib.lib()
    canon = _layer(layout=lib.MOE_LAYOUT_CANONICAL, w_gate=1 << 40, w_up=2 << 40, w_down=3 << 40,
                   s_gate=4 << 40, s_up=5 << 40, s_down=6 << 40)
    dst = lib.MoeLayer(w_gate=7 << 40, w_up=8 << 40, w_down=9 << 40, s_gate=10 << 40, s_up=11 << 40, s_down=0)
    assert L.moe_prepare_weights(ctypes.byref(canon), ctypes.byref(dst), None) == lib.MOE_ERR_INVALID_ARG
    assert "s_down" in lib.last_error()
    assert dst.layout == 0 and dst.n_experts == 0  # left unchanged
    dst.s_down = (12 << 40) + 8  # misaligned
    assert L.moe_prepare_weights(ctypes.byref(canon), ctypes.byref(dst), None) == lib.MOE_ERR_INVALID_ARG
    dst.s_down = (1 << 40) + 4096  # inside the canonical w_gate
    assert L.moe_prepare_weights(ctypes.byref(canon), ctypes.byref(dst), None) == lib.MOE_ERR_INVALID_ARG
    assert "overlaps" in lib.last_error()
    dst.s_down = (9 << 40) + 256  # inside another destination
    assert L.moe_prepare_weights(ctypes.byref(canon), ctypes.byref(dst), None) == lib.MOE_ERR_INVALID_ARG
    dev = _layer()  # already in the device layout
    assert L.moe_prepare_weights(ctypes.byref(dev), ctypes.byref(dst), None) == lib.MOE_ERR_UNSUPPORTED
    assert L.moe_prepare_weights(ctypes.byref(_layer(layout=lib.MOE_LAYOUT_CANONICAL, fmt_down=9)),
                                 ctypes.byref(dst), None) == lib.MOE_ERR_UNSUPPORTED
    assert L.moe_prepare_weights(ctypes.byref(canon), None, None) == lib.MOE_ERR_INVALID_ARG


def test_workspace_sizes_cover_their_buffers():
    layer = _layer()
    E, d, f, k = 384, 4096, 2048, 6
    assert lib.workspace_bytes(layer, 1, lib.MOE_OP_ROUTE) >= E * 4
    # decode: quantized x chunks and quantized SwiGLU outputs of k routed + 1
    # shared expert per token (128 bytes + one fp32 scale per 64 values)
    assert lib.workspace_bytes(layer, 8, lib.MOE_OP_DECODE) >= 8 * (d // 64) * 132 + (8 * k + 8) * (f // 64) * 132
    # prefill: fp16 H [T*k][f] + fp32 Ye [T*k][d] + shared H/Y + routing buffers
    T = 1024
    need = T * k * f * 2 + T * k * d * 4 + T * f * 2 + T * d * 4 + (3 * E + 2 * T * k) * 4
    assert lib.workspace_bytes(layer, T, lib.MOE_OP_PREFILL) >= need
    assert lib.workspace_bytes(layer, T, lib.MOE_OP_LAYER) >= lib.workspace_bytes(layer, T, lib.MOE_OP_PREFILL)
    assert lib.workspace_bytes(layer, 1, lib.MOE_OP_LAYER) >= lib.workspace_bytes(layer, 1, lib.MOE_OP_DECODE)


def test_prefill_workspace_counts_the_dense_shared_expert():
    """A Q8 shared expert on the prefill path runs as dense GEMMs on fp16
    copies of its three matrices (2 * 3 * d * f bytes), fp32 gate/up outputs
    and operands on the token count rounded up to 64 rows; other shared
    formats need none of that."""
    d, f = 4096, 2048
    for T in (1, 100, 1024):
        Tg = (T + 63) // 64 * 64
        q8 = lib.workspace_bytes(_layer(), T, lib.MOE_OP_PREFILL)
        q2k = lib.workspace_bytes(_layer(fmt_shared=2), T, lib.MOE_OP_PREFILL)
        extra = 6 * d * f + Tg * 2 * f * 4 + (2 * f + d) * 4 + (Tg - T) * (d * 2 + f * 2 + d * 4)
        assert extra <= q8 - q2k <= extra + 16 * 256, (T, q8 - q2k, extra)
        assert lib.workspace_bytes(_layer(fmt_shared=2), T, lib.MOE_OP_PREFILL) == \
            lib.workspace_bytes(_layer(fmt_shared=1), T, lib.MOE_OP_PREFILL)


def test_route_and_bucket_validation():
    L = lib.lib()
    assert L.moe_route_topk(256, None, 384, 4096, 512, 0, 1, 0, 768, 1024, 1280, 1 << 20, None) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(256, None, 2000, 4096, 512, 0, 1, 6, 768, 1024, 1280, 1 << 20, None) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(256, None, 384, 4096, 512, 0, 1, 6, 768, 1024, 1280, 0, None) == lib.MOE_ERR_WORKSPACE
    assert L.moe_route_topk(256, None, 384, 4096, 512, 3, 1, 6, 768, 1024, 1280, 1 << 20, None) == lib.MOE_ERR_UNSUPPORTED
    assert L.moe_bucket(256, 4, 6, 384, 0, 512, 768, 1024, None) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_bucket(256, 4, 0, 384, 256, 512, 768, 1024, None) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_bucket(0, 0, 6, 384, 0, 0, 0, 0, None) == lib.MOE_OK


def test_repack_validation():
    L = lib.lib()
    assert L.moe_repack(9, 1, 16, 256, 256, 512, 0, None) == lib.MOE_ERR_UNSUPPORTED
    assert L.moe_repack(5, 1, 16, 48, 256, 512, 0, None) == lib.MOE_ERR_INVALID_ARG  # MXFP4: K % 32
    assert L.moe_repack(4, 1, 16, 100, 256, 512, 0, None) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_repack(1, 1, 16, 100, 256, 512, 0, None) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_repack(1, 1, 16, 256, 256, 256, 0, None) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_repack(1, 1, 16, 256, 256, 512, 3, None) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_repack(3, 1, 16, 32, 0, 512, 0, None) == lib.MOE_ERR_INVALID_ARG
