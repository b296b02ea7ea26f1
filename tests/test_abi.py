"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments before touching a device.  No kernels run here."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxmoe.h")

mx = pytest.importorskip("mxfp4_weight_mixture_amd", reason="libmxmoe.so is not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_every_declared_function_is_exported():
    names = _declared()
    assert "moe_route" in names and "moe_layer_prefill_streamed" in names and len(names) >= 18
    out = subprocess.run(["nm", "-D", "--defined-only", mx.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(moe_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(mx.lib, n)


def test_abi_version_and_enum_names():
    assert mx.lib.moe_abi_version() == mx.ABI_VERSION == 3
    # each enum value round-trips through the library's names (the binding checked it at import too)
    for kind, table in mx.ENUM_KINDS.items():
        for name, value in table.items():
            assert mx.lib.moe_enum_name(kind, value).decode() == name
        assert mx.lib.moe_enum_name(kind, -1) is None
    assert mx.lib.moe_enum_name(99, 0) is None
    assert mx.lib.moe_status_string(2) == b"MOE_ERR_SHAPE"
    assert mx.lib.moe_status_string(1234) == b"unknown status"


def test_enum_values_match_the_header_text():
    text = open(HEADER).read()
    for table in mx.ENUM_KINDS.values():
        for name, value in table.items():
            m = re.search(rf"\b{name}\s*=\s*(\d+)", text)
            assert m and int(m.group(1)) == value, name


def _status(st):
    return st, mx.lib.moe_last_error_message().decode()


def test_route_rejects_bad_sizes_before_any_device_call():
    p = ctypes.c_void_p(16)
    st, msg = _status(mx.lib.moe_route(p, -1, 4, 2, p, p, None))
    assert st == mx.STATUS["MOE_ERR_SHAPE"] and "T" in msg
    st, _ = _status(mx.lib.moe_route(p, 4, 2000, 2, p, p, None))
    assert st == mx.STATUS["MOE_ERR_SHAPE"]
    st, _ = _status(mx.lib.moe_route(p, 4, 8, 9, p, p, None))
    assert st == mx.STATUS["MOE_ERR_SHAPE"]
    st, _ = _status(mx.lib.moe_route(None, 4, 8, 2, p, p, None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"]


def test_permute_workspace_checks():
    p = ctypes.c_void_p(16)
    need = mx.lib.moe_permute_workspace_size(100, 16, 4)
    assert need > 0
    st, msg = _status(mx.lib.moe_permute(p, 100, 16, 4, p, p, p, p, need - 1, None))
    assert st == mx.STATUS["MOE_ERR_WORKSPACE"] and str(need) in msg


def _gemm_args(**kw):
    p = 16
    base = dict(a=p, a_scales=None, a_gather=None, w_packed=p, w_scales=p, expert_offsets=p, c=p,
                c_scales=None, a_dtype=0, a_gather_div=1, a_rows=64, rows=64, E=2, N=256, K=128,
                epilogue=0, c_dtype=1)
    base.update(kw)
    return mx.GemmArgs(**base)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(K=100), "MOE_ERR_SHAPE", "multiples of 32"),
    (dict(N=96, epilogue=1), "MOE_ERR_SHAPE", "gate + up"),
    (dict(a_dtype=1), "MOE_ERR_INVALID_ARG", "a_scales"),
    (dict(epilogue=7), "MOE_ERR_INVALID_ARG", "epilogue"),
    (dict(c_dtype=2, epilogue=1), "MOE_ERR_NOT_IMPLEMENTED", "MXFP8"),
    (dict(a_rows=10), "MOE_ERR_SHAPE", "fewer than rows"),
])
def test_gemm_argument_errors(kw, status, needle):
    args = _gemm_args(**kw)
    st, msg = _status(mx.lib.moe_mxfp4_grouped_gemm(ctypes.byref(args), ctypes.c_void_p(16), 1 << 20, None))
    assert st == mx.STATUS[status] and needle in msg, msg


def test_layer_rejects_fc1_fc2_size_rules():
    # H, I must be whole MX blocks; E within the router's range
    args = mx.LayerArgs(T=4, H=100, I=64, E=4, k=2, layout=1, act_dtype=0, inter_dtype=1)
    st, msg = _status(mx.lib.moe_layer_forward(ctypes.byref(args), None))
    assert st == mx.STATUS["MOE_ERR_SHAPE"] and "multiples" in msg
    args = mx.LayerArgs(T=4, H=128, I=64, E=4, k=2, layout=0, act_dtype=0, inter_dtype=1)
    st, msg = _status(mx.lib.moe_layer_forward(ctypes.byref(args), None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "SwiGLU" in msg


def test_streamed_argument_errors():
    args = mx.StreamedArgs(num_layers=2, T=4, H=128, I=64, E=4, k=2, layout=1, chain=0, depth=3, num_blobs=1)
    st, msg = _status(mx.lib.moe_layer_prefill_streamed(ctypes.byref(args), None, None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "depth" in msg
    args = mx.StreamedArgs(num_layers=2, T=4, H=128, I=64, E=4, k=2, layout=1, chain=0, depth=2, num_blobs=1,
                           expert_copy=3)
    st, msg = _status(mx.lib.moe_layer_prefill_streamed(ctypes.byref(args), None, None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "expert_copy" in msg
    args = mx.StreamedArgs(num_layers=2, T=4, H=128, I=64, E=4, k=2, layout=1, chain=0, depth=2, num_blobs=1,
                           expert_copy=mx.COPY["MOE_COPY_AUTO"], routed_copy_max_tokens=-1)
    st, msg = _status(mx.lib.moe_layer_prefill_streamed(ctypes.byref(args), None, None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "routed_copy_max_tokens" in msg


def test_routed_copy_rejects_misaligned_blobs_before_any_device_call():
    blob = (ctypes.c_uint8 * 4096)()
    ptrs = (ctypes.c_void_p * 1)(ctypes.addressof(blob) + 8)
    slots = (ctypes.c_void_p * 2)(256, 512)
    args = mx.StreamedArgs(num_layers=1, T=4, H=128, I=64, E=4, k=2, layout=1, chain=0, depth=2, num_blobs=1,
                           host_blobs=ptrs, blob_bytes=1 << 20, device_slot=slots, logits=256, x=256, out=256,
                           workspace=256, workspace_bytes=1 << 30, expert_copy=mx.COPY["MOE_COPY_ROUTED"])
    st, msg = _status(mx.lib.moe_layer_prefill_streamed(ctypes.byref(args), None, None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "16-byte aligned blobs" in msg


def test_streamed_depth_2_needs_two_streams_before_any_device_call():
    blob = (ctypes.c_uint8 * 4096)()
    ptrs = (ctypes.c_void_p * 1)(ctypes.addressof(blob))
    slots = (ctypes.c_void_p * 2)(256, 512)
    args = mx.StreamedArgs(num_layers=2, T=4, H=128, I=64, E=4, k=2, layout=1, chain=0, depth=2, num_blobs=1,
                           host_blobs=ptrs, blob_bytes=1 << 20, device_slot=slots, logits=256, x=256, out=256,
                           workspace=256, workspace_bytes=1 << 30)
    for cs in (None, 4096):
        st, msg = _status(mx.lib.moe_layer_prefill_streamed(ctypes.byref(args), cs, cs))
        assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "distinct" in msg


def test_static_scratch_gemm_checks_before_any_device_call():
    st, msg = _status(mx.lib.moe_mxfp4_grouped_gemm_static(None, None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"]
    # 1.1 M rows over 896 experts need more planner scratch than the static array holds
    args = mx.GemmArgs(a=256, w_packed=256, w_scales=256, expert_offsets=256, c=256, a_dtype=0, a_gather_div=1,
                       a_rows=1_100_000, rows=1_100_000, E=896, N=7168, K=3584, epilogue=0, c_dtype=1, w_format=0)
    assert mx.lib.moe_grouped_gemm_workspace_size(ctypes.byref(args)) > (1 << 20)
    st, msg = _status(mx.lib.moe_mxfp4_grouped_gemm_static(ctypes.byref(args), None))
    assert st == mx.STATUS["MOE_ERR_WORKSPACE"] and "static" in msg
    # bad arguments are the same errors as the workspace entry point's
    args.K = 100
    st, msg = _status(mx.lib.moe_mxfp4_grouped_gemm_static(ctypes.byref(args), None))
    assert st == mx.STATUS["MOE_ERR_SHAPE"]


def test_blob_layout_sections_are_aligned_and_ordered():
    H, I, E = 4096, 2048, 256
    offs = [mx.blob_section_offset(H, I, E, w) for w in range(4)]
    assert offs[0] == 0 and all(o % 256 == 0 for o in offs)
    assert offs == sorted(offs)
    assert offs[1] == E * 2 * I * H // 2
    total = mx.blob_bytes(H, I, E)
    # 3*H*I weights per expert at 4 bits + one scale byte per 32: ~3.42 GB per layer
    assert total == E * 3 * H * I * 17 // 32


def test_layer_graph_argument_errors():
    """Graph capture rejects a missing handle, missing args and the null stream
    before any device call; destroying NULL is a no-op, launching it an error."""
    args = mx.LayerArgs(T=4, H=128, I=64, E=4, k=2, layout=1, act_dtype=0, inter_dtype=1)
    h = ctypes.c_void_p()
    st, msg = _status(mx.lib.moe_layer_graph_create(ctypes.byref(args), None, ctypes.byref(h)))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "null stream" in msg and not h.value
    st, msg = _status(mx.lib.moe_layer_graph_create(ctypes.byref(args), ctypes.c_void_p(16), None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "handle" in msg
    st, msg = _status(mx.lib.moe_layer_graph_create(None, ctypes.c_void_p(16), ctypes.byref(h)))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "null args" in msg
    assert mx.lib.moe_layer_graph_destroy(None) == 0
    st, msg = _status(mx.lib.moe_layer_graph_launch(None, None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "handle" in msg


def test_weight_tiling_sizes_and_argument_errors():
    """The tiled order keeps the canonical byte counts; shapes it does not take
    (K % 512, N % 256) and bad arguments are refused before any device call,
    and a grouped GEMM or layer that names tiled weights of such a shape too."""
    E, N, K = 3, 512, 1024
    assert mx.lib.moe_tiled_weight_bytes(E, N, K, 0) == E * N * K // 2
    assert mx.lib.moe_tiled_weight_bytes(E, N, K, 1) == E * N * K // 32
    assert mx.lib.moe_tiled_weight_bytes(E, 384, K, 0) == 0 and mx.lib.moe_tiled_weight_bytes(E, N, 768, 1) == 0
    assert mx.lib.moe_tiled_weight_bytes(E, N, K, 2) == 0
    p = ctypes.c_void_p(16)
    st, msg = _status(mx.lib.moe_mxfp4_tile_weights(p, p, E, 384, K, 0, p, p, None))
    assert st == mx.STATUS["MOE_ERR_SHAPE"] and "N % 256" in msg
    st, msg = _status(mx.lib.moe_mxfp4_untile_weights(p, p, E, N, 640, 0, p, p, None))
    assert st == mx.STATUS["MOE_ERR_SHAPE"] and "K % 512" in msg
    st, msg = _status(mx.lib.moe_mxfp4_tile_weights(p, p, E, N, K, 3, p, p, None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "epilogue" in msg
    st, msg = _status(mx.lib.moe_mxfp4_tile_weights(None, p, E, N, K, 0, p, p, None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "null" in msg
    a, b = ctypes.c_void_p(1 << 20), ctypes.c_void_p((1 << 20) + 4096)
    st, msg = _status(mx.lib.moe_mxfp4_tile_weights(a, ctypes.c_void_p(1 << 30), E, N, K, 0, b,
                                                    ctypes.c_void_p(1 << 31), None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "overlap" in msg
    args = _gemm_args(K=640, w_format=1)
    st, msg = _status(mx.lib.moe_mxfp4_grouped_gemm(ctypes.byref(args), ctypes.c_void_p(16), 1 << 20, None))
    assert st == mx.STATUS["MOE_ERR_SHAPE"] and "tiled" in msg
    args = _gemm_args(w_format=7)
    st, msg = _status(mx.lib.moe_mxfp4_grouped_gemm(ctypes.byref(args), ctypes.c_void_p(16), 1 << 20, None))
    assert st == mx.STATUS["MOE_ERR_INVALID_ARG"] and "w_format" in msg
    largs = mx.LayerArgs(T=4, H=512, I=256, E=4, k=2, layout=1, act_dtype=0, inter_dtype=1, w_format=1)
    st, msg = _status(mx.lib.moe_layer_forward(ctypes.byref(largs), None))
    assert st == mx.STATUS["MOE_ERR_SHAPE"] and "tiled" in msg
