"""Python binding of libmxmoe.so: an MXFP4-weight mixture-of-experts layer for MI355X.

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch tensors on the current HIP device; PyTorch provides device
memory and streams.  The library must be built first
(``python -m mxfp4_weight_mixture_amd.build``); importing this package
without it raises ImportError -- there is no other implementation to fall
back to.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxmoe.so")
ABI_VERSION = 3

# mirrors of include/mxmoe.h; checked against the library at import
STATUS = {"MOE_OK": 0, "MOE_ERR_INVALID_ARG": 1, "MOE_ERR_SHAPE": 2, "MOE_ERR_UNSUPPORTED_DEVICE": 3,
          "MOE_ERR_NOT_PINNED": 4, "MOE_ERR_WORKSPACE": 5, "MOE_ERR_HIP": 6, "MOE_ERR_NOT_IMPLEMENTED": 7}
ACT = {"MOE_ACT_BF16": 0, "MOE_ACT_MXFP8_E4M3": 1}
OUT = {"MOE_OUT_FP32": 0, "MOE_OUT_BF16": 1, "MOE_OUT_MXFP8_E4M3": 2}
EPI = {"MOE_EPI_NONE": 0, "MOE_EPI_SWIGLU_SPLIT": 1, "MOE_EPI_SWIGLU_INTERLEAVED": 2}
CHAIN = {"MOE_CHAIN_RMS": 0, "MOE_CHAIN_INDEPENDENT": 1}
WFORMAT = {"MOE_W_CANONICAL": 0, "MOE_W_TILED": 1}
COPY = {"MOE_COPY_ALL": 0, "MOE_COPY_ROUTED": 1, "MOE_COPY_AUTO": 2}
ENUM_KINDS = {0: STATUS, 1: ACT, 2: OUT, 3: EPI, 4: CHAIN, 5: WFORMAT, 6: COPY}
EXPERT_COPY = {"all": COPY["MOE_COPY_ALL"], "routed": COPY["MOE_COPY_ROUTED"], "auto": COPY["MOE_COPY_AUTO"]}
W_FORMAT = {"canonical": WFORMAT["MOE_W_CANONICAL"], "tiled": WFORMAT["MOE_W_TILED"]}

LAYOUT = {"split": EPI["MOE_EPI_SWIGLU_SPLIT"], "interleaved": EPI["MOE_EPI_SWIGLU_INTERLEAVED"]}

_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        name = {v: k for k, v in STATUS.items()}.get(status, str(status))
        super().__init__(f"{name}: {message}")


class GemmArgs(ctypes.Structure):
    _fields_ = [("a", _vp), ("a_scales", _vp), ("a_gather", _vp), ("w_packed", _vp), ("w_scales", _vp),
                ("expert_offsets", _vp), ("c", _vp), ("c_scales", _vp), ("a_dtype", _i32),
                ("a_gather_div", _i32), ("a_rows", _i32), ("rows", _i32), ("E", _i32), ("N", _i32),
                ("K", _i32), ("epilogue", _i32), ("c_dtype", _i32), ("w_format", _i32)]


class LayerArgs(ctypes.Structure):
    _fields_ = [("T", _i32), ("H", _i32), ("I", _i32), ("E", _i32), ("k", _i32), ("layout", _i32),
                ("act_dtype", _i32), ("inter_dtype", _i32), ("logits", _vp), ("x", _vp), ("x_scales", _vp),
                ("w1_packed", _vp), ("w1_scales", _vp), ("w2_packed", _vp), ("w2_scales", _vp),
                ("out", _vp), ("x_next", _vp), ("workspace", _vp), ("workspace_bytes", _sz), ("w_format", _i32)]


class StreamedArgs(ctypes.Structure):
    _fields_ = [("num_layers", _i32), ("T", _i32), ("H", _i32), ("I", _i32), ("E", _i32), ("k", _i32),
                ("layout", _i32), ("chain", _i32), ("depth", _i32), ("num_blobs", _i32),
                ("host_blobs", ctypes.POINTER(_vp)), ("blob_bytes", _sz), ("device_slot", _vp * 2),
                ("logits", _vp), ("x", _vp), ("out", _vp), ("layer_inputs", _vp), ("events", _vp),
                ("workspace", _vp), ("workspace_bytes", _sz), ("w_format", _i32), ("expert_copy", _i32),
                ("routed_copy_max_tokens", _i32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m mxfp4_weight_mixture_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sigs = {
        "moe_abi_version": (ctypes.c_int, []),
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_last_error_message": (ctypes.c_char_p, []),
        "moe_enum_name": (ctypes.c_char_p, [ctypes.c_int, ctypes.c_int]),
        "moe_device_supported": (ctypes.c_int, []),
        "moe_route": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp]),
        "moe_permute_workspace_size": (_sz, [_i32, _i32, _i32]),
        "moe_permute": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
        "moe_grouped_gemm_workspace_size": (_sz, [ctypes.POINTER(GemmArgs)]),
        "moe_mxfp4_grouped_gemm": (ctypes.c_int, [ctypes.POINTER(GemmArgs), _vp, _sz, _vp]),
        "moe_mxfp4_grouped_gemm_static": (ctypes.c_int, [ctypes.POINTER(GemmArgs), _vp]),
        "moe_combine": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]),
        "moe_layer_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
        "moe_layer_workspace_offset": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
        "moe_layer_forward": (ctypes.c_int, [ctypes.POINTER(LayerArgs), _vp]),
        "moe_blob_bytes": (_sz, [_i32, _i32, _i32]),
        "moe_blob_section_offset": (_sz, [_i32, _i32, _i32, _i32]),
        "moe_streamed_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
        "moe_layer_prefill_streamed": (ctypes.c_int, [ctypes.POINTER(StreamedArgs), _vp, _vp]),
        "moe_tiled_weight_bytes": (_sz, [_i32, _i32, _i32, _i32]),
        "moe_mxfp4_tile_weights": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
        "moe_mxfp4_untile_weights": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
        "moe_layer_graph_create": (ctypes.c_int, [ctypes.POINTER(LayerArgs), _vp, ctypes.POINTER(_vp)]),
        "moe_layer_graph_launch": (ctypes.c_int, [_vp, _vp]),
        "moe_layer_graph_destroy": (ctypes.c_int, [_vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe_abi_version() != ABI_VERSION:
        raise ImportError(f"libmxmoe ABI {lib.moe_abi_version()} != binding ABI {ABI_VERSION}")
    for kind, table in ENUM_KINDS.items():
        for name, value in table.items():
            got = lib.moe_enum_name(kind, value)
            if got is None or got.decode() != name:
                raise ImportError(f"enum mismatch: kind {kind} value {value}: library says {got}, binding {name}")
        if lib.moe_enum_name(kind, max(table.values()) + 1) is not None:
            raise ImportError(f"enum kind {kind} has values the binding does not know")
    return lib


lib = _load()


def _check(status: int):
    if status != 0:
        raise MoeError(status, (lib.moe_last_error_message() or b"").decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _u8(n: int, device) -> torch.Tensor:
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def _keep_until_done(stream, *tensors):
    """Tensors allocated here on the current stream but used by work enqueued on
    `stream`: tell the caching allocator so, so that it does not hand their memory
    to a later allocation before that work has finished."""
    if stream is None or stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


_COPY_STREAMS = {}


def _copy_stream_for(device) -> "torch.cuda.Stream":
    """One side stream per device for the streamed prefill's copies when the caller gives none."""
    idx = torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    if idx not in _COPY_STREAMS:
        _COPY_STREAMS[idx] = torch.cuda.Stream(device=idx)
    return _COPY_STREAMS[idx]


def device_supported() -> bool:
    return lib.moe_device_supported() == 1


# ----------------------------------------------------------------- calls

def route(logits: torch.Tensor, k: int, stream=None):
    """moe_route: logits fp32 [T][E] -> (topk_ids int32 [T][k], topk_w fp32 [T][k])."""
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib.moe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(stream)))
    _keep_until_done(stream, ids, w)
    return ids, w


def permute(topk_ids: torch.Tensor, E: int, stream=None):
    """moe_permute: topk_ids [T][k] -> (expert_offsets [E+1], perm_src [T*k], dest_row [T*k])."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ps = torch.empty(T * k, dtype=torch.int32, device=dev)
    dr = torch.empty(T * k, dtype=torch.int32, device=dev)
    n = lib.moe_permute_workspace_size(T, E, k)
    ws = _u8(n, dev)
    _check(lib.moe_permute(_ptr(topk_ids), T, E, k, _ptr(off), _ptr(ps), _ptr(dr), _ptr(ws), n,
                           _stream(stream)))
    _keep_until_done(stream, off, ps, dr, ws)
    return off, ps, dr


def grouped_gemm(a: torch.Tensor, w_packed: torch.Tensor, w_scales: torch.Tensor,
                 expert_offsets: torch.Tensor, *, a_scales: Optional[torch.Tensor] = None,
                 a_gather: Optional[torch.Tensor] = None, a_gather_div: int = 1, rows: Optional[int] = None,
                 epilogue: str = "none", out_dtype: str = "bf16", w_format: str = "canonical",
                 stream=None) -> torch.Tensor:
    """moe_mxfp4_grouped_gemm.  a: bf16 [a_rows][K] or uint8 E4M3 codes (with a_scales).

    w_packed [E][N][K/2], w_scales [E][N][K/32].  Returns C [rows][N or N/2]
    (fp32 or bf16), or for out_dtype "mxfp8" the pair (E4M3 codes uint8
    [rows][N/2], E8M0 scales uint8 [rows][N/64]).
    """
    E, N, K2 = w_packed.shape
    K = 2 * K2
    if rows is None:
        rows = a_gather.numel() if a_gather is not None else a.shape[0]
    epi = {"none": 0, "split": 1, "interleaved": 2}[epilogue]
    n_out = N if epi == 0 else N // 2
    c_dt = {"fp32": 0, "bf16": 1, "mxfp8": 2}[out_dtype]
    c_scales = None
    if c_dt == 2:
        c = torch.empty((rows, n_out), dtype=torch.uint8, device=a.device)
        c_scales = torch.empty((rows, n_out // 32), dtype=torch.uint8, device=a.device)
    else:
        c = torch.empty((rows, n_out), dtype=torch.float32 if c_dt == 0 else torch.bfloat16, device=a.device)
    args = GemmArgs(a=a.data_ptr(), a_scales=a_scales.data_ptr() if a_scales is not None else None,
                    a_gather=a_gather.data_ptr() if a_gather is not None else None,
                    w_packed=w_packed.data_ptr(), w_scales=w_scales.data_ptr(),
                    expert_offsets=expert_offsets.data_ptr(), c=c.data_ptr(),
                    c_scales=c_scales.data_ptr() if c_scales is not None else None,
                    a_dtype=1 if a_scales is not None else 0, a_gather_div=a_gather_div,
                    a_rows=a.shape[0], rows=rows, E=E, N=N, K=K, epilogue=epi, c_dtype=c_dt,
                    w_format=W_FORMAT[w_format])
    n = lib.moe_grouped_gemm_workspace_size(ctypes.byref(args))
    ws = _u8(n, a.device)
    _check(lib.moe_mxfp4_grouped_gemm(ctypes.byref(args), _ptr(ws), n, _stream(stream)))
    _keep_until_done(stream, c, c_scales, ws)
    return (c, c_scales) if c_dt == 2 else c


def tile_weights(w_packed: torch.Tensor, w_scales: torch.Tensor, epilogue: str = "none", stream=None):
    """moe_mxfp4_tile_weights: canonical [E][N][K/2] + [E][N][K/32] -> the tiled order.

    Returns uint8 tensors of the same shapes (the bytes are reordered; the
    shapes only carry E, N, K).  epilogue: the one the matrix is used with."""
    E, N, K2 = w_packed.shape
    tp, ts = torch.empty_like(w_packed), torch.empty_like(w_scales)
    _check(lib.moe_mxfp4_tile_weights(_ptr(w_packed), _ptr(w_scales), E, N, 2 * K2,
                                      {"none": 0, "split": 1, "interleaved": 2}[epilogue], _ptr(tp), _ptr(ts),
                                      _stream(stream)))
    _keep_until_done(stream, tp, ts)
    return tp, ts


def untile_weights(t_packed: torch.Tensor, t_scales: torch.Tensor, epilogue: str = "none", stream=None):
    """moe_mxfp4_untile_weights: the inverse of tile_weights."""
    E, N, K2 = t_packed.shape
    wp, ws = torch.empty_like(t_packed), torch.empty_like(t_scales)
    _check(lib.moe_mxfp4_untile_weights(_ptr(t_packed), _ptr(t_scales), E, N, 2 * K2,
                                        {"none": 0, "split": 1, "interleaved": 2}[epilogue], _ptr(wp), _ptr(ws),
                                        _stream(stream)))
    _keep_until_done(stream, wp, ws)
    return wp, ws


def combine(y: torch.Tensor, dest_row: torch.Tensor, topk_w: torch.Tensor, *, rms_next: bool = False,
            stream=None):
    """moe_combine: y [T*k][H] (fp32 or bf16) -> out fp32 [T][H] (and bf16 x_next if rms_next)."""
    T, k = topk_w.shape
    H = y.shape[1]
    out = torch.empty((T, H), dtype=torch.float32, device=y.device)
    xn = torch.empty((T, H), dtype=torch.bfloat16, device=y.device) if rms_next else None
    dt = 1 if y.dtype == torch.bfloat16 else 0
    _check(lib.moe_combine(_ptr(y), dt, _ptr(dest_row), _ptr(topk_w), T, k, H, _ptr(out), _ptr(xn),
                           _stream(stream)))
    _keep_until_done(stream, out, xn)
    return (out, xn) if rms_next else out


class Layer:
    """A resident layer: weights stay on the device; forward() runs the five steps on one stream."""

    def __init__(self, w1_packed, w1_scales, w2_packed, w2_scales, k: int, layout: str = "split",
                 inter: str = "bf16", w_format: str = "canonical", tile: bool = False):
        """inter: precision of the SwiGLU output fed to FC2, "bf16" or "mxfp8".
        w_format: the order of the given weights, "canonical" or "tiled" (W1 tiled
        with `layout`, W2 with "none").  tile=True: canonical weights are tiled
        here once and the layer keeps only the tiled copy."""
        if tile:
            if w_format != "canonical":
                raise ValueError("tile=True takes canonical weights")
            w1_packed, w1_scales = tile_weights(w1_packed, w1_scales, layout)
            w2_packed, w2_scales = tile_weights(w2_packed, w2_scales, "none")
            w_format = "tiled"
        self.w_format = W_FORMAT[w_format]
        self.w1p, self.w1s, self.w2p, self.w2s = w1_packed, w1_scales, w2_packed, w2_scales
        self.E, two_i, h2 = w1_packed.shape
        self.I, self.H = two_i // 2, 2 * h2
        self.k = k
        self.layout = LAYOUT[layout]
        self.inter = OUT[{"bf16": "MOE_OUT_BF16", "mxfp8": "MOE_OUT_MXFP8_E4M3"}[inter]]
        self._ws = None

    def workspace_bytes(self, T: int) -> int:
        return lib.moe_layer_workspace_size(T, self.H, self.I, self.E, self.k, self.inter)

    def _args(self, T, logits, x, x_scales, out, x_next, ws):
        return LayerArgs(T=T, H=self.H, I=self.I, E=self.E, k=self.k, layout=self.layout,
                         act_dtype=1 if x_scales is not None else 0, inter_dtype=self.inter,
                         logits=logits.data_ptr(), x=x.data_ptr(),
                         x_scales=x_scales.data_ptr() if x_scales is not None else None,
                         w1_packed=self.w1p.data_ptr(), w1_scales=self.w1s.data_ptr(),
                         w2_packed=self.w2p.data_ptr(), w2_scales=self.w2s.data_ptr(), out=out.data_ptr(),
                         x_next=x_next.data_ptr() if x_next is not None else None,
                         workspace=ws.data_ptr(), workspace_bytes=ws.numel(), w_format=self.w_format)

    def forward(self, logits: torch.Tensor, x: torch.Tensor, x_scales: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, x_next: Optional[torch.Tensor] = None, stream=None):
        T = logits.shape[0]
        n = self.workspace_bytes(T)
        if self._ws is None or self._ws.numel() < n:
            self._ws = _u8(n, logits.device)
        if out is None:
            out = torch.empty((T, self.H), dtype=torch.float32, device=logits.device)
        args = self._args(T, logits, x, x_scales, out, x_next, self._ws)
        _check(lib.moe_layer_forward(ctypes.byref(args), _stream(stream)))
        # the workspace may be replaced by a larger one on a later call while this one still runs
        _keep_until_done(stream, self._ws, out)
        return out

    def capture(self, logits: torch.Tensor, x: torch.Tensor, x_scales: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, x_next: Optional[torch.Tensor] = None) -> "LayerGraph":
        """moe_layer_graph_create: this layer on these buffers, captured once; see LayerGraph."""
        return LayerGraph(self, logits, x, x_scales, out, x_next)

    def routing(self, T: int):
        """Views of the routing arrays the last forward() wrote into its workspace."""
        def view(which, count, dtype):
            off = lib.moe_layer_workspace_offset(T, self.H, self.I, self.E, self.k, self.inter, which)
            return self._ws[off: off + 4 * count].view(dtype)
        Tk = T * self.k
        return dict(ids=view(0, Tk, torch.int32).view(T, self.k), w=view(1, Tk, torch.float32).view(T, self.k),
                    offsets=view(2, self.E + 1, torch.int32), perm_src=view(3, Tk, torch.int32),
                    dest_row=view(4, Tk, torch.int32))


class LayerGraph:
    """A resident layer captured into a HIP graph (moe_layer_graph_*).

    The graph owns its workspace and keeps the tensors it was captured on:
    replay() runs the five steps with one launch, reading the current contents
    of logits / x / x_scales and writing `out` (and x_next).  Replays on one
    graph must not overlap each other.
    """

    def __init__(self, layer: Layer, logits, x, x_scales=None, out=None, x_next=None):
        T = logits.shape[0]
        dev = logits.device
        self.layer, self.T = layer, T
        self.logits, self.x, self.x_scales, self.x_next = logits, x, x_scales, x_next
        self.out = out if out is not None else torch.empty((T, layer.H), dtype=torch.float32, device=dev)
        self.ws = _u8(layer.workspace_bytes(T), dev)
        args = layer._args(T, logits, x, x_scales, self.out, x_next, self.ws)
        # capture needs a created stream; nothing runs during the capture
        side = torch.cuda.Stream(device=dev)
        self._h = ctypes.c_void_p()
        _check(lib.moe_layer_graph_create(ctypes.byref(args), ctypes.c_void_p(side.cuda_stream),
                                          ctypes.byref(self._h)))

    def replay(self, stream=None) -> torch.Tensor:
        if not self._h:
            raise MoeError(STATUS["MOE_ERR_INVALID_ARG"], "graph already destroyed")
        _check(lib.moe_layer_graph_launch(self._h, _stream(stream)))
        return self.out

    def routing(self):
        """Views of the routing arrays the last replay wrote into the graph's workspace."""
        L = self.layer
        def view(which, count, dtype):
            off = lib.moe_layer_workspace_offset(self.T, L.H, L.I, L.E, L.k, L.inter, which)
            return self.ws[off: off + 4 * count].view(dtype)
        Tk = self.T * L.k
        return dict(ids=view(0, Tk, torch.int32).view(self.T, L.k), w=view(1, Tk, torch.float32).view(self.T, L.k),
                    offsets=view(2, L.E + 1, torch.int32), perm_src=view(3, Tk, torch.int32),
                    dest_row=view(4, Tk, torch.int32))

    def close(self):
        """moe_layer_graph_destroy; waits for the device first so that no replay is still running."""
        if self._h:
            torch.cuda.synchronize(self.out.device)
            h, self._h = self._h, ctypes.c_void_p()
            _check(lib.moe_layer_graph_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def blob_bytes(H: int, I: int, E: int) -> int:
    return lib.moe_blob_bytes(H, I, E)


def blob_section_offset(H: int, I: int, E: int, which: int) -> int:
    return lib.moe_blob_section_offset(H, I, E, which)


def prefill_streamed(host_blobs: Sequence[torch.Tensor], slots: Sequence[torch.Tensor], logits: torch.Tensor,
                     x: torch.Tensor, out: torch.Tensor, *, T: int, H: int, I: int, E: int, k: int,
                     num_layers: int, layout: str = "split", chain: str = "rms", depth: int = 2,
                     layer_inputs: Optional[torch.Tensor] = None, events=None, workspace=None,
                     compute_stream=None, copy_stream=None, w_format: str = "canonical",
                     expert_copy: str = "all", routed_copy_max_tokens: int = 0):
    """moe_layer_prefill_streamed.  host_blobs: pinned uint8 CPU tensors (layer L uses blob L % n).

    expert_copy: "all" moves every expert of a layer, "routed" only the experts
    its routing hits, "auto" routed when T <= routed_copy_max_tokens.
    copy_stream: the stream the weight copies run on; None uses one dedicated
    side stream per device (never the compute stream, which would serialise the
    pipeline).
    """
    nb = len(host_blobs)
    arr = (_vp * nb)(*[b.data_ptr() for b in host_blobs])
    need = lib.moe_streamed_workspace_size(T, H, I, E, k)
    if workspace is None or workspace.numel() < need:
        workspace = _u8(need, x.device)
    ev_arr = None
    if events is not None:
        ev_arr = (_vp * len(events))(*[e.cuda_event for e in events])
    args = StreamedArgs(num_layers=num_layers, T=T, H=H, I=I, E=E, k=k, layout=LAYOUT[layout],
                        chain=CHAIN["MOE_CHAIN_RMS" if chain == "rms" else "MOE_CHAIN_INDEPENDENT"],
                        depth=depth, num_blobs=nb, host_blobs=arr,
                        blob_bytes=min(b.numel() for b in host_blobs),
                        device_slot=(_vp * 2)(slots[0].data_ptr(), slots[1].data_ptr() if len(slots) > 1 else 0),
                        logits=logits.data_ptr(), x=x.data_ptr(), out=out.data_ptr(),
                        layer_inputs=layer_inputs.data_ptr() if layer_inputs is not None else None,
                        events=ctypes.cast(ev_arr, _vp) if ev_arr is not None else None,
                        workspace=workspace.data_ptr(), workspace_bytes=workspace.numel(),
                        w_format=W_FORMAT[w_format], expert_copy=EXPERT_COPY[expert_copy],
                        routed_copy_max_tokens=routed_copy_max_tokens)
    cs = _stream(compute_stream)
    if copy_stream is None:
        # a copy on the compute stream would serialise the pipeline
        copy_stream = _copy_stream_for(x.device)
    _check(lib.moe_layer_prefill_streamed(ctypes.byref(args), cs, _stream(copy_stream)))
    _keep_until_done(compute_stream, workspace)
    if copy_stream != torch.cuda.current_stream(x.device):
        workspace.record_stream(copy_stream)
    return workspace
