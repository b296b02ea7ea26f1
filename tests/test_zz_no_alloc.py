"""moe_mxfp4_grouped_gemm_static (the grouped GEMM whose scratch is a static
device array, for callers that cannot allocate) against moe_mxfp4_grouped_gemm
with a caller workspace: the same kernels, so the outputs must be bitwise
equal.  Two calls in a row through the C ABI, the second smaller than the
first, so that the second runs on the array the first left behind."""
import ctypes

import pytest
import torch

from workloads import gen
from tests.gpu_util import device_weights

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_weight_mixture_amd")
DEV = "cuda"


def _problem(T, H, I, E, k, act, layout, cfg_id):
    s = gen.LayerShape(T=T, H=H, I=I, E=E, k=k, act=act, layout=layout, cfg_id=cfg_id)
    li = gen.layer_inputs(s)
    w = device_weights(s)
    logits = torch.from_numpy(li.logits).to(DEV)
    ids, tw = mx.route(logits, k)
    off, ps, dr = mx.permute(ids, E)
    if act == "mxfp8":
        x, xs = li.x_codes.to(DEV), li.x_scales.to(DEV)
    else:
        x, xs = li.x_bf16.to(DEV), None
    return s, w, x, xs, off, ps


def _fc1_args(s, w, x, xs, off, ps, out_dtype):
    rows, n_out = s.T * s.k, s.I
    mx8 = out_dtype == "mxfp8"
    c = torch.empty((rows, n_out), dtype=torch.uint8 if mx8 else torch.bfloat16, device=DEV)
    cs = torch.empty((rows, n_out // 32), dtype=torch.uint8, device=DEV) if mx8 else None
    args = mx.GemmArgs(a=x.data_ptr(), a_scales=xs.data_ptr() if xs is not None else None, a_gather=ps.data_ptr(),
                       w_packed=w[0].data_ptr(), w_scales=w[1].data_ptr(), expert_offsets=off.data_ptr(),
                       c=c.data_ptr(), c_scales=cs.data_ptr() if mx8 else None,
                       a_dtype=1 if xs is not None else 0, a_gather_div=s.k, a_rows=s.T, rows=rows, E=s.E,
                       N=2 * s.I, K=s.H, epilogue=mx.LAYOUT[s.layout], c_dtype=2 if mx8 else 1, w_format=0)
    return args, c, cs


def _fc2_args(s, w, a, off):
    rows = s.T * s.k
    c = torch.empty((rows, s.H), dtype=torch.float32, device=DEV)
    args = mx.GemmArgs(a=a.data_ptr(), a_scales=None, a_gather=None, w_packed=w[2].data_ptr(),
                       w_scales=w[3].data_ptr(), expert_offsets=off.data_ptr(), c=c.data_ptr(), c_scales=None,
                       a_dtype=0, a_gather_div=1, a_rows=rows, rows=rows, E=s.E, N=s.H, K=s.I, epilogue=0,
                       c_dtype=0, w_format=0)
    return args, c


def _with_workspace(args):
    n = mx.lib.moe_grouped_gemm_workspace_size(ctypes.byref(args))
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    mx._check(mx.lib.moe_mxfp4_grouped_gemm(ctypes.byref(args), ctypes.c_void_p(ws.data_ptr()), n,
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    torch.cuda.synchronize()


def _static(args):
    mx._check(mx.lib.moe_mxfp4_grouped_gemm_static(ctypes.byref(args),
                                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    torch.cuda.synchronize()


def test_static_scratch_gemm_equals_workspace_gemm_on_two_calls():
    # call 1: MXFP8 activations gathered through the permutation, SwiGLU with MXFP8 output,
    # enough rows per expert for every row-tile class
    s, w, x, xs, off, ps = _problem(T=1500, H=1024, I=512, E=12, k=4, act="mxfp8", layout="interleaved",
                                    cfg_id=170)
    args, c_ref, cs_ref = _fc1_args(s, w, x, xs, off, ps, "mxfp8")
    _with_workspace(args)
    ref = (c_ref.clone(), cs_ref.clone())
    c_ref.fill_(0x7F)
    cs_ref.fill_(0x00)
    _static(args)
    assert torch.equal(c_ref, ref[0]) and torch.equal(cs_ref, ref[1])
    print(f"[no-alloc] call 1: {s.T * s.k} rows, {s.E} experts: bitwise equal", flush=True)

    # call 2, smaller: bf16 activations, split SwiGLU to bf16, then FC2 to fp32 on its output
    s, w, x, xs, off, ps = _problem(T=90, H=512, I=256, E=5, k=2, act="bf16", layout="split", cfg_id=171)
    args, c_ref, _ = _fc1_args(s, w, x, xs, off, ps, "bf16")
    _with_workspace(args)
    ref = c_ref.clone()
    c_ref.zero_()
    _static(args)
    assert torch.equal(c_ref, ref)
    args2, y = _fc2_args(s, w, ref, off)
    _with_workspace(args2)
    y_ref = y.clone()
    y.fill_(float("nan"))
    _static(args2)
    assert torch.equal(y, y_ref) and torch.isfinite(y).all()
    print(f"[no-alloc] call 2: {s.T * s.k} rows, {s.E} experts: bitwise equal (FC1 and FC2)", flush=True)
