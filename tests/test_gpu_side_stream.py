"""Every binding call on a caller-given side stream equals the same call on the
current stream, bitwise, while the current stream keeps allocating and
filling memory: the scratch and outputs the binding allocates for a
side-stream call must not be handed to another allocation before the
side-stream work that uses them has run."""
import pytest
import torch

from workloads import gen
from tests.gpu_util import device_weights, device_x

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_weight_mixture_amd")
DEV = "cuda"


def _steps(w, logits, x, logits2, x2, k, E, layout, stream=None, churn=None):
    """route -> permute -> FC1 -> FC2 -> combine through the binding's calls, then the resident layer."""
    def step(v):
        if churn is not None:
            churn()
        return v
    ids, tw = step(mx.route(logits, k, stream=stream))
    off, ps, dr = step(mx.permute(ids, E, stream=stream))
    act = step(mx.grouped_gemm(x, w[0], w[1], off, a_gather=ps, a_gather_div=k, epilogue=layout,
                               out_dtype="bf16", stream=stream))
    y = step(mx.grouped_gemm(act, w[2], w[3], off, out_dtype="bf16", stream=stream))
    out = step(mx.combine(y, dr, tw, stream=stream))
    layer = mx.Layer(*w, k=k, layout=layout)
    lo = step(layer.forward(logits, x, stream=stream))
    # a second, larger batch replaces the layer's workspace while the first may still run
    lo2 = step(layer.forward(logits2, x2, stream=stream))
    return [ids, tw, off, ps, dr, act, y, out, lo, lo2]


def test_side_stream_calls_equal_current_stream_calls():
    s = gen.LayerShape(T=700, H=512, I=256, E=8, k=2, cfg_id=160, layout="split")
    li = gen.layer_inputs(s)
    w = device_weights(s)
    x, _ = device_x(li)
    logits = torch.from_numpy(li.logits).to(DEV)
    logits2, x2 = torch.cat([logits, logits]), torch.cat([x, x])
    ref = _steps(w, logits, x, logits2, x2, s.k, s.E, s.layout)
    torch.cuda.synchronize()

    junk = []

    def churn():
        # allocations on the current stream, filled at once, of the sizes the calls use
        for n in (1 << 12, 1 << 16, 1 << 20, 1 << 22):
            junk.append(torch.full((n,), 0x5A, dtype=torch.uint8, device=DEV))
        del junk[:-8]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = _steps(w, logits, x, logits2, x2, s.k, s.E, s.layout, stream=side, churn=churn)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(ref, got)):
        assert torch.equal(a, b), f"result {i} differs on the side stream"
