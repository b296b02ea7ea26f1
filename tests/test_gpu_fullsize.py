"""Full-size workloads, in the launch configuration the benchmark times: routing
and permutation bit-exact over every token, and the layer output on sampled
tokens against the oracle (which regenerates only the experts those tokens use)."""
import time

import numpy as np
import pytest
import torch

from oracle import moe as omoe
from workloads import gen
from tests.gpu_util import cpu_weights, device_weights, device_x, rel_err, x_as_f64

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_weight_mixture_amd")
DEV = "cuda"


def pick_tokens(ids, n):
    """n tokens chosen greedily to share experts (keeps the oracle's dequantisation small)."""
    chosen, used = [], set()
    cand = list(range(ids.shape[0]))
    for _ in range(n):
        best = min(cand, key=lambda t: (len(set(ids[t].tolist()) - used), t))
        chosen.append(best)
        used |= set(ids[best].tolist())
        cand.remove(best)
    return np.array(chosen)


def _full(name, n_sample, tol, inter="bf16", **over):
    t0 = time.time()
    s = gen.preset(name, **over)
    li = gen.layer_inputs(s)
    w = device_weights(s)
    layer = mx.Layer(*w, k=s.k, layout=s.layout, inter=inter)
    x, xs = device_x(li)
    out = layer.forward(torch.from_numpy(li.logits).to(DEV), x, xs)
    torch.cuda.synchronize()
    r = {k: v.cpu().numpy() for k, v in layer.routing(s.T).items()}
    out = out.cpu().numpy()
    del w, layer, x, xs
    torch.cuda.empty_cache()
    print(f"[{name} inter={inter}] gpu done {time.time() - t0:.1f}s", flush=True)

    rid, rw = omoe.route(li.logits, s.k)
    np.testing.assert_array_equal(r["ids"], rid)
    np.testing.assert_allclose(r["w"], rw, rtol=1e-6)
    roff, rps, rdr = omoe.permute(rid, s.E)
    np.testing.assert_array_equal(r["offsets"], roff)
    np.testing.assert_array_equal(r["perm_src"], rps)
    np.testing.assert_array_equal(r["dest_row"], rdr)
    assert np.all(np.isfinite(out))

    toks = pick_tokens(rid, n_sample)
    xa = x_as_f64(li)
    ref = omoe.moe_tokens(xa[toks], rid[toks], rw[toks], cpu_weights(s), s.layout)
    err = rel_err(out[toks], ref)
    print(f"[{name} inter={inter}] tokens {toks.tolist()} experts {len(np.unique(rid[toks]))} "
          f"rel err {err:.3e} ({time.time() - t0:.1f}s)", flush=True)
    assert err <= tol


def test_prefill896_mxfp8_full_size():
    _full("prefill896_mxfp8", 6, 5e-2)


def test_prefill896_mxfp8_full_size_mxfp8_intermediate():
    _full("prefill896_mxfp8", 6, 5e-2, inter="mxfp8")


def test_prefill256_full_size():
    _full("prefill256", 6, 2e-2)


def test_decode_t1_full_size():
    _full("decode", 1, 2e-2, T=1)


def test_prefill896_repeat_runs_bitwise_identical():
    """Five passes of the full-size layer (MXFP8 intermediate: FC1's epilogue
    stages its fp32 tile through LDS between two barriers) agree bitwise: a
    barrier that let a wave read the staged tile before another wave's LDS
    writes had landed showed up here as an occasional garbage block."""
    s = gen.preset("prefill896_mxfp8")
    li = gen.layer_inputs(s)
    w = device_weights(s)
    layer = mx.Layer(*w, k=s.k, layout=s.layout, inter="mxfp8")
    x, xs = device_x(li)
    logits = torch.from_numpy(li.logits).to(DEV)
    first = layer.forward(logits, x, xs).clone()
    for _ in range(4):
        assert torch.equal(layer.forward(logits, x, xs), first)
    assert torch.isfinite(first).all()


@pytest.mark.parametrize("name,over,inter", [("prefill896_mxfp8", {}, "mxfp8"), ("decode", {"T": 32}, "bf16"),
                                             ("prefill256", {}, "bf16")])
def test_full_size_tiled_weights_equal_canonical_bitwise(name, over, inter):
    """The benchmark's configuration runs on load-time tiled weights; at the full
    sizes its layer output equals the canonical-weight layer's bitwise."""
    s = gen.preset(name, **over)
    li = gen.layer_inputs(s)
    w = device_weights(s)
    x, xs = device_x(li)
    logits = torch.from_numpy(li.logits).to(DEV)
    ref = mx.Layer(*w, k=s.k, layout=s.layout, inter=inter).forward(logits, x, xs).clone()
    tiled = mx.Layer(*w, k=s.k, layout=s.layout, inter=inter, tile=True)
    del w
    got = tiled.forward(logits, x, xs)
    torch.cuda.synchronize()
    assert torch.equal(ref, got)
    print(f"[{name}] tiled == canonical bitwise", flush=True)
