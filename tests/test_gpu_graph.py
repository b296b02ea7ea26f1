"""Graph capture and replay of the resident layer (moe_layer_graph_*): every
replay equals the eager layer bitwise, with eager work and synchronisations
between the replays, a replay reads its input buffers' current contents, and
at the decode shape every replay's whole output meets the acceptance bound
against the oracle.  Token counts 1/2/8/32 at the decode shape are the
Phase-1 list of the Kimi-K3 page; the tiny shapes cover both activation
types and layouts."""
import numpy as np
import pytest
import torch

from oracle import moe as omoe
from workloads import gen
from tests.gpu_util import device_weights, device_x, full_oracle, rel_err

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_weight_mixture_amd")
DEV = "cuda"


def _replays_match_eager(layer, li, replays=3, ref=None, tol=None):
    """ref: the oracle's output for li; each replay's whole output is held to tol against it."""
    x, xs = device_x(li)
    logits = torch.from_numpy(li.logits).to(DEV)
    eager = layer.forward(logits, x, xs).clone()
    eager_r = {k: v.clone() for k, v in layer.routing(li.shape.T).items()}
    g = layer.capture(logits, x, xs)
    try:
        for i in range(replays):
            out = g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {i} differs from the eager layer"
            if ref is not None:
                err = rel_err(out.cpu().numpy(), ref)
                assert err <= tol, f"replay {i}: max|replay-oracle|/max|oracle| = {err:.3e} > {tol}"
            for k, v in g.routing().items():
                assert torch.equal(v, eager_r[k]), (i, k)
            # the program's own eager work between replays
            again = layer.forward(logits, x, xs)
            torch.cuda.synchronize()
            assert torch.equal(again, eager)
        # routing of the replay is the oracle's (bit-exact ids)
        rid, _ = omoe.route(li.logits, li.shape.k)
        np.testing.assert_array_equal(g.routing()["ids"].cpu().numpy(), rid)
    finally:
        g.close()
    return eager


@pytest.mark.parametrize("act,layout,inter", [("bf16", "split", "bf16"), ("bf16", "interleaved", "bf16"),
                                              ("mxfp8", "interleaved", "bf16"), ("mxfp8", "split", "bf16")])
def test_tiny_graph_replay_equals_eager(act, layout, inter):
    s = gen.preset("tiny", act=act, layout=layout)
    li = gen.layer_inputs(s)
    layer = mx.Layer(*device_weights(s), k=s.k, layout=layout, inter=inter)
    out = _replays_match_eager(layer, li)
    assert torch.isfinite(out).all()


def test_graph_replay_reads_current_inputs():
    """Capture on one set of buffers, then overwrite them with another token
    batch: the replay computes the new batch (equal to an eager call on it)."""
    s = gen.preset("tiny", T=96, H=512, I=256, E=8, k=2, layout="split")
    li = gen.layer_inputs(s)
    li2 = gen.layer_inputs(gen.preset("tiny", T=96, H=512, I=256, E=8, k=2, layout="split", seed=7))
    layer = mx.Layer(*device_weights(s), k=s.k, layout="split")
    x, _ = device_x(li)
    logits = torch.from_numpy(li.logits).to(DEV)
    first = layer.forward(logits, x).clone()
    g = layer.capture(logits, x)
    try:
        assert torch.equal(g.replay(), first)
        torch.cuda.synchronize()
        x2, _ = device_x(li2)
        logits2 = torch.from_numpy(li2.logits).to(DEV)
        want = layer.forward(logits2, x2).clone()
        x.copy_(x2)
        logits.copy_(logits2)
        got = g.replay()
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        assert not torch.equal(got, first)
    finally:
        g.close()


@pytest.mark.timeout(600)
def test_decode_graph_replay_equals_eager_and_oracle_at_1_2_8_32_tokens():
    s0 = gen.preset("decode")
    w = device_weights(s0)
    layer = mx.Layer(*w, k=s0.k, layout=s0.layout)
    for T in (1, 2, 8, 32):
        s = gen.preset("decode", T=T)
        li = gen.layer_inputs(s)
        # decode weights do not depend on T: the same device bytes feed the oracle
        ref, _ = full_oracle(s, li, w, label=f"decode T={T}")
        out = _replays_match_eager(layer, li, ref=ref, tol=2e-2)
        assert out.shape == (T, s0.H) and torch.isfinite(out).all()
        print(f"[decode T={T}] graph replays equal the eager layer; whole output "
              f"{rel_err(out.cpu().numpy(), ref):.3e} vs the oracle", flush=True)


def test_graph_of_empty_batch_is_a_no_op():
    s = gen.preset("tiny")
    layer = mx.Layer(*device_weights(s), k=s.k)
    logits = torch.empty((0, s.E), dtype=torch.float32, device=DEV)
    x = torch.empty((0, s.H), dtype=torch.bfloat16, device=DEV)
    g = layer.capture(logits, x)
    try:
        assert g.replay().shape == (0, s.H)
        torch.cuda.synchronize()
    finally:
        g.close()
