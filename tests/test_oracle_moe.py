"""Pins of the oracle's layer (oracle/moe.py): library routines, brute force, identities."""
import math

import numpy as np
import pytest
import torch

from oracle import moe, mx
from workloads import gen


def _rand_weights(rng, E, H, I, lo=121, hi=128):
    ws = []
    for _ in range(E):
        ws.append((rng.integers(0, 256, (2 * I, H // 2), dtype=np.uint8),
                   rng.integers(lo, hi, (2 * I, H // 32), dtype=np.uint8),
                   rng.integers(0, 256, (H, I // 2), dtype=np.uint8),
                   rng.integers(lo, hi, (H, I // 32), dtype=np.uint8)))
    return ws


# ------------------------------------------------------------------ routing

@pytest.mark.parametrize("T,E,k", [(64, 4, 2), (33, 256, 6), (17, 896, 16), (5, 7, 7)])
def test_route_matches_numpy_stable_argsort(T, E, k):
    lg = np.random.default_rng(T * E).standard_normal((T, E)).astype(np.float32)
    ids, w = moe.route(lg, k)
    ref = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(ids, ref)


def test_route_bruteforce_fp64_with_ties():
    g = np.random.default_rng(5)
    lg = g.integers(-3, 4, (40, 9)).astype(np.float32)      # many exact ties
    ids, w = moe.route(lg, 4)
    for t in range(40):
        order = sorted(range(9), key=lambda e: (-float(lg[t, e]), e))[:4]
        assert list(ids[t]) == order
        m = max(float(v) for v in lg[t])
        p = [math.exp(float(lg[t, e]) - m) for e in order]
        s = sum(p)
        np.testing.assert_allclose(w[t], [q / s for q in p], rtol=1e-15)


def test_route_weight_identities():
    g = np.random.default_rng(6)
    lg = (g.standard_normal((50, 32)) * 3).astype(np.float32)
    ids, w = moe.route(lg, 5)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)
    top = np.take_along_axis(lg, ids, axis=1).astype(np.float64)
    # ratios of the kept weights are exp of logit differences (softmax law)
    np.testing.assert_allclose(w[:, 1:] / w[:, :1], np.exp(top[:, 1:] - top[:, :1]), rtol=1e-13)
    for t in range(50):
        assert len(set(ids[t])) == 5


def test_route_equals_full_softmax_then_renormalise():
    g = np.random.default_rng(7)
    lg = g.standard_normal((20, 12)).astype(np.float32)
    ids, w = moe.route(lg, 3)
    full = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    kept = np.take_along_axis(full, ids, axis=1)
    np.testing.assert_allclose(w, kept / kept.sum(axis=1, keepdims=True), rtol=1e-13)


# -------------------------------------------------------------- permutation

@pytest.mark.parametrize("T,E,k", [(32, 4, 2), (100, 16, 3), (7, 64, 7), (1, 5, 1)])
def test_permute_matches_stable_argsort(T, E, k):
    g = np.random.default_rng(T + E)
    lg = g.standard_normal((T, E)).astype(np.float32)
    ids, _ = moe.route(lg, k)
    off, perm_src, dest_row = moe.permute(ids, E)
    flat = ids.ravel()
    np.testing.assert_array_equal(perm_src, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(np.diff(off), np.bincount(flat, minlength=E))
    assert off[0] == 0 and off[-1] == T * k
    np.testing.assert_array_equal(dest_row[perm_src], np.arange(T * k))


def test_permute_empty_and_single_expert():
    off, ps, dr = moe.permute(np.zeros((0, 2), dtype=np.int32), 3)
    assert list(off) == [0, 0, 0, 0] and ps.size == 0 and dr.size == 0
    ids = np.full((6, 1), 2, dtype=np.int32)
    off, ps, dr = moe.permute(ids, 4)
    assert list(off) == [0, 0, 0, 6, 6]
    np.testing.assert_array_equal(ps, np.arange(6))


# ------------------------------------------------------------ activation

def test_silu_identities():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(moe.silu(z) - moe.silu(-z), z, rtol=1e-13, atol=1e-13)
    assert moe.silu(np.array(0.0)) == 0.0
    assert abs(moe.silu(np.array(40.0)) - 40.0) < 1e-12
    assert abs(moe.silu(np.array(-40.0))) < 1e-15
    # sigmoid(z) = silu(z) / z, compared with torch's sigmoid
    zz = z[z != 0]
    np.testing.assert_allclose(moe.silu(zz) / zz, torch.sigmoid(torch.from_numpy(zz)).numpy(), rtol=1e-13)


@pytest.mark.parametrize("layout", ["split", "interleaved"])
def test_gate_and_up_rows_are_where_the_layout_says(layout):
    g = np.random.default_rng(8)
    H, I = 64, 32
    X = g.standard_normal((6, H))
    (w1p, w1s, w2p, w2s), = _rand_weights(g, 1, H, I)
    W1 = mx.dequant_mxfp4(w1p, w1s)
    W2 = mx.dequant_mxfp4(w2p, w2s)
    gate_rows = np.arange(I) if layout == "split" else 2 * np.arange(I)
    up_rows = I + np.arange(I) if layout == "split" else 2 * np.arange(I) + 1
    base = moe.expert_mlp(X, W1, W2, layout)
    assert np.abs(base).max() > 0
    # zero the up rows -> zero output; zero the gate rows -> zero output (silu(0) = 0)
    for rows in (up_rows, gate_rows):
        Wz = W1.copy()
        Wz[rows] = 0
        assert np.all(moe.expert_mlp(X, Wz, W2, layout) == 0)
    # the output is linear in the up rows (x2 exactly) but not in the gate rows
    Wu = W1.copy()
    Wu[up_rows] *= 2
    np.testing.assert_array_equal(moe.expert_mlp(X, Wu, W2, layout), 2 * base)
    Wg = W1.copy()
    Wg[gate_rows] *= 2
    assert not np.allclose(moe.expert_mlp(X, Wg, W2, layout), 2 * base)


# ------------------------------------------------------------- expert MLP

def _brute_expert(X, W1, W2, layout):
    n, H = X.shape
    I = W1.shape[0] // 2
    Y = np.zeros((n, H))
    for r in range(n):
        act = []
        for i in range(I):
            gr, ur = (i, I + i) if layout == "split" else (2 * i, 2 * i + 1)
            gv = sum(X[r, h] * W1[gr, h] for h in range(H))
            uv = sum(X[r, h] * W1[ur, h] for h in range(H))
            act.append(gv / (1 + math.exp(-gv)) * uv)
        for h in range(H):
            Y[r, h] = sum(act[i] * W2[h, i] for i in range(I))
    return Y


@pytest.mark.parametrize("layout", ["split", "interleaved"])
def test_expert_mlp_bruteforce(layout):
    g = np.random.default_rng(9)
    H, I = 32, 32
    X = g.standard_normal((3, H))
    (w1p, w1s, w2p, w2s), = _rand_weights(g, 1, H, I)
    W1, W2 = mx.dequant_mxfp4(w1p, w1s), mx.dequant_mxfp4(w2p, w2s)
    np.testing.assert_allclose(moe.expert_mlp(X, W1, W2, layout), _brute_expert(X, W1, W2, layout),
                               rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- combine

def test_combine_one_hot_and_k1():
    g = np.random.default_rng(10)
    Y = g.standard_normal((12, 8))
    dest = g.permutation(12).astype(np.int32)
    w = np.zeros((4, 3))
    w[:, 1] = 1.0
    out = moe.combine(Y, dest, w)
    np.testing.assert_array_equal(out, Y[dest.reshape(4, 3)[:, 1]])
    w1 = np.ones((12, 1))
    np.testing.assert_array_equal(moe.combine(Y, dest, w1), Y[dest])


# ------------------------------------------------------------ whole layer

def _brute_layer(xv, lg, k, ws, layout):
    """Pure-Python layer: sorted() routing, explicit dequantisation, loops."""
    T, E = lg.shape
    H = xv.shape[1]
    out = np.zeros((T, H))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:k]
        m = max(float(v) for v in lg[t])
        p = [math.exp(float(lg[t, e]) - m) for e in order]
        for j, e in enumerate(order):
            w1p, w1s, w2p, w2s = ws[e]
            W1 = _brute_dequant(w1p, w1s)
            W2 = _brute_dequant(w2p, w2s)
            y = _brute_expert(xv[t:t + 1], W1, W2, layout)[0]
            out[t] += (p[j] / sum(p)) * y
    return out


E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _brute_dequant(p, s):
    N, K2 = p.shape
    W = np.empty((N, 2 * K2))
    for n in range(N):
        for kk in range(2 * K2):
            c = (int(p[n, kk // 2]) >> (4 * (kk % 2))) & 15
            v = E2M1[c & 7] * (-1 if c & 8 else 1)
            W[n, kk] = v * 2.0 ** (int(s[n, kk // 32]) - 127)
    return W


@pytest.mark.parametrize("layout", ["split", "interleaved"])
def test_layer_bruteforce_tiny(layout):
    g = np.random.default_rng(11)
    T, H, I, E, k = 5, 32, 32, 3, 2
    xv = g.standard_normal((T, H))
    lg = g.standard_normal((T, E)).astype(np.float32)
    ws = _rand_weights(g, E, H, I)
    out = moe.moe_layer(xv, lg, k, lambda e: ws[e], layout)
    np.testing.assert_allclose(out, _brute_layer(xv, lg, k, ws, layout), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("layout", ["split", "interleaved"])
def test_dense_one_expert_equivalence(layout):
    g = np.random.default_rng(12)
    T, H, I = 9, 64, 64
    xv = g.standard_normal((T, H))
    ws = _rand_weights(g, 1, H, I)
    lg = g.standard_normal((T, 1)).astype(np.float32)
    out = moe.moe_layer(xv, lg, 1, lambda e: ws[e], layout)
    W1 = mx.dequant_mxfp4(ws[0][0], ws[0][1])
    W2 = mx.dequant_mxfp4(ws[0][2], ws[0][3])
    gr = np.arange(I) if layout == "split" else 2 * np.arange(I)
    ur = I + np.arange(I) if layout == "split" else 2 * np.arange(I) + 1
    dense = (torch.nn.functional.silu(torch.from_numpy(xv @ W1[gr].T)).numpy() * (xv @ W1[ur].T)) @ W2.T
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-12)
    # E > 1 with one dominant expert and k = 1: the same plain MLP
    ws4 = _rand_weights(g, 4, H, I)
    ws4[2] = ws[0]
    lg4 = g.standard_normal((T, 4)).astype(np.float32)
    lg4[:, 2] = 1e4
    out4 = moe.moe_layer(xv, lg4, 1, lambda e: ws4[e], layout)
    np.testing.assert_allclose(out4, dense, rtol=1e-12, atol=1e-12)


def test_token_order_permutation_invariance():
    g = np.random.default_rng(13)
    T, H, I, E, k = 24, 64, 32, 5, 2
    xv = g.standard_normal((T, H))
    lg = g.standard_normal((T, E)).astype(np.float32)
    ws = _rand_weights(g, E, H, I)
    out = moe.moe_layer(xv, lg, k, lambda e: ws[e], "split")
    perm = g.permutation(T)
    outp = moe.moe_layer(xv[perm], lg[perm], k, lambda e: ws[e], "split")
    np.testing.assert_allclose(outp, out[perm], rtol=1e-12, atol=1e-12)


def test_moe_tokens_equals_layer_rows():
    g = np.random.default_rng(14)
    T, H, I, E, k = 16, 64, 32, 6, 3
    xv = g.standard_normal((T, H))
    lg = g.standard_normal((T, E)).astype(np.float32)
    ws = _rand_weights(g, E, H, I)
    out = moe.moe_layer(xv, lg, k, lambda e: ws[e], "interleaved")
    ids, w = moe.route(lg, k)
    sel = np.array([0, 5, 11])
    part = moe.moe_tokens(xv[sel], ids[sel], w[sel], lambda e: ws[e], "interleaved")
    np.testing.assert_allclose(part, out[sel], rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------- stacked layers

def test_rms_rescale_and_bf16_rounding():
    g = np.random.default_rng(15)
    y = g.standard_normal((7, 256)) * 1e5
    r = moe.rms_rescale(y)
    np.testing.assert_allclose(np.sqrt(np.mean(r ** 2, axis=1)), 1.0, rtol=1e-14)
    bits = moe.to_bf16_bits(r)
    ref = torch.from_numpy(r.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    np.testing.assert_array_equal(bits, ref)


def test_streamed_layers_stay_finite_and_chain():
    shape = gen.LayerShape(T=8, H=64, I=32, E=4, k=2, cfg_id=99, layers=3)
    x0 = gen.activations_bf16(shape).view(torch.int16).numpy()
    lgs = [gen.router_logits(shape, L) for L in range(3)]
    wts = lambda L, e: [t.numpy() for t in gen.expert_weights(shape, e, L)]
    outs = moe.streamed_layers(x0, lgs, 2, wts, "split")
    assert len(outs) == 3 and all(np.all(np.isfinite(o)) for o in outs)
    # layer 1 consumes bf16(rms_rescale(layer 0))
    x1 = mx.bf16_value(moe.to_bf16_bits(moe.rms_rescale(outs[0])))
    y1 = moe.moe_layer(x1, lgs[1], 2, lambda e: wts(1, e), "split")
    np.testing.assert_array_equal(y1, outs[1])


def test_tiny_workload_golden_fixture():
    """Frozen oracle result on the tiny workload (tests/golden/make_golden.py wrote it)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_layer.json")) as f:
        doc = json.load(f)
    s = gen.preset("tiny")
    li = gen.layer_inputs(s)
    x = moe.activations(x_bf16=li.x_bf16.view(torch.int16).numpy())
    wts = lambda e: [t.numpy() for t in gen.expert_weights(s, e)]
    out, it = moe.moe_layer(x, li.logits, s.k, wts, s.layout, return_intermediates=True)
    assert it["ids"].tolist() == doc["ids"]
    assert it["offsets"].tolist() == doc["offsets"]
    assert it["perm_src"].tolist() == doc["perm_src"]
    np.testing.assert_allclose(it["w"], doc["w"], rtol=1e-15)
    np.testing.assert_allclose(out[:2], doc["out_rows_0_1"], rtol=1e-12)
    np.testing.assert_allclose(out.sum(axis=1), doc["out_row_sums"], rtol=1e-9, atol=1e-9 * doc["out_abs_max"])
