"""The MoE layer with MXFP4 expert weights, written out plainly (oracle side).

Test infrastructure: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use this package.  It shares no code with the HIP
path; float64 throughout.

What the pages fix, and where:
* top-k expert selection per token: 256 experts / top-6 (ktransformers
  issue #2172, "Environment"), 896 experts / top-16 ("Kimi-K3 SM120
  FlashInfer MXFP4 MoE", Phase-0 audit table);
* dispatch of the routed tokens to the expert compute (issue #2172,
  "Impact": the MoE method is applied to the dispatch output);
* a gated activation makes FC1 twice as wide as FC2's inner size (Kimi-K3
  page, on-machine evidence: the "256 vs. 128" inter-size check);
* the gate/up row arrangement must be stated explicitly (Kimi-K3 page,
  Phase-1 gates, item 2);
* the fused MoE ends in the weighted top-k combine (Kimi-K3 page, goal).

What the pages leave open, and the reading taken here:
* router: softmax over the experts, keep the k largest, renormalise over
  the k kept.  Selection uses the fp32 logits (softmax is monotone), ties
  go to the lower expert index, slots are in selection order.  Weights
  are exp(l_j - max) / sum over the k kept: the full-softmax denominator
  cancels.
* permutation: stable counting sort of the flat pairs f = t*k + j by
  expert.
* activation: SwiGLU, act = silu(gate) * up, silu(z) = z / (1 + e**-z);
  layouts "split" (gate rows [0, I), up rows [I, 2I)) and "interleaved"
  (gate row 2i, up row 2i+1).
* combine: out[t] = sum_j w[t][j] * Y[row of (t, j)], j ascending.
* stacked layers: x_{L+1} = bf16(y_L / rms(y_L)) per token (the pages
  give no norm or residual between layers; this keeps 43 random layers
  finite).
"""
from __future__ import annotations

import numpy as np

from .mx import dequant_mxfp4, dequant_mxfp8, bf16_value


# ---------------------------------------------------------------- routing

def route(logits, k):
    """Top-k experts per token and their renormalised softmax weights.

    logits: fp32 [T][E].  Returns ids int32 [T][k] (best first; equal
    logits -> lower index first) and w float64 [T][k].
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # order by (logit descending, index ascending); lexsort's last key is primary
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -lg.astype(np.float64)), axis=1)
    ids = order[:, :k].astype(np.int32)
    top = np.take_along_axis(lg, ids, axis=1).astype(np.float64)
    m = lg.astype(np.float64).max(axis=1, keepdims=True)
    p = np.exp(top - m)
    w = p / p.sum(axis=1, keepdims=True)
    return ids, w


# ------------------------------------------------------------ permutation

def permute(ids, E):
    """Stable counting sort of the (token, slot) pairs by expert.

    ids: int [T][k].  Returns offsets int32 [E+1] (exclusive prefix of the
    per-expert counts), perm_src int32 [T*k] (permuted row -> flat index
    f = t*k + j) and dest_row int32 [T*k] (f -> permuted row).
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    seen = np.zeros(E, dtype=np.int64)
    perm_src = np.empty(flat.size, dtype=np.int32)
    dest_row = np.empty(flat.size, dtype=np.int32)
    for f, e in enumerate(flat):
        row = offsets[e] + seen[e]
        seen[e] += 1
        perm_src[row] = f
        dest_row[f] = row
    return offsets.astype(np.int32), perm_src, dest_row


# ------------------------------------------------------------ expert MLP

def silu(z):
    return z / (1.0 + np.exp(-z))


def gate_up(h1, layout):
    """Split FC1's output [n][2I] into (gate, up) [n][I] per the row layout."""
    two_i = h1.shape[-1]
    if layout == "split":
        return h1[..., : two_i // 2], h1[..., two_i // 2:]
    if layout == "interleaved":
        return h1[..., 0::2], h1[..., 1::2]
    raise ValueError(layout)


def expert_mlp(X, W1, W2, layout):
    """One expert on its rows.  X [n][H], W1 [2I][H], W2 [H][I] (float64) -> Y [n][H]."""
    h1 = X @ W1.T
    g, u = gate_up(h1, layout)
    act = silu(g) * u
    return act @ W2.T


# ---------------------------------------------------------------- combine

def combine(Y, dest_row, w):
    """out[t] = sum_{j ascending} w[t][j] * Y[dest_row[t*k + j]]."""
    T, k = w.shape
    out = np.zeros((T, Y.shape[1]), dtype=np.float64)
    rows = np.asarray(dest_row).reshape(T, k)
    for j in range(k):
        out += w[:, j:j + 1] * Y[rows[:, j]]
    return out


# ------------------------------------------------------------- one layer

def activations(x_bf16=None, x_codes=None, x_scales=None):
    """Layer input as float64: bf16 bit patterns, or MXFP8 codes + E8M0 scales."""
    if x_codes is not None:
        return dequant_mxfp8(x_codes, x_scales)
    return bf16_value(x_bf16)


def moe_layer(x, logits, k, weights, layout, return_intermediates=False):
    """The whole layer.

    x: float64 [T][H]; logits fp32 [T][E]; weights(e) -> (w1_packed,
    w1_scales, w2_packed, w2_scales) for expert e (uint8 arrays, MXFP4).
    Experts are dequantised one at a time and only when they received
    tokens.  Returns out float64 [T][H] (and the routing arrays).
    """
    T, E = np.asarray(logits).shape
    ids, w = route(logits, k)
    offsets, perm_src, dest_row = permute(ids, E)
    Y = np.zeros((T * k, x.shape[1]), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        w1p, w1s, w2p, w2s = weights(e)
        W1 = dequant_mxfp4(w1p, w1s)
        W2 = dequant_mxfp4(w2p, w2s)
        X = x[perm_src[lo:hi] // k]
        Y[lo:hi] = expert_mlp(X, W1, W2, layout)
    out = combine(Y, dest_row, w)
    if return_intermediates:
        return out, dict(ids=ids, w=w, offsets=offsets, perm_src=perm_src,
                         dest_row=dest_row, Y=Y)
    return out


def moe_tokens(x_rows, ids, w, weights, layout):
    """The layer's output for a few tokens, given their routing.

    x_rows float64 [n][H]; ids int [n][k]; w [n][k].  Each expert that
    any of these tokens uses is dequantised once.  Used to check sampled
    tokens of full-size workloads.
    """
    n, k = ids.shape
    Yt = np.zeros((n, k, x_rows.shape[1]), dtype=np.float64)
    for e in np.unique(ids):
        tok, slot = np.nonzero(ids == e)
        w1p, w1s, w2p, w2s = weights(int(e))
        Yt[tok, slot] = expert_mlp(x_rows[tok], dequant_mxfp4(w1p, w1s),
                                   dequant_mxfp4(w2p, w2s), layout)
    out = np.zeros((n, x_rows.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * Yt[:, j]
    return out


# ---------------------------------------------------- stacked / streamed

def rms_rescale(y):
    """Per-token y / sqrt(mean_h y**2) (float64); the next layer's input before bf16 rounding."""
    r = np.sqrt(np.mean(np.square(y), axis=1, keepdims=True))
    return y / r


def to_bf16_bits(v):
    """float64 -> bf16 bit patterns, via fp32 and round-to-nearest-even."""
    f = np.asarray(v, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def streamed_layers(x0_bits, logits_per_layer, k, weights_per_layer, layout):
    """The stacked layers without teacher forcing: returns every layer's output."""
    x = bf16_value(x0_bits)
    outs = []
    for L, lg in enumerate(logits_per_layer):
        y = moe_layer(x, lg, k, lambda e, L=L: weights_per_layer(L, e), layout)
        outs.append(y)
        x = bf16_value(to_bf16_bits(rms_rescale(y)))
    return outs
