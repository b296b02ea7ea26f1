"""Seeded synthetic inputs for the MXFP4 mixture-of-experts layer.

This module only *produces* inputs.  It holds none of the layer's own
arithmetic (no decoding of MX numbers, no routing, no matmul): both the
CPU oracle and the GPU path consume exactly the arrays made here.

Shapes and value laws follow the workloads described on the pages: the
DeepSeek-V4-Flash shape (256 experts, top-6, 43 layers, native MXFP4;
ktransformers issue #2172, "Environment") and the Kimi-K3 shape (hidden
7168, expert hidden 3584, 896 experts, top-16; "Kimi-K3 SM120 FlashInfer
MXFP4 MoE", Phase-0 audit table).  Token counts 1/2/8/32 come from the
Phase-1 coverage list of the same page.

Weights (the bulk of every workload) come from a counter-based generator:
byte stream = MurmurHash3's 32-bit finaliser ``fmix32`` (Appleby, public
domain) applied twice to ``counter XOR key``.  It is written with torch
int64 ops whose products never exceed 2**63, so the *same* function runs
on the CPU (oracle side, one expert at a time) and on the GPU (bulk
generation of tens of GB), bit-identically.

Activations and router logits come from numpy's PCG64 with a
``SeedSequence(seed, spawn_key=(config, tensor, index))``.

MXFP8 inputs (the Kimi-K3-shaped prefill workload) are quantised here from
the bf16 activations, with the OCP Microscaling (MX) v1.0 conversion rule
(shared scale X = floor(log2(amax)) - emax(E4M3) = ... - 8, elements rounded
to nearest-even and saturated at +-448).  That quantisation is input
preparation: the layer consumes the resulting bytes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

# tensor ids of the spawn keys / counter-generator keys
T_X, T_LOGITS, T_BIAS, T_W1, T_S1, T_W2, T_S2 = range(7)

M32 = (1 << 32) - 1


@dataclass(frozen=True)
class LayerShape:
    """One MoE layer's sizes and value laws."""
    T: int                 # tokens
    H: int                 # hidden size (FC1 K, FC2 N)
    I: int                 # expert intermediate size (FC1 N = 2*I, FC2 K)
    E: int                 # experts
    k: int                 # experts per token
    layout: str = "split"  # "split": gate rows [0,I), up rows [I,2I); "interleaved": gate 2i, up 2i+1
    act: str = "bf16"      # "bf16" or "mxfp8"
    logit_sigma: float = 1.0
    bias: Optional[str] = None   # None, "hot" (2% of experts +2.0) or "zipf" (-1.1*ln(rank))
    cfg_id: int = 0        # namespace of the seeds
    seed: int = 0
    layers: int = 1        # >1 only for the streamed stack

    def __post_init__(self):
        if self.H % 32 or self.I % 32:
            raise ValueError("H and I must be multiples of the 32-element MX block")
        if not (1 <= self.k <= self.E):
            raise ValueError("need 1 <= k <= E")


# Workload presets.  Sizes are the pages' model shapes; value laws are the
# synthetic ones the workload descriptions give.
PRESETS = {
    # FlashInfer's minimal MXFP8xMXFP4 fused-MoE test scale (Kimi-K3 page,
    # on-machine evidence): hidden 128, 2-4 experts, top-2, inter 128.
    "tiny": LayerShape(T=32, H=128, I=128, E=4, k=2, layout="split", cfg_id=1),
    # Kimi-K3 shape, decode-sized token counts (Phase-1 list: 1/2/8/32).
    "decode": LayerShape(T=32, H=7168, I=3584, E=896, k=16, bias="hot", cfg_id=2),
    # DeepSeek-V4-Flash shape (256 experts, top-6), one resident layer.
    "prefill256": LayerShape(T=4096, H=4096, I=2048, E=256, k=6, logit_sigma=1.5, cfg_id=3),
    # Kimi-K3 shape, MXFP8 activations, Zipf-skewed routing, interleaved gate/up.
    "prefill896_mxfp8": LayerShape(T=8192, H=7168, I=3584, E=896, k=16, act="mxfp8",
                                   bias="zipf", layout="interleaved", cfg_id=4),
    # 43 stacked DeepSeek-V4-Flash-shaped layers streamed from pinned host memory.
    "streamed": LayerShape(T=16384, H=4096, I=2048, E=256, k=6, logit_sigma=1.5,
                           cfg_id=5, layers=43),
}


def preset(name: str, **overrides) -> LayerShape:
    return replace(PRESETS[name], **overrides)


# ---------------------------------------------------------------------------
# counter-based generator (torch int64, device-agnostic, bit-exact)
# ---------------------------------------------------------------------------

def _mul32(a: torch.Tensor, c: int) -> torch.Tensor:
    """(a * c) mod 2**32 for 0 <= a < 2**32, without int64 overflow."""
    lo = c & 0xFFFF
    hi = c >> 16
    return (a * lo + (((a * hi) & 0xFFFF) << 16)) & M32


def fmix32(h: torch.Tensor) -> torch.Tensor:
    """MurmurHash3's 32-bit finaliser on int64 tensors holding 0..2**32-1."""
    h = h ^ (h >> 16)
    h = _mul32(h, 0x85EBCA6B)
    h = h ^ (h >> 13)
    h = _mul32(h, 0xC2B2AE35)
    h = h ^ (h >> 16)
    return h


def _fmix32_int(h: int) -> int:
    h &= M32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & M32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & M32
    h ^= h >> 16
    return h


def stream_key(seed: int, cfg_id: int, tensor_id: int, index: int) -> int:
    k = _fmix32_int(seed ^ 0x6D786D6F)
    for v in (cfg_id, tensor_id, index):
        k = _fmix32_int(k ^ (v & M32))
        k = _fmix32_int((k + 0x9E3779B9) & M32)
    return k


def counter_words(key: int, start: int, count: int, device) -> torch.Tensor:
    """32-bit words number start..start+count-1 of the stream `key` (int64 tensor)."""
    i = torch.arange(start, start + count, dtype=torch.int64, device=device) & M32
    h = fmix32(i ^ key)
    return fmix32((h + key) & M32)


def _words_to_bytes(w: torch.Tensor) -> torch.Tensor:
    """int64 words (0..2**32-1) -> little-endian bytes (uint8, 4 per word)."""
    w32 = torch.where(w >= (1 << 31), w - (1 << 32), w).to(torch.int32)
    return w32.view(torch.uint8)


def random_bytes(key: int, nbytes: int, device) -> torch.Tensor:
    """Uniform bytes (every byte = two independent uniform 4-bit codes)."""
    nwords = (nbytes + 3) // 4
    return _words_to_bytes(counter_words(key, 0, nwords, device))[:nbytes]


def random_scales(key: int, count: int, device, lo: int = 121, hi: int = 127) -> torch.Tensor:
    """E8M0 bytes uniform over lo..hi inclusive (2**-6 .. 2**0 for the default)."""
    w = counter_words(key, 0, count, device)
    return (lo + (w >> 8) % (hi - lo + 1)).to(torch.uint8)


def expert_weights(shape: LayerShape, expert: int, layer: int = 0, device="cpu"):
    """MXFP4 weights of one expert.

    Returns (w1_packed [2I][H/2], w1_scales [2I][H/32], w2_packed [H][I/2],
    w2_scales [H][I/32]), all uint8.  Packed bytes hold element 2j in the low
    nibble and 2j+1 in the high nibble; the 32-element scale blocks run along
    the contiguous (reduction) axis.
    """
    H, I = shape.H, shape.I
    idx = layer * shape.E + expert
    k = lambda t: stream_key(shape.seed, shape.cfg_id, t, idx)
    w1p = random_bytes(k(T_W1), 2 * I * H // 2, device).view(2 * I, H // 2)
    w1s = random_scales(k(T_S1), 2 * I * H // 32, device).view(2 * I, H // 32)
    w2p = random_bytes(k(T_W2), H * I // 2, device).view(H, I // 2)
    w2s = random_scales(k(T_S2), H * I // 32, device).view(H, I // 32)
    return w1p, w1s, w2p, w2s


def _batched_stream(keys, count: int, device) -> torch.Tensor:
    """Words 0..count-1 of several streams at once: [len(keys)][count] (int64)."""
    k = torch.tensor(keys, dtype=torch.int64, device=device).unsqueeze(1)
    i = torch.arange(count, dtype=torch.int64, device=device).unsqueeze(0)
    h = fmix32(i ^ k)
    return fmix32((h + k) & M32)


def all_expert_weights(shape: LayerShape, layer: int = 0, device="cpu", experts=None, chunk: int = 16):
    """Weights of all experts stacked: [E][2I][H/2], [E][2I][H/32], [E][H][I/2], [E][H][I/32].

    Byte-identical to expert_weights() per expert; generated a chunk of experts
    per tensor op so that tens of GB take a few hundred device launches.
    """
    E = shape.E if experts is None else experts
    H, I = shape.H, shape.I
    out = (torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=device),
           torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=device),
           torch.empty((E, H, I // 2), dtype=torch.uint8, device=device),
           torch.empty((E, H, I // 32), dtype=torch.uint8, device=device))
    kinds = ((T_W1, False), (T_S1, True), (T_W2, False), (T_S2, True))
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        for t, (tid, is_scale) in zip(out, kinds):
            keys = [stream_key(shape.seed, shape.cfg_id, tid, layer * shape.E + e) for e in range(e0, e1)]
            n = t[0].numel()
            if is_scale:
                w = _batched_stream(keys, n, device)
                t[e0:e1].copy_((121 + (w >> 8) % 7).to(torch.uint8).view(e1 - e0, *t.shape[1:]))
            else:
                w = _batched_stream(keys, (n + 3) // 4, device)
                b = _words_to_bytes(w.reshape(-1)).view(e1 - e0, -1)[:, :n]
                t[e0:e1].copy_(b.reshape(e1 - e0, *t.shape[1:]))
            del w
    return out


# ---------------------------------------------------------------------------
# activations and router logits (numpy PCG64)
# ---------------------------------------------------------------------------

def _rng(shape: LayerShape, tensor_id: int, index: int) -> np.random.Generator:
    ss = np.random.SeedSequence(shape.seed, spawn_key=(shape.cfg_id, tensor_id, index))
    return np.random.Generator(np.random.PCG64(ss))


def activations_bf16(shape: LayerShape, index: int = 0) -> torch.Tensor:
    """x ~ N(0,1), drawn in fp32, rounded to bf16 (nearest-even).  [T][H] bf16 on CPU."""
    g = _rng(shape, T_X, index if index else shape.T)
    x = g.standard_normal((shape.T, shape.H), dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


def expert_bias(shape: LayerShape) -> np.ndarray:
    """Per-expert additive router bias (fp32 [E]); zeros when the workload has none."""
    E = shape.E
    b = np.zeros(E, dtype=np.float32)
    g = _rng(shape, T_BIAS, 0)
    if shape.bias == "hot":
        # 2 % of the experts, chosen without replacement, get +2.0
        n_hot = int(round(0.02 * E))
        b[g.choice(E, size=n_hot, replace=False)] = 2.0
    elif shape.bias == "zipf":
        # Zipf(s=1.1) popularity over a random ranking: p(rank r) ~ r**-1.1,
        # applied through the softmax as the log-popularity -1.1*ln(r).
        ranks = g.permutation(E) + 1
        b = (-1.1 * np.log(ranks.astype(np.float64))).astype(np.float32)
    elif shape.bias is not None:
        raise ValueError(shape.bias)
    return b


def router_logits(shape: LayerShape, layer: int = 0, index: int = 0) -> np.ndarray:
    """fp32 [T][E]: N(0, sigma) plus the per-expert bias (fp32 add)."""
    g = _rng(shape, T_LOGITS, layer * 1000 + (index if index else shape.T))
    z = g.standard_normal((shape.T, shape.E), dtype=np.float32)
    if shape.logit_sigma != 1.0:
        z = (z * np.float32(shape.logit_sigma)).astype(np.float32)
    return (z + expert_bias(shape)[None, :]).astype(np.float32)


# ---------------------------------------------------------------------------
# MXFP8 (E4M3 + E8M0 block-of-32) quantisation of the bf16 activations
# ---------------------------------------------------------------------------

E4M3_EMAX = 8        # exponent of E4M3's largest normal (448 = 1.75 * 2**8)
E4M3_MAX = 448.0


def quantize_mxfp8(x: torch.Tensor):
    """OCP MX conversion of a [rows][K] tensor (K % 32 == 0) to MXFP8 E4M3.

    Per block of 32: X = floor(log2(max|v|)) - 8 (clamped to [-127, 127]);
    scale byte = X + 127; elements = v * 2**-X rounded to nearest-even on the
    E4M3 grid, saturated at +-448.  An all-zero block gets X = -127.
    Returns (codes uint8 [rows][K], scales uint8 [rows][K/32]).
    """
    rows, K = x.shape
    v = x.to(torch.float64).reshape(rows, K // 32, 32)
    amax = v.abs().amax(dim=2)
    # floor(log2(amax)) exactly, via frexp: amax = m * 2**e with m in [0.5, 1)
    _, e = torch.frexp(amax)
    X = (e.to(torch.int64) - 1) - E4M3_EMAX
    X = torch.where(amax > 0, X, torch.full_like(X, -127)).clamp(-127, 127)
    q = v * torch.pow(2.0, -X.to(torch.float64)).unsqueeze(2)   # exact (power of two)
    sign = torch.signbit(q)
    a = q.abs()
    # E4M3 grid: 3 mantissa bits, exponent bias 7, min normal 2**-6, subnormal step 2**-9
    _, ea = torch.frexp(a)
    ea = (ea.to(torch.int64) - 1).clamp(min=-6)
    step = torch.pow(2.0, (ea - 3).to(torch.float64))
    r = torch.round(a / step) * step          # torch.round is half-to-even
    r = torch.clamp(r, max=E4M3_MAX)
    # encode r (a grid value) into the byte s.eeee.mmm
    _, er = torch.frexp(r)
    er = (er.to(torch.int64) - 1)
    is_sub = r < 2.0 ** -6
    exp_field = torch.where(is_sub, torch.zeros_like(er), er + 7)
    mant = torch.where(is_sub, torch.round(r / 2.0 ** -9),
                       torch.round((r / torch.pow(2.0, er.to(torch.float64)) - 1.0) * 8))
    code = (exp_field << 3) | mant.to(torch.int64)
    code = code | (sign.to(torch.int64) << 7)
    codes = code.reshape(rows, K).to(torch.uint8)
    scales = (X + 127).to(torch.uint8)
    return codes, scales


# ---------------------------------------------------------------------------
# one workload's host-side inputs
# ---------------------------------------------------------------------------

@dataclass
class LayerInputs:
    shape: LayerShape
    x_bf16: torch.Tensor                 # [T][H] bf16 (CPU)
    logits: np.ndarray                   # [T][E] fp32
    x_codes: Optional[torch.Tensor] = None   # [T][H] uint8 E4M3 (MXFP8 workloads)
    x_scales: Optional[torch.Tensor] = None  # [T][H/32] uint8 E8M0
    extra: dict = field(default_factory=dict)


def layer_inputs(shape: LayerShape, index: int = 0, layer: int = 0) -> LayerInputs:
    x = activations_bf16(shape, index)
    lg = router_logits(shape, layer, index)
    li = LayerInputs(shape, x, lg)
    if shape.act == "mxfp8":
        li.x_codes, li.x_scales = quantize_mxfp8(x.float())
    return li


def flops(shape: LayerShape) -> float:
    """Algorithmic flops of one layer: FC1 (2I x H) + FC2 (H x I) for T*k rows."""
    return 2.0 * shape.T * shape.k * 3 * shape.H * shape.I


def expert_bytes(shape: LayerShape) -> int:
    """MXFP4 bytes of one expert: 3*H*I weights at 4 bits + one E8M0 byte per 32."""
    n = 3 * shape.H * shape.I
    return n // 2 + n // 32
