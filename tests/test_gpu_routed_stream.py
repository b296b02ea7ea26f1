"""Routed expert copy in the streamed prefill: only the experts a layer's
routing hits cross the host link, and the results are bitwise those of the
all-experts stream.

The hit set is checked against the oracle's routing of the same logits (not
against the GPU's own routing): every expert the oracle routes a token to is
copied byte for byte, every other expert's slot bytes are left untouched.
"""
import numpy as np
import pytest
import torch

from oracle import moe as omoe
from workloads import gen

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_weight_mixture_amd")
DEV = "cuda"
FILL = 0xA5


def _blobs(s, n_blobs, w_format="canonical"):
    H, I, E = s.H, s.I, s.E
    nbytes = mx.blob_bytes(H, I, E)
    blobs = []
    for b in range(n_blobs):
        blob = torch.zeros(nbytes, dtype=torch.uint8, pin_memory=True)
        w1p, w1s, w2p, w2s = gen.all_expert_weights(s, layer=b, device=DEV)
        if w_format == "tiled":
            w1p, w1s = mx.tile_weights(w1p, w1s, epilogue=s.layout)
            w2p, w2s = mx.tile_weights(w2p, w2s, epilogue="none")
        for which, t in enumerate((w1p, w1s, w2p, w2s)):
            o = mx.blob_section_offset(H, I, E, which)
            blob[o:o + t.numel()] = t.reshape(-1).cpu()
        blobs.append(blob)
    torch.cuda.synchronize()
    return blobs


def _stream(s, blobs, L, depth=2, chain="rms", expert_copy="all", max_tokens=0, w_format="canonical",
            slots=None):
    nbytes = blobs[0].numel()
    if slots is None:
        slots = [torch.full((nbytes,), FILL, dtype=torch.uint8, device=DEV) for _ in range(2)]
    logits = torch.from_numpy(np.stack([gen.router_logits(s, l) for l in range(L)])).to(DEV)
    x = gen.activations_bf16(s).to(DEV)
    out = torch.empty((s.T, s.H), dtype=torch.float32, device=DEV)
    caps = torch.empty((L, s.T, s.H), dtype=torch.bfloat16, device=DEV)
    copy = torch.cuda.Stream()
    mx.prefill_streamed(blobs, slots, logits, x, out, T=s.T, H=s.H, I=s.I, E=s.E, k=s.k, num_layers=L,
                        layout=s.layout, chain=chain, depth=depth, layer_inputs=caps, copy_stream=copy,
                        w_format=w_format, expert_copy=expert_copy, routed_copy_max_tokens=max_tokens)
    torch.cuda.synchronize()
    return out, caps, slots, logits


def _expert_ranges(s):
    """(section offset, bytes per expert) of the four blob sections."""
    H, I = s.H, s.I
    per = [2 * I * (H // 2), 2 * I * (H // 32), H * (I // 2), H * (I // 32)]
    return [(mx.blob_section_offset(H, I, s.E, w), per[w]) for w in range(4)]


def _check_slot(s, slot, blob, hit):
    """Hit experts' bytes equal the blob's; the others still hold FILL."""
    sl = slot.cpu().numpy()
    bl = blob.numpy()
    for off, per in _expert_ranges(s):
        for e in range(s.E):
            a, b = off + e * per, off + (e + 1) * per
            if e in hit:
                assert np.array_equal(sl[a:b], bl[a:b]), f"expert {e} not copied"
            else:
                assert (sl[a:b] == FILL).all(), f"expert {e} has no routed row but was written"


@pytest.mark.parametrize("depth", [2, 1])
@pytest.mark.parametrize("chain", ["rms", "independent"])
def test_routed_copy_equals_all_experts_bitwise(depth, chain):
    # 6 tokens x top-2 over 16 experts: most experts are idle in every layer
    s = gen.LayerShape(T=6, H=256, I=128, E=16, k=2, cfg_id=150, layers=4)
    blobs = _blobs(s, 2)
    out_a, caps_a, _, logits = _stream(s, blobs, 4, depth, chain, "all")
    out_r, caps_r, _, _ = _stream(s, blobs, 4, depth, chain, "routed")
    assert torch.equal(out_a, out_r) and torch.equal(caps_a, caps_r)
    hits = [set(np.unique(omoe.route(logits[l].cpu().numpy(), s.k)[0]).tolist()) for l in range(4)]
    assert all(len(h) < s.E for h in hits)


def test_routed_copy_writes_exactly_the_hit_experts():
    s = gen.LayerShape(T=5, H=256, I=128, E=24, k=3, cfg_id=151, layers=1)
    blobs = _blobs(s, 1)
    _, _, slots, logits = _stream(s, blobs, 1, depth=1, expert_copy="routed")
    hit = set(np.unique(omoe.route(logits[0].cpu().numpy(), s.k)[0]).tolist())
    assert 0 < len(hit) < s.E
    _check_slot(s, slots[0], blobs[0], hit)


def test_routed_copy_slots_alternate_per_layer():
    # depth 2: layer L fills slot L % 2 with layer L's hit experts of blob L % 2
    s = gen.LayerShape(T=3, H=128, I=64, E=32, k=2, cfg_id=152, layers=2)
    blobs = _blobs(s, 2)
    _, _, slots, logits = _stream(s, blobs, 2, depth=2, expert_copy="routed")
    for L in range(2):
        hit = set(np.unique(omoe.route(logits[L].cpu().numpy(), s.k)[0]).tolist())
        _check_slot(s, slots[L], blobs[L], hit)


def test_auto_copy_follows_the_token_threshold():
    s = gen.LayerShape(T=4, H=128, I=64, E=16, k=2, cfg_id=153, layers=1)
    blobs = _blobs(s, 1)
    out_all, _, slots, logits = _stream(s, blobs, 1, depth=1, expert_copy="auto", max_tokens=s.T - 1)
    _check_slot(s, slots[0], blobs[0], set(range(s.E)))        # T above the threshold: every expert
    out_r, _, slots, _ = _stream(s, blobs, 1, depth=1, expert_copy="auto", max_tokens=s.T)
    hit = set(np.unique(omoe.route(logits[0].cpu().numpy(), s.k)[0]).tolist())
    _check_slot(s, slots[0], blobs[0], hit)                     # T at the threshold: routed only
    assert torch.equal(out_all, out_r)


def test_routed_copy_on_tiled_blobs_equals_all_experts():
    s = gen.LayerShape(T=4, H=512, I=512, E=8, k=2, cfg_id=154, layers=2)
    blobs = _blobs(s, 2, w_format="tiled")
    out_a, caps_a, _, _ = _stream(s, blobs, 3, expert_copy="all", w_format="tiled")
    out_r, caps_r, _, _ = _stream(s, blobs, 3, expert_copy="routed", w_format="tiled")
    assert torch.equal(out_a, out_r) and torch.equal(caps_a, caps_r)
    # and the tiled stream equals the canonical one
    out_c, caps_c, _, _ = _stream(s, _blobs(s, 2), 3, expert_copy="routed")
    assert torch.equal(out_c, out_r) and torch.equal(caps_c, caps_r)


def test_routed_copy_many_tokens_hits_every_expert():
    # enough tokens that every expert is hit: the routed stream copies the whole blob
    s = gen.LayerShape(T=300, H=256, I=128, E=8, k=2, cfg_id=155, layers=1)
    blobs = _blobs(s, 1)
    out_a, _, _, _ = _stream(s, blobs, 1, depth=1, expert_copy="all")
    out_r, _, slots, logits = _stream(s, blobs, 1, depth=1, expert_copy="routed")
    assert torch.equal(out_a, out_r)
    hit = set(np.unique(omoe.route(logits[0].cpu().numpy(), s.k)[0]).tolist())
    assert hit == set(range(s.E))
    _check_slot(s, slots[0], blobs[0], hit)


def test_routed_copy_zero_tokens_copies_nothing():
    s = gen.LayerShape(T=0, H=128, I=64, E=4, k=2, cfg_id=156, layers=2)
    nbytes = mx.blob_bytes(s.H, s.I, s.E)
    blobs = [torch.zeros(nbytes, dtype=torch.uint8, pin_memory=True)]
    slots = [torch.full((nbytes,), FILL, dtype=torch.uint8, device=DEV) for _ in range(2)]
    # zero-size tensors have no address; the call still wants non-null pointers
    logits = torch.zeros(1, dtype=torch.float32, device=DEV)
    x = torch.zeros(1, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(1, dtype=torch.float32, device=DEV)
    mx.prefill_streamed(blobs, slots, logits, x, out, T=0, H=s.H, I=s.I, E=s.E, k=s.k, num_layers=2,
                        expert_copy="routed")
    torch.cuda.synchronize()
    assert all((sl == FILL).all() for sl in slots)
