"""Load-time weight tiling (moe_mxfp4_tile_weights / untile): the round trip
to the canonical layout is bitwise, the tiled order is a pure reordering, and
the grouped GEMM and the layer on tiled weights equal their canonical-weight
results bitwise (same kernels, same products, same summation order) over
every row-tile class, both activation types, every epilogue and output."""
import numpy as np
import pytest
import torch

from oracle import moe as omoe
from workloads import gen
from tests.gpu_util import device_weights, device_x

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_weight_mixture_amd")
DEV = "cuda"


def _rand_w(E, N, K, seed):
    g = np.random.default_rng(seed)
    wp = torch.from_numpy(g.integers(0, 256, (E, N, K // 2), dtype=np.uint8)).to(DEV)
    ws = torch.from_numpy(g.integers(118, 131, (E, N, K // 32), dtype=np.uint8)).to(DEV)
    return wp, ws


@pytest.mark.parametrize("E,N,K", [(3, 512, 1024), (1, 256, 512), (5, 768, 1536)])
@pytest.mark.parametrize("epi", ["none", "split", "interleaved"])
def test_tile_round_trip_is_bitwise(E, N, K, epi):
    wp, ws = _rand_w(E, N, K, seed=E + N + K)
    tp, ts = mx.tile_weights(wp, ws, epi)
    torch.cuda.synchronize()
    assert not torch.equal(tp, wp)                       # reordered ...
    assert torch.equal(torch.sort(tp.flatten())[0], torch.sort(wp.flatten())[0])   # ... not changed
    assert torch.equal(torch.sort(ts.flatten())[0], torch.sort(ws.flatten())[0])
    bp, bs = mx.untile_weights(tp, ts, epi)
    torch.cuda.synchronize()
    assert torch.equal(bp, wp) and torch.equal(bs, ws)


def test_tiled_block_holds_the_stage_in_lds_order():
    """Spot check of the documented order: byte q of the 16 KB block of (expert
    e, n-tile nt, stage s) is chunk uu % 4 of the stage bytes of tile column
    2*(q//128) + uu//4, uu = slot XOR the line swizzle; for MOE_EPI_NONE tile
    column j of n-tile nt is weight row 256*nt + j."""
    E, N, K = 2, 512, 1024
    wp, ws = _rand_w(E, N, K, seed=5)
    tp, _ = mx.tile_weights(wp, ws, "none")
    w, t = wp.cpu().numpy(), tp.cpu().numpy().reshape(-1)
    nst, n_tiles = K // 128, N // 256
    g = np.random.default_rng(0)
    for _ in range(200):
        e, nt, s, q = int(g.integers(E)), int(g.integers(n_tiles)), int(g.integers(nst)), int(g.integers(1024))
        line, slot = q // 8, q % 8
        swz = ((line >> 1) & 3) ^ ((line & 1) << 1)
        uu = slot ^ swz
        j = 2 * line + (uu >> 2)
        row = 256 * nt + j
        blk = ((e * n_tiles + nt) * nst + s) * 16384 + line * 128 + slot * 16
        np.testing.assert_array_equal(t[blk: blk + 16], w[e, row, s * 64 + (uu & 3) * 16: s * 64 + (uu & 3) * 16 + 16])


def _gemm_pair(a, a_sc, gather, div, wp, ws, off, epi, out):
    kw = dict(a_scales=a_sc, a_gather=gather, a_gather_div=div, epilogue=epi, out_dtype=out)
    ref = mx.grouped_gemm(a, wp, ws, off, **kw)
    tp, ts = mx.tile_weights(wp, ws, epi)
    got = mx.grouped_gemm(a, tp, ts, off, w_format="tiled", **kw)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("epi,out", [("none", "bf16"), ("none", "fp32"), ("split", "bf16"),
                                     ("interleaved", "bf16"), ("interleaved", "mxfp8"), ("split", "fp32")])
def test_gemm_on_tiled_weights_equals_canonical_bitwise(fp8, epi, out):
    if out == "mxfp8" and not fp8:
        pytest.skip("the MXFP8 intermediate follows MXFP8 activations")
    g = np.random.default_rng(21)
    counts = [1, 33, 64, 65, 100, 129, 256, 300]     # every row-tile class, ragged tails
    E, N, K = len(counts), 512, 1024
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(DEV)
    rows = int(sum(counts))
    x = torch.from_numpy(g.standard_normal((rows, K)).astype(np.float32)).to(torch.bfloat16)
    if fp8:
        codes, scales = gen.quantize_mxfp8(x.float())
        a, a_sc = codes.to(DEV), scales.to(DEV)
    else:
        a, a_sc = x.to(DEV), None
    wp, ws = _rand_w(E, N, K, seed=9)
    ref, got = _gemm_pair(a, a_sc, None, 1, wp, ws, off, epi, out)
    if out == "mxfp8":
        assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    else:
        assert torch.equal(ref, got)


def test_gemm_on_tiled_weights_with_gathered_rows():
    g = np.random.default_rng(4)
    T, k, E, N, K = 200, 4, 9, 768, 512
    ids, _ = omoe.route(g.standard_normal((T, E)).astype(np.float32), k)
    off, perm_src, _ = omoe.permute(ids, E)
    x = torch.from_numpy(g.standard_normal((T, K)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    wp, ws = _rand_w(E, N, K, seed=2)
    ref, got = _gemm_pair(x, None, torch.from_numpy(perm_src).to(DEV), k, wp, ws,
                          torch.from_numpy(off).to(DEV), "split", "bf16")
    assert torch.equal(ref, got)


@pytest.mark.parametrize("act,layout,inter", [("bf16", "split", "bf16"), ("mxfp8", "interleaved", "mxfp8"),
                                              ("mxfp8", "split", "bf16")])
def test_layer_on_tiled_weights_equals_canonical_bitwise(act, layout, inter):
    s = gen.preset("tiny", T=300, H=1024, I=512, E=6, k=3, act=act, layout=layout)
    li = gen.layer_inputs(s)
    w = device_weights(s)
    x, xs = device_x(li)
    logits = torch.from_numpy(li.logits).to(DEV)
    ref = mx.Layer(*w, k=s.k, layout=layout, inter=inter).forward(logits, x, xs)
    got = mx.Layer(*w, k=s.k, layout=layout, inter=inter, tile=True).forward(logits, x, xs)
    torch.cuda.synchronize()
    assert torch.equal(ref, got)
