"""Each ABI call on the GPU against the oracle: routing and permutation bit-exact,
the grouped GEMM bitwise on one-hot inputs and within fp32 rounding on random ones,
the combine within fp32 rounding."""
import numpy as np
import pytest
import torch

from oracle import moe as omoe
from oracle import mx as omx
from workloads import gen
from tests.gpu_util import rel_err

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_weight_mixture_amd")
DEV = "cuda"


def test_device_is_gfx950():
    assert mx.device_supported(), "the GPU path only runs on gfx950"


# ---------------------------------------------------------------- routing

@pytest.mark.parametrize("T,E,k,sigma", [
    (32, 4, 2, 1.0), (1, 896, 16, 1.0), (257, 896, 16, 1.0), (3, 7, 7, 1.0), (100, 256, 6, 1.5),
    (64, 1024, 64, 1.0), (5, 1, 1, 1.0), (130, 65, 3, 1.0),
])
def test_route_bit_exact(T, E, k, sigma):
    g = np.random.default_rng(T * 1000 + E)
    lg = (g.standard_normal((T, E)) * sigma).astype(np.float32)
    ids, w = mx.route(torch.from_numpy(lg).to(DEV), k)
    rid, rw = omoe.route(lg, k)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=0)


def test_route_ties_signed_zero_and_nan():
    g = np.random.default_rng(1)
    lg = g.integers(-2, 3, (200, 40)).astype(np.float32)   # heavy ties
    lg[0, :] = 0.0
    lg[0, ::2] = -0.0                                       # -0 == +0: lower id first
    lg[1, 5] = np.nan                                       # NaN sorts last
    lg[2, :] = -np.inf
    lg[2, 7] = 1.0
    ids, w = mx.route(torch.from_numpy(lg).to(DEV), 8)
    rid, rw = omoe.route(lg, 8)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    assert 5 not in ids[1].tolist()
    ok = np.isfinite(rw).all(axis=1)
    np.testing.assert_allclose(w.cpu().numpy()[ok], rw[ok], rtol=1e-6)


def test_route_zipf_workload_full_size():
    s = gen.preset("prefill896_mxfp8")
    lg = gen.router_logits(s)
    ids, w = mx.route(torch.from_numpy(lg).to(DEV), s.k)
    rid, rw = omoe.route(lg, s.k)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-6)


# ------------------------------------------------------------ permutation

def _perm_check(ids_np, E):
    ids = torch.from_numpy(ids_np.astype(np.int32)).to(DEV)
    off, ps, dr = mx.permute(ids, E)
    roff, rps, rdr = omoe.permute(ids_np, E)
    np.testing.assert_array_equal(off.cpu().numpy(), roff)
    np.testing.assert_array_equal(ps.cpu().numpy(), rps)
    np.testing.assert_array_equal(dr.cpu().numpy(), rdr)


# T*k <= 1024 runs the one-block permutation; (64, 896, 16) is exactly one chunk, (1025, 7, 1) one entry more
@pytest.mark.parametrize("T,E,k", [(32, 4, 2), (257, 896, 16), (1, 5, 1), (4096, 256, 6), (3, 1, 1),
                                   (64, 896, 16), (1025, 7, 1), (100, 8192, 8), (1, 896, 16)])
def test_permute_bit_exact(T, E, k):
    g = np.random.default_rng(T + E + k)
    lg = g.standard_normal((T, E)).astype(np.float32)
    ids, _ = omoe.route(lg, k)
    _perm_check(ids, E)


def test_permute_skewed_full_size_and_degenerate():
    s = gen.preset("prefill896_mxfp8")
    ids, _ = omoe.route(gen.router_logits(s), s.k)
    _perm_check(ids, s.E)                              # 131072 pairs, Zipf-skewed
    _perm_check(np.full((3000, 1), 7, dtype=np.int32), 9)   # every token to one expert
    off, ps, dr = mx.permute(torch.zeros((0, 2), dtype=torch.int32, device=DEV), 6)
    assert off.cpu().tolist() == [0] * 7 and ps.numel() == 0


@pytest.mark.parametrize("T,E,k,seed", [
    (9000, 8192, 8, 0),      # the largest E (13 id bits), 71 chunks: the column scan carries across 64
    (1500, 1024, 4, 1),      # ids with bit 9 set next to the last chunk's unused lanes
    (70000, 3, 2, 2),        # 137 chunks, few experts: long same-expert runs in every 64 entries
])
def test_permute_uniform_ids_many_chunks(T, E, k, seed):
    g = np.random.default_rng(seed)
    ids = g.integers(0, E, (T, k), dtype=np.int32)    # repeats within a token are allowed here
    _perm_check(ids, E)


# ------------------------------------------------------ grouped GEMM

def _rand_w(E, N, K, seed, lo=121, hi=127):
    g = np.random.default_rng(seed)
    wp = g.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    ws = g.integers(lo, hi + 1, (E, N, K // 32), dtype=np.uint8)
    return wp, ws


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


# 160: register-staged kernels; 512 / 1024 / 1536 / 2560: three-stage DMA kernels with
# one to five groups of four stages
@pytest.mark.parametrize("K", [160, 512, 1024, 1536, 2560])
@pytest.mark.parametrize("fp8", [False, True])
# [96, 97, 200, 72]: the bf16 128-row tile on either side of the 96 rows up to
# which it leaves its last 32-row fragment out (200 = a full tile + 72)
@pytest.mark.parametrize("counts", [[40, 0, 300], [1, 33, 64, 65, 129, 256, 257], [96, 97, 200, 72]])
def test_gemm_one_hot_rows_return_the_dequantised_weights_bitwise(fp8, counts, K):
    """A row r of expert e is the unit vector on column (r - off[e]) % K, so
    C[r][n] = dequant(W_e)[n][(r - off[e]) % K] exactly (one nonzero product)."""
    E, N = len(counts), 320
    wp, ws = _rand_w(E, N, K, seed=len(counts) + fp8, lo=100, hi=150)
    off = _offsets(counts)
    rows = int(off[-1])
    col = np.concatenate([np.arange(c) % K for c in counts]).astype(np.int64)
    if fp8:
        codes = np.zeros((rows, K), dtype=np.uint8)
        codes[np.arange(rows), col] = 0x38                   # E4M3 1.0
        sc = np.full((rows, K // 32), 127, dtype=np.uint8)
        sc[::3] = 128                                        # every third row scaled by 2
        a = torch.from_numpy(codes).to(DEV)
        a_sc = torch.from_numpy(sc).to(DEV)
    else:
        a32 = np.zeros((rows, K), dtype=np.float32)
        a32[np.arange(rows), col] = 1.0
        a = torch.from_numpy(a32).to(torch.bfloat16).to(DEV)
        a_sc = None
    c = mx.grouped_gemm(a, torch.from_numpy(wp).to(DEV), torch.from_numpy(ws).to(DEV),
                        torch.from_numpy(off).to(DEV), a_scales=a_sc, out_dtype="fp32")
    got = c.cpu().numpy()
    want = np.empty((rows, N))
    for e in range(E):
        W = omx.dequant_mxfp4(wp[e], ws[e])
        for r in range(off[e], off[e + 1]):
            want[r] = W[:, col[r]]
    if fp8:
        want[::3] *= 2
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


def _gemm_oracle(a64, gather, div, wp, ws, off, layout):
    rows = int(off[-1])
    out = None
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        src = gather[lo:hi] // div if gather is not None else np.arange(lo, hi)
        h = a64[src] @ omx.dequant_mxfp4(wp[e], ws[e]).T
        if layout != "none":
            gt, up = omoe.gate_up(h, layout)
            h = omoe.silu(gt) * up
        if out is None:
            out = np.zeros((rows, h.shape[1]))
        out[lo:hi] = h
    return out


@pytest.mark.parametrize("K", [288, 512])   # ragged K stage vs whole 128-element stages
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("layout", ["none", "split", "interleaved"])
def test_gemm_random_against_oracle(fp8, layout, K):
    g = np.random.default_rng(7)
    T, k, E, N = 150, 3, 5, 384
    ids, _ = omoe.route(g.standard_normal((T, E)).astype(np.float32), k)
    ids[:40] = np.array([0, 1, 2])       # load expert 0..2 heavily: > 64 rows each
    off, perm_src, _ = omoe.permute(ids, E)
    x = torch.from_numpy(g.standard_normal((T, K)).astype(np.float32)).to(torch.bfloat16)
    wp, ws = _rand_w(E, N, K, seed=3)
    if fp8:
        codes, scales = gen.quantize_mxfp8(x.float())
        a = codes.to(DEV)
        a_sc = scales.to(DEV)
        a64 = omx.dequant_mxfp8(codes.numpy(), scales.numpy())
    else:
        a = x.to(DEV)
        a_sc = None
        a64 = omx.bf16_value(x.view(torch.int16).numpy())
    c = mx.grouped_gemm(a, torch.from_numpy(wp).to(DEV), torch.from_numpy(ws).to(DEV),
                        torch.from_numpy(off).to(DEV), a_scales=a_sc,
                        a_gather=torch.from_numpy(perm_src).to(DEV), a_gather_div=k,
                        epilogue=layout, out_dtype="fp32")
    want = _gemm_oracle(a64, perm_src, k, wp, ws, off, layout)
    assert c.shape == want.shape
    # bf16 MFMA: fp32 accumulation (measured ~1e-6).  Scaled FP8 x FP4 MFMA:
    # its internal accumulation is slightly coarser (measured 1.5e-5 to 1.7e-5).
    assert rel_err(c.cpu().numpy(), want) < (1e-4 if fp8 else 1e-5)


@pytest.mark.parametrize("K", [1024, 2048, 4096])
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("layout", ["none", "split"])
def test_gemm_small_tiles_long_k_against_oracle(fp8, layout, K):
    """Experts of at most 32 rows (the 32-row class, which streams weights) with
    long K and gathered rows, against the oracle."""
    g = np.random.default_rng(K + fp8)
    counts = [1, 7, 32, 0, 19, 32, 3]
    E, N = len(counts), 512
    off = _offsets(counts)
    rows = int(off[-1])
    T, div = rows // 2 + 1, 2
    perm_src = g.permutation(2 * T)[:rows].astype(np.int32)      # rows gathered from x[perm_src // 2]
    x = torch.from_numpy(g.standard_normal((T, K)).astype(np.float32)).to(torch.bfloat16)
    wp, ws = _rand_w(E, N, K, seed=K)
    if fp8:
        codes, scales = gen.quantize_mxfp8(x.float())
        a, a_sc = codes.to(DEV), scales.to(DEV)
        a64 = omx.dequant_mxfp8(codes.numpy(), scales.numpy())
    else:
        a, a_sc = x.to(DEV), None
        a64 = omx.bf16_value(x.view(torch.int16).numpy())
    c = mx.grouped_gemm(a, torch.from_numpy(wp).to(DEV), torch.from_numpy(ws).to(DEV),
                        torch.from_numpy(off).to(DEV), a_scales=a_sc,
                        a_gather=torch.from_numpy(perm_src).to(DEV), a_gather_div=div,
                        epilogue=layout, out_dtype="fp32")
    want = _gemm_oracle(a64, perm_src, div, wp, ws, off, layout)
    assert rel_err(c.cpu().numpy(), want) < (1e-4 if fp8 else 1e-5)


@pytest.mark.parametrize("K", [1024, 1536, 4096])
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("layout,out", [("none", "fp32"), ("none", "bf16"), ("split", "bf16")])
def test_gemm_32_and_64_row_classes_agree_bitwise(fp8, layout, out, K):
    """Two experts with the same weights in one call: expert 0 gets 32 rows
    (32-row tile class), expert 1 the same 32 rows plus one (64-row class).
    Both tiles accumulate every output in the same K order, so expert 0's rows
    equal expert 1's first 32 bitwise."""
    g = np.random.default_rng(3 * K + fp8)
    N = 512
    x = torch.from_numpy(g.standard_normal((33, K)).astype(np.float32)).to(torch.bfloat16)
    wp, ws = _rand_w(1, N, K, seed=K + 1)
    wp, ws = np.concatenate([wp, wp]), np.concatenate([ws, ws])
    rows = torch.cat([torch.arange(32), torch.arange(33)]).to(torch.int32)
    if fp8:
        codes, scales = gen.quantize_mxfp8(x.float())
        a, a_sc = codes[rows].to(DEV), scales[rows].to(DEV)
    else:
        a, a_sc = x[rows].to(DEV), None
    w = (torch.from_numpy(wp).to(DEV), torch.from_numpy(ws).to(DEV))
    c = mx.grouped_gemm(a, *w, torch.from_numpy(_offsets([32, 33])).to(DEV), a_scales=a_sc,
                        epilogue=layout, out_dtype=out)
    assert torch.equal(c[:32], c[32:64])


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("layout,out", [("none", "fp32"), ("none", "bf16"), ("split", "bf16"),
                                        ("interleaved", "mxfp8")])
def test_gemm_decode_shaped_call_matches_oracle_and_repeats_bitwise(fp8, layout, out):
    """A call of 32 rows in all (the decode shape: only the 32-row tile class
    runs) over a long K meets the oracle's bound (the MXFP8 output checked
    through its decoded values), and repeated calls are bitwise identical."""
    if out == "mxfp8" and not fp8:
        fp8 = True
    g = np.random.default_rng(41 + fp8)
    K, N, counts = 4096, 512, [1, 0, 24, 7]
    off = _offsets(counts)
    rows = sum(counts)
    x = torch.from_numpy(g.standard_normal((rows, K)).astype(np.float32)).to(torch.bfloat16)
    wp, ws = _rand_w(len(counts), N, K, seed=77)
    if fp8:
        codes, scales = gen.quantize_mxfp8(x.float())
        a, a_sc = codes.to(DEV), scales.to(DEV)
        a64 = omx.dequant_mxfp8(codes.numpy(), scales.numpy())
    else:
        a, a_sc = x.to(DEV), None
        a64 = omx.bf16_value(x.view(torch.int16).numpy())
    args = dict(a_scales=a_sc, epilogue=layout, out_dtype=out)
    w = (torch.from_numpy(wp).to(DEV), torch.from_numpy(ws).to(DEV), torch.from_numpy(off).to(DEV))
    c = mx.grouped_gemm(a, *w, **args)
    again = mx.grouped_gemm(a, *w, **args)
    torch.cuda.synchronize()
    if out == "mxfp8":
        assert torch.equal(c[0], again[0]) and torch.equal(c[1], again[1])
        got = omx.dequant_mxfp8(c[0].cpu().numpy(), c[1].cpu().numpy())
    else:
        assert torch.equal(c, again)
        got = c.float().cpu().numpy()
    want = _gemm_oracle(a64, np.arange(rows, dtype=np.int32), 1, wp, ws, off, layout)
    tol = {"fp32": 1e-4 if fp8 else 1e-5, "bf16": 1e-2, "mxfp8": 5e-2}[out]
    assert rel_err(got, want) < tol


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("layout", ["split", "interleaved"])
def test_gemm_mxfp8_output_encodes_the_fp32_result(fp8, layout):
    """The MXFP8 epilogue encodes the same fp32 SwiGLU values the fp32 epilogue
    writes; the oracle's encoder, given those fp32 values, must produce the same
    codes and scale bytes (the quantisation decided in the same precision)."""
    g = np.random.default_rng(12)
    K, N = 512, 448                                     # N_out = 224: seven blocks per row
    counts = [300, 0, 5, 129]
    off = _offsets(counts)
    rows = int(off[-1])
    x = torch.from_numpy(g.standard_normal((rows, K)).astype(np.float32)).to(torch.bfloat16)
    x[7] = 0                                            # a zero row: all-zero blocks
    wp, ws = _rand_w(len(counts), N, K, seed=5)
    if fp8:
        codes, scales = gen.quantize_mxfp8(x.float())
        a, a_sc = codes.to(DEV), scales.to(DEV)
    else:
        a, a_sc = x.to(DEV), None
    args = (a, torch.from_numpy(wp).to(DEV), torch.from_numpy(ws).to(DEV), torch.from_numpy(off).to(DEV))
    c32 = mx.grouped_gemm(*args, a_scales=a_sc, epilogue=layout, out_dtype="fp32").cpu().numpy()
    c8, s8 = mx.grouped_gemm(*args, a_scales=a_sc, epilogue=layout, out_dtype="mxfp8")
    want_c, want_s = omx.quantize_mxfp8(c32.astype(np.float64))
    np.testing.assert_array_equal(s8.cpu().numpy(), want_s)
    got = c8.cpu().numpy()
    bad = np.argwhere(got != want_c)
    assert bad.size == 0, f"{len(bad)} code mismatches, first {bad[:5].tolist()}"
    assert np.all(want_s[7] == 0) and np.all(got[7] == 0)


def test_gemm_mxfp8_output_needs_swiglu_and_whole_stages():
    E, N, K = 1, 128, 256
    wp, ws = _rand_w(E, N, K, seed=6)
    a = torch.zeros((4, K), dtype=torch.bfloat16, device=DEV)
    args = (a, torch.from_numpy(wp).to(DEV), torch.from_numpy(ws).to(DEV), torch.from_numpy(_offsets([4])).to(DEV))
    for epi in ("none", "split"):                       # no SwiGLU / K % 512 != 0
        with pytest.raises(mx.MoeError) as ei:
            mx.grouped_gemm(*args, epilogue=epi, out_dtype="mxfp8")
        assert ei.value.status == mx.STATUS["MOE_ERR_NOT_IMPLEMENTED"]


def test_gemm_bf16_output_rounding():
    g = np.random.default_rng(8)
    E, N, K = 2, 256, 256
    off = _offsets([100, 28])
    a = torch.from_numpy(g.standard_normal((128, K)).astype(np.float32)).to(torch.bfloat16)
    wp, ws = _rand_w(E, N, K, seed=4)
    args = (a.to(DEV), torch.from_numpy(wp).to(DEV), torch.from_numpy(ws).to(DEV), torch.from_numpy(off).to(DEV))
    c32 = mx.grouped_gemm(*args, out_dtype="fp32")
    c16 = mx.grouped_gemm(*args, out_dtype="bf16")
    assert torch.equal(c32.to(torch.bfloat16), c16)


# ------------------------------------------------------------ combine

@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16])
def test_combine_against_oracle(ydt):
    g = np.random.default_rng(9)
    T, k, H = 77, 5, 264
    dest = g.permutation(T * k).astype(np.int32)
    w = g.random((T, k)).astype(np.float32)
    y = torch.from_numpy(g.standard_normal((T * k, H)).astype(np.float32)).to(ydt)
    out, xn = mx.combine(y.to(DEV), torch.from_numpy(dest).to(DEV), torch.from_numpy(w).to(DEV), rms_next=True)
    want = omoe.combine(y.double().numpy(), dest, w.astype(np.float64))
    assert rel_err(out.cpu().numpy(), want) < 1e-6
    ref_next = omoe.rms_rescale(want)
    got_next = xn.float().cpu().numpy()
    assert np.all(np.abs(got_next - ref_next) <= 2.0 ** -7 * np.abs(ref_next) + 1e-30)


def test_combine_one_hot_is_a_bitwise_gather():
    g = np.random.default_rng(10)
    T, k, H = 40, 3, 128
    dest = g.permutation(T * k).astype(np.int32)
    w = np.zeros((T, k), dtype=np.float32)
    w[:, 2] = 1.0
    y = torch.from_numpy(g.standard_normal((T * k, H)).astype(np.float32))
    out = mx.combine(y.to(DEV), torch.from_numpy(dest).to(DEV), torch.from_numpy(w).to(DEV))
    assert torch.equal(out.cpu(), y[dest.reshape(T, k)[:, 2]])
