"""The seeded input generator: determinism, exactness of the int64 hash, value laws."""
import numpy as np
import torch

from workloads import gen


def test_fmix32_int64_matches_exact_32bit_arithmetic():
    g = np.random.default_rng(0)
    vals = [int(v) for v in g.integers(0, 2 ** 32, 2000, dtype=np.uint64)] + [0, 1, 2 ** 32 - 1, 2 ** 31]
    got = gen.fmix32(torch.tensor(vals, dtype=torch.int64)).tolist()
    assert got == [gen._fmix32_int(v) for v in vals]


def test_counter_words_are_deterministic_and_sliceable():
    k = gen.stream_key(0, 1, gen.T_W1, 3)
    a = gen.counter_words(k, 0, 1000, "cpu")
    b = gen.counter_words(k, 400, 100, "cpu")
    assert torch.equal(a[400:500], b)
    assert int(a.min()) >= 0 and int(a.max()) < 2 ** 32
    assert not torch.equal(a, gen.counter_words(gen.stream_key(0, 1, gen.T_W1, 4), 0, 1000, "cpu"))


def test_weight_laws():
    s = gen.LayerShape(T=4, H=256, I=128, E=2, k=1)
    w1p, w1s, w2p, w2s = gen.expert_weights(s, 1)
    assert w1p.shape == (256, 128) and w1s.shape == (256, 8)
    assert w2p.shape == (256, 64) and w2s.shape == (256, 4)
    for sc in (w1s, w2s):
        assert int(sc.min()) == 121 and int(sc.max()) == 127
    nib = torch.cat([(w1p & 15).flatten(), (w1p >> 4).flatten()]).long()
    counts = torch.bincount(nib, minlength=16).double()
    assert counts.min() > 0.85 * counts.mean() and counts.max() < 1.15 * counts.mean()


def test_biases():
    hot = gen.expert_bias(gen.preset("decode"))
    assert (hot == 2.0).sum() == 18 and set(np.unique(hot)) == {0.0, 2.0}
    z = gen.expert_bias(gen.preset("prefill896_mxfp8"))
    assert z.max() == 0.0 and np.isclose(z.min(), -1.1 * np.log(896), rtol=1e-6)
    assert len(np.unique(z)) == 896


def test_inputs_are_seeded():
    s = gen.preset("tiny")
    a, b = gen.layer_inputs(s), gen.layer_inputs(s)
    assert torch.equal(a.x_bf16, b.x_bf16) and np.array_equal(a.logits, b.logits)
    assert a.x_bf16.shape == (32, 128) and a.logits.shape == (32, 4)
    assert abs(float(a.x_bf16.float().std()) - 1.0) < 0.1


def test_batched_weight_generation_matches_per_expert():
    s = gen.LayerShape(T=4, H=256, I=96, E=11, k=2, cfg_id=78)
    a = gen.all_expert_weights(s, layer=3, chunk=4)
    for e in range(s.E):
        b = gen.expert_weights(s, e, 3)
        assert all(torch.equal(x[e], y) for x, y in zip(a, b)), e
