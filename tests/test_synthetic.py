"""The seeded input generators shared by the GPU path, the oracle tests and
the bench: the token laws the workloads name and the storage rounding.

* bf16 storage: round to nearest, ties to even, bit for bit as torch's own
  float32 -> bfloat16 conversion (random values, exact ties on both parities,
  subnormals, signed zeros), and an exact widening back.
* Zipf(1.1) over 65,536 ids (the d12 / d20 / d24 token law): the law's own
  figures (normaliser sum_k k^-1.1 = 7.2857, P(id 0) = 0.1373, the ten and
  256 most frequent ids carrying 36.8 % and 66.5 % of the mass), and the d20
  batch's draw against them: hits on the most frequent ids within 5 sigma of
  the binomial mean, the count of distinct ids within 1 % of its expectation.
* next-token targets: targets[:, t] = idx[:, t + 1] from one [B, T + 1] draw.
* weights: N(0, 0.02) draws, the residual scalars around their initial values.
"""
import numpy as np
import torch

from decoder_only_transformer_gpt_amd import synthetic


def torch_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_bit_for_bit():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32) * np.float32(0.02),
        rng.standard_normal(10_000).astype(np.float32) * np.float32(1e4),
        # exact ties: low 16 bits 0x8000 above an even and an odd bf16 mantissa
        (np.arange(0x3F80, 0x3F80 + 512, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        (np.arange(0xBF00, 0xBF00 + 512, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        # just below and just above a tie
        (np.arange(0x4000, 0x4000 + 256, dtype=np.uint32) << 16 | 0x7FFF).view(np.float32),
        (np.arange(0x4000, 0x4000 + 256, dtype=np.uint32) << 16 | 0x8001).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.0e38], dtype=np.float32),
    ])
    bits = synthetic.f32_to_bf16_bits(x)
    assert np.array_equal(bits, torch_bf16_bits(x))
    back = synthetic.bf16_bits_to_f32(bits)
    assert np.array_equal(synthetic.f32_to_bf16_bits(back), bits)          # widening is exact
    assert np.array_equal(back, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy())


def zipf_law(V=65536, s=1.1):
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    return w.sum(), w / w.sum()


def test_zipf_law_figures():
    H, p = zipf_law()
    assert round(H, 4) == 7.2857
    assert round(p[0], 4) == 0.1373
    assert round(p[:10].sum(), 3) == 0.368
    assert round(p[:256].sum(), 3) == 0.665


def test_zipf_tokens_of_the_d20_batch_follow_the_law():
    B, T, V = 32, 2048, 65536
    idx, tgt = synthetic.make_tokens(B, T, V, "zipf", seed=1)
    assert idx.dtype == np.int32 and idx.shape == (B, T) and tgt.shape == (B, T)
    assert idx.min() >= 0 and idx.max() < V
    N = idx.size
    _, p = zipf_law(V)
    counts = np.bincount(idx.reshape(-1), minlength=V)
    for i in range(16):
        mean, sd = N * p[i], np.sqrt(N * p[i] * (1 - p[i]))
        assert abs(counts[i] - mean) <= 5 * sd, (i, counts[i], mean)
    distinct = np.count_nonzero(counts)
    expected = np.sum(1.0 - (1.0 - p) ** N)
    assert abs(distinct - expected) <= 0.01 * expected, (distinct, expected)


def test_targets_are_the_next_tokens():
    for law in ("uniform", "zipf"):
        idx, tgt = synthetic.make_tokens(4, 100, 512, law, seed=3)
        assert np.array_equal(idx[:, 1:], tgt[:, :-1])
        assert idx.min() >= 0 and max(idx.max(), tgt.max()) < 512
    u, _ = synthetic.make_tokens(8, 4096, 512, "uniform", seed=4)
    c = np.bincount(u.reshape(-1), minlength=512)
    assert c.min() > 0 and abs(c.mean() - 64) < 1e-9 and c.max() < 64 + 6 * 8


def test_weights_follow_the_recipe():
    shapes = [("wte", 512, 128), ("h0.w_qkv", 384, 128), ("lm_head", 512, 128),
              ("resid_lambdas", 1, 64), ("x0_lambdas", 1, 64), ("ve_gates", 1, 64)]
    storage, values = synthetic.make_weights(shapes, seed=0, dtype="bf16")
    assert storage.dtype == np.uint16 and np.array_equal(synthetic.bf16_bits_to_f32(storage), values)
    off, got = 0, {}
    for name, r, c in shapes:
        got[name] = values[off:off + r * c]
        off += r * c
    for name in ("wte", "h0.w_qkv", "lm_head"):
        assert abs(got[name].std() - 0.02) < 0.02 * 0.02 and abs(got[name].mean()) < 0.02 * 0.02
    for name, init in (("resid_lambdas", 1.0), ("x0_lambdas", 0.1), ("ve_gates", 1.0)):
        assert abs(got[name].mean() - init) < 0.05 and 0.05 < got[name].std() < 0.15
    f32, f32v = synthetic.make_weights(shapes, seed=0, dtype="f32")
    assert f32.dtype == np.float32 and np.array_equal(synthetic.f32_to_bf16_bits(f32v), storage)
