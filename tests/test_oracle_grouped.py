"""Pins for the grouped oracle (local sample + local log-mass per vocabulary
group, then a Gumbel-max draw of the group) against what the mathematics
fixes: its two reductions to the plain sampler, scipy's logsumexp, the
categorical law by chi-square, and the T -> 0 limit.

FlashSampling (arXiv 2603.15854): the tensor-parallel paragraphs of
Section 3 (local sample and local log-mass per shard) and the abstract
(exactness by hierarchical factorisation of the categorical distribution).
"""
import numpy as np
import pytest
from scipy import special, stats

import oracle
from lm_head_gemm_amd import inputs


def _head(seed, B, D, V, dtype="bf16", sigma=0.05):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((B, D), dtype=np.float32)
    W = rng.standard_normal((V, D), dtype=np.float32) * np.float32(sigma)
    if dtype == "bf16":
        return inputs.f32_to_bf16_bits(H), inputs.f32_to_bf16_bits(W)
    return H, W


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,seed,step", [(1.0, 0, 0), (0.6, 7, 3), (1.7, 2**40 + 5, 2**33 + 1)])
def test_one_group_is_the_plain_sample(dtype, T, seed, step):
    """With a single group the group draw has nothing to choose: the result is
    the local sample over the whole vocabulary, i.e. the plain Gumbel-max."""
    H, W = _head(11, 5, 96, 777, dtype)
    plain = oracle.sample(H, W, T, seed, step).idx
    for G in (777, 780, 4096):
        got = oracle.sample_grouped(H, W, T, seed, step, G)
        assert np.array_equal(got.idx, plain)
        assert np.all(got.group == 0)


@pytest.mark.parametrize("T,seed,step", [(1.0, 3, 0), (0.5, 9, 2**32 + 7)])
def test_groups_of_one_token_are_a_plain_sample_with_the_group_noise(T, seed, step):
    """With one token per group the local sample is the token and its log-mass
    is l_v / T, so the result is argmax_v (l_v / T + h_v): a plain Gumbel-max
    whose noise comes from the group stream. The stream is rebuilt here from
    the scalar Philox (pinned against rocRAND) at counter
    (0xC0000000 | v >> 2, row, step mod 2^32, step >> 32), word v & 3."""
    B, D, V = 3, 64, 53
    H, W = _head(5, B, D, V)
    l = oracle.exact_logits(H, W)
    words = np.empty((B, V), dtype=np.uint64)
    for b in range(B):
        for v in range(V):
            ctr = (0xC0000000 | (v >> 2), b, step & 0xFFFFFFFF, step >> 32)
            words[b, v] = oracle.philox4x32_10_scalar(ctr, (seed & 0xFFFFFFFF, seed >> 32))[v & 3]
    h = oracle.gumbel_from_words(words)
    want = oracle.argmax_lowest(l / T + h)
    got = oracle.sample_grouped(H, W, T, seed, step, 1)
    assert np.array_equal(got.idx, want)
    assert np.array_equal(got.group, want)


def test_group_stream_is_not_the_token_stream():
    g_tok = oracle.philox_words(1, 2, np.arange(4), 0, 64)
    g_grp = oracle.group_philox_words(1, 2, np.arange(4), 0, 64)
    assert not np.any(g_tok == g_grp)


def test_log_mass_matches_scipy_logsumexp():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 37)) * 30
    x[3, 5] = np.nan
    x[4, :] = np.nan
    x[6, :] = -np.inf
    x[7, 2] = -np.inf
    got = oracle.log_mass(x)
    for r in range(x.shape[0]):
        keep = x[r][~np.isnan(x[r])]
        want = special.logsumexp(keep) if keep.size and np.isfinite(keep).any() else -np.inf
        assert got[r] == pytest.approx(want, rel=1e-14, abs=1e-12) if np.isfinite(want) else got[r] == want


def test_log_masses_of_a_partition_combine_to_the_whole():
    """log-mass is additive over a partition in the exp domain, ragged groups included."""
    H, W = _head(8, 4, 48, 301)
    T = 0.7
    lt = oracle.exact_logits(H, W) / T
    res = oracle.sample_grouped(H, W, T, 0, 0, 37)
    whole = special.logsumexp(lt, axis=1)
    assert np.allclose(special.logsumexp(res.mass, axis=1), whole, rtol=0, atol=1e-12)


def test_temperature_zero_is_greedy():
    H, W = _head(4, 6, 64, 500)
    plain = oracle.sample(H, W, 0.0, 0, 0).idx
    for G in (1, 64, 100, 500):
        assert np.array_equal(oracle.sample_grouped(H, W, 0.0, 0, 0, G).idx, plain)


def test_nan_and_negative_infinity():
    H, W = _head(6, 4, 32, 90, "f32")
    H[1, :] = np.nan                  # every logit NaN
    W[40, :] = np.nan                 # one NaN token in every row
    res = oracle.sample_grouped(H, W, 1.0, 2, 3, 16)
    assert res.idx[1] == -1
    assert not np.any(res.idx[[0, 2, 3]] == 40)
    Hn = np.full((1, 32), -np.inf, dtype=np.float32)
    Wp = np.abs(W[:10]) + 1           # all logits -inf: lowest index, as the plain sampler
    assert oracle.sample_grouped(Hn, Wp, 1.0, 0, 0, 3).idx[0] == oracle.sample(Hn, Wp, 1.0, 0, 0).idx[0] == 0


def _grouped_draws(G, T, n_steps, mass_rule=None):
    """n_steps x 1000 draws at V = 64 from identical rows. mass_rule, if given,
    replaces the log-mass (a planted mistake, applied to a local copy of the
    rule, on the CPU only)."""
    h, w = inputs.chi2_inputs(1)
    rows = np.arange(1000)
    H = np.repeat(h[None, :], 1000, axis=0)
    l = oracle.exact_logits(H[:1], w)[0]
    V = 64
    K = (V + G - 1) // G
    bounds = [(k * G, min(V, (k + 1) * G)) for k in range(K)]
    out = []
    for step in range(n_steps):
        if mass_rule is None:
            out.append(oracle.sample_grouped(H, w, T, 0, step, G).idx)
            continue
        s = l[None, :] / T + oracle.gumbel_noise(0, step, rows, 0, V)
        x = np.stack([oracle.argmax_lowest(s[:, a:b], offset=a) for a, b in bounds], axis=1)
        m = np.array([mass_rule(l[a:b] / T) for a, b in bounds])
        t = m[None, :] + oracle.group_noise(0, step, rows, K)
        out.append(x[np.arange(1000), oracle.argmax_lowest(t)])
    return l, np.concatenate(out)


@pytest.mark.parametrize("G", [8, 5, 1])
def test_grouped_chi_square_matches_softmax(G):
    T = 0.8
    l, idx = _grouped_draws(G, T, 1000)
    p = np.exp((l - l.max()) / T)
    p /= p.sum()
    counts = np.bincount(idx, minlength=64)
    assert counts.sum() == 10**6
    assert stats.chisquare(counts, p * 10**6).pvalue > 1e-3


def test_grouped_chi_square_rejects_max_as_group_mass():
    """Drawing the group by its largest logit instead of its log-mass is biased
    towards groups with one dominant token; chi-square must reject it."""
    T = 0.8
    l, good = _grouped_draws(8, T, 300)
    _, bad = _grouped_draws(8, T, 300, mass_rule=np.max)
    p = np.exp((l - l.max()) / T)
    p /= p.sum()
    n = 300 * 1000
    pg = stats.chisquare(np.bincount(good, minlength=64), p * n).pvalue
    pb = stats.chisquare(np.bincount(bad, minlength=64), p * n).pvalue
    assert pg > 1e-3 and pb < 1e-6
