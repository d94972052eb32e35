"""Pins for the oracle sampler against what the pages and the mathematics fix.

FlashSampling (arXiv 2603.15854), Section 3: Gumbel-max sampling
(s = l~ + g, sample = argmax s), its exactness under vocab tiling (argmax
decomposes over a partition), and the chi-square check of sampling
correctness in the evaluation (the pages use V = 512 and 10^4 samples; here
V = 64 and 10^6 draws).
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

import oracle
from lm_head_gemm_amd import inputs

EULER_GAMMA = 0.57721566490153286061


def _bf16(x):
    return inputs.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------- logits

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_logits_equal_exact_rational_dot(dtype):
    rng = np.random.default_rng(5)
    B, D, V = 3, 40, 17
    h = rng.standard_normal((B, D)).astype(np.float32)
    w = (rng.standard_normal((V, D)) * 0.05).astype(np.float32)
    if dtype == "bf16":
        h, w = _bf16(h), _bf16(w)
        hv, wv = inputs.bf16_bits_to_f32(h), inputs.bf16_bits_to_f32(w)
    else:
        hv, wv = h, w
    got = oracle.exact_logits(h, w)
    for b in range(B):
        for v in range(V):
            exact = sum(Fraction(float(hv[b, d])) * Fraction(float(wv[v, d])) for d in range(D))
            assert abs(got[b, v] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def test_logits_use_rows_of_w_not_columns():
    """A transposed operand would pair H with columns of W; a non-square W catches it."""
    h = np.array([[1.0, 0.0, 0.0]], dtype=np.float32)
    w = np.array([[2.0, 3.0, 5.0], [7.0, 11.0, 13.0]], dtype=np.float32)
    assert np.array_equal(oracle.exact_logits(h, w), [[2.0, 7.0]])


# ---------------------------------------------------------------- argmax / ties

def test_argmax_lowest_ties_and_nan():
    s = np.array([
        [1.0, 3.0, 3.0, 2.0],
        [np.nan, 5.0, np.nan, 5.0],
        [np.nan, np.nan, np.nan, np.nan],
        [-np.inf, -np.inf, np.nan, -np.inf],
        [np.inf, 1.0, np.inf, np.nan],
    ])
    assert oracle.argmax_lowest(s).tolist() == [1, 1, -1, 0, 0]
    assert oracle.argmax_lowest(s, offset=10).tolist() == [11, 11, -1, 10, 10]


def test_greedy_ties_go_to_lowest_index():
    rng = np.random.default_rng(2)
    D, V = 32, 300
    w = _bf16(rng.standard_normal((V, D)) * 0.05)
    w[250] = w[40]  # duplicate rows give exactly equal logits
    w[41] = w[40]
    h = _bf16(rng.standard_normal((1, D)))
    l = oracle.exact_logits(h, w)[0]
    # make row 40 the maximum by construction: align it with h
    w[40] = w[41] = w[250] = _bf16(inputs.bf16_bits_to_f32(h[0]) * 0.5)
    res = oracle.sample(h, w, 0.0, 0, 0, vocab_chunk=64)
    assert res.idx[0] == 40 and res.second_idx[0] == 41 and res.margin[0] == 0.0
    del l


# ---------------------------------------------------------------- partition invariance

def _head(seed, B, D, V, sigma=0.05):
    rng = np.random.default_rng(seed)
    h = _bf16(rng.standard_normal((B, D)))
    w = _bf16(rng.standard_normal((V, D)) * sigma)
    return h, w


@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
def test_partition_invariance(T):
    """argmax decomposes over any vocab partition: the two-stage tiled result
    equals the direct one for every tile size and for random ragged tilings."""
    B, D, V = 6, 48, 1000
    h, w = _head(11, B, D, V)
    direct = oracle.sample(h, w, T, 1, 3, vocab_chunk=128).idx
    for tile in (1, 3, 64, 256, 1000, V):
        bounds = list(range(0, V, tile)) + [V]
        assert np.array_equal(oracle.sample_two_stage(h, w, T, 1, 3, bounds), direct)
    rng = np.random.default_rng(0)
    for _ in range(5):
        cuts = np.sort(rng.choice(np.arange(1, V), size=rng.integers(1, 40), replace=False))
        bounds = [0] + cuts.tolist() + [V]
        assert np.array_equal(oracle.sample_two_stage(h, w, T, 1, 3, bounds), direct)
    # the chunking inside sample() is not allowed to matter either
    for chunk in (1, 7, 999, 4096):
        assert np.array_equal(oracle.sample(h, w, T, 1, 3, vocab_chunk=chunk).idx, direct)


def test_partition_invariance_with_exact_ties():
    B, D, V = 2, 16, 200
    h, w = _head(3, B, D, V)
    for dup in (17, 63, 64, 150, 199):
        w[dup] = w[5]
    direct = oracle.sample(h, w, 0.0, 0, 0, vocab_chunk=50).idx
    for tile in (1, 3, 64, 100):
        bounds = list(range(0, V, tile)) + [V]
        assert np.array_equal(oracle.sample_two_stage(h, w, 0.0, 0, 0, bounds), direct)


def test_top2_against_brute_force():
    B, D, V = 5, 24, 333
    h, w = _head(4, B, D, V)
    res = oracle.sample(h, w, 0.8, 9, 2, vocab_chunk=40)
    s = oracle.perturbed_scores(h, w, 0.8, 9, 2)
    for b in range(B):
        order = sorted(range(V), key=lambda v: (-s[b, v], v))
        assert res.idx[b] == order[0] and res.second_idx[b] == order[1]
        assert res.best[b] == s[b, order[0]] and res.second[b] == s[b, order[1]]


def test_rows_subset_and_batch_prefix():
    """Noise is keyed by the row index, so selecting rows or truncating the
    batch never changes a row's sample."""
    B, D, V = 8, 32, 500
    h, w = _head(6, B, D, V)
    full = oracle.sample(h, w, 1.0, 5, 1).idx
    assert np.array_equal(oracle.sample(h, w, 1.0, 5, 1, rows=[2, 7, 0]).idx, full[[2, 7, 0]])
    assert np.array_equal(oracle.sample(h[:3], w, 1.0, 5, 1).idx, full[:3])


# ---------------------------------------------------------------- T -> 0

def test_temperature_to_zero_is_argmax():
    """g lies in [-3.13, 22.874] on the lattice, so when the top-2 logit gap
    exceeds 26.004 T the Gumbel-max sample must be the plain argmax."""
    B, D, V = 16, 64, 2000
    h, w = _head(8, B, D, V, sigma=0.2)
    l = oracle.exact_logits(h, w)
    srt = np.sort(l, axis=1)
    gap = srt[:, -1] - srt[:, -2]
    T = float(gap.min()) / 26.01
    res = oracle.sample(h, w, T, 0, 0)
    assert np.array_equal(res.idx, np.argmax(l, axis=1))
    assert np.array_equal(oracle.sample(h, w, 0.0, 0, 0).idx, np.argmax(l, axis=1))
    # and at a moderate temperature the samples do differ from the argmax on some rows
    assert not np.array_equal(oracle.sample(h, w, 1.0, 0, 0).idx, np.argmax(l, axis=1))


# ---------------------------------------------------------------- distribution

@pytest.fixture(scope="module")
def chi2_draws():
    """10^6 draws: 1000 identical rows x 1000 steps of a V = 64 head."""
    h, w = inputs.chi2_inputs(0)
    H = np.repeat(h[None, :], 1000, axis=0)
    idx = np.empty((1000, 1000), dtype=np.int64)
    best = np.empty((1000, 1000))
    for step in range(1000):
        r = oracle.sample(H, w, 1.0, 0, step)
        idx[step] = r.idx
        best[step] = r.best
    l = oracle.exact_logits(h, w)[0]
    return l, idx.ravel(), best.ravel()


@pytest.mark.slow
def test_chi_square_matches_softmax(chi2_draws):
    l, idx, _ = chi2_draws
    p = np.exp(l - l.max())
    p /= p.sum()
    counts = np.bincount(idx, minlength=64)
    assert counts.sum() == 10**6
    res = stats.chisquare(counts, p * 10**6)
    assert res.pvalue > 1e-3, res


@pytest.mark.slow
def test_max_statistic_is_gumbel_of_logsumexp(chi2_draws):
    """max_v (l_v + g_v) ~ Gumbel(logsumexp(l)): mean lse + gamma, sd pi/sqrt(6)."""
    l, _, best = chi2_draws
    lse = np.log(np.exp(l - l.max()).sum()) + l.max()
    sd = np.pi / np.sqrt(6.0)
    assert abs(best.mean() - (lse + EULER_GAMMA)) < 4 * sd / np.sqrt(best.size)
    assert abs(best.std() - sd) < 0.01


def test_chi_square_rejects_temperature_outside_the_noise():
    """Dividing the perturbed score by T, (l + g) / T, leaves the argmax
    unchanged and samples softmax(l) instead of softmax(l / T); the chi-square
    pin must reject it. Planted in a local copy of the oracle's score rule."""
    h, w = inputs.chi2_inputs(0)
    T = 0.5
    H = np.repeat(h[None, :], 1000, axis=0)
    l = oracle.exact_logits(H[:1], w)[0]
    good, bad = [], []
    for step in range(100):
        g = oracle.gumbel_noise(0, step, np.arange(1000), 0, 64)
        good.append(oracle.argmax_lowest(l[None, :] / T + g))
        bad.append(oracle.argmax_lowest((l[None, :] + g) / T))
    p = np.exp((l - l.max()) / T)
    p /= p.sum()
    n = 100 * 1000
    pg = stats.chisquare(np.bincount(np.concatenate(good), minlength=64), p * n).pvalue
    pb = stats.chisquare(np.bincount(np.concatenate(bad), minlength=64), p * n).pvalue
    assert pg > 1e-3 and pb < 1e-6


def test_oracle_noise_depends_on_seed_step_row():
    a = oracle.gumbel_noise(0, 0, [0, 1], 0, 64)
    assert not np.array_equal(a[0], a[1])
    assert not np.array_equal(a, oracle.gumbel_noise(1, 0, [0, 1], 0, 64))
    assert not np.array_equal(a, oracle.gumbel_noise(0, 1, [0, 1], 0, 64))
    assert not np.array_equal(a, oracle.gumbel_noise(0, 2**32, [0, 1], 0, 64))
    assert np.array_equal(a, oracle.gumbel_noise(0, 0, [0, 1], 0, 64))
