"""The grouped variant on the GPU (local sample + local log-mass per
vocabulary group, then a Gumbel-max draw of the group; FlashSampling, arXiv
2603.15854, Section 3, tensor-parallel paragraphs) against
oracle.sample_grouped, through the C ABI: small shapes over both tiled MFMA
kernels, ragged vocab, several batch tiles and group sizes; the reductions to
the plain sampler; the categorical law by chi-square (full sizes: tests/test_gpu_full_size.py).
"""
import numpy as np
import pytest

import oracle
from lm_head_gemm_amd import inputs
from tests._util import check_grouped_parity, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fs():
    import torch
    assert torch.cuda.is_available()
    from lm_head_gemm_amd import flashsample
    return flashsample


def _rand_head(seed, B, D, V, sigma=0.05):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((B, D), dtype=np.float32)
    w = rng.standard_normal((V, D), dtype=np.float32) * np.float32(sigma)
    return inputs.f32_to_bf16_bits(h), inputs.f32_to_bf16_bits(w)


@pytest.mark.parametrize("tile,G", [(64, 64), (64, 192), (128, 128), (128, 512), (256, 256), (256, 1024)])
@pytest.mark.parametrize("B,D,V", [(1, 64, 1000), (5, 520, 2001), (33, 1032, 4099), (70, 264, 3000),
                                   (150, 512, 2053), (300, 264, 1100)])
def test_grouped_parity(fs, tile, G, B, D, V):
    H, W = _rand_head(B * 13 + D + V + G, B, D, V)
    Hd = to_device(H)
    tw = fs.TiledWeights(to_device(W))
    for T, seed, step in ((1.0, 0, 0), (0.6, 77, 2**32 + 1), (1.3, 2**40 + 3, 5)):
        tok = fs.sample_fused(Hd, tw, T, seed, step, variant="mfma", vocab_tile=tile, group_size=G).cpu().numpy()
        check_grouped_parity(H, W, T, seed, step, G, np.arange(B), tok)


@pytest.mark.parametrize("B", [3, 40, 100])
def test_one_group_and_greedy_equal_the_plain_call(fs, B):
    """A single group (G >= V) leaves the group draw nothing to choose: the
    token is the plain Gumbel-max, bit for bit; T = 0 is the plain greedy."""
    D, V = 256, 3001
    H, W = _rand_head(B + 5, B, D, V)
    Hd = to_device(H)
    tw = fs.TiledWeights(to_device(W))
    for T in (1.0, 0.7):
        plain = fs.sample_fused(Hd, tw, T, 4, 9).cpu().numpy()
        one = fs.sample_fused(Hd, tw, T, 4, 9, group_size=4096).cpu().numpy()
        assert np.array_equal(one, plain)
    plain0 = fs.sample_fused(Hd, tw, 0.0, 4, 9).cpu().numpy()
    assert np.array_equal(fs.sample_fused(Hd, tw, 0.0, 4, 9, group_size=256).cpu().numpy(), plain0)


def test_grouped_with_logits_store(fs):
    import torch
    B, D, V = 20, 264, 1500
    H, W = _rand_head(3, B, D, V)
    Hd = to_device(H)
    tw = fs.TiledWeights(to_device(W))
    l32 = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda")
    tok = fs.sample_fused(Hd, tw, 0.9, 1, 2, group_size=256, logits=l32).cpu().numpy()
    assert np.max(np.abs(l32.cpu().numpy().astype(np.float64) - oracle.exact_logits(H, W))) < 1e-4
    check_grouped_parity(H, W, 0.9, 1, 2, 256, np.arange(B), tok)


def test_grouped_nan_rows(fs):
    B, D, V = 4, 64, 700
    H, W = _rand_head(9, B, D, V)
    H[2, :] = 0x7FC0                  # bf16 NaN: every logit of row 2 is NaN
    W[300, :] = 0x7FC0                # one NaN token in every row
    Hd = to_device(H)
    tw = fs.TiledWeights(to_device(W))
    tok = fs.sample_fused(Hd, tw, 1.0, 0, 0, variant="mfma", vocab_tile=64, group_size=128).cpu().numpy()
    ref = oracle.sample_grouped(H, W, 1.0, 0, 0, 128)
    assert tok[2] == -1 == ref.idx[2]
    assert not np.any(tok == 300)
    rows = np.array([0, 1, 3])
    check_grouped_parity(H, W, 1.0, 0, 0, 128, rows, tok[rows])


def test_grouped_chi_square_on_device(fs):
    """10^6 GPU draws (1000 identical rows x 1000 steps) at V = 256 in four
    groups of 64 follow softmax(l / T)."""
    from scipy import stats
    h, w = inputs.chi2_inputs(2)
    rng = np.random.default_rng(3)
    w = np.concatenate([w, rng.standard_normal((192, 256), dtype=np.float32) * np.float32(0.05)])
    H = inputs.f32_to_bf16_bits(np.repeat(h[None, :], 1000, axis=0))
    W = inputs.f32_to_bf16_bits(w)
    Hd = to_device(H)
    tw = fs.TiledWeights(to_device(W))
    T = 0.8
    counts = np.zeros(256, dtype=np.int64)
    for step in range(1000):
        tok = fs.sample_fused(Hd, tw, T, 11, step, variant="mfma", vocab_tile=64, group_size=64)
        counts += np.bincount(tok.cpu().numpy(), minlength=256)
    l = oracle.exact_logits(H[:1], W)[0]
    p = np.exp((l - l.max()) / T)
    p /= p.sum()
    assert counts.sum() == 10**6
    assert stats.chisquare(counts, p * 10**6).pvalue > 1e-3


@pytest.mark.parametrize("tile,G", [(64, 128), (128, 256), (256, 512)])
@pytest.mark.parametrize("B,D,V", [(3, 256, 1000), (40, 512, 3001), (150, 256, 2053)])
def test_grouped_parity_row_major(fs, tile, G, B, D, V):
    """Row-major W with D a multiple of 256: the MFMA kernels read the rows
    directly and carry the same log-mass epilogue."""
    H, W = _rand_head(B * 17 + D + V + G, B, D, V)
    Hd, Wd = to_device(H), to_device(W)
    for T, seed, step in ((1.0, 2, 0), (0.7, 9, 2**32 + 3)):
        tok = fs.sample_fused(Hd, Wd, T, seed, step, variant="mfma", vocab_tile=tile, group_size=G).cpu().numpy()
        check_grouped_parity(H, W, T, seed, step, G, np.arange(B), tok)
