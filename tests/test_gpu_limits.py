"""Edge sizes through the C ABI against the oracle: the largest hidden size a
GEMV kernel can stage (one H row filling the 160 KB LDS), the largest batch
the ABI accepts, and a vocabulary of two million rows (16K vocab tiles, the
large-grid Stage 2). FlashSampling, arXiv 2603.15854, Section 3.
"""
import numpy as np
import pytest

import oracle
from lm_head_gemm_amd import inputs
from tests._util import check_parity, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fs():
    import torch
    assert torch.cuda.is_available()
    from lm_head_gemm_amd import flashsample
    return flashsample


def _rand_head(seed, B, D, V, dtype="bf16", sigma=0.05):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((B, D), dtype=np.float32)
    w = rng.standard_normal((V, D), dtype=np.float32) * np.float32(sigma / np.sqrt(D / 256))
    if dtype == "bf16":
        return inputs.f32_to_bf16_bits(h), inputs.f32_to_bf16_bits(w)
    return h, w


@pytest.mark.parametrize("dtype,D,B", [("f32", 40704, 3), ("bf16", 81408, 2), ("bf16", 81408, 9)])
def test_largest_hidden_size(fs, dtype, D, B):
    """D * element size = 159 KiB, the largest accepted: the whole H row fills
    the LDS of the GEMV kernels (bf16 B <= 2 and every fp32 batch) beside their
    reduction arrays; the MFMA kernels (bf16 B = 9) stage H in chunks.
    Row-major and tiled W."""
    V = 700
    H, W = _rand_head(D + B, B, D, V, dtype)
    Hd, Wd = to_device(H), to_device(W)
    heads = [Wd] + ([fs.TiledWeights(Wd)] if dtype == "bf16" else [])
    for Wx in heads:
        for T, seed, step in ((1.0, 1, 2), (0.0, 0, 0)):
            tok = fs.sample_fused(Hd, Wx, T, seed, step).cpu().numpy()
            check_parity(H, W, T, seed, step, np.arange(B), tok)


def test_hidden_size_past_the_lds_is_rejected(fs):
    import torch
    from lm_head_gemm_amd.flashsample import FlashSampleError
    H = torch.zeros((1, 40708), dtype=torch.float32, device="cuda")
    W = torch.zeros((10, 40708), dtype=torch.float32, device="cuda")
    with pytest.raises(FlashSampleError):
        fs.sample_fused(H, W, 1.0, 0, 0)


def test_largest_batch(fs):
    """B = 65536, the ABI's maximum: 512 batch tiles of the wide kernel, 1024
    of the row-major MFMA kernel; two-stage and single-pass agree."""
    B, D, V = 65536, 64, 300
    H, W = _rand_head(4, B, D, V)
    Hd, Wd = to_device(H), to_device(W)
    tw = fs.TiledWeights(Wd)
    rows = np.unique(np.concatenate([[0, 1, B - 1], np.random.default_rng(0).choice(B, 40, replace=False)]))
    ref = oracle.sample(H, W, 0.9, 6, 1, rows=rows)
    for Wx in (Wd, tw):
        two = fs.sample_fused(Hd, Wx, 0.9, 6, 1).cpu().numpy()
        one = fs.sample_fused(Hd, Wx, 0.9, 6, 1, single_pass=True).cpu().numpy()
        assert np.array_equal(one, two)
        assert two.min() >= 0 and two.max() < V
        check_parity(H, W, 0.9, 6, 1, rows, two[rows], ref=ref)


def test_two_million_vocab_rows(fs):
    """V = 2^21 + 3: 16385 vocab tiles of 128 rows (Stage 2 over the large
    candidate buffer), ragged last tile; GEMV and MFMA, both layouts."""
    D, V = 64, (1 << 21) + 3
    H, W = _rand_head(8, 5, D, V)
    Hd, Wd = to_device(H), to_device(W)
    tw = fs.TiledWeights(Wd)
    ref = oracle.sample(H, W, 1.0, 3, 4, vocab_chunk=1 << 18)
    for B in (2, 5):
        for Wx in (Wd, tw):
            tok = fs.sample_fused(Hd[:B], Wx, 1.0, 3, 4).cpu().numpy()
            sub = oracle.SampleResult(ref.idx[:B], ref.best[:B], ref.second[:B], ref.second_idx[:B])
            check_parity(H, W, 1.0, 3, 4, np.arange(B), tok, ref=sub)


def test_launch_beyond_dispatch_limit_is_refused(fs):
    """65536 rows over an 8M-row vocabulary need more work-items in one launch
    dimension than a dispatch can count (2^32): the call fails with FS_ERR_HIP
    (hipErrorInvalidConfiguration) before anything is enqueued, and the output
    is left untouched. (Single-pass, so the workspace stays small.)"""
    import torch
    B, D, V = 65536, 8, 8 << 20
    H = torch.zeros(B, D, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(V, D, dtype=torch.bfloat16, device="cuda")
    out = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(fs.FlashSampleError) as err:
        fs.sample_fused(H, W, 1.0, 0, 0, out=out, single_pass=True)
    assert err.value.status == fs.FS_ERR_HIP
    assert fs._lib.fs_last_hip_error() == 9   # hipErrorInvalidConfiguration
    torch.cuda.synchronize()
    assert int((out != -7).sum()) == 0
