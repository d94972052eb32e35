"""The allocation-free entry point (fs_sample_fused_noalloc: the fused call
with the library's static per-GPU scratch array in place of a workspace)
through the C ABI, against fs_sample_fused_ex with a caller workspace: the
same tokens on two calls in a row, the second with a smaller input, for
two-stage, single-pass (whose keys the entry point zeroes itself, after a
two-stage call has left the array dirty) and grouped sampling; sizes past the
array are refused before anything is enqueued."""
import numpy as np
import pytest

from lm_head_gemm_amd import inputs
from tests._util import check_parity, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fs():
    import torch
    assert torch.cuda.is_available()
    from lm_head_gemm_amd import flashsample
    return flashsample


def _head(seed, B, D, V, dtype="bf16"):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((B, D), dtype=np.float32)
    w = rng.standard_normal((V, D), dtype=np.float32) * np.float32(0.05)
    if dtype == "bf16":
        return inputs.f32_to_bf16_bits(h), inputs.f32_to_bf16_bits(w)
    return h, w


def _pair(fs, H, W, tiled, T, seed, step, **kw):
    import torch
    Hd, Wd = to_device(H), to_device(W)
    Wx = fs.TiledWeights(Wd) if tiled else Wd
    want = fs.sample_fused(Hd, Wx, T, seed, step, **kw).cpu().numpy()
    out = torch.full((H.shape[0],), -7, dtype=torch.int32, device="cuda")
    got = fs.sample_fused_noalloc(Hd, Wx, T, seed, step, out=out, **kw)
    assert got is out
    return want, out.cpu().numpy()


@pytest.mark.parametrize("kw", [{}, {"single_pass": True}, {"group_size": 512}])
def test_noalloc_equals_workspace_call_twice_then_smaller(fs, kw):
    # a large call first (fills much of the scratch array), then a smaller one
    H1, W1 = _head(1, 300, 1024, 20011)
    H2, W2 = _head(2, 17, 512, 3001)
    for H, W, tiled, T, seed, step in ((H1, W1, True, 1.0, 3, 5), (H2, W2, False, 0.7, 9, 2**32 + 1)):
        if kw.get("group_size") and not tiled and W.shape[1] % 256:
            continue
        want, got = _pair(fs, H, W, tiled, T, seed, step, **kw)
        assert np.array_equal(got, want)
        if not kw.get("group_size"):
            check_parity(H, W, T, seed, step, np.arange(H.shape[0]), got)


@pytest.mark.parametrize("single_pass", [False, True])
def test_noalloc_split_last_round(fs, single_pass):
    """A vocabulary whose nearly empty last round of 128-row tiles runs as
    64-row tiles (more candidate slots in the scratch array): the same tokens
    as the call with a workspace."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    H, W = _head(6, 64, 256, (2 * cus + cus // 5) * 128 + 9)
    for step in range(2):
        want, got = _pair(fs, H, W, True, 1.0, 4, step, single_pass=single_pass)
        assert np.array_equal(got, want)


def test_noalloc_single_pass_after_a_dirty_two_stage_call(fs):
    H, W = _head(3, 40, 512, 5003)
    Hd, Wd = to_device(H), to_device(W)
    big, _ = _head(4, 200, 512, 5003)
    fs.sample_fused_noalloc(to_device(big), Wd, 1.0, 1, 1)      # leaves candidate keys in the array
    for step in range(3):
        want = fs.sample_fused(Hd, Wd, 1.0, 7, step).cpu().numpy()
        got = fs.sample_fused_noalloc(Hd, Wd, 1.0, 7, step, single_pass=True).cpu().numpy()
        assert np.array_equal(got, want)


def test_noalloc_fp32_and_greedy(fs):
    H, W = _head(5, 9, 256, 4099, "f32")
    for T in (1.0, 0.0):
        want, got = _pair(fs, H, W, False, T, 2, 3)
        assert np.array_equal(got, want)


def test_noalloc_refuses_sizes_past_the_scratch_array(fs):
    import torch
    B, D, V = 4096, 256, 128256
    need = fs.workspace_bytes(B, D, V, tiled=False)
    assert need > fs.NOALLOC_SCRATCH_BYTES
    H = torch.zeros((B, D), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((V, D), dtype=torch.bfloat16, device="cuda")
    out = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(fs.FlashSampleError, match="FS_ERR_WORKSPACE_TOO_SMALL"):
        fs.sample_fused_noalloc(H, W, 1.0, 0, 0, out=out)
    torch.cuda.synchronize()
    assert int((out != -7).sum()) == 0   # nothing was enqueued
