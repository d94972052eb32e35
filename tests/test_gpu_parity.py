"""Parity of the HIP sampler with the CPU oracle (FlashSampling, arXiv
2603.15854, Section 3), through the C ABI.

Small cases span several vocab tiles, ragged tails, several batch tiles and
the degenerate cases (V = 1, greedy ties, NaN rows). The full-size workloads
are checked row by row in tests/test_gpu_full_size.py.
"""
import os

import numpy as np
import pytest

import oracle
from lm_head_gemm_amd import inputs
from tests._util import TOL, check_grouped_parity, check_parity, to_device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def assert_bf16_logits(got16, exact, acc_tol=1e-4):
    """bf16 logits = round-to-nearest of the fp32 accumulators, which lie
    within acc_tol of the exact logits: |got - exact| <= u (|exact| + acc_tol)
    + acc_tol, with u = 2^-8 the unit roundoff of an 8-bit significand."""
    u = 2.0 ** -8
    err = np.abs(got16 - exact)
    bound = u * (np.abs(exact) + acc_tol) + acc_tol
    assert np.all(err <= bound), float(np.max(err - bound))


@pytest.fixture(scope="module")
def fs():
    import torch
    assert torch.cuda.is_available()
    from lm_head_gemm_amd import flashsample
    return flashsample


def _rand_head(seed, B, D, V, dtype="bf16", sigma=0.05):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((B, D), dtype=np.float32)
    w = rng.standard_normal((V, D), dtype=np.float32) * np.float32(sigma)
    if dtype == "bf16":
        return inputs.f32_to_bf16_bits(h), inputs.f32_to_bf16_bits(w)
    return h, w


# ------------------------------------------------------------------ tiny fp32 workload

def test_tiny_f32_64_steps_match_golden(fs):
    wl = inputs.WORKLOADS["tiny_f32"]
    H, W = inputs.make_hidden(wl), inputs.make_weights(wl)
    Hd, Wd = to_device(H), to_device(W)
    want = {}
    with open(os.path.join(GOLDEN, "tiny_f32_tokens.txt")) as f:
        for line in f:
            if not line.startswith("#"):
                p = line.split()
                want[int(p[0])] = (int(p[1]), float(p[3]))
    for tile in (wl.vocab_tile, 0):
        for step in wl.steps:
            tok = int(fs.sample_fused(Hd, Wd, wl.temperature, wl.seed, step, vocab_tile=tile).cpu()[0])
            idx, margin = want[step]
            if margin > TOL:
                assert tok == idx, f"step {step} tile {tile}: {tok} != {idx}"
            else:
                check_parity(H, W, wl.temperature, wl.seed, step, [0], [tok])


# ------------------------------------------------------------------ small shapes

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,D,V", [
    (1, 64, 1), (1, 64, 5), (1, 256, 1000), (2, 200, 4099), (3, 1032, 3000),
    (5, 512, 777), (8, 4096, 2053), (13, 264, 1500),
])
@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
def test_small_shapes(fs, dtype, B, D, V, T):
    H, W = _rand_head(B * 1000 + D + V, B, D, V, dtype)
    Hd, Wd = to_device(H), to_device(W)
    for seed, step in ((0, 0), (12345, 2**32 + 7)):
        tok = fs.sample_fused(Hd, Wd, T, seed, step).cpu().numpy()
        check_parity(H, W, T, seed, step, np.arange(B), tok)


@pytest.mark.parametrize("variant,tile", [("gemv", 16), ("gemv", 48), ("gemv", 64), ("gemv", 256),
                                          ("gemv", 1008), ("gemv", 4096), ("mfma", 64), ("mfma", 128)])
def test_vocab_tile_invariance(fs, variant, tile):
    B, D, V = 6, 512, 5003
    H, W = _rand_head(7, B, D, V)
    Hd, Wd = to_device(H), to_device(W)
    ref = fs.sample_fused(Hd, Wd, 0.9, 3, 11).cpu().numpy()
    got = fs.sample_fused(Hd, Wd, 0.9, 3, 11, variant=variant, vocab_tile=tile).cpu().numpy()
    r = oracle.sample(H, W, 0.9, 3, 11)
    firm = r.margin > TOL
    assert np.array_equal(got[firm], ref[firm])
    check_parity(H, W, 0.9, 3, 11, np.arange(B), got)


@pytest.mark.parametrize("B,D,V", [(3, 4096, 3000), (4, 8192, 1001), (2, 8192, 2053), (4, 7168, 700),
                                   (1, 8192, 257), (9, 3584, 1001), (40, 512, 4099), (64, 768, 130)])
def test_row_major_small_batch_plans(fs, B, D, V):
    """Row-major bf16 W: 256-row GEMV tiles at B <= 2 on heads 8192 wide, the
    row-direct matrix-core kernel (128-row tiles, 256-byte row runs through a
    wave-private LDS transpose, rotated K order) from B = 3 on, with ragged
    last tiles; every row against the oracle, single-pass equal, and the
    tokens equal to the GEMV kernel's on rows the margin decides."""
    H, W = _rand_head(B * 11 + D + V, B, D, V)
    Hd, Wd = to_device(H), to_device(W)
    assert fs.num_vocab_tiles(B, D, V) == -(-V // (256 if B <= 2 else 128))   # bf16
    for T, seed, step in ((1.0, 5, 6), (0.0, 0, 0)):
        tok = fs.sample_fused(Hd, Wd, T, seed, step).cpu().numpy()
        check_parity(H, W, T, seed, step, np.arange(B), tok)
        one = fs.sample_fused(Hd, Wd, T, seed, step, single_pass=True).cpu().numpy()
        assert np.array_equal(tok, one)
        other = fs.sample_fused(Hd, Wd, T, seed, step, variant="gemv" if B > 2 else "mfma").cpu().numpy()
        firm = oracle.sample(H, W, T, seed, step).margin > TOL
        assert np.array_equal(tok[firm], other[firm])


@pytest.mark.parametrize("variant,tile", [("mfma", 64), ("mfma", 128), ("gemv", 64), ("gemv", 1008)])
@pytest.mark.parametrize("B,D,V", [
    (1, 64, 5), (5, 520, 2001), (16, 256, 777), (17, 1032, 3000), (64, 4096, 2053),
    (65, 264, 4099), (130, 512, 1500), (300, 128, 1000),
])
def test_forced_variants(fs, variant, tile, B, D, V):
    """Both Stage-1 kernel families at several tiles, batch tiles, ragged
    vocab and K tails (D not a multiple of the K chunk)."""
    H, W = _rand_head(B * 7 + D + V, B, D, V)
    Hd, Wd = to_device(H), to_device(W)
    for T, seed, step in ((1.0, 0, 0), (0.6, 77, 2**32 + 1), (0.0, 0, 0)):
        tok = fs.sample_fused(Hd, Wd, T, seed, step, variant=variant, vocab_tile=tile).cpu().numpy()
        check_parity(H, W, T, seed, step, np.arange(B), tok)


def test_mfma_store_logits_matches_exact(fs):
    import torch
    B, D, V = 70, 1032, 1001
    H, W = _rand_head(5, B, D, V)
    Hd, Wd = to_device(H), to_device(W)
    exact = oracle.exact_logits(H, W)
    l32 = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda")
    fs.sample_fused(Hd, Wd, 1.0, 0, 0, variant="mfma", logits=l32)
    assert np.max(np.abs(l32.cpu().numpy().astype(np.float64) - exact)) < 1e-4


def _numpy_tiled(W):
    """The tiled layout written out from its definition: block (m, c) of 16
    rows x 256 columns at block index ((m // 8) * nC + c) * 8 + m % 8; inside
    it step t, piece lane = (r, q) = (lane % 16, lane // 16) holds
    W[16m + r, 256c + 32t + 8q : +8]; zero past V (to a whole group of 8
    blocks) and past D."""
    V, D = W.shape
    nM, nC = -(-V // 16), -(-D // 256)
    nG = -(-nM // 8)
    P = np.zeros((nG * 8 * 16, nC * 256), dtype=W.dtype)
    P[:V, :D] = W
    # blocks[m, c, t, lane, 8]
    blocks = np.empty((nG * 8, nC, 8, 64, 8), dtype=W.dtype)
    for lane in range(64):
        r, q = lane % 16, lane // 16
        for t in range(8):
            cols = np.arange(nC)[:, None] * 256 + 32 * t + 8 * q + np.arange(8)[None, :]
            blocks[:, :, t, lane, :] = P.reshape(nG * 8, 16, -1)[:, r, :][:, cols]
    out = blocks.reshape(nG, 8, nC, 8, 64, 8).transpose(0, 2, 1, 3, 4, 5)
    return np.ascontiguousarray(out).reshape(-1)


@pytest.mark.parametrize("V,D", [(1, 8), (17, 264), (1000, 512), (4099, 1032)])
def test_pack_weights_tiled_layout(fs, V, D):
    import torch
    _, W = _rand_head(V + D, 1, D, V)
    tw = fs.TiledWeights(to_device(W))
    got = tw.data.cpu().numpy().view(np.uint16)
    want = _numpy_tiled(W)
    assert got.shape == want.shape and np.array_equal(got, want)


@pytest.mark.parametrize("variant,tile", [("auto", 0), ("gemv", 64), ("gemv", 128), ("mfma", 64), ("mfma", 128),
                                          ("mfma", 256)])
@pytest.mark.parametrize("B,D,V", [
    (1, 64, 5), (2, 520, 2001), (3, 256, 777), (4, 1032, 3000), (16, 256, 4099),
    (33, 4096, 2053), (64, 264, 1500), (100, 512, 1000), (129, 1032, 3001), (260, 264, 4099),
])
def test_tiled_layout_parity(fs, variant, tile, B, D, V):
    H, W = _rand_head(B * 11 + D + V, B, D, V)
    Hd = to_device(H)
    tw = fs.TiledWeights(to_device(W))
    for T, seed, step in ((1.0, 0, 0), (0.6, 77, 2**32 + 1), (0.0, 0, 0)):
        tok = fs.sample_fused(Hd, tw, T, seed, step, variant=variant, vocab_tile=tile).cpu().numpy()
        check_parity(H, W, T, seed, step, np.arange(B), tok)


def test_tiled_unfused_and_store(fs):
    import torch
    B, D, V = 37, 1032, 2001
    H, W = _rand_head(21, B, D, V)
    Hd = to_device(H)
    tw = fs.TiledWeights(to_device(W))
    exact = oracle.exact_logits(H, W)
    l32 = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda")
    tok = fs.sample_fused(Hd, tw, 1.0, 4, 4, logits=l32).cpu().numpy()
    assert np.max(np.abs(l32.cpu().numpy().astype(np.float64) - exact)) < 1e-4
    check_parity(H, W, 1.0, 4, 4, np.arange(B), tok)
    for var in ("gemv", "mfma"):
        tok = fs.sample_unfused(Hd[:3] if var == "gemv" else Hd, tw, 1.0, 4, 4, logits_dtype=torch.float32,
                                variant=var).cpu().numpy()
        rows = np.arange(3 if var == "gemv" else B)
        check_parity(H[rows], W, 1.0, 4, 4, rows, tok)


@pytest.mark.parametrize("B", [150, 300])
def test_tiled_wide_store_and_unfused(fs, B):
    """The 256-row wide kernel (batches above 64) in its store and store-only
    forms: logits exact to fp32 rounding, ragged V and D; two batch tiles
    (W loads non-temporal) and three (cached W loads)."""
    import torch
    D, V = 1032, 2001
    H, W = _rand_head(23, B, D, V)
    Hd = to_device(H)
    tw = fs.TiledWeights(to_device(W))
    assert fs.num_vocab_tiles(B, D, V, tiled=True) == (V + 255) // 256
    exact = oracle.exact_logits(H, W)
    l32 = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda")
    tok = fs.sample_fused(Hd, tw, 1.0, 4, 4, logits=l32).cpu().numpy()
    assert np.max(np.abs(l32.cpu().numpy().astype(np.float64) - exact)) < 1e-4
    check_parity(H, W, 1.0, 4, 4, np.arange(B), tok)
    l16 = torch.zeros((B, V + 5), dtype=torch.bfloat16, device="cuda")
    fs.sample_fused(Hd, tw, 1.0, 4, 4, logits=l16[:, :V])
    got16 = l16[:, :V].float().cpu().numpy().astype(np.float64)
    assert_bf16_logits(got16, exact)
    assert int(l16[:, V:].count_nonzero()) == 0
    for ld in (torch.float32, torch.bfloat16):
        tok = fs.sample_unfused(Hd, tw, 0.8, 6, 1, logits_dtype=ld).cpu().numpy()
        if ld == torch.float32:
            check_parity(H, W, 0.8, 6, 1, np.arange(B), tok)
        else:
            assert tok.min() >= 0 and tok.max() < V


@pytest.mark.parametrize("B,D,V", [(129, 256, 999), (300, 512, 3001), (513, 1280, 2053), (1000, 768, 1234)])
def test_tiled_wide_two_workgroups_per_cu(fs, B, D, V):
    """The wide tile in 128 registers (two or more batch tiles on the tiled
    layout with D a multiple of 256): ragged V and last batch tile, every row
    against the oracle (sampling, another temperature and step, greedy),
    single-pass equal to two-stage, stored logits exact to fp32 rounding, the
    unfused baseline and the grouped variant's log-masses."""
    import torch
    H, W = _rand_head(B + 3 * D + V, B, D, V)
    Hd = to_device(H)
    tw = fs.TiledWeights(to_device(W))
    assert fs.num_vocab_tiles(B, D, V, tiled=True) == (V + 255) // 256
    rows = np.arange(B)
    for T, seed, step in ((1.0, 3, 7), (0.6, 77, 2**32 + 1), (0.0, 0, 0)):
        tok = fs.sample_fused(Hd, tw, T, seed, step).cpu().numpy()
        check_parity(H, W, T, seed, step, rows, tok)
        assert np.array_equal(tok, fs.sample_fused(Hd, tw, T, seed, step, single_pass=True).cpu().numpy())
    exact = oracle.exact_logits(H, W)
    l32 = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda")
    tok = fs.sample_fused(Hd, tw, 1.0, 4, 4, logits=l32).cpu().numpy()
    assert np.max(np.abs(l32.cpu().numpy().astype(np.float64) - exact)) < 1e-4
    check_parity(H, W, 1.0, 4, 4, rows, tok)
    tok = fs.sample_unfused(Hd, tw, 0.8, 6, 1, logits_dtype=torch.float32).cpu().numpy()
    check_parity(H, W, 0.8, 6, 1, rows, tok)
    tok = fs.sample_fused(Hd, tw, 0.9, 1, 2, group_size=512).cpu().numpy()
    check_grouped_parity(H, W, 0.9, 1, 2, 512, rows, tok)


def test_tiled_wide_one_batch_tile_of_256(fs):
    """B = 129 .. 256 on vocabularies whose 256-row tiles fill the last round
    of one-per-CU workgroups completely or to seven eighths (the 256-column
    form of the wide tile): every row against the oracle, greedy, single-pass,
    stored logits, the unfused baseline and the grouped variant."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for B, D, V in [(200, 256, cus * 256 - 7), (256, 512, (cus + 7 * cus // 8) * 256 - 100),
                    (129, 768, (2 * cus) * 256 - 255)]:
        H, W = _rand_head(B + D + V, B, D, V)
        Hd = to_device(H)
        tw = fs.TiledWeights(to_device(W))
        rows = np.arange(B)
        for T, seed, step in ((1.0, 8, 3), (0.0, 0, 0)):
            tok = fs.sample_fused(Hd, tw, T, seed, step).cpu().numpy()
            check_parity(H, W, T, seed, step, rows, tok)
            assert np.array_equal(tok, fs.sample_fused(Hd, tw, T, seed, step, single_pass=True).cpu().numpy())
        l32 = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda")
        tok = fs.sample_fused(Hd, tw, 1.0, 4, 4, logits=l32).cpu().numpy()
        assert np.max(np.abs(l32.cpu().numpy().astype(np.float64) - oracle.exact_logits(H, W))) < 1e-4
        check_parity(H, W, 1.0, 4, 4, rows, tok)
        del l32
        tok = fs.sample_unfused(Hd, tw, 0.8, 6, 1, logits_dtype=torch.float32).cpu().numpy()
        check_parity(H, W, 0.8, 6, 1, rows, tok)
        tok = fs.sample_fused(Hd, tw, 0.9, 1, 2, group_size=4096).cpu().numpy()
        check_grouped_parity(H, W, 0.9, 1, 2, 4096, rows, tok)


def test_tiled_ragged_last_round_split(fs):
    """B = 17 .. 64 on vocabularies whose 128-row tiles leave the last round
    of two-per-CU workgroups at most a quarter full (those tiles then run as
    two 64-row tiles each, the plan counting them): one split tile, a last
    64-row tile with no vocab row, a ragged D, 1 to 5 K blocks (each way
    the loop that keeps W two blocks ahead can end). Every row against the
    oracle, greedy, single-pass, the grouped variant and stored logits
    (paths without the 64-row tiles)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for B, D, V in [(64, 256, (2 * cus + cus // 3) * 128 + 5), (40, 512, (4 * cus + 1) * 128),
                    (24, 264, (2 * cus + cus // 2) * 128 - 3), (17, 1024, (2 * cus + cus // 8) * 128 + 70),
                    (33, 768, (2 * cus + cus // 6) * 128 + 17), (48, 1280, (2 * cus + cus // 7) * 128)]:
        assert fs.num_vocab_tiles(B, D, V, tiled=True) > -(-V // 128)   # 64-row tiles planned
        H, W = _rand_head(B + D + V, B, D, V)
        Hd = to_device(H)
        tw = fs.TiledWeights(to_device(W))
        rows = np.arange(B)
        for T, seed, step in ((1.0, 5, 2), (0.0, 0, 0)):
            tok = fs.sample_fused(Hd, tw, T, seed, step).cpu().numpy()
            check_parity(H, W, T, seed, step, rows, tok)
            for _ in range(2):   # the second call finds the single-pass counters returned to zero
                assert np.array_equal(tok, fs.sample_fused(Hd, tw, T, seed, step, single_pass=True).cpu().numpy())
        tok = fs.sample_fused(Hd, tw, 0.9, 1, 2, group_size=4096).cpu().numpy()
        check_grouped_parity(H, W, 0.9, 1, 2, 4096, rows, tok)
        l16 = torch.empty((B, V), dtype=torch.bfloat16, device="cuda")
        tok = fs.sample_fused(Hd, tw, 1.0, 5, 2, logits=l16).cpu().numpy()
        check_parity(H, W, 1.0, 5, 2, rows, tok)
        assert_bf16_logits(l16.float().cpu().numpy().astype(np.float64), oracle.exact_logits(H, W))
        del l16


def test_wide_tile_huge_h_stride(fs):
    """H rows 2^22 + 256 elements apart (past the 32-bit offsets of the
    two-workgroup wide tile, which then hands the call to the one-workgroup
    wide kernel): every row against the oracle, the same tokens as with a
    contiguous H."""
    import torch
    B, D, V = 130, 256, 999
    H, W = _rand_head(77, B, D, V)
    big = torch.zeros((B, (1 << 22) + 256), dtype=torch.bfloat16, device="cuda")
    big[:, 128:128 + D] = to_device(H)
    Hs = big[:, 128:128 + D]
    assert Hs.stride(0) == (1 << 22) + 256
    tw = fs.TiledWeights(to_device(W))
    tok = fs.sample_fused(Hs, tw, 1.0, 5, 6).cpu().numpy()
    check_parity(H, W, 1.0, 5, 6, np.arange(B), tok)
    assert np.array_equal(tok, fs.sample_fused(to_device(H), tw, 1.0, 5, 6).cpu().numpy())
    del big


@pytest.mark.parametrize("layout,variant,dtype", [
    ("rows", "gemv", "bf16"), ("rows", "mfma", "bf16"), ("rows", "gemv", "f32"), ("rows", "mfma", "f32"),
    ("tiled", "gemv", "bf16"), ("tiled", "mfma", "bf16"),
])
@pytest.mark.parametrize("B,D,V", [(1, 256, 4099), (3, 520, 2001), (17, 1032, 3000), (64, 264, 1500),
                                   (130, 512, 1000)])
def test_single_pass_equals_two_stage(fs, layout, variant, dtype, B, D, V):
    """Stage 2 folded into Stage 1 (atomic maximum + last workgroup) gives
    the two-stage tokens, and leaves its workspace zero for the next call."""
    import torch
    if layout == "tiled" and dtype == "f32":
        pytest.skip("tiled layout is bf16 only")
    H, W = _rand_head(B * 5 + D + V, B, D, V, dtype)
    Hd, Wd = to_device(H), to_device(W)
    Wx = fs.TiledWeights(Wd) if layout == "tiled" else Wd
    nbytes = fs.workspace_bytes(B, D, V, Hd.dtype, variant=variant, tiled=layout == "tiled", single_pass=True)
    ws = torch.full((nbytes,), 7, dtype=torch.uint8, device="cuda")
    fs.workspace_reset(ws)
    for T, seed, step in ((1.0, 0, 0), (0.7, 5, 2**32 + 3), (0.0, 0, 0), (1.0, 9, 1)):
        two = fs.sample_fused(Hd, Wx, T, seed, step, variant=variant).cpu().numpy()
        one = fs.sample_fused(Hd, Wx, T, seed, step, variant=variant, single_pass=True, workspace=ws).cpu().numpy()
        assert np.array_equal(one, two)
        assert int(ws.count_nonzero()) == 0
        check_parity(H, W, T, seed, step, np.arange(B), one)


@pytest.mark.parametrize("B,D", [(2, 128), (5, 256), (64, 256), (9, 260), (64, 1032), (150, 132)])
@pytest.mark.parametrize("variant", ["auto", "gemv", "mfma"])
def test_f32_heads_past_one_row(fs, B, D, variant):
    """fp32 heads: the GEMV kernel's 2- and 4-row batch tiles (one or four
    16-byte chunks per lane in flight) and the fp32 matrix-core kernel
    (v_mfma_f32_16x16x4_f32; ragged K block, ragged batch and vocab tiles),
    sampling, greedy, the logits store and the unfused baseline."""
    import torch
    V = 1500
    H, W = _rand_head(B + D, B, D, V, "f32")
    Hd, Wd = to_device(H), to_device(W)
    for T, seed, step in ((1.0, 3, 1), (0.0, 0, 0)):
        tok = fs.sample_fused(Hd, Wd, T, seed, step, variant=variant).cpu().numpy()
        check_parity(H, W, T, seed, step, np.arange(B), tok)
    exact = oracle.exact_logits(H, W)
    l32 = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda")
    fs.sample_fused(Hd, Wd, 1.0, 3, 1, variant=variant, logits=l32)
    assert np.max(np.abs(l32.cpu().numpy().astype(np.float64) - exact)) < 1e-4
    tok = fs.sample_unfused(Hd, Wd, 0.8, 6, 2, variant=variant, logits_dtype=torch.float32).cpu().numpy()
    check_parity(H, W, 0.8, 6, 2, np.arange(B), tok)


def test_batch_prefix_and_repeat_determinism(fs):
    B, D, V = 13, 256, 3001
    H, W = _rand_head(9, B, D, V)
    Hd, Wd = to_device(H), to_device(W)
    full = fs.sample_fused(Hd, Wd, 1.0, 5, 2).cpu().numpy()
    for b in (1, 4, 8, 9):
        assert np.array_equal(fs.sample_fused(Hd[:b], Wd, 1.0, 5, 2).cpu().numpy(), full[:b])
    for _ in range(100):
        assert np.array_equal(fs.sample_fused(Hd, Wd, 1.0, 5, 2).cpu().numpy(), full)


@pytest.mark.parametrize("dtype,B,D", [
    ("bf16", 1, 512), ("bf16", 2, 4096), ("bf16", 4, 4096), ("bf16", 8, 512), ("bf16", 40, 768),
    ("bf16", 100, 512), ("bf16", 6, 520), ("bf16", 70, 1032),
    ("f32", 1, 256), ("f32", 2, 260), ("f32", 9, 256), ("f32", 70, 132),
])
def test_padded_leading_dimensions(fs, dtype, B, D):
    """Row-major W and H that are column slices of wider buffers (ldw = D + 264,
    ldh = D + 40): every row-major Stage-1 kernel family (GEMV up to two rows
    and the four-row GEMV plan on the 4096-wide head, the row-direct matrix-core
    kernels for D a multiple of 256 with 64/128-row and wide 256-row tiles, the
    LDS-transposing kernel for other D, the fp32 GEMV and matrix-core kernels)
    gives the oracle's tokens, the same tokens as contiguous copies, and stores
    the same logits."""
    import torch
    V = 2053
    Hc, Wc = _rand_head(B * 3 + D, B, D, V, dtype)
    Hd, Wd = to_device(Hc), to_device(Wc)
    Wwide = torch.zeros((V, D + 264), dtype=Wd.dtype, device="cuda")
    Wwide[:, :D] = Wd
    Wwide[:, D:] = float("nan")            # never read
    Hwide = torch.zeros((B, D + 40), dtype=Hd.dtype, device="cuda")
    Hwide[:, :D] = Hd
    Hwide[:, D:] = float("nan")
    Ws, Hs = Wwide[:, :D], Hwide[:, :D]
    assert Ws.stride(0) == D + 264 and Hs.stride(0) == D + 40
    for T, seed, step in ((1.0, 4, 3), (0.0, 0, 0)):
        tok = fs.sample_fused(Hs, Ws, T, seed, step).cpu().numpy()
        check_parity(Hc, Wc, T, seed, step, np.arange(B), tok)
        assert np.array_equal(tok, fs.sample_fused(Hd, Wd, T, seed, step).cpu().numpy())
        single = fs.sample_fused(Hs, Ws, T, seed, step, single_pass=True).cpu().numpy()
        assert np.array_equal(tok, single)
    l_pad = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda")
    l_ref = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda")
    fs.sample_fused(Hs, Ws, 1.0, 4, 3, logits=l_pad)
    fs.sample_fused(Hd, Wd, 1.0, 4, 3, logits=l_ref)
    assert torch.equal(l_pad, l_ref)
    tok = fs.sample_unfused(Hs, Ws, 0.8, 6, 1, logits_dtype=torch.float32).cpu().numpy()
    check_parity(Hc, Wc, 0.8, 6, 1, np.arange(B), tok)


def test_greedy_ties_lowest_index(fs):
    B, D, V = 3, 64, 999
    H, W = _rand_head(1, B, D, V)
    hv = inputs.bf16_bits_to_f32(H)
    for b, dup in enumerate((17, 500, 998)):
        W[dup] = inputs.f32_to_bf16_bits(hv[b] * np.float32(0.5))
        W[dup + 1 if dup + 1 < V else 0] = W[dup]
    W[0] = W[998]  # tie between 998 and 0: lowest index is 0
    Hd, Wd = to_device(H), to_device(W)
    got = fs.sample_fused(Hd, Wd, 0.0, 0, 0).cpu().numpy()
    want = oracle.sample(H, W, 0.0, 0, 0).idx
    assert got.tolist() == want.tolist()
    assert want[2] == 0


def test_nan_row_returns_minus_one(fs):
    B, D, V = 3, 64, 300
    H, W = _rand_head(2, B, D, V, "f32")
    H[1, :] = np.nan
    Hd, Wd = to_device(H), to_device(W)
    for T in (1.0, 0.0):
        got = fs.sample_fused(Hd, Wd, T, 1, 1).cpu().numpy()
        assert got[1] == -1
        check_parity(H[[0, 2]], W, T, 1, 1, [0], [got[0]])
        # row 2's noise is keyed by its row index 2
        r = oracle.sample(H, W, T, 1, 1, rows=[2])
        assert r.margin[0] <= TOL or got[2] == r.idx[0]


def test_tiled_split_last_round_ties_and_nan_rows(fs):
    """Exact ties and an all-NaN row where the last round runs as 64-row
    tiles. Two equal W rows in tiles of one kind (both 128-row, or both
    64-row, the two halves of one split tile included) get bit-equal logits,
    so greedy takes the lower index; across the seam between the kinds the
    sums are taken in another order, so either index is a correct answer
    (the tie rule for near-ties). Sampled rows against the oracle,
    single-pass equal to two-stage; the NaN row gives -1."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B, D, V = 24, 256, (2 * cus + cus // 8) * 128 + 40
    n128 = -(-V // 128)
    split = fs.num_vocab_tiles(B, D, V, tiled=True) - n128
    assert split > 0
    first = 128 * (n128 - split)              # first row of the 64-row tiles
    same = [(3, 700), (first + 63, first + 64), (first + 64 * 3 + 5, first + 64 * 5 + 9)]
    cross = [(first - 1, first), (0, V - 1)]
    pairs = same + cross
    H, W = _rand_head(11, B, D, V)
    hv = inputs.bf16_bits_to_f32(H)
    for b, (lo, hi) in enumerate(pairs):
        W[lo] = inputs.f32_to_bf16_bits(hv[b] * np.float32(0.5))
        W[hi] = W[lo]
    nan_row = len(pairs)
    H[nan_row, :] = inputs.f32_to_bf16_bits(np.full(D, np.nan, dtype=np.float32))
    Hd, tw = to_device(H), fs.TiledWeights(to_device(W))
    rows = np.array([b for b in range(B) if b != nan_row])
    for T in (0.0, 1.0):
        tok = fs.sample_fused(Hd, tw, T, 3, 1).cpu().numpy()
        assert tok[nan_row] == -1
        check_parity(H, W, T, 3, 1, rows, tok[rows])
        if T == 0.0:
            for b, (lo, hi) in enumerate(pairs):
                assert tok[b] == lo if b < len(same) else tok[b] in (lo, hi), (b, tok[b], lo, hi)
        assert np.array_equal(tok, fs.sample_fused(Hd, tw, T, 3, 1, single_pass=True).cpu().numpy())


def test_out_of_range_noise_keys(fs):
    """Large seeds and steps whose high words are non-zero."""
    B, D, V = 4, 128, 2000
    H, W = _rand_head(3, B, D, V)
    Hd, Wd = to_device(H), to_device(W)
    for seed, step in ((2**64 - 1, 2**64 - 1), (2**40 + 3, 2**33)):
        tok = fs.sample_fused(Hd, Wd, 1.0, seed, step).cpu().numpy()
        check_parity(H, W, 1.0, seed, step, np.arange(B), tok)


# ------------------------------------------------------------------ unfused baseline and logits store

@pytest.mark.parametrize("B,D,V", [(1, 256, 4099), (5, 1032, 3000), (8, 4096, 2053)])
def test_unfused_f32_logits_parity(fs, B, D, V):
    import torch
    H, W = _rand_head(B + D, B, D, V)
    Hd, Wd = to_device(H), to_device(W)
    for T in (1.0, 0.0):
        tok = fs.sample_unfused(Hd, Wd, T, 7, 3, logits_dtype=torch.float32).cpu().numpy()
        check_parity(H, W, T, 7, 3, np.arange(B), tok)
        tok16 = fs.sample_unfused(Hd, Wd, T, 7, 3, logits_dtype=torch.bfloat16).cpu().numpy()
        assert tok16.min() >= 0 and tok16.max() < V


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_store_logits_option(fs, dtype):
    import torch
    B, D, V = 5, 520, 2001
    H, W = _rand_head(4, B, D, V, dtype)
    Hd, Wd = to_device(H), to_device(W)
    exact = oracle.exact_logits(H, W)
    l32 = torch.full((B, V + 3), float("nan"), dtype=torch.float32, device="cuda")
    tok = fs.sample_fused(Hd, Wd, 1.0, 0, 0, logits=l32[:, :V]).cpu().numpy()
    got = l32[:, :V].cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - exact)) < 1e-4
    assert np.isnan(l32[:, V:].cpu().numpy()).all()  # nothing written past V
    check_parity(H, W, 1.0, 0, 0, np.arange(B), tok)
    l16 = torch.zeros((B, V), dtype=torch.bfloat16, device="cuda")
    fs.sample_fused(Hd, Wd, 1.0, 0, 0, logits=l16)
    got16 = l16.float().cpu().numpy().astype(np.float64)
    assert_bf16_logits(got16, exact)


# ------------------------------------------------------------------ distribution

def test_chi_square_on_device(fs):
    """V = 64 head, 10^6 draws (1000 identical rows x 1000 steps): the device
    reproduces the oracle's draws and passes chi-square against softmax."""
    import torch
    from scipy import stats
    h, w = inputs.chi2_inputs(0)
    H = np.repeat(h[None, :], 1000, axis=0)
    Hd, Wd = to_device(H), to_device(w)
    out = torch.empty((1000, 1000), dtype=torch.int32, device="cuda")
    for step in range(1000):
        fs.sample_fused(Hd, Wd, 1.0, 0, step, out=out[step])
    draws = out.cpu().numpy()
    mism = 0
    for step in range(0, 1000, 50):
        r = oracle.sample(H, w, 1.0, 0, step)
        firm = r.margin > TOL
        mism += int(np.sum(draws[step][firm] != r.idx[firm]))
    assert mism == 0
    l = oracle.exact_logits(h, w)[0]
    p = np.exp(l - l.max())
    p /= p.sum()
    counts = np.bincount(draws.ravel(), minlength=64)
    assert stats.chisquare(counts, p * counts.sum()).pvalue > 1e-3


@pytest.mark.parametrize("B", [65, 150, 300])
def test_row_major_wide_kernel(fs, B):
    """Row-major W with D a multiple of 256 above 64 rows: the row-major wide
    kernel (vocab tile 256, 128-column batch tiles, 256-byte row runs through a
    wave-private LDS transpose, rotated K order); sampling, greedy, logits
    store and the unfused path; the tiled layout's tokens on every row the
    oracle's margin decides (the two accumulate the K blocks in different
    orders, so exact near-ties may differ)."""
    import torch
    D, V = 512, 2053
    H, W = _rand_head(B + 31, B, D, V)
    Hd, Wd = to_device(H), to_device(W)
    assert fs.num_vocab_tiles(B, D, V) == (V + 255) // 256
    tw = fs.TiledWeights(Wd)
    for T, seed, step in ((1.0, 0, 0), (0.6, 77, 2**32 + 1), (0.0, 0, 0)):
        tok = fs.sample_fused(Hd, Wd, T, seed, step).cpu().numpy()
        check_parity(H, W, T, seed, step, np.arange(B), tok)
        firm = oracle.sample(H, W, T, seed, step).margin > TOL
        assert np.array_equal(tok[firm], fs.sample_fused(Hd, tw, T, seed, step).cpu().numpy()[firm])
    l32 = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda")
    fs.sample_fused(Hd, Wd, 1.0, 0, 0, logits=l32)
    assert np.max(np.abs(l32.cpu().numpy().astype(np.float64) - oracle.exact_logits(H, W))) < 1e-4
    tok = fs.sample_unfused(Hd, Wd, 1.0, 4, 4, logits_dtype=torch.float32).cpu().numpy()
    check_parity(H, W, 1.0, 4, 4, np.arange(B), tok)


@pytest.mark.parametrize("B,D,V", [(300, 544, 3000), (513, 288, 1001), (1000, 1024, 2053), (257, 7168, 700),
                                   (5, 256, 999)])
def test_big_tile_parity(fs, B, D, V):
    """The opt-in 256 x 256 tile (batch_tile 256: operands copied straight into
    LDS; tiled layout, D a multiple of 32) with ragged V, B and K blocks:
    every row against the oracle, greedy, single-pass, and the same tokens
    as the default wide kernel, whose accumulation order is the same."""
    H, W = _rand_head(B + D + V, B, D, V)
    Hd = to_device(H)
    tw = fs.TiledWeights(to_device(W))
    rows = np.arange(B)
    for T, seed, step in ((1.0, 2, 9), (0.0, 0, 0)):
        tok = fs.sample_fused(Hd, tw, T, seed, step, batch_tile=256).cpu().numpy()
        check_parity(H, W, T, seed, step, rows, tok)
        one = fs.sample_fused(Hd, tw, T, seed, step, batch_tile=256, single_pass=True).cpu().numpy()
        assert np.array_equal(tok, one)
        wide = fs.sample_fused(Hd, tw, T, seed, step, variant="mfma", vocab_tile=256).cpu().numpy()
        assert np.array_equal(tok, wide)


def test_concurrent_streams_with_distinct_workspaces(fs):
    """Calls on two streams with their own workspaces and outputs overlap
    safely and give the sequential results (the header's concurrency rule)."""
    import torch
    B, D, V = 40, 512, 3001
    H, W = _rand_head(41, B, D, V)
    Hd, Wd = to_device(H), to_device(W)
    tw = fs.TiledWeights(Wd)
    want = [fs.sample_fused(Hd, tw, 1.0, 3, step).cpu().numpy() for step in range(8)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    ws = [torch.empty(fs.workspace_bytes(B, D, V, tiled=True), dtype=torch.uint8, device="cuda") for _ in range(2)]
    outs = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(8)]
    torch.cuda.synchronize()
    for step in range(8):
        k = step % 2
        with torch.cuda.stream(streams[k]):
            fs.sample_fused(Hd, tw, 1.0, 3, step, out=outs[step], workspace=ws[k], stream=streams[k])
    torch.cuda.synchronize()
    for step in range(8):
        assert np.array_equal(outs[step].cpu().numpy(), want[step])


@pytest.mark.parametrize("single_pass", [False, True])
@pytest.mark.parametrize("B,D,V", [(24, 1024, 2053), (300, 512, 3001)])
def test_graph_capture_and_replay(fs, single_pass, B, D, V):
    """A fused call enqueues only kernel launches, so it can be captured in a
    HIP graph: every replay (with new hidden states copied into the captured
    input between replays, and eager calls in between) equals the eager call.
    Narrow tile (24 rows) and the register-ring wide tile (300 rows)."""
    _graph_capture_check(fs, single_pass, B, D, V)


@pytest.mark.parametrize("single_pass", [False, True])
def test_graph_capture_split_last_round(fs, single_pass):
    """The same with a nearly empty last round of 128-row tiles, which runs
    as 64-row tiles (the plan's extra candidate slots included)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    _graph_capture_check(fs, single_pass, 64, 256, (2 * cus + cus // 5) * 128 + 9)


def _graph_capture_check(fs, single_pass, B, D, V):
    import torch
    H, W = _rand_head(43, B, D, V)
    Hd = to_device(H)
    tw = fs.TiledWeights(to_device(W))
    rng = np.random.default_rng(5)
    ws = torch.empty(fs.workspace_bytes(B, D, V, tiled=True, single_pass=single_pass), dtype=torch.uint8, device="cuda")
    fs.workspace_reset(ws)
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    static_h = Hd.clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):   # warm the call on the capture stream first
        fs.sample_fused(static_h, tw, 0.9, 7, 11, out=out, workspace=ws, single_pass=single_pass, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fs.sample_fused(static_h, tw, 0.9, 7, 11, out=out, workspace=ws, single_pass=single_pass, stream=s)
    torch.cuda.synchronize()
    eager_ws = torch.empty_like(ws)
    fs.workspace_reset(eager_ws)
    for rep in range(4):
        Hn = inputs.f32_to_bf16_bits(rng.standard_normal((B, D), dtype=np.float32))
        static_h.copy_(to_device(Hn))
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        eager = fs.sample_fused(static_h, tw, 0.9, 7, 11, workspace=eager_ws, single_pass=single_pass).cpu().numpy()
        assert np.array_equal(got, eager), f"replay {rep}"
        check_parity(Hn, W, 0.9, 7, 11, np.arange(B), got)
