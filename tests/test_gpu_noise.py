"""Device noise equals the oracle's: Philox words bit for bit, Gumbel values
within 1e-5 of the fp64 oracle (checked on the extreme and middle ranges of
the 32-bit word lattice and on a strided sweep of all of it)."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fs():
    import torch
    assert torch.cuda.is_available()
    from lm_head_gemm_amd import flashsample
    return flashsample


@pytest.mark.parametrize("seed,step,b,v0,n", [
    (0, 0, 0, 0, 4096),
    (1, 0, 255, 5, 128251),
    (4, 2**32 + 5, 1023, 129279 - 4099, 4099),
    (0x123456789ABCDEF, 63, 7, 3, 1000),
])
def test_philox_words_bit_exact(fs, seed, step, b, v0, n):
    got = fs.test_philox(seed, step, b, v0, n).cpu().numpy().view(np.uint32).astype(np.uint64)
    want = oracle.philox_words(seed, step, b, v0, v0 + n)
    assert np.array_equal(got, want)


def test_philox_zero_counter_published_vector(fs):
    """Seed 0, step 0, row 0, vocab 0..3 is the all-zero counter and key: the
    device words equal the generator's published known answer (fixture)."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "philox4x32_10_kat.txt")
    with open(path) as f:
        zero = [l.split() for l in f if l.strip() and not l.startswith("#")][0]
    assert all(int(w, 16) == 0 for w in zero[:6])
    got = fs.test_philox(0, 0, 0, 0, 4).cpu().numpy().view(np.uint32)
    assert [int(w) for w in got] == [int(w, 16) for w in zero[6:10]]


def test_gumbel_map_accuracy(fs):
    import torch
    edge = 1 << 22
    words = np.concatenate([
        np.arange(0, edge, dtype=np.uint64),
        np.arange(2**31 - edge, 2**31 + edge, dtype=np.uint64),
        np.arange(2**32 - edge, 2**32, dtype=np.uint64),
        np.arange(0, 2**32, 61, dtype=np.uint64),
    ])
    worst = 0.0
    for chunk in np.array_split(words, 16):
        w32 = torch.from_numpy(chunk.astype(np.uint32).view(np.int32)).cuda()
        g = fs.test_gumbel(w32).cpu().numpy().astype(np.float64)
        ref = oracle.gumbel_from_words(chunk)
        worst = max(worst, float(np.max(np.abs(g - ref))))
    print(f"max |g_gpu - g_fp64| = {worst:.3e}")
    assert worst <= 1e-5


@pytest.mark.timeout(1800)
def test_gumbel_map_every_word(fs):
    """All 2^32 words through the device Gumbel map, each against the fp64
    oracle: |g_gpu - g_fp64| <= 1e-5 everywhere. The device evaluates chunks
    of 2^28 words; host threads compare slices of each chunk."""
    import os
    import time
    from concurrent.futures import ThreadPoolExecutor

    import torch

    chunk, piece = 1 << 28, 1 << 22
    try:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        threads = 4

    def compare(g, start, a):
        words = np.arange(start + a, start + a + piece, dtype=np.uint64)
        err = np.abs(g[a:a + piece].astype(np.float64) - oracle.gumbel_from_words(words))
        i = int(np.argmax(err))
        return float(err[i]), int(words[i])

    worst, worst_word = 0.0, -1
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for start in range(0, 1 << 32, chunk):
            w = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda").to(torch.int32)
            g = fs.test_gumbel(w).cpu().numpy()
            del w
            for e, word in ex.map(lambda a: compare(g, start, a), range(0, chunk, piece)):
                if e > worst:
                    worst, worst_word = e, word
    print(f"all 2^32 words: max |g_gpu - g_fp64| = {worst:.3e} at word {worst_word:#010x} "
          f"({time.perf_counter() - t0:.0f} s, {threads} host threads)", flush=True)
    assert worst <= 1e-5
