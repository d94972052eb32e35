"""The C ABI library loads, exports every entry point include/*.h declares, and
rejects invalid arguments synchronously with the documented status codes
(no device is needed: nothing is launched on a validation error)."""
import ctypes
import glob
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "lm_head_gemm_amd", "libflashsample.so")

OK, INVALID, UNSUPPORTED, WS_SMALL, HIP = 0, 1, 2, 3, 4
BF16, F32 = 0, 1
FAKE = 0x100000  # aligned, never dereferenced: every call below fails validation first


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^[A-Za-z_][\w \*]*?\b(fs_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (python -m lm_head_gemm_amd.build)")
    from lm_head_gemm_amd import flashsample  # sets argtypes/restypes
    return flashsample._lib


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("fs_sample_fused", "fs_sample_unfused", "fs_workspace_bytes", "fs_status_string",
                 "fs_sample_fused_ex", "fs_unfused_workspace_bytes", "fs_last_hip_error"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def test_status_strings(lib):
    assert lib.fs_status_string(OK) == b"FS_OK"
    assert lib.fs_status_string(WS_SMALL) == b"FS_ERR_WORKSPACE_TOO_SMALL"
    assert lib.fs_status_string(99) == b"FS_ERR_UNKNOWN"
    assert lib.fs_last_hip_error() == 0


def test_default_plan_tile_counts(lib):
    """Default vocab tiles per plan on row-major W (no compute): GEMV 16-row
    tiles at B <= 2 (256-row tiles on bf16 heads 8192 wide and more), the
    row-direct matrix-core kernel's 128-row tiles from B = 3 to 64 when D is a
    multiple of 256, the wide kernel's 256 rows from 65 on, and the
    LDS-transposing kernel's 64 (B <= 32) or 128 rows for other D."""
    V = 128256
    nt = lambda B, D, dt=BF16: lib.fs_num_vocab_tiles(B, D, V, dt, None)
    assert nt(1, 4096) == nt(2, 7168) == nt(2, 3584) == math.ceil(V / 16)
    assert nt(1, 8192) == nt(2, 8192) == math.ceil(V / 256)
    assert nt(3, 4096) == nt(4, 7168) == nt(4, 8192) == nt(64, 3584) == math.ceil(V / 128)
    assert nt(65, 4096) == nt(1024, 7168) == math.ceil(V / 256)
    assert nt(3, 4104) == nt(32, 4104) == math.ceil(V / 64)
    assert nt(33, 4104) == math.ceil(V / 128)
    assert nt(3, 4096, F32) == math.ceil(V / 128)     # fp32 heads: the fp32 matrix-core kernel


def test_workspace_sizes(lib):
    from lm_head_gemm_amd.flashsample import FsOptions
    nt = lib.fs_num_vocab_tiles(1, 4096, 128256, BF16, None)
    assert nt > 0
    ws = lib.fs_workspace_bytes(1, 4096, 128256, BF16)
    assert ws >= 8 * nt and ws % 256 == 0
    assert lib.fs_workspace_bytes(0, 4096, 128256, BF16) == 0
    assert lib.fs_workspace_bytes(1, 4096, 2**31, BF16) == 0
    assert lib.fs_workspace_bytes(1, 4096, 10, 7) == 0
    o = FsOptions()
    g = lib.fs_vocab_tile_granule(1)
    o.vocab_tile = 3 * g
    assert lib.fs_num_vocab_tiles(2, 64, 1000, BF16, ctypes.byref(o)) == math.ceil(1000 / (3 * g))
    o.vocab_tile = g + 1
    assert lib.fs_num_vocab_tiles(2, 64, 1000, BF16, ctypes.byref(o)) == -1
    assert lib.fs_workspace_bytes_ex(2, 64, 1000, BF16, ctypes.byref(o)) == 0
    uw = lib.fs_unfused_workspace_bytes(4, 4096, 1000, BF16, F32)
    assert uw >= 4 * 1000 * 4


def _fused(lib, **kw):
    a = dict(H=FAKE, ldh=64, W=FAKE, ldw=64, dtype=BF16, B=2, D=64, V=1000, T=1.0, seed=0, step=0,
             ws=FAKE, wsb=1 << 20, out=FAKE, stream=None, opts=None)
    a.update(kw)
    args = [a["H"], a["ldh"], a["W"], a["ldw"], a["dtype"], a["B"], a["D"], a["V"], a["T"], a["seed"],
            a["step"], a["ws"], a["wsb"], a["out"], a["stream"]]
    if a["opts"] is None:
        return lib.fs_sample_fused(*args)
    return lib.fs_sample_fused_ex(*args, ctypes.byref(a["opts"]))


@pytest.mark.parametrize("kw,status", [
    (dict(H=None), INVALID), (dict(W=None), INVALID), (dict(ws=None), INVALID), (dict(out=None), INVALID),
    (dict(B=0), INVALID), (dict(B=-3), INVALID), (dict(D=0), INVALID), (dict(V=0), INVALID),
    (dict(V=2**31), INVALID), (dict(B=2**20), INVALID),
    (dict(ldh=32), INVALID), (dict(ldw=63), INVALID),
    (dict(T=-1.0), INVALID), (dict(T=float("nan")), INVALID), (dict(T=float("inf")), INVALID),
    (dict(dtype=7), UNSUPPORTED),
    (dict(H=FAKE + 2), UNSUPPORTED), (dict(W=FAKE + 8), UNSUPPORTED), (dict(ws=FAKE + 4), UNSUPPORTED),
    (dict(D=12, ldh=12, ldw=12), UNSUPPORTED), (dict(ldh=68), UNSUPPORTED),
    (dict(D=128 * 1024, ldh=128 * 1024, ldw=128 * 1024), UNSUPPORTED),
    (dict(D=81416, ldh=81416, ldw=81416), UNSUPPORTED),   # H row past 159 KiB
    (dict(wsb=8), WS_SMALL),
])
def test_fused_validation(lib, kw, status):
    assert _fused(lib, **kw) == status


def test_fused_option_validation(lib):
    from lm_head_gemm_amd.flashsample import FsOptions
    o = FsOptions()
    o.variant = 9
    assert _fused(lib, opts=o) == INVALID
    o = FsOptions()
    o.vocab_tile = 17
    assert _fused(lib, opts=o) == INVALID
    o = FsOptions()
    o.vocab_tile = -16
    assert _fused(lib, opts=o) == INVALID
    o = FsOptions()
    o.logits = FAKE
    o.ld_logits = 999
    assert _fused(lib, opts=o) == INVALID
    o.ld_logits = 1000
    o.logits_dtype = 5
    assert _fused(lib, opts=o) == UNSUPPORTED
    o.logits_dtype = F32
    o.logits = FAKE + 4
    assert _fused(lib, opts=o) == UNSUPPORTED
    o.logits = FAKE
    assert _fused(lib, opts=o, wsb=0) == WS_SMALL


def test_unfused_validation(lib):
    base = [FAKE, 64, FAKE, 64, BF16, 2, 64, 1000, 1.0, 0, 0]
    assert lib.fs_sample_unfused(*base, 9, FAKE, 1 << 20, FAKE, None) == UNSUPPORTED
    assert lib.fs_sample_unfused(*base, F32, FAKE, 16, FAKE, None) == WS_SMALL
    bad = list(base)
    bad[0] = None
    assert lib.fs_sample_unfused(*bad, F32, FAKE, 1 << 20, FAKE, None) == INVALID
    bad = list(base)
    bad[8] = -0.5
    assert lib.fs_sample_unfused(*bad, F32, FAKE, 1 << 20, FAKE, None) == INVALID


def test_test_hooks_validation(lib):
    assert lib.fs_test_philox(0, 0, 0, 0, 0, FAKE, None) == INVALID
    assert lib.fs_test_philox(0, 0, -1, 0, 4, FAKE, None) == INVALID
    assert lib.fs_test_philox(0, 0, 0, 0, 4, None, None) == INVALID
    assert lib.fs_test_gumbel(None, 4, FAKE, None) == INVALID
    assert lib.fs_test_gumbel(FAKE, 0, FAKE, None) == INVALID


def test_tiled_layout_validation(lib):
    from lm_head_gemm_amd.flashsample import FsOptions
    assert lib.fs_tiled_weights_bytes(4099, 1032, BF16) == 264 * 5 * 8192   # 257 blocks -> 33 groups of 8
    assert lib.fs_tiled_weights_bytes(16, 256, BF16) == 8 * 8192
    assert lib.fs_tiled_weights_bytes(16, 256, F32) == 0
    assert lib.fs_tiled_weights_bytes(0, 256, BF16) == 0
    assert lib.fs_pack_weights_tiled(None, 64, 10, 64, BF16, FAKE, 1 << 20, None) == INVALID
    assert lib.fs_pack_weights_tiled(FAKE, 32, 10, 64, BF16, FAKE, 1 << 20, None) == INVALID
    assert lib.fs_pack_weights_tiled(FAKE, 64, 10, 64, F32, FAKE, 1 << 20, None) == UNSUPPORTED
    assert lib.fs_pack_weights_tiled(FAKE, 64, 10, 64, BF16, FAKE + 8, 1 << 20, None) == UNSUPPORTED
    assert lib.fs_pack_weights_tiled(FAKE, 64, 10, 64, BF16, FAKE, 100, None) == WS_SMALL
    o = FsOptions()
    o.weights_layout = 2
    assert _fused(lib, opts=o) == INVALID
    o = FsOptions()
    o.reserved = 1
    assert _fused(lib, opts=o) == INVALID
    # single pass: B keys + 33 counter slots of 256 bytes, independent of the tile count
    o = FsOptions()
    o.single_pass = 1
    assert lib.fs_workspace_bytes_ex(3, 64, 100000, BF16, ctypes.byref(o)) == 256 + 33 * 256
    assert lib.fs_workspace_bytes_ex(1000, 64, 100000, BF16, ctypes.byref(o)) == 8192 + 33 * 256
    assert _fused(lib, opts=o, wsb=256 + 33 * 256 - 1) == WS_SMALL
    assert lib.fs_workspace_reset(None, 256, None) == INVALID
    assert lib.fs_workspace_reset(FAKE, 12, None) == INVALID
    assert lib.fs_workspace_reset(FAKE + 8, 256, None) == UNSUPPORTED
    o = FsOptions()
    o.weights_layout = 1
    assert _fused(lib, opts=o, dtype=F32) == UNSUPPORTED
    o.vocab_tile = 96
    assert _fused(lib, opts=o) == INVALID
    o.vocab_tile = 128
    o.batch_tile = 48
    assert _fused(lib, opts=o) == INVALID
    # ldw is ignored for the tiled layout; the other checks still apply
    o.batch_tile = 0
    assert _fused(lib, opts=o, ldw=0, wsb=8) == WS_SMALL
    # the 256-row wide tile: MFMA only, default from B = 65 on, batch tile 128 only there
    o = FsOptions()
    o.weights_layout = 1
    assert lib.fs_num_vocab_tiles(64, 4096, 128256, BF16, ctypes.byref(o)) == 1002
    assert lib.fs_num_vocab_tiles(65, 4096, 128256, BF16, ctypes.byref(o)) == 501
    o.vocab_tile = 256
    assert lib.fs_num_vocab_tiles(8, 4096, 1000, BF16, ctypes.byref(o)) == 4
    o.batch_tile = 64
    assert lib.fs_num_vocab_tiles(8, 4096, 1000, BF16, ctypes.byref(o)) == -1
    o.batch_tile = 128
    assert lib.fs_num_vocab_tiles(8, 4096, 1000, BF16, ctypes.byref(o)) == 4
    o.vocab_tile = 128
    assert lib.fs_num_vocab_tiles(8, 4096, 1000, BF16, ctypes.byref(o)) == -1
    o.vocab_tile = 256
    o.batch_tile = 0
    o.variant = 1  # GEMV
    assert lib.fs_num_vocab_tiles(8, 4096, 1000, BF16, ctypes.byref(o)) == -1
    # the opt-in 256 x 256 tile (batch_tile 256): tiled bf16, D a multiple of
    # 32, plain sampling only
    o = FsOptions()
    o.weights_layout = 1
    o.batch_tile = 256
    assert lib.fs_num_vocab_tiles(300, 4096, 1000, BF16, ctypes.byref(o)) == 4
    assert lib.fs_workspace_bytes_ex(300, 4096, 1000, BF16, ctypes.byref(o)) == 300 * 4 * 8 + 128
    assert lib.fs_num_vocab_tiles(300, 4104, 1000, BF16, ctypes.byref(o)) == -1        # D % 32 != 0
    o.vocab_tile = 128
    assert lib.fs_num_vocab_tiles(300, 4096, 1000, BF16, ctypes.byref(o)) == -1
    o.vocab_tile = 0
    o.group_size = 1024
    assert _fused(lib, opts=o, B=300, D=4096, V=1000, ldh=4096, ldw=4096) == UNSUPPORTED
    o.group_size = 0
    o.logits = FAKE
    o.ld_logits = 1000
    assert _fused(lib, opts=o, B=300, D=4096, V=1000, ldh=4096, ldw=4096) == UNSUPPORTED
    o.logits = None
    assert _fused(lib, opts=o, B=300, D=4096, V=1000, ldh=4096, ldw=4096, dtype=F32) == UNSUPPORTED
    o.weights_layout = 0
    assert lib.fs_num_vocab_tiles(300, 4096, 1000, BF16, ctypes.byref(o)) == -1         # row-major W
    o.weights_layout = 1
    ub = [FAKE, 4096, FAKE, 4096, BF16, 300, 4096, 1000, 1.0, 0, 0, F32, FAKE, 1 << 30, FAKE, None]
    assert lib.fs_sample_unfused_ex(*ub, ctypes.byref(o)) == UNSUPPORTED
    base = [FAKE, 64, FAKE, 64, BF16, 2, 64, 1000, 1.0, 0, 0, F32, FAKE, 1 << 20, FAKE, None]
    o = FsOptions()
    o.weights_layout = 3
    assert lib.fs_sample_unfused_ex(*base, ctypes.byref(o)) == INVALID


def test_grouped_option_validation(lib):
    """group_size: tiled bf16 MFMA, two-stage only, a multiple of the vocab tile;
    the workspace adds one fp32 log-mass per (tile, row)."""
    from lm_head_gemm_amd.flashsample import FsOptions
    o = FsOptions()
    o.weights_layout = 1
    o.group_size = -256
    assert _fused(lib, opts=o) == INVALID
    o.group_size = 256
    nt = lib.fs_num_vocab_tiles(8, 4096, 128256, BF16, ctypes.byref(o))
    assert nt == 1002  # MFMA default tile 128 below B = 65
    want = -(-8 * nt * 8 // 256) * 256 + -(-8 * nt * 4 // 256) * 256
    assert lib.fs_workspace_bytes_ex(8, 4096, 128256, BF16, ctypes.byref(o)) == want
    o.group_size = 192            # not a multiple of the 128-row tile
    assert lib.fs_workspace_bytes_ex(8, 4096, 128256, BF16, ctypes.byref(o)) == 0
    assert _fused(lib, opts=o) == INVALID
    o.group_size = 128
    assert lib.fs_workspace_bytes_ex(100, 4096, 128256, BF16, ctypes.byref(o)) == 0  # wide tile is 256
    o.group_size = 256
    o.single_pass = 1
    assert _fused(lib, opts=o) == UNSUPPORTED
    o.single_pass = 0
    o.variant = 1                 # GEMV
    assert _fused(lib, opts=o) == UNSUPPORTED
    o = FsOptions()               # row-major W: only with D a multiple of 256
    o.group_size = 256
    assert _fused(lib, opts=o) == UNSUPPORTED
    assert _fused(lib, opts=o, D=256, ldh=256, ldw=256, wsb=8) == WS_SMALL
    assert lib.fs_num_vocab_tiles(100, 512, 5000, BF16, ctypes.byref(o)) == 20   # wide tile from B = 65
    o.vocab_tile = 256
    assert lib.fs_num_vocab_tiles(100, 520, 5000, BF16, ctypes.byref(o)) == -1   # not for other D
    base = [FAKE, 64, FAKE, 64, BF16, 2, 64, 1000, 1.0, 0, 0, F32, FAKE, 1 << 20, FAKE, None]
    o.weights_layout = 1
    assert lib.fs_sample_unfused_ex(*base, ctypes.byref(o)) == UNSUPPORTED


def test_f32_matrix_core_options(lib):
    """fp32 heads: GEMV up to 2 rows, the fp32 matrix-core kernel above
    (row-major only, 128-row vocab tiles, batch tiles 16/32/64)."""
    from lm_head_gemm_amd.flashsample import FsOptions
    V = 1000
    assert lib.fs_num_vocab_tiles(2, 256, V, F32, None) == math.ceil(V / 16)
    assert lib.fs_num_vocab_tiles(3, 256, V, F32, None) == math.ceil(V / 128)
    o = FsOptions()
    o.variant = 2  # MFMA
    assert lib.fs_num_vocab_tiles(1, 256, V, F32, ctypes.byref(o)) == math.ceil(V / 128)
    o.vocab_tile = 64
    assert lib.fs_num_vocab_tiles(1, 256, V, F32, ctypes.byref(o)) == -1
    o.vocab_tile = 128
    o.batch_tile = 32
    assert lib.fs_num_vocab_tiles(40, 256, V, F32, ctypes.byref(o)) == math.ceil(V / 128)
    o.batch_tile = 128
    assert lib.fs_num_vocab_tiles(40, 256, V, F32, ctypes.byref(o)) == -1
    o = FsOptions()
    o.group_size = 1024
    assert _fused(lib, opts=o, dtype=F32, B=16) == UNSUPPORTED
    o = FsOptions()
    o.weights_layout = 1
    o.variant = 2
    assert _fused(lib, opts=o, dtype=F32, B=16) == UNSUPPORTED


def test_workspace_size_argument_order(lib):
    """The sizing calls take (B, D, V) in the order of the sampling calls'
    size arguments (not (B, V, D)): pinned by a shape where swapping D and V
    changes the answer."""
    B, D, V = 2, 64, 100000
    tiles = math.ceil(V / 16)                         # GEMV plan, 16-row vocab tiles
    assert lib.fs_num_vocab_tiles(B, D, V, BF16, None) == tiles
    assert lib.fs_workspace_bytes(B, D, V, BF16) == -(-B * tiles * 8 // 256) * 256
    assert lib.fs_workspace_bytes(B, V, D, BF16) != lib.fs_workspace_bytes(B, D, V, BF16)
    # unfused: [B, round_up(V, 8)] logits, then one key per (row, 2048-entry part)
    logits = -(-B * (-(-V // 8) * 8) * 4 // 256) * 256
    parts = -(-B * math.ceil(V / 2048) * 8 // 256) * 256
    assert lib.fs_unfused_workspace_bytes(B, D, V, BF16, F32) == logits + parts
    assert lib.fs_unfused_workspace_bytes(B, V, D, BF16, F32) != logits + parts


def _noalloc(lib, **kw):
    a = dict(H=FAKE, ldh=64, W=FAKE, ldw=64, dtype=BF16, B=2, D=64, V=1000, T=1.0, seed=0, step=0,
             out=FAKE, stream=None, opts=None)
    a.update(kw)
    from lm_head_gemm_amd.flashsample import FsOptions
    o = a["opts"] if a["opts"] is not None else FsOptions()
    return lib.fs_sample_fused_noalloc(a["H"], a["ldh"], a["W"], a["ldw"], a["dtype"], a["B"], a["D"], a["V"],
                                       a["T"], a["seed"], a["step"], a["out"], a["stream"], ctypes.byref(o))


@pytest.mark.parametrize("kw,status", [
    (dict(H=None), INVALID), (dict(W=None), INVALID), (dict(out=None), INVALID), (dict(B=0), INVALID),
    (dict(ldw=63), INVALID), (dict(T=float("nan")), INVALID), (dict(dtype=7), UNSUPPORTED),
    (dict(H=FAKE + 2), UNSUPPORTED),
    # candidates past the 8 MiB scratch array: 4096 rows x 8016 tiles x 8 bytes
    (dict(B=4096, V=128256), WS_SMALL),
])
def test_noalloc_validation(lib, kw, status):
    """The allocation-free entry point validates like the fused call (its
    workspace is the static scratch array) before touching the device, and
    refuses sizes whose workspace does not fit the array."""
    assert _noalloc(lib, **kw) == status


def test_noalloc_scratch_fits_the_workloads(lib):
    """Two-stage workspaces of every workload's largest batch (row-major and
    tiled plans) fit the scratch array, and so does the grouped variant at
    B = 1024; the first size past it is refused."""
    from lm_head_gemm_amd.flashsample import FsOptions, NOALLOC_SCRATCH_BYTES
    assert NOALLOC_SCRATCH_BYTES == 8 << 20
    o = FsOptions()
    for B, D, V in ((256, 4096, 128256), (256, 3584, 152064), (512, 8192, 128256), (1024, 7168, 129280)):
        for layout in (0, 1):
            o.weights_layout = layout
            assert 0 < lib.fs_workspace_bytes_ex(B, D, V, BF16, ctypes.byref(o)) <= NOALLOC_SCRATCH_BYTES
    o.weights_layout = 1
    o.group_size = 16384
    assert lib.fs_workspace_bytes_ex(1024, 7168, 129280, BF16, ctypes.byref(o)) <= NOALLOC_SCRATCH_BYTES
