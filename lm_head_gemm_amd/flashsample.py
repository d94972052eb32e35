"""Python binding of libflashsample (argument marshalling only).

Every step of sampling runs in the library's HIP kernels; PyTorch supplies
device memory and the current stream. The function names follow the C ABI in
include/flashsample.h. Importing this module loads the library and fails
loudly if it has not been built (python -m lm_head_gemm_amd.build).
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime the library binds to

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflashsample.so")

FS_OK = 0
FS_ERR_INVALID_ARGUMENT = 1
FS_ERR_UNSUPPORTED = 2
FS_ERR_WORKSPACE_TOO_SMALL = 3
FS_ERR_HIP = 4

FS_DTYPE_BF16 = 0
FS_DTYPE_F32 = 1

FS_VARIANT_AUTO = 0
FS_VARIANT_GEMV = 1
FS_VARIANT_MFMA = 2

VARIANTS = {"auto": FS_VARIANT_AUTO, "gemv": FS_VARIANT_GEMV, "mfma": FS_VARIANT_MFMA}

FS_LAYOUT_ROWS = 0
FS_LAYOUT_TILED = 1


class FsOptions(ctypes.Structure):
    _fields_ = [
        ("variant", ctypes.c_int32),
        ("vocab_tile", ctypes.c_int32),
        ("logits", ctypes.c_void_p),
        ("ld_logits", ctypes.c_int64),
        ("logits_dtype", ctypes.c_int32),
        ("batch_tile", ctypes.c_int32),
        ("stage1_start", ctypes.c_void_p),
        ("stage1_stop", ctypes.c_void_p),
        ("weights_layout", ctypes.c_int32),
        ("single_pass", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class FlashSampleError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.fs_status_string(status).decode()
        if status == FS_ERR_HIP:
            msg += f" (hipError_t {_lib.fs_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m lm_head_gemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_i64, c_u64, c_sz, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p
    lib.fs_status_string.restype = ctypes.c_char_p
    lib.fs_status_string.argtypes = [ctypes.c_int]
    lib.fs_last_hip_error.restype = ctypes.c_int
    lib.fs_num_vocab_tiles.restype = c_i64
    lib.fs_num_vocab_tiles.argtypes = [c_i64, c_i64, c_i64, ctypes.c_int, ctypes.POINTER(FsOptions)]
    lib.fs_vocab_tile_granule.restype = ctypes.c_int32
    lib.fs_vocab_tile_granule.argtypes = [ctypes.c_int]
    lib.fs_workspace_bytes.restype = c_sz
    lib.fs_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, ctypes.c_int]
    lib.fs_workspace_bytes_ex.restype = c_sz
    lib.fs_workspace_bytes_ex.argtypes = [c_i64, c_i64, c_i64, ctypes.c_int, ctypes.POINTER(FsOptions)]
    fused = [vp, c_i64, vp, c_i64, ctypes.c_int, c_i64, c_i64, c_i64, ctypes.c_float, c_u64, c_u64,
             vp, c_sz, vp, vp]
    lib.fs_sample_fused.restype = ctypes.c_int
    lib.fs_sample_fused.argtypes = fused
    lib.fs_sample_fused_ex.restype = ctypes.c_int
    lib.fs_sample_fused_ex.argtypes = fused + [ctypes.POINTER(FsOptions)]
    lib.fs_sample_fused_noalloc.restype = ctypes.c_int
    lib.fs_sample_fused_noalloc.argtypes = [vp, c_i64, vp, c_i64, ctypes.c_int, c_i64, c_i64, c_i64,
                                            ctypes.c_float, c_u64, c_u64, vp, vp, ctypes.POINTER(FsOptions)]
    lib.fs_unfused_workspace_bytes.restype = c_sz
    lib.fs_unfused_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, ctypes.c_int, ctypes.c_int]
    unfused = [vp, c_i64, vp, c_i64, ctypes.c_int, c_i64, c_i64, c_i64, ctypes.c_float, c_u64, c_u64,
               ctypes.c_int, vp, c_sz, vp, vp]
    lib.fs_sample_unfused.restype = ctypes.c_int
    lib.fs_sample_unfused.argtypes = unfused
    lib.fs_sample_unfused_ex.restype = ctypes.c_int
    lib.fs_sample_unfused_ex.argtypes = unfused + [ctypes.POINTER(FsOptions)]
    lib.fs_tiled_weights_bytes.restype = c_sz
    lib.fs_tiled_weights_bytes.argtypes = [c_i64, c_i64, ctypes.c_int]
    lib.fs_pack_weights_tiled.restype = ctypes.c_int
    lib.fs_pack_weights_tiled.argtypes = [vp, c_i64, c_i64, c_i64, ctypes.c_int, vp, c_sz, vp]
    lib.fs_test_philox.restype = ctypes.c_int
    lib.fs_test_philox.argtypes = [c_u64, c_u64, c_i64, c_i64, c_i64, vp, vp]
    lib.fs_test_gumbel.restype = ctypes.c_int
    lib.fs_test_gumbel.argtypes = [vp, c_i64, vp, vp]
    lib.fs_workspace_reset.restype = ctypes.c_int
    lib.fs_workspace_reset.argtypes = [vp, c_sz, vp]
    lib.fs_probe_read_blocks.restype = c_i64
    lib.fs_probe_read_blocks.argtypes = [c_i64, c_i64]
    lib.fs_probe_read.restype = ctypes.c_int
    lib.fs_probe_read.argtypes = [vp, c_i64, c_i64, vp, vp]
    return lib


_lib = _load()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return FS_DTYPE_BF16
    if t == torch.float32:
        return FS_DTYPE_F32
    raise TypeError(f"unsupported dtype {t}")


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(st: int, where: str):
    if st != FS_OK:
        raise FlashSampleError(st, where)


class TiledWeights:
    """A bf16 LM head [V, D] repacked once into the tiled layout
    (fs_pack_weights_tiled): blocks of 16 vocab rows x 256 columns, each 8 KiB
    contiguous in matrix-core operand order. Pass it wherever W is taken."""

    def __init__(self, W: torch.Tensor, stream=None):
        if not W.is_cuda or W.dtype != torch.bfloat16 or W.dim() != 2 or W.stride(1) != 1:
            raise ValueError("TiledWeights needs a bf16 device tensor [V, D] with contiguous rows")
        self.V, self.D = W.shape
        nbytes = int(_lib.fs_tiled_weights_bytes(self.V, self.D, FS_DTYPE_BF16))
        self.data = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
        _check(_lib.fs_pack_weights_tiled(W.data_ptr(), W.stride(0), self.V, self.D, FS_DTYPE_BF16,
                                          self.data.data_ptr(), nbytes, _stream(stream)),
               "fs_pack_weights_tiled")
        self.dtype = W.dtype
        self.device = W.device

    @property
    def shape(self):
        return (self.V, self.D)


def _weights(W):
    """(pointer, ldw, V, D, layout) of a row-major tensor or TiledWeights."""
    if isinstance(W, TiledWeights):
        return W.data.data_ptr(), W.D, W.V, W.D, FS_LAYOUT_TILED
    return W.data_ptr(), W.stride(0), W.shape[0], W.shape[1], FS_LAYOUT_ROWS


def _check_inputs(H: torch.Tensor, W):
    if not (H.is_cuda and W.device.type == "cuda"):
        raise ValueError("H and W must be device tensors")
    if H.dim() != 2 or len(W.shape) != 2 or H.shape[1] != W.shape[1]:
        raise ValueError(f"H [B, D] and W [V, D] expected, got {tuple(H.shape)} and {tuple(W.shape)}")
    if H.dtype != W.dtype:
        raise ValueError("H and W must share a dtype")
    if H.stride(1) != 1 or (isinstance(W, torch.Tensor) and W.stride(1) != 1):
        raise ValueError("H and W rows must be contiguous")


def make_options(variant="auto", vocab_tile=0, logits=None, events=None, batch_tile=0,
                 layout=FS_LAYOUT_ROWS, single_pass=False, group_size=0) -> FsOptions:
    o = FsOptions()
    o.single_pass = int(bool(single_pass))
    o.group_size = int(group_size)
    o.variant = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    o.vocab_tile = int(vocab_tile)
    o.batch_tile = int(batch_tile)
    o.weights_layout = int(layout)
    if logits is not None:
        o.logits = logits.data_ptr()
        o.ld_logits = logits.stride(0)
        o.logits_dtype = _dtype_code(logits.dtype)
    if events is not None:
        o.stage1_start = events[0].cuda_event
        o.stage1_stop = events[1].cuda_event
    return o


def workspace_reset(workspace: torch.Tensor, stream=None) -> None:
    """Zeroes a workspace with the library's fill kernel (fs_workspace_reset)."""
    _check(_lib.fs_workspace_reset(workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "fs_workspace_reset")


def num_vocab_tiles(B, D, V, dtype=torch.bfloat16, variant="auto", vocab_tile=0, tiled=False) -> int:
    o = make_options(variant, vocab_tile, layout=FS_LAYOUT_TILED if tiled else FS_LAYOUT_ROWS)
    return int(_lib.fs_num_vocab_tiles(B, D, V, _dtype_code(dtype), ctypes.byref(o)))


def workspace_bytes(B, D, V, dtype=torch.bfloat16, variant="auto", vocab_tile=0, tiled=False,
                    single_pass=False, group_size=0, batch_tile=0) -> int:
    o = make_options(variant, vocab_tile, layout=FS_LAYOUT_TILED if tiled else FS_LAYOUT_ROWS,
                     single_pass=single_pass, group_size=group_size, batch_tile=batch_tile)
    return int(_lib.fs_workspace_bytes_ex(B, D, V, _dtype_code(dtype), ctypes.byref(o)))


def unfused_workspace_bytes(B, D, V, dtype=torch.bfloat16, logits_dtype=torch.bfloat16) -> int:
    return int(_lib.fs_unfused_workspace_bytes(B, D, V, _dtype_code(dtype), _dtype_code(logits_dtype)))


def sample_fused(H: torch.Tensor, W, temperature: float, seed: int, step: int,
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 variant="auto", vocab_tile: int = 0, logits: torch.Tensor | None = None,
                 events=None, stream=None, batch_tile: int = 0, single_pass: bool = False,
                 group_size: int = 0) -> torch.Tensor:
    """One token per row of H from softmax(H W^T / T) (Gumbel-max, fused).
    W is a row-major [V, D] tensor or a TiledWeights. With single_pass, a
    caller-provided workspace must have been zeroed once (workspace_reset).
    group_size > 0 selects the grouped variant (bf16; tiled weights, or
    row-major ones with D a multiple of 256): the group of group_size vocab
    entries is drawn from its log-mass, the token is that group's local
    Gumbel-max sample."""
    _check_inputs(H, W)
    B, D = H.shape
    wptr, ldw, V, _, layout = _weights(W)
    o = make_options(variant, vocab_tile, logits, events, batch_tile, layout, single_pass, group_size)
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=H.device)
    if workspace is None:
        nbytes = int(_lib.fs_workspace_bytes_ex(B, D, V, _dtype_code(H.dtype), ctypes.byref(o)))
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=H.device)
        if single_pass:
            workspace_reset(workspace, stream)
    st = _lib.fs_sample_fused_ex(H.data_ptr(), H.stride(0), wptr, ldw, _dtype_code(H.dtype), B, D, V,
                                 float(temperature), int(seed), int(step), workspace.data_ptr(),
                                 workspace.numel(), out.data_ptr(), _stream(stream), ctypes.byref(o))
    _check(st, "fs_sample_fused_ex")
    return out


# Bytes of the library's static per-GPU scratch array (FS_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 8 << 20


def sample_fused_noalloc(H: torch.Tensor, W, temperature: float, seed: int, step: int,
                         out: torch.Tensor | None = None, variant="auto", vocab_tile: int = 0,
                         logits: torch.Tensor | None = None, stream=None, batch_tile: int = 0,
                         single_pass: bool = False, group_size: int = 0) -> torch.Tensor:
    """sample_fused without a workspace (fs_sample_fused_noalloc): the library
    uses its static per-GPU scratch array instead, so the C call allocates
    nothing. Calls on one GPU must not overlap in time."""
    _check_inputs(H, W)
    B, D = H.shape
    wptr, ldw, V, _, layout = _weights(W)
    o = make_options(variant, vocab_tile, logits, None, batch_tile, layout, single_pass, group_size)
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=H.device)
    st = _lib.fs_sample_fused_noalloc(H.data_ptr(), H.stride(0), wptr, ldw, _dtype_code(H.dtype), B, D, V,
                                      float(temperature), int(seed), int(step), out.data_ptr(), _stream(stream),
                                      ctypes.byref(o))
    _check(st, "fs_sample_fused_noalloc")
    return out


def sample_unfused(H: torch.Tensor, W, temperature: float, seed: int, step: int,
                   logits_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None, stream=None, variant="auto",
                   vocab_tile: int = 0, batch_tile: int = 0) -> torch.Tensor:
    """The IO-model baseline: GEMM writes logits, a sampler kernel reads them."""
    _check_inputs(H, W)
    B, D = H.shape
    wptr, ldw, V, _, layout = _weights(W)
    o = make_options(variant, vocab_tile, None, None, batch_tile, layout)
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=H.device)
    if workspace is None:
        nbytes = unfused_workspace_bytes(B, D, V, H.dtype, logits_dtype)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=H.device)
    st = _lib.fs_sample_unfused_ex(H.data_ptr(), H.stride(0), wptr, ldw, _dtype_code(H.dtype), B, D, V,
                                   float(temperature), int(seed), int(step), _dtype_code(logits_dtype),
                                   workspace.data_ptr(), workspace.numel(), out.data_ptr(), _stream(stream),
                                   ctypes.byref(o))
    _check(st, "fs_sample_unfused_ex")
    return out


def test_philox(seed: int, step: int, b: int, v0: int, n: int, device="cuda") -> torch.Tensor:
    out = torch.empty(n, dtype=torch.int32, device=device)
    _check(_lib.fs_test_philox(seed, step, b, v0, n, out.data_ptr(), _stream(None)), "fs_test_philox")
    return out


def test_gumbel(words: torch.Tensor) -> torch.Tensor:
    assert words.dtype == torch.int32 and words.is_cuda and words.is_contiguous()
    out = torch.empty(words.numel(), dtype=torch.float32, device=words.device)
    _check(_lib.fs_test_gumbel(words.data_ptr(), words.numel(), out.data_ptr(), _stream(None)),
           "fs_test_gumbel")
    return out


def probe_read(src: torch.Tensor, chunk_bytes: int = 1 << 19, sink: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """Streams all bytes of a contiguous device tensor (see fs_probe_read)."""
    assert src.is_cuda and src.is_contiguous()
    nbytes = src.numel() * src.element_size()
    nblk = int(_lib.fs_probe_read_blocks(nbytes, chunk_bytes))
    if nblk < 0:
        raise ValueError("probe_read: bytes and chunk must be positive multiples of 16")
    if sink is None:
        sink = torch.empty(nblk, dtype=torch.int32, device=src.device)
    _check(_lib.fs_probe_read(src.data_ptr(), nbytes, chunk_bytes, sink.data_ptr(), _stream(stream)),
           "fs_probe_read")
    return sink
