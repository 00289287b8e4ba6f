"""ctypes binding of libmla (include/mla.h): argument marshalling only.

Every step of the decode runs in the HIP kernels of libmla.so; this module
turns torch tensors into the pointers and sizes of the C ABI and raises
MlaError on a non-OK status.  Importing it fails loudly when the library has
not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")

# status codes (mla_status)
MLA_OK = 0
MLA_ERR_NULL = 1
MLA_ERR_DTYPE = 2
MLA_ERR_SHAPE = 3
MLA_ERR_UNSUPPORTED = 4
MLA_ERR_LAUNCH = 5
MLA_ERR_DEVICE = 6

MLA_CACHE_BF16 = 0
MLA_CACHE_FP8_E4M3 = 1

NUM_HEADS = 128
LATENT_DIM = 512
ROPE_DIM = 64
ROW_DIM = 576
BLOCK_SIZE = 64

# every symbol include/mla.h declares
EXPORTED_SYMBOLS = ("mla_decode", "mla_combine", "mla_num_splits_hint", "mla_partial_out_bytes",
                    "mla_partial_lse_bytes", "mla_status_string", "mla_version")


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class LatentCacheDesc(ctypes.Structure):
    """Mirror of struct mla_latent_cache."""
    _fields_ = [("dtype", ctypes.c_int32), ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int64),
                ("rows", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("rope", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmla.so is not built at {LIB_PATH}; run __graft_entry__.build() "
                          "or python mla_latent_kv_39_amd/build_lib.py")
    # torch first: its HIP runtime is then the one libmla.so binds to.  Loaded
    # the other way round the process holds two HIP runtimes, and the tensors
    # of one are not valid in the other.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.mla_decode.restype = i32
    lib.mla_decode.argtypes = [vp, vp, ctypes.POINTER(LatentCacheDesc), vp, i32, vp, i32, i32, f32, i32,
                               vp, vp, vp, vp, vp]
    lib.mla_combine.restype = i32
    lib.mla_combine.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp]
    lib.mla_num_splits_hint.restype = i32
    lib.mla_num_splits_hint.argtypes = [i32, i32, i32, i32]
    lib.mla_partial_out_bytes.restype = sz
    lib.mla_partial_out_bytes.argtypes = [i32, i32]
    lib.mla_partial_lse_bytes.restype = sz
    lib.mla_partial_lse_bytes.argtypes = [i32, i32]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [i32]
    lib.mla_version.restype = i32
    lib.mla_version.argtypes = []
    return lib


_lib = _load()


def library():
    """The loaded ctypes CDLL."""
    return _lib


def status_string(status: int) -> str:
    return _lib.mla_status_string(int(status)).decode()


def mla_version() -> int:
    return int(_lib.mla_version())


def mla_num_splits_hint(device: int, batch: int, s_q: int, max_blocks_per_seq: int = 0) -> int:
    return int(_lib.mla_num_splits_hint(int(device), int(batch), int(s_q), int(max_blocks_per_seq)))


def mla_partial_out_bytes(num_splits: int, s_q: int) -> int:
    return int(_lib.mla_partial_out_bytes(int(num_splits), int(s_q)))


def mla_partial_lse_bytes(num_splits: int, s_q: int) -> int:
    return int(_lib.mla_partial_lse_bytes(int(num_splits), int(s_q)))


# ------------------------------------------------------------------ tensors
def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream) or None
    if isinstance(stream, int):
        return stream or None
    return int(stream.cuda_stream) or None


def _need(t, dtype, shape, name):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    return t


@dataclass
class LatentCache:
    """Device-resident latent cache: bf16 rows [NB, 64, 576], or the fp8 bundle
    (e4m3 bytes [NB, 64, 512] as uint8, fp32 scales [NB, 64, 4], bf16 rope [NB, 64, 64])."""
    dtype: int
    rows: object
    scales: object = None
    rope: object = None

    @property
    def num_blocks(self) -> int:
        return int(self.rows.shape[0])

    def desc(self) -> LatentCacheDesc:
        return LatentCacheDesc(int(self.dtype), int(self.rows.shape[1]), self.num_blocks, _ptr(self.rows),
                               _ptr(self.scales), _ptr(self.rope))


def mla_decode(q_absorbed, q_rope, cache: LatentCache, block_table, seq_lens, scale: float, num_splits: int,
               partial_out, partial_lse, out_latent, lse, max_blocks_per_seq: Optional[int] = None,
               stream=None) -> None:
    """Enqueue mla_decode (see include/mla.h) on `stream` (default: torch's current stream)."""
    import torch
    B, S = int(q_absorbed.shape[0]), int(q_absorbed.shape[1])
    _need(q_absorbed, torch.bfloat16, (B, S, NUM_HEADS, LATENT_DIM), "q_absorbed")
    _need(q_rope, torch.bfloat16, (B, S, NUM_HEADS, ROPE_DIM), "q_rope")
    _need(seq_lens, torch.int32, (B,), "seq_lens")
    _need(out_latent, torch.float32, (B, S, NUM_HEADS, LATENT_DIM), "out_latent")
    _need(lse, torch.float32, (B, S, NUM_HEADS), "lse")
    if block_table is not None:
        _need(block_table, torch.int32, tuple(block_table.shape), "block_table")
        mb = int(block_table.shape[1])
    else:
        if max_blocks_per_seq is None:
            raise ValueError("max_blocks_per_seq is required for a contiguous cache")
        mb = int(max_blocks_per_seq)
    if num_splits > 1:
        _need(partial_out, torch.uint8, (mla_partial_out_bytes(num_splits, S),), "partial_out")
        _need(partial_lse, torch.float32, (num_splits, 2, S, NUM_HEADS), "partial_lse")
    d = cache.desc()
    st = _lib.mla_decode(_ptr(q_absorbed), _ptr(q_rope), ctypes.byref(d), _ptr(block_table), mb, _ptr(seq_lens),
                         B, S, float(scale), int(num_splits), _ptr(partial_out), _ptr(partial_lse),
                         _ptr(out_latent), _ptr(lse), _stream_handle(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode")


def mla_combine(partial_out, partial_lse, seq_lens, num_splits: int, out_latent, lse, stream=None) -> None:
    """Enqueue mla_combine (see include/mla.h)."""
    import torch
    B, S = int(out_latent.shape[0]), int(out_latent.shape[1])
    if int(num_splits) > 1:
        _need(partial_out, torch.uint8, (mla_partial_out_bytes(num_splits, S),), "partial_out")
        _need(partial_lse, torch.float32, (num_splits, 2, S, NUM_HEADS), "partial_lse")
    _need(seq_lens, torch.int32, (B,), "seq_lens")
    _need(out_latent, torch.float32, (B, S, NUM_HEADS, LATENT_DIM), "out_latent")
    _need(lse, torch.float32, (B, S, NUM_HEADS), "lse")
    st = _lib.mla_combine(_ptr(partial_out), _ptr(partial_lse), _ptr(seq_lens), B, S, int(num_splits),
                          _ptr(out_latent), _ptr(lse), _stream_handle(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_combine")
