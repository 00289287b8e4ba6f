"""ctypes binding of libmla (include/mla.h): argument marshalling only.

Every step of the decode runs in the HIP kernels of libmla.so; this module
turns torch tensors into the mla_tensor descriptors of the C ABI and raises
MlaError on a non-OK status.  Shapes, dtypes and strides are checked by the
library itself; the binding only makes sure that what it hands over is device
memory (a host pointer would reach the GPU).  Importing it fails loudly when
the library has not been built.
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
MLA_ERR_SCRATCH = 7
NOALLOC_MAX_SPLIT_TOKENS = 256

# element types (mla_dtype)
MLA_DTYPE_BF16 = 0
MLA_DTYPE_FP32 = 1
MLA_DTYPE_INT32 = 2
MLA_DTYPE_FP8_E4M3 = 3
MLA_DTYPE_UINT8 = 4

# latent cache kinds of LatentCache
MLA_CACHE_BF16 = 0
MLA_CACHE_FP8_E4M3 = 1

NUM_HEADS = 128
LATENT_DIM = 512
ROPE_DIM = 64
ROW_DIM = 576
BLOCK_SIZE = 64
MAX_RANK = 5

# every symbol include/mla.h declares
EXPORTED_SYMBOLS = ("mla_decode", "mla_combine", "mla_decode_noalloc", "mla_num_splits_hint",
                    "mla_partial_out_bytes", "mla_partial_lse_bytes", "mla_absorb_query", "mla_absorb_output",
                    "mla_kv_project", "mla_kv_project_split", "mla_kv_project_splits", "mla_cache_append",
                    "mla_check_indices", "mla_init",
                    "mla_status_string", "mla_version")
ROPE_BASE = 10000.0


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class MlaTensor(ctypes.Structure):
    """Mirror of struct mla_tensor."""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("shape", ctypes.c_int64 * MAX_RANK), ("strides", ctypes.c_int64 * MAX_RANK)]


class MlaLatentCache(ctypes.Structure):
    """Mirror of struct mla_latent_cache."""
    _fields_ = [("rows", MlaTensor), ("scales", MlaTensor), ("rope", MlaTensor)]


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
    T, C = ctypes.POINTER(MlaTensor), ctypes.POINTER(MlaLatentCache)
    lib.mla_decode.restype = i32
    lib.mla_decode.argtypes = [T, T, C, T, T, f32, T, T, T, T, vp]
    lib.mla_combine.restype = i32
    lib.mla_combine.argtypes = [T, T, T, T, T, vp]
    lib.mla_decode_noalloc.restype = i32
    lib.mla_decode_noalloc.argtypes = [T, T, C, T, T, f32, T, T, i32, vp]
    lib.mla_absorb_query.restype = i32
    lib.mla_absorb_query.argtypes = [T, T, T, T, f32, T, T, vp]
    lib.mla_absorb_output.restype = i32
    lib.mla_absorb_output.argtypes = [T, T, T, vp]
    lib.mla_kv_project.restype = i32
    lib.mla_kv_project.argtypes = [T, T, T, vp]
    lib.mla_kv_project_split.restype = i32
    lib.mla_kv_project_split.argtypes = [T, T, T, T, vp]
    lib.mla_kv_project_splits.restype = i32
    lib.mla_kv_project_splits.argtypes = [ctypes.c_int64, ctypes.c_int64]
    lib.mla_cache_append.restype = i32
    lib.mla_cache_append.argtypes = [T, T, T, C, f32, vp]
    lib.mla_check_indices.restype = i32
    lib.mla_check_indices.argtypes = [C, T, T, T, vp]
    lib.mla_init.restype = i32
    lib.mla_init.argtypes = [i32]
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


def mla_init(device: int = 0) -> None:
    """Load the library's code object on `device` now (see include/mla.h)."""
    st = _lib.mla_init(int(device))
    if st != MLA_OK:
        raise MlaError(st, "mla_init")


# ------------------------------------------------------------------ tensors
_DTYPE_CODES = None


def _dtype_code(t) -> int:
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch
        codes = {torch.bfloat16: MLA_DTYPE_BF16, torch.float32: MLA_DTYPE_FP32, torch.int32: MLA_DTYPE_INT32,
                 torch.uint8: MLA_DTYPE_UINT8}
        if hasattr(torch, "float8_e4m3fn"):
            codes[torch.float8_e4m3fn] = MLA_DTYPE_FP8_E4M3
        _DTYPE_CODES = codes
    # any other element type goes through with a code the library rejects (MLA_ERR_DTYPE)
    return _DTYPE_CODES.get(t.dtype, 255)


def tensor(t, dtype: Optional[int] = None, device_only: bool = True) -> MlaTensor:
    """The mla_tensor of a torch tensor (None -> an empty descriptor).  dtype
    overrides the element type code (e4m3 codes held in a uint8 tensor).
    Built with one constructor call: a launch marshals ten of these, and
    field-by-field assignment cost more host time than a short kernel."""
    if t is None:
        return MlaTensor()
    if device_only and not t.is_cuda:
        raise ValueError(f"tensor on {t.device} passed to libmla: device tensors only")
    shape = tuple(t.shape)
    n = len(shape)
    if n > MAX_RANK:
        raise ValueError(f"rank {n} above {MAX_RANK}")
    pad = (0,) * (MAX_RANK - n)
    return MlaTensor(t.data_ptr() or None, _dtype_code(t) if dtype is None else int(dtype), n,
                     shape + pad, tuple(t.stride()) + pad)


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream) or None
    if isinstance(stream, int):
        return stream or None
    return int(stream.cuda_stream) or None


def _ref(d: MlaTensor):
    return None if d.data is None and d.rank == 0 else ctypes.byref(d)


@dataclass
class LatentCache:
    """Device-resident latent cache: bf16 rows [NB, 64, 576], or the e4m3
    bundle (codes [NB, 64, 512] as uint8 or float8_e4m3fn, fp32 scales
    [NB, 64, 4], bf16 rope [NB, 64, 64]).  A contiguous cache (no block table)
    is [B * max_blocks, 64, .] or [B, L_cap, .]."""
    dtype: int
    rows: object
    scales: object = None
    rope: object = None

    @property
    def num_blocks(self) -> int:
        return int(self.rows.shape[0])

    def desc(self) -> MlaLatentCache:
        c = MlaLatentCache()
        fp8 = self.dtype == MLA_CACHE_FP8_E4M3
        c.rows = tensor(self.rows, MLA_DTYPE_FP8_E4M3 if fp8 else None)
        c.scales = tensor(self.scales)
        c.rope = tensor(self.rope)
        return c


def mla_decode(q_absorbed, q_rope, cache: LatentCache, block_table, seq_lens, scale: float, out_latent, lse,
               partial_out=None, partial_lse=None, stream=None) -> None:
    """Enqueue mla_decode (see include/mla.h) on `stream` (default: torch's
    current stream).  The split count is partial_lse's leading dimension (1
    without partials)."""
    c = cache.desc()
    args = [tensor(q_absorbed), tensor(q_rope), c, tensor(block_table), tensor(seq_lens), tensor(out_latent),
            tensor(lse), tensor(partial_out), tensor(partial_lse)]
    st = _lib.mla_decode(_ref(args[0]), _ref(args[1]), ctypes.byref(c), _ref(args[3]), _ref(args[4]),
                         float(scale), _ref(args[5]), _ref(args[6]), _ref(args[7]), _ref(args[8]),
                         _stream_handle(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode")


class PreparedStep:
    """One decode step (mla_decode, then mla_combine) with its descriptors
    built once, for a loop that launches on the same buffers every step:
    their contents may change between launches, their addresses, shapes
    and dtypes may not.  Each launch then costs two foreign calls instead of
    marshalling a dozen descriptors (tens of microseconds of host time,
    longer than a short decode).  The library still validates every call."""

    def __init__(self, q_absorbed, q_rope, cache: LatentCache, block_table, seq_lens, scale: float, out_latent,
                 lse, partial_out=None, partial_lse=None):
        self._tensors = (q_absorbed, q_rope, cache, block_table, seq_lens, out_latent, lse, partial_out,
                         partial_lse)   # kept alive while the descriptors point at them
        self._cache = cache.desc()
        self._desc = [tensor(x) for x in (q_absorbed, q_rope, block_table, seq_lens, out_latent, lse,
                                          partial_out, partial_lse)]
        qa, qr, bt, sl, out, ls, po, pl = [_ref(d) for d in self._desc]
        self._decode_args = (qa, qr, ctypes.byref(self._cache), bt, sl, ctypes.c_float(scale), out, ls, po, pl)
        self._combine_args = (po, pl, sl, out, ls)

    def __call__(self, stream=None) -> None:
        """Enqueue the step on `stream` (default: torch's current stream)."""
        s = _stream_handle(stream)
        st = _lib.mla_decode(*self._decode_args, s)
        if st != MLA_OK:
            raise MlaError(st, "mla_decode")
        st = _lib.mla_combine(*self._combine_args, s)
        if st != MLA_OK:
            raise MlaError(st, "mla_combine")

    def decode(self, stream=None) -> None:
        """Enqueue mla_decode alone."""
        st = _lib.mla_decode(*self._decode_args, _stream_handle(stream))
        if st != MLA_OK:
            raise MlaError(st, "mla_decode")


def mla_decode_noalloc(q_absorbed, q_rope, cache: LatentCache, block_table, seq_lens, scale: float, out_latent,
                       lse, num_splits: int, stream=None) -> None:
    """Enqueue mla_decode_noalloc (decode + combine with the library's static
    scratch for the partials; see include/mla.h)."""
    c = cache.desc()
    args = [tensor(q_absorbed), tensor(q_rope), c, tensor(block_table), tensor(seq_lens), tensor(out_latent),
            tensor(lse)]
    st = _lib.mla_decode_noalloc(_ref(args[0]), _ref(args[1]), ctypes.byref(c), _ref(args[3]), _ref(args[4]),
                                 float(scale), _ref(args[5]), _ref(args[6]), int(num_splits),
                                 _stream_handle(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_noalloc")


def mla_combine(partial_out, partial_lse, seq_lens, out_latent, lse, stream=None) -> None:
    """Enqueue mla_combine (see include/mla.h)."""
    args = [tensor(partial_out), tensor(partial_lse), tensor(seq_lens), tensor(out_latent), tensor(lse)]
    st = _lib.mla_combine(*[_ref(a) for a in args], _stream_handle(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_combine")


def mla_check_indices(cache: LatentCache, block_table, seq_lens, counts, stream=None) -> None:
    """Enqueue mla_check_indices: counts (int32 [2], device) <- bad lengths,
    bad block-table entries."""
    c = cache.desc()
    args = [tensor(block_table), tensor(seq_lens), tensor(counts)]
    st = _lib.mla_check_indices(ctypes.byref(c), *[_ref(a) for a in args], _stream_handle(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_check_indices")


def mla_absorb_query(q_c, q_r, w_uk_t, seq_lens, q_absorbed, q_rope, rope_base: float = ROPE_BASE,
                     stream=None) -> None:
    """Enqueue mla_absorb_query: q_absorbed = W^UK_h^T q^C_h, q_rope = RoPE(q^R, position)."""
    args = [tensor(x) for x in (q_c, q_r, w_uk_t, seq_lens)] + [tensor(q_absorbed), tensor(q_rope)]
    st = _lib.mla_absorb_query(*[_ref(a) for a in args[:4]], float(rope_base), _ref(args[4]), _ref(args[5]),
                               _stream_handle(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_absorb_query")


def mla_absorb_output(out_latent, w_uv, out_values, stream=None) -> None:
    """Enqueue mla_absorb_output: out_values = W^UV_h out_latent_h per head."""
    args = [tensor(out_latent), tensor(w_uv), tensor(out_values)]
    st = _lib.mla_absorb_output(*[_ref(a) for a in args], _stream_handle(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_absorb_output")


def mla_kv_project(hidden, w_kv, kv, stream=None) -> None:
    """Enqueue mla_kv_project: kv = [W^DKV ; W^KR] hidden (fp32)."""
    args = [tensor(hidden), tensor(w_kv), tensor(kv)]
    st = _lib.mla_kv_project(*[_ref(a) for a in args], _stream_handle(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_kv_project")


def mla_kv_project_splits(tokens: int, d: int) -> int:
    """The slice count mla_kv_project_split fills the GPU with (0: shape not taken)."""
    return int(_lib.mla_kv_project_splits(int(tokens), int(d)))


def mla_kv_project_split(hidden, w_kv, kv, workspace, stream=None) -> None:
    """Enqueue mla_kv_project_split: kv as mla_kv_project, K cut into workspace.shape[0] slices
    (workspace: fp32 [S, T, 576], overwritten)."""
    args = [tensor(hidden), tensor(w_kv), tensor(kv), tensor(workspace)]
    st = _lib.mla_kv_project_split(*[_ref(a) for a in args], _stream_handle(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_kv_project_split")


def mla_cache_append(kv, seq_lens, block_table, cache: LatentCache, rope_base: float = ROPE_BASE,
                     stream=None) -> None:
    """Enqueue mla_cache_append: each new token's row into its page slot (bf16 or e4m3)."""
    c = cache.desc()
    args = [tensor(kv), tensor(seq_lens), tensor(block_table)]
    st = _lib.mla_cache_append(*[_ref(a) for a in args], ctypes.byref(c), float(rope_base), _stream_handle(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_cache_append")
