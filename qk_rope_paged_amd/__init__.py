"""Python binding of the qk_rope_paged C ABI (include/qk_rope_paged.h).

Argument marshalling only: every step of the pass runs in the HIP library
``libqk_rope_paged.so`` that sits next to this file.  Importing the package
fails loudly when that library is missing; there is no fallback path.

Tensors are torch tensors on the GPU (any dtype whose storage holds the
right bits: bfloat16 / int16 / uint16 for bf16 data, float32 / int32 for
fp32).  Streams default to torch's current stream.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqk_rope_paged.so")

QRP_OK, QRP_EINVAL, QRP_EALIGN, QRP_EUNSUPPORTED, QRP_EGEOMETRY, QRP_EHIP, QRP_EDATA = (
    0, -1, -2, -3, -4, -5, -6)
QRP_F32, QRP_BF16, QRP_F16, QRP_FP8 = 0, 1, 2, 3
STATUS_NAMES = {0: "QRP_OK", -1: "QRP_EINVAL", -2: "QRP_EALIGN", -3: "QRP_EUNSUPPORTED",
                -4: "QRP_EGEOMETRY", -5: "QRP_EHIP", -6: "QRP_EDATA"}

# entry points declared in include/qk_rope_paged.h
EXPORTS = ("rope_split_store_paged", "qk_rmsnorm_rope_paged", "dual_band", "kv_cache_radd",
           "fused_qk_rope_bshd_continuous_batch", "matmul_fused_partial_rmsnorm",
           "matmul_fused_partial_rmsnorm_noalloc",
           "qrp_gemv_norm_workspace_bytes", "qrp_validate", "qrp_validate_host",
           "qrp_last_error", "qrp_abi_version", "qrp_set_launch_override")


class QrpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class QrpPagedCache(ctypes.Structure):
    _fields_ = [("blocks", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_uint32), ("head_dim", ctypes.c_uint32),
                ("page_size", ctypes.c_uint32), ("num_layers", ctypes.c_uint32),
                ("kv_planes", ctypes.c_uint32), ("num_pages", ctypes.c_uint64),
                ("page_stride", ctypes.c_int64), ("plane_stride", ctypes.c_int64),
                ("layer_stride", ctypes.c_int64), ("slot_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64),
                ("cache_lengths", ctypes.c_void_p), ("lookup_table", ctypes.c_void_p),
                ("cache_batch", ctypes.c_uint32), ("max_pages_per_seq", ctypes.c_uint32),
                ("scales", ctypes.c_void_p), ("scale_dtype", ctypes.c_int32),
                ("scale_page_stride", ctypes.c_int64), ("scale_plane_stride", ctypes.c_int64),
                ("scale_layer_stride", ctypes.c_int64), ("scale_slot_stride", ctypes.c_int64),
                ("scale_head_stride", ctypes.c_int64)]


class QrpRope(ctypes.Structure):
    _fields_ = [("freqs_cis", ctypes.c_void_p), ("freq_dtype", ctypes.c_int32),
                ("max_seq_len", ctypes.c_uint32), ("rope_dim", ctypes.c_uint32),
                ("interleaved", ctypes.c_int32), ("rope_tail", ctypes.c_int32)]


class QrpBand(ctypes.Structure):
    _fields_ = [("q_col", ctypes.c_uint64), ("n_q_heads", ctypes.c_uint32),
                ("k_col", ctypes.c_int64), ("v_col", ctypes.c_int64),
                ("q_gamma", ctypes.c_void_p), ("k_gamma", ctypes.c_void_p),
                ("epsilon", ctypes.c_float), ("cache", ctypes.POINTER(QrpPagedCache)),
                ("q_output", ctypes.c_void_p), ("q_out_row_stride", ctypes.c_uint64)]


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    # One HIP runtime per process: PyTorch-ROCm ships its own libamdhip64
    # (same soname as the system one it was not linked by name against), so
    # torch is loaded first and the library then binds to that runtime.
    # Loading the library first would leave two runtimes in the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python qk_rope_paged_amd/build.py` "
            "(or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(path)
    P, U32, U64, I32, F = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32, ctypes.c_float
    PC, PR, PB = ctypes.POINTER(QrpPagedCache), ctypes.POINTER(QrpRope), ctypes.POINTER(QrpBand)
    sig = {
        "rope_split_store_paged": [P, I32, U32, U64, U32, P, U32, PR, PC, U32, P, I32, U64, P],
        "qk_rmsnorm_rope_paged": [P, I32, U32, U64, PB, F, I32, P, U32, PR, U32, P],
        "dual_band": [P, I32, U32, U64, PB, PB, F, I32, P, U32, PR, U32, P],
        "kv_cache_radd": [P, I32, U32, U64, P, U32, U32, PC, U32, P],
        "fused_qk_rope_bshd_continuous_batch": [P, I32, U32, U32, U32, P, PR, PC, U32, P, P],
        "matmul_fused_partial_rmsnorm": [P, U64, P, U64, P, U64, U32, P, U64, U32, U32, P, U32,
                                         F, F, I32, I32, P, U64, P],
        "matmul_fused_partial_rmsnorm_noalloc": [P, U64, P, U64, P, U64, U32, P, U64, U32, U32,
                                                 P, U32, F, F, I32, I32, P],
        "qrp_validate": [P, U32, U32, U32, PC, U32, P],
        "qrp_validate_host": [P, U32, U32, U32, P, P, U32, U32, U32, U64, U32],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = I32
    lib.qrp_last_error.argtypes = []
    lib.qrp_last_error.restype = ctypes.c_char_p
    lib.qrp_gemv_norm_workspace_bytes.argtypes = [U32, U32, I32]
    lib.qrp_gemv_norm_workspace_bytes.restype = U64
    lib.qrp_abi_version.argtypes = []
    lib.qrp_abi_version.restype = I32
    lib.qrp_set_launch_override.argtypes = [I32, I32, ctypes.POINTER(I32)]
    lib.qrp_set_launch_override.restype = I32
    return lib


lib = _load()


def last_error() -> str:
    return lib.qrp_last_error().decode()


# launch-shape knobs (include/qk_rope_paged.h: qrp_set_launch_override)
QRP_KNOB_PACK, QRP_KNOB_PASSES_PER_WAVE, QRP_KNOB_WAVES_PER_BLOCK, QRP_KNOB_XCD_REMAP = 0, 1, 2, 3
QRP_KNOB_TAIL_UNITS, QRP_KNOB_LDS_BYTES = 4, 5
_KNOBS = {"pack": QRP_KNOB_PACK, "passes_per_wave": QRP_KNOB_PASSES_PER_WAVE,
          "waves_per_block": QRP_KNOB_WAVES_PER_BLOCK, "xcd_remap": QRP_KNOB_XCD_REMAP,
          "tail_units": QRP_KNOB_TAIL_UNITS, "lds_bytes": QRP_KNOB_LDS_BYTES}


def set_launch_override(knob: int, value: int) -> int:
    """Set one launch-shape knob (-1: the library's choice); returns the old value."""
    prev = ctypes.c_int32(0)
    _check(lib.qrp_set_launch_override(knob, value, ctypes.byref(prev)), True)
    return prev.value


class launch_overrides:
    """Context manager: ``with launch_overrides(pack=1, passes_per_wave=2): ...``
    sets the named knobs (None or -1: the library's choice) and restores
    their old values on exit."""

    def __init__(self, **knobs):
        unknown = set(knobs) - set(_KNOBS)
        if unknown:
            raise ValueError(f"unknown launch knobs {sorted(unknown)}")
        self._set = {_KNOBS[k]: (-1 if v is None else int(v)) for k, v in knobs.items()}
        self._old = {}

    def __enter__(self):
        for k, v in self._set.items():
            self._old[k] = set_launch_override(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self._old.items():
            set_launch_override(k, v)
        return False


def _check(status: int, raise_on_error: bool) -> int:
    if status != QRP_OK and raise_on_error:
        raise QrpError(status, last_error())
    return status


class PreparedCall:
    """A library call with its arguments marshalled once (``prepare=True``):
    calling it costs one ctypes call, for tight launch loops."""

    def __init__(self, fn, args, keep, raise_on_error):
        self._fn, self._args, self._keep, self._raise = fn, args, keep, raise_on_error

    def __call__(self) -> int:
        return _check(self._fn(*self._args), self._raise)


def _call(fn, args, keep, raise_on_error, prepare):
    if prepare:
        return PreparedCall(fn, args, keep, raise_on_error)
    return _check(fn(*args), raise_on_error)


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclass
class PagedCache:
    """A paged K/V cache: device pool + metadata, with element strides.

    ``blocks`` is the pool tensor; ``cache_lengths`` ([cache_batch]) and
    ``lookup_table`` ([cache_batch, max_pages_per_seq]) are uint32 data held
    in int32 tensors.  ``to_c()`` gives the C struct."""
    blocks: object
    dtype: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_layers: int
    kv_planes: int
    num_pages: int
    page_stride: int
    plane_stride: int
    layer_stride: int
    slot_stride: int
    head_stride: int
    cache_lengths: object
    lookup_table: object
    cache_batch: int
    max_pages_per_seq: int
    scales: object = None            # QRP_FP8 caches: one scale per row
    scale_dtype: int = QRP_F32
    scale_page_stride: int = 0
    scale_plane_stride: int = 0
    scale_layer_stride: int = 0
    scale_slot_stride: int = 0
    scale_head_stride: int = 0

    def to_c(self) -> QrpPagedCache:
        return QrpPagedCache(
            blocks=_ptr(self.blocks), dtype=self.dtype, num_kv_heads=self.num_kv_heads,
            head_dim=self.head_dim, page_size=self.page_size, num_layers=self.num_layers,
            kv_planes=self.kv_planes, num_pages=self.num_pages, page_stride=self.page_stride,
            plane_stride=self.plane_stride, layer_stride=self.layer_stride,
            slot_stride=self.slot_stride, head_stride=self.head_stride,
            cache_lengths=_ptr(self.cache_lengths), lookup_table=_ptr(self.lookup_table),
            cache_batch=self.cache_batch, max_pages_per_seq=self.max_pages_per_seq,
            scales=_ptr(self.scales), scale_dtype=self.scale_dtype,
            scale_page_stride=self.scale_page_stride, scale_plane_stride=self.scale_plane_stride,
            scale_layer_stride=self.scale_layer_stride, scale_slot_stride=self.scale_slot_stride,
            scale_head_stride=self.scale_head_stride)


@dataclass
class Rope:
    freqs_cis: object        # [max_seq_len, rope_dim] of freq_dtype (float32 or bf16 words)
    max_seq_len: int
    rope_dim: int
    interleaved: bool
    freq_dtype: int = QRP_F32
    rope_tail: bool = False          # rotate the last rope_dim dims of a head

    def to_c(self) -> QrpRope:
        return QrpRope(freqs_cis=_ptr(self.freqs_cis), freq_dtype=self.freq_dtype,
                       max_seq_len=self.max_seq_len, rope_dim=self.rope_dim,
                       interleaved=int(bool(self.interleaved)),
                       rope_tail=int(bool(self.rope_tail)))


@dataclass
class Band:
    q_col: int
    n_q_heads: int
    k_col: int
    v_col: int
    q_gamma: object
    k_gamma: object
    epsilon: float
    cache: PagedCache
    q_output: object
    q_out_row_stride: int

    def to_c(self, keep: list) -> QrpBand:
        cc = self.cache.to_c()
        keep.append(cc)
        return QrpBand(q_col=self.q_col, n_q_heads=self.n_q_heads, k_col=self.k_col,
                       v_col=self.v_col, q_gamma=_ptr(self.q_gamma), k_gamma=_ptr(self.k_gamma),
                       epsilon=self.epsilon, cache=ctypes.pointer(cc), q_output=_ptr(self.q_output),
                       q_out_row_stride=self.q_out_row_stride)


def rope_split_store_paged(qkv, dtype: int, total_seq_len: int, qkv_row_stride: int,
                           n_q_heads: int, input_row_offsets, batch_size: int, rope: Rope,
                           cache: PagedCache, layer_idx: int, q_output, q_out_dtype: int,
                           q_out_row_stride: int, stream=None, raise_on_error: bool = True,
                           prepare: bool = False):
    cr, cc = rope.to_c(), cache.to_c()
    args = (_ptr(qkv), dtype, total_seq_len, qkv_row_stride, n_q_heads, _ptr(input_row_offsets),
            batch_size, ctypes.byref(cr), ctypes.byref(cc), layer_idx, _ptr(q_output),
            q_out_dtype, q_out_row_stride, _stream(stream))
    return _call(lib.rope_split_store_paged, args, [cr, cc], raise_on_error, prepare)


def qk_rmsnorm_rope_paged(qkv, dtype: int, total_seq_len: int, qkv_row_stride: int, band: Band,
                          weight_offset: float, multiply_before_cast: bool, input_row_offsets,
                          batch_size: int, rope: Rope, layer_idx: int, stream=None,
                          raise_on_error: bool = True, prepare: bool = False):
    keep: list = []
    cb, cr = band.to_c(keep), rope.to_c()
    args = (_ptr(qkv), dtype, total_seq_len, qkv_row_stride, ctypes.byref(cb), weight_offset,
            int(bool(multiply_before_cast)), _ptr(input_row_offsets), batch_size,
            ctypes.byref(cr), layer_idx, _stream(stream))
    return _call(lib.qk_rmsnorm_rope_paged, args, keep + [cb, cr], raise_on_error, prepare)


def dual_band(buf, dtype: int, total_seq_len: int, buf_row_stride: int, main_band: Band,
              index_band: Band, weight_offset: float, multiply_before_cast: bool,
              input_row_offsets, batch_size: int, rope: Rope, layer_idx: int, stream=None,
              raise_on_error: bool = True, prepare: bool = False):
    keep: list = []
    cm, ci, cr = main_band.to_c(keep), index_band.to_c(keep), rope.to_c()
    args = (_ptr(buf), dtype, total_seq_len, buf_row_stride, ctypes.byref(cm), ctypes.byref(ci),
            weight_offset, int(bool(multiply_before_cast)), _ptr(input_row_offsets), batch_size,
            ctypes.byref(cr), layer_idx, _stream(stream))
    return _call(lib.dual_band, args, keep + [cm, ci, cr], raise_on_error, prepare)


def kv_cache_radd(a, dtype: int, total_rows: int, a_row_stride: int, input_row_offsets,
                  batch_size: int, batch_offset: int, cache: PagedCache, layer_idx: int,
                  stream=None, raise_on_error: bool = True, prepare: bool = False):
    cc = cache.to_c()
    args = (_ptr(a), dtype, total_rows, a_row_stride, _ptr(input_row_offsets), batch_size,
            batch_offset, ctypes.byref(cc), layer_idx, _stream(stream))
    return _call(lib.kv_cache_radd, args, [cc], raise_on_error, prepare)


def fused_qk_rope_bshd_continuous_batch(q_proj, dtype: int, batch_size: int, seq_len: int,
                                        n_q_heads: int, valid_lengths, rope: Rope,
                                        cache: PagedCache, layer_idx: int, output, stream=None,
                                        raise_on_error: bool = True, prepare: bool = False):
    cc, rc = cache.to_c(), rope.to_c()
    args = (_ptr(q_proj), dtype, batch_size, seq_len, n_q_heads, _ptr(valid_lengths),
            ctypes.byref(rc), ctypes.byref(cc), layer_idx, _ptr(output), _stream(stream))
    return _call(lib.fused_qk_rope_bshd_continuous_batch, args, [cc, rc], raise_on_error, prepare)


def gemv_norm_workspace_bytes(m: int, n_normed: int, transpose_b: int = 1) -> int:
    return int(lib.qrp_gemv_norm_workspace_bytes(m, n_normed, transpose_b))


def matmul_fused_partial_rmsnorm(normed_output, normed_row_stride: int, unnormed_output,
                                 unnormed_row_stride: int, input, input_row_stride: int, m: int,
                                 weight, weight_row_stride: int, n: int, k: int, gamma,
                                 n_normed: int, epsilon: float, weight_offset: float, dtype: int,
                                 workspace, workspace_bytes: int, transpose_b: int = 1,
                                 stream=None, raise_on_error: bool = True, prepare: bool = False):
    """The fused GEMV + partial RMSNorm; `workspace` is a zero-filled device
    buffer of at least gemv_norm_workspace_bytes(m, n_normed, transpose_b)
    bytes."""
    args = (_ptr(normed_output), normed_row_stride, _ptr(unnormed_output), unnormed_row_stride,
            _ptr(input), input_row_stride, m, _ptr(weight), weight_row_stride, n, k, _ptr(gamma),
            n_normed, epsilon, weight_offset, dtype, transpose_b, _ptr(workspace),
            workspace_bytes, _stream(stream))
    return _call(lib.matmul_fused_partial_rmsnorm, args, [], raise_on_error, prepare)


def matmul_fused_partial_rmsnorm_noalloc(normed_output, normed_row_stride: int, unnormed_output,
                                         unnormed_row_stride: int, input, input_row_stride: int,
                                         m: int, weight, weight_row_stride: int, n: int, k: int,
                                         gamma, n_normed: int, epsilon: float,
                                         weight_offset: float, dtype: int, transpose_b: int = 1,
                                         stream=None, raise_on_error: bool = True,
                                         prepare: bool = False):
    """The same op with the library's own scratch (m * n_normed <= 131072);
    calls that overlap on one GPU race."""
    args = (_ptr(normed_output), normed_row_stride, _ptr(unnormed_output), unnormed_row_stride,
            _ptr(input), input_row_stride, m, _ptr(weight), weight_row_stride, n, k, _ptr(gamma),
            n_normed, epsilon, weight_offset, dtype, transpose_b, _stream(stream))
    return _call(lib.matmul_fused_partial_rmsnorm_noalloc, args, [], raise_on_error, prepare)


def qrp_validate(input_row_offsets, batch_size: int, total_seq_len: int, batch_offset: int,
                 cache: PagedCache, max_seq_len: int, stream=None,
                 raise_on_error: bool = False) -> int:
    cc = cache.to_c()
    st = lib.qrp_validate(_ptr(input_row_offsets), batch_size, total_seq_len, batch_offset,
                          ctypes.byref(cc), max_seq_len, _stream(stream))
    return _check(st, raise_on_error)


def qrp_validate_host(offsets, batch_size: int, total_seq_len: int, batch_offset: int,
                      cache_lengths, lookup_table, cache_batch: int, max_pages_per_seq: int,
                      page_size: int, num_pages: int, max_seq_len: int) -> int:
    """Host-array form; numpy uint32 arrays."""
    import numpy as np

    off = np.ascontiguousarray(offsets, dtype=np.uint32)
    lens = np.ascontiguousarray(cache_lengths, dtype=np.uint32)
    tab = np.ascontiguousarray(lookup_table, dtype=np.uint32)
    return lib.qrp_validate_host(off.ctypes.data, batch_size, total_seq_len, batch_offset,
                                 lens.ctypes.data, tab.ctypes.data, cache_batch,
                                 max_pages_per_seq, page_size, num_pages, max_seq_len)


def abi_version() -> int:
    return lib.qrp_abi_version()
