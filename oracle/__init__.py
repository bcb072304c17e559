"""CPU oracle for the ragged RoPE / split / paged-store pass -- TEST INFRASTRUCTURE.

A plain single-threaded C implementation (``qrp_oracle.c``) of what the pass
computes, in double precision, plus this ctypes adapter.  Only the
test-suite, the smoke check and the benchmark's CPU-baseline leg may import
it.  It shares no code with the HIP library and never calls it.

``run_case`` takes a workload from :mod:`synth.cases` (duck-typed: only its
attributes are read) and returns the oracle's outputs, the cache pools after
the operation and the unrounded values needed for tolerance checks.
Pools larger than ``compact_over`` bytes are run on a compacted copy that
holds only the pages the batch touches; ``page_map`` then maps each compact
page back to its id in the full pool.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "qrp_oracle.c")

ORC_F32, ORC_BF16, ORC_F16, ORC_FP8 = 0, 1, 2, 3
_DT = {"f32": ORC_F32, "bf16": ORC_BF16, "f16": ORC_F16, "fp8": ORC_FP8}
_SENT = {"f32": np.uint32(0x7FBADBAD), "bf16": np.uint16(0x7FBA), "f16": np.uint16(0x7DBA),
         "fp8": np.uint8(0x7F)}
_BITS = {"f32": np.uint32, "bf16": np.uint16, "f16": np.uint16, "fp8": np.uint8}
NO_PAGE = 0xFFFFFFFF


def build() -> str:
    """Compile the oracle with gcc (plain C11, no fp contraction, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", SRC, "-o", LIB_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    return LIB_PATH


class OrcCache(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_uint32), ("head_dim", ctypes.c_uint32),
                ("page_size", ctypes.c_uint32), ("kv_planes", ctypes.c_uint32),
                ("num_layers", ctypes.c_uint32), ("num_pages", ctypes.c_uint64),
                ("page_stride", ctypes.c_int64), ("plane_stride", ctypes.c_int64),
                ("layer_stride", ctypes.c_int64), ("slot_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64),
                ("cache_lengths", ctypes.c_void_p), ("lookup_table", ctypes.c_void_p),
                ("cache_batch", ctypes.c_uint32), ("max_pages_per_seq", ctypes.c_uint32),
                ("scales", ctypes.c_void_p), ("scale_dtype", ctypes.c_int32),
                ("s_page_stride", ctypes.c_int64), ("s_plane_stride", ctypes.c_int64),
                ("s_layer_stride", ctypes.c_int64), ("s_slot_stride", ctypes.c_int64),
                ("s_head_stride", ctypes.c_int64)]


class OrcTrace(ctypes.Structure):
    _fields_ = [("q_exact", ctypes.c_void_p), ("q_mag", ctypes.c_void_p),
                ("k_exact", ctypes.c_void_p), ("k_mag", ctypes.c_void_p),
                ("k_row_off", ctypes.c_void_p), ("v_row_off", ctypes.c_void_p),
                ("k_scale_off", ctypes.c_void_p), ("v_scale_off", ctypes.c_void_p),
                ("q_pre", ctypes.c_void_p), ("k_pre", ctypes.c_void_p)]


class OrcBand(ctypes.Structure):
    _fields_ = [("q_col", ctypes.c_uint64), ("n_q_heads", ctypes.c_uint32),
                ("k_col", ctypes.c_int64), ("v_col", ctypes.c_int64),
                ("q_gamma", ctypes.c_void_p), ("k_gamma", ctypes.c_void_p),
                ("epsilon", ctypes.c_float), ("cache", ctypes.POINTER(OrcCache)),
                ("q_output", ctypes.c_void_p), ("q_out_row_stride", ctypes.c_uint64)]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P, U32, U64, I32, I64, F = (ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64,
                                ctypes.c_int32, ctypes.c_int64, ctypes.c_float)
    lib.orc_round_bf16.argtypes = [ctypes.c_double]
    lib.orc_round_bf16.restype = ctypes.c_uint16
    lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_double.restype = ctypes.c_double
    lib.orc_round_f16.argtypes = [ctypes.c_double]
    lib.orc_round_f16.restype = ctypes.c_uint16
    lib.orc_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_double.restype = ctypes.c_double
    lib.orc_round_e4m3.argtypes = [ctypes.c_double]
    lib.orc_round_e4m3.restype = ctypes.c_uint8
    lib.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_to_double.restype = ctypes.c_double
    lib.orc_rope_split_store_paged.argtypes = [P, I32, U32, U64, U32, P, U32, P, U32, U32, I32,
                                               I32, ctypes.POINTER(OrcCache), U32, P, I32, U64,
                                               ctypes.POINTER(OrcTrace)]
    lib.orc_rope_split_store_paged.restype = I32
    lib.orc_qk_rmsnorm_rope_paged.argtypes = [P, I32, U32, U64, ctypes.POINTER(OrcBand), F, I32,
                                              P, U32, P, U32, U32, I32, I32, U32,
                                              ctypes.POINTER(OrcTrace)]
    lib.orc_qk_rmsnorm_rope_paged.restype = I32
    lib.orc_dual_band.argtypes = [P, I32, U32, U64, ctypes.POINTER(OrcBand),
                                  ctypes.POINTER(OrcBand), F, I32, P, U32, P, U32, U32, I32, I32,
                                  U32, ctypes.POINTER(OrcTrace), ctypes.POINTER(OrcTrace)]
    lib.orc_dual_band.restype = I32
    lib.orc_kv_cache_radd.argtypes = [P, I32, U32, U64, P, U32, U32, ctypes.POINTER(OrcCache),
                                      U32, ctypes.POINTER(OrcTrace)]
    lib.orc_kv_cache_radd.restype = I32
    lib.orc_fused_qk_rope_bshd.argtypes = [P, I32, U32, U32, U32, P, P, U32, U32, I32, I32,
                                           ctypes.POINTER(OrcCache), U32, P,
                                           ctypes.POINTER(OrcTrace)]
    lib.orc_fused_qk_rope_bshd.restype = I32
    lib.orc_matmul_fused_partial_rmsnorm.argtypes = [P, U64, P, U64, P, U64, U32, P, U64, U32,
                                                     U32, P, U32, F, F, I32, I32, P, P, P]
    lib.orc_matmul_fused_partial_rmsnorm.restype = I32
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def round_bf16(x: float) -> int:
    return int(load().orc_round_bf16(float(x)))


def bf16_to_double(b: int) -> float:
    return float(load().orc_bf16_to_double(int(b)))


def round_f16(x: float) -> int:
    return int(load().orc_round_f16(float(x)))


def f16_to_double(h: int) -> float:
    return float(load().orc_f16_to_double(int(h)))


def round_e4m3(x: float) -> int:
    return int(load().orc_round_e4m3(float(x)))


def e4m3_to_double(q: int) -> float:
    return float(load().orc_e4m3_to_double(int(q)))


@dataclass
class OracleResult:
    status: int
    seconds: float = 0.0                                       # wall time of the C call
    q_out: List[np.ndarray] = field(default_factory=list)     # per band, raw bits
    pools: List[np.ndarray] = field(default_factory=list)     # per cache, after the op
    scales: List[Optional[np.ndarray]] = field(default_factory=list)   # per FP8 cache, after
    page_maps: List[Optional[np.ndarray]] = field(default_factory=list)
    traces: List[dict] = field(default_factory=list)          # per band


def touched_pages(case, ci: int) -> np.ndarray:
    """Distinct page ids of cache ``ci`` that the batch's tokens land on."""
    cache = case.caches[ci]
    off = np.asarray(case.offsets, dtype=np.int64)
    T = int(off[-1])
    if T == 0:
        return np.zeros(0, dtype=np.int64)
    seq = np.searchsorted(off, np.arange(T), side="right") - 1
    local = np.arange(T) - off[seq]
    if case.op == "bshd":                    # only rows below the valid length touch the cache
        real = local < np.asarray(case.lengths, dtype=np.int64)[seq]
        seq, local = seq[real], local[real]
        if len(seq) == 0:
            return np.zeros(0, dtype=np.int64)
    cseq = seq + case.batch_offset
    pos = cache.cache_lengths.astype(np.int64)[cseq] + local
    pages = cache.lookup_table[cseq, pos // cache.page_size].astype(np.int64)
    return np.unique(pages)


def _orc_cache(cache, pool: np.ndarray, table: np.ndarray, num_pages: int, keep: list,
               scales: Optional[np.ndarray] = None) -> OrcCache:
    st = cache.strides
    lens = np.ascontiguousarray(cache.cache_lengths, dtype=np.uint32)
    table = np.ascontiguousarray(table, dtype=np.uint32)
    keep += [lens, table, pool, scales]
    sst = cache.scale_strides if scales is not None else dict(
        s_page_stride=0, s_plane_stride=0, s_layer_stride=0, s_slot_stride=0, s_head_stride=0)
    return OrcCache(scales=_ptr(scales),
                    scale_dtype=_DT[cache.scale_dtype] if scales is not None else 0, **sst,
                    pool=_ptr(pool), dtype=_DT[cache.dtype], num_kv_heads=cache.num_kv_heads,
                    head_dim=cache.head_dim, page_size=cache.page_size,
                    kv_planes=cache.kv_planes, num_layers=cache.num_layers, num_pages=num_pages,
                    page_stride=st["page_stride"], plane_stride=st["plane_stride"],
                    layer_stride=st["layer_stride"], slot_stride=st["slot_stride"],
                    head_stride=st["head_stride"], cache_lengths=_ptr(lens),
                    lookup_table=_ptr(table), cache_batch=cache.cache_batch,
                    max_pages_per_seq=cache.max_pages_per_seq)


def _trace(T: int, Hq: int, Hk: int, D: int, keep: list) -> tuple:
    tr = dict(q_exact=np.zeros((T, Hq, D)), q_mag=np.zeros((T, Hq, D)),
              k_exact=np.zeros((T, Hk, D)), k_mag=np.zeros((T, Hk, D)),
              k_row_off=np.full((T, Hk), -1, dtype=np.int64),
              v_row_off=np.full((T, Hk), -1, dtype=np.int64),
              k_scale_off=np.full((T, Hk), -1, dtype=np.int64),
              v_scale_off=np.full((T, Hk), -1, dtype=np.int64),
              q_pre=np.full((T, Hq, D), np.nan), k_pre=np.full((T, Hk, D), np.nan))
    keep.append(tr)
    return tr, OrcTrace(**{k: _ptr(v) for k, v in tr.items()})


def run_case(case, trace: bool = True, compact_over: int = 1 << 31) -> OracleResult:
    lib = load()
    keep: list = []
    dt = _DT[case.dtype]
    T = case.T
    buf = np.ascontiguousarray(case.buf)
    off = np.ascontiguousarray(case.offsets, dtype=np.uint32)
    freqs = None if case.freqs is None else np.ascontiguousarray(case.freqs, dtype=np.float32)
    keep += [buf, off, freqs]

    res = OracleResult(status=0)
    ocaches = []
    for ci, cache in enumerate(case.caches):
        if cache.nbytes > compact_over:
            pages = touched_pages(case, ci)
            remap = np.full(cache.num_pages, NO_PAGE, dtype=np.uint64)
            remap[pages] = np.arange(len(pages), dtype=np.uint64)
            tab = cache.lookup_table.astype(np.uint64)
            valid = tab != NO_PAGE
            ctab = np.full(tab.shape, NO_PAGE, dtype=np.uint64)
            ctab[valid] = remap[tab[valid]]
            pool = cache.materialize(pages)
            scl = cache.materialize_scales(pages)
            res.page_maps.append(pages)
            oc = _orc_cache(cache, pool, ctab.astype(np.uint32), len(pages), keep, scl)
        else:
            pool = cache.materialize()
            scl = cache.materialize_scales()
            res.page_maps.append(None)
            oc = _orc_cache(cache, pool, cache.lookup_table, cache.num_pages, keep, scl)
        res.pools.append(pool)
        res.scales.append(scl)
        ocaches.append(oc)
    keep.append(ocaches)

    if case.op == "store":
        cache = case.caches[0]
        D, Hk, Hq = cache.head_dim, cache.num_kv_heads, case.n_q_heads
        qdt = case.q_dtype
        q_out = np.full((T, case.q_out_row_stride), _SENT[qdt], dtype=_BITS[qdt])
        tr, otr = _trace(T, Hq, Hk, D, keep) if trace else (None, None)
        t0 = time.perf_counter()
        st = lib.orc_rope_split_store_paged(
            _ptr(buf), dt, T, case.row_stride, Hq, _ptr(off), case.batch, _ptr(freqs),
            case.max_seq_len, case.rope_dim, int(case.interleaved), int(case.rope_tail),
            ctypes.byref(ocaches[0]), case.layer_idx, _ptr(q_out), _DT[qdt], case.q_out_row_stride,
            ctypes.byref(otr) if otr is not None else None)
        res.q_out.append(q_out)
        res.traces.append(tr)
    elif case.op in ("norm", "dual"):
        obands, q_outs, trs, otrs = [], [], [], []
        for band in case.bands:
            cache = case.caches[band.cache]
            D, Hk = cache.head_dim, cache.num_kv_heads
            q_out = np.full((T, band.q_out_row_stride), _SENT[case.dtype], dtype=_BITS[case.dtype])
            qg = None if band.q_gamma is None else np.ascontiguousarray(band.q_gamma)
            kg = None if band.k_gamma is None else np.ascontiguousarray(band.k_gamma)
            keep += [q_out, qg, kg]
            obands.append(OrcBand(q_col=band.q_col, n_q_heads=band.n_q_heads, k_col=band.k_col,
                                  v_col=band.v_col, q_gamma=_ptr(qg), k_gamma=_ptr(kg),
                                  epsilon=band.epsilon,
                                  cache=ctypes.pointer(ocaches[band.cache]),
                                  q_output=_ptr(q_out), q_out_row_stride=band.q_out_row_stride))
            q_outs.append(q_out)
            tr, otr = _trace(T, band.n_q_heads, Hk, D, keep) if trace else (None, None)
            trs.append(tr)
            otrs.append(otr)
        keep.append(obands)
        t0 = time.perf_counter()
        if case.op == "norm":
            st = lib.orc_qk_rmsnorm_rope_paged(
                _ptr(buf), dt, T, case.row_stride, ctypes.byref(obands[0]),
                case.weight_offset, int(case.multiply_before_cast), _ptr(off), case.batch,
                _ptr(freqs), case.max_seq_len, case.rope_dim, int(case.interleaved),
                int(case.rope_tail), case.layer_idx,
                ctypes.byref(otrs[0]) if otrs[0] is not None else None)
        else:
            st = lib.orc_dual_band(
                _ptr(buf), dt, T, case.row_stride, ctypes.byref(obands[0]),
                ctypes.byref(obands[1]), case.weight_offset, int(case.multiply_before_cast),
                _ptr(off), case.batch, _ptr(freqs), case.max_seq_len, case.rope_dim,
                int(case.interleaved), int(case.rope_tail), case.layer_idx,
                ctypes.byref(otrs[0]) if otrs[0] is not None else None,
                ctypes.byref(otrs[1]) if otrs[1] is not None else None)
        res.q_out += q_outs
        res.traces += trs
    elif case.op == "radd":
        cache = case.caches[0]
        Hk = cache.num_kv_heads
        tr = {k: np.full((T, Hk), -1, dtype=np.int64)
              for k in ("k_row_off", "v_row_off", "k_scale_off", "v_scale_off")}
        keep.append(tr)
        otr = OrcTrace(**{k: _ptr(v) for k, v in tr.items()})
        t0 = time.perf_counter()
        st = lib.orc_kv_cache_radd(_ptr(buf), dt, T, case.row_stride, _ptr(off), case.batch,
                                   case.batch_offset, ctypes.byref(ocaches[0]), case.layer_idx,
                                   ctypes.byref(otr))
        res.traces.append(tr)
    elif case.op == "bshd":
        cache = case.caches[0]
        D, Hk, Hq = cache.head_dim, cache.num_kv_heads, case.n_q_heads
        out = np.full((T, Hq * D), _SENT[case.dtype], dtype=_BITS[case.dtype])
        valid = np.ascontiguousarray(case.lengths, dtype=np.uint32)
        keep += [out, valid]
        tr, otr = _trace(T, Hq, Hk, D, keep) if trace else (None, None)
        t0 = time.perf_counter()
        st = lib.orc_fused_qk_rope_bshd(
            _ptr(buf), dt, case.batch, case.seq_len, Hq, _ptr(valid), _ptr(freqs),
            case.max_seq_len, case.rope_dim, int(case.interleaved), int(case.rope_tail),
            ctypes.byref(ocaches[0]), case.layer_idx, _ptr(out),
            ctypes.byref(otr) if otr is not None else None)
        res.q_out.append(out)
        res.traces.append(tr)
    else:
        raise ValueError(case.op)
    res.seconds = time.perf_counter() - t0
    res.status = int(st)
    return res


@dataclass
class GemvResult:
    status: int
    seconds: float = 0.0
    normed: Optional[np.ndarray] = None     # raw bits [m, normed_row_stride]
    unnormed: Optional[np.ndarray] = None   # raw bits [m, unnormed_row_stride]
    y_exact: Optional[np.ndarray] = None    # [m, n] y before rounding
    abs_dot: Optional[np.ndarray] = None    # [m, n] sum_k |x_k w_jk|
    r: Optional[np.ndarray] = None          # [m] reciprocal root of each row's norm


def run_gemv(case, trace: bool = True) -> GemvResult:
    """The fused GEMV + partial RMSNorm on a case from synth.cases.make_gemv_case
    (duck-typed).  Outputs start as sentinels, so padding columns stay visible."""
    lib = load()
    dt = _DT[case.dtype]
    m, n = case.m, case.n
    x = np.ascontiguousarray(case.x)
    w = np.ascontiguousarray(case.w)
    g = np.ascontiguousarray(case.gamma)
    normed = np.full((m, case.normed_row_stride), _SENT[case.dtype], dtype=_BITS[case.dtype])
    unnormed = np.full((m, case.unnormed_row_stride), _SENT[case.dtype], dtype=_BITS[case.dtype])
    y = np.zeros((m, n)) if trace else None
    a = np.zeros((m, n)) if trace else None
    r = np.zeros(m) if trace else None
    t0 = time.perf_counter()
    st = lib.orc_matmul_fused_partial_rmsnorm(
        _ptr(normed), case.normed_row_stride, _ptr(unnormed), case.unnormed_row_stride,
        _ptr(x), x.shape[1], m, _ptr(w), w.shape[1], n, case.k, _ptr(g), case.n_normed,
        case.epsilon, case.weight_offset, dt, int(getattr(case, "transpose_b", 1)), _ptr(y),
        _ptr(a), _ptr(r))
    return GemvResult(status=int(st), seconds=time.perf_counter() - t0, normed=normed,
                      unnormed=unnormed, y_exact=y, abs_dot=a, r=r)
