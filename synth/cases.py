"""Seeded synthetic workloads for the ragged RoPE / split / paged-store pass.

A :class:`Case` holds host numpy arrays only: the flat input buffer (raw bits
of its dtype), ragged row offsets, the freqs_cis table, one or two paged
caches and the scalar arguments.  Tests, the benchmark and the smoke check
turn a case into arguments for the HIP library and, separately, for the CPU
oracle.  Nothing here computes any part of the method itself.

Workload shapes follow the configurations the pass is measured on:

* ``tiny_fp32``  tiny fp32 interleaved store (batch 2, lengths {3, 5}, cache lengths
  {0, 4}, 4 Q / 2 KV heads, head_dim 64, page 16, 8 pages);
* ``prefill``    Llama-3-8B-shaped bf16 prefill store, half-split RoPE (batch 8,
  lengths U[128, 2048], 32 Q / 8 KV heads, head_dim 128, theta 5e5, page 128,
  32 layers, layer 17);
* ``decode``     the matching decode (256 sequences x 1 token, cache lengths
  U[0, 8191], interleaved, 20000-page pool);
* ``dual``       dual-band RMSNorm + RoPE (main 64 Q / 8 KV heads, index 16 Q heads
  + single-head K-only cache, head_dim 128, rope_dim 64, page 64);
* ``radd``       K/V radd (8 KV heads, head_dim 128, batch 32 of a 64-sequence
  cache at batch_offset 4, page 128, layer 3).

``small=True`` gives a reduced variant of each that the oracle finishes in
well under a second while still spanning several work tiles and a ragged tail.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from . import prng

F32, BF16, F16 = "f32", "bf16", "f16"
FP8 = "fp8"                             # OCP e4m3 codes with a scale per cache row (caches only)
# signalling-NaN patterns
SENTINEL = {F32: np.uint32(0x7FBADBAD), BF16: np.uint16(0x7FBA), F16: np.uint16(0x7DBA),
            FP8: np.uint8(0x7F)}
BITS_DTYPE = {F32: np.uint32, BF16: np.uint16, F16: np.uint16, FP8: np.uint8}
ELEM_BYTES = {F32: 4, BF16: 2, F16: 2, FP8: 1}
# the finite e4m3 codes (S.1111.111 is NaN)
FP8_FINITE_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
NO_PAGE = np.uint32(0xFFFFFFFF)

# stream numbers (one per generated array)
S_LENS, S_CLEN, S_PERM, S_BUF, S_GAMMA, S_A, S_PREFILL, S_SPECIAL = 1, 2, 3, 4, 5, 6, 7, 8
S_X, S_W = 9, 10


def to_bits(values: np.ndarray, dtype: str) -> np.ndarray:
    """Doubles -> raw bits of ``dtype`` (binary16: numpy's RNE; bf16: binary32
    RNE, then bf16 RNE)."""
    if dtype == F16:
        return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)
    f = np.asarray(values, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    if dtype == F32:
        return u.copy()
    rounded = (u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F16:
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == F32:
        return bits.view(np.float32).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def freqs_table(max_seq_len: int, rope_dim: int, base: float, freq_dtype: str = F32) -> np.ndarray:
    """freqs_cis[p, 2i] = cos(p * base^(-2i/R)), [p, 2i+1] = sin(...), fp64 -> fp32
    (a bf16 table: -> fp32 -> bf16; an f16 table: fp64 -> f16; the float32
    array then holds those values)."""
    i = np.arange(rope_dim // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / rope_dim)
    ang = np.arange(max_seq_len, dtype=np.float64)[:, None] * inv[None, :]
    tab = np.empty((max_seq_len, rope_dim), dtype=np.float64)
    tab[:, 0::2] = np.cos(ang)
    tab[:, 1::2] = np.sin(ang)
    if freq_dtype in (BF16, F16):
        return bits_to_f64(to_bits(tab, freq_dtype), freq_dtype).astype(np.float32)
    return tab.astype(np.float32)


@dataclass
class PagedCache:
    """Paged pool, page-major: [num_pages][kv_planes][num_layers][page_size][Hk][D].

    The pool is held lazily: every element is the sentinel except the rows
    listed in ``prefill`` (page, plane, layer, slot, values[Hk, D]), so a
    20000-page pool costs nothing until someone materialises it."""
    dtype: str
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_layers: int
    kv_planes: int
    num_pages: int
    cache_lengths: np.ndarray          # uint32 [cache_batch]
    lookup_table: np.ndarray           # uint32 [cache_batch, max_pages_per_seq]
    prefill: list = field(default_factory=list)
    scale_dtype: Optional[str] = None   # FP8 caches: F32 or BF16 scales, one per row
    prefill_scales: list = field(default_factory=list)   # FP8: [n, Hk] scale bits per prefill entry

    @property
    def cache_batch(self) -> int:
        return int(self.lookup_table.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.lookup_table.shape[1])

    @property
    def shape(self) -> tuple:
        return (self.num_pages, self.kv_planes, self.num_layers, self.page_size,
                self.num_kv_heads, self.head_dim)

    @property
    def strides(self) -> dict:
        """Element strides of the page-major layout (C order of ``shape``)."""
        st = np.empty(6, dtype=np.int64)
        acc = 1
        for i in range(5, -1, -1):
            st[i] = acc
            acc *= self.shape[i]
        return dict(page_stride=int(st[0]), plane_stride=int(st[1]), layer_stride=int(st[2]),
                    slot_stride=int(st[3]), head_stride=int(st[4]))

    @property
    def page_elems(self) -> int:
        return int(np.prod(self.shape[1:]))

    @property
    def scale_shape(self) -> tuple:
        """FP8 caches: one scale per (page, plane, layer, slot, head) row."""
        return self.shape[:5]

    @property
    def scale_strides(self) -> dict:
        st = np.empty(5, dtype=np.int64)
        acc = 1
        for i in range(4, -1, -1):
            st[i] = acc
            acc *= self.scale_shape[i]
        return dict(s_page_stride=int(st[0]), s_plane_stride=int(st[1]),
                    s_layer_stride=int(st[2]), s_slot_stride=int(st[3]),
                    s_head_stride=int(st[4]))

    def materialize_scales(self, pages: Optional[np.ndarray] = None) -> Optional[np.ndarray]:
        """FP8 caches: the scales array (sentinel except prefilled rows); with
        ``pages`` only those pages, in that order.  None for other caches."""
        if self.dtype != FP8:
            return None
        n = self.num_pages if pages is None else len(pages)
        sc_ = np.full((n,) + self.scale_shape[1:], SENTINEL[self.scale_dtype],
                      dtype=BITS_DTYPE[self.scale_dtype])
        pg, pl, ly, sl, _ = self.prefill_arrays()
        if len(pg):
            vals = np.concatenate(self.prefill_scales)
            if pages is not None:
                remap = np.full(self.num_pages, -1, dtype=np.int64)
                remap[np.asarray(pages, dtype=np.int64)] = np.arange(len(pages))
                pg = remap[pg]
                keep = pg >= 0
                pg, pl, ly, sl, vals = pg[keep], pl[keep], ly[keep], sl[keep], vals[keep]
            sc_[pg, pl, ly, sl] = vals
        return sc_

    @property
    def nbytes(self) -> int:
        return self.num_pages * self.page_elems * ELEM_BYTES[self.dtype]

    @property
    def scale_nbytes(self) -> int:
        if self.dtype != FP8:
            return 0
        return int(np.prod(self.scale_shape)) * ELEM_BYTES[self.scale_dtype]

    def prefill_arrays(self):
        """(pages, planes, layers, slots) int64 arrays and values [n, Hk, D] bits."""
        if not self.prefill:
            z = np.zeros(0, dtype=np.int64)
            return z, z, z, z, np.zeros((0, self.num_kv_heads, self.head_dim),
                                        dtype=BITS_DTYPE[self.dtype])
        cols = [np.concatenate([np.asarray(p[i], dtype=np.int64) for p in self.prefill])
                for i in range(4)]
        vals = np.concatenate([p[4] for p in self.prefill])
        return cols[0], cols[1], cols[2], cols[3], vals

    def materialize(self, pages: Optional[np.ndarray] = None) -> np.ndarray:
        """The pool as a numpy array; with ``pages`` only those pages, in that order."""
        n = self.num_pages if pages is None else len(pages)
        pool = np.full((n,) + self.shape[1:], SENTINEL[self.dtype], dtype=BITS_DTYPE[self.dtype])
        pg, pl, ly, sl, vals = self.prefill_arrays()
        if len(pg):
            if pages is not None:
                remap = np.full(self.num_pages, -1, dtype=np.int64)
                remap[np.asarray(pages, dtype=np.int64)] = np.arange(len(pages))
                pg = remap[pg]
                keep = pg >= 0
                pg, pl, ly, sl, vals = pg[keep], pl[keep], ly[keep], sl[keep], vals[keep]
            pool[pg, pl, ly, sl] = vals
        return pool


@dataclass
class Band:
    q_col: int
    n_q_heads: int
    k_col: int                          # < 0: K already in the cache (in place)
    v_col: int                          # < 0: no V
    q_gamma: Optional[np.ndarray]       # raw bits [D] or None
    k_gamma: Optional[np.ndarray]
    epsilon: float
    cache: int                          # index into Case.caches
    q_out_row_stride: int


@dataclass
class Case:
    name: str
    op: str                             # 'store' | 'norm' | 'dual' | 'radd' | 'bshd'
    dtype: str
    seed: int
    lengths: np.ndarray                 # int64 [B]
    offsets: np.ndarray                 # uint32 [B + 1]
    buf: np.ndarray                     # raw bits [T, row_stride]
    freqs: Optional[np.ndarray]         # float32 [max_seq_len, rope_dim]
    rope_dim: int
    interleaved: bool
    caches: List[PagedCache]
    layer_idx: int = 0
    batch_offset: int = 0
    n_q_heads: int = 0                  # store op
    q_out_row_stride: int = 0           # store op
    bands: List[Band] = field(default_factory=list)
    weight_offset: float = 0.0
    multiply_before_cast: bool = True
    freq_dtype: str = F32               # table entries: f32, or bf16 / f16 values held in float32
    seq_len: int = 0                    # bshd: padded rows per sequence (lengths = valid lengths)
    q_out_dtype: Optional[str] = None   # store op: Q output dtype (None: dtype)
    rope_tail: bool = False             # a partial rope rotates the last rope_dim dims

    @property
    def q_dtype(self) -> str:
        return self.q_out_dtype or self.dtype

    @property
    def T(self) -> int:
        return int(self.offsets[-1])

    @property
    def batch(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def row_stride(self) -> int:
        return int(self.buf.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.freqs.shape[0]) if self.freqs is not None else 0


# ---------------------------------------------------------------------------
# builders
# ---------------------------------------------------------------------------

def _offsets(lengths: np.ndarray) -> np.ndarray:
    off = np.zeros(len(lengths) + 1, dtype=np.uint64)
    off[1:] = np.cumsum(lengths)
    return off.astype(np.uint32)


def _paged_cache(seed: int, stream: int, dtype: str, Hk: int, D: int, P: int, L: int, planes: int,
                 cache_lengths: np.ndarray, rows_needed: np.ndarray, max_pages: int,
                 num_pages: Optional[int], slack: float,
                 scale_dtype: Optional[str] = None) -> PagedCache:
    """Pool + page table: sequence b takes the next ceil(rows_needed[b] / P) ids
    of a seeded permutation of the pool; left-over table entries take the
    remaining ids while any remain, then NO_PAGE."""
    need = [(int(r) + P - 1) // P for r in rows_needed]
    if max(need, default=0) > max_pages:
        raise ValueError("max_pages_per_seq too small for the lengths drawn")
    total = sum(need)
    if num_pages is None:
        num_pages = max(1, int(np.ceil(total * (1.0 + slack))))
    if total > num_pages:
        raise ValueError("pool too small")
    perm = prng.permutation(seed, stream, num_pages).astype(np.uint32)
    cb = len(rows_needed)
    table = np.full((cb, max_pages), NO_PAGE, dtype=np.uint32)
    k = 0
    for b in range(cb):
        table[b, :need[b]] = perm[k:k + need[b]]
        k += need[b]
    for b in range(cb):
        for j in range(need[b], max_pages):
            if k >= num_pages:
                break
            table[b, j] = perm[k]
            k += 1
    return PagedCache(dtype=dtype, num_kv_heads=Hk, head_dim=D, page_size=P, num_layers=L,
                      kv_planes=planes, num_pages=num_pages,
                      cache_lengths=np.asarray(cache_lengths, dtype=np.uint32), lookup_table=table,
                      scale_dtype=(scale_dtype or F32) if dtype == FP8 else None)


def _prefill_rows(cache: PagedCache, seed: int, stream: int, layer: int, planes, seqs,
                  starts, counts, std: float = 1.0) -> None:
    """N(0, std^2) into rows [start, start + count) of the given sequences."""
    P, H, D = cache.page_size, cache.num_kv_heads, cache.head_dim
    pos_list, seq_list = [], []
    for s, st, cnt in zip(seqs, starts, counts):
        pos_list.append(np.arange(int(st), int(st) + int(cnt), dtype=np.int64))
        seq_list.append(np.full(int(cnt), int(s), dtype=np.int64))
    pos = np.concatenate(pos_list) if pos_list else np.zeros(0, np.int64)
    seq = np.concatenate(seq_list) if seq_list else np.zeros(0, np.int64)
    n_rows = len(pos) * len(planes)
    if cache.dtype == FP8:
        # random finite codes and positive scales around 2^-7 (448 * scale ~ 2..5)
        pick = prng.integers(seed, stream, n_rows * H * D, 0, len(FP8_FINITE_CODES) - 1)
        vals = FP8_FINITE_CODES[pick]
        u = prng.uniform01(seed, stream + 500, n_rows * H)
        scales = to_bits((0.5 + u) * 2.0 ** -7, cache.scale_dtype)
        scales = scales.reshape(len(planes), len(pos), H)
    else:
        vals = to_bits(prng.normal(seed, stream, n_rows * H * D, std=std), cache.dtype)
    vals = vals.reshape(len(planes), len(pos), H, D)
    pages = cache.lookup_table[seq, pos // P].astype(np.int64)
    for k, plane in enumerate(planes):
        cache.prefill.append((pages, np.full(len(pos), plane, np.int64),
                              np.full(len(pos), layer, np.int64), pos % P, vals[k]))
        if cache.dtype == FP8:
            cache.prefill_scales.append(scales[k])


def make_store_case(name: str, seed: int, dtype: str, lengths, cache_lengths, Hq: int, Hk: int,
                    D: int, rope_dim: int, interleaved: bool, theta: float, max_seq_len: int,
                    P: int, L: int, layer: int, num_pages: Optional[int] = None,
                    max_pages: Optional[int] = None, slack: float = 0.25,
                    q_out_pad: int = 0, row_pad: int = 0, specials: bool = False,
                    freq_dtype: str = F32, cache_dtype: Optional[str] = None,
                    scale_dtype: str = F32, q_out_dtype: Optional[str] = None,
                    rope_tail: bool = False) -> Case:
    """rope_split_store_paged workload: qkv [T, (Hq + 2Hk) D (+row_pad)] N(0, 1).
    ``cache_dtype`` FP8 stores e4m3 rows with ``scale_dtype`` scales;
    ``q_out_dtype`` sets Q's output dtype (default: dtype)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cache_lengths = np.asarray(cache_lengths, dtype=np.int64)
    rows = cache_lengths + lengths
    if max_pages is None:
        max_pages = max(1, (max_seq_len + P - 1) // P)
    cache = _paged_cache(seed, S_PERM, cache_dtype or dtype, Hk, D, P, L, 2, cache_lengths, rows,
                         max_pages, num_pages, slack, scale_dtype)
    off = _offsets(lengths)
    T = int(off[-1])
    width = (Hq + 2 * Hk) * D
    stride = width + row_pad
    buf = np.zeros((T, stride), dtype=BITS_DTYPE[dtype])
    buf[:, :width] = to_bits(prng.normal(seed, S_BUF, T * width), dtype).reshape(T, width)
    if row_pad:
        buf[:, width:] = SENTINEL[dtype]
    if specials and T:
        _inject_specials(buf, seed, dtype, Hq, Hk, D, rope_dim)
    return Case(name=name, op="store", dtype=dtype, seed=seed, lengths=lengths, offsets=off,
                buf=buf, freqs=freqs_table(max_seq_len, rope_dim, theta, freq_dtype),
                rope_dim=rope_dim, interleaved=interleaved, caches=[cache], layer_idx=layer,
                n_q_heads=Hq, q_out_row_stride=Hq * D + q_out_pad, freq_dtype=freq_dtype,
                q_out_dtype=q_out_dtype, rope_tail=rope_tail)


def _special_values(dtype: str) -> np.ndarray:
    """+-0, +-inf, quiet/signalling NaNs with payloads, subnormals, extremes."""
    if dtype == F16:
        return np.array([0x0000, 0x8000, 0x7C00, 0xFC00, 0x7E01, 0x7C01, 0xFDBA, 0x0001, 0x83FF,
                         0x7BFF, 0x0400], dtype=np.uint16)
    if dtype == F32:
        return np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00001, 0x7F800001,
                         0xFFBADBAD, 0x00000001, 0x807FFFFF, 0x7F7FFFFF, 0x00800000],
                        dtype=np.uint32)
    return np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC1, 0x7F81, 0xFFBA, 0x0001, 0x807F,
                     0x7F7F, 0x0080], dtype=np.uint16)


def _inject_specials(buf, seed, dtype, Hq, Hk, D, rope_dim):
    """Put special bit patterns into V columns and un-roped Q/K dims only."""
    T = buf.shape[0]
    sv = _special_values(dtype)
    cols = [(Hq + Hk) * D + j for j in range(Hk * D)]                 # all V columns
    for h in range(Hq + Hk):
        cols += [h * D + j for j in range(rope_dim, D)]               # un-roped dims
    cols = np.asarray(cols, dtype=np.int64)
    n = max(1, (T * len(cols)) // 16)
    pick_t = prng.integers(seed, S_SPECIAL, n, 0, T - 1)
    pick_c = cols[prng.integers(seed, S_SPECIAL + 100, n, 0, len(cols) - 1)]
    pick_v = sv[prng.integers(seed, S_SPECIAL + 200, n, 0, len(sv) - 1)]
    buf[pick_t, pick_c] = pick_v


def make_norm_case(name: str, seed: int, dtype: str, lengths, cache_lengths, Hq: int, Hk: int,
                   D: int, rope_dim: int, interleaved: bool, theta: float, max_seq_len: int,
                   P: int, L: int, layer: int, k_in_cache: bool, q_norm: bool = True,
                   k_norm: bool = True, eps: float = 1e-6, weight_offset: float = 0.0,
                   multiply_before_cast: bool = True, slack: float = 0.25,
                   gamma_std: float = 0.1, freq_dtype: str = F32,
                   cache_dtype: Optional[str] = None, scale_dtype: str = F32,
                   rope_tail: bool = False) -> Case:
    """Single-band qk_rmsnorm_rope_paged workload.  Buffer [T, (Hq+2Hk) D] =
    Q | K | V; with ``k_in_cache`` K is prefilled in the cache and updated in
    place (the buffer's K and V columns are then unread)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cache_lengths = np.asarray(cache_lengths, dtype=np.int64)
    rows = cache_lengths + lengths
    max_pages = max(1, (max_seq_len + P - 1) // P)
    cache = _paged_cache(seed, S_PERM, cache_dtype or dtype, Hk, D, P, L, 2, cache_lengths, rows,
                         max_pages, None, slack, scale_dtype)
    off = _offsets(lengths)
    T = int(off[-1])
    width = (Hq + 2 * Hk) * D
    buf = to_bits(prng.normal(seed, S_BUF, T * width), dtype).reshape(T, width)
    if k_in_cache:
        _prefill_rows(cache, seed, S_PREFILL, layer, [0], range(len(lengths)), cache_lengths,
                      lengths)
    g = to_bits(prng.normal(seed, S_GAMMA, 2 * D, mean=1.0, std=gamma_std), dtype).reshape(2, D)
    band = Band(q_col=0, n_q_heads=Hq, k_col=-1 if k_in_cache else Hq * D,
                v_col=-1 if k_in_cache else (Hq + Hk) * D,
                q_gamma=g[0] if q_norm else None, k_gamma=g[1] if k_norm else None,
                epsilon=eps, cache=0, q_out_row_stride=Hq * D)
    return Case(name=name, op="norm", dtype=dtype, seed=seed, lengths=lengths, offsets=off,
                buf=buf, freqs=freqs_table(max_seq_len, rope_dim, theta, freq_dtype),
                rope_dim=rope_dim, interleaved=interleaved, caches=[cache], layer_idx=layer,
                bands=[band], weight_offset=weight_offset,
                multiply_before_cast=multiply_before_cast, freq_dtype=freq_dtype,
                rope_tail=rope_tail)


def make_dual_case(name: str, seed: int, dtype: str, lengths, Hq_main: int, Hk_main: int,
                   Hq_index: int, D: int, rope_dim: int, interleaved: bool, theta: float,
                   max_seq_len: int, P_main: int, P_index: int, eps_main: float = 1e-6,
                   eps_index: float = 1e-6, weight_offset: float = 0.0,
                   multiply_before_cast: bool = True, slack: float = 0.25,
                   cache_lengths=None, freq_dtype: str = F32,
                   main_cache_dtype: Optional[str] = None,
                   index_cache_dtype: Optional[str] = None, scale_dtype: str = F32,
                   rope_tail: bool = False, index_cache_lengths=None) -> Case:
    """Dual-band workload: buffer [T, (Hq_main + 2 Hk_main + Hq_index) D] =
    Q-main | K-main | V-main | Q-index; both bands' K caches updated in place.
    The index cache has cache lengths of its own when ``index_cache_lengths``
    is given (else the main cache's)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    B = len(lengths)
    cl = np.zeros(B, dtype=np.int64) if cache_lengths is None else np.asarray(cache_lengths,
                                                                             dtype=np.int64)
    cli = cl if index_cache_lengths is None else np.asarray(index_cache_lengths, dtype=np.int64)
    mp_main = max(1, (max_seq_len + P_main - 1) // P_main)
    mp_index = max(1, (max_seq_len + P_index - 1) // P_index)
    main = _paged_cache(seed, S_PERM, main_cache_dtype or dtype, Hk_main, D, P_main, 1, 2, cl,
                        cl + lengths, mp_main, None, slack, scale_dtype)
    index = _paged_cache(seed, S_PERM + 1000, index_cache_dtype or dtype, 1, D, P_index, 1, 1, cli,
                         cli + lengths, mp_index, None, slack, scale_dtype)
    off = _offsets(lengths)
    T = int(off[-1])
    width = (Hq_main + 2 * Hk_main + Hq_index) * D
    buf = to_bits(prng.normal(seed, S_BUF, T * width), dtype).reshape(T, width)
    _prefill_rows(main, seed, S_PREFILL, 0, [0], range(B), cl, lengths)
    _prefill_rows(index, seed, S_PREFILL + 1000, 0, [0], range(B), cli, lengths)
    g = to_bits(prng.normal(seed, S_GAMMA, 4 * D, mean=1.0, std=0.1), dtype).reshape(4, D)
    main_band = Band(q_col=0, n_q_heads=Hq_main, k_col=-1, v_col=-1, q_gamma=g[0], k_gamma=g[1],
                     epsilon=eps_main, cache=0, q_out_row_stride=Hq_main * D)
    index_band = Band(q_col=(Hq_main + 2 * Hk_main) * D, n_q_heads=Hq_index, k_col=-1, v_col=-1,
                      q_gamma=g[2], k_gamma=g[3], epsilon=eps_index, cache=1,
                      q_out_row_stride=Hq_index * D)
    return Case(name=name, op="dual", dtype=dtype, seed=seed, lengths=lengths, offsets=off,
                buf=buf, freqs=freqs_table(max_seq_len, rope_dim, theta, freq_dtype),
                rope_dim=rope_dim, interleaved=interleaved, caches=[main, index], layer_idx=0,
                bands=[main_band, index_band], weight_offset=weight_offset,
                multiply_before_cast=multiply_before_cast, freq_dtype=freq_dtype,
                rope_tail=rope_tail)


def make_radd_case(name: str, seed: int, dtype: str, lengths, cache_lengths, batch_offset: int,
                   Hk: int, D: int, P: int, L: int, layer: int, a_std: float = 0.02,
                   slack: float = 0.25, a_values: Optional[np.ndarray] = None,
                   cache_dtype: Optional[str] = None, scale_dtype: str = F32) -> Case:
    """kv_cache_radd workload: a [T, 2 Hk D] N(0, a_std^2) added into rows
    [cache_len, cache_len + len) of cache sequences batch_offset + b, which
    hold N(0, 1) before the call."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cache_lengths = np.asarray(cache_lengths, dtype=np.int64)
    B = len(lengths)
    cb = len(cache_lengths)
    if batch_offset + B > cb:
        raise ValueError("batch_offset + batch exceeds the cache batch")
    rows = np.zeros(cb, dtype=np.int64)
    active = np.arange(batch_offset, batch_offset + B)
    rows[active] = cache_lengths[active] + lengths
    max_pages = max(1, int((rows.max() + P - 1) // P))
    cache = _paged_cache(seed, S_PERM, cache_dtype or dtype, Hk, D, P, L, 2, cache_lengths, rows,
                         max_pages, None, slack, scale_dtype)
    off = _offsets(lengths)
    T = int(off[-1])
    width = 2 * Hk * D
    if a_values is None:
        buf = to_bits(prng.normal(seed, S_A, T * width, std=a_std), dtype).reshape(T, width)
    else:
        buf = np.asarray(a_values).reshape(T, width)
    _prefill_rows(cache, seed, S_PREFILL, layer, [0, 1], active, cache_lengths[active], lengths)
    return Case(name=name, op="radd", dtype=dtype, seed=seed, lengths=lengths, offsets=off,
                buf=buf, freqs=None, rope_dim=0, interleaved=True, caches=[cache],
                layer_idx=layer, batch_offset=batch_offset)


def make_bshd_case(name: str, seed: int, dtype: str, valid_lengths, seq_len: int, cache_lengths,
                   Hq: int, Hk: int, D: int, rope_dim: int, interleaved: bool, theta: float,
                   max_seq_len: int, capacity: int, L: int, layer: int,
                   num_blocks: Optional[int] = None, slack: float = 0.25,
                   freq_dtype: Optional[str] = None, cache_dtype: Optional[str] = None,
                   scale_dtype: str = F32, rope_tail: bool = False) -> Case:
    """Padded continuous-batching workload: q_proj [B, seq_len, Hq, D] N(0, 1)
    held as [B * seq_len, Hq * D]; a continuous-batching cache of blocks of
    ``capacity`` rows (one page per sequence, a seeded permutation of the
    blocks), whose K and V rows [cache_len, cache_len + min(valid, seq_len))
    hold N(0, 1) (the projection's K and V).  The table has the op's dtype
    unless ``freq_dtype`` says otherwise."""
    valid = np.asarray(valid_lengths, dtype=np.int64)
    cl = np.asarray(cache_lengths, dtype=np.int64)
    B = len(valid)
    real = np.minimum(valid, seq_len)
    cache = _paged_cache(seed, S_PERM, cache_dtype or dtype, Hk, D, capacity, L, 2, cl, cl + real, 1,
                         num_blocks, slack, scale_dtype)
    T = B * seq_len
    width = Hq * D
    buf = to_bits(prng.normal(seed, S_BUF, T * width), dtype).reshape(T, width)
    _prefill_rows(cache, seed, S_PREFILL, layer, [0, 1], range(B), cl, real)
    off = (np.arange(B + 1, dtype=np.int64) * seq_len).astype(np.uint32)
    fdt = dtype if freq_dtype is None else freq_dtype
    return Case(name=name, op="bshd", dtype=dtype, seed=seed, lengths=valid, offsets=off, buf=buf,
                freqs=freqs_table(max_seq_len, rope_dim, theta, fdt), rope_dim=rope_dim,
                interleaved=interleaved, caches=[cache], layer_idx=layer, n_q_heads=Hq,
                q_out_row_stride=width, freq_dtype=fdt, seq_len=seq_len, rope_tail=rope_tail)


# ---------------------------------------------------------------------------
# the workloads
# ---------------------------------------------------------------------------

def tiny_fp32(seed: int = 1) -> Case:
    return make_store_case("tiny_fp32", seed, F32, [3, 5], [0, 4], Hq=4, Hk=2, D=64,
                           rope_dim=64, interleaved=True, theta=1e4, max_seq_len=64, P=16, L=1,
                           layer=0, num_pages=8, max_pages=4)


def _kv(name: str, cache_dtype: Optional[str]) -> str:
    return name if cache_dtype is None else f"{name}_{cache_dtype}"


def prefill(seed: int = 2, small: bool = False, cache_dtype: Optional[str] = None) -> Case:
    if small:
        B = 4
        lens = prng.integers(seed, S_LENS, B, 1, 300)
        return make_store_case(_kv("prefill_small", cache_dtype), seed, BF16, lens,
                               np.zeros(B, np.int64), Hq=32, Hk=8, D=128, rope_dim=128,
                               interleaved=False, theta=5e5, max_seq_len=8192, P=128, L=4,
                               layer=2, cache_dtype=cache_dtype)
    B = 8
    lens = prng.integers(seed, S_LENS, B, 128, 2048)
    return make_store_case(_kv("prefill", cache_dtype), seed, BF16, lens, np.zeros(B, np.int64),
                           Hq=32, Hk=8, D=128, rope_dim=128, interleaved=False, theta=5e5,
                           max_seq_len=8192, P=128, L=32, layer=17, cache_dtype=cache_dtype)


def decode(seed: int = 3, small: bool = False, cache_dtype: Optional[str] = None) -> Case:
    B = 32 if small else 256
    lens = np.ones(B, dtype=np.int64)
    clen = prng.integers(seed, S_CLEN, B, 0, 8191)
    return make_store_case(_kv("decode_small" if small else "decode", cache_dtype), seed, BF16,
                           lens, clen, Hq=32, Hk=8, D=128, rope_dim=128, interleaved=True,
                           theta=5e5, max_seq_len=8192, P=128, L=1, layer=0,
                           num_pages=1400 if small else 20000, max_pages=64,
                           cache_dtype=cache_dtype)


def dual(seed: int = 4, small: bool = False, cache_dtype: Optional[str] = None) -> Case:
    B = 4 if small else 16
    lens = prng.integers(seed, S_LENS, B, 1, 150 if small else 1024)
    return make_dual_case(_kv("dual_small" if small else "dual", cache_dtype), seed, BF16, lens,
                          Hq_main=64, Hk_main=8, Hq_index=16, D=128, rope_dim=64,
                          interleaved=True, theta=1e4, max_seq_len=8192, P_main=64, P_index=64,
                          main_cache_dtype=cache_dtype, index_cache_dtype=cache_dtype)


def radd(seed: int = 5, small: bool = False, cache_dtype: Optional[str] = None) -> Case:
    if small:
        B, cb, boff = 6, 12, 4
        lens = prng.integers(seed, S_LENS, B, 1, 64)
        clen = prng.integers(seed, S_CLEN, cb, 0, 600)
    else:
        B, cb, boff = 32, 64, 4
        lens = prng.integers(seed, S_LENS, B, 16, 512)
        clen = prng.integers(seed, S_CLEN, cb, 0, 4096)
    return make_radd_case(_kv("radd_small" if small else "radd", cache_dtype), seed, BF16, lens,
                          clen, boff, Hk=8, D=128, P=128, L=4, layer=3, cache_dtype=cache_dtype)


def bshd(seed: int = 6, small: bool = False, cache_dtype: Optional[str] = None) -> Case:
    """Padded continuous batching on the prefill shapes: every sequence padded
    to the longest length the prefill batch draws (2048), valid lengths drawn
    as the prefill lengths are, a bf16 table (the op's dtype)."""
    if small:
        B, S = 4, 300
        valid = prng.integers(seed, S_LENS, B, 0, S)
        clen = prng.integers(seed, S_CLEN, B, 0, 500)
        return make_bshd_case(_kv("bshd_small", cache_dtype), seed, BF16, valid, S, clen, Hq=32,
                              Hk=8, D=128, rope_dim=128, interleaved=False, theta=5e5,
                              max_seq_len=1024, capacity=1024, L=2, layer=1,
                              cache_dtype=cache_dtype)
    B, S = 8, 2048
    valid = prng.integers(seed, S_LENS, B, 128, S)
    return make_bshd_case(_kv("bshd", cache_dtype), seed, BF16, valid, S, np.zeros(B, np.int64),
                          Hq=32, Hk=8, D=128, rope_dim=128, interleaved=False, theta=5e5,
                          max_seq_len=8192, capacity=8192, L=1, layer=0, cache_dtype=cache_dtype)


def prefill_tp8(seed: int = 2, small: bool = False, cache_dtype: Optional[str] = None) -> Case:
    """The prefill at one GPU's share under 8-way head (tensor) parallelism:
    a column-parallel QKV projection leaves each GPU Hq/8 = 4 Q heads and
    Hk/8 = 1 KV head, against a cache holding that one head."""
    B = 4 if small else 8
    lens = prng.integers(seed, S_LENS, B, 1, 300) if small else \
        prng.integers(seed, S_LENS, B, 128, 2048)
    return make_store_case(_kv("prefill_tp8_small" if small else "prefill_tp8", cache_dtype),
                           seed, BF16, lens, np.zeros(B, np.int64), Hq=4, Hk=1, D=128,
                           rope_dim=128, interleaved=False, theta=5e5, max_seq_len=8192, P=128,
                           L=4 if small else 32, layer=2 if small else 17,
                           cache_dtype=cache_dtype)


def decode_tp8(seed: int = 3, small: bool = False, cache_dtype: Optional[str] = None) -> Case:
    """The decode at one GPU's share under 8-way head parallelism: 4 Q heads
    and 1 KV head per token."""
    B = 32 if small else 256
    lens = np.ones(B, dtype=np.int64)
    clen = prng.integers(seed, S_CLEN, B, 0, 8191)
    return make_store_case(_kv("decode_tp8_small" if small else "decode_tp8", cache_dtype), seed,
                           BF16, lens, clen, Hq=4, Hk=1, D=128, rope_dim=128, interleaved=True,
                           theta=5e5, max_seq_len=8192, P=128, L=1, layer=0,
                           num_pages=1400 if small else 20000, max_pages=64,
                           cache_dtype=cache_dtype)


def dual_tp8(seed: int = 4, small: bool = False, cache_dtype: Optional[str] = None) -> Case:
    """The dual band at one GPU's share under 8-way head parallelism: main
    band 8 Q heads and 1 KV head; index band 2 Q heads and its single K head
    (a one-head cache cannot split: every rank keeps it whole)."""
    B = 4 if small else 16
    lens = prng.integers(seed, S_LENS, B, 1, 150 if small else 1024)
    return make_dual_case(_kv("dual_tp8_small" if small else "dual_tp8", cache_dtype), seed,
                          BF16, lens, Hq_main=8, Hk_main=1, Hq_index=2, D=128, rope_dim=64,
                          interleaved=True, theta=1e4, max_seq_len=8192, P_main=64, P_index=64,
                          main_cache_dtype=cache_dtype, index_cache_dtype=cache_dtype)


def _with_cache(fn, cache_dtype):
    def make(seed: Optional[int] = None, small: bool = False) -> Case:
        return fn(small=small, cache_dtype=cache_dtype) if seed is None else \
            fn(seed, small=small, cache_dtype=cache_dtype)
    make.__name__ = f"{fn.__name__}_{cache_dtype}"
    return make


WORKLOADS = {"tiny_fp32": tiny_fp32, "prefill": prefill, "decode": decode, "dual": dual,
             "radd": radd, "bshd": bshd, "prefill_tp8": prefill_tp8, "decode_tp8": decode_tp8,
             "dual_tp8": dual_tp8}
# the same workloads over FP8 caches (bf16 inputs; f32 scales, one per row)
WORKLOADS.update({f"{k}_fp8": _with_cache(WORKLOADS[k], FP8)
                  for k in ("prefill", "decode", "dual", "radd", "bshd")})


# ---------------------------------------------------------------------------
# fused GEMV + partial RMSNorm
# ---------------------------------------------------------------------------

@dataclass
class GemvCase:
    """y = x W^T for m input rows; the first n_normed columns RMS-normalised
    with gamma, the rest passed through.  Arrays hold raw bits of dtype, row
    strides in elements are the arrays' second dimensions (padding columns of
    x and W hold sentinels) and the output strides below."""
    name: str
    seed: int
    dtype: str
    m: int
    k: int
    n: int
    n_normed: int
    x: np.ndarray                 # [m, x_stride]
    w: np.ndarray                 # [n, w_stride]
    gamma: np.ndarray             # [n_normed] (one element when n_normed is 0)
    epsilon: float
    weight_offset: float
    normed_row_stride: int
    unnormed_row_stride: int
    op: str = "gemv_norm"
    transpose_b: int = 1          # 1: w is W [n, w_stride]; 0: w is W^T stored [k, w_stride]

    @property
    def T(self) -> int:     # input rows: the tokens of a step
        return self.m


def make_gemv_case(name: str, seed: int, dtype: str, m: int, k: int, n: int, n_normed: int,
                   epsilon: float = 1e-6, weight_offset: float = 0.0, x_pad: int = 0,
                   w_pad: int = 0, out_pad: int = 0, transpose_b: bool = True) -> GemvCase:
    """x ~ N(0, 1), W ~ N(0, 1/k) (so y is about N(0, 1)), gamma ~ N(1, 0.1).
    W's values do not depend on transpose_b: with transpose_b False the same
    [n, k] matrix is stored transposed, as [k, n + w_pad]."""
    x = np.full((m, k + x_pad), SENTINEL[dtype], dtype=BITS_DTYPE[dtype])
    x[:, :k] = to_bits(prng.normal(seed, S_X, m * k), dtype).reshape(m, k)
    wv = to_bits(prng.normal(seed, S_W, n * k, std=1.0 / np.sqrt(max(k, 1))), dtype).reshape(n, k)
    if transpose_b:
        w = np.full((n, k + w_pad), SENTINEL[dtype], dtype=BITS_DTYPE[dtype])
        w[:, :k] = wv
    else:
        w = np.full((k, n + w_pad), SENTINEL[dtype], dtype=BITS_DTYPE[dtype])
        w[:, :n] = wv.T
    gamma = to_bits(prng.normal(seed, S_GAMMA, max(n_normed, 1), mean=1.0, std=0.1), dtype)
    return GemvCase(name=name, seed=seed, dtype=dtype, m=m, k=k, n=n, n_normed=n_normed, x=x,
                    w=w, gamma=gamma, epsilon=epsilon, weight_offset=weight_offset,
                    normed_row_stride=max(n_normed, 1) + out_pad,
                    unnormed_row_stride=max(n - n_normed, 1) + out_pad,
                    transpose_b=1 if transpose_b else 0)


def gemv_norm(seed: int = 7, small: bool = False, transpose_b: bool = True) -> GemvCase:
    """One input row (a GEMV) of hidden size 7168 into 1536 normed and 576
    passed-through columns (the shape of a low-rank query / key-value
    projection); bf16.  The small form keeps the split at a tenth the size.
    transpose_b False stores the same W as [k][n]."""
    sfx = "" if transpose_b else "_t"
    if small:
        return make_gemv_case("gemv_norm_small" + sfx, seed, BF16, 1, 704, 216, 152,
                              transpose_b=transpose_b)
    return make_gemv_case("gemv_norm" + sfx, seed, BF16, 1, 7168, 2112, 1536,
                          transpose_b=transpose_b)


def gemv_norm_t(seed: int = 7, small: bool = False) -> GemvCase:
    """The gemv_norm projection with W stored [k][n] (transpose_b False)."""
    return gemv_norm(seed, small, transpose_b=False)


def gemv_norm_rows4(seed: int = 7, small: bool = False) -> GemvCase:
    """The same projection over four rows at once (a few decode tokens)."""
    if small:
        return make_gemv_case("gemv_norm_rows4_small", seed, BF16, 4, 704, 216, 152)
    return make_gemv_case("gemv_norm_rows4", seed, BF16, 4, 7168, 2112, 1536)


GEMV_WORKLOADS = {"gemv_norm": gemv_norm, "gemv_norm_rows4": gemv_norm_rows4,
                  "gemv_norm_t": gemv_norm_t}
