"""Device side of the tests and the benchmark: put a synthetic case on the GPU
and run it through the C ABI (via the thin Python binding).

Buffers hold raw bits (int16 for bf16 and f16, int32 for fp32, uint8 for
FP8 cache codes; FP8 scales as int32 / int16 bits of f32 / bf16).  Output buffers and
cache pools start as the signalling-NaN sentinel so that any stray write,
or any float round trip of a copied value, shows up in a bit comparison.
``q_output`` buffers carry GUARD sentinel rows before and after the rows
the call may write.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np
import torch

import qk_rope_paged_amd as qrp
from synth import cases as sc

GUARD = 2
TORCH_BITS = {sc.F32: torch.int32, sc.BF16: torch.int16, sc.F16: torch.int16, sc.FP8: torch.uint8}
QRP_DT = {sc.F32: qrp.QRP_F32, sc.BF16: qrp.QRP_BF16, sc.F16: qrp.QRP_F16, sc.FP8: qrp.QRP_FP8}


def bits_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(device)
    signed = a.view(np.int16 if a.dtype == np.uint16 else np.int32)
    return torch.from_numpy(signed).to(device)


def sentinel_int(dtype: str) -> int:
    s = int(sc.SENTINEL[dtype])
    if dtype == sc.FP8:
        return s                                   # a uint8 tensor
    bits = 32 if dtype == sc.F32 else 16
    return s - (1 << bits) if s >= 1 << (bits - 1) else s


def to_numpy_bits(t: torch.Tensor, dtype: str) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(sc.BITS_DTYPE[dtype])


@dataclass
class DeviceCache:
    host: sc.PagedCache
    pool: torch.Tensor                 # flat raw bits
    cache_lengths: torch.Tensor
    lookup_table: torch.Tensor
    desc: qrp.PagedCache = None
    scales: torch.Tensor = None        # FP8 caches: flat scale bits

    def pages(self, page_ids: np.ndarray) -> np.ndarray:
        """Copy the given pages back, shaped like the host pool."""
        view = self.pool.view(self.host.num_pages, self.host.page_elems)
        idx = torch.from_numpy(np.asarray(page_ids, dtype=np.int64)).to(self.pool.device)
        sel = view.index_select(0, idx)
        return to_numpy_bits(sel, self.host.dtype).reshape((len(page_ids),) + self.host.shape[1:])

    def scale_pages(self, page_ids: np.ndarray) -> np.ndarray:
        """FP8 caches: the scales of the given pages, shaped like the host's."""
        h = self.host
        per_page = int(np.prod(h.scale_shape[1:]))
        view = self.scales.view(h.num_pages, per_page)
        idx = torch.from_numpy(np.asarray(page_ids, dtype=np.int64)).to(self.scales.device)
        sel = view.index_select(0, idx)
        return to_numpy_bits(sel, h.scale_dtype).reshape((len(page_ids),) + h.scale_shape[1:])


def upload_cache(c: sc.PagedCache, device="cuda") -> DeviceCache:
    n = c.num_pages * c.page_elems
    pool = torch.full((n,), sentinel_int(c.dtype), dtype=TORCH_BITS[c.dtype], device=device)
    pg, pl, ly, sl, vals = c.prefill_arrays()
    if len(pg):
        row0 = np.ravel_multi_index((pg, pl, ly, sl, np.zeros_like(pg), np.zeros_like(pg)), c.shape)
        idx = row0[:, None] + np.arange(c.num_kv_heads * c.head_dim)[None, :]
        pool[torch.from_numpy(idx.reshape(-1)).to(device)] = bits_tensor(vals.reshape(-1), device)
    lens = torch.from_numpy(c.cache_lengths.astype(np.uint32).view(np.int32)).to(device)
    tab = torch.from_numpy(np.ascontiguousarray(c.lookup_table, dtype=np.uint32).view(np.int32)).to(device)
    st = c.strides
    scales, extra = None, {}
    if c.dtype == sc.FP8:
        scales = bits_tensor(c.materialize_scales().reshape(-1), device)
        sst = c.scale_strides
        extra = dict(scales=scales, scale_dtype=QRP_DT[c.scale_dtype],
                     scale_page_stride=sst["s_page_stride"], scale_plane_stride=sst["s_plane_stride"],
                     scale_layer_stride=sst["s_layer_stride"], scale_slot_stride=sst["s_slot_stride"],
                     scale_head_stride=sst["s_head_stride"])
    desc = qrp.PagedCache(**extra, blocks=pool, dtype=QRP_DT[c.dtype], num_kv_heads=c.num_kv_heads,
                          head_dim=c.head_dim, page_size=c.page_size, num_layers=c.num_layers,
                          kv_planes=c.kv_planes, num_pages=c.num_pages,
                          page_stride=st["page_stride"], plane_stride=st["plane_stride"],
                          layer_stride=st["layer_stride"], slot_stride=st["slot_stride"],
                          head_stride=st["head_stride"], cache_lengths=lens, lookup_table=tab,
                          cache_batch=c.cache_batch, max_pages_per_seq=c.max_pages_per_seq)
    return DeviceCache(host=c, pool=pool, cache_lengths=lens, lookup_table=tab, desc=desc,
                       scales=scales)


@dataclass
class DeviceCase:
    case: sc.Case
    buf: torch.Tensor
    offsets: torch.Tensor
    freqs: torch.Tensor
    caches: List[DeviceCache]
    q_out: List[torch.Tensor] = field(default_factory=list)      # with guard rows
    gammas: list = field(default_factory=list)
    valid: torch.Tensor = None                                    # bshd: valid lengths

    def q_out_rows(self, i: int) -> torch.Tensor:
        return self.q_out[i][GUARD:GUARD + self.case.T]


def upload(case: sc.Case, device="cuda") -> DeviceCase:
    buf = bits_tensor(case.buf, device) if case.buf.size else torch.zeros(
        (0, case.row_stride), dtype=TORCH_BITS[case.dtype], device=device)
    off = torch.from_numpy(case.offsets.astype(np.uint32).view(np.int32)).to(device)
    if case.freqs is None:
        freqs = torch.zeros(4, dtype=torch.float32, device=device)
    elif case.freq_dtype == sc.BF16:
        # the table holds bf16 values in float32: ship their top 16 bits
        hi = (np.ascontiguousarray(case.freqs, np.float32).view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal(hi.astype(np.uint32) << 16, case.freqs.view(np.uint32))
        freqs = bits_tensor(hi, device)
    elif case.freq_dtype == sc.F16:
        # binary16 values held in float32: the conversion back is exact
        h = np.ascontiguousarray(case.freqs, np.float32).astype(np.float16)
        assert np.array_equal(h.astype(np.float32), case.freqs)
        freqs = bits_tensor(h.view(np.uint16), device)
    else:
        freqs = torch.from_numpy(np.ascontiguousarray(case.freqs)).to(device)
    dc = DeviceCase(case=case, buf=buf, offsets=off, freqs=freqs,
                    caches=[upload_cache(c, device) for c in case.caches])
    strides = ([case.q_out_row_stride] if case.op in ("store", "bshd")
               else [b.q_out_row_stride for b in case.bands])
    if case.op == "bshd":
        dc.valid = torch.from_numpy(np.asarray(case.lengths, np.uint32).view(np.int32)).to(device)
    qdt = case.q_dtype
    for s in strides:
        dc.q_out.append(torch.full((case.T + 2 * GUARD, max(s, 1)), sentinel_int(qdt),
                                   dtype=TORCH_BITS[qdt], device=device))
    for b in case.bands:
        dc.gammas.append((None if b.q_gamma is None else bits_tensor(b.q_gamma, device),
                          None if b.k_gamma is None else bits_tensor(b.k_gamma, device)))
    return dc


def rope_of(dc: DeviceCase) -> qrp.Rope:
    c = dc.case
    return qrp.Rope(freqs_cis=dc.freqs, max_seq_len=c.max_seq_len, rope_dim=c.rope_dim,
                    interleaved=c.interleaved, freq_dtype=QRP_DT[c.freq_dtype],
                    rope_tail=c.rope_tail)


def band_of(dc: DeviceCase, i: int) -> qrp.Band:
    b = dc.case.bands[i]
    qg, kg = dc.gammas[i]
    return qrp.Band(q_col=b.q_col, n_q_heads=b.n_q_heads, k_col=b.k_col, v_col=b.v_col,
                    q_gamma=qg, k_gamma=kg, epsilon=b.epsilon, cache=dc.caches[b.cache].desc,
                    q_output=dc.q_out_rows(i), q_out_row_stride=b.q_out_row_stride)


# launch-shape overrides held around every unprepared run() call (a test
# sets them with monkeypatch.setattr), e.g. {"pack": 0}
OVERRIDES: dict = {}


def knobs(remap=None, ppw=None, wpb=None, pack=None, tail=None, lds=None):
    """qrp.launch_overrides from the tests' settings: "0" or 0 for a count
    (passes per wave, waves per block) is the library's choice."""
    def count(v):
        return None if v is None or int(v) == 0 else int(v)
    kw = {}
    if remap is not None:
        kw["xcd_remap"] = int(remap)
    if ppw is not None:
        kw["passes_per_wave"] = count(ppw)
    if wpb is not None:
        kw["waves_per_block"] = count(wpb)
    if pack is not None:
        kw["pack"] = int(pack)
    if tail is not None:
        kw["tail_units"] = int(tail)
    if lds is not None:
        kw["lds_bytes"] = int(lds)
    return qrp.launch_overrides(**kw)


def run(dc: DeviceCase, stream=None, raise_on_error=True, op=None, prepare=False):
    """One call of the case's operation through the C ABI (or, with
    ``prepare``, the call bound to its marshalled arguments)."""
    if OVERRIDES and not prepare:
        with knobs(**OVERRIDES):
            return _run(dc, stream, raise_on_error, op, prepare)
    return _run(dc, stream, raise_on_error, op, prepare)


def _run(dc: DeviceCase, stream, raise_on_error, op, prepare):
    c = dc.case
    op = op or c.op
    dt = QRP_DT[c.dtype]
    kw = dict(stream=stream, raise_on_error=raise_on_error, prepare=prepare)
    if op == "store":
        return qrp.rope_split_store_paged(
            dc.buf, dt, c.T, c.row_stride, c.n_q_heads, dc.offsets, c.batch, rope_of(dc),
            dc.caches[0].desc, c.layer_idx, dc.q_out_rows(0), QRP_DT[c.q_dtype],
            c.q_out_row_stride, **kw)
    if op == "norm":
        return qrp.qk_rmsnorm_rope_paged(
            dc.buf, dt, c.T, c.row_stride, band_of(dc, 0), c.weight_offset,
            c.multiply_before_cast, dc.offsets, c.batch, rope_of(dc), c.layer_idx, **kw)
    if op == "dual":
        return qrp.dual_band(
            dc.buf, dt, c.T, c.row_stride, band_of(dc, 0), band_of(dc, 1), c.weight_offset,
            c.multiply_before_cast, dc.offsets, c.batch, rope_of(dc), c.layer_idx, **kw)
    if op == "radd":
        return qrp.kv_cache_radd(
            dc.buf, dt, c.T, c.row_stride, dc.offsets, c.batch, c.batch_offset,
            dc.caches[0].desc, c.layer_idx, **kw)
    if op == "bshd":
        return qrp.fused_qk_rope_bshd_continuous_batch(
            dc.buf, dt, c.batch, c.seq_len, c.n_q_heads, dc.valid, rope_of(dc),
            dc.caches[0].desc, c.layer_idx, dc.q_out_rows(0), **kw)
    raise ValueError(op)


# ---------------------------------------------------------------------------
# fused GEMV + partial RMSNorm
# ---------------------------------------------------------------------------

@dataclass
class DeviceGemv:
    case: sc.GemvCase
    x: torch.Tensor
    w: torch.Tensor
    gamma: torch.Tensor
    normed: torch.Tensor
    unnormed: torch.Tensor
    workspace: torch.Tensor            # uint8, zero-filled once


def upload_gemv(case, device="cuda", workspace: torch.Tensor = None) -> DeviceGemv:
    """Operands as raw bits; outputs start as sentinels; a zero-filled
    workspace of the size the library asks for (or the one given)."""
    bits = TORCH_BITS[case.dtype]
    s = sentinel_int(case.dtype)
    normed = torch.full((case.m, case.normed_row_stride), s, dtype=bits, device=device)
    unnormed = torch.full((case.m, case.unnormed_row_stride), s, dtype=bits, device=device)
    if workspace is None:
        nbytes = max(qrp.gemv_norm_workspace_bytes(case.m, case.n_normed,
                                                   int(getattr(case, "transpose_b", 1))), 256)
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    return DeviceGemv(case=case, x=bits_tensor(case.x, device), w=bits_tensor(case.w, device),
                      gamma=bits_tensor(case.gamma, device), normed=normed, unnormed=unnormed,
                      workspace=workspace)


def run_gemv(dg: DeviceGemv, stream=None, raise_on_error=True, prepare=False,
             no_workspace=False):
    c = dg.case
    ws = None if no_workspace else dg.workspace
    return qrp.matmul_fused_partial_rmsnorm(
        dg.normed if c.n_normed else None, c.normed_row_stride,
        dg.unnormed if c.n_normed < c.n else None, c.unnormed_row_stride,
        dg.x, c.x.shape[1], c.m, dg.w, c.w.shape[1], c.n, c.k, dg.gamma, c.n_normed,
        c.epsilon, c.weight_offset, QRP_DT[c.dtype], ws,
        0 if ws is None else ws.numel(), transpose_b=int(getattr(c, "transpose_b", 1)),
        stream=stream, raise_on_error=raise_on_error, prepare=prepare)
