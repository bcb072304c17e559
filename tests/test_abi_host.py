"""Host-side checks of the C ABI, no GPU needed.

* the library loads and exports every function include/qk_rope_paged.h
  declares;
* the package ends up with one HIP runtime in the process (torch's);
* every invalid-argument path returns its status code before anything is
  launched (the pointers below are never dereferenced: the calls fail on the
  host first);
* qrp_validate_host finds each kind of inconsistent metadata.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import qk_rope_paged_amd as qrp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qk_rope_paged.h")
FAKE = 0x10000          # 16-byte aligned stand-in for a device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:int32_t|uint64_t|const char\s*\*)\s*(\w+)\s*\(", text, flags=re.M)


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert set(names) >= {"rope_split_store_paged", "qk_rmsnorm_rope_paged", "dual_band",
                          "kv_cache_radd", "qrp_validate", "qrp_validate_host",
                          "qrp_last_error", "qrp_abi_version"}
    lib = ctypes.CDLL(qrp.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(qrp.EXPORTS)
    assert qrp.abi_version() == 8


def test_launch_overrides_set_restore_and_reject():
    old = qrp.set_launch_override(qrp.QRP_KNOB_PACK, 1)
    assert qrp.set_launch_override(qrp.QRP_KNOB_PACK, old) == 1
    with qrp.launch_overrides(pack=0, passes_per_wave=2, waves_per_block=4, xcd_remap=1):
        assert qrp.set_launch_override(qrp.QRP_KNOB_PASSES_PER_WAVE, 2) == 2
        assert qrp.set_launch_override(qrp.QRP_KNOB_XCD_REMAP, 1) == 1
    assert qrp.set_launch_override(qrp.QRP_KNOB_PASSES_PER_WAVE, -1) == -1
    with qrp.launch_overrides(tail_units=7):
        assert qrp.set_launch_override(qrp.QRP_KNOB_TAIL_UNITS, 0) == 7
    for knob, value in ((6, 0), (-1, 0), (qrp.QRP_KNOB_LDS_BYTES, 65537), (qrp.QRP_KNOB_PACK, 2), (qrp.QRP_KNOB_TAIL_UNITS, -2),
                        (qrp.QRP_KNOB_PASSES_PER_WAVE, 0), (qrp.QRP_KNOB_WAVES_PER_BLOCK, 5),
                        (qrp.QRP_KNOB_XCD_REMAP, -2), (qrp.QRP_KNOB_XCD_REMAP, 3)):
        with pytest.raises(qrp.QrpError):
            qrp.set_launch_override(knob, value)
    with pytest.raises(ValueError):
        qrp.launch_overrides(bogus=1)


def test_launch_override_environment_is_read_once_at_load():
    # a fresh process: the variables set the first values; changing the
    # environment afterwards changes nothing
    import subprocess
    import sys
    code = ("import os, qk_rope_paged_amd as q\n"
            "os.environ['QRP_PACK'] = '0'\n"
            "print(q.set_launch_override(q.QRP_KNOB_PACK, -1),"
            " q.set_launch_override(q.QRP_KNOB_PASSES_PER_WAVE, -1),"
            " q.set_launch_override(q.QRP_KNOB_WAVES_PER_BLOCK, -1),"
            " q.set_launch_override(q.QRP_KNOB_XCD_REMAP, -1),"
            " q.set_launch_override(q.QRP_KNOB_TAIL_UNITS, -1),"
            " q.set_launch_override(q.QRP_KNOB_LDS_BYTES, -1))\n")
    env = dict(os.environ, QRP_PACK="1", QRP_PASSES_PER_WAVE="0", QRP_WAVES_PER_BLOCK="2",
               QRP_XCD_REMAP="1", QRP_TAIL_UNITS="0", QRP_LDS_BYTES="70000")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, check=True).stdout.split()
    # QRP_LDS_BYTES past 65536 is out of range: the library's choice stays
    assert out == ["1", "-1", "2", "1", "0", "-1"]


def test_noalloc_gemv_rejects_sizes_past_its_scratch_on_the_host():
    # m * n_normed above the library's scratch: QRP_EINVAL before any device call
    st = qrp.matmul_fused_partial_rmsnorm_noalloc(
        FAKE, 65537, FAKE, 64, FAKE, 64, 2, FAKE, 64, 65600, 64, FAKE, 65537, 1e-6, 0.0,
        qrp.QRP_BF16, stream=0, raise_on_error=False)
    assert st == qrp.QRP_EINVAL and "scratch" in qrp.last_error()
    # the workspace form is still checked as before
    st = qrp.matmul_fused_partial_rmsnorm(FAKE, 64, FAKE, 16, FAKE, 64, 1, FAKE, 64, 80, 64, FAKE,
                                          64, 1e-6, 0.0, qrp.QRP_BF16, FAKE, 16, stream=0,
                                          raise_on_error=False)
    assert st == qrp.QRP_EINVAL and "workspace" in qrp.last_error()


def test_one_hip_runtime_in_process():
    maps = open("/proc/self/maps").read()
    libs = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(libs) <= 1, libs


def _cache(**kw):
    d = dict(blocks=FAKE, dtype=qrp.QRP_BF16, num_kv_heads=8, head_dim=128, page_size=128,
             num_layers=2, kv_planes=2, num_pages=16, page_stride=2 * 2 * 128 * 8 * 128,
             plane_stride=2 * 128 * 8 * 128, layer_stride=128 * 8 * 128, slot_stride=8 * 128,
             head_stride=128, cache_lengths=FAKE, lookup_table=FAKE, cache_batch=4,
             max_pages_per_seq=4)
    d.update(kw)
    return qrp.PagedCache(**d)


def _rope(**kw):
    d = dict(freqs_cis=FAKE, max_seq_len=512, rope_dim=128, interleaved=True)
    d.update(kw)
    return qrp.Rope(**d)


def _store(cache=None, rope=None, **kw):
    a = dict(qkv=FAKE, dtype=qrp.QRP_BF16, total_seq_len=8, qkv_row_stride=48 * 128, n_q_heads=32,
             input_row_offsets=FAKE, batch_size=2, rope=rope or _rope(), cache=cache or _cache(),
             layer_idx=1, q_output=FAKE, q_out_dtype=qrp.QRP_BF16, q_out_row_stride=32 * 128,
             stream=0, raise_on_error=False)
    a.update(kw)
    return qrp.rope_split_store_paged(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), qrp.QRP_EUNSUPPORTED),
    (dict(q_out_dtype=7), qrp.QRP_EUNSUPPORTED),
    (dict(batch_size=0), qrp.QRP_EINVAL),
    (dict(input_row_offsets=None), qrp.QRP_EINVAL),
    (dict(qkv=None), qrp.QRP_EINVAL),
    (dict(q_output=None), qrp.QRP_EINVAL),
    (dict(qkv=FAKE + 8), qrp.QRP_EALIGN),
    (dict(q_output=FAKE + 4), qrp.QRP_EALIGN),
    (dict(qkv_row_stride=48 * 128 + 4), qrp.QRP_EALIGN),
    (dict(qkv_row_stride=47 * 128), qrp.QRP_EINVAL),
    (dict(q_out_row_stride=31 * 128), qrp.QRP_EINVAL),
    (dict(n_q_heads=0), qrp.QRP_EINVAL),
    (dict(layer_idx=2), qrp.QRP_EINVAL),
    (dict(batch_size=5), qrp.QRP_EINVAL),
    (dict(cache=_cache(head_dim=96)), qrp.QRP_EUNSUPPORTED),
    (dict(cache=_cache(dtype=qrp.QRP_F32)), qrp.QRP_EUNSUPPORTED),
    (dict(cache=_cache(kv_planes=1)), qrp.QRP_EINVAL),
    (dict(cache=_cache(page_size=0)), qrp.QRP_EINVAL),
    (dict(cache=_cache(blocks=FAKE + 2)), qrp.QRP_EALIGN),
    (dict(cache=_cache(head_stride=100)), qrp.QRP_EALIGN),
    (dict(cache=_cache(lookup_table=None)), qrp.QRP_EINVAL),
    (dict(rope=_rope(rope_dim=130)), qrp.QRP_EINVAL),
    (dict(rope=_rope(rope_dim=7)), qrp.QRP_EINVAL),
    (dict(rope=_rope(rope_dim=8)), qrp.QRP_EUNSUPPORTED),
    (dict(rope=_rope(max_seq_len=0)), qrp.QRP_EINVAL),
    (dict(rope=_rope(freqs_cis=None)), qrp.QRP_EINVAL),
    (dict(rope=_rope(freq_dtype=3)), qrp.QRP_EUNSUPPORTED),
    (dict(rope=_rope(freq_dtype=9)), qrp.QRP_EUNSUPPORTED),
    (dict(rope=_rope(freqs_cis=FAKE + 8, freq_dtype=qrp.QRP_BF16)), qrp.QRP_EALIGN),
    (dict(dtype=qrp.QRP_F16, q_out_dtype=qrp.QRP_F16), qrp.QRP_EUNSUPPORTED),   # cache is bf16
    (dict(dtype=qrp.QRP_F16, q_out_dtype=qrp.QRP_BF16, cache=_cache(dtype=qrp.QRP_F16),
          q_out_row_stride=32 * 128 + 4), qrp.QRP_EALIGN),
    (dict(dtype=qrp.QRP_F16, q_out_dtype=qrp.QRP_F16, cache=_cache(dtype=qrp.QRP_F16),
          rope=_rope(rope_dim=8)), qrp.QRP_EUNSUPPORTED),
    (dict(dtype=qrp.QRP_F16, q_out_dtype=qrp.QRP_F16, cache=_cache(dtype=qrp.QRP_F16),
          qkv=FAKE + 8), qrp.QRP_EALIGN),
])
def test_store_argument_errors(kw, code):
    assert _store(**kw) == code
    assert qrp.last_error() != ""


def test_empty_batch_returns_ok_without_touching_anything():
    assert _store(total_seq_len=0, qkv=None, q_output=None, input_row_offsets=None) == qrp.QRP_OK


def _band(cache=None, **kw):
    d = dict(q_col=0, n_q_heads=64, k_col=-1, v_col=-1, q_gamma=FAKE, k_gamma=FAKE, epsilon=1e-6,
             cache=cache or _cache(), q_output=FAKE, q_out_row_stride=64 * 128)
    d.update(kw)
    return qrp.Band(**d)


def _dual(main=None, index=None, **kw):
    idx_cache = _cache(num_kv_heads=1, kv_planes=1, page_stride=128 * 128, plane_stride=128 * 128,
                       layer_stride=128 * 128, slot_stride=128)
    a = dict(buf=FAKE, dtype=qrp.QRP_BF16, total_seq_len=8, buf_row_stride=96 * 128,
             main_band=main or _band(),
             index_band=index or _band(cache=idx_cache, q_col=80 * 128, n_q_heads=16,
                                       q_out_row_stride=16 * 128),
             weight_offset=0.0, multiply_before_cast=True, input_row_offsets=FAKE, batch_size=2,
             rope=_rope(rope_dim=64), layer_idx=0, stream=0, raise_on_error=False)
    a.update(kw)
    return qrp.dual_band(**a)


def test_dual_band_geometry_and_argument_errors():
    assert _dual(index=_band(cache=_cache(head_dim=64, num_kv_heads=1), n_q_heads=16)) == \
        qrp.QRP_EGEOMETRY
    assert _dual(index=_band(cache=_cache(dtype=qrp.QRP_F32), n_q_heads=16)) == \
        qrp.QRP_EUNSUPPORTED                                           # cache dtype != op dtype
    assert _dual(main=_band(k_col=64 * 128, v_col=72 * 128)) == qrp.QRP_EUNSUPPORTED
    assert _dual(main=_band(q_col=40 * 128)) == qrp.QRP_EINVAL          # Q past the row end
    assert _dual(main=_band(q_gamma=FAKE + 2)) == qrp.QRP_EALIGN
    assert _dual(main=_band(q_output=None)) == qrp.QRP_EINVAL
    assert _dual(buf_row_stride=96 * 128 + 3) == qrp.QRP_EALIGN


def test_norm_band_errors():
    def call(band, **kw):
        a = dict(qkv=FAKE, dtype=qrp.QRP_BF16, total_seq_len=4, qkv_row_stride=48 * 128,
                 band=band, weight_offset=0.0, multiply_before_cast=True, input_row_offsets=FAKE,
                 batch_size=1, rope=_rope(), layer_idx=0, stream=0, raise_on_error=False)
        a.update(kw)
        return qrp.qk_rmsnorm_rope_paged(**a)
    assert call(_band(n_q_heads=32, v_col=40 * 128)) == qrp.QRP_EINVAL      # V without K column
    assert call(_band(n_q_heads=32, k_col=32 * 128, v_col=40 * 128,
                      cache=_cache(kv_planes=1))) == qrp.QRP_EINVAL          # V without V plane
    assert call(_band(n_q_heads=32, k_col=41 * 128)) == qrp.QRP_EINVAL      # K past the row end
    assert call(_band(n_q_heads=32, q_col=4)) == qrp.QRP_EALIGN


def test_radd_errors():
    def call(**kw):
        a = dict(a=FAKE, dtype=qrp.QRP_BF16, total_rows=4, a_row_stride=2 * 8 * 128,
                 input_row_offsets=FAKE, batch_size=2, batch_offset=2, cache=_cache(),
                 layer_idx=0, stream=0, raise_on_error=False)
        a.update(kw)
        return qrp.kv_cache_radd(**a)
    assert call(batch_offset=3) == qrp.QRP_EINVAL                  # 3 + 2 > cache_batch 4
    assert call(a_row_stride=2 * 8 * 128 - 8) == qrp.QRP_EINVAL
    assert call(cache=_cache(kv_planes=1)) == qrp.QRP_EINVAL
    assert call(a=FAKE + 6) == qrp.QRP_EALIGN
    assert call(total_rows=0, a=None) == qrp.QRP_OK


def test_raise_on_error_raises():
    with pytest.raises(qrp.QrpError) as e:
        _store(dtype=9, raise_on_error=True)
    assert e.value.status == qrp.QRP_EUNSUPPORTED


# --------------------------------------------------------------------------
# qrp_validate_host
# --------------------------------------------------------------------------

def _meta():
    off = np.array([0, 3, 3, 8], np.uint32)               # sequence 1 is empty
    lens = np.array([0, 40, 4, 0], np.uint32)
    tab = np.arange(16, dtype=np.uint32).reshape(4, 4)
    return off, lens, tab


def _validate(off, lens, tab, B=3, T=8, boff=0, P=16, num_pages=16, msl=64):
    return qrp.qrp_validate_host(off, B, T, boff, lens, tab, tab.shape[0], tab.shape[1], P,
                                 num_pages, msl)


def test_validate_accepts_good_metadata():
    off, lens, tab = _meta()
    assert _validate(off, lens, tab) == qrp.QRP_OK
    assert _validate(off, lens, tab, boff=1) == qrp.QRP_OK


@pytest.mark.parametrize("mutate,fragment", [
    (lambda o, l, t: o.__setitem__(0, 1), "offsets[0]"),
    (lambda o, l, t: o.__setitem__(2, 2), "decrease"),
    (lambda o, l, t: o.__setitem__(3, 9), "total_seq_len"),
    (lambda o, l, t: l.__setitem__(2, 60), "max_seq_len"),
    (lambda o, l, t: t.__setitem__((2, 0), 99), "num_pages"),
    (lambda o, l, t: (t.__setitem__((2, 0), 0), l.__setitem__(2, 1)), "same cache row"),
])
def test_validate_finds_bad_metadata(mutate, fragment):
    off, lens, tab = _meta()
    mutate(off, lens, tab)
    assert _validate(off, lens, tab) == qrp.QRP_EDATA
    assert fragment in qrp.last_error()


def test_validate_allows_shared_pages_with_distinct_rows():
    off, lens, tab = _meta()
    tab[2, 0] = 0            # sequence 2 writes rows 4..8 of the page sequence 0 writes rows 0..2 of
    assert _validate(off, lens, tab) == qrp.QRP_OK


def test_validate_page_index_and_batch_offset_bounds():
    off, lens, tab = _meta()
    lens[2] = 60                                              # positions 60..64 -> page index 4
    assert _validate(off, lens, tab, msl=0) == qrp.QRP_EDATA
    assert "max_pages_per_seq" in qrp.last_error()
    off, lens, tab = _meta()
    assert _validate(off, lens, tab, boff=2) == qrp.QRP_EDATA   # 2 + 3 > 4 sequences


def _bshd(cache=None, rope=None, **kw):
    a = dict(q_proj=FAKE, dtype=qrp.QRP_BF16, batch_size=2, seq_len=16, n_q_heads=32,
             valid_lengths=FAKE, rope=rope or _rope(), cache=cache or _cache(), layer_idx=1,
             output=FAKE + 4096, stream=0, raise_on_error=False)
    a.update(kw)
    return qrp.fused_qk_rope_bshd_continuous_batch(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), qrp.QRP_EUNSUPPORTED),
    (dict(q_proj=None), qrp.QRP_EINVAL),
    (dict(output=None), qrp.QRP_EINVAL),
    (dict(valid_lengths=None), qrp.QRP_EINVAL),
    (dict(n_q_heads=0), qrp.QRP_EINVAL),
    (dict(q_proj=FAKE + 8), qrp.QRP_EALIGN),
    (dict(output=FAKE + 2), qrp.QRP_EALIGN),
    (dict(valid_lengths=FAKE + 2), qrp.QRP_EALIGN),
    (dict(batch_size=5), qrp.QRP_EINVAL),
    (dict(batch_size=4, seq_len=1 << 30), qrp.QRP_EINVAL),
    (dict(layer_idx=2), qrp.QRP_EINVAL),
    (dict(cache=_cache(dtype=qrp.QRP_F16)), qrp.QRP_EUNSUPPORTED),
    (dict(cache=_cache(head_dim=80)), qrp.QRP_EUNSUPPORTED),
    (dict(rope=_rope(rope_dim=130)), qrp.QRP_EINVAL),
    (dict(rope=_rope(freq_dtype=4)), qrp.QRP_EUNSUPPORTED),
    (dict(rope=_rope(max_seq_len=0)), qrp.QRP_EINVAL),
])
def test_bshd_argument_errors(kw, code):
    assert _bshd(**kw) == code
    assert qrp.last_error() != ""


def test_bshd_empty_grid_returns_ok_without_touching_anything():
    assert _bshd(batch_size=0, q_proj=None, output=None, valid_lengths=None) == qrp.QRP_OK
    assert _bshd(seq_len=0, q_proj=None, output=None, valid_lengths=None) == qrp.QRP_OK



def _fp8_cache(**kw):
    d = dict(dtype=qrp.QRP_FP8, scales=FAKE + (1 << 20), scale_dtype=qrp.QRP_F32,
             scale_page_stride=2 * 2 * 128 * 8, scale_plane_stride=2 * 128 * 8,
             scale_layer_stride=128 * 8, scale_slot_stride=8, scale_head_stride=1)
    d.update(kw)
    return _cache(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(cache=_fp8_cache(scales=None)), qrp.QRP_EINVAL),
    (dict(cache=_fp8_cache(scale_dtype=qrp.QRP_F16)), qrp.QRP_EUNSUPPORTED),
    (dict(cache=_fp8_cache(scale_dtype=qrp.QRP_FP8)), qrp.QRP_EUNSUPPORTED),
    (dict(cache=_fp8_cache(scales=FAKE + 2)), qrp.QRP_EALIGN),
    (dict(cache=_fp8_cache(scale_slot_stride=-8)), qrp.QRP_EINVAL),
    (dict(cache=_fp8_cache(head_stride=100)), qrp.QRP_EALIGN),
    (dict(cache=_fp8_cache(), qkv=FAKE + 4), qrp.QRP_EALIGN),
    (dict(cache=_fp8_cache(), q_out_dtype=qrp.QRP_FP8), qrp.QRP_EUNSUPPORTED),
    (dict(cache=_fp8_cache(), q_out_dtype=qrp.QRP_F32, q_out_row_stride=32 * 128 + 2),
     qrp.QRP_EALIGN),
])
def test_fp8_cache_and_q_dtype_argument_errors(kw, code):
    assert _store(**kw) == code
    assert qrp.last_error() != ""


def test_dual_band_mixed_fp8_and_plain_caches_pass_the_host_checks():
    # one plain and one FP8 cache is a supported pairing: every host check
    # passes and the call gets as far as the launch (QRP_EHIP without a GPU)
    idx_cache = _fp8_cache(num_kv_heads=1, kv_planes=1, page_stride=128 * 128,
                           plane_stride=128 * 128, layer_stride=128 * 128, slot_stride=128)
    st = _dual(index=_band(cache=idx_cache, q_col=80 * 128, n_q_heads=16,
                           q_out_row_stride=16 * 128))
    assert st in (qrp.QRP_OK, qrp.QRP_EHIP), qrp.last_error()
    # the FP8 side is still checked like any FP8 cache
    bad = _fp8_cache(num_kv_heads=1, kv_planes=1, page_stride=128 * 128, plane_stride=128 * 128,
                     layer_stride=128 * 128, slot_stride=128, scales=None)
    assert _dual(index=_band(cache=bad, q_col=80 * 128, n_q_heads=16,
                             q_out_row_stride=16 * 128)) == qrp.QRP_EINVAL


def _gemv(**kw):
    a = dict(normed_output=FAKE, normed_row_stride=1536, unnormed_output=FAKE,
             unnormed_row_stride=576, input=FAKE, input_row_stride=7168, m=1, weight=FAKE,
             weight_row_stride=7168, n=2112, k=7168, gamma=FAKE, n_normed=1536, epsilon=1e-6,
             weight_offset=0.0, dtype=qrp.QRP_BF16, workspace=FAKE,
             workspace_bytes=qrp.gemv_norm_workspace_bytes(1, 1536), stream=0,
             raise_on_error=False)
    a.update(kw)
    return qrp.matmul_fused_partial_rmsnorm(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=qrp.QRP_FP8), qrp.QRP_EUNSUPPORTED),
    (dict(transpose_b=2), qrp.QRP_EINVAL),
    (dict(transpose_b=0, weight_row_stride=2104), qrp.QRP_EINVAL),   # W [k][n]: stride < n
    (dict(transpose_b=0, weight_row_stride=2116), qrp.QRP_EALIGN),   # not 16-byte rows
    (dict(transpose_b=0, weight_row_stride=2112), qrp.QRP_EINVAL),   # [n][k]-sized workspace
    (dict(transpose_b=0, weight_row_stride=2112, n_normed=0, normed_output=None, gamma=None,
          workspace=None, workspace_bytes=0), qrp.QRP_EINVAL),       # [k][n] always needs one
    (dict(m=9), qrp.QRP_EUNSUPPORTED),
    (dict(n_normed=2113), qrp.QRP_EINVAL),
    (dict(input=None), qrp.QRP_EINVAL),
    (dict(weight=None), qrp.QRP_EINVAL),
    (dict(gamma=None), qrp.QRP_EINVAL),
    (dict(normed_output=None), qrp.QRP_EINVAL),
    (dict(workspace=None), qrp.QRP_EINVAL),
    (dict(unnormed_output=None), qrp.QRP_EINVAL),
    (dict(workspace_bytes=qrp.gemv_norm_workspace_bytes(1, 1536) - 4), qrp.QRP_EINVAL),
    (dict(m=2), qrp.QRP_EINVAL),                              # workspace sized for one row
    (dict(input=FAKE + 8), qrp.QRP_EALIGN),
    (dict(weight=FAKE + 8), qrp.QRP_EALIGN),
    (dict(workspace=FAKE + 8), qrp.QRP_EALIGN),
    (dict(normed_output=FAKE + 1), qrp.QRP_EALIGN),
    (dict(gamma=FAKE + 1), qrp.QRP_EALIGN),
    (dict(k=7164, input_row_stride=7164, weight_row_stride=7164), qrp.QRP_EALIGN),
    (dict(weight_row_stride=7172), qrp.QRP_EALIGN),
    (dict(input_row_stride=7160), qrp.QRP_EINVAL),
    (dict(weight_row_stride=7160), qrp.QRP_EINVAL),
    (dict(normed_row_stride=1535), qrp.QRP_EINVAL),
    (dict(unnormed_row_stride=575), qrp.QRP_EINVAL),
    (dict(n=1 << 31, unnormed_row_stride=(1 << 31) - 1536), qrp.QRP_EINVAL),
])
def test_gemv_norm_argument_errors(kw, code):
    assert _gemv(**kw) == code
    assert qrp.last_error() != ""


def test_gemv_norm_degenerate_sizes_and_workspace_size():
    # nothing to compute: no launch, no pointer read
    assert _gemv(m=0, input=None, weight=None, workspace=None) == qrp.QRP_OK
    assert _gemv(n=0, n_normed=0, input=None, weight=None) == qrp.QRP_OK
    # the workspace is the counters plus m * n_normed binary32 values; with W
    # stored [n][k] none without a norm; with W stored [k][n] the slices'
    # partial sums follow, from a 256-byte boundary
    assert qrp.gemv_norm_workspace_bytes(3, 100) == 1280 + 4 * 3 * 100
    assert qrp.gemv_norm_workspace_bytes(8, 0) == 0
    assert qrp.gemv_norm_workspace_bytes(3, 100, 0) == 1280 + 1280 + 65536 * 3
    assert qrp.gemv_norm_workspace_bytes(8, 0, 0) == 1280 + 65536 * 8
    assert qrp.gemv_norm_workspace_bytes(1, 1536, 0) == 1280 + 6144 + 65536
