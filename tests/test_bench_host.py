"""Host logic of bench.py, on the CPU: the byte model against a hand count,
and the source hash that decides whether a committed counter summary still
describes the kernels."""
from __future__ import annotations

import bench
from synth import cases as sc


def test_algorithmic_bytes_of_the_tiny_case_by_hand():
    # tiny_fp32: fp32, 2 sequences of 3 and 5 tokens at cache lengths 0 and 4,
    # 4 Q and 2 KV heads of 64, page size 16, rope width 64
    case = sc.tiny_fp32()
    head = 64 * 4
    per_token = 4 * head * 2 + 2 * head * 2 + 2 * head * 2   # Q, K, V read and written
    freqs = 8 * 64 * 4              # positions 0-2 and 4-8: 8 distinct rows
    metadata = 3 * 4 + 2 * 4 + 2 * 4  # offsets, cache lengths, one page entry per sequence
    assert bench.algorithmic_bytes(case) == 8 * per_token + freqs + metadata


def test_code_only_strips_comments_and_keeps_literals():
    src = ('int a = 1;  // trailing\n'
           '/* block\n   comment */\n'
           '\n'
           'const char* s = "not // a comment /* either */";\n'
           "char c = '/';  /* x */ int b = 2;\n")
    assert bench._code_only(src) == ('int a = 1;\n'
                                     'const char* s = "not // a comment /* either */";\n'
                                     "char c = '/';   int b = 2;")


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    f = tmp_path / "k.hpp"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ("k.hpp",))
    f.write_text("int f() { return 1; }\n")
    h0 = bench.kernel_source_hash()
    f.write_text("// a note\nint f() { return 1; }  /* same code */\n\n")
    assert bench.kernel_source_hash() == h0
    f.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != h0


def test_cpu_model_reads_proc_cpuinfo():
    # a string on any host (empty where /proc/cpuinfo has no model line)
    assert isinstance(bench._cpu_model(), str)


def test_gemv_bytes_by_hand_and_its_own_source_hash():
    # one bf16 row of 7168 into 2112 columns, 1536 of them normed
    case = bench.make_case("gemv_norm")
    w, x, gamma, out = 2112 * 7168 * 2, 7168 * 2, 1536 * 2, 2112 * 2
    assert bench.algorithmic_bytes(case) == w + x + gamma + out
    assert bench.case_tokens(case) == 1
    assert bench.kernel_name("gemv_norm") == bench.GEMV_KERNEL_NAME
    assert bench.source_hash_for("gemv_norm") != bench.source_hash_for("prefill")
    four = bench.make_case("gemv_norm_rows4")
    assert bench.algorithmic_bytes(four) == w + 4 * x + gamma + 4 * out
    assert bench.case_tokens(four) == 4


def test_percentiles_nearest_rank():
    p = bench.percentiles(list(range(1, 101)))
    assert p == {10: 11, 50: 51, 90: 91}
    assert bench.percentiles([5.0]) == {10: 5.0, 50: 5.0, 90: 5.0}


def test_counter_summary_gives_traffic_and_tcc_hit_rate(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "qk_rope_paged_amd" / "csrc"
    src.mkdir(parents=True)
    for rel in bench.KERNEL_SOURCES:
        (tmp_path / rel).write_text("int k;\n")
    h = bench.kernel_source_hash()
    (tmp_path / "profiles" / "band_kernel_decode_traffic.txt").write_text(
        "# header\n"
        f"kernel_source_sha256: {h}\n"
        "seed_3_bytes: 100 50   # read, written\n"
        "seed_103_bytes: 300 150   # read, written\n"
        "tcc_hit_rate: 0.4500   # TCC_HIT / (TCC_HIT + TCC_MISS)\n")
    assert bench.traffic_from_profiles("decode", [3, 103, 3, 103]) == 300
    assert bench.tcc_hit_rate_from_profiles("decode") == 0.45
    # a summary of other kernel code is not used
    (tmp_path / bench.KERNEL_SOURCES[0]).write_text("int k2;\n")
    assert bench.traffic_from_profiles("decode", [3]) is None
    assert bench.tcc_hit_rate_from_profiles("decode") is None
