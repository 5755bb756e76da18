"""Host-side checks of bench.py (no GPU): its algorithmic byte and FLOP counts against the
per-step figures worked out independently from the workload shapes, and its refusal of more
than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import dsa_inputs as DI  # noqa: E402


# Decode, 32 x 16384: k_I 32*16384*256 + rows 32*2048*1152 + q/out 32*64*(576+512)*2
# + q_I/w 32*32*(256+4). IndexShare: one k_I stream and four layers of rows, q and out.
# Mixed lengths: the k_I rows of every sequence, min(2048, L) rows each, q/out/q_I/w per query.
# MTP, 32 x 16384 with 4 new tokens each: the k_I rows once per sequence (32*16384*256), rows,
# q/out and q_I/w per token (128 tokens).
@pytest.mark.parametrize("name,step,mla", [
    ("decode_b32_l16k", 214_437_888, 79_953_920),
    ("indexshare_b8_l256k", 616_891_392, 19_988_480),
    ("mixed_b16_l512_1m", 949_534_848, 33_706_624),
    ("mtp_b32_l16k_q4", 32 * 16384 * 256 + 128 * (2048 * 1152 + 64 * 1088 * 2 + 32 * 260),
     128 * (2048 * 1152 + 64 * 1088 * 2)),
])
def test_step_bytes(name, step, mla):
    case = DI.CASES[name]
    assert bench.step_bytes(case) == step
    assert bench.mla_bytes(case) == mla


def test_decode_bytes_closed_form():
    b, L, k = 32, 16384, 2048
    want = b * L * 128 * 2 + b * k * 576 * 2 + b * 64 * (576 + 512) * 2 + b * 32 * (128 * 2 + 4)
    assert bench.step_bytes(DI.CASES["decode_b32_l16k"]) == want


def test_prefill_key_rows_counted_once():
    """The chunk's 8192 queries share one key stream: 65536 rows of 256 B, not one per query."""
    case = DI.CASES["prefill_chunk8k_l64k"]
    assert bench.indexer_bytes(case) == 65536 * 256 + 8192 * 32 * 260


def test_prefill_flops():
    case = DI.CASES["prefill_chunk8k_l64k"]
    # queries at positions 57344..65535 each see p + 1 keys: sum = 8192*57344 + 8192*8193/2
    pairs = 8192 * 57344 + 8192 * 8193 // 2
    assert bench.indexer_flops(case) == 2 * 32 * 128 * pairs == 4_123_202_158_592
    assert bench.mla_flops(case) == 2 * 64 * (576 + 512) * 2048 * 8192 == 2_336_462_209_024


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_record_needs_every_current_source(tmp_path, monkeypatch):
    """A traffic record counts only while it lists every kernel source of the tree with the
    digest the counters were taken at: a changed, added or missing source voids it."""
    csrc = tmp_path / "long_context_lightning_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (csrc / "a.hip").write_text("int a;  // comment\n")
    (csrc / "b.hpp").write_text("int b;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))

    def write(shas):
        rec = {"code_sha256": shas, "kernel": "sparse_mla", "traffic_bytes_per_launch": 123}
        (tmp_path / "profiles" / "w_hbm_traffic.md").write_text("traffic-record: " + json.dumps(rec) + "\n")

    good = {n: bench.code_digest(str(csrc / n)) for n in ("a.hip", "b.hpp")}
    write(good)
    assert bench.traffic_record("w", "sparse_mla") == 123
    (csrc / "a.hip").write_text("int a;  // another comment\n")          # comments only
    assert bench.traffic_record("w", "sparse_mla") == 123
    write({"a.hip": good["a.hip"]})                                      # b.hpp not covered
    assert bench.traffic_record("w", "sparse_mla") is None
    write(good)
    (csrc / "c.hpp").write_text("int c;\n")                              # a source added
    assert bench.traffic_record("w", "sparse_mla") is None
    (csrc / "c.hpp").unlink()
    (csrc / "b.hpp").write_text("int b2;\n")                             # code changed
    assert bench.traffic_record("w", "sparse_mla") is None


def test_fp32_workload_bytes():
    """The tiny fp32 prefill (one sequence of 256 tokens, indexer 4 x 32, top-64, 8 heads over
    80-wide rows with 64 value columns) counts 4-byte elements: key rows 256*32*4 = 32768;
    gathered rows sum_t min(64, t+1) = 2080 + 192*64 = 14368 rows of 80*4 B = 4597760; queries
    and outputs 256*8*(80+64)*4 = 1179648; q_I and w 256*4*(32*4+4) = 135168."""
    case = DI.CASES["tiny_prefill_fp32"]
    assert bench.step_bytes(case, 4, 4) == 32768 + 4597760 + 1179648 + 135168
    assert bench.indexer_bytes(case, 4) == 32768 + 135168
    assert bench.mla_bytes(case, 4) == 4597760 + 1179648
