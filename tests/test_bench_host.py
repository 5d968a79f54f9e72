"""Host-side logic of bench.py (no GPU): the one-GPU rule, the gating of the
stored HBM-traffic counters by kernel source, and the algorithmic byte count
the roofline divides by."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from video_dit_trainable_amd.configs import WORKLOADS, compulsory_bytes, gather_bytes, op_bytes  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_stored_traffic_is_gated_by_the_kernel_source(tmp_path, monkeypatch):
    rec = {"bwd_dkdv/train720": {"bytes_per_launch": 123, "source_sha256_16": bench.source_hash("bwd_dkdv")},
           "fine_fwd/train720": {"bytes_per_launch": 456, "source_sha256_16": "0000000000000000"}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.stored_traffic("bwd_dkdv", "train720") == 123   # counters taken on this source
    assert bench.stored_traffic("fine_fwd", "train720") is None  # source changed since
    assert bench.stored_traffic("bwd_dq", "train720") is None    # never measured
    assert bench.stored_traffic("bwd_dkdv", "train720pad") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.stored_traffic("bwd_dkdv", "train720") is None


def test_source_hash_covers_the_shared_header():
    # the fine backward kernels share a source file, so they share a hash; the
    # router's differs
    assert bench.source_hash("bwd_dkdv") == bench.source_hash("bwd_dq")
    assert bench.source_hash("bwd_dkdv") != bench.source_hash("router_lse")
    assert len(bench.source_hash("fine_fwd")) == 16


def test_dkdv_gather_bytes_at_720p():
    # the per-unit figure times the units of one launch, counted by hand:
    # 20 heads x 3,432 query cubes x top64 = 4,392,960 selected pairs, each
    # gathering a 64 x 128 bf16 Q tile and dO tile (32 KiB), the 64 rows'
    # (lse, delta) fp32 pairs (512 B) and one 4-byte list entry; per head,
    # K, V, dK, dV once (4 x 219,648 x 128 x 2 B), the coarse dK_c, dV_c rows
    # (2 x 3,432 x 128 x 4 B) and the 3,433 CSC column pointers
    pairs = 20 * 3432 * 64
    per_pair = 2 * 64 * 128 * 2 + 64 * 8 + 4
    per_head = 4 * 219648 * 128 * 2 + 2 * 3432 * 128 * 4 + 3433 * 4
    want = pairs * per_pair + 20 * per_head
    assert pairs == 4_392_960
    assert gather_bytes(WORKLOADS["train720"])["bwd_dkdv"] == want == 150_784_233_680


def test_compulsory_bytes_at_720p():
    # forward: Q, K, V read and O_f written once (4 x 219,648 x 128 bf16 per
    # head), the fp32 LSE of every row, the CSR (219,648 entries + 3,433 row
    # pointers); 20 heads: the 4.52 GB floor of the fine forward
    tok = 219648 * 128 * 2
    idx = 219648 * 4 + 3433 * 4
    fwd = 20 * (4 * tok + 219648 * 4 + idx)
    cb = compulsory_bytes(WORKLOADS["train720"])
    assert cb["fine_fwd"] == fwd
    assert 4.5e9 < fwd < 4.55e9
    # each backward kernel reads or writes six per-token tensors once (dK/dV:
    # Q, K, V, dO in, dK, dV out; dQ: Q, K, V, dO, O_f in, dQ out), plus the
    # per-row statistics, the lists and the coarse rows (under 2% more)
    for n in ("bwd_dkdv", "bwd_dq"):
        assert 20 * 6 * tok < cb[n] < 1.02 * 20 * 6 * tok


def test_topk_bytes_count_every_pass():
    # five passes over the 3,432^2 fp32 scores of each of 20 heads is most of
    # what the per-sequence TopK moves
    w = WORKLOADS["train720"]
    five = 20 * 5 * 3432 * 3432 * 4
    assert five < op_bytes(w)["topk"] < 1.05 * five


def test_forward_only_topk_bytes_leave_out_the_csc():
    # forward-only workloads call TopK with no CSC: no selection bitmap and
    # no column lists, only the five score passes and the CSR
    w = WORKLOADS["infer720"]
    five = 20 * 5 * 3432 * 3432 * 4
    csr = 20 * (219648 * 4 + 3433 * 4)
    assert op_bytes(w)["topk"] == five + csr
    assert op_bytes(w)["topk"] < op_bytes(WORKLOADS["train720"])["topk"]


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_every_workload_is_described_with_its_grid(name):
    w = WORKLOADS[name]
    text = bench.describe(w)
    t, y, x = w.grid
    assert f"{t}x{y}x{x}" in text
    assert f"d={w.head_dim}" in text


def test_dense_context_figure_only_on_plain_video_workloads():
    # the dense-attention context runs over all L tokens of Q, K, V; text rows
    # and pad slots are not tokens of that attention, so those workloads skip
    for name in ("train720text", "train720pad"):
        out = bench.dense_attention(WORKLOADS[name], None, None, None, None, 1.0, 1.0)
        assert set(out) == {"skipped"}
