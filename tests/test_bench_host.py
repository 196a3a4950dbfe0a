"""Host-side checks of bench.py (CPU only): the algorithmic byte and flop
counts behind the roofline figures, the traffic record's staleness guard and
the one-GPU exit.

The expected counts are written out part by part from the layouts the kernels
read and write (fp32 S [2F][d] and Z [2F] per (request, head), bf16 q/k/v
[L][d], fp32 out [L][d], bf16 W [d][F] per head), not through bench.py's own
formulas.  The transfer's matrix-core count is compared with the per-sweep
counts that rocprofv3's SQ_INSTS_VALU_MFMA_MOPS_BF16 reported for the three
kernels (944, 1,184 and 1,200 instructions per 32-token tile and head).
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_step_bytes_serving_workload():
    B, H, L, d, F = 128, 16, 32, 128, 128
    state = 2 * F * d * 4 + 2 * F * 4          # S and Z of one (request, head)
    blk = 3 * L * d * 2 + L * d * 4            # q, k, v in, out
    w = H * d * F * 2                          # W once per head
    assert B * H * (state + blk) + w == 354_942_976
    assert bench.step_bytes(B, H, L, d, F) == 354_942_976


def test_commit_bytes_one_block():
    B, H, T, d, F = 128, 16, 32, 128, 128
    rmw = 2 * (2 * F * d * 4 + 2 * F * 4)      # S and Z read and written
    kv = 2 * T * d * 2
    assert B * H * (rmw + kv) + H * d * F * 2 == 575_143_936
    assert bench.commit_bytes(B, H, T, d, F) == 575_143_936


def test_transfer_counts():
    assert bench.transfer_flops(128, 128, 32) == 475_136
    assert bench.transfer_mfma_bf16(128) == 944 + 1_184 + 1_200


def test_stale_traffic_record_is_refused():
    assert bench.load_traffic("0000000000000000") is None


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
