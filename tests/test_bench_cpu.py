"""Host logic of bench.py: the single-GPU refusal, the algorithmic byte and
FLOP models behind the roofline fractions, and the committed counter records
the bench line reports (no GPU needed)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_prefill_byte_model():
    # Per token-head: q, k, v, o in bf16 (256 B each at d = 128), g in fp32
    # (512 B), beta (4 B): 1540 B; plus one 64 KB fp32 state read and written
    # per (sequence, head).
    assert bench.prefill_alg_bytes(1, 1, 128, 128, 0) == 1540
    assert bench.prefill_alg_bytes(131072, 32, 128, 128, 1) == \
        131072 * 32 * 1540 + 2 * 32 * 128 * 128 * 4 == 6463422464
    # zero initial states are not read
    assert bench.prefill_alg_bytes(10, 2, 128, 128, 3, has_s0=False) == \
        10 * 2 * 1540 + 3 * 2 * 128 * 128 * 4
    # one log-decay per (token, head) instead of d_k of them
    assert bench.scalar_gate_alg_bytes(1, 1, 128, 128, 0) == 1540 - 512 + 4


def test_fp32_prefill_byte_model():
    # q, k, v, o in fp32 (512 B each at d = 128), g in fp32 (512 B), beta (4 B)
    assert bench.prefill_f32_alg_bytes(1, 1, 128, 128, 0) == 5 * 512 + 4 == 2564
    assert bench.prefill_f32_alg_bytes(4096, 8, 128, 128, 2) == \
        4096 * 8 * 2564 + 2 * 2 * 8 * 128 * 128 * 4


def test_prefill_flop_model():
    # 2 (5 C d + 3 d^2) = 180,224 FLOP per token-head at C = 64, d = 128
    assert bench.prefill_alg_flops(1, 1, 64, 128) == 180224
    assert bench.prefill_alg_flops(131072, 32, 64, 128) == 131072 * 32 * 180224


def test_decode_byte_model():
    # per (session, head): 2 x 64 KB of fp32 state, q k v o in bf16, g fp32, beta
    per_pair = 2 * 128 * 128 * 4 + 4 * 256 + 512 + 4
    assert per_pair == 132612
    assert bench.decode_alg_bytes(128, 32, 128, 128) == 128 * 32 * per_pair == 543178752


def test_counter_records_are_well_formed():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        recs = json.load(f)
    cal = recs.pop("calibration")
    assert cal["fetch_kib_per_gib_copy"] > 0 and cal["write_kib_per_gib_copy"] > 0
    assert "kda_chunk_fwd:T131072_H32" in recs and "kda_decode_step:N128_H32" in recs
    for key, rec in recs.items():
        for name in rec["sources"]:
            assert os.path.exists(os.path.join(ROOT, "gated_delta_rule_80_amd", "csrc", name)), name
        assert len(rec["sources_sha256"]) == 64
        total = sum(v["read"] + v["write"] for v in rec["per_kernel"].values())
        assert total == rec["hbm_bytes_per_launch"], key
        for v in rec.get("mfma_counters", {}).values():
            assert 0.0 <= v["mfma_busy_frac"] <= 1.0


def test_unknown_counter_record_reports_nothing():
    assert bench.measured_traffic("no such workload") is None
    assert bench.measured_mfma("no such workload") is None
