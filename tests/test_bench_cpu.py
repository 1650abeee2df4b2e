"""Host-side pieces of bench.py, on the CPU: the algorithmic bytes it divides
by, the bf16 distance it reports for FAST mode, and its refusal of more than
one GPU."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_of_the_qwen_image_step():
    rows, d, b = 2 * 4608, 3072, 2
    tensor = rows * d * 2                                  # one [9216, 3072] bf16 tensor
    assert bench.BYTES["ln_modulate"] == 2 * tensor + 2 * b * d * 2 == 113_270_784
    assert bench.BYTES["rmsnorm_scale"] == 2 * tensor + d * 2 + b * d * 2 == 113_264_640
    assert bench.BYTES["rmsnorm_tanh_residual"] == 3 * tensor + d * 2 + b * d * 2
    assert bench.BYTES["residual_gate_add"] == 3 * tensor + b * d * 2 == 169_881_600
    # Q, K, V read from the merged projection and written to the joint buffers,
    # four 128-element weights, fp32 cos/sin [4608, 64]
    assert bench.BYTES["qk_norm_rope"] == 6 * tensor + 4 * 128 * 2 + 2 * 4608 * 64 * 4 \
        == 342_098_944


def test_algorithmic_bytes_of_the_wan_block():
    tensor = 75600 * 5120 * 2
    assert bench.WAN_BYTES["ln_modulate_per_token"] == 4 * tensor == 3_096_576_000
    assert bench.WAN_BYTES["rmsnorm_tanh_residual_per_token"] == 4 * tensor + 5120 * 2
    assert bench.WAN_BYTES["rmsnorm_tanh_residual_per_batch"] == 3 * tensor + 2 * 5120 * 2 \
        == 2_322_452_480


def test_bf16_line_is_monotone_and_merges_zeros():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bench._bf16_values(codes)
    ok = ~bench._bf16_nan(codes)
    line = bench._bf16_line(codes[ok])
    order = np.argsort(vals[ok], kind="stable")
    assert np.all(np.diff(line[order]) >= 0)
    assert bench._bf16_line(np.array([0x0000, 0x8000], dtype=np.uint16)).tolist() == [0, 0]
    # neighbours one step apart, across zero too
    pair = np.array([0x0001, 0x8001, 0x3F80, 0x3F81], dtype=np.uint16)
    assert np.abs(np.diff(bench._bf16_line(pair)))[[0, 2]].tolist() == [2, 1]
    assert bench._bf16_nan(np.array([0x7FC0, 0xFF81, 0x7F80], dtype=np.uint16)).tolist() == \
        [True, True, False]


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_fast_targets_mark_the_literal_two_step_bound():
    import bench
    res = {"ln": dict(max_ulp=4, frac_within_1ulp=0.999999),
           "rms": dict(max_ulp=0, frac_within_1ulp=1.0),
           "chain": dict(psnr_db=189.9)}
    t = bench.fast_targets(res, ["ln", "rms"])
    assert t["max_2_steps_literal"] == dict(met=False, over=["ln"])
    assert t["within_1_step_at_least_99.9pct"]["met"] is True
    assert t["chain_psnr_at_least_40_db"]["met"] is True
    res["ln"] = dict(max_ulp=2, frac_within_1ulp=0.998)
    res["chain"] = dict(psnr_db=39.0)
    t = bench.fast_targets(res, ["ln", "rms"])
    assert t["max_2_steps_literal"]["met"] is True
    assert t["within_1_step_at_least_99.9pct"]["met"] is False
    assert t["chain_psnr_at_least_40_db"]["met"] is False


def test_fast_targets_serialize_with_numpy_inputs():
    import json
    import bench
    res = {"ln": dict(max_ulp=np.int64(4), frac_within_1ulp=np.float64(0.999999)),
           "chain": dict(psnr_db=np.float64(189.86))}
    t = bench.fast_targets(res, ["ln"])
    back = json.loads(json.dumps(t))
    assert back["max_2_steps_literal"] == {"met": False, "over": ["ln"]}
    assert back["chain_psnr_at_least_40_db"]["met"] is True


def test_result_line_serializes_numpy_scalars():
    import json
    import bench
    line = json.dumps({"a": np.bool_(True), "b": np.int64(3), "c": np.float32(0.5)},
                      default=bench._json_scalar)
    assert json.loads(line) == {"a": True, "b": 3, "c": 0.5}
