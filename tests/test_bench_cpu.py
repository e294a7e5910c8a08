"""Host-side checks of bench.py (no GPU): the algorithmic byte and flop counts its roofline figures divide by,
recomputed here from their definitions for the benchmarked workloads, and the one-GPU contract."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_state_pass_bytes_lm_layer():
    # q, k, v read and o written once per token-head in bf16 (2 bytes), plus the fp32 final state per head
    B, H, L, d = 8, 16, 4096, 128
    expect = B * H * L * 4 * d * 2 + B * H * d * d * 4
    assert bench.chain_algorithmic(B, H, L, d, d) == expect == 545_259_520


def test_forward_bytes_and_flops_lm_layer():
    B, H, L, d, C = 8, 16, 4096, 128, 64
    nbytes, flops = bench.fwd_algorithmic(B, H, L, d, d, C)
    # the state pass's bytes plus beta (fp32) once per token-head
    assert nbytes == 545_259_520 + B * H * L * 4 == 547_356_672
    # per chunk: K S, Q S and K^T Delta (2 C d^2 each), the lower blocks of K K^T and Q K^T (C^2 d each),
    # T diag(alpha) R and lower(Q K^T) Delta (C^2 d each), the substitution C^3 / 3
    per_chunk = 3 * 2 * C * d * d + 2 * C * C * d + 2 * C * C * d + C ** 3 / 3
    assert abs(flops - per_chunk * B * H * L / C) < 1.0
    # arithmetic intensity below the bf16 ridge (2.5 PFLOP/s over 8 TB/s): the forward is HBM-bound
    assert flops / nbytes < bench.BF16_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)


def test_decode_bytes():
    # 256 sequences x 32 heads: the fp32 state read and written once, q, k, v, o in bf16 and beta
    NH, d = 256 * 32, 128
    assert bench.decode_algorithmic(NH, d, d) == NH * (2 * 4 * d * d + 4 * d * 2 + 4) == 1_082_163_200


def test_ut_bytes():
    B, H, L, d = 8, 16, 4096, 128
    assert bench.ut_algorithmic(B, H, L, d) == B * H * L * (d * 2 + 4) == 136_314_880


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "one GPU" in r.stdout
