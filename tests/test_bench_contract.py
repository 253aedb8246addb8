"""bench.py on the CPU: the one-GPU refusal and the algorithmic byte and flop
models behind every roofline fraction it reports."""
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_byte_model_bf16_head():
    # decode head, M = 64, fp32 logits, no bias: weight read once, the hidden
    # rows read once, the logits written once
    M, H, V = 64, 4096, 128256
    weight = 128256 * 4096 * 2
    hidden = 64 * 4096 * 2
    logits = 64 * 128256 * 4
    assert bench.bytes_bf16(M, H, V, 4, False) == weight + hidden + logits == 1_084_030_976
    # a bias adds one fp32 read per column; bf16 logits halve the write
    assert bench.bytes_bf16(M, H, V, 2, True) == weight + hidden + 128256 * 4 + logits // 2


def test_byte_model_nvfp4_head():
    # H = 2048, V = 151936, M = 1: half a byte per code, one E4M3 scale byte
    # per 16 codes, bf16 hidden row and bf16 logits
    codes = 151936 * 2048 // 2
    scales = 151936 * 2048 // 16
    assert codes == 155_582_464 and scales == 19_447_808
    assert bench.bytes_nvfp4(1, 2048, 151936) == codes + scales + 2048 * 2 + 151936 * 2 == 175_338_240


def test_flop_model():
    # one multiply and one add per (row, column, K element)
    assert bench.flops(2048, 4096, 151936) == 2 * 2048 * 4096 * 151936
    assert bench.flops(1, 1, 1) == 2
