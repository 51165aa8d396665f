"""CPU checks of bench.py's contract that need no GPU: it measures one GPU
and says so when asked for more, and its byte constants follow the row
format."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                      # no JSON line for a run that did not happen


def test_bench_row_bytes():
    sys.path.insert(0, ROOT)
    import bench
    # a (token, head) row: 16 b bytes of codes plus four fp16 scales and zeros
    assert [bench.row_bytes(b) for b in (1, 2, 4)] == [32, 48, 80]
    assert bench.DECODE_BYTES_PER_TOKEN_HEAD == 2 * 48
    assert bench.QUANT_BYTES_PER_TOKEN_HEAD == 2 * 256 + 2 * 48
