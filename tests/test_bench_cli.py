"""The bench's command-line contract and byte accounting, on the CPU."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=ROOT)
    assert run.returncode == 2
    assert "one GPU" in run.stderr and run.stdout == ""


def test_step_bytes_of_the_4096_token_batch():
    """Bytes one step must move, summed by hand for 4096 tokens x 14336-byte
    rows, top-8 of 256 experts in 8 ranks, int64 routing, every token live,
    31130 expert-major rows and 20919 rank rows:
      routing read         4096 * 8 * 8               =     262144
      token rows read      4096 * 14336               =   58720256
      rows written         (20919 + 31130) * 14336    =  746174464
      int32 layout outputs 4 * (2*256 + 2*8 + 2 + 2*32768 + 31130 + 20919)
                                                      =     472460
    """
    total, layout, rows = bench.algorithmic_bytes(4096, 8, 256, 8, 8, 14336, 0, 4096, 31130, 20919)
    assert (total, layout, rows) == (805629324, 262144 + 472460, 58720256 + 746174464)
    # The scatter launch alone: token rows read, rows written, both slot maps
    # read (2 * 4 bytes per pair) and the expert counts and psums read.
    assert bench.scatter_launch_bytes(4096, 8, 256, 14336, 0, 4096, 31130, 20919) == (
        58720256 + 746174464 + 4096 * 8 * 8 + 4 * (2 * 256 + 1))


def test_scale_factors_count_with_their_rows():
    # 56 fp32 scale factors per row add 224 bytes to every row read or written.
    base = bench.algorithmic_bytes(100, 4, 16, 4, 8, 7168, 0, 90, 300, 200)[0]
    with_sf = bench.algorithmic_bytes(100, 4, 16, 4, 8, 7168, 56, 90, 300, 200)[0]
    assert with_sf - base == 224 * (90 + 300 + 200)
