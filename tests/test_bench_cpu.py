"""Host-side checks of bench.py: its byte models against sums worked out by
hand for the OPT-6.7B-shaped layer, and its refusal to run on more than one GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_bytes_per_head_opt67b():
    # k = 256 slots, d = 128, bf16: K and V rows 2*256*128*2 = 131072; score
    # read+write and pos read 12*256 = 3072; q, k_new, v_new read and the new
    # K, V rows written 5*128*2 = 1280; fp32 output 4*128 = 512; the new
    # slot's position and the evicted position 8.
    assert bench.decode_bytes_per_head(256, 128, 2) == 131072 + 3072 + 1280 + 512 + 8


def test_fullcache_bytes_and_ratio_large_batch():
    # 1536 positions, d = 128, fp16: K and V 2*1536*128*2 = 786432, query 256,
    # fp32 output 512.
    full = bench.fullcache_bytes_per_head(1536, 128, 2)
    assert full == 786432 + 256 + 512
    ratio = full / bench.decode_bytes_per_head(256, 128, 2)
    assert 5.78 < ratio < 5.80


def test_quant_bytes_per_head_u4():
    # 4-bit codes: rows of 64 bytes; K and V codes 2*256*64 = 32768; value
    # grids 8*256 = 2048; score/pos 12*256 = 3072; q, k_new, v_new 3*128*2 =
    # 768; key grids 8*128 = 1024; output 512; new codes 2*64 = 128; 16.
    assert bench.decode_bytes_per_head_quant(256, 128, 2, 4) == 32768 + 2048 + 3072 + 768 + 1024 + 512 + 128 + 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
