"""Host-side logic of bench.py (no GPU): which LM-head kernel a shape selects, the algorithmic
byte and flop counts behind the roofline fields, and the command-line contract."""
import os
import subprocess
import sys

import pytest

import bench
from workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("M,H,Vt,calls,kernel", [
    (6, 3072, 32768, False, "lmhead_gemv"),          # configs 2 and 3
    (8, 4096, 65536, False, "lmhead_mfma_rows"),     # 8 rows of 4096 exceed the GEMV's registers
    (9, 4096, 65536, False, "lmhead_mfma_rows"),     # config 5's shape at one sequence
    (192, 4096, 65536, False, "lmhead_mfma_rows"),   # the largest all-rows block on 256 columns
    (193, 4096, 65536, False, "lmhead_mfma_dma8"),
    (256, 3072, 32768, False, "lmhead_mfma_rows"),   # 128-column blocks: one block up to 256 rows
    (384, 3072, 32768, False, "lmhead_mfma_rows"),   # and two up to 384
    (385, 3072, 32768, False, "lmhead_mfma_dma8"),   # 256 square tiles beat 128 tall ones
    (512, 3072, 32768, False, "lmhead_mfma_dma8"),   # config 4
    (288, 4096, 65536, False, "lmhead_mfma_tall"),   # 256 tall tiles against 512 square ones
    (2304, 4096, 65536, False, "lmhead_mfma_tall"),  # config 5, fused call
    (2304, 4096, 65536, True, "lmhead_mfma_dma8"),   # config 5, separate calls
    (100, 520, 32768, False, "lmhead_mfma"),         # H % 32 != 0 up to 128 rows
    (300, 520, 32768, False, "lmhead_mfma_big"),
])
def test_head_kernel_names(M, H, Vt, calls, kernel):
    assert bench.head_kernel(M, H, calls, Vt) == kernel


def test_gemv_register_limit():
    # the GEMV holds M * ceil(H / 512) <= 48 slices of 512 columns and at most 8 of them per row
    assert bench.gemv_head(6, 4096) and not bench.gemv_head(7, 4096)
    assert bench.gemv_head(8, 3072) and not bench.gemv_head(1, 4608)


def test_algorithmic_counts_config5():
    cfg = CONFIGS[5]
    M = cfg.B * cfg.R
    assert M == 2304
    assert bench.lmhead_flops(cfg) == 2.0 * 2304 * 4096 * 65536
    # kept head rows + hidden rows + fp32 logits + keep ids
    assert bench.lmhead_bytes(cfg) == 65536 * 4096 * 2 + 2304 * 4096 * 2 + 2304 * 65536 * 4 + 65536 * 4
    assert not bench.small_batch_block(cfg)


def test_small_batch_block_is_the_gemv_path():
    assert bench.small_batch_block(CONFIGS[3]) and bench.small_batch_block(CONFIGS[2])
    assert not bench.small_batch_block(CONFIGS[3], greedy=True)
    assert not bench.small_batch_block(CONFIGS[5].scaled(B=1))  # 9 rows: an MFMA head


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_sequences_applies_to_block_configs_only():
    r = _run("--config", "1", "--sequences", "4")
    assert r.returncode != 0 and "--sequences" in r.stderr
