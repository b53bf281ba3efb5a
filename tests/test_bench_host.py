"""Host-side checks of bench.py (no GPU): the one-GPU contract and the algorithmic byte counts
that the roofline divides by the measured time.

The byte counts follow the per-unit figures of the path: a dense step moves one K and one V
row per (sequence, KV head, position) plus one fp32 logit per (sequence, query head,
position), plus q, out and lse once per head; a fast step moves one K and one V row and one
int32 index per attended (sequence, KV head, position), plus q, out and lse.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_kv_attention_dense_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120,
                       env={**os.environ, "WORLD_SIZE": "1"})
    assert r.returncode == 2
    assert "single MI355X" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name,expect", [
    # 4 sequences x 8 KV heads x 131072 positions x (2 rows x 256 B + 4 heads x 4 B)
    # + q (bf16) and out (fp32) of 128 heads x 128 dims + lse of 128 heads
    ("sink_128k_b4", 4 * 8 * 131072 * (512 + 16) + 128 * 128 * (2 + 4) + 128 * 4),
    # 1 sequence x 8 KV heads x 524288 positions x (512 B + 8 heads x 4 B), 64 query heads
    ("gqa8_512k", 8 * 524288 * (512 + 32) + 64 * 128 * (2 + 4) + 64 * 4),
    # its share on one of 8 GPUs split by KV head: 1 KV head, 8 query heads
    ("gqa8_512k_tp8", 1 * 524288 * (512 + 32) + 8 * 128 * (2 + 4) + 8 * 4),
    # 2048 positions, fp32 rows of 64 dims (2 x 256 B), 4 heads x 4 B of logits
    ("tiny_2k_f32", 1 * 2048 * (512 + 16) + 4 * 64 * (4 + 4) + 4 * 4),
])
def test_dense_bytes_per_launch(name, expect):
    wl = synth.WORKLOADS[name]
    assert bench.dense_bytes(wl, synth.slow_step_lengths(wl)) == expect


def test_fast_bytes_count_index_rows_recent_rows_and_skip_masked_groups():
    wl = synth.WORKLOADS["gqa8_512k"]
    lens = [wl.n0 + 1]
    n_idx = [[wl.n_sink + wl.k_sel] * wl.Hkv]
    heads = wl.B * wl.Hq * (wl.d * (wl.elem_bytes + 4) + 4)
    per_group = (wl.n_sink + wl.k_sel + wl.n_recent) * 2 * wl.d * wl.elem_bytes + \
        (wl.n_sink + wl.k_sel) * 4
    assert bench.fast_bytes(wl, lens, n_idx, None) == wl.Hkv * per_group + heads
    # every head of KV group 3 masked: the group reads no rows; a partly masked group still does
    mask = [[0] * wl.Hq]
    for i in range(3 * wl.G, 4 * wl.G):
        mask[0][i] = 1
    mask[0][0] = 1
    assert bench.fast_bytes(wl, lens, n_idx, mask) == (wl.Hkv - 1) * per_group + heads


def test_fast_bytes_clip_the_recent_window_to_the_length():
    wl = synth.WORKLOADS["tiny_2k_f32"]
    got = bench.fast_bytes(wl, [10], [[3]], None)
    assert got == (3 + 10) * 2 * wl.d * 4 + 3 * 4 + wl.Hq * (wl.d * 8 + 4)
