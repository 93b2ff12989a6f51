"""Host checks of the algorithmic byte and FLOP counts that bench.py divides by
measured times (the roofline figures rest on them), on a tiny case counted by
hand."""
import numpy as np
import pytest
import torch

import msa_synth


def test_algorithmic_counts_by_hand():
    import bench
    # two decode rows at positions 299 and 127 (3 and 1 blocks), G 2, d_idx 64, n_idx 4
    case = msa_synth.build_case("t", seed=5, ctx_lens=[300, 128], G=2, Hg=4, d_idx=64, k=2)
    sel = torch.tensor([[[0, 2, -1], [1, 2, -1]],     # row 0: block 2 is its own (44 tokens)
                        [[0, -1, -1], [0, -1, -1]]],  # row 1: only its own block (128 tokens)
                       dtype=torch.int32)
    a = bench.algorithmic(case, sel)
    G, d_idx, n_idx, D, Hg = 2, 64, 4, 128, 4
    # key index: every visible token of every row, per group
    assert a["kidx"] == (300 + 128) * G * d_idx * 2
    assert a["qidx"] == 2 * G * n_idx * d_idx * 2
    assert a["score_bytes"] == a["kidx"] + a["qidx"] + 2 * G * case.nb * 4
    assert a["index_flops"] == (300 + 128) * G * n_idx * d_idx * 2
    # attention: visible tokens of the selected blocks, per (row, group)
    tokens = (128 + 44) + (128 + 44) + 128 + 128
    assert a["attn_flops"] == 4.0 * D * tokens * Hg
    # full blocks of K and V for every selected block (6 of them)
    assert a["kv_bytes"] == 6 * 128 * D * 2 * 2
    assert a["qo_bytes"] == 2 * G * Hg * D * 2 * 2
    assert a["part_bytes"] == 2 * G * Hg * 3 * (D * 2 + 4)


def test_multi_gpu_request_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True,
                       text=True, cwd=bench_root())
    assert r.returncode != 0 and "one GPU" in r.stderr


def bench_root():
    import os
    return os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_profile_traffic_binds_to_workload_and_source(tmp_path):
    """A committed counter summary is used only for the workload it was taken on
    and only while the kernel sources hash to the recorded value."""
    import hashlib
    import json
    import bench
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel source\n")
    h = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    prof = tmp_path / "traffic.json"
    prof.write_text(json.dumps({"workload": "decode-64k-b8", "kernel_source_sha256_16": h,
                                "hbm_bytes_per_launch": 1234}))
    assert bench.traffic_from_profile("decode-64k-b8", str(prof), [str(src)]) == 1234
    assert bench.traffic_from_profile("decode-1m-b4", str(prof), [str(src)]) is None
    src.write_text("// kernel source, changed\n")
    assert bench.traffic_from_profile("decode-64k-b8", str(prof), [str(src)]) is None
    assert bench.traffic_from_profile("decode-64k-b8", str(tmp_path / "missing.json"),
                                      [str(src)]) is None

