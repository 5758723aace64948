"""The benchmark's host-side pieces, without a GPU: the one-GPU contract, the
FLOP count behind every TFLOP/s figure, and that the committed counter
profiles belong to the kernel sources as they stand."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("causal", [True, False])
def test_visible_pairs_matches_a_brute_force_count(causal):
    # ragged lengths with qo > kv, qo < kv and empty sequences
    qo_len = [5, 0, 7, 33, 1, 12]
    kv_len = [5, 4, 3, 40, 0, 30]
    qo = np.cumsum([0] + qo_len).tolist()
    kv = np.cumsum([0] + kv_len).tolist()
    brute = 0
    for ql, kl in zip(qo_len, kv_len):
        for i in range(ql):
            for j in range(kl):
                if not causal or j < kl - ql + i + 1:
                    brute += 1
    assert bench.visible_pairs(qo, kv, causal) == brute


@pytest.mark.parametrize("profile,source", [
    ("prefill_bf16_deepseek_v3_batch.txt", "mla_ragged_chunked_amd/csrc/prefill_bf16.hip"),
    ("prefill_absorbed_deepseek_v3_batch.txt", "mla_ragged_chunked_amd/csrc/prefill_absorbed.hip"),
    ("merge_state_16384x128_bf16.txt", "mla_ragged_chunked_amd/csrc/merge.hip"),
    ("decompress_kv_8x4096_128heads.txt", "mla_ragged_chunked_amd/csrc/decompress.hip"),
    ("prefill_fp32_deepseek_v3_lengths_16heads.txt", "mla_ragged_chunked_amd/csrc/prefill_fp32.hip"),
])
def test_committed_profiles_match_the_kernel_sources(profile, source):
    # the bench reports a kernel's measured traffic only while the profile's
    # source hash matches the code; a kernel change needs a new profile
    traffic = bench.profile_traffic(profile, source)
    assert traffic is not None and traffic > 0


def test_every_profile_names_the_current_source():
    # each committed summary records the hash of the kernel source it was
    # taken with; a kernel change needs a new profile
    import glob
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    files = sorted(glob.glob(os.path.join(root, "profiles", "*.txt")))
    assert files
    for f in files:
        fields = dict(line.split(": ", 1) for line in open(f).read().splitlines()[:6]
                      if ": " in line)
        assert "source" in fields and "source_code_sha256_16" in fields, f
        src = os.path.join(root, fields["source"].strip())
        assert bench.code_hash(src) == fields["source_code_sha256_16"].strip(), f
