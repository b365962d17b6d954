"""The benchmark's byte accounting, pinned to closed forms worked out by hand
for the workload shapes, and its one-GPU contract.  No GPU needed.

Per launch, a codec kernel moves the fp16 tokens it reads or writes, plus
the packed code words and the fp16 scale/zero sidecars, padding slots
included: keys have ceil(n/G) groups of G*b/32 word rows of D words and D
sidecars each; values have ceil(D/G) groups per token, G*b/32 words and one
sidecar pair each."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_llama_shape_round_trip_bytes():
    # 8192 slices x 3968 tokens x 128 channels, 2/2-bit, G = 32
    fp16 = 8192 * 3968 * 128 * 2                      # 8,321,499,136
    k_words = 8192 * 124 * 2 * 128 * 4                # 124 groups x 2 word rows
    k_stats = 2 * 8192 * 124 * 128 * 2
    v_words = 8192 * 3968 * 8 * 4                     # 4 groups x 2 words per token
    v_stats = 2 * 8192 * 3968 * 4 * 2
    assert fp16 + k_words + k_stats == 9_881_780_224
    assert fp16 + v_words + v_stats == 9_881_780_224
    got = [bench.algorithmic_bytes(kind, d, 8192, 3968, 128, 32, 2)
           for kind in "kv" for d in ("encode", "decode")]
    assert got == [9_881_780_224] * 4
    assert sum(got) == 39_527_120_896                 # the round trip of the shape table


def test_mistral_shape_round_trip_bytes():
    # 4096 slices x 16256 tokens x 128 channels, keys 2-bit, values 4-bit
    k = bench.algorithmic_bytes("k", "encode", 4096, 16256, 128, 32, 2)
    v = bench.algorithmic_bytes("v", "encode", 4096, 16256, 128, 32, 4)
    assert k == 17_045_651_456 + 2_130_706_432 + 1_065_353_216
    assert v == 17_045_651_456 + 4_261_412_864 + 1_065_353_216
    assert 2 * (k + v) == 85_228_257_280


def test_single_layer_round_trip_bytes():
    # 8 slices x 384 tokens x 128 channels, 4/4-bit: 12 key groups, 4 value groups
    k = bench.algorithmic_bytes("k", "encode", 8, 384, 128, 32, 4)
    v = bench.algorithmic_bytes("v", "encode", 8, 384, 128, 32, 4)
    assert k == v == 786_432 + 196_608 + 49_152
    assert 2 * (k + v) == 4_128_768


def test_partial_groups_count_their_padding():
    # 1000 tokens at G = 64: 16 key groups (the last holds 40 tokens) and
    # D = 96 at G = 64: 2 value groups per token (the last holds 32 channels)
    k = bench.algorithmic_bytes("k", "encode", 1, 1000, 96, 64, 4)
    v = bench.algorithmic_bytes("v", "encode", 1, 1000, 96, 64, 4)
    assert k == 1000 * 96 * 2 + 16 * 8 * 96 * 4 + 2 * 16 * 96 * 2
    assert v == 1000 * 96 * 2 + 1000 * 2 * 8 * 4 + 2 * 1000 * 2 * 2


def test_attention_bytes_llama_shape():
    # what attention must move: the packed prefix, the fp16 residual, q and
    # the output; the partial sums of a split plan (5 splits, 1 head, 128 + 2
    # floats each, written by the attention kernel and read back by the
    # merge kernel) are counted on their own
    payload = 1_040_187_392 + 520_093_696 + 1_040_187_392 + 520_093_696
    resid = 2 * 8192 * 128 * 128 * 2
    q = out = 8192 * 128 * 2
    partials = 8192 * 5 * 130 * 4
    got = bench.attention_bytes(8192, 3968, 128, 128, 32, 2, 2, 1, 5)
    assert got == {"method": payload + resid + q + out, "partials": 2 * partials}
    assert got["method"] == 3_661_627_392
    assert got["method"] + got["partials"] == 3_704_225_792
    # one split: no partial sums
    one = bench.attention_bytes(8192, 3968, 128, 128, 32, 2, 2, 1, 1)
    assert one == {"method": payload + resid + q + out, "partials": 0}


def test_attention_bytes_mistral_shape():
    # 4096 slices x 16256 quantized tokens, keys 2-bit and values 4-bit,
    # 4 query heads per KV slice, 128 fp16 residual tokens
    payload = (4096 * 508 * 2 * 128 * 4 + 2 * 4096 * 508 * 128 * 2
               + 4096 * 16256 * 16 * 4 + 2 * 4096 * 16256 * 4 * 2)
    got = bench.attention_bytes(4096, 16256, 128, 128, 32, 2, 4, 4, 9)
    assert got["method"] == payload + 2 * 4096 * 128 * 128 * 2 + 2 * 4096 * 4 * 128 * 2
    assert got["partials"] == 2 * 4096 * 9 * 4 * 130 * 4


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stdout
