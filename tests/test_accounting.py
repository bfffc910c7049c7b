"""Byte/FLOP accounting pinned to the worked KV-cache examples of the lecture page
"추론 최적화" (section 2 and exercises 1-2), stored in tests/golden/kv_cache_bytes.txt."""
import os

import pytest

from attention_gqa_decode_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "kv_cache_bytes.txt")


def rows():
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            yield [float(x) for x in line.split()]


@pytest.mark.parametrize("row", list(rows()))
def test_kv_bytes_match_worked_examples(row):
    layers, kvh, hd, b, per_tok, tokens, total, tol = row
    got = acc.kv_cache_bytes_per_token(int(layers), int(kvh), int(hd), int(b))
    assert got == int(per_tok)
    assert abs(got * tokens - total) <= tol * total


def test_gqa8_is_a_quarter_of_mha():
    assert acc.kv_cache_bytes_per_token(32, 8, 128, 2) * 4 == acc.kv_cache_bytes_per_token(32, 32, 128, 2)


def test_decode_bytes_llama3_shape():
    # 16 requests x 8 KV heads x 8192 tokens x 128 x 2 (K,V) x 2 bytes = 512 MiB of KV
    b = acc.decode_bytes([8192] * 16, 16, 32, 8, 128)
    assert b == 536870912 + 16 * 32 * 128 * 2 + 16 * 32 * 128 * 4


def test_prefill_flops_small_case_by_enumeration():
    B, ISL, Hq, Hsz = 1, 5, 2, 4
    pairs = sum(i + 1 for i in range(ISL))
    assert acc.prefill_causal_flops(B, ISL, Hq, Hsz) == 4 * Hsz * Hq * pairs
