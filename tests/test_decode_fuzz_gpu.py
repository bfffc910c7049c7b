"""GPU parity of decode over seeded random combinations of every option at once.

Each case draws a head dimension, group size, kv heads, batch, ragged lengths (zeros
included when one token is decoded), cache capacity, bf16 or FP8 E4M3 caches with
power-of-two scales, contiguous or paged caches (block sizes 16..64), one or several
drafted tokens, host or device lengths, the schedule (automatic, stream-K with forced
LeanTile sizes and workgroup counts, or the fixed split), and an optional score
multiplier.  The output is compared with the fp64 oracle of the same arithmetic: decode,
decode over E4M3 codes, or multi-token decode ("LeanAttention" digest, section on the
piecewise exact softmax; lecture page "추론 최적화", §5, for the drafted tokens).

With power-of-two scales every scaled E4M3 value is exact in bf16, so the FP8 multi-token
reference is the multi-token oracle over those exact values.
"""
import math

import numpy as np
import pytest
import torch

import attention_gqa_decode_amd as A
import oracle
from attention_gqa_decode_amd import workloads as W
from attention_gqa_decode_amd.workloads import bits, codes
from gpu_util import DECODE_TOL, note

pytestmark = pytest.mark.gpu

CASES = 40
MAX_COLUMNS, MAX_COLUMN_ELEMS = 64, 64 * 128  # the library's query-column limits


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def e4m3_table():
    return oracle.fp8_e4m3_to_f64(np.arange(256, dtype=np.uint8))


def draw(i):
    rng = np.random.default_rng(5000 + i)
    Hsz = int(rng.choice([64, 128, 256]))
    while True:
        G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        q_len = int(rng.choice([1, 1, 1, 2, 3, 5]))
        if G * q_len <= MAX_COLUMNS and G * q_len * Hsz <= MAX_COLUMN_ELEMS:
            break
    KH = int(rng.integers(1, 4))
    B = int(rng.integers(1, 7))
    sl = []
    for _ in range(B):  # a context holds at least the drafted tokens
        r = rng.random()
        if r < 0.1 and q_len == 1:
            sl.append(0)
        elif r < 0.35:
            sl.append(int(rng.integers(q_len, 65)))
        else:
            sl.append(max(q_len, int(np.exp(rng.uniform(np.log(65), np.log(3000))))))
    cfg = dict(Hsz=Hsz, G=G, KH=KH, B=B, q_len=q_len, sl=sl, S=max(max(sl), 1) + int(rng.integers(0, 40)),
               fp8=bool(rng.random() < 0.4), paged=bool(rng.random() < 0.4), bs=int(rng.choice([16, 32, 64])),
               dev=bool(rng.random() < 0.3), mult=float(rng.choice([1.0, 1.0, 8.0])),
               ks=float(rng.choice([0.5, 1.0, 2.0])), vs=float(rng.choice([0.5, 1.0, 2.0])))
    sched = rng.integers(0, 3)
    if sched == 0:
        cfg.update(schedule=A.ATTN_SCHEDULE_AUTO, tile_keys=0, num_ctas=0, num_splits=0)
    elif sched == 1:
        cfg.update(schedule=A.ATTN_SCHEDULE_STREAM_K, tile_keys=int(rng.choice([0, 1, 16, 48, 128, 1024])),
                   num_ctas=int(rng.choice([0, 1, 5, 37, 300])), num_splits=0)
    else:
        cfg.update(schedule=A.ATTN_SCHEDULE_FIXED_SPLIT, tile_keys=int(rng.choice([0, 16, 128])), num_ctas=0,
                   num_splits=int(rng.choice([0, 1, 3])))
    return cfg


def as_bf16_bits(x):
    """float64 values exact in bf16 -> their uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("i", range(CASES))
def test_random_option_combination(i, e4m3_table):
    c = draw(i)
    Hq = c["G"] * c["KH"]
    note(f"fuzz case {i}: {c}")
    shape = W.DecodeShape("fz", c["B"], Hq, c["KH"], c["Hsz"], tuple(c["sl"]), seed=7000 + i)
    if c["fp8"]:
        q1, k, v, _ = W.decode_inputs_fp8(shape, device="cuda", k_scale=c["ks"], v_scale=c["vs"], S=c["S"])
    else:
        q1, k, v, _ = W.decode_inputs(shape, device="cuda", S=c["S"])
    q = W.randn_bf16((c["B"], Hq, c["q_len"], c["Hsz"]), 7500 + i, "cuda") if c["q_len"] > 1 else q1
    scale = c["mult"] / math.sqrt(c["Hsz"])
    kw = dict(scale=scale if c["mult"] != 1.0 else 0.0, tile_keys=c["tile_keys"], num_ctas=c["num_ctas"],
              schedule=c["schedule"], num_splits=c["num_splits"])
    if c["fp8"]:
        kw.update(k_scale=c["ks"], v_scale=c["vs"])
    seqlens = torch.tensor(c["sl"], dtype=torch.int32, device="cuda") if c["dev"] else c["sl"]
    if c["paged"]:
        kp, vp, table = W.paged_layout(k, v, c["sl"], c["bs"], seed=9000 + i)
        got = A.attn_decode_paged(q, kp, vp, table, seqlens, **kw)
    elif c["q_len"] > 1:
        got = A.attn_decode_multi(q, k, v, seqlens, **kw)
    else:
        got = A.attn_decode_ex(q, k, v, seqlens, **kw)
    torch.cuda.synchronize()
    got = got.cpu().double().numpy()

    if c["q_len"] > 1:
        if c["fp8"]:
            kb = as_bf16_bits(e4m3_table[codes(k)] * c["ks"])
            vb = as_bf16_bits(e4m3_table[codes(v)] * c["vs"])
        else:
            kb, vb = bits(k), bits(v)
        ref = oracle.decode_multi(bits(q), kb, vb, c["sl"], c["KH"], scale)
    elif c["fp8"]:
        ref = oracle.decode_fp8(bits(q), codes(k), codes(v), c["sl"], Hq, c["KH"], scale, c["ks"], c["vs"])
    else:
        ref = oracle.decode(bits(q), bits(k), bits(v), c["sl"], Hq, c["KH"], scale)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    err = float(np.abs(got - ref).max())
    note(f"  max |err| {err:.3e}")
    assert err <= DECODE_TOL
