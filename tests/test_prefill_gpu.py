"""GPU parity of causal prefill against the fp64 oracle.

The output is bf16, so the bar is |gpu - oracle| <= 2e-3 + half a bf16 ulp of the oracle
value (the rounding of the output alone can reach half an ulp).  Small prompts are
checked on every row; the full 8192-token workload on its first and last rows plus a
seeded sample.
"""
import math

import numpy as np
import pytest
import torch

import attention_gqa_decode_amd as A
import oracle
from attention_gqa_decode_amd import workloads as W
from attention_gqa_decode_amd.workloads import bits
from gpu_util import bf16_half_ulp, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_and_check(B, ISL, Hq, KH, Hsz, seed, rows=None):
    s = W.PrefillShape("t", B, ISL, Hq, KH, Hsz, seed=seed)
    q, k, v = W.prefill_inputs(s, device="cuda")
    out = A.attn_prefill_causal(q, k, v)
    torch.cuda.synchronize()
    got = out.float().cpu().double().numpy().reshape(-1, Hsz)
    ref = oracle.prefill_causal(bits(q), bits(k), bits(v), KH, 1 / math.sqrt(Hsz), rows=rows).reshape(-1, Hsz)
    sel = np.arange(got.shape[0]) if rows is None else np.asarray(rows)
    g, r = got[sel], ref[sel]
    assert np.all(np.isfinite(g))
    excess = np.abs(g - r) - (2e-3 + bf16_half_ulp(r))
    note(f"  max |err| {np.abs(g - r).max():.3e}, worst excess over bound {excess.max():.3e}")
    if excess.max() > 0:
        worst = np.argsort(excess.max(axis=1))[::-1][:8]
        for j in worst:
            flat = int(sel[j])
            bhq, i = divmod(flat, ISL)
            col = int(excess[j].argmax())
            note(f"    row {i} of (b, h) {divmod(bhq, Hq)} col {col}: gpu {g[j, col]:.6f} oracle {r[j, col]:.6f}")
    assert excess.max() <= 0, f"max |err| {np.abs(g - r).max():.3e}"


@pytest.mark.parametrize("ISL", [1, 5, 64, 128, 129, 255, 256, 257, 300, 700])
def test_small_prompts(ISL):
    note(f"prefill B=2 ISL={ISL} Hq=8 KH=2")
    run_and_check(2, ISL, 8, 2, 128, seed=ISL)


@pytest.mark.parametrize("Hsz", [64, 256])
@pytest.mark.parametrize("ISL", [1, 63, 64, 127, 129, 255, 256, 257, 700])
def test_other_head_dims(ISL, Hsz):
    note(f"prefill Hsz={Hsz} B=2 ISL={ISL} Hq=8 KH=2")
    run_and_check(2, ISL, 8, 2, Hsz, seed=640 + ISL + Hsz)


@pytest.mark.parametrize("Hsz", [64, 256])
def test_other_head_dims_long_sampled_rows(Hsz):
    s = W.PrefillShape("t", 1, 4096, 16, 4, Hsz, seed=Hsz)
    note(f"prefill Hsz={Hsz} B=1 ISL={s.ISL} Hq={s.Hq} KH={s.KH}, sampled rows")
    rng = np.random.default_rng(Hsz)
    picks = list(range(0, 32)) + list(range(s.ISL - 32, s.ISL)) + rng.choice(s.ISL, 32, replace=False).tolist()
    rows = np.array([h * s.ISL + i for h in (0, 7, 15) for i in picks])
    run_and_check(s.B, s.ISL, s.Hq, s.KH, s.Hsz, seed=s.seed, rows=rows)


@pytest.mark.parametrize("Hq,KH", [(4, 1), (8, 8), (16, 2)])
def test_group_sizes(Hq, KH):
    note(f"prefill ISL=1000 Hq={Hq} KH={KH}")
    run_and_check(1, 1000, Hq, KH, 128, seed=Hq * 10 + KH)


def test_row0_is_v0():
    s = W.PrefillShape("t", 1, 256, 8, 2, 128, seed=3)
    q, k, v = W.prefill_inputs(s, device="cuda")
    out = A.attn_prefill_causal(q, k, v)
    torch.cuda.synchronize()
    for h in range(8):
        assert torch.equal(out[0, h, 0], v[0, h // 4, 0])


def test_full_size_sampled_rows():
    s = W.prefill_workload()
    note(f"prefill full-size B={s.B} ISL={s.ISL} Hq={s.Hq} KH={s.KH}")
    rng = np.random.default_rng(5)
    heads = [0, 5, 17, 31]
    picks = list(range(0, 64)) + list(range(s.ISL - 64, s.ISL)) + rng.choice(s.ISL, 64, replace=False).tolist()
    rows = np.array([h * s.ISL + i for h in heads for i in picks])
    run_and_check(s.B, s.ISL, s.Hq, s.KH, s.Hsz, seed=s.seed, rows=rows)


def draw_prefill(i):
    """A seeded random prefill: batch, group size (odd ones too), kv heads, head dimension
    and prompt length, so that both work orders (kv-head pairs a multiple of the 8 XCDs or
    not) and ragged last blocks come up."""
    rng = np.random.default_rng(6100 + i)
    G = int(rng.choice([1, 2, 3, 4, 8]))
    KH = int(rng.choice([1, 2, 3, 4, 8]))
    B = int(rng.integers(1, 4))
    Hsz = int(rng.choice([64, 128, 256]))
    ISL = int(rng.integers(1, 600))
    return B, ISL, G * KH, KH, Hsz


@pytest.mark.parametrize("i", range(12))
def test_random_shapes(i):
    B, ISL, Hq, KH, Hsz = draw_prefill(i)
    note(f"prefill random case {i}: B={B} ISL={ISL} Hq={Hq} KH={KH} Hsz={Hsz}")
    run_and_check(B, ISL, Hq, KH, Hsz, seed=6200 + i)
