"""GPU parity of the decode path (tile kernel + merge kernel) against the fp64 oracle.

Bar: max |err| <= 2e-3 on the fp32 outputs for bf16 unit-scale inputs.  Shapes cover the
small case the oracle finishes at once, several tiles with ragged tails, the full-size
Llama-3-8B-shaped, long-context MQA (and its x8-score variant) and ragged workloads, the
(G, Hsz) sweep, forced LeanTile sizes and CTA counts, and the degenerate cases (empty
context, one key, constant V, a planted huge score, GQA vs repeated-KV MHA).
"""
import math

import numpy as np
import pytest
import torch

import attention_gqa_decode_amd as A
from attention_gqa_decode_amd import workloads as W
from gpu_util import DECODE_TOL, decode_err, gpu_decode, note, oracle_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def inputs(B, Hq, KH, Hsz, seqlens, seed, S=None):
    shape = W.DecodeShape("t", B, Hq, KH, Hsz, tuple(seqlens), seed=seed)
    q, k, v, sl = W.decode_inputs(shape, device="cuda", S=S)
    return q, k, v, sl.tolist()


def test_tiny_workload():
    s = W.decode_workload("tiny")
    note(f"decode tiny {s}")
    q, k, v, sl = W.decode_inputs(s, device="cuda")
    err, _ = decode_err(q, k, v, sl.tolist())
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL


@pytest.mark.parametrize("Hsz", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_shapes_ragged(Hsz, G):
    KH = 2
    sl = [1, 100, 517, 33]
    note(f"decode shapes Hsz={Hsz} G={G} sl={sl}")
    q, k, v, sl = inputs(4, G * KH, KH, Hsz, sl, seed=10 * G + Hsz)
    err, _ = decode_err(q, k, v, sl)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL


@pytest.mark.parametrize("T", [1, 16, 48, 256, 1024])
@pytest.mark.parametrize("P", [1, 3, 7, 256, 1000])
def test_forced_splits(T, P):
    note(f"decode forced split T={T} P={P}")
    q, k, v, sl = inputs(2, 8, 2, 128, [1000, 333], seed=7)
    err, got = decode_err(q, k, v, sl, tile_keys=T, num_ctas=P)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    base = gpu_decode(q, k, v, sl)
    assert np.abs(got - base).max() <= 1e-5  # schedules differ only by fp32 rounding


def test_empty_and_single_key_contexts():
    note("decode empty/single-key contexts")
    q, k, v, sl = inputs(4, 8, 2, 128, [0, 1, 0, 5], seed=3)
    got = gpu_decode(q, k, v, sl)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    vf = v.float().cpu().numpy()
    for h in range(8):
        np.testing.assert_array_equal(got[1, h], vf[1, h // 4, 0])
    err, _ = decode_err(q, k, v, sl)
    assert err <= DECODE_TOL


def test_all_contexts_empty():
    q, k, v, _ = inputs(2, 4, 1, 64, [1, 1], seed=4)
    out = torch.full((2, 4, 64), 7.0, device="cuda")
    A.attn_decode_ex(q, k, v, [0, 0], out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_constant_values_give_the_constant():
    note("decode constant V")
    q, k, v, sl = inputs(3, 16, 4, 128, [4000, 1, 777], seed=5)
    v.fill_(-1.375)
    got = gpu_decode(q, k, v, sl, tile_keys=64, num_ctas=37)
    assert np.abs(got + 1.375).max() <= 1e-6


def test_planted_huge_score():
    # one key scores ~ +200 (exp overflows fp32 without the running max); others are < 10
    note("decode planted huge score")
    Hsz, L, hit = 128, 5000, 3210
    q, k, v, sl = inputs(1, 4, 1, Hsz, [L], seed=6)
    q.zero_()
    q[0, :, 0] = 48.0
    k[0, 0, :, 0] = k[0, 0, :, 0].clamp(-1, 1)
    k[0, 0, hit, 0] = 48.0
    got = gpu_decode(q, k, v, sl, tile_keys=256, num_ctas=13)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got[0], np.broadcast_to(v[0, 0, hit].float().cpu().numpy(), (4, Hsz)), atol=1e-6)
    err, _ = decode_err(q, k, v, sl)
    assert err <= DECODE_TOL


def test_gqa_equals_mha_with_repeated_kv():
    note("decode GQA vs repeated-KV MHA")
    q, k, v, sl = inputs(2, 16, 2, 128, [3000, 1234], seed=8)
    gqa = gpu_decode(q, k, v, sl)
    mha = gpu_decode(q, k.repeat_interleave(8, dim=1).contiguous(), v.repeat_interleave(8, dim=1).contiguous(), sl)
    assert np.abs(gqa - mha).max() <= 1e-5


def test_caller_workspace_matches_library_workspace():
    q, k, v, sl = inputs(2, 8, 2, 128, [4096, 999], seed=9)
    need = A.attn_decode_workspace_bytes(2, 8, 2, 128, 64)
    ws = torch.zeros(need // 4, dtype=torch.float32, device="cuda")
    a = gpu_decode(q, k, v, sl, num_ctas=64, workspace=ws)
    b = gpu_decode(q, k, v, sl, num_ctas=64)
    # the same plan; waves claim blocks dynamically, so only the summation order may differ
    assert np.abs(a - b).max() <= 1e-5
    assert np.abs(a - oracle_decode(q, k, v, sl, 2, 1 / math.sqrt(128))).max() <= DECODE_TOL
    counters = ws[: A.ATTN_DECODE_COUNTER_BYTES // 4].view(torch.int32)
    assert int(counters.abs().sum()) == 0, "merge counters must be left at zero"
    with pytest.raises(A.AttnError) as e:
        A.attn_decode_ex(q, k, v, sl, num_ctas=64, workspace=ws[:16])
    assert e.value.status == A.ATTN_ERR_WORKSPACE


def test_one_workspace_across_cta_counts():
    # the counter region sits at a fixed offset, so slots written with one P never alias
    # the counters of a later call with another P
    note("decode one caller workspace, P = 64, 700, 64, 3")
    q, k, v, sl = inputs(2, 8, 2, 128, [5000, 777], seed=13)
    need = A.attn_decode_workspace_bytes(2, 8, 2, 128, 700)
    ws = torch.zeros(need // 4, dtype=torch.float32, device="cuda")
    ref = oracle_decode(q, k, v, sl, 2, 1 / math.sqrt(128))
    for P in [64, 700, 64, 3]:
        got = gpu_decode(q, k, v, sl, tile_keys=16, num_ctas=P, workspace=ws)
        assert np.abs(got - ref).max() <= DECODE_TOL, P


@pytest.mark.parametrize("P", [16, 17, 300, 4096])
def test_one_head_over_many_ctas(P):
    # one head split over P CTAs: at the in-kernel merge's width (16), just past it and far
    # past it (the wide merge kernel)
    L = 16 * P + 5
    note(f"decode one head over P={P}: L={L}, T=16")
    q, k, v, sl = inputs(1, 8, 1, 128, [L], seed=14 + P)
    err, got = decode_err(q, k, v, sl, tile_keys=16, num_ctas=P)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    again = gpu_decode(q, k, v, sl, tile_keys=16, num_ctas=P)
    assert np.abs(got - again).max() <= 1e-5  # counters were reset: a second call merges the same way


def test_repeated_calls_agree():
    # waves claim blocks dynamically, so the summation order (not the result) may change
    # from call to call: the pages promise exactness, not bitwise equality across schedules
    q, k, v, sl = inputs(4, 32, 8, 128, [3000, 9000, 1, 4500], seed=15)
    outs = [gpu_decode(q, k, v, sl) for _ in range(4)]
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 1e-5


def test_simple_entry_matches_ex():
    q, k, v, sl = inputs(3, 8, 2, 128, [100, 2048, 50], seed=11)
    a = A.attn_decode(q, k, v, sl)
    torch.cuda.synchronize()
    b = gpu_decode(q, k, v, sl)
    assert np.abs(a.cpu().double().numpy() - b).max() <= 1e-5  # same plan, dynamic block order


def test_cache_capacity_larger_than_contexts():
    q, k, v, sl = inputs(2, 8, 4, 64, [700, 31], seed=12, S=1500)
    err, _ = decode_err(q, k, v, sl)
    assert err <= DECODE_TOL


# ------------------------------------------------------------------ full-size workloads

@pytest.mark.parametrize("name", ["llama3_8b", "long_mqa", "long_mqa_x8", "ragged"])
def test_full_size_workloads(name):
    s = W.decode_workload(name)
    note(f"decode full-size {name}: B={s.B} Hq={s.Hq} KH={s.KH} Hsz={s.Hsz} sum(L)={sum(s.seqlens)}")
    q, k, v, sl = W.decode_inputs(s, device="cuda")
    err, _ = decode_err(q, k, v, sl.tolist(), scale_mult=s.score_mult)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    del q, k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("Hsz", [64, 128, 256])
def test_ragged_sweep_points(G, Hsz):
    s = W.ragged_sweep_point(G, Hsz)
    note(f"decode sweep G={G} Hsz={Hsz}: KH={s.KH} sum(L)={sum(s.seqlens)}")
    q, k, v, sl = W.decode_inputs(s, device="cuda")
    rows = np.random.default_rng(G * 1000 + Hsz).choice(s.B * s.Hq, 96, replace=False)
    err, _ = decode_err(q, k, v, sl.tolist(), rows=rows)
    note(f"  max err {err:.3e} over {len(rows)} sampled rows")
    assert err <= DECODE_TOL
    del q, k, v
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ schedules

@pytest.mark.parametrize("splits", [0, 1, 2, 7, 64])
def test_fixed_split_schedule(splits):
    # FlashDecoding-style baseline: every (request, kv head) context cut into `splits`
    # chunks (0 = fill the GPU once); ragged lengths, empty and one-key contexts included
    note(f"decode fixed split S={splits}")
    q, k, v, sl = inputs(5, 16, 4, 128, [3000, 0, 1, 700, 5555], seed=20 + splits)
    err, got = decode_err(q, k, v, sl, schedule=A.ATTN_SCHEDULE_FIXED_SPLIT, num_splits=splits)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    assert np.all(got[1] == 0)
    base = gpu_decode(q, k, v, sl, schedule=A.ATTN_SCHEDULE_STREAM_K)
    assert np.abs(got - base).max() <= 1e-5


def test_auto_schedule_many_segments():
    # 256 requests x 8 kv heads: at least twice the resident workgroups, so the selector
    # runs one workgroup per (request, kv head) with no reduction
    rng = np.random.default_rng(21)
    sl = rng.integers(1, 400, 256).tolist()
    note(f"decode auto schedule, B=256 KH=8, sum(L)={sum(sl)}")
    q, k, v, sl = inputs(256, 32, 8, 64, sl, seed=21)
    rows = np.random.default_rng(22).choice(256 * 32, 200, replace=False)
    err, got = decode_err(q, k, v, sl, rows=rows)
    assert err <= DECODE_TOL
    sk = gpu_decode(q, k, v, sl, schedule=A.ATTN_SCHEDULE_STREAM_K)
    assert np.abs(got - sk).max() <= 1e-5


def test_default_ctas_many_segments():
    # 64 requests x 32 kv heads (G=1): far more segments than resident workgroups, so the
    # default stream-K launch runs several workgroups per slot.  A workspace sized with
    # num_ctas = 0 must cover that call, and the result matches the oracle and a launch of
    # one workgroup per slot.
    rng = np.random.default_rng(31)
    sl = rng.integers(1, 3000, 64).tolist()
    note(f"decode default CTAs, B=64 KH=32 G=1, sum(L)={sum(sl)}")
    q, k, v, sl = inputs(64, 32, 32, 128, sl, seed=31)
    need = A.attn_decode_workspace_bytes(64, 32, 32, 128, 0)
    assert need > A.attn_decode_workspace_bytes(64, 32, 32, 128, 256)
    ws = torch.zeros(need // 4 + 1, dtype=torch.int32, device="cuda")
    rows = np.random.default_rng(32).choice(64 * 32, 256, replace=False)
    err, got = decode_err(q, k, v, sl, rows=rows, workspace=ws, schedule=A.ATTN_SCHEDULE_STREAM_K)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    one = gpu_decode(q, k, v, sl, schedule=A.ATTN_SCHEDULE_STREAM_K, num_ctas=256)
    assert np.abs(got - one).max() <= 1e-5


@pytest.mark.parametrize("name", ["long_mqa", "ragged"])
def test_fixed_split_full_size(name):
    s = W.decode_workload(name)
    note(f"decode fixed split full-size {name}")
    q, k, v, sl = W.decode_inputs(s, device="cuda")
    err, _ = decode_err(q, k, v, sl.tolist(), scale_mult=s.score_mult, schedule=A.ATTN_SCHEDULE_FIXED_SPLIT)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    del q, k, v
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ wide heads

def ctas_per_head(sl, KH, T, P):
    """CTAs holding a piece of each (request, kv head) under the stream-K plan."""
    _, _, cta, seg = A.attn_decode_plan(sl, KH, T, P)
    out = []
    for s in range(len(sl) * KH):
        if seg[s + 1] == seg[s]:
            out.append(0)
            continue
        lo = np.searchsorted(cta, seg[s], side="right") - 1
        hi = np.searchsorted(cta, seg[s + 1] - 1, side="right") - 1
        out.append(int(hi - lo + 1))
    return np.array(out)


@pytest.mark.parametrize("Hsz", [64, 128, 256])
def test_wide_and_narrow_heads_in_one_call(Hsz):
    # request 0's heads span well over 16 CTAs (merged by the wide merge kernel), request 2's
    # a few (merged inside the tile kernel), request 1's one (finished by its CTA)
    sl = [120000, 300, 3000, 0]
    T, P = 128, 256
    widths = ctas_per_head(sl, 2, T, P)
    note(f"decode wide+narrow heads Hsz={Hsz}: CTAs per head {widths.tolist()}")
    assert widths.max() > 16 and ((widths > 1) & (widths <= 16)).any()
    q, k, v, sl = inputs(4, 8, 2, Hsz, sl, seed=90 + Hsz)
    err, got = decode_err(q, k, v, sl, tile_keys=T, num_ctas=P)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    assert np.all(got[3] == 0)


@pytest.mark.parametrize("P", [17, 255, 4096])
def test_wide_head_widths(P):
    # one head split over P CTAs, from just above the in-kernel merge width to the maximum
    q, k, v, sl = inputs(1, 8, 1, 128, [65536], seed=91)
    T = 16
    assert ctas_per_head(sl, 1, T, P).max() == P
    err, _ = decode_err(q, k, v, sl, tile_keys=T, num_ctas=P)
    note(f"decode one head over P={P}: max err {err:.3e}")
    assert err <= DECODE_TOL
    # a second call reuses the workspace: same values up to the fp32 summation order that
    # the waves' dynamic block claims choose
    again = gpu_decode(q, k, v, sl, tile_keys=T, num_ctas=P)
    assert np.abs(again - gpu_decode(q, k, v, sl, tile_keys=T, num_ctas=P)).max() <= 1e-5
