"""GPU parity of decode with more than 16 query columns per kv head, against the fp64 oracle.

A workgroup holds the G query heads of a kv head (times q_len drafted tokens) as MFMA
columns, in blocks of 16, so one pass over K/V serves all of them.  Cases:
  * MQA over many query heads ("필수 LLM 최적화 기법(2)", section 1-1: models with 32 or
    64 query heads sharing one K/V head), with the long context of the MQA shape;
  * speculative verification at the lecture page's draft lengths ("추론 최적화", section 5,
    gamma around 5) over Llama-3's group of 4 and over G = 8;
  * the edges of the column blocks (17, 32, 33, 64 columns), forced splits that put piece
    boundaries everywhere, FP8 and paged caches, device seqlens, and the limits.
Bar: max |err| <= 2e-3 on the fp32 outputs.
"""
import math

import numpy as np
import pytest
import torch

import attention_gqa_decode_amd as A
import oracle
from attention_gqa_decode_amd import workloads as W
from attention_gqa_decode_amd.workloads import bits
from gpu_util import DECODE_TOL, decode_err, gpu_decode, note, oracle_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def inputs(B, Hq, KH, Hsz, seqlens, seed):
    shape = W.DecodeShape("c", B, Hq, KH, Hsz, tuple(seqlens), seed=seed)
    q, k, v, sl = W.decode_inputs(shape, device="cuda")
    return q, k, v, sl.tolist()


@pytest.mark.parametrize("Hsz,G", [(64, 17), (64, 32), (64, 33), (64, 64), (128, 17), (128, 24), (128, 32),
                                   (128, 33), (128, 48), (128, 64), (256, 17), (256, 32)])
def test_wide_groups(Hsz, G):
    KH = 2
    sl = [1, 100, 517, 3000]
    note(f"decode wide group Hsz={Hsz} G={G} sl={sl}")
    q, k, v, sl = inputs(4, G * KH, KH, Hsz, sl, seed=500 + G + Hsz)
    err, got = decode_err(q, k, v, sl)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    # forced splits: pieces end inside blocks, heads merged in-kernel and by the wide merge
    for T, P in [(16, 37), (48, 300)]:
        err2, got2 = decode_err(q, k, v, sl, tile_keys=T, num_ctas=P)
        note(f"  T={T} P={P}: max err {err2:.3e}")
        assert err2 <= DECODE_TOL
        assert np.abs(got2 - got).max() <= 1e-5


@pytest.mark.parametrize("Hq", [32, 64])
def test_mqa_many_heads_long_context(Hq):
    # one K/V head under Hq query heads at 65,536 keys: every CTA of the GPU streams part
    # of the one context, and the head's partials are merged by the wide merge
    L = 65536
    note(f"decode MQA Hq={Hq} KH=1 L={L}")
    q, k, v, sl = inputs(1, Hq, 1, 128, [L], seed=600 + Hq)
    err, got = decode_err(q, k, v, sl)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    # the same heads as Hq / 16 separate groups of 16 give the same numbers
    parts = []
    for h0 in range(0, Hq, 16):
        parts.append(gpu_decode(q[:, h0:h0 + 16].contiguous(), k, v, sl))
    assert np.abs(np.concatenate(parts, axis=1) - got).max() <= 1e-5


def multi_err(q, k, v, sl, **kw):
    KH, Hsz = k.shape[1], k.shape[3]
    got = A.attn_decode_multi(q, k, v, sl, **kw)
    torch.cuda.synchronize()
    got = got.cpu().double().numpy().reshape(-1, Hsz)
    ref = oracle.decode_multi(bits(q), bits(k), bits(v), sl, KH, 1 / math.sqrt(Hsz)).reshape(-1, Hsz)
    assert np.all(np.isfinite(got))
    return float(np.abs(got - ref).max()), got


@pytest.mark.parametrize("G,gamma,Hsz", [(4, 5, 128), (4, 8, 128), (8, 5, 128), (8, 8, 64), (16, 2, 128),
                                         (2, 16, 64), (32, 2, 128), (4, 8, 256), (16, 2, 256), (64, 1, 128)])
def test_multi_token_many_columns(G, gamma, Hsz):
    sl = [gamma, 0, 700, 64, 2049]
    note(f"multi-token decode G={G} gamma={gamma} Hsz={Hsz} ({G * gamma} columns)")
    shape = W.DecodeShape("m", len(sl), 2 * G, 2, Hsz, tuple(sl), seed=700 + G * gamma + Hsz)
    q = W.randn_bf16((len(sl), 2 * G, gamma, Hsz), shape.seed, "cuda")
    _, k, v, _ = W.decode_inputs(shape, device="cuda")
    err, got = multi_err(q, k, v, sl)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    assert np.all(got.reshape(len(sl), -1)[1] == 0)
    err2, _ = multi_err(q, k, v, sl, tile_keys=16, num_ctas=300)
    note(f"  forced split: max err {err2:.3e}")
    assert err2 <= DECODE_TOL


def test_llama3_verification_full_size():
    # Llama-3-8B-shaped batch verifying gamma = 8 drafted tokens (32 columns per kv head);
    # sampled rows against the oracle
    s = W.decode_workload("llama3_8b")
    gamma = 8
    note(f"multi-token llama3_8b gamma={gamma}")
    q = W.randn_bf16((s.B, s.Hq, gamma, s.Hsz), s.seed + 17, "cuda")
    _, k, v, sl = W.decode_inputs(s, device="cuda")
    sl = sl.tolist()
    got = A.attn_decode_multi(q, k, v, sl)
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(s.B * s.Hq * gamma, 256, replace=False)
    ref = oracle.decode_multi(bits(q), bits(k), bits(v), sl, s.KH, 1 / math.sqrt(s.Hsz), rows=rows)
    g = got.cpu().double().numpy().reshape(-1, s.Hsz)
    err = float(np.abs(g[rows] - ref.reshape(-1, s.Hsz)[rows]).max())
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL


def test_wide_group_fp8_and_paged():
    G, KH, Hsz = 32, 2, 128
    sl = [900, 33, 4100]
    shape = W.DecodeShape("f", len(sl), G * KH, KH, Hsz, tuple(sl), seed=810)
    q, k8, v8, _ = W.decode_inputs_fp8(shape, device="cuda", k_scale=0.5, v_scale=2.0)
    got = A.attn_decode_ex(q, k8, v8, sl, k_scale=0.5, v_scale=2.0)
    torch.cuda.synchronize()
    ref = oracle.decode_fp8(bits(q), W.codes(k8), W.codes(v8), np.asarray(sl), G * KH, KH, 1 / math.sqrt(Hsz),
                            0.5, 2.0)
    err = float(np.abs(got.cpu().double().numpy() - ref).max())
    note(f"FP8 G=32: max err {err:.3e}")
    assert err <= DECODE_TOL
    q, k, v, sl = inputs(len(sl), G * KH, KH, Hsz, sl, seed=811)
    kp, vp, table = W.paged_layout(k, v, sl, 16, seed=3)
    got = A.attn_decode_paged(q, kp, vp, table, sl)
    torch.cuda.synchronize()
    assert np.abs(got.cpu().double().numpy() - gpu_decode(q, k, v, sl)).max() <= 1e-5


def test_wide_group_device_seqlens():
    G, KH, Hsz = 48, 1, 128
    sl = [3000, 0, 129]
    q, k, v, _ = inputs(len(sl), G * KH, KH, Hsz, sl, seed=812)
    dev = torch.tensor(sl, dtype=torch.int32, device="cuda")
    got = A.attn_decode_ex(q, k, v, dev)
    torch.cuda.synchronize()
    ref = oracle_decode(q, k, v, sl, KH, 1 / math.sqrt(Hsz))
    err = float(np.abs(got.cpu().double().numpy() - ref).max())
    note(f"device seqlens G=48: max err {err:.3e}")
    assert err <= DECODE_TOL


def test_column_limits_rejected():
    q, k, v, sl = inputs(1, 2 * 65, 2, 64, [10], seed=813)
    with pytest.raises(A.AttnError) as e:
        A.attn_decode_ex(q, k, v, sl)
    assert e.value.status == A.ATTN_ERR_UNSUPPORTED
    q, k, v, sl = inputs(1, 33, 1, 256, [10], seed=814)
    with pytest.raises(A.AttnError) as e:
        A.attn_decode_ex(q, k, v, sl)
    assert e.value.status == A.ATTN_ERR_UNSUPPORTED
