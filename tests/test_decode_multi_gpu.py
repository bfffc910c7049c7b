"""GPU parity of multi-token decode (speculative verification) against the fp64 oracle.

gamma drafted tokens per request sit at the end of the cache; query t attends keys
0 .. L_b - gamma + t (lecture page "추론 최적화", section 5: the target model checks the
drafted positions at once).  The gamma x G query columns share one pass over K/V.
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
from gpu_util import DECODE_TOL, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def multi_inputs(B, Hq, KH, Hsz, gamma, seqlens, seed):
    shape = W.DecodeShape("m", B, Hq, KH, Hsz, tuple(seqlens), seed=seed)
    q = W.randn_bf16((B, Hq, gamma, Hsz), seed, "cuda")
    _, k, v, _ = W.decode_inputs(shape, device="cuda")
    return q, k, v, list(seqlens)


def multi_err(q, k, v, sl, rows=None, **kw):
    KH, Hsz = k.shape[1], k.shape[3]
    got = A.attn_decode_multi(q, k, v, sl, **kw)
    torch.cuda.synchronize()
    got = got.cpu().double().numpy().reshape(-1, Hsz)
    ref = oracle.decode_multi(bits(q), bits(k), bits(v), sl, KH, 1 / math.sqrt(Hsz), rows=rows).reshape(-1, Hsz)
    sel = np.arange(got.shape[0]) if rows is None else np.asarray(rows)
    assert np.all(np.isfinite(got[sel]))
    return float(np.abs(got[sel] - ref[sel]).max()), got


@pytest.mark.parametrize("G,gamma", [(4, 2), (4, 4), (8, 2), (1, 16), (2, 5), (16, 1)])
@pytest.mark.parametrize("Hsz", [64, 128])
def test_multi_token_shapes(G, gamma, Hsz):
    sl = [gamma, 0, 700, 64, 2049]
    note(f"multi-token decode G={G} gamma={gamma} Hsz={Hsz}")
    q, k, v, sl = multi_inputs(len(sl), 2 * G, 2, Hsz, gamma, sl, seed=80 + G * gamma + Hsz)
    err, got = multi_err(q, k, v, sl)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    assert np.all(got.reshape(len(sl), -1)[1] == 0)


@pytest.mark.parametrize("T,P", [(16, 9), (1, 64), (48, 300), (1024, 2)])
def test_multi_token_forced_splits(T, P):
    # small LeanTiles put piece boundaries inside the drafted tokens, so some pieces hold
    # keys that only the later drafted tokens may see
    q, k, v, sl = multi_inputs(2, 8, 2, 128, 4, [1000, 37], seed=81)
    err, _ = multi_err(q, k, v, sl, tile_keys=T, num_ctas=P)
    assert err <= DECODE_TOL


def test_multi_token_gamma1_equals_decode():
    q, k, v, sl = multi_inputs(3, 16, 4, 128, 1, [900, 1, 4000], seed=82)
    a = A.attn_decode_multi(q, k, v, sl)
    b = A.attn_decode_ex(q[:, :, 0].contiguous(), k, v, sl)
    torch.cuda.synchronize()
    assert (a[:, :, 0] - b).abs().max().item() <= 1e-5


def test_multi_token_fp8_cache():
    shape = W.DecodeShape("m", 2, 8, 2, 128, (3000, 500), seed=83)
    q = W.randn_bf16((2, 8, 3, 128), 83, "cuda")
    _, k, v, _ = W.decode_inputs_fp8(shape, device="cuda", k_scale=0.5, v_scale=2.0)
    got = A.attn_decode_multi(q, k, v, [3000, 500], k_scale=0.5, v_scale=2.0)
    kb = k.view(torch.float8_e4m3fn).to(torch.bfloat16)
    vb = v.view(torch.float8_e4m3fn).to(torch.bfloat16)
    base = A.attn_decode_multi(q, kb, vb, [3000, 500], scale=0.5 / math.sqrt(128))
    torch.cuda.synchronize()
    assert (got - 2.0 * base).abs().max().item() <= 1e-5


def test_multi_token_full_size_llama3():
    s = W.decode_workload("llama3_8b")
    gamma = 4
    note(f"multi-token decode full-size llama3_8b, gamma={gamma}")
    q, k, v, sl = multi_inputs(s.B, s.Hq, s.KH, s.Hsz, gamma, s.seqlens, seed=84)
    rows = np.random.default_rng(85).choice(s.B * s.Hq * gamma, 256, replace=False)
    err, _ = multi_err(q, k, v, sl, rows=rows)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    del q, k, v
    torch.cuda.empty_cache()


def test_multi_token_wide_head_with_masked_partials():
    # G = 1, gamma = 16, 16-key tiles over 300 CTAs: each head is merged by the wide merge
    # kernel, and the partials of the last keys hold no key that the first drafted tokens
    # may see (their running max is -inf)
    q, k, v, sl = multi_inputs(1, 2, 2, 128, 16, [3000], seed=84)
    err, _ = multi_err(q, k, v, sl, tile_keys=16, num_ctas=300)
    note(f"multi-token wide head: max err {err:.3e}")
    assert err <= DECODE_TOL
