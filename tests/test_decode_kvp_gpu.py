"""GPU parity of the KV-sequence split (decode over key shards, then ``attn_merge_shards``).

With the KV sequence of each request cut into S shards (as across S devices), every shard
runs the decode kernel at its own shape and also returns ``out_lse``, the log2 of each
row's softmax denominator.  ``attn_merge_shards`` then rescales the shard rows to their
common max: the LeanAttention digest's exact merge of partial states, applied to shard
outputs.  The merged rows must match the fp64 oracle over the whole sequence (max |err| <=
2e-3) and the single-call decode (1e-5); ``out_lse`` itself must match the oracle's
log-sum-exp of the scores.
"""
import math

import numpy as np
import pytest
import torch

import attention_gqa_decode_amd as A
import oracle
from attention_gqa_decode_amd import workloads as W
from attention_gqa_decode_amd.workloads import bits
from gpu_util import DECODE_TOL, gpu_decode, note, oracle_decode

pytestmark = pytest.mark.gpu
LN2 = math.log(2.0)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def inputs(B, Hq, KH, Hsz, seqlens, seed, S=None):
    shape = W.DecodeShape("k", B, Hq, KH, Hsz, tuple(seqlens), seed=seed)
    q, k, v, sl = W.decode_inputs(shape, device="cuda", S=S)
    return q, k, v, sl.tolist()


def oracle_lse2(q, k, v, sl, KH, scale, rows):
    """log2 sum_j exp(scale q.k_j) per (b, h) row, from the oracle's partial state over all keys."""
    Hq = q.shape[1]
    qb, kb, vb = bits(q), bits(k), bits(v)
    out = []
    for r in rows:
        b, h = divmod(int(r), Hq)
        if sl[b] == 0:
            out.append(-math.inf)
            continue
        m, l, _ = oracle.partial_state(qb, kb, vb, Hq, KH, scale, b, h, 0, sl[b])
        out.append((m + math.log(l)) / LN2)
    return np.array(out)


@pytest.mark.parametrize("sl,KH,G,kw", [
    ([3000, 0, 1, 700], 2, 4, {}),                               # whole heads, a split head, an empty row
    ([5000, 777], 2, 4, dict(tile_keys=16, num_ctas=20)),        # heads merged inside the decode kernel
    ([40000], 1, 8, dict(tile_keys=64, num_ctas=256)),           # one head over 256 CTAs (wide merge)
])
def test_out_lse_matches_oracle(sl, KH, G, kw):
    q, k, v, sl = inputs(len(sl), G * KH, KH, 128, sl, seed=400 + len(sl))
    B, Hq = len(sl), G * KH
    lse = torch.empty(B * Hq, dtype=torch.float32, device="cuda")
    got = A.attn_decode_ex(q, k, v, sl, out_lse=lse, **kw)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(128)
    ref = oracle_lse2(q, k, v, sl, KH, scale, range(B * Hq))
    g = lse.cpu().double().numpy()
    fin = np.isfinite(ref)
    note(f"out_lse sl={sl} {kw}: max |err| {np.abs(g[fin] - ref[fin]).max():.3e}")
    assert np.array_equal(np.isfinite(g), fin) and np.all(g[~fin] < 0)
    assert np.abs(g[fin] - ref[fin]).max() <= 1e-4 * max(1.0, np.abs(ref[fin]).max())
    # the output itself is unchanged by asking for the lse
    assert np.abs(got.cpu().double().numpy() - gpu_decode(q, k, v, sl, **kw)).max() <= 1e-5


def shard_decode(q, k, v, sl, S, **kw):
    """Decode each of S contiguous key shards of every request; returns (outs, lses)."""
    B, Hq, Hsz = q.shape
    L = k.shape[2]
    cut = [L * s // S for s in range(S + 1)]
    outs = torch.empty((S, B, Hq, Hsz), dtype=torch.float32, device="cuda")
    lses = torch.empty((S, B, Hq), dtype=torch.float32, device="cuda")
    for s in range(S):
        ks, vs = k[:, :, cut[s]:cut[s + 1]].contiguous(), v[:, :, cut[s]:cut[s + 1]].contiguous()
        sls = [max(0, min(Lb, cut[s + 1]) - cut[s]) for Lb in sl]
        A.attn_decode_ex(q, ks, vs, sls, out=outs[s], out_lse=lses[s], **kw)
    torch.cuda.synchronize()
    return outs, lses


def test_long_context_split_eight_ways():
    # the long-context MQA shape (B=1, Hq=8, KH=1, L=262144) cut into 8 shards of 32768
    # keys, one per device in a KV-sequence split, each decoded at its real shape
    s = W.decode_workload("long_mqa")
    q, k, v, sl = W.decode_inputs(s, device="cuda")
    sl = sl.tolist()
    outs, lses = shard_decode(q, k, v, sl, 8)
    merged_lse = torch.empty((1, 8), dtype=torch.float32, device="cuda")
    got = A.attn_merge_shards(outs, lses, lse_out=merged_lse)
    torch.cuda.synchronize()
    g = got.cpu().double().numpy()
    ref = oracle_decode(q, k, v, sl, 1, 1 / math.sqrt(128))
    err = float(np.abs(g - ref).max())
    note(f"long_mqa over 8 KV shards: max err {err:.3e}")
    assert err <= DECODE_TOL
    assert np.abs(g - gpu_decode(q, k, v, sl)).max() <= 1e-5
    ref_lse = oracle_lse2(q, k, v, sl, 1, 1 / math.sqrt(128), range(8))
    assert np.abs(merged_lse.cpu().double().numpy().ravel() - ref_lse).max() <= 1e-4 * np.abs(ref_lse).max()


@pytest.mark.parametrize("S", [2, 3, 7])
def test_ragged_requests_over_uneven_shards(S):
    # ragged lengths: some requests end inside the first shards, so later shards hold no
    # key of them (lse = -inf, they contribute nothing); one request is empty everywhere
    sl = [9000, 150, 0, 4097, 31]
    q, k, v, sl = inputs(len(sl), 16, 4, 128, sl, seed=410 + S)
    outs, lses = shard_decode(q, k, v, sl, S)
    got = A.attn_merge_shards(outs, lses)
    torch.cuda.synchronize()
    g = got.cpu().double().numpy()
    ref = oracle_decode(q, k, v, sl, 4, 1 / math.sqrt(128))
    err = float(np.abs(g - ref).max())
    note(f"ragged over {S} KV shards: max err {err:.3e}")
    assert err <= DECODE_TOL
    assert np.all(g[2] == 0)


def test_merge_of_one_shard_is_the_identity():
    q, k, v, sl = inputs(2, 8, 2, 64, [500, 33], seed=420)
    outs, lses = shard_decode(q, k, v, sl, 1)
    got = A.attn_merge_shards(outs, lses)
    torch.cuda.synchronize()
    assert torch.equal(got, outs[0])
