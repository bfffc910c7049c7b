"""CPU checks of the seeded input generators (no attention arithmetic in them)."""
import numpy as np
import pytest
import torch

from attention_gqa_decode_amd import workloads as W


def paged_by_loop(k, v, seqlens, block_size, seed, spare=7):
    """The block scatter written out one logical block at a time."""
    B, KH, S, Hsz = k.shape
    nb = [(int(L) + block_size - 1) // block_size for L in seqlens]
    total = sum(nb) + spare
    perm = np.random.default_rng(seed).permutation(total)
    table = np.full((B, max(max(nb), 1) + 2), -1, dtype=np.int32)
    kp = torch.zeros((total, KH, block_size, Hsz), dtype=k.dtype)
    vp = torch.zeros_like(kp)
    o = 0
    for b in range(B):
        for i in range(nb[b]):
            blk = int(perm[o])
            o += 1
            table[b, i] = blk
            n = min(block_size, int(seqlens[b]) - i * block_size)
            kp[blk, :, :n] = k[b, :, i * block_size:i * block_size + n]
            vp[blk, :, :n] = v[b, :, i * block_size:i * block_size + n]
    return kp, vp, torch.from_numpy(table)


@pytest.mark.parametrize("seqlens,block_size", [
    ([37, 0, 64, 5], 16),   # ragged tails and an empty request
    ([100], 32),
    ([16, 48], 16),         # whole blocks only
    ([1, 1, 1], 64),
])
@pytest.mark.parametrize("fp8", [False, True])
def test_paged_layout_matches_block_by_block_scatter(seqlens, block_size, fp8):
    shape = W.DecodeShape("p", len(seqlens), 4, 2, 64, tuple(seqlens), seed=5)
    S = max(max(seqlens), 1) + 9  # rows past every length hold values that must not be copied
    if fp8:
        _, k, v, _ = W.decode_inputs_fp8(shape, device="cpu", S=S)
    else:
        _, k, v, _ = W.decode_inputs(shape, device="cpu", S=S)
    got = W.paged_layout(k, v, seqlens, block_size, seed=11)
    ref = paged_by_loop(k, v, seqlens, block_size, seed=11)
    for g, r in zip(got, ref):
        assert g.dtype == r.dtype and g.shape == r.shape
        assert torch.equal(g.view(torch.uint8) if g.dtype == torch.bfloat16 else g,
                           r.view(torch.uint8) if r.dtype == torch.bfloat16 else r)
