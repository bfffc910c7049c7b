"""GPU check of the cross-CTA merge protocol on repeated calls.

Partial states of a split head are written by CTAs that sit on different XCDs (consecutive
CTAs go to different XCDs) and read by the CTA that arrives last at the head's counter, or
by the wide-merge kernel.  The library reuses one workspace from call to call, so a merge
that read a partial before it was written would pick up the previous call's value.  Here
consecutive calls alternate between two unrelated K/V sets of the same shape (same plan,
same slots): a stale read would mix the two problems and miss the oracle by far more than
the tolerance.  Heads are split over 2..16 CTAs (the in-kernel merge) and over more than
16 (the merge kernel); the merge is the exact combine of partial softmax states
("LeanAttention" digest, section on the piecewise exact softmax).
"""
import math

import numpy as np
import pytest
import torch

from attention_gqa_decode_amd import workloads as W
from gpu_util import DECODE_TOL, gpu_decode, note, oracle_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def two_problems(B, Hq, KH, Hsz, sl, seed):
    # the second problem has other keys and values shifted by +1, so its outputs sit near 1
    # while the first one's sit near 0 (a long softmax average of N(0, 1) values)
    out = []
    for s, shift in ((seed, 0.0), (seed + 1, 1.0)):
        shape = W.DecodeShape("m", B, Hq, KH, Hsz, tuple(sl), seed=s)
        q, k, v, _ = W.decode_inputs(shape, device="cuda")
        v = (v.float() + shift).to(torch.bfloat16)
        out.append((q, k, v, oracle_decode(q, k, v, sl, KH, 1 / math.sqrt(Hsz))))
    return out


# (seqlens, KH, forced tile keys, CTAs): heads split over 2, 5, 16 and about 60 CTAs
@pytest.mark.parametrize("sl,KH,T,P", [
    ([4096, 4096], 2, 64, 8),
    ([3000, 5000, 700], 2, 32, 29),
    ([8192], 2, 16, 32),
    ([20000], 1, 64, 60),
])
def test_alternating_problems_merge_their_own_partials(sl, KH, T, P):
    probs = two_problems(len(sl), 8 * KH, KH, 128, sl, seed=900 + P)
    note(f"merge coherence sl={sl} KH={KH} T={T} P={P}, 24 alternating calls")
    errs = []
    for i in range(24):
        q, k, v, ref = probs[i % 2]
        got = gpu_decode(q, k, v, sl, tile_keys=T, num_ctas=P)
        errs.append(float(np.abs(got - ref).max()))
    note(f"  worst err {max(errs):.3e}")
    assert max(errs) <= DECODE_TOL
    # the two problems differ far beyond the tolerance, so a mixed-up partial cannot hide
    assert np.abs(probs[0][3] - probs[1][3]).min() > 100 * DECODE_TOL
