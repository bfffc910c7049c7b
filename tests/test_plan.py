"""CPU tests of the LeanTile planner (host export and the shared plan header).

The work split follows the LeanAttention digest, sections "조각별로 합칠 수 있는 정확한
소프트맥스" (global tile ids over (batch, head, context range), stream-K style) and
"하드웨어에 맞춘 작업 단위" (tile count from total work and unit count).  Properties:
every key of every (request, kv head) is covered exactly once, CTA loads differ by at
most one tile, only a CTA's first and last pieces are partial, every partial slot is
written once, and the merge reads exactly the slots the tile kernel wrote.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    out = tmp_path_factory.mktemp("plan") / "libplan_harness.so"
    src = os.path.join(ROOT, "tests", "harness", "plan_harness.cpp")
    subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-Wall", "-Werror", "-o", str(out), src],
                   check=True)
    lib = ctypes.CDLL(str(out))
    lib.harness_pieces.restype = ctypes.c_int64
    lib.harness_pieces.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_int64]
    lib.harness_segment_ctas.restype = ctypes.c_int
    lib.harness_segment_ctas.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.harness_muldiv.restype = ctypes.c_int64
    lib.harness_muldiv.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    lib.harness_cta_begin.restype = ctypes.c_int64
    lib.harness_cta_begin.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    lib.harness_cta_of_tile.restype = ctypes.c_int
    lib.harness_cta_of_tile.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int64]
    lib.harness_whole_segments_makespan.restype = ctypes.c_int64
    lib.harness_whole_segments_makespan.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                    ctypes.c_int]
    lib.harness_merge_slots.restype = ctypes.c_int
    lib.harness_merge_slots.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
    return lib


def pieces(harness, sl, KH, T, P, splits=0):
    sl = np.ascontiguousarray(sl, dtype=np.int32)
    n = harness.harness_pieces(sl.ctypes.data, len(sl), KH, T, P, splits, None, 0)
    rows = np.zeros((max(n, 1), 8), dtype=np.int64)
    harness.harness_pieces(sl.ctypes.data, len(sl), KH, T, P, splits, rows.ctypes.data, n)
    return rows[:n]


def merge_slots(harness, sl, KH, T, P, s, splits=0):
    sl = np.ascontiguousarray(sl, dtype=np.int32)
    buf = np.zeros(4 * P + 4, dtype=np.int32)
    k = harness.harness_merge_slots(sl.ctypes.data, len(sl), KH, T, P, splits, s, buf.ctypes.data, len(buf))
    return buf[:k].tolist()


def total_tiles(sl, KH, T):
    return sum(KH * ((L + T - 1) // T) for L in sl)


CASES = [
    ([1024], 2, 256, 8),
    ([8192] * 16, 8, 256, 256),
    ([262144], 1, 256, 256),
    ([262144], 1, 16, 1000),
    ([0, 1, 5, 0, 300, 17], 3, 16, 7),
    ([518, 64654, 3000, 777], 8, 100, 13),
    ([1], 1, 1, 1),
    ([33, 31, 0], 2, 1024, 3),
]


@pytest.mark.parametrize("sl,KH,T,P", CASES)
def test_every_key_covered_once_and_slots_consistent(harness, sl, KH, T, P, splits=0):
    N = total_tiles(sl, KH, T)
    if splits:
        P = len(sl) * KH * splits
    else:
        P = min(P, N) if N else 1
    rows = pieces(harness, sl, KH, T, P, splits)
    cover = {}
    per_cta_tiles = np.zeros(P, dtype=np.int64)
    written = {}
    for c, b, kh, tb, te, kb, ke, slot in rows:
        assert 0 <= kb < ke <= sl[b]
        cover.setdefault((b, kh), []).append((kb, ke))
        per_cta_tiles[c] += te - tb
        if slot >= 0:
            assert slot in (2 * c, 2 * c + 1)
            assert slot not in written, "partial slot written twice"
            written[slot] = (b, kh)
    for b, L in enumerate(sl):
        for kh in range(KH):
            segs = sorted(cover.get((b, kh), []))
            if L == 0:
                assert not segs
                continue
            assert segs[0][0] == 0 and segs[-1][1] == L
            for (a0, a1), (b0, b1) in zip(segs, segs[1:]):
                assert a1 == b0, "gap or overlap between pieces"
            expect = merge_slots(harness, sl, KH, T, P, b * KH + kh, splits)
            got = sorted(s for s, seg in written.items() if seg == (b, kh))
            if len(segs) == 1:
                assert expect == [] and got == []
            else:
                assert sorted(expect) == got
    if N:
        assert per_cta_tiles.sum() == N
        if splits:
            # fixed split: CTA s*S + j holds chunk j of segment s, chunks within a tile of each other
            for b, L in enumerate(sl):
                n = (L + T - 1) // T
                for kh in range(KH):
                    loads = per_cta_tiles[(b * KH + kh) * splits:(b * KH + kh + 1) * splits]
                    assert loads.sum() == n
                    chunks = min(n, splits)
                    assert np.all(loads[chunks:] == 0)
                    if chunks:
                        assert loads[:chunks].max() - loads[:chunks].min() <= 1 and loads[:chunks].min() >= 1
        else:
            assert per_cta_tiles.max() - per_cta_tiles.min() <= 1


@pytest.mark.parametrize("seed", range(20))
def test_random_plans(harness, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    KH = int(rng.integers(1, 9))
    sl = rng.integers(0, 5000, B)
    sl[rng.random(B) < 0.2] = 0
    T = int(rng.choice([1, 16, 32, 48, 100, 256, 1024]))
    P = int(rng.integers(1, 600))
    test_every_key_covered_once_and_slots_consistent(harness, sl.tolist(), KH, T, P)


@pytest.mark.parametrize("sl,KH,T,splits", [
    ([1024], 2, 256, 4),
    ([8192] * 16, 8, 256, 2),
    ([262144], 1, 256, 256),
    ([0, 1, 5, 0, 300, 17], 3, 16, 7),
    ([518, 64654, 3000, 777], 8, 100, 13),
    ([33, 31, 0], 2, 1024, 1),
])
def test_fixed_split_covers_every_key_once(harness, sl, KH, T, splits):
    test_every_key_covered_once_and_slots_consistent(harness, sl, KH, T, 0, splits=splits)


@pytest.mark.parametrize("seed", range(10))
def test_random_fixed_split_plans(harness, seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 30))
    KH = int(rng.integers(1, 9))
    sl = rng.integers(0, 5000, B)
    sl[rng.random(B) < 0.2] = 0
    T = int(rng.choice([1, 16, 32, 100, 256]))
    splits = int(rng.integers(1, max(2, 4096 // (B * KH))))
    test_every_key_covered_once_and_slots_consistent(harness, sl.tolist(), KH, T, 0, splits=splits)


def test_library_planner_matches_header(harness):
    import attention_gqa_decode_amd as A
    sl = [518, 64654, 3000, 0, 777]
    N, P, cta, seg = A.attn_decode_plan(sl, 8, 100, 13)
    assert N == total_tiles(sl, 8, 100) and P == 13
    assert cta[0] == 0 and cta[-1] == N and np.all(np.diff(cta) >= 1)
    assert np.all(np.diff(cta) - np.diff(cta).min() <= 1)
    assert seg[-1] == N and np.all(np.diff(seg) >= 0)
    rows = pieces(harness, sl, 8, 100, 13)
    for c in range(P):
        mine = rows[rows[:, 0] == c]
        assert mine[0, 3] == cta[c] and mine[-1, 4] == cta[c + 1]


# ------------------------------------------------------- split heads and wide merge

MERGE_FAN_IN, MAX_CTAS = 16, 4096   # heads split over more CTAs go to the wide merge kernel
MAX_WIDE_HEADS = (MAX_CTAS + MERGE_FAN_IN - 2) // (MERGE_FAN_IN - 1)


def segment_ctas(harness, sl, KH, T, P, splits=0):
    sl = np.ascontiguousarray(sl, dtype=np.int32)
    c_lo = np.zeros(len(sl) * KH, dtype=np.int32)
    n = np.zeros(len(sl) * KH, dtype=np.int32)
    wide = harness.harness_segment_ctas(sl.ctypes.data, len(sl), KH, T, P, splits, MERGE_FAN_IN, c_lo.ctypes.data,
                                        n.ctypes.data)
    return c_lo, n, wide


@pytest.mark.parametrize("sl,KH,T,P,splits", [
    ([262144], 1, 256, 256, 0),                # one long head over every CTA
    ([5000, 0, 17, 70000, 3], 3, 64, 97, 0),
    ([8192] * 16, 8, 256, 256, 0),
    ([100, 2000, 40000], 2, 16, 1000, 0),
    ([4000, 33, 0, 9000], 2, 64, 0, 20),      # fixed split with more than 16 chunks per head
])
def test_segment_ctas_match_the_pieces(harness, sl, KH, T, P, splits):
    """The CTAs that plan_segment_ctas names for a head are exactly those that hold one of its
    pieces, and the heads split over more than 16 CTAs are counted as wide."""
    c_lo, n, wide = segment_ctas(harness, sl, KH, T, P, splits)
    rows = pieces(harness, sl, KH, T, P, splits)
    for s in range(len(sl) * KH):
        b, kh = divmod(s, KH)
        owners = sorted(set(rows[(rows[:, 1] == b) & (rows[:, 2] == kh)][:, 0].tolist()))
        if not owners:
            assert n[s] == 0
            continue
        assert owners == list(range(owners[0], owners[0] + len(owners)))
        assert (c_lo[s], n[s]) == (owners[0], len(owners))
    assert wide == int((n > MERGE_FAN_IN).sum())


def test_wide_heads_stay_within_the_kernel_argument_list(harness):
    """A head split over more than 16 CTAs owns the whole ranges of at least 15 of them, so a
    plan of at most 4096 CTAs has at most ceil(4096 / 15) such heads (the merge kernel's
    list).  Checked on the densest packing: heads just long enough to span 17 CTAs."""
    rng = np.random.default_rng(3)
    worst = 0
    for per_cta in [1, 2, 3, 4]:
        for extra in [1, per_cta, 2 * per_cta - 1]:
            L = 15 * per_cta + extra          # tiles of T = 1 key per head
            KH = 2
            B = min(256, MAX_CTAS * per_cta // (KH * L) + 1)
            _, n, wide = segment_ctas(harness, [L] * B, KH, 1, MAX_CTAS, 0)
            worst = max(worst, wide)
            assert wide <= MAX_WIDE_HEADS
    for _ in range(20):
        B = int(rng.integers(1, 257))
        sl = rng.integers(0, 4000, size=B)
        KH = int(rng.integers(1, 9))
        P = int(min(MAX_CTAS, max(1, KH * sl.sum())))
        _, _, wide = segment_ctas(harness, sl, KH, 1, P, 0)
        assert wide <= MAX_WIDE_HEADS
    assert worst > 200  # the packing above really comes close to the bound


# ------------------------------------------------- exact integer arithmetic limits

def test_muldiv_is_exact_floor(harness):
    """floor(a b / d) through a double quotient equals exact integer division on the whole
    domain the planner uses (a b < 2^53): random draws, and numerators one below, at and
    one above a multiple of d, where a rounding error would show."""
    rng = np.random.default_rng(7)
    cases = []
    for _ in range(20000):
        d = int(rng.integers(1, 1 << 31))
        x = int(rng.integers(0, 1 << 53))
        cases.append((x, 1, d))
    for _ in range(20000):
        d = int(rng.integers(1, 1 << 31))
        k = int(rng.integers(0, ((1 << 53) - 2) // d))
        for x in (k * d - 1, k * d, k * d + 1):
            if 0 <= x < (1 << 53):
                cases.append((x, 1, d))
    for _ in range(20000):  # the stream-K form c * N / P
        P = int(rng.integers(1, 4097))
        N = int(rng.integers(1, 1 << 31))
        cases.append((int(rng.integers(0, P + 1)), N, P))
    for a, b, d in cases:
        assert harness.harness_muldiv(a, b, d) == (a * b) // d, (a, b, d)


@pytest.mark.parametrize("N", [(1 << 31) - 1, (1 << 31) - 2, 1_000_000_007, 4097, 4096])
@pytest.mark.parametrize("P", [4096, 4095, 977, 3, 1])
def test_stream_k_ranges_at_the_limits(harness, N, P):
    """CTA c's first tile is floor(c N / P) and the owner of tile t is the largest c with
    floor(c N / P) <= t, at N near 2^31 tiles and P up to the CTA limit."""
    if P > N:
        return
    rng = np.random.default_rng(N % 1000 + P)
    cs = sorted({0, 1, P - 1, P, *map(int, rng.integers(0, P + 1, 50))})
    for c in cs:
        assert harness.harness_cta_begin(N, P, c) == c * N // P, c
    ts = {0, N - 1}
    for c in cs[:-1]:
        b = c * N // P
        ts.update(x for x in (b - 1, b, b + 1) if 0 <= x < N)
    ts.update(map(int, rng.integers(0, N, 50)))
    for t in sorted(ts):
        c = harness.harness_cta_of_tile(N, P, t)
        assert c * N // P <= t < (c + 1) * N // P, (t, c)


# ------------------------------------------------------------------ selector


def makespan(harness, sl, KH, T, R):
    sl = np.ascontiguousarray(sl, dtype=np.int32)
    return harness.harness_whole_segments_makespan(sl.ctypes.data, len(sl), KH, T, R)


def makespan_naive(sl, KH, T, R):
    """Segments in order, each onto the slot that frees first (lowest index on ties)."""
    slots = [0] * R
    end = 0
    for L in sl:
        n = -(-int(L) // T)
        for _ in range(KH):
            i = min(range(R), key=lambda j: slots[j])
            slots[i] += n
            end = max(end, slots[i])
    return end


def test_whole_segments_makespan_matches_a_naive_dispatch(harness):
    rng = np.random.default_rng(7)
    for _ in range(200):
        B = int(rng.integers(1, 40))
        KH = int(rng.integers(1, 9))
        T = int(rng.choice([16, 64, 256]))
        R = int(rng.integers(1, 70))
        sl = rng.integers(0, 3000, B)
        assert makespan(harness, sl, KH, T, R) == makespan_naive(sl, KH, T, R), (B, KH, T, R)


def test_selector_rule_on_the_shapes_that_decide_it(harness):
    """Whole segments (no partial states) only when they finish within stream-K's even share."""
    from attention_gqa_decode_amd import workloads as W

    def whole_wins(sl, KH, T, R):
        N = sum(KH * (-(-int(L) // T)) for L in sl)
        return makespan(harness, sl, KH, T, R) <= -(-N // R)

    # many short uniform requests: every slot gets the same number of segments
    assert whole_wins([300] * 256, 8, 256, 512)
    # the ragged batch and its (G, Hsz) sweep points: a few long contexts would finish last
    for G in (1, 2, 4, 8, 16):
        for Hsz, T, R in ((64, 256, 512), (128, 256, 256), (256, 128, 256)):
            s = W.ragged_sweep_point(G, Hsz)
            assert not whole_wins(s.seqlens, s.KH, T, R), (G, Hsz)
    # a uniform long batch with fewer segments than slots leaves slots idle
    assert not whole_wins([8192] * 16, 8, 256, 256)
