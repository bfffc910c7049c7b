// plan.h -- the LeanTile work split, shared by the host planner and the kernels.
//
// Source: "LeanAttention" digest (siliconandsystems.com), sections "조각별로 합칠
// 수 있는 정확한 소프트맥스" (a global work id maps tiles of (batch, head,
// context range) to CTAs, stream-K style) and "하드웨어에 맞춘 작업 단위" (tile
// count follows from the total work and the number of compute units; resident
// CTAs take the next tile instead of a fixed split).
//
// Numbering.  Segment s = b*KH + kh is the context of request b under kv head
// kh; it holds n_b = ceil(L_b / T) LeanTiles of T keys.  Tiles are numbered in
// segment order: batch b owns tiles [tile_prefix[b], tile_prefix[b+1]) with
// tile_prefix[b+1] - tile_prefix[b] = KH * n_b, and within the batch kv head
// kh owns the kh-th run of n_b tiles.  With N tiles and P CTAs, CTA c owns
// [floor(cN/P), floor((c+1)N/P)); the planner keeps P <= N so no CTA is empty
// and the loads of any two CTAs differ by at most one tile.
//
// Pieces and partial slots.  The part of a segment inside one CTA's range is
// a piece.  A piece that is the whole segment is finished by its CTA.  Only a
// CTA's first and last pieces can be partial, so each CTA c owns two partial
// slots: 2c for its first piece and 2c+1 for its last piece.  A segment whose
// tiles span CTAs c_lo..c_hi (c_lo < c_hi) leaves one partial in each of them:
// CTA c_lo's slot is 2*c_lo if the segment starts exactly where c_lo's range
// starts (then it is c_lo's first piece) and 2*c_lo+1 otherwise; every later
// CTA holds the segment as its first piece, slot 2c.
//
// Fixed split (the FlashDecoding-style baseline of the digest's section
// "모양이 다른 프리필과 디코드": a fixed number of splits per launch).  Every
// segment s is cut into S_s = min(S, n_s) chunks of near-equal tile counts,
// chunk j = local tiles [floor(j n_s / S_s), floor((j+1) n_s / S_s)); CTA
// c = s*S + j takes chunk j, so P = B*KH*S and CTAs with j >= S_s own nothing.
// Chunks never cross segments, so every CTA holds at most one piece and the
// slot and merge rules above apply unchanged.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define ATTN_HD __host__ __device__ inline
#else
#define ATTN_HD inline
#endif

#ifndef ATTN_MAX_BATCH
#define ATTN_MAX_BATCH 256
#endif

enum : int { kPlanStreamK = 0, kPlanFixedSplit = 1 };

struct LeanPlan {
    int B;
    int KH;
    int T;      // keys per LeanTile
    int P;      // CTAs (stream-K: 1 <= P <= N when N > 0; fixed split: B*KH*splits)
    int64_t N;  // total tiles
    int mode;   // kPlanStreamK or kPlanFixedSplit
    int splits; // fixed split: CTAs per segment (S)
    int32_t seqlen[ATTN_MAX_BATCH];           // L_b
    int32_t tile_prefix[ATTN_MAX_BATCH + 1];  // tiles before batch b (all its kv heads)
};

// floor(a * b / d) for integers with 0 <= a * b < 2^53 and d > 0.  The double
// quotient is the correctly rounded x / d of an exactly represented x = a * b;
// when x / d is not an integer it lies at least 1/d below the next integer,
// while the rounding error is at most (x / d) * 2^-53 < 1/d, so the floor is
// exact.  This replaces 64-bit integer division, which the GPU runs as a long
// dependent instruction sequence, on the kernels' start-up path.
ATTN_HD int64_t plan_muldiv(int64_t a, int64_t b, int64_t d) {
    return (int64_t)__builtin_floor((double)(a * b) / (double)d);
}

ATTN_HD int plan_tiles_per_segment(const LeanPlan &p, int b) {
    return (p.tile_prefix[b + 1] - p.tile_prefix[b]) / p.KH;
}

// First tile of CTA c; plan_cta_begin(p, P) == N.
ATTN_HD int64_t plan_cta_begin(const LeanPlan &p, int c) {
    if (p.mode == kPlanStreamK) return plan_muldiv(c, p.N, p.P);  // c N < 2^12 2^31
    const int s = c / p.splits, j = c % p.splits;
    if (s >= p.B * p.KH) return p.N;
    const int b = s / p.KH, kh = s % p.KH;
    const int n = plan_tiles_per_segment(p, b);
    const int64_t seg_begin = p.tile_prefix[b] + (int64_t)kh * n;
    const int chunks = n < p.splits ? n : p.splits;
    if (chunks == 0) return seg_begin;
    const int jj = j < chunks ? j : chunks;
    return seg_begin + plan_muldiv(jj, n, chunks);
}

ATTN_HD int plan_batch_of_tile(const LeanPlan &p, int64_t t);

// CTA whose range contains tile t (0 <= t < N).
ATTN_HD int plan_cta_of_tile(const LeanPlan &p, int64_t t) {
    if (p.mode == kPlanStreamK) return (int)plan_muldiv((t + 1) * p.P - 1, 1, p.N);  // largest c with floor(cN/P) <= t
    const int b = plan_batch_of_tile(p, t);
    const int n = plan_tiles_per_segment(p, b);
    const int local = (int)(t - p.tile_prefix[b]);
    const int kh = local / n;
    const int u = local - kh * n;
    const int chunks = n < p.splits ? n : p.splits;
    const int j = (int)plan_muldiv((int64_t)(u + 1) * chunks - 1, 1, n);  // largest j with floor(j n / chunks) <= u
    return (b * p.KH + kh) * p.splits + j;
}

// Batch owning tile t (0 <= t < N): the b with tile_prefix[b] <= t < tile_prefix[b+1].
ATTN_HD int plan_batch_of_tile(const LeanPlan &p, int64_t t) {
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (p.tile_prefix[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

struct LeanPiece {
    int b, kh;
    int64_t seg_begin, seg_end;    // tiles of the whole segment
    int64_t tile_begin, tile_end;  // tiles of this piece
    int key_begin, key_end;        // keys of this piece, 0 <= key_begin < key_end <= L_b
};

// The piece that starts at tile t inside a CTA range ending at cta_end.
ATTN_HD LeanPiece plan_piece_at(const LeanPlan &p, int64_t t, int64_t cta_end) {
    LeanPiece pc;
    pc.b = plan_batch_of_tile(p, t);
    int nb = plan_tiles_per_segment(p, pc.b);
    const int local = (int)(t - p.tile_prefix[pc.b]);  // tiles fit in 31 bits
    pc.kh = local / nb;
    pc.seg_begin = p.tile_prefix[pc.b] + (int64_t)pc.kh * nb;
    pc.seg_end = pc.seg_begin + nb;
    pc.tile_begin = t;
    pc.tile_end = pc.seg_end < cta_end ? pc.seg_end : cta_end;
    int L = p.seqlen[pc.b];
    pc.key_begin = (int)((pc.tile_begin - pc.seg_begin) * p.T);
    int64_t ke = (pc.tile_end - pc.seg_begin) * (int64_t)p.T;
    pc.key_end = ke < L ? (int)ke : L;
    return pc;
}

// Partial slot of CTA c's piece in a split segment that starts at tile seg_begin.
ATTN_HD int plan_slot(const LeanPlan &p, int c, int64_t seg_begin) {
    return 2 * c + (seg_begin <= plan_cta_begin(p, c) ? 0 : 1);
}

// The CTAs c_lo .. c_lo + n - 1 hold the pieces of the segment with tiles
// [seg_begin, seg_end) (non-empty).  n > 1 means the head is split and leaves
// one partial in each of them: partial i sits in slot plan_slot(p, c_lo,
// seg_begin) for i = 0 and in slot 2 (c_lo + i) otherwise.
struct SegmentCtas {
    int c_lo;
    int n;
};

ATTN_HD SegmentCtas plan_segment_ctas(const LeanPlan &p, int64_t seg_begin, int64_t seg_end) {
    SegmentCtas s;
    s.c_lo = plan_cta_of_tile(p, seg_begin);
    s.n = plan_cta_of_tile(p, seg_end - 1) - s.c_lo + 1;
    return s;
}

// Selector support (host side).  One workgroup per segment, launched in
// segment order onto R resident slots, each segment taking the slot that
// frees first (the dispatcher hands out workgroups as slots free up): the
// makespan in tiles, from a binary min-heap over the slots' finish times.
// `heap` must hold R entries.  Stream-K's makespan is ceil(N / R) plus its
// merges, so running every segment whole pays only when this comes out no
// longer than that: many segments of similar length.  A ragged batch, where
// a few long contexts finish last, does not ("LeanAttention" digest, section
// "모양이 다른 프리필과 디코드": fixed splits leave partial waves and idle units).
inline int64_t plan_whole_segments_makespan(const LeanPlan &p, int R, int64_t *heap) {
    if (R < 1) R = 1;
    int used = 0;
    int64_t makespan = 0;
    for (int b = 0; b < p.B; ++b) {
        const int64_t n = plan_tiles_per_segment(p, b);
        for (int kh = 0; kh < p.KH; ++kh) {
            int64_t t;
            if (used < R) {  // a free slot: push its finish time
                t = n;
                int i = used++;
                while (i > 0 && heap[(i - 1) / 2] > t) {
                    heap[i] = heap[(i - 1) / 2];
                    i = (i - 1) / 2;
                }
                heap[i] = t;
            } else {  // the earliest slot takes it: replace the root and sift down
                t = heap[0] + n;
                int i = 0;
                for (;;) {
                    int c = 2 * i + 1;
                    if (c >= used) break;
                    if (c + 1 < used && heap[c + 1] < heap[c]) ++c;
                    if (heap[c] >= t) break;
                    heap[i] = heap[c];
                    i = c;
                }
                heap[i] = t;
            }
            makespan = t > makespan ? t : makespan;
        }
    }
    return makespan;
}
