// Host-only harness over the LeanTile plan header the kernels use.  It walks
// every CTA's tile range exactly as the decode tile kernel does and lists, for
// every segment, the partial slots the merge kernel would read.  Built with g++
// by tests/test_plan.py; no GPU involved.
#include <stdint.h>

#include <vector>

#include "../../attention_gqa_decode_amd/csrc/plan.h"

extern "C" {

// Plan as the library builds it; splits > 0 selects the fixed split (P = B*KH*splits).
static LeanPlan make_plan(const int32_t *seqlens, int B, int KH, int T, int P, int splits) {
    LeanPlan p;
    p.B = B;
    p.KH = KH;
    p.T = T;
    int64_t acc = 0;
    for (int b = 0; b < B; ++b) {
        p.seqlen[b] = seqlens[b];
        p.tile_prefix[b] = (int32_t)acc;
        acc += (int64_t)KH * ((seqlens[b] + (int64_t)T - 1) / T);
    }
    p.tile_prefix[B] = (int32_t)acc;
    p.N = acc;
    p.mode = splits > 0 ? kPlanFixedSplit : kPlanStreamK;
    p.splits = splits > 0 ? splits : 1;
    p.P = splits > 0 ? B * KH * splits : P;
    return p;
}

// The kernels' exact floor(a b / d) and the stream-K range functions on a plan
// of N tiles over P CTAs (only N, P and the mode matter to them).
int64_t harness_muldiv(int64_t a, int64_t b, int64_t d) { return plan_muldiv(a, b, d); }

static LeanPlan streamk_plan(int64_t N, int P) {
    LeanPlan p = {};
    p.B = 1;
    p.KH = 1;
    p.T = 1;
    p.N = N;
    p.P = P;
    p.mode = kPlanStreamK;
    p.splits = 1;
    return p;
}

int64_t harness_cta_begin(int64_t N, int P, int c) { return plan_cta_begin(streamk_plan(N, P), c); }

int harness_cta_of_tile(int64_t N, int P, int64_t t) { return plan_cta_of_tile(streamk_plan(N, P), t); }

// rows of 8 int64: cta, b, kh, tile_begin, tile_end, key_begin, key_end, slot (-1 = whole segment)
int64_t harness_pieces(const int32_t *seqlens, int B, int KH, int T, int P, int splits, int64_t *rows,
                       int64_t max_rows) {
    LeanPlan p = make_plan(seqlens, B, KH, T, P, splits);
    P = p.P;
    int64_t n = 0;
    for (int c = 0; c < P; ++c) {
        int64_t t = plan_cta_begin(p, c), te = plan_cta_begin(p, c + 1);
        while (t < te) {
            LeanPiece pc = plan_piece_at(p, t, te);
            bool whole = pc.tile_begin == pc.seg_begin && pc.tile_end == pc.seg_end;
            if (n < max_rows) {
                int64_t *r = rows + 8 * n;
                r[0] = c; r[1] = pc.b; r[2] = pc.kh; r[3] = pc.tile_begin; r[4] = pc.tile_end;
                r[5] = pc.key_begin; r[6] = pc.key_end; r[7] = whole ? -1 : plan_slot(p, c, pc.seg_begin);
            }
            ++n;
            t = pc.tile_end;
        }
    }
    return n;
}

// For segment s = b*KH + kh: writes the slots the merge kernel reads, returns their count
// (0 when the segment is finished by one CTA or is empty).
int harness_merge_slots(const int32_t *seqlens, int B, int KH, int T, int P, int splits, int s, int32_t *slots,
                        int max_slots) {
    LeanPlan p = make_plan(seqlens, B, KH, T, P, splits);
    int b = s / KH, kh = s % KH;
    int nb = plan_tiles_per_segment(p, b);
    if (nb == 0) return 0;
    int64_t seg_begin = p.tile_prefix[b] + (int64_t)kh * nb;
    int c_lo = plan_cta_of_tile(p, seg_begin), c_hi = plan_cta_of_tile(p, seg_begin + nb - 1);
    if (c_lo == c_hi) return 0;
    int k = c_hi - c_lo + 1;
    for (int i = 0; i < k && i < max_slots; ++i) slots[i] = i == 0 ? plan_slot(p, c_lo, seg_begin) : 2 * (c_lo + i);
    return k;
}

// For every segment s = b*KH + kh: the first CTA and the number of CTAs that
// hold its pieces, from plan_segment_ctas (n = 0 for an empty segment).
// Returns how many segments are split over more than `width` CTAs.
int harness_segment_ctas(const int32_t *seqlens, int B, int KH, int T, int P, int splits, int width, int32_t *c_lo,
                         int32_t *n) {
    LeanPlan p = make_plan(seqlens, B, KH, T, P, splits);
    int wide = 0;
    for (int b = 0; b < B; ++b) {
        const int nb = plan_tiles_per_segment(p, b);
        for (int kh = 0; kh < KH; ++kh) {
            const int s = b * KH + kh;
            c_lo[s] = n[s] = 0;
            if (nb == 0) continue;
            const int64_t s0 = p.tile_prefix[b] + (int64_t)kh * nb;
            const SegmentCtas sc = plan_segment_ctas(p, s0, s0 + nb);
            c_lo[s] = sc.c_lo;
            n[s] = sc.n;
            wide += sc.n > width;
        }
    }
    return wide;
}

// The selector's makespan of one workgroup per segment over R resident slots.
int64_t harness_whole_segments_makespan(const int32_t *seqlens, int B, int KH, int T, int R) {
    LeanPlan p = make_plan(seqlens, B, KH, T, R, 0);
    std::vector<int64_t> heap(R > 0 ? R : 1);
    return plan_whole_segments_makespan(p, R, heap.data());
}
}

