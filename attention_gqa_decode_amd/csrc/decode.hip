// decode.hip -- GQA decode on gfx950: the LeanTile kernel, with the merge of split heads fused in.
//
// What runs (sources by page title and section):
//  * co-design page "장문 컨텍스트 추론을 위한 어텐션 공동 설계", sections
//    "FlashAttention과 GEMM 모양" and "그룹 크기(G)의 영향": QK^T -> online
//    softmax (running max m and sum l) -> PV fused over streamed K/V tiles; in
//    decode the matmul M dimension is the group size G, so one pass over a K/V
//    byte serves all G query heads of the group.
//  * "LeanAttention" digest, sections "조각별로 합칠 수 있는 정확한 소프트맥스"
//    and "하드웨어에 맞춘 작업 단위": LeanTiles numbered globally and split evenly
//    over resident CTAs; partial (m, l, O) states merged by rescaling to the
//    common max.  The work split itself lives in plan.h.
//
// gfx950 mapping.  A workgroup is 8 wave64s, or 4 where the query columns'
// accumulators need more than 256 registers per wave (DecodeCfg).  Inside a
// piece (one (b, kv head) context range) each wave claims blocks of 16 or 32
// keys from an LDS counter and never synchronises with the other waves until
// the piece ends.  Per block a wave
//   1. streams the K and V rows from HBM with fully coalesced, non-temporal
//      loads (16 bytes of bf16, or 8 bytes of FP8 codes that are widened to
//      bf16 on the way; each load instruction covers whole 128-byte lines; a
//      measured 6.7-7.1 TB/s pattern, against ~6.0 TB/s when each instruction
//      takes 64 bytes of 16 rows) into registers, while the previous block is
//      being computed, and parks them in its own LDS stage;
//   2. BMM1 on v_mfma_f32_16x16x32_bf16 with A = K (16 keys x 32 d, read from
//      the stage), B = Q^T (32 d x 16 query columns: the G heads times the
//      drafted tokens, in blocks of 16, columns past them zero): S^T lands
//      with the column index on lanes and four consecutive keys per lane;
//   3. online softmax in the log2 domain; the row max over the block needs two
//      cross-lane steps (lanes 16 and 32 apart);
//   4. V^T straight from the row-major V stage: transposing LDS reads
//      (ds_read_b64_tr_b16) hand each lane four consecutive keys of one d;
//   5. BMM2 on MFMA with A = V^T (16 d x 32 keys), B = P^T (32 keys x 16 heads);
//      P is split into bf16 hi + lo parts (two MFMAs), so the weights keep
//      ~2^-17 relative accuracy instead of bf16's 2^-9.
//  The key order inside each MFMA contraction is chosen so that the lanes that
//  hold S^T after step 2 already hold the P^T operand of step 5, and step 4
//  reads V^T in that same key order: no shuffles beyond the two row-max steps.
//  At the end of a piece every wave parks its state in LDS and, after one
//  barrier, each thread merges one float4 column over the waves (max,
//  rescale, sum) and writes it either as the final output or, when the head
//  is split over several CTAs, into a partial slot.  A head split
//  over at most 16 CTAs is merged by the CTA that arrives last at its atomic
//  counter, which rescales the partials to their common max.  A wider head is
//  merged by merge_wide_kernel, launched next on the stream: one CU reads only
//  about 20-30 GB/s of freshly written partials, so a single merging CTA (or a
//  tree of them) would sit on the critical path for microseconds, while the
//  merge kernel reads them with one workgroup per 16 output columns.  No CTA
//  ever waits for another, so neither merge needs co-residency.
#include "common.h"

#include <hip/hip_ext.h>

#include <atomic>
#include <type_traits>

namespace attn {
namespace {

constexpr float kLazyMax = 8.f;  // lazy running-max threshold in log2 units (weights <= 256)

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load_row8(const uint16_t *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Four keys of one d column of a row-major bf16 LDS stage with row stride rs:
// within each 16-lane block, lane t reads 8 bytes at row key0 + t/4, columns
// d0 + 4 (t % 4) .. +3, and the transposing read (ds_read_b64_tr_b16) hands
// lane i the column d0 + i at rows key0 .. key0 + 3.
__device__ __forceinline__ i16x4 v_cols(const uint16_t *stage, int rs, int key0, int d0, int t) {
    const uint16_t *p = stage + (key0 + (t >> 2)) * rs + d0 + 4 * (t & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)((__attribute__((address_space(3))) uint16_t *)p));
}

// Max and sum of a column's value over the four 16-lane groups.
__device__ __forceinline__ float wave_max_over_groups(float x) {
    float a, b;
    swap16(x, a, b);
    return pair_max32(fmaxf(a, b));
}

__device__ __forceinline__ float wave_sum_over_groups(float x) {
    float a, b;
    swap16(x, a, b);
    return pair_sum32(a + b);
}

// Launch shape for head dimension HSZ and NCB blocks of 16 MFMA columns (the
// query columns: G heads x q_len drafted tokens, at most 16 x NCB of them).
//  * KPB keys per wave block: 32, or 16 at HSZ = 256 (so one block is 16 KiB
//    of bf16 K+V there and its staging takes 64 registers per lane), with 64
//    columns at HSZ = 128 (whose accumulators leave no room for more), and for
//    bf16 at HSZ = 128 with up to 16 columns: there the 8 KiB blocks measured
//    1-3% faster than 16 KiB ones (each wave's load-to-use chain is shorter and
//    the LeanTile finer), while at HSZ = 64, with more columns and for FP8 the
//    larger block was as fast or faster.
//  * W waves per workgroup: 8 (two per SIMD, 256 registers each) where the
//    wave fits, else 4 (one per SIMD, up to 512 registers with the AGPRs).
template <int HSZ, int NCB, bool FP8>
struct DecodeCfg {
    static constexpr int KPB = HSZ == 256 || HSZ * NCB >= 512 || (HSZ == 128 && NCB == 1 && !FP8) ? 16 : 32;
    static constexpr int KB = KPB / 16;                  // 16-key MFMA row blocks per wave block
    static constexpr int W = NCB == 1 ? 8 : (NCB == 2 && HSZ == 64 ? 8 : 4);
    static constexpr int NCMAX = 16 * NCB;               // MFMA columns
    static constexpr int NS = HSZ / 32;                  // MFMA K steps over d
    static constexpr int ND = HSZ / 16;                  // 16-wide d blocks of the output
    static constexpr int RS = HSZ + 8;                   // staged row stride (bf16), 16 B pad
    static constexpr int STAGE = 2 * KPB * RS;           // bf16 per wave: K rows then V rows
};

// One wave's next block in registers: fully coalesced loads (lane l of load j
// reads chunk (64j + l) of the block, row-major over keys), marked
// non-temporal because every byte is used exactly once.  Rows past klast are
// clamped re-reads of row klast (their scores are masked later).  A chunk is 8
// elements: 16 bytes of bf16, or 8 bytes of FP8 E4M3 codes, which widen to the
// same 16 bytes of bf16, so every lane parks one contiguous 16-byte run per
// chunk and the LDS stores of a wave cover whole rows without bank conflicts.
template <int HSZ, bool FP8, int KPB>
struct KvCfg {
    static constexpr int EPC = 8;                                     // elements per chunk
    static constexpr int CPR = HSZ / EPC;                             // chunks per row
    static constexpr int LOADS = 2 * KPB * CPR / 64;                  // chunks per lane per block (K + V)
    static_assert(KPB * CPR % 64 == 0, "a block's chunks split evenly over the lanes");
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int HSZ, bool FP8, int KPB>
struct Staged {
    typedef typename std::conditional<FP8, u32x2, u32x4>::type chunk_t;
    chunk_t r[KvCfg<HSZ, FP8, KPB>::LOADS];
};

// Where the rows of one (request, kv head) context live.  Contiguous: row j of
// the context is row j of [S][Hsz] at kbase/vbase.  Paged: row j sits in
// physical block table[j >> log2_bs] of the pools [num_blocks][KH][bs][Hsz],
// at in-block row j & (bs - 1); out-of-range block ids are clamped into the
// pool, so a bad table gives wrong numbers, never an out-of-bounds access.
template <bool PAGED>
struct KvRows {
    const uint8_t *kbase, *vbase;  // contiguous: this context; paged: the pools
    const int32_t *table;          // paged: this request's row of the block table
    int kh, KH, log2_bs, max_block;
    __device__ __forceinline__ int64_t row_offset(int key, int row_bytes) const {
        if constexpr (!PAGED) {
            return (int64_t)key * row_bytes;
        } else {
            int blk = table[key >> log2_bs];
            blk = blk < 0 ? 0 : (blk > max_block ? max_block : blk);
            return ((((int64_t)blk * KH + kh) << log2_bs) + (key & ((1 << log2_bs) - 1))) * row_bytes;
        }
    }
};

template <int HSZ, bool FP8, bool PAGED, int KPB>
__device__ __forceinline__ void load_block(Staged<HSZ, FP8, KPB> &st, const KvRows<PAGED> &kv, int key0, int klast,
                                           int lane) {
    using K = KvCfg<HSZ, FP8, KPB>;
    constexpr int HALF = K::LOADS / 2;
    constexpr int EB = FP8 ? 1 : 2;  // bytes per element
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
        const int c = 64 * j + lane;
        int key = key0 + c / K::CPR;
        key = key < klast ? key : klast;
        const int64_t off = kv.row_offset(key, HSZ * EB) + K::EPC * (c % K::CPR) * EB;
        using chunk_t = typename Staged<HSZ, FP8, KPB>::chunk_t;
        st.r[j] = __builtin_nontemporal_load(reinterpret_cast<const chunk_t *>(kv.kbase + off));
        st.r[HALF + j] = __builtin_nontemporal_load(reinterpret_cast<const chunk_t *>(kv.vbase + off));
    }
}

// 8 E4M3 codes -> 8 bf16 (16 bytes), exactly: every E4M3 value is a bf16
// value, and the conversion runs with scale 1.
__device__ __forceinline__ u32x4 fp8x8_to_bf16(const u32x2 &w) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        r[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
        r[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
    }
    return r;
}

// Registers -> this wave's LDS stage as bf16, rows padded by 16 bytes
// (row-parallel 16-byte reads of the MFMA operands then hit distinct banks).
template <int HSZ, bool FP8, int KPB>
__device__ __forceinline__ void store_block(const Staged<HSZ, FP8, KPB> &st, uint16_t *stage, int lane) {
    constexpr int RS = HSZ + 8;
    using K = KvCfg<HSZ, FP8, KPB>;
    constexpr int HALF = K::LOADS / 2;
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
        const int c = 64 * j + lane;
        const int row = c / K::CPR, col = K::EPC * (c % K::CPR);
        uint16_t *kd = stage + row * RS + col;
        uint16_t *vd = stage + (KPB + row) * RS + col;
        if constexpr (FP8) {
            *reinterpret_cast<u32x4 *>(kd) = fp8x8_to_bf16(st.r[j]);
            *reinterpret_cast<u32x4 *>(vd) = fp8x8_to_bf16(st.r[HALF + j]);
        } else {
            *reinterpret_cast<u32x4 *>(kd) = st.r[j];
            *reinterpret_cast<u32x4 *>(vd) = st.r[HALF + j];
        }
    }
}

__device__ __forceinline__ bf16x8 lds_row8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// BMM1 -> online softmax -> BMM2 for one staged block of KPB keys of one wave.
// Column block cb holds MFMA columns 16 cb .. 16 cb + 15; in every lane
// (col, grp) its keys after kmax[cb] (the piece's end, or the causal limit of
// the lane's drafted token) are masked when `mask` is set (uniform: the block
// reaches past some column's limit).  Each K and V operand read from LDS
// serves all NCB column blocks.
// The running max is a lazily moved reference: it moves only when a block's
// max exceeds it by more than kLazyMax (log2 units), so the weights stay at
// most 2^kLazyMax and O and l are rescaled only on the rare blocks that move
// it.  Any reference gives the same softmax, so this is exact up to rounding.
template <int HSZ, int NCB, int KPB>
__device__ __forceinline__ void process_block(const uint16_t *stage, const bf16x8 (&qop)[NCB][HSZ / 32],
                                              int key0, const int (&kmax)[NCB], bool mask, int col, int grp,
                                              float scale_log2, float (&m_run)[NCB], float (&l_run)[NCB],
                                              f32x4 (&oacc)[NCB][HSZ / 16]) {
    using C = DecodeCfg<HSZ, NCB, false>;  // the stage layout does not depend on the cache type
    constexpr int NS = C::NS;
    constexpr int ND = C::ND;
    constexpr int KB = KPB / 16;
    const float NEG_INF = -__builtin_inff();
    const uint16_t *krow = stage + col * C::RS + 8 * grp;  // key col of 16-key row block 0
    // BMM1: S^T[key][c] for keys key0 + 16kb + 4grp + i in lane (c = 16cb + col, grp)
    f32x4 sc[NCB][KB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sc[cb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const bf16x8 a = lds_row8(krow + 16 * kb * C::RS + 32 * s);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) sc[cb][kb] = mfma_bf16(a, qop[cb][s], sc[cb][kb]);
        }
    // online softmax per column block; P enters BMM2 as its bf16 hi and lo parts
    bf16x8 phi[NCB], plo[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        float x[4 * KB];
        float mx = NEG_INF;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float xv = sc[cb][kb][i] * scale_log2;
                if (mask) xv = key0 + 16 * kb + 4 * grp + i <= kmax[cb] ? xv : NEG_INF;
                x[4 * kb + i] = xv;
                mx = fmaxf(mx, xv);
            }
        mx = wave_max_over_groups(mx);
        const bool move = mx > m_run[cb] + kLazyMax;  // always true on a column's first key
        const float m_new = move ? mx : m_run[cb];
        // -inf only while a drafted token's column has seen no key yet (its limit lies before this block)
        const float m_use = m_new == NEG_INF ? 0.f : m_new;
        if (__builtin_amdgcn_ballot_w64(move)) {  // alpha is 1 on the columns that did not move
            const float alpha = __builtin_amdgcn_exp2f(m_run[cb] - m_use);
            l_run[cb] *= alpha;
#pragma unroll
            for (int db = 0; db < ND; ++db) oacc[cb][db] *= alpha;
        }
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4 * KB; ++i) {
            const float pv = __builtin_amdgcn_exp2f(x[i] - m_use);
            ps += pv;
            const __bf16 hi = (__bf16)pv;
            phi[cb][i] = hi;
            plo[cb][i] = (__bf16)(pv - (float)hi);
        }
        l_run[cb] += ps;
        m_run[cb] = m_new;
    }
    // BMM2: the V^T operand comes straight out of the row-major V stage through
    // transposing reads.  Lane (i, grp) gets V[4 grp + j][16 db + i] (and, with
    // 32-key blocks, V[16 + 4 grp + j][16 db + i]), j = 0..3: the key order of
    // this lane's S^T accumulator, so P needs no shuffle.
    const uint16_t *vstage = stage + KPB * C::RS;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
        const i16x4 a = v_cols(vstage, C::RS, 4 * grp, 16 * db, col);
        if constexpr (KB == 2) {
            const i16x4 b = v_cols(vstage, C::RS, 16 + 4 * grp, 16 * db, col);
            const bf16x8 vt = __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                oacc[cb][db] = mfma_bf16(vt, phi[cb], oacc[cb][db]);
                oacc[cb][db] = mfma_bf16(vt, plo[cb], oacc[cb][db]);
            }
        } else {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const i16x4 ph = __builtin_bit_cast(i16x4, bf16x4{phi[cb][0], phi[cb][1], phi[cb][2], phi[cb][3]});
                const i16x4 pl = __builtin_bit_cast(i16x4, bf16x4{plo[cb][0], plo[cb][1], plo[cb][2], plo[cb][3]});
                oacc[cb][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ph, oacc[cb][db], 0, 0, 0);
                oacc[cb][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pl, oacc[cb][db], 0, 0, 0);
            }
        }
    }
}

// Partial slots and merge counters are shared between CTAs that may sit on
// different XCDs, whose L2 caches are not coherent with each other.  Every
// access to a slot goes through agent-scope atomic loads and stores (relaxed
// order): on gfx950 these carry device scope in the instruction (sc1), so a
// store is written through to the device-wide coherence point and a load
// reads from it, bypassing the XCD's L2; no L2 writeback or invalidate is
// involved.  Every writing wave waits for its slot stores to be acknowledged
// (s_waitcnt vmcnt(0), after which they are performed at that point) before
// the workgroup barrier; one thread then arrives at the head's counter with a
// device-scope atomic add, which is issued after the barrier and so after
// every acknowledged slot store of the workgroup.  The CTA that sees the last
// arrival issues its slot loads only after that atomic returned.  The order is
// therefore enforced by the instruction stream and the device-scope accesses
// themselves.  An acquire-release add (an L2 writeback before the arrival and
// an L2 invalidate after it, the HIP memory model's formal route) measured
// 3.5% slower on the Llama-3-8B-shaped batch and 11% slower on the ragged
// batch with one query head per kv head, so it is not used.
// (Whole-vector bit casts only: a bit cast of a single vector element is not
// reliable with this compiler.)
__device__ __forceinline__ void st_shared_f4(float *p, const f32x4 &v) {
    const u64x2 w = __builtin_bit_cast(u64x2, v);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), w[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p) + 1, w[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f32x4 ld_shared_f4(const float *p) {
    u64x2 w;
    w[0] = __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w[1] = __hip_atomic_load(reinterpret_cast<const uint64_t *>(p) + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_bit_cast(f32x4, w);
}

__device__ __forceinline__ void st_shared_f(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float ld_shared_f(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until every memory access this wave issued has completed.
__device__ __forceinline__ void wait_memory() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Slot of partial i of a split segment whose pieces sit in CTAs c_lo, c_lo+1, ...
__device__ __forceinline__ int partial_slot(const LeanPlan &pl, int c_lo, int64_t seg_begin, int i) {
    return i == 0 ? plan_slot(pl, c_lo, seg_begin) : 2 * (c_lo + i);
}

// Called by every thread of CTA c right after it wrote its partial of the split
// segment (b, kh) into its slot (each writing wave has waited for its stores).
// A head whose partials sit in at most kMergeFanIn CTAs is merged here: the
// CTA that arrives last at the head's counter reads every partial, rescales
// them to their common max and writes the output.  Wider heads are left to
// merge_wide_kernel, which reads their partials with many workgroups at once.
// All control flow is uniform over the CTA.
template <int HSZ, int NT, int NCMAX>
__device__ void merge_up(const DecodeParams &p, const LeanPlan &pl, const LeanPiece &pc, int *flag) {
    const int NC = p.NC, G = p.G;
    const int tid = threadIdx.x;
    const SegmentCtas sc = plan_segment_ctas(pl, pc.seg_begin, pc.seg_end);
    const int c_lo = sc.c_lo, n = sc.n;  // partials of this head
    if (n > kMergeFanIn) return;
    __syncthreads();  // every wave's slot stores have completed
    if (tid == 0) {
        int *cnt = p.counters + partial_slot(pl, c_lo, pc.seg_begin, 0);
        const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == n - 1;
        if (last) atomicExch(cnt, 0);  // counters are zero again for the next call
        *flag = last;
    }
    __syncthreads();
    if (!*flag) return;
    const int units = NC * HSZ / 4;
    auto merge_unit = [&](int u) {
        const int g = u / (HSZ / 4), d4 = u % (HSZ / 4);
        float mv[kMergeFanIn], lv[kMergeFanIn];
        f32x4 ov[kMergeFanIn];
#pragma unroll
        for (int j = 0; j < kMergeFanIn; ++j) {
            mv[j] = -__builtin_inff();
            lv[j] = 0.f;
            ov[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (j < n) {
                const float *sp = p.ws + (int64_t)partial_slot(pl, c_lo, pc.seg_begin, j) * p.slot_floats;
                mv[j] = ld_shared_f(sp + NC * HSZ + g);
                lv[j] = ld_shared_f(sp + NC * HSZ + NC + g);
                ov[j] = ld_shared_f4(sp + g * HSZ + 4 * d4);
            }
        }
        float M = mv[0];
#pragma unroll
        for (int j = 1; j < kMergeFanIn; ++j) M = fmaxf(M, mv[j]);
        // M is -inf only for a drafted token whose limit lies before every member's keys
        const float Muse = M == -__builtin_inff() ? 0.f : M;
        float L = 0.f;
        f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kMergeFanIn; ++j) {
            const float f = j < n ? __builtin_amdgcn_exp2f(mv[j] - Muse) : 0.f;
            L += lv[j] * f;
            O += ov[j] * f;
        }
        // column g: token g / G, head g % G
        const int64_t orow = ((int64_t)pc.b * p.Hq + pc.kh * G + g % G) * p.qlen + g / G;
        *reinterpret_cast<f32x4 *>(p.out + orow * HSZ + 4 * d4) = O * (p.v_scale / L);
        if (p.lse && d4 == 0) p.lse[orow] = M + __log2f(L);
    };
    // A short loop is unrolled (its loads then overlap); a long one, with 32 or
    // more columns, runs as a loop so its registers stay within the kernel's budget.
    constexpr int UNITS = NCMAX * HSZ / 4 / NT + 1;  // float4 outputs per thread, upper bound
    if constexpr (UNITS <= 3) {
#pragma unroll
        for (int r = 0; r < UNITS; ++r)
            if (tid + r * NT < units) merge_unit(tid + r * NT);
    } else {
        for (int u = tid; u < units; u += NT) merge_unit(u);
    }
}

// (M, L, O) <- the rescaled sum of two partial states of one column; an empty
// state has M = -inf and contributes nothing.
__device__ __forceinline__ void combine_state(float &M, float &L, f32x4 &O, float M2, float L2, const f32x4 &O2) {
    const float Mn = fmaxf(M, M2);
    const float f1 = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    const float f2 = M2 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M2 - Mn);
    L = L * f1 + L2 * f2;
    O = O * f1 + O2 * f2;
    M = Mn;
}

// Merge of the heads whose partials sit in more than kMergeFanIn CTAs (long
// contexts over few kv heads), launched after the tile kernel.  Workgroup
// (x, y) takes columns [16x, 16x + 16) of the NC x HSZ state of wide head y:
// thread t covers float4 column t % 4 over the partials t / 4, t / 4 + 64, ...
// (online rescaling), then the 64 threads of each column combine their states
// through lane shuffles and LDS.  The same rescaled sum as the in-kernel merge
// ("LeanAttention" digest, section "조각별로 합칠 수 있는 정확한 소프트맥스"),
// spread over many CUs instead of read by the one CTA that arrives last.
template <int HSZ>
__global__ __launch_bounds__(256) void merge_wide_kernel(const WideMergeParams mp) {
    WideHead hd;
    if (mp.count_dev) {  // list built on the device: the grid covers the most heads there can be
        if ((int)blockIdx.y >= *mp.count_dev) return;
        hd = mp.head_dev[blockIdx.y];
    } else {
        hd = mp.head[blockIdx.y];
    }
    const int b = hd.bkh & 255, kh = hd.bkh >> 8;
    const int c_lo = hd.cta & 4095, n = ((hd.cta >> 12) & 4095) + 1;
    const int slot0 = 2 * c_lo + (hd.cta >> 24);
    const int NC = mp.NC, G = mp.G;
    const int g = blockIdx.x * 16 / HSZ;
    const int col = blockIdx.x * 16 % HSZ + 4 * (threadIdx.x & 3);
    const int lane_j = threadIdx.x >> 2;
    float M = -__builtin_inff(), L = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    constexpr int R = 4;  // partials per thread per round of loads
    for (int j0 = 0; j0 < n; j0 += 64 * R) {
        float mv[R], lv[R];
        f32x4 ov[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int j = j0 + lane_j + 64 * r;
            mv[r] = -__builtin_inff();
            lv[r] = 0.f;
            ov[r] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (j < n) {
                const float *sp = mp.ws + (int64_t)(j == 0 ? slot0 : 2 * (c_lo + j)) * mp.slot_floats;
                mv[r] = ld_shared_f(sp + NC * HSZ + g);
                lv[r] = ld_shared_f(sp + NC * HSZ + NC + g);
                ov[r] = ld_shared_f4(sp + g * HSZ + col);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) combine_state(M, L, O, mv[r], lv[r], ov[r]);
    }
    // the 16 partial lanes of a column within the wave: lane bits 2..5
#pragma unroll
    for (int sh = 4; sh < 64; sh <<= 1) {
        const float M2 = __shfl_xor(M, sh), L2 = __shfl_xor(L, sh);
        f32x4 O2;
        O2[0] = __shfl_xor(O[0], sh);
        O2[1] = __shfl_xor(O[1], sh);
        O2[2] = __shfl_xor(O[2], sh);
        O2[3] = __shfl_xor(O[3], sh);
        combine_state(M, L, O, M2, L2, O2);
    }
    __shared__ float red[4][4][8];  // [wave][column][M, L, O0..3]
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane < 4) {
        float *r = red[wave][lane];
        r[0] = M;
        r[1] = L;
        r[2] = O[0];
        r[3] = O[1];
        r[4] = O[2];
        r[5] = O[3];
    }
    __syncthreads();
    if (threadIdx.x < 4) {
        const int u = threadIdx.x;
        for (int w = 1; w < 4; ++w) {
            const float *r = red[w][u];
            combine_state(M, L, O, r[0], r[1], f32x4{r[2], r[3], r[4], r[5]});
        }
        // column g: token g / G, head g % G
        const int64_t orow = ((int64_t)b * mp.Hq + kh * G + g % G) * mp.qlen + g / G;
        *reinterpret_cast<f32x4 *>(mp.out + orow * HSZ + col) = O * (mp.v_scale / L);
        if (mp.lse && col == 0) mp.lse[orow] = M + __log2f(L);
    }
}

// The LeanPlan of a call whose seqlens live in device memory, built by every
// CTA of the decode kernel into its own LDS (so the call needs no host read of
// the lengths, no extra kernel, and can be captured in a graph): L_b clamped
// into [0, stride], the tile prefix (one scan over the batch, in wave 0 with
// lane shuffles), N, and P = min(launched CTAs, N) for stream-K.  The same
// numbering as the host planner (plan.h), so the rest of the kernel cannot tell
// the two apart.  `base` carries B, KH, T, the mode, the splits and the
// launched P.  The caller's barrier publishes `lp`.
static_assert(ATTN_MAX_BATCH == 256, "the device plan scans 256 request slots");
template <int NT>
__device__ void build_plan_lds(const int32_t *seqlens, const LeanPlan &base, int64_t stride, LeanPlan &lp) {
    static_assert(NT >= 64, "one wave builds the plan");
    const int tid = threadIdx.x;
    if (tid < 64) {
        // wave 0: lane i takes requests 4i .. 4i+3, then one inclusive scan over the lanes
        const int B = base.B, KH = base.KH;
        int64_t tiles[4], own = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 4 * tid + j;
            int L = 0;
            if (b < B) {
                L = seqlens[b];
                L = L < 0 ? 0 : (L > stride ? (int)stride : L);
            }
            lp.seqlen[b] = L;
            tiles[j] = (int64_t)KH * ((L + (int64_t)base.T - 1) / base.T);
            own += tiles[j];
        }
        int64_t incl = own;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int64_t v = __shfl_up(incl, off);
            if (tid >= off) incl += v;
        }
        const int64_t N = __shfl(incl, 63);
        int64_t pre = incl - own;  // tiles before request 4i
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 4 * tid + j;
            lp.tile_prefix[b] = (int32_t)(b < B ? pre : N);
            pre += tiles[j];
        }
        if (tid == 0) {
            lp.tile_prefix[256] = (int32_t)N;
            lp.B = B;
            lp.KH = KH;
            lp.T = base.T;
            lp.N = N;
            lp.mode = base.mode;
            lp.splits = base.splits;
            lp.P = base.mode == kPlanStreamK ? (int)(N < base.P ? (N > 0 ? N : 1) : base.P) : base.P;
        }
    }
}

// The heads of a device-built plan split over more than kMergeFanIn CTAs, for
// merge_wide_kernel (which runs after the decode kernel): written by CTA 0
// once its own pieces are done.  All NT threads call it; *count gets the total.
template <int NT>
__device__ void write_wide_list(const LeanPlan &lp, int *nwide, int *count, WideHead *wide) {
    const int tid = threadIdx.x;
    if (tid == 0) *nwide = 0;
    __syncthreads();
    // A stream-K CTA owns at least floor(N/P) tiles, so a segment spread over more
    // than kMergeFanIn CTAs has more than (kMergeFanIn - 1) floor(N/P) tiles:
    // shorter ones are skipped without locating their CTAs.
    const int64_t min_wide = lp.mode == kPlanStreamK ? (int64_t)(kMergeFanIn - 1) * (lp.N / lp.P) : 0;
    for (int s = tid; s < lp.B * lp.KH; s += NT) {
        const int b = s / lp.KH, kh = s - b * lp.KH;
        const int nb = plan_tiles_per_segment(lp, b);
        if (nb == 0 || nb <= min_wide) continue;
        const int64_t s0 = lp.tile_prefix[b] + (int64_t)kh * nb;
        const SegmentCtas sc = plan_segment_ctas(lp, s0, s0 + nb);
        if (sc.n > kMergeFanIn) {
            const int i = atomicAdd(nwide, 1);  // at most kMaxWideHeads (see WideMergeParams)
            if (i < kMaxWideHeads) {
                wide[i].bkh = b | kh << 8;
                wide[i].cta = sc.c_lo | (sc.n - 1) << 12 | (plan_slot(lp, sc.c_lo, s0) & 1) << 24;
            }
        }
    }
    __syncthreads();
    if (tid == 0) *count = *nwide < kMaxWideHeads ? *nwide : kMaxWideHeads;
}

// K/V rows of the context of request b under kv head kh.
template <int HSZ, bool FP8, bool PAGED>
__device__ __forceinline__ KvRows<PAGED> piece_rows(const DecodeParams &p, const LeanPlan &pl, int b, int kh) {
    KvRows<PAGED> kv;
    if constexpr (PAGED) {
        kv.kbase = reinterpret_cast<const uint8_t *>(p.k);
        kv.vbase = reinterpret_cast<const uint8_t *>(p.v);
        kv.table = p.block_table + (int64_t)b * p.max_blocks_per_seq;
        kv.kh = kh;
        kv.KH = pl.KH;
        kv.log2_bs = p.log2_block_size;
        kv.max_block = p.num_blocks - 1;
    } else {
        const int64_t kvrow = ((int64_t)b * pl.KH + kh) * p.kv_stride;
        kv.kbase = reinterpret_cast<const uint8_t *>(p.k) + kvrow * HSZ * (FP8 ? 1 : 2);
        kv.vbase = reinterpret_cast<const uint8_t *>(p.v) + kvrow * HSZ * (FP8 ? 1 : 2);
        kv.table = nullptr;
        kv.kh = kv.KH = kv.log2_bs = kv.max_block = 0;
    }
    return kv;
}

// Piece fields are the same on every lane; reading them out of lane 0 keeps
// them in scalar registers (values loaded from LDS land in vector registers).
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint64_t u = (uint64_t)x;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ LeanPiece uniform_piece(const LeanPiece &x) {
    LeanPiece u;
    u.b = __builtin_amdgcn_readfirstlane(x.b);
    u.kh = __builtin_amdgcn_readfirstlane(x.kh);
    u.seg_begin = uniform64(x.seg_begin);
    u.seg_end = uniform64(x.seg_end);
    u.tile_begin = uniform64(x.tile_begin);
    u.tile_end = uniform64(x.tile_end);
    u.key_begin = __builtin_amdgcn_readfirstlane(x.key_begin);
    u.key_end = __builtin_amdgcn_readfirstlane(x.key_end);
    return u;
}

template <int KPB>
__device__ __forceinline__ int piece_blocks(const LeanPiece &pc) {
    return (pc.key_end - pc.key_begin + KPB - 1) / KPB;
}

template <int HSZ, bool FP8, bool PAGED, int NCB>
__global__ __launch_bounds__((DecodeCfg<HSZ, NCB, FP8>::W * 64)) void decode_tiles_kernel(const DecodeParams p) {
    using C = DecodeCfg<HSZ, NCB, FP8>;
    constexpr int NS = C::NS;
    constexpr int ND = C::ND;
    constexpr int W = C::W;
    constexpr int KPB = C::KPB;
    constexpr int NCMAX = C::NCMAX;
    constexpr int OSTRIDE = HSZ + 4;  // padded LDS row of the cross-wave reduction
    extern __shared__ __attribute__((aligned(16))) float smem[];
    // streaming phase: one K/V stage per wave; piece epilogue: the reduction buffers
    uint16_t *stages = reinterpret_cast<uint16_t *>(smem);
    float *sm_m = smem;                  // [W][NCMAX]
    float *sm_l = smem + W * NCMAX;      // [W][NCMAX]
    float *sm_o = smem + 2 * W * NCMAX;  // [W][NC][OSTRIDE]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: block indices stay scalar
    const int col = lane & 15;  // column within a 16-column block (Q, P, O), key row (K, V) or d (V^T)
    const int grp = lane >> 4;  // 8-wide slice of the MFMA contraction
    const int c = blockIdx.x;
    const int G = p.G, NC = p.NC;
    const float NEG_INF = -__builtin_inff();
    uint16_t *stage = stages + wave * C::STAGE;

    __shared__ int merge_flag;
    __shared__ int blk_next;  // next unclaimed block of the current piece
    // The plan is read many times (piece lookups, merge slots): one copy in LDS
    // costs a single round of vector loads instead of chains of dependent
    // scalar loads from the argument segment.
    __shared__ LeanPlan plan_lds;
    if (p.seqlens_dev) {  // device seqlens: the plan is built here (the stages serve as scan scratch)
        build_plan_lds<W * 64>(p.seqlens_dev, p.plan, p.kv_stride, plan_lds);
        if (threadIdx.x == 0) blk_next = W;
    } else {
        constexpr int WORDS = (int)(sizeof(LeanPlan) / sizeof(int));
        int *dst = reinterpret_cast<int *>(&plan_lds);
        const int *src = reinterpret_cast<const int *>(&p.plan);
        for (int i = threadIdx.x; i < WORDS; i += W * 64) dst[i] = src[i];
        if (threadIdx.x == 0) blk_next = W;
    }
    __syncthreads();
    const LeanPlan &pl = plan_lds;
    // a plan built on the device uses min(P, N) of the launched CTAs
    if (c >= __builtin_amdgcn_readfirstlane(pl.P)) return;

    // The first piece's first blocks are requested before any other set-up:
    // every wave's start-up instructions then run while they are in flight.
    int64_t t = plan_cta_begin(pl, c);
    const int64_t t_end = plan_cta_begin(pl, c + 1);
    Staged<HSZ, FP8, KPB> st;
    LeanPiece pc0 = {};
    if (t < t_end) {
        pc0 = uniform_piece(plan_piece_at(pl, t, t_end));
        if (wave < piece_blocks<KPB>(pc0))
            load_block<HSZ, FP8, PAGED, KPB>(st, piece_rows<HSZ, FP8, PAGED>(p, pl, pc0.b, pc0.kh),
                                             pc0.key_begin + wave * KPB, pc0.key_end - 1, lane);
    }

    // Requests with an empty context own no tiles: their output rows are zero.
    for (int b = c; b < pl.B; b += pl.P) {
        if (pl.seqlen[b] != 0) continue;
        float *orow = p.out + (int64_t)b * p.Hq * p.qlen * HSZ;
        for (int e = threadIdx.x; e < p.Hq * p.qlen * HSZ / 4; e += W * 64)
            reinterpret_cast<f32x4 *>(orow)[e] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (p.lse)
            for (int e = threadIdx.x; e < p.Hq * p.qlen; e += W * 64) p.lse[(int64_t)b * p.Hq * p.qlen + e] = -__builtin_inff();
    }

    // Column c = 16 cb + col holds query token c / G of head kh G + c % G of the
    // piece (q is [B][Hq][qlen][Hsz]); columns past NC are zero.
    bf16x8 qop[NCB][NS];
    auto load_q = [&](const LeanPiece &pq) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int cc = 16 * cb + col;
            const int ccol = cc < NC ? cc : 0;
            const uint16_t *qrow = p.q + (((int64_t)pq.b * p.Hq + pq.kh * G + ccol % G) * p.qlen + ccol / G) * HSZ;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                bf16x8 z = {};
                qop[cb][s] = cc < NC ? load_row8(qrow + 32 * s + 8 * grp) : z;
            }
        }
    };
    // At HSZ = 256 with 8 waves the next piece's queries would not fit beside the
    // epilogue's registers: there they are loaded when the piece starts.
    constexpr bool kPrefetchQ = !(HSZ == 256 && W == 8);
    bool first_piece = true;
    LeanPiece pc_next = pc0;
    while (t < t_end) {
        const LeanPiece pc = pc_next;
        const KvRows<PAGED> kv = piece_rows<HSZ, FP8, PAGED>(p, pl, pc.b, pc.kh);
        const int h0 = pc.kh * G;

        float m_run[NCB];  // running max (log2 domain) of column c
        float l_run[NCB];  // this lane's share of the running sum
        f32x4 oacc[NCB][ND];  // O[c][16*db + 4*grp + i]
        int kmax[NCB];
        const int nblk = piece_blocks<KPB>(pc);
        const int klast = pc.key_end - 1;
        if (first_piece || !kPrefetchQ) load_q(pc);  // else requested before the previous epilogue
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int cc = 16 * cb + col;
            const int ccol = cc < NC ? cc : 0;
            m_run[cb] = NEG_INF;
            l_run[cb] = 0.f;
#pragma unroll
            for (int db = 0; db < ND; ++db) oacc[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
            // drafted token t sees keys up to L_b - qlen + t
            const int climit = pl.seqlen[pc.b] - p.qlen + ccol / G;
            kmax[cb] = klast < climit ? klast : climit;
        }
        // blocks ending at or before kmin (every column's limit) need no mask
        const int climit0 = pl.seqlen[pc.b] - p.qlen;  // the limit of drafted token 0
        const int kmin = klast < climit0 ? klast : climit0;
        // Block w starts on wave w; every wave claims its next block from an
        // LDS counter when it starts computing one, so waves whose loads come
        // back sooner take more blocks and all waves of the CTA finish within
        // about one block of each other.  The claimed block is loading while
        // the current one is computed out of the wave's LDS stage; LDS traffic
        // of one wave executes in issue order, so no barrier is needed.
        int blk = wave;
        first_piece = false;
        while (blk < nblk) {
            store_block<HSZ, FP8, KPB>(st, stage, lane);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            int nxt = 0;
            if (lane == 0) nxt = atomicAdd(&blk_next, 1);
            nxt = __builtin_amdgcn_readfirstlane(nxt);
            if (nxt < nblk) load_block<HSZ, FP8, PAGED, KPB>(st, kv, pc.key_begin + nxt * KPB, klast, lane);
            __builtin_amdgcn_sched_barrier(0);
            const int key0 = pc.key_begin + blk * KPB;
            process_block<HSZ, NCB, KPB>(stage, qop, key0, kmax, key0 + KPB - 1 > kmin, col, grp, p.scale_log2, m_run,
                                         l_run, oacc);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            blk = nxt;
        }

        // The staging registers and the query operands are free now: the next
        // piece's first block and queries are requested before this piece's
        // epilogue, whose barriers and stores then hide their latency.
        if (pc.tile_end < t_end) {
            pc_next = uniform_piece(plan_piece_at(pl, pc.tile_end, t_end));
            if (wave < piece_blocks<KPB>(pc_next))
                load_block<HSZ, FP8, PAGED, KPB>(st, piece_rows<HSZ, FP8, PAGED>(p, pl, pc_next.b, pc_next.kh),
                                                 pc_next.key_begin + wave * KPB, pc_next.key_end - 1, lane);
            if constexpr (kPrefetchQ) load_q(pc_next);
        }

        // ---- merge the W wave states of this piece ----
        // Every wave parks its (m, l, O) in LDS; after one barrier each thread
        // merges one float4 column of the piece's NC x HSZ state over the W
        // waves (rescale to the common max, sum) and stores it straight to the
        // output or to the partial slot.
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) l_run[cb] = wave_sum_over_groups(l_run[cb]);
        __syncthreads();  // every wave left the streaming loop: stages and block counter are free
        if (threadIdx.x == 0) blk_next = W;  // for the next piece (later barriers publish it)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int cc = 16 * cb + col;
            if (grp == 0) {
                sm_m[wave * NCMAX + cc] = m_run[cb];
                sm_l[wave * NCMAX + cc] = l_run[cb];
            }
            if (cc < NC) {
                float *dst = sm_o + (wave * NC + cc) * OSTRIDE + 4 * grp;
#pragma unroll
                for (int db = 0; db < ND; ++db) *reinterpret_cast<f32x4 *>(dst + 16 * db) = oacc[cb][db];
            }
        }
        __syncthreads();

        const bool whole = pc.tile_begin == pc.seg_begin && pc.tile_end == pc.seg_end;
        const int64_t so = whole ? 0 : (int64_t)plan_slot(pl, c, pc.seg_begin) * p.slot_floats;
        const int units = NC * HSZ / 4;
        auto reduce_unit = [&](int u) {
            const int g = u / (HSZ / 4), d4 = u % (HSZ / 4);
            float M = NEG_INF;
#pragma unroll
            for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w * NCMAX + g]);
            float Lt = 0.f;
            f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float mw = sm_m[w * NCMAX + g];
                const float f = mw == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(mw - M);
                Lt += sm_l[w * NCMAX + g] * f;
                O += *reinterpret_cast<const f32x4 *>(sm_o + (w * NC + g) * OSTRIDE + 4 * d4) * f;
            }
            if (whole) {
                // column g: token g / G, head g % G
                const int64_t orow = ((int64_t)pc.b * p.Hq + h0 + g % G) * p.qlen + g / G;
                *reinterpret_cast<f32x4 *>(p.out + orow * HSZ + 4 * d4) = O * (p.v_scale / Lt);
                if (p.lse && d4 == 0) p.lse[orow] = M + __log2f(Lt);
            } else {
                st_shared_f4(p.ws + so + g * HSZ + 4 * d4, O);
                if (d4 == 0) {
                    st_shared_f(p.ws + so + NC * HSZ + g, M);
                    st_shared_f(p.ws + so + NC * HSZ + NC + g, Lt);
                }
            }
        };
        constexpr int UNITS = (NCMAX * HSZ / 4 + W * 64 - 1) / (W * 64);  // float4 columns per thread, at most
        if constexpr (UNITS <= 2) {
#pragma unroll
            for (int r = 0; r < UNITS; ++r)
                if ((int)threadIdx.x + r * W * 64 < units) reduce_unit(threadIdx.x + r * W * 64);
        } else {
            for (int u = threadIdx.x; u < units; u += W * 64) reduce_unit(u);
        }
        if (!whole) wait_memory();
        if (!whole) merge_up<HSZ, W * 64, NCMAX>(p, pl, pc, &merge_flag);
        t = pc.tile_end;
        if (t < t_end) __syncthreads();  // the reduction buffers are read before the next piece's stages reuse them
    }
    if (p.seqlens_dev && c == 0) {
        __syncthreads();  // the last piece's merge has read merge_flag
        write_wide_list<W * 64>(pl, &merge_flag, p.wide_count, p.wide_list);
    }
}

template <int HSZ, int NCB, bool FP8>
size_t decode_tiles_lds_bytes(int NC) {
    using C = DecodeCfg<HSZ, NCB, FP8>;
    const size_t stage = (size_t)C::W * C::STAGE * sizeof(uint16_t);
    const size_t reduce = (size_t)(2 * C::W * C::NCMAX + C::W * NC * (HSZ + 4)) * sizeof(float);
    return stage > reduce ? stage : reduce;
}

// Column blocks of 16 for NC query columns: 1, 2 or 4.
inline int column_blocks(int NC) { return NC <= 16 ? 1 : (NC <= 32 ? 2 : 4); }

// With timing events the launch goes through hipExtLaunchKernelGGL, which binds
// the events to the kernel's own start and end timestamps (no separate marker
// packets around it).
template <int HSZ, bool FP8, bool PAGED, int NCB>
hipError_t launch_tiles_t(const DecodeParams &p, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
    using C = DecodeCfg<HSZ, NCB, FP8>;
    const size_t lds = decode_tiles_lds_bytes<HSZ, NCB, FP8>(p.NC);
    static std::atomic<int> lds_set[kMaxLdsDevices];
    hipError_t e =
        ensure_lds_limit(reinterpret_cast<const void *>(decode_tiles_kernel<HSZ, FP8, PAGED, NCB>), lds_set, lds);
    if (e != hipSuccess) return e;
    if (ev_begin || ev_end)
        hipExtLaunchKernelGGL((decode_tiles_kernel<HSZ, FP8, PAGED, NCB>), dim3(p.plan.P), dim3(C::W * 64),
                              (uint32_t)lds, stream, ev_begin, ev_end, 0u, p);
    else
        hipLaunchKernelGGL((decode_tiles_kernel<HSZ, FP8, PAGED, NCB>), dim3(p.plan.P), dim3(C::W * 64), lds, stream,
                           p);
    return hipGetLastError();
}

template <int HSZ, int NCB>
hipError_t launch_tiles_n(const DecodeParams &p, bool fp8, hipStream_t stream, hipEvent_t ev_begin,
                          hipEvent_t ev_end) {
    const bool paged = p.block_table != nullptr;
    if (fp8)
        return paged ? launch_tiles_t<HSZ, true, true, NCB>(p, stream, ev_begin, ev_end)
                     : launch_tiles_t<HSZ, true, false, NCB>(p, stream, ev_begin, ev_end);
    return paged ? launch_tiles_t<HSZ, false, true, NCB>(p, stream, ev_begin, ev_end)
                 : launch_tiles_t<HSZ, false, false, NCB>(p, stream, ev_begin, ev_end);
}

template <int HSZ>
hipError_t launch_tiles_h(const DecodeParams &p, bool fp8, hipStream_t stream, hipEvent_t ev_begin,
                          hipEvent_t ev_end) {
    switch (column_blocks(p.NC)) {
        case 1: return launch_tiles_n<HSZ, 1>(p, fp8, stream, ev_begin, ev_end);
        case 2: return launch_tiles_n<HSZ, 2>(p, fp8, stream, ev_begin, ev_end);
        default:
            if constexpr (HSZ * 64 <= kMaxColumnElems) return launch_tiles_n<HSZ, 4>(p, fp8, stream, ev_begin, ev_end);
            return hipErrorInvalidValue;
    }
}

template <int HSZ>
hipError_t launch_merge_wide_h(const WideMergeParams &mp, hipStream_t stream, hipEvent_t ev_end) {
    if (ev_end)
        hipExtLaunchKernelGGL(merge_wide_kernel<HSZ>, dim3(mp.NC * HSZ / 16, mp.count), dim3(256), 0u, stream,
                              nullptr, ev_end, 0u, mp);
    else
        hipLaunchKernelGGL(merge_wide_kernel<HSZ>, dim3(mp.NC * HSZ / 16, mp.count), dim3(256), 0, stream, mp);
    return hipGetLastError();
}

template <int HSZ, int NCB>
int occupancy_t(int NC) {
    using C = DecodeCfg<HSZ, NCB, false>;
    int blocks = 0;
    const size_t lds = decode_tiles_lds_bytes<HSZ, NCB, false>(NC);
    const void *fn = reinterpret_cast<const void *>(decode_tiles_kernel<HSZ, false, false, NCB>);
    if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_tiles_kernel<HSZ, false, false, NCB>, C::W * 64,
                                                     lds) != hipSuccess)
        return 1;
    return blocks > 0 ? blocks : 1;
}

template <int HSZ>
int occupancy_h(int NC) {
    switch (column_blocks(NC)) {
        case 1: return occupancy_t<HSZ, 1>(NC);
        case 2: return occupancy_t<HSZ, 2>(NC);
        default:
            if constexpr (HSZ * 64 <= kMaxColumnElems) return occupancy_t<HSZ, 4>(NC);
            return 1;
    }
}

// Default LeanTile: every wave's first round of blocks.
template <class C>
constexpr int tile_keys_of() { return C::W * C::KPB; }

template <int HSZ>
int tile_keys_h(int NC) {
    switch (column_blocks(NC)) {
        case 1: return tile_keys_of<DecodeCfg<HSZ, 1, false>>();
        case 2: return tile_keys_of<DecodeCfg<HSZ, 2, false>>();
        default: return tile_keys_of<DecodeCfg<HSZ, 4, false>>();
    }
}

}  // namespace

// Raises a kernel's dynamic-LDS limit (default 64 KiB; gfx950 has 160 KiB per
// CU) to the largest size any call asks for, once per device and size, so
// that launches captured into a graph make no attribute calls.  `done` holds
// one entry per device (kMaxLdsDevices); the attribute call may run twice when
// two threads race on a new size, which is harmless.
hipError_t ensure_lds_limit(const void *fn, std::atomic<int> *done, size_t lds) {
    if (lds <= 65536) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::atomic<int> &d = done[dev < kMaxLdsDevices ? dev : kMaxLdsDevices - 1];
    if (d.load(std::memory_order_acquire) >= (int)lds && dev < kMaxLdsDevices) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int cur = d.load(std::memory_order_relaxed);
    while (cur < (int)lds && !d.compare_exchange_weak(cur, (int)lds)) {
    }
    return hipSuccess;
}

int decode_tile_keys(int Hsz, int NC) {
    switch (Hsz) {
        case 64: return tile_keys_h<64>(NC);
        case 128: return tile_keys_h<128>(NC);
        default: return tile_keys_h<256>(NC);
    }
}

hipError_t launch_decode_tiles(const DecodeParams &p, int Hsz, bool fp8, hipStream_t stream, hipEvent_t ev_begin,
                               hipEvent_t ev_end) {
    switch (Hsz) {
        case 64: return launch_tiles_h<64>(p, fp8, stream, ev_begin, ev_end);
        case 128: return launch_tiles_h<128>(p, fp8, stream, ev_begin, ev_end);
        case 256: return launch_tiles_h<256>(p, fp8, stream, ev_begin, ev_end);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_merge_wide(const WideMergeParams &mp, int Hsz, hipStream_t stream, hipEvent_t ev_end) {
    switch (Hsz) {
        case 64: return launch_merge_wide_h<64>(mp, stream, ev_end);
        case 128: return launch_merge_wide_h<128>(mp, stream, ev_end);
        case 256: return launch_merge_wide_h<256>(mp, stream, ev_end);
        default: return hipErrorInvalidValue;
    }
}

// Merge of S decode outputs over disjoint key ranges of the same rows (KV
// split across devices or calls): each shard's normalised row O_s comes with
// lse_s = log2 of its softmax denominator, so the whole row is
// sum_s O_s 2^(lse_s - M) / sum_s 2^(lse_s - M) with M = max_s lse_s, the same
// associative rescale as the merge of partial states ("LeanAttention" digest,
// section "조각별로 합칠 수 있는 정확한 소프트맥스").  Thread per float4 of a
// row; a shard with lse = -inf (no keys) contributes nothing.
__global__ __launch_bounds__(256) void merge_shards_kernel(const float *outs, const float *lses, int S, int64_t rows,
                                                           int Hsz, float *out, float *lse_out) {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int per_row = Hsz / 4;
    if (u >= rows * per_row) return;
    const int64_t r = u / per_row;
    const int d4 = (int)(u - r * per_row);
    float M = -__builtin_inff();
    for (int sh = 0; sh < S; ++sh) M = fmaxf(M, lses[sh * rows + r]);
    float L = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    if (M != -__builtin_inff()) {
        for (int sh = 0; sh < S; ++sh) {
            const float ls = lses[sh * rows + r];
            if (ls == -__builtin_inff()) continue;
            const float w = __builtin_amdgcn_exp2f(ls - M);
            L += w;
            O += *reinterpret_cast<const f32x4 *>(outs + (sh * rows + r) * Hsz + 4 * d4) * w;
        }
        O *= 1.f / L;
    }
    *reinterpret_cast<f32x4 *>(out + r * Hsz + 4 * d4) = O;
    if (lse_out && d4 == 0) lse_out[r] = M == -__builtin_inff() ? M : M + __log2f(L);
}

// Zero-fills `bytes` (a multiple of 4) with plain vector stores; used for the
// arrival counters of a freshly allocated workspace.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

hipError_t launch_zero_fill(void *ptr, size_t bytes, hipStream_t stream) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<uint32_t *>(ptr), n);
    return hipGetLastError();
}

hipError_t launch_merge_shards(const float *outs, const float *lses, int S, int64_t rows, int Hsz, float *out,
                               float *lse_out, hipStream_t stream) {
    const int64_t n = rows * (Hsz / 4);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(merge_shards_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, outs, lses, S, rows,
                       Hsz, out, lse_out);
    return hipGetLastError();
}

int decode_tiles_occupancy(int Hsz, int NC) {
    switch (Hsz) {
        case 64: return occupancy_h<64>(NC);
        case 128: return occupancy_h<128>(NC);
        default: return occupancy_h<256>(NC);
    }
}

}  // namespace attn
