// prefill.hip -- causal GQA prefill on gfx950 MFMA (QK^T in bf16, PV in fp16).
//
// Source: co-design page "장문 컨텍스트 추론을 위한 어텐션 공동 설계", sections
// "프리필과 디코드의 차이" (prefill has GEMM-M = ISL x G and is compute bound)
// and "FlashAttention과 GEMM 모양" (BMM1 -> online softmax -> BMM2 over
// streamed K/V tiles, no materialised score matrix); "LeanAttention" digest,
// section "모양이 다른 프리필과 디코드" (parallelism over the query length).
// Causal, top-left aligned: query row i sees keys 0..i.
//
// gfx950 mapping.  A workgroup of 8 wave64s owns 256 query rows of one query
// head (32 rows per wave) and walks the K/V blocks of 64 keys up to the
// diagonal; it fills a CU (two waves per SIMD, up to 256 VGPRs per lane, 74 KiB
// of LDS), so one wave's softmax overlaps its sibling's matrix products, and
// each staged K/V block serves eight waves (half the staging per product of
// two 4-wave workgroups).  Waves whose rows end before a block skip it.
//  * Staging: each block's K (bf16) and V (converted to fp16, exact inside
//    fp16's normal range) go through registers into one of two LDS stages
//    while the other stage is being computed: one barrier per block.  K rows
//    are padded to 272 bytes (row-parallel 16-byte operand reads hit distinct
//    banks), V rows to 320 bytes (the transposed reads below hit distinct banks).
//  * BMM1 in the transposed form S^T = K Q^T on v_mfma_f32_32x32x16_bf16: a
//    query row sits on lane (l % 32), so the row max and sum need one exchange
//    with lane l ^ 32; Q^T stays in registers for the whole key loop.
//  * Online softmax in the log2 domain with a lazily moved reference max: it
//    moves only when a block's max exceeds it by more than 2^8, so P <= 256
//    stays inside fp16 and the O/l rescale runs only on the rare blocks that
//    move it.  P is rounded to fp16 (2^-11 relative) and the running sum adds
//    the rounded values (v_dot2_f32_f16), so the weights stay normalised exactly.
//  * BMM2 as O^T = V^T P^T on v_mfma_f32_32x32x16_f16.  V^T comes straight
//    from the row-major V stage through ds_read_b64_tr_b16 (each read hands a
//    lane four consecutive keys of one d), and the key order inside every
//    16-key contraction is chosen so that the lanes holding S^T already hold
//    the P^T operand: no shuffles and no transposed staging.
//  * Order: each XCD takes the work of whole kv heads (their K/V then stays in
//    its L2), and inside it the query blocks go longest first.
#include "common.h"

namespace attn {
namespace {

constexpr int PF_BN = 64;   // keys per K/V block
constexpr int PF_NKT = PF_BN / 32;  // 32-key tiles of BMM1 per block
constexpr int PF_NCH = PF_BN / 16;  // 16-key contractions of BMM2 per block
// Sizes that follow the head dimension (64, 128 or 256).  The row pitches keep
// the operand reads conflict-free: K rows of 16 B more than a row (row-parallel
// 16-byte reads), V rows of 64 B more (the transposed reads of four rows).  At
// 256 a wave's Q^T and O^T alone take 192 registers per lane, so the workgroup
// is 4 waves with one wave per SIMD (512 registers each, AGPRs included) and
// owns 128 query rows; otherwise 8 waves, two per SIMD, own 256 rows.
template <int HSZ>
struct PfDims {
    static constexpr int WAVES = HSZ == 256 ? 4 : 8;
    static constexpr int WPE = HSZ == 256 ? 1 : 2;    // waves per SIMD
    static constexpr int NT = WAVES * 64;
    static constexpr int BM = 32 * WAVES;             // query rows per workgroup
    static constexpr int KP = HSZ + 8;               // K stage row pitch (bf16 elements): 144 or 272 B
    static constexpr int VP = HSZ + 32;              // V stage row pitch (fp16 elements): 192 or 320 B
    static constexpr int KSTAGE = PF_BN * KP;        // elements
    static constexpr int VSTAGE = PF_BN * VP;
    static constexpr int STAGE = KSTAGE + VSTAGE;
    static constexpr int CH = HSZ / 8;               // 16-byte chunks per row
    static constexpr int LOADS = PF_BN * CH / NT;    // 16-byte chunks per thread per block (K, and again V)
    static_assert(PF_BN * CH % NT == 0, "a block's chunks split evenly over the threads");
};
constexpr int PF_XCDS = 8;
constexpr float kLazy = 8.f;  // lazy-rescale threshold in log2 units (weights <= 256)

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x16 mfma_qk(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_pv(const f16x8 &a, const f16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 8 bf16 (one 16-byte chunk) -> 8 fp16, exact for |v| in fp16's normal range.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(const u32x4 &w) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = w[i];
        const f16x2 h = {(_Float16)__builtin_bit_cast(float, x << 16), (_Float16)__builtin_bit_cast(float, x & 0xffff0000u)};
        r[i] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
}

// Four consecutive keys of one d column of the row-major fp16 V stage.  Within
// each 16-lane block, lane t reads 8 bytes at row key0 + t/4, columns
// d0 + 4 (t % 4) .. +3; the transposing read then hands lane i the column
// d0 + i at rows key0 .. key0+3.
template <int VP>
__device__ __forceinline__ i16x4 v_cols(const uint16_t *vstage, int key0, int d0, int t) {
    const uint16_t *p = vstage + (key0 + (t >> 2)) * VP + d0 + 4 * (t & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)((__attribute__((address_space(3))) uint16_t *)p));
}

template <int HSZ>
__global__ __launch_bounds__(PfDims<HSZ>::NT) __attribute__((amdgpu_waves_per_eu(PfDims<HSZ>::WPE)))
void prefill_causal_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    uint16_t *__restrict__ out, int B, int ISL, int Hq, int KH, float scale_log2, int nqb) {
    using D = PfDims<HSZ>;
    constexpr int PF_HSZ = HSZ;
    constexpr int PF_KP = D::KP, PF_VP = D::VP, PF_KSTAGE = D::KSTAGE, PF_STAGE = D::STAGE;
    constexpr int PF_CH = D::CH, PF_LOADS = D::LOADS;
    constexpr int PF_NT = D::NT, PF_BM = D::BM;
    extern __shared__ __attribute__((aligned(16))) uint16_t pf_smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: row-block tests stay scalar
    const int l32 = lane & 31, h = lane >> 5;  // query column of the 32x32 tiles, lane half
    const int G = Hq / KH;

    // ---- work item: XCD-aware when the (b, kv head) pairs split evenly over the XCDs ----
    const int x = blockIdx.x;
    const int npair = B * KH;
    int pair, g, qb;
    if (npair % PF_XCDS == 0) {
        const int xcd = x % PF_XCDS, rank = x / PF_XCDS, per = npair / PF_XCDS;
        g = rank % G;
        const int rest = rank / G;
        pair = (rest % per) * PF_XCDS + xcd;
        qb = nqb - 1 - rest / per;
    } else {
        g = x % G;
        const int rest = x / G;
        pair = rest % npair;
        qb = nqb - 1 - rest / npair;
    }
    const int b = pair / KH, kh = pair % KH;
    const int hq = kh * G + g;

    const int64_t bh = (int64_t)b * Hq + hq;
    const uint16_t *qh = q + bh * ISL * PF_HSZ;
    const uint16_t *kbase = k + ((int64_t)b * KH + kh) * ISL * PF_HSZ;
    const uint16_t *vbase = v + ((int64_t)b * KH + kh) * ISL * PF_HSZ;
    const int q0 = qb * PF_BM + 32 * wave;  // first query row of this wave
    const float NEG_INF = -__builtin_inff();

    // Q^T operands: lane holds query q0 + l32, d = 16s + 8h .. +7.
    bf16x8 qop[PF_HSZ / 16];
    {
        int row = q0 + l32;
        row = row < ISL ? row : ISL - 1;
#pragma unroll
        for (int s = 0; s < PF_HSZ / 16; ++s)
            qop[s] = *reinterpret_cast<const bf16x8 *>(qh + (int64_t)row * PF_HSZ + 16 * s + 8 * h);
    }

    f32x16 oacc[PF_HSZ / 32];  // O^T[d = 32dt + 8(r/4) + 4h + r%4][query l32]
#pragma unroll
    for (int dt = 0; dt < PF_HSZ / 32; ++dt) oacc[dt] = f32x16{};
    float m_run = NEG_INF, l_run = 0.f;

    int last_key = qb * PF_BM + PF_BM - 1;
    last_key = last_key < ISL - 1 ? last_key : ISL - 1;
    const int nkv = last_key / PF_BN + 1;

    u32x4 kst[PF_LOADS], vst[PF_LOADS];
    // Chunk r of a block is the 16-byte word r * PF_NT + tid of its row-major
    // keys x Hsz slab: a whole block is contiguous, so only the last block of a
    // ragged ISL needs its rows clamped.
    auto load_block = [&](int kvb) {
        if (kvb * PF_BN + PF_BN <= ISL) {
            const uint16_t *kb = kbase + (int64_t)kvb * PF_BN * PF_HSZ + 8 * tid;
            const uint16_t *vb = vbase + (int64_t)kvb * PF_BN * PF_HSZ + 8 * tid;
#pragma unroll
            for (int r = 0; r < PF_LOADS; ++r) {
                kst[r] = *reinterpret_cast<const u32x4 *>(kb + r * PF_NT * 8);
                vst[r] = *reinterpret_cast<const u32x4 *>(vb + r * PF_NT * 8);
            }
        } else {
#pragma unroll
            for (int r = 0; r < PF_LOADS; ++r) {
                const int idx = r * PF_NT + tid;
                int key = kvb * PF_BN + idx / PF_CH;
                key = key < ISL ? key : ISL - 1;
                const int64_t off = (int64_t)key * PF_HSZ + 8 * (idx % PF_CH);
                kst[r] = *reinterpret_cast<const u32x4 *>(kbase + off);
                vst[r] = *reinterpret_cast<const u32x4 *>(vbase + off);
            }
        }
    };
    auto store_block = [&](int stage) {
        uint16_t *ks = pf_smem + stage * PF_STAGE;
        uint16_t *vs = ks + PF_KSTAGE;
#pragma unroll
        for (int r = 0; r < PF_LOADS; ++r) {
            const int idx = r * PF_NT + tid;
            const int row = idx / PF_CH, ch = idx % PF_CH;
            *reinterpret_cast<u32x4 *>(ks + row * PF_KP + 8 * ch) = kst[r];
            *reinterpret_cast<u32x4 *>(vs + row * PF_VP + 8 * ch) = bf16x8_to_f16x8(vst[r]);
        }
    };

    load_block(0);
    store_block(0);
    __syncthreads();
    for (int kvb = 0; kvb < nkv; ++kvb) {
        const int stage = kvb & 1;
        if (kvb + 1 < nkv) load_block(kvb + 1);
        const int key_base = kvb * PF_BN;
        if (key_base <= q0 + 31) {  // some key of the block is visible to some row of this wave
            const uint16_t *ks = pf_smem + stage * PF_STAGE;
            const uint16_t *vs = ks + PF_KSTAGE;
            // ---- BMM1: S^T[key = 32kt + 8(r/4) + 4h + r%4][query l32] ----
            // The key tiles' chains alternate, and the K operand reads run four
            // ahead of the products that use them, so LDS latency overlaps the MFMAs
            // instead of sitting between every pair of them.
            f32x16 sc[PF_NKT];
#pragma unroll
            for (int kt = 0; kt < PF_NKT; ++kt) sc[kt] = f32x16{};
            bf16x8 kop[PF_HSZ / 16][PF_NKT];
#pragma unroll
            for (int s = 0; s < PF_HSZ / 16; ++s)
#pragma unroll
                for (int kt = 0; kt < PF_NKT; ++kt)
                    kop[s][kt] = *reinterpret_cast<const bf16x8 *>(ks + (32 * kt + l32) * PF_KP + 8 * h + 16 * s);
#pragma unroll
            for (int s = 0; s < PF_HSZ / 16; ++s)
#pragma unroll
                for (int kt = 0; kt < PF_NKT; ++kt) sc[kt] = mfma_qk(kop[s][kt], qop[s], sc[kt]);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS reads
#pragma unroll
            for (int i = 0; i < PF_NKT * (PF_HSZ / 16) - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            // ---- online softmax (log2 domain, lazy rescale) ----
            // Only the blocks that reach past the wave's first row need the causal
            // mask; the test is uniform over the wave, so the others skip it.
            if (key_base + PF_BN - 1 > q0) {
                const int lim = q0 + l32 - key_base - 4 * h;  // key offset limit of this lane's row
#pragma unroll
                for (int kt = 0; kt < PF_NKT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (32 * kt + 8 * (r >> 2) + (r & 3) > lim) sc[kt][r] = NEG_INF;
            }
            float mx = NEG_INF;  // max raw score of this query over the block
#pragma unroll
            for (int kt = 0; kt < PF_NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kt][r]);
            mx = pair_max32(mx) * scale_log2;
            // The reference max moves only when the block max exceeds it by more
            // than kLazy (log2 units): the weights then stay <= 2^kLazy, far inside
            // fp16, and O and l are rescaled only on the rare blocks that move it.
            // Any reference value gives the same softmax, so this is exact up to rounding.
            const bool move = mx > m_run + kLazy;  // always true on the first block (m_run = -inf)
            const float m_new = move ? mx : m_run;
            if (__builtin_amdgcn_ballot_w64(move)) {
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < PF_HSZ / 32; ++dt) oacc[dt] *= alpha;
            }
            m_run = m_new;
            // ---- P and BMM2, one 16-key chunk at a time: O^T += V^T P^T, contraction
            //      slot 8h + e of chunk c is key 16c + 4h + e (e < 4) or 16c + 8 + 4h +
            //      (e - 4) (e >= 4).  The chunk's four MFMAs run while the next chunk's
            //      exponentials issue. ----
            const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
            const int t = lane & 15;
#pragma unroll
            for (int c = 0; c < PF_NCH; ++c) {
                f16x8 pb;  // P^T operand of chunk c
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pb[e] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[c >> 1][8 * (c & 1) + e], scale_log2, -m_new));
                // the running sum adds the fp16-rounded weights the product uses
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const f16x2 pair = {pb[e], pb[e + 1]};
                    l_run = __builtin_amdgcn_fdot2(pair, ones, l_run, false);
                }
#pragma unroll
                for (int dt = 0; dt < PF_HSZ / 32; ++dt) {
                    const int d0 = 32 * dt + 16 * ((lane >> 4) & 1);
                    const i16x4 lo = v_cols<PF_VP>(vs, 16 * c + 4 * h, d0, t);
                    const i16x4 hi = v_cols<PF_VP>(vs, 16 * c + 8 + 4 * h, d0, t);
                    const f16x8 a = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[dt] = mfma_pv(a, pb, oacc[dt]);
                }
            }
        }
        if (kvb + 1 < nkv) store_block(stage ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l, rounded to bf16 once ----
    const float lt = pair_sum32(l_run);
    const int row = q0 + l32;
    if (row < ISL) {
        const float inv = 1.f / lt;
        uint16_t *orow = out + (bh * ISL + row) * PF_HSZ;
#pragma unroll
        for (int dt = 0; dt < PF_HSZ / 32; ++dt)
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) {
                bf16x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = (__bf16)(oacc[dt][4 * m4 + i] * inv);
                *reinterpret_cast<bf16x4 *>(orow + 32 * dt + 8 * m4 + 4 * h) = o;
            }
    }
}

}  // namespace

namespace {

template <int HSZ>
hipError_t launch_prefill_h(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *out, int B, int ISL,
                            int Hq, int KH, float scale_log2, hipStream_t stream) {
    const int nqb = (ISL + PfDims<HSZ>::BM - 1) / PfDims<HSZ>::BM;
    const int64_t nblocks = (int64_t)nqb * B * Hq;
    if (nblocks > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = (size_t)2 * PfDims<HSZ>::STAGE * sizeof(uint16_t);
    static std::atomic<int> lds_set[kMaxLdsDevices];  // per device: above the 64 KiB default
    const hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(prefill_causal_kernel<HSZ>), lds_set, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_causal_kernel<HSZ>, dim3((unsigned)nblocks), dim3(PfDims<HSZ>::NT), lds, stream, q, k, v, out, B,
                       ISL, Hq, KH, scale_log2, nqb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_causal(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *out,
                                 int B, int ISL, int Hq, int KH, int Hsz, float scale_log2,
                                 hipStream_t stream) {
    switch (Hsz) {
        case 64: return launch_prefill_h<64>(q, k, v, out, B, ISL, Hq, KH, scale_log2, stream);
        case 128: return launch_prefill_h<128>(q, k, v, out, B, ISL, Hq, KH, scale_log2, stream);
        case 256: return launch_prefill_h<256>(q, k, v, out, B, ISL, Hq, KH, scale_log2, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
