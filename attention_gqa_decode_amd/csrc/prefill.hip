// prefill.hip -- causal GQA prefill on gfx950 MFMA (QK^T in bf16, PV in fp16).
//
// Source: co-design page "장문 컨텍스트 추론을 위한 어텐션 공동 설계", sections
// "프리필과 디코드의 차이" (prefill has GEMM-M = ISL x G and is compute bound)
// and "FlashAttention과 GEMM 모양" (BMM1 -> online softmax -> BMM2 over
// streamed K/V tiles, no materialised score matrix); "LeanAttention" digest,
// section "모양이 다른 프리필과 디코드" (parallelism over the query length).
// Causal, top-left aligned: query row i sees keys 0..i.
//
// gfx950 mapping.  A workgroup of 4 wave64s owns 128 query rows of one query
// head (32 rows per wave) and walks the K/V blocks of 64 keys up to the
// diagonal.  K is staged row-major in LDS; V is staged transposed (V^T[d][key],
// written as packed key pairs) so that the PV product can read its MFMA
// operand with two 8-byte LDS reads.  Both products run on
// v_mfma_f32_16x16x32_bf16 in the transposed form S^T = K Q^T and
// O^T = V^T P^T: the query row sits on the lane index, so the row max and row
// sum need only two cross-lane steps, and the lanes holding S^T already hold
// the P^T operand (same key order trick as the decode kernel).  The second
// product runs in fp16 (v_mfma_f32_16x16x32_f16): V is converted bf16 -> fp16
// while it is staged (exact inside fp16's range, |v| < 65504) and P in [0, 1]
// is rounded to fp16 (2^-11 relative, four times finer than bf16, whose 2^-9
// weight error alone breaks a 2e-3 bound on rows with few keys).  The running
// sum l accumulates the same rounded P, so rounding perturbs the weights but
// not their normalisation.  Blocks are issued longest-first (late query
// blocks see the most keys).
#include "common.h"

namespace attn {
namespace {

constexpr int PF_BM = 128;   // query rows per workgroup
constexpr int PF_BN = 64;    // keys per K/V block
constexpr int PF_WAVES = 4;  // 32 query rows per wave

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_pf(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_pv(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
    const f16x2 h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float max_over_groups(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float sum_over_groups(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

template <int HSZ>
__global__ __launch_bounds__(PF_WAVES * 64) void prefill_causal_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    uint16_t *__restrict__ out, int B, int ISL, int Hq, int KH, float scale_log2, int nqb) {
    constexpr int NS = HSZ / 32;
    constexpr int ND = HSZ / 16;
    constexpr int KSTR = HSZ + 8;    // bf16 per K row in LDS (16-byte aligned rows)
    constexpr int VSTR = PF_BN + 4;  // bf16 per V^T row in LDS (8-byte aligned rows)
    constexpr int KCH = HSZ / 8;     // 16-byte chunks per row
    constexpr int NT = PF_WAVES * 64;
    constexpr int KLOADS = PF_BN * KCH / NT;        // K chunks per thread per block
    constexpr int VLOADS = (PF_BN / 2) * KCH / NT;  // V key-pair chunks per thread per block
    __shared__ __attribute__((aligned(16))) uint16_t sk[PF_BN * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t svt[HSZ * VSTR];  // fp16 V^T

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int nbh = B * Hq;
    const int qb = nqb - 1 - (int)(blockIdx.x / nbh);  // longest first
    const int bh = (int)(blockIdx.x % nbh);
    const int b = bh / Hq, h = bh % Hq;
    const int kh = h / (Hq / KH);
    const float NEG_INF = -__builtin_inff();

    const int row0 = qb * PF_BM + 32 * wave;
    const uint16_t *qh = q + (int64_t)bh * ISL * HSZ;
    const uint16_t *kbase = k + ((int64_t)b * KH + kh) * ISL * HSZ;
    const uint16_t *vbase = v + ((int64_t)b * KH + kh) * ISL * HSZ;

    bf16x8 qop[2][NS];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        int row = row0 + 16 * rb + col;
        row = row < ISL ? row : ISL - 1;
#pragma unroll
        for (int s = 0; s < NS; ++s)
            qop[rb][s] = *reinterpret_cast<const bf16x8 *>(qh + (int64_t)row * HSZ + 32 * s + 8 * grp);
    }

    float m[2] = {NEG_INF, NEG_INF};
    float l[2] = {0.f, 0.f};
    f32x4 oacc[2][ND];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

    int last_key = qb * PF_BM + PF_BM - 1;
    last_key = last_key < ISL - 1 ? last_key : ISL - 1;
    const int nkv = last_key / PF_BN + 1;

    u32x4 kst[KLOADS], vst[VLOADS][2];
    auto load_block = [&](int kvb) {
        const int kb0 = kvb * PF_BN;
#pragma unroll
        for (int r = 0; r < KLOADS; ++r) {
            const int idx = r * NT + tid;
            int key = kb0 + idx / KCH;
            key = key < ISL ? key : ISL - 1;
            kst[r] = *reinterpret_cast<const u32x4 *>(kbase + (int64_t)key * HSZ + 8 * (idx % KCH));
        }
#pragma unroll
        for (int r = 0; r < VLOADS; ++r) {
            const int idx = r * NT + tid;
            const int pr = idx / KCH, ch = idx % KCH;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                int key = kb0 + 2 * pr + e;
                key = key < ISL ? key : ISL - 1;
                vst[r][e] = *reinterpret_cast<const u32x4 *>(vbase + (int64_t)key * HSZ + 8 * ch);
            }
        }
    };
    auto store_block = [&]() {
#pragma unroll
        for (int r = 0; r < KLOADS; ++r) {
            const int idx = r * NT + tid;
            *reinterpret_cast<u32x4 *>(sk + (idx / KCH) * KSTR + 8 * (idx % KCH)) = kst[r];
        }
#pragma unroll
        for (int r = 0; r < VLOADS; ++r) {
            const int idx = r * NT + tid;
            const int pr = idx / KCH, ch = idx % KCH;
            uint32_t *dst = reinterpret_cast<uint32_t *>(svt) + ((8 * ch) * VSTR + 2 * pr) / 2;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t a = vst[r][0][w], c = vst[r][1][w];
                // d = 8ch + 2w (low halves) and 8ch + 2w + 1 (high halves); keys 2pr, 2pr+1.
                // bf16 -> fp32 is exact; fp32 -> fp16 is exact for |v| in fp16's normal range.
                dst[(2 * w) * VSTR / 2] = pack_f16(bf16_lo(a), bf16_lo(c));
                dst[(2 * w + 1) * VSTR / 2] = pack_f16(bf16_hi(a), bf16_hi(c));
            }
        }
    };

    load_block(0);
    for (int kvb = 0; kvb < nkv; ++kvb) {
        __syncthreads();
        store_block();
        __syncthreads();
        if (kvb + 1 < nkv) load_block(kvb + 1);
        const int key_base = kvb * PF_BN;
        if (key_base > row0 + 31) continue;  // block entirely above this wave's diagonal

        f32x4 sc[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) sc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sk + (16 * kb + col) * KSTR + 32 * s + 8 * grp);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) sc[kb][rb] = mfma_pf(a, qop[rb][s], sc[kb][rb]);
            }

        const bool diag = key_base + PF_BN - 1 > row0;  // some key of the block lies past some row
        f16x8 pb[2][2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int row = row0 + 16 * rb + col;
            float x[16];
            float mx = NEG_INF;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = key_base + 16 * kb + 4 * grp + i;
                    float xv = sc[kb][rb][i] * scale_log2;
                    if (diag && key > row) xv = NEG_INF;
                    x[4 * kb + i] = xv;
                    mx = fmaxf(mx, xv);
                }
            mx = max_over_groups(mx);
            const float m_new = fmaxf(m[rb], mx);
            const float m_use = m_new == NEG_INF ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m[rb] - m_use);
            float ps = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const _Float16 pr = (_Float16)__builtin_amdgcn_exp2f(x[j] - m_use);
                ps += (float)pr;
                // k-slot order inside a 32-key chunk kc: slots 0-3 <- 16-key block 2kc, 4-7 <- 2kc+1
                const int kb = j >> 2, i = j & 3;
                pb[rb][kb >> 1][4 * (kb & 1) + i] = pr;
            }
            l[rb] = l[rb] * alpha + ps;
            m[rb] = m_new;
#pragma unroll
            for (int db = 0; db < ND; ++db) oacc[rb][db] *= alpha;
        }

#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                const uint16_t *vrow = svt + (16 * db + col) * VSTR + 32 * kc + 4 * grp;
                const f16x4 lo = *reinterpret_cast<const f16x4 *>(vrow);
                const f16x4 hi = *reinterpret_cast<const f16x4 *>(vrow + 16);
                const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) oacc[rb][db] = mfma_pv(a, pb[rb][kc], oacc[rb][db]);
            }
    }

#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float lt = sum_over_groups(l[rb]);
        const int row = row0 + 16 * rb + col;
        if (row >= ISL) continue;
        const float inv = 1.f / lt;
        uint16_t *orow = out + ((int64_t)bh * ISL + row) * HSZ + 4 * grp;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            bf16x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (__bf16)(oacc[rb][db][i] * inv);
            *reinterpret_cast<bf16x4 *>(orow + 16 * db) = o;
        }
    }
}

}  // namespace

hipError_t launch_prefill_causal(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *out,
                                 int B, int ISL, int Hq, int KH, int Hsz, float scale_log2,
                                 hipStream_t stream) {
    if (Hsz != 128) return hipErrorInvalidValue;
    const int nqb = (ISL + PF_BM - 1) / PF_BM;
    const int64_t nblocks = (int64_t)nqb * B * Hq;
    if (nblocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prefill_causal_kernel<128>, dim3((unsigned)nblocks), dim3(PF_WAVES * 64), 0, stream,
                       q, k, v, out, B, ISL, Hq, KH, scale_log2, nqb);
    return hipGetLastError();
}

}  // namespace attn
