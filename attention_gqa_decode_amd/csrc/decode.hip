// decode.hip -- GQA decode on gfx950: LeanTile tile kernel and partial-state merge kernel.
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
// gfx950 mapping.  A workgroup is 8 wave64s.  Inside a piece (one (b, kv head)
// context range) the waves take 32-key blocks round-robin and never
// synchronise until the piece ends.  Per block a wave
//   1. loads K and V rows straight from HBM into registers in the MFMA operand
//      layout (16-byte loads; lane = key row, lane group = 8-wide d chunk);
//   2. BMM1 on v_mfma_f32_16x16x32_bf16 with A = K (16 keys x 32 d), B = Q^T
//      (32 d x 16 heads, rows >= G are zero): S^T lands with the head index on
//      lanes and four consecutive keys per lane;
//   3. online softmax in the log2 domain; the row max over the block needs two
//      cross-lane steps (lanes 16 and 32 apart);
//   4. V^T without LDS: an MFMA against a 0/1 selection matrix re-distributes a
//      16-key x 32-d tile of V so that each lane holds four consecutive keys of
//      one d (exact: one product by 1.0 plus zeros);
//   5. BMM2 on MFMA with A = V^T (16 d x 32 keys), B = P^T (32 keys x 16 heads);
//      P is split into bf16 hi + lo parts (two MFMAs), so the weights keep
//      ~2^-17 relative accuracy instead of bf16's 2^-9.
//  The key order inside each MFMA contraction is chosen so that the lanes that
//  hold S^T after step 2 already hold the P^T operand of step 5 and the lanes
//  of step 4's output already hold the V^T operand: no shuffles and no LDS in
//  the streaming loop.  At the end of a piece the 8 wave states are merged
//  through LDS (max, rescale, tree sum) and written either as the final output
//  or as a partial slot for the merge kernel.
#include "common.h"

namespace attn {
namespace {

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load_row8(const uint16_t *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ __forceinline__ float wave_max_over_groups(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float wave_sum_over_groups(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

template <int HSZ>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_tiles_kernel(const DecodeParams p) {
    constexpr int NS = HSZ / 32;  // MFMA K steps over d
    constexpr int ND = HSZ / 16;  // 16-wide d blocks of the output
    constexpr int W = kDecodeWaves;
    constexpr int OSTRIDE = HSZ + 4;  // padded LDS row of the cross-wave reduction
    extern __shared__ float smem[];
    float *sm_m = smem;           // [W][16]
    float *sm_l = smem + W * 16;  // [W][16]
    float *sm_o = smem + 2 * W * 16;  // [W/2][G][OSTRIDE]

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;  // head g (Q, P, O), key row (K, V) or d (V^T)
    const int grp = lane >> 4;  // 8-wide slice of the MFMA contraction
    const int c = blockIdx.x;
    const LeanPlan &pl = p.plan;
    const int G = p.G;
    const float NEG_INF = -__builtin_inff();

    // 0/1 selection operands: sel[h] picks d = 16h + col out of a 32-d chunk.
    bf16x8 sel[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) sel[h][i] = (__bf16)((8 * grp + i == 16 * h + col) ? 1.0f : 0.0f);

    int64_t t = plan_cta_begin(pl, c);
    const int64_t t_end = plan_cta_begin(pl, c + 1);
    while (t < t_end) {
        const LeanPiece pc = plan_piece_at(pl, t, t_end);
        const int64_t kvrow = ((int64_t)pc.b * pl.KH + pc.kh) * p.kv_stride;
        const uint16_t *kbase = p.k + kvrow * HSZ;
        const uint16_t *vbase = p.v + kvrow * HSZ;
        const int h0 = pc.kh * G;

        bf16x8 qop[NS];
        const uint16_t *qrow = p.q + ((int64_t)pc.b * p.Hq + h0 + (col < G ? col : 0)) * HSZ;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            bf16x8 z = {};
            qop[s] = col < G ? load_row8(qrow + 32 * s + 8 * grp) : z;
        }

        float m_run = NEG_INF;  // running max (log2 domain) of head `col`
        float l_run = 0.f;      // this lane's share of the running sum
        f32x4 oacc[ND];         // O[col][16*db + 4*grp + i]
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

        const int nblk = (pc.key_end - pc.key_begin + kKeysPerBlock - 1) / kKeysPerBlock;
        const int klast = pc.key_end - 1;
        for (int blk = wave; blk < nblk; blk += W) {
            const int key0 = pc.key_begin + blk * kKeysPerBlock;
            bf16x8 kr[2][NS], vr[2][NS];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                int key = key0 + 16 * kb + col;
                key = key < klast ? key : klast;  // rows past the piece are re-reads, masked below
                const int64_t off = (int64_t)key * HSZ + 8 * grp;
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    kr[kb][s] = load_row8(kbase + off + 32 * s);
                    vr[kb][s] = load_row8(vbase + off + 32 * s);
                }
            }
            // BMM1: S^T[key][g] for keys key0 + 16kb + 4grp + i in lane (g = col, grp)
            f32x4 sc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NS; ++s) sc[kb] = mfma_bf16(kr[kb][s], qop[s], sc[kb]);
            }
            float x[8];
            float mx = NEG_INF;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = key0 + 16 * kb + 4 * grp + i;
                    const float xv = key <= klast ? sc[kb][i] * p.scale_log2 : NEG_INF;
                    x[4 * kb + i] = xv;
                    mx = fmaxf(mx, xv);
                }
            mx = wave_max_over_groups(mx);
            const float m_new = fmaxf(m_run, mx);  // finite: every block holds a valid key
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            float ps = 0.f;
            bf16x8 phi, plo;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float pv = __builtin_amdgcn_exp2f(x[i] - m_new);
                ps += pv;
                const __bf16 hi = (__bf16)pv;
                phi[i] = hi;
                plo[i] = (__bf16)(pv - (float)hi);
            }
            l_run = l_run * alpha + ps;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
            // V^T via selection MFMAs, then BMM2 with the hi and lo parts of P
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    const f32x4 t0 = mfma_bf16(vr[0][s], sel[h], z);
                    const f32x4 t1 = mfma_bf16(vr[1][s], sel[h], z);
                    bf16x8 vt;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        vt[i] = (__bf16)t0[i];
                        vt[4 + i] = (__bf16)t1[i];
                    }
                    const int db = 2 * s + h;
                    oacc[db] = mfma_bf16(vt, phi, oacc[db]);
                    oacc[db] = mfma_bf16(vt, plo, oacc[db]);
                }
        }

        // ---- merge the W wave states of this piece ----
        l_run = wave_sum_over_groups(l_run);
        __syncthreads();  // LDS of the previous piece is free
        if (grp == 0) {
            sm_m[wave * 16 + col] = m_run;
            sm_l[wave * 16 + col] = l_run;
        }
        __syncthreads();
        float M = NEG_INF;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w * 16 + col]);
        float Lt = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float mw = sm_m[w * 16 + col];
            Lt += mw == NEG_INF ? 0.f : sm_l[w * 16 + col] * __builtin_amdgcn_exp2f(mw - M);
        }
        const float f = m_run == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db] *= f;
#pragma unroll
        for (int half = W / 2; half >= 1; half >>= 1) {
            if (wave >= half && wave < 2 * half && col < G) {
                float *dst = sm_o + ((wave - half) * G + col) * OSTRIDE + 4 * grp;
#pragma unroll
                for (int db = 0; db < ND; ++db) *reinterpret_cast<f32x4 *>(dst + 16 * db) = oacc[db];
            }
            __syncthreads();
            if (wave < half && col < G) {
                const float *src = sm_o + (wave * G + col) * OSTRIDE + 4 * grp;
#pragma unroll
                for (int db = 0; db < ND; ++db) oacc[db] += *reinterpret_cast<const f32x4 *>(src + 16 * db);
            }
            __syncthreads();
        }

        if (wave == 0 && col < G) {
            if (pc.tile_begin == pc.seg_begin && pc.tile_end == pc.seg_end) {
                const float inv = 1.f / Lt;
                float *dst = p.out + ((int64_t)pc.b * p.Hq + h0 + col) * HSZ + 4 * grp;
#pragma unroll
                for (int db = 0; db < ND; ++db) *reinterpret_cast<f32x4 *>(dst + 16 * db) = oacc[db] * inv;
            } else {
                float *slot = p.ws + (int64_t)plan_slot(pl, c, pc.seg_begin) * p.slot_floats;
                float *dst = slot + col * HSZ + 4 * grp;
#pragma unroll
                for (int db = 0; db < ND; ++db) *reinterpret_cast<f32x4 *>(dst + 16 * db) = oacc[db];
                if (grp == 0) {
                    slot[G * HSZ + col] = M;
                    slot[G * HSZ + G + col] = Lt;
                }
            }
        }
        t = pc.tile_end;
    }
}

// One workgroup per (segment, head of the group, 32-wide d chunk).  Segments
// finished inside one CTA are skipped; empty segments (L_b = 0) get zero rows.
constexpr int kMergeThreads = 256;
constexpr int kMergeLanesPerPartial = 32;
constexpr int kMergeGroups = kMergeThreads / kMergeLanesPerPartial;

template <int HSZ>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const DecodeParams p) {
    __shared__ float red_m[kMergeGroups];
    __shared__ float red_o[kMergeGroups][kMergeLanesPerPartial];
    __shared__ float red_l[kMergeGroups];
    const LeanPlan &pl = p.plan;
    const int s = blockIdx.x, g = blockIdx.y, dc = blockIdx.z;
    const int b = s / pl.KH, kh = s % pl.KH;
    const int G = p.G;
    const int tid = threadIdx.x;
    const int pgrp = tid / kMergeLanesPerPartial, dd = tid % kMergeLanesPerPartial;
    const int d = dc * kMergeLanesPerPartial + dd;
    float *orow = p.out + ((int64_t)b * p.Hq + kh * G + g) * HSZ;
    const int nb = plan_tiles_per_segment(pl, b);
    if (nb == 0) {
        if (pgrp == 0) orow[d] = 0.f;
        return;
    }
    const int64_t seg_begin = pl.tile_prefix[b] + (int64_t)kh * nb;
    const int c_lo = plan_cta_of_tile(pl, seg_begin);
    const int c_hi = plan_cta_of_tile(pl, seg_begin + nb - 1);
    if (c_lo == c_hi) return;
    const int k = c_hi - c_lo + 1;
    const int slot0 = plan_slot(pl, c_lo, seg_begin);
    const float NEG_INF = -__builtin_inff();

    float mx = NEG_INF;
    for (int i = pgrp; i < k; i += kMergeGroups) {
        const int slot = i == 0 ? slot0 : 2 * (c_lo + i);
        mx = fmaxf(mx, p.ws[(int64_t)slot * p.slot_floats + G * HSZ + g]);
    }
    if (dd == 0) red_m[pgrp] = mx;
    __syncthreads();
    float M = NEG_INF;
#pragma unroll
    for (int j = 0; j < kMergeGroups; ++j) M = fmaxf(M, red_m[j]);

    float acc = 0.f, lsum = 0.f;
    for (int i = pgrp; i < k; i += kMergeGroups) {
        const int slot = i == 0 ? slot0 : 2 * (c_lo + i);
        const float *sp = p.ws + (int64_t)slot * p.slot_floats;
        const float f = __builtin_amdgcn_exp2f(sp[G * HSZ + g] - M);
        acc += f * sp[g * HSZ + d];
        lsum += f * sp[G * HSZ + G + g];
    }
    red_o[pgrp][dd] = acc;
    if (dd == 0) red_l[pgrp] = lsum;
    __syncthreads();
    if (pgrp == 0) {
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int j = 0; j < kMergeGroups; ++j) {
            o += red_o[j][dd];
            l += red_l[j];
        }
        orow[d] = o / l;
    }
}

template <int HSZ>
size_t decode_tiles_lds_bytes(int G) {
    return (size_t)(2 * kDecodeWaves * 16 + (kDecodeWaves / 2) * G * (HSZ + 4)) * sizeof(float);
}

size_t tiles_lds_bytes(int Hsz, int G) {
    switch (Hsz) {
        case 64: return decode_tiles_lds_bytes<64>(G);
        case 128: return decode_tiles_lds_bytes<128>(G);
        default: return decode_tiles_lds_bytes<256>(G);
    }
}

template <int HSZ>
hipError_t launch_tiles_t(const DecodeParams &p, hipStream_t stream) {
    const size_t lds = decode_tiles_lds_bytes<HSZ>(p.G);
    if (lds > 65536) {  // above the default dynamic-LDS limit; gfx950 has 160 KiB per CU
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(decode_tiles_kernel<HSZ>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(decode_tiles_kernel<HSZ>, dim3(p.plan.P), dim3(kDecodeWaves * 64), lds, stream, p);
    return hipGetLastError();
}

template <int HSZ>
hipError_t launch_merge_t(const DecodeParams &p, hipStream_t stream) {
    dim3 grid(p.plan.B * p.plan.KH, p.G, HSZ / kMergeLanesPerPartial);
    hipLaunchKernelGGL(decode_merge_kernel<HSZ>, grid, dim3(kMergeThreads), 0, stream, p);
    return hipGetLastError();
}

template <int HSZ>
int occupancy_t(int G) {
    int blocks = 0;
    const size_t lds = decode_tiles_lds_bytes<HSZ>(G);
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(decode_tiles_kernel<HSZ>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_tiles_kernel<HSZ>, kDecodeWaves * 64,
                                                     decode_tiles_lds_bytes<HSZ>(G)) != hipSuccess)
        return 1;
    return blocks > 0 ? blocks : 1;
}

}  // namespace

hipError_t launch_decode_tiles(const DecodeParams &p, int Hsz, hipStream_t stream) {
    switch (Hsz) {
        case 64: return launch_tiles_t<64>(p, stream);
        case 128: return launch_tiles_t<128>(p, stream);
        case 256: return launch_tiles_t<256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_merge(const DecodeParams &p, int Hsz, hipStream_t stream) {
    switch (Hsz) {
        case 64: return launch_merge_t<64>(p, stream);
        case 128: return launch_merge_t<128>(p, stream);
        case 256: return launch_merge_t<256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

int decode_tiles_occupancy(int Hsz, int G) {
    switch (Hsz) {
        case 64: return occupancy_t<64>(G);
        case 128: return occupancy_t<128>(G);
        default: return occupancy_t<256>(G);
    }
}

}  // namespace attn
