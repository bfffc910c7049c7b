// common.h -- types and launcher declarations shared by the HIP sources of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "plan.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

// Lane l together with lane l ^ 16 (swap16) or lane l ^ 32 (swap32) of a
// wave64, through the gfx950 cross-lane swaps instead of an LDS permute: the
// swap exchanges 16-lane rows (or 32-lane halves) between two registers, so
// after swapping two copies of x one copy holds every lane's own value and the
// other its partner's, in an order that depends on the lane (checked on the
// GPU lane by lane).  Max and sum of the pair are then the same on both lanes
// of it.  Every lane of the wave must be active.  The swaps are written in asm
// with both registers as in-out operands: the compiler's builtin returns the
// first register's result for both of its outputs.  The nops give the wait
// states around a swap of registers that a VALU instruction has just written.
__device__ __forceinline__ void swap16(float x, float &a, float &b) {
    a = x;
    b = x;
    __asm__("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(float x, float &a, float &b) {
    a = x;
    b = x;
    __asm__("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float pair_max32(float x) {
    float a, b;
    swap32(x, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum32(float x) {
    float a, b;
    swap32(x, a, b);
    return a + b;
}

// Query columns one decode workgroup holds: G query heads x q_len drafted
// tokens, in blocks of 16 MFMA columns.  At most kMaxColumns of them, and
// columns x Hsz at most kMaxColumnElems (their output accumulators live in
// registers: 64 columns at Hsz 64 or 128, 32 at Hsz 256).
constexpr int kMaxColumns = 64;
constexpr int kMaxColumnElems = 64 * 128;
inline bool decode_columns_supported(int NC, int Hsz) {
    return NC >= 1 && NC <= kMaxColumns && NC * Hsz <= kMaxColumnElems;
}

// Kernel arguments of the decode tile kernel (passed by value: the plan rides in kernargs).
struct DecodeParams {
    const uint16_t *q;   // bf16 [B][Hq][Hsz]
    const uint16_t *k;   // [B][KH][S][Hsz], bf16 or (reinterpreted) FP8 E4M3 bytes
    const uint16_t *v;   // same layout as k
    float *out;          // fp32 [B][Hq][Hsz]
    float *lse;          // optional fp32 [B][Hq][qlen]: log2 of each row's softmax denominator (NULL = none)
    float *ws;           // partial slots, each slot_floats long
    int *counters;       // arrival counters [2 * kMaxCtas], zero between calls
    int64_t kv_stride;   // S
    int Hq;
    int G;
    int qlen;            // query tokens per request (1 = plain decode; gamma for drafted tokens)
    int NC;              // MFMA columns in use: G * qlen <= 16, column c = (token c / G, head c % G)
    int slot_floats;     // NC*Hsz (O) + NC (m) + NC (l), rounded up to a multiple of 4
    float scale_log2;    // softmax scale * key scale * log2(e)
    float v_scale;       // value scale (1 for bf16 caches)
    const int32_t *block_table;  // paged KV: [B][max_blocks_per_seq] block ids (NULL = contiguous)
    int max_blocks_per_seq;
    int log2_block_size;
    int num_blocks;
    // Device seqlens (non-NULL): every CTA builds the plan from these lengths, and
    // `plan` carries only B, KH, T, mode, splits and the launched P; CTA 0 lists
    // the heads split over more than kMergeFanIn CTAs in wide_list / *wide_count.
    const int32_t *seqlens_dev;
    int *wide_count;
    struct WideHead *wide_list;
    LeanPlan plan;
};

// Partial slot layout: O[NC][Hsz] unnormalised, then m[NC] (log2 domain), then l[NC].
inline int decode_slot_floats(int NC, int Hsz) { return (NC * Hsz + 2 * NC + 3) & ~3; }

// Split heads whose partials sit in at most kMergeFanIn CTAs are merged inside
// the tile kernel by the CTA that arrives last; wider heads (at most
// kMaxWideHeads of them: each one has at least kMergeFanIn - 1 CTAs to
// itself) by merge_wide_kernel.
constexpr int kMergeFanIn = 16;
constexpr int kMaxCtas = 4096;
constexpr int kMaxWideHeads = (kMaxCtas + kMergeFanIn - 2) / (kMergeFanIn - 1);

// A wide head for merge_wide_kernel, packed so one scalar load fetches it:
// bkh = b | kh << 8; cta = c_lo | (n - 1) << 12 | (slot of partial 0 is odd) << 24.
struct WideHead {
    int32_t bkh;
    int32_t cta;
};

struct WideMergeParams {
    const int *count_dev;          // non-NULL: the list was built on the device, head_dev[0 .. *count_dev)
    const WideHead *head_dev;
    const float *ws;      // partial slots
    float *out;           // fp32 [B][Hq][qlen][Hsz]
    float *lse;           // optional [B][Hq][qlen]
    int slot_floats;
    int NC, G, Hq, qlen;
    float v_scale;
    int count;            // wide heads
    WideHead head[kMaxWideHeads];
};

// Workspace layout: int counters[2 * kMaxCtas] (a fixed-size region, so its
// place never depends on P), then a plan area that a call with device seqlens
// uses for the wide-head count and list (written by the decode kernel's CTA 0
// for the merge kernel), then float slots[2P][slot_floats].
constexpr size_t kCounterBytes = (size_t)2 * kMaxCtas * sizeof(int);
constexpr size_t kPlanAreaBytes = 8192;
constexpr size_t kWideCountOffset = 4096;  // within the plan area
constexpr size_t kWideListOffset = 4112;
static_assert(sizeof(LeanPlan) <= kWideCountOffset, "plan area too small for the plan");
static_assert(kWideListOffset + kMaxWideHeads * sizeof(WideHead) <= kPlanAreaBytes, "plan area too small for the list");
inline size_t decode_workspace_bytes(int P, int NC, int Hsz) {
    return kCounterBytes + kPlanAreaBytes + (size_t)2 * P * decode_slot_floats(NC, Hsz) * sizeof(float);
}

// Raises `fn`'s dynamic-LDS limit to `lds` bytes on the current device if it is
// above the 64 KiB default; `done` is a kMaxLdsDevices-entry record of the
// largest size already set per device (zero-initialised, one per kernel).
constexpr int kMaxLdsDevices = 64;
hipError_t ensure_lds_limit(const void *fn, std::atomic<int> *done, size_t lds);

// Launchers (return hipError_t of the launch).
// Optional timing events are bound to the kernels' own start and end timestamps.
hipError_t launch_decode_tiles(const DecodeParams &p, int Hsz, bool fp8, hipStream_t stream,
                               hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr);
hipError_t launch_merge_wide(const WideMergeParams &mp, int Hsz, hipStream_t stream, hipEvent_t ev_end = nullptr);
hipError_t launch_zero_fill(void *ptr, size_t bytes, hipStream_t stream);
hipError_t launch_merge_shards(const float *outs, const float *lses, int S, int64_t rows, int Hsz, float *out,
                               float *lse_out, hipStream_t stream);
int decode_tiles_occupancy(int Hsz, int NC);  // resident decode workgroups per CU
int decode_tile_keys(int Hsz, int NC);       // default LeanTile: one block per wave
hipError_t launch_prefill_causal(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *out,
                                 int B, int ISL, int Hq, int KH, int Hsz, float scale_log2,
                                 hipStream_t stream);
hipError_t launch_copy_probe(const void *src, void *dst, size_t bytes, hipStream_t stream);
hipError_t launch_read_probe(const void *src, size_t bytes, void *sink, hipStream_t stream);

}  // namespace attn
