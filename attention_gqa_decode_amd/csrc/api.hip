// api.hip -- the C ABI (include/attn_gqa.h): validation, LeanTile planning, workspace, launches.
//
// Every argument check runs before anything is enqueued, so argument errors
// are reported synchronously and leave no trace on the device.  Only the
// checks that depend on the library's default workgroup count (a caller
// workspace too small for it) come after a device query.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/attn_gqa.h"
#include "common.h"

static_assert(ATTN_MAX_COLUMNS == attn::kMaxColumns, "column limit mismatch");
static_assert(ATTN_MAX_COLUMN_ELEMS == attn::kMaxColumnElems, "column limit mismatch");
static_assert(ATTN_MAX_CTAS == attn::kMaxCtas, "CTA limit mismatch");
static_assert(ATTN_DECODE_COUNTER_BYTES == attn::kCounterBytes, "counter region mismatch");
static_assert(ATTN_DECODE_PLAN_BYTES == attn::kPlanAreaBytes, "plan area mismatch");

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int fail_hip(hipError_t e, const char *what) {
    return fail(ATTN_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;      // library-owned partial-state buffers
// Resident decode workgroups per (device, head dimension, query columns), 0 until
// first queried.  A fixed table, so a decode call allocates no host memory.
constexpr int kResidentDevices = 64;
std::atomic<int> g_resident[kResidentDevices][3][attn::kMaxColumns + 1];

int device_default_ctas(int Hsz, int NC, int *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    if (dev < 0 || dev >= kResidentDevices) return fail(ATTN_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kResidentDevices);
    std::atomic<int> &slot = g_resident[dev][Hsz == 64 ? 0 : (Hsz == 128 ? 1 : 2)][NC];
    int r = slot.load(std::memory_order_acquire);
    if (r > 0) {
        *out = r;
        return ATTN_OK;
    }
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute(MultiprocessorCount)");
    r = cus * attn::decode_tiles_occupancy(Hsz, NC);
    slot.store(r, std::memory_order_release);  // concurrent first queries store the same value
    *out = r;
    return ATTN_OK;
}

// Stream-K workgroups when the caller leaves num_ctas at 0.  One per resident
// slot, or, when the (request, kv head) segments outnumber the slots k >= 2
// times, k per slot (at most 4): a workgroup's time then depends on how many
// pieces (segment starts and ends) its tile range holds, not only on its tile
// count, and with several workgroups per slot the hardware starts the next
// one wherever a slot frees, which evens the slots out.  Measured on MI355X:
// the ragged sweep's G=1 points run 6-10% faster, G=2 2% faster; batches
// with fewer segments than slots keep one workgroup per slot (more would only
// add partial states).
int stream_k_default_ctas(int64_t segments, int resident) {
    int64_t k = resident > 0 ? segments / resident : 1;
    k = k < 1 ? 1 : (k > 4 ? 4 : k);
    const int64_t P = k * resident;
    return (int)(P < attn::kMaxCtas ? P : attn::kMaxCtas);
}

int library_workspace(hipStream_t stream, size_t bytes, void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_mu);
    Workspace &w = g_ws[std::make_pair(dev, stream)];
    if (w.bytes < bytes) {
        if (w.ptr) {
            e = hipStreamSynchronize(stream);  // earlier launches on this stream may still read it
            if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
            e = hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
            if (e != hipSuccess) return fail_hip(e, "hipFree(workspace)");
        }
        size_t grow = bytes + bytes / 4;
        e = hipMalloc(&w.ptr, grow);
        if (e != hipSuccess) {
            w.ptr = nullptr;
            return fail_hip(e, "hipMalloc(workspace)");
        }
        w.bytes = grow;
        // the arrival counters must start at zero; the kernel leaves them zero
        e = attn::launch_zero_fill(w.ptr, grow, stream);
        if (e != hipSuccess) return fail_hip(e, "workspace zero fill");
    }
    *ptr = w.ptr;
    return ATTN_OK;
}

// Shape checks shared by attn_decode_ex and attn_decode_workspace_bytes.
int check_decode_dims(int B, int Hq, int KH, int Hsz) {
    if (B <= 0 || Hq <= 0 || KH <= 0) return fail(ATTN_ERR_SHAPE, "B, Hq and KH must be positive (B=%d Hq=%d KH=%d)", B, Hq, KH);
    if (Hq % KH != 0) return fail(ATTN_ERR_SHAPE, "Hq=%d is not a multiple of KH=%d", Hq, KH);
    if (Hsz != 64 && Hsz != 128 && Hsz != 256) return fail(ATTN_ERR_UNSUPPORTED, "Hsz=%d (supported: 64, 128, 256)", Hsz);
    if (!attn::decode_columns_supported(Hq / KH, Hsz))
        return fail(ATTN_ERR_UNSUPPORTED, "group size G=%d at Hsz=%d exceeds the column limit (G <= %d, G*Hsz <= %d)",
                    Hq / KH, Hsz, attn::kMaxColumns, attn::kMaxColumnElems);
    if (B > ATTN_MAX_BATCH) return fail(ATTN_ERR_UNSUPPORTED, "B=%d exceeds %d", B, ATTN_MAX_BATCH);
    return ATTN_OK;
}

// Host half of the LeanTile plan: tile prefix over batches and the tile count N.
int build_plan(const int32_t *seqlens, int B, int KH, int T, int64_t stride, LeanPlan *plan) {
    plan->B = B;
    plan->KH = KH;
    plan->T = T;
    int64_t acc = 0;
    for (int b = 0; b < B; ++b) {
        const int32_t L = seqlens[b];
        if (L < 0) return fail(ATTN_ERR_SHAPE, "seqlens[%d]=%d is negative", b, L);
        if (stride >= 0 && L > stride) return fail(ATTN_ERR_SHAPE, "seqlens[%d]=%d exceeds kv_stride=%lld", b, L, (long long)stride);
        plan->seqlen[b] = L;
        plan->tile_prefix[b] = (int32_t)acc;
        acc += (int64_t)KH * ((L + (int64_t)T - 1) / T);
        if (acc > 0x7fffffffLL) return fail(ATTN_ERR_UNSUPPORTED, "too many LeanTiles (%lld); raise tile_keys", (long long)acc);
    }
    plan->tile_prefix[B] = (int32_t)acc;
    plan->N = acc;
    plan->P = 1;
    plan->mode = kPlanStreamK;
    plan->splits = 1;
    return ATTN_OK;
}

// Splits per segment of the fixed-split schedule when the caller gives none:
// enough CTAs to fill every resident slot once (the FlashDecoding default),
// never more than the longest segment's tiles, within the merge-counter range.
int default_splits(const LeanPlan &p, int resident) {
    const int segs = p.B * p.KH;
    int nmax = 0;
    for (int b = 0; b < p.B; ++b) {
        const int n = plan_tiles_per_segment(p, b);
        nmax = n > nmax ? n : nmax;
    }
    int S = (resident + segs - 1) / segs;
    if (S > nmax) S = nmax;
    if (S > attn::kMaxCtas / segs) S = attn::kMaxCtas / segs;
    return S < 1 ? 1 : S;
}

// One pass over the segments: whether any of them is split over several CTAs
// (*split), and the list of those split over more than kMergeFanIn CTAs (their
// merge runs in merge_wide_kernel).  Each such head owns the whole ranges of
// at least kMergeFanIn - 1 CTAs, so there are at most kMaxWideHeads of them;
// returns false if the list would still overflow.
bool scan_segments(const LeanPlan &p, bool *split, attn::WideMergeParams *wide) {
    *split = false;
    wide->count = 0;
    for (int b = 0; b < p.B; ++b) {
        const int nb = plan_tiles_per_segment(p, b);
        if (nb == 0) continue;
        for (int kh = 0; kh < p.KH; ++kh) {
            const int64_t s0 = p.tile_prefix[b] + (int64_t)kh * nb;
            const int n = plan_segment_ctas(p, s0, s0 + nb).n;
            *split |= n > 1;
            if (n > attn::kMergeFanIn) {
                if (wide->count == attn::kMaxWideHeads) return false;
                const int c_lo = plan_cta_of_tile(p, s0);
                attn::WideHead &h = wide->head[wide->count++];
                h.bkh = b | kh << 8;
                h.cta = c_lo | (n - 1) << 12 | (plan_slot(p, c_lo, s0) & 1) << 24;
            }
        }
    }
    return true;
}

}  // namespace

extern "C" {

const char *attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "null pointer argument";
        case ATTN_ERR_SHAPE: return "inconsistent shape";
        case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
        case ATTN_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
        case ATTN_ERR_WORKSPACE: return "workspace too small";
        case ATTN_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *attn_last_error(void) { return g_last_error.c_str(); }

size_t attn_decode_multi_workspace_bytes(int B, int Hq, int KH, int Hsz, int q_len, int num_ctas) {
    if (check_decode_dims(B, Hq, KH, Hsz) != ATTN_OK || num_ctas < 0 || q_len < 0) return 0;
    const int NC = (Hq / KH) * (q_len > 1 ? q_len : 1);
    if (!attn::decode_columns_supported(NC, Hsz)) return 0;
    int P = num_ctas;
    if (P == 0) {
        // the larger of the two default counts: stream-K's, and the fixed split's
        // B*KH*S with S = ceil(resident / (B*KH)) (capped so B*KH*S <= ATTN_MAX_CTAS),
        // which only splits, and so only needs slots, when S >= 2
        int resident = 0;
        if (device_default_ctas(Hsz, NC, &resident) != ATTN_OK) return 0;
        P = stream_k_default_ctas((int64_t)B * KH, resident);
        const int64_t segs = (int64_t)B * KH;
        int64_t S = (resident + segs - 1) / segs;
        if (S > attn::kMaxCtas / segs) S = attn::kMaxCtas / segs;
        if (S >= 2 && segs * S > P) P = (int)(segs * S);
    }
    if (P > attn::kMaxCtas) return 0;
    return attn::decode_workspace_bytes(P, NC, Hsz);
}

size_t attn_decode_workspace_bytes(int B, int Hq, int KH, int Hsz, int num_ctas) {
    return attn_decode_multi_workspace_bytes(B, Hq, KH, Hsz, 1, num_ctas);
}

}  // extern "C"

namespace {

// Where the partial-state workspace of a decode call comes from.
enum class WorkspaceSource { Caller, Library, Scratch };

// The workspace of attn_decode_noalloc: a device array of fixed size in the
// library's code object, so that entry point never allocates.  Each device the
// library runs on holds its own copy until the process ends.  `scratch` is the
// host-side stand-in of the array; the device address of a device's copy comes
// from hipGetSymbolAddress (scratch_pointer) and is the only address used.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
static_assert(ATTN_NOALLOC_SCRATCH_BYTES == kScratchBytes, "scratch size mismatch");

constexpr int kScratchDevices = 64;
void *g_scratch_ptr[kScratchDevices];  // per device, set once under g_mu

// The current device's copy of `scratch`, resolved once per device.
int scratch_pointer(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    if (dev < 0 || dev >= kScratchDevices) return fail(ATTN_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kScratchDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return ATTN_OK;
}

int decode_impl(const attn_decode_args *a, hipStream_t stream, WorkspaceSource src) {
    if (!a) return fail(ATTN_ERR_NULL, "args is NULL");
    if (!a->q || !a->k_cache || !a->v_cache || !a->seqlens || !a->out)
        return fail(ATTN_ERR_NULL, "q, k_cache, v_cache, seqlens and out must be non-NULL");
    int st = check_decode_dims(a->B, a->Hq, a->KH, a->Hsz);
    if (st != ATTN_OK) return st;
    if (!aligned16(a->q) || !aligned16(a->k_cache) || !aligned16(a->v_cache) || !aligned16(a->out))
        return fail(ATTN_ERR_ALIGN, "q, k_cache, v_cache and out must be 16-byte aligned");
    if (a->kv_stride < 0) return fail(ATTN_ERR_SHAPE, "kv_stride=%lld is negative", (long long)a->kv_stride);
    if (a->tile_keys < 0 || a->num_ctas < 0) return fail(ATTN_ERR_SHAPE, "tile_keys and num_ctas must be >= 0");
    if (a->num_ctas > attn::kMaxCtas) return fail(ATTN_ERR_UNSUPPORTED, "num_ctas=%d exceeds %d", a->num_ctas, attn::kMaxCtas);
    if (a->q_len < 0) return fail(ATTN_ERR_SHAPE, "q_len=%d is negative", a->q_len);
    const int qlen = a->q_len > 1 ? a->q_len : 1;
    if ((int64_t)(a->Hq / a->KH) * qlen > attn::kMaxColumns ||
        !attn::decode_columns_supported((a->Hq / a->KH) * qlen, a->Hsz))
        return fail(ATTN_ERR_UNSUPPORTED, "G*q_len=%lld query columns at Hsz=%d exceed the limit (<= %d, columns*Hsz <= %d)",
                    (long long)(a->Hq / a->KH) * qlen, a->Hsz, attn::kMaxColumns, attn::kMaxColumnElems);
    const bool dev_sl = a->seqlens_on_device != 0;
    if (dev_sl) {
        if (((uintptr_t)a->seqlens & 3u) != 0) return fail(ATTN_ERR_ALIGN, "device seqlens must be 4-byte aligned");
        if (!a->block_table && a->kv_stride == 0)
            return fail(ATTN_ERR_SHAPE, "device seqlens need an explicit kv_stride (or a block table)");
    } else {
        for (int b = 0; b < a->B; ++b)
            if (a->seqlens[b] != 0 && a->seqlens[b] < qlen)
                return fail(ATTN_ERR_SHAPE, "seqlens[%d]=%d holds fewer keys than q_len=%d", b, a->seqlens[b], qlen);
    }
    if (a->schedule < ATTN_SCHEDULE_AUTO || a->schedule > ATTN_SCHEDULE_FIXED_SPLIT)
        return fail(ATTN_ERR_SHAPE, "schedule=%d is not an ATTN_SCHEDULE_* value", a->schedule);
    if (a->num_splits < 0) return fail(ATTN_ERR_SHAPE, "num_splits=%d is negative", a->num_splits);
    if (a->kv_dtype != ATTN_KV_BF16 && a->kv_dtype != ATTN_KV_FP8_E4M3)
        return fail(ATTN_ERR_SHAPE, "kv_dtype=%d is not an ATTN_KV_* value", a->kv_dtype);
    if (!(a->k_scale == a->k_scale) || isinf(a->k_scale) || !(a->v_scale == a->v_scale) || isinf(a->v_scale))
        return fail(ATTN_ERR_SHAPE, "k_scale and v_scale must be finite");
    if (a->kv_dtype == ATTN_KV_BF16 && (a->k_scale > 0.f || a->v_scale > 0.f) && (a->k_scale != 1.f || a->v_scale != 1.f))
        return fail(ATTN_ERR_SHAPE, "k_scale and v_scale apply to FP8 caches only");
    if (a->schedule == ATTN_SCHEDULE_FIXED_SPLIT && a->num_ctas != 0)
        return fail(ATTN_ERR_SHAPE, "num_ctas is set by the fixed-split schedule (B*KH*num_splits); pass 0");
    if (a->schedule == ATTN_SCHEDULE_FIXED_SPLIT && a->num_splits > 1 &&
        (int64_t)a->B * a->KH * a->num_splits > attn::kMaxCtas)
        return fail(ATTN_ERR_UNSUPPORTED, "B*KH*num_splits=%lld exceeds %d", (long long)a->B * a->KH * a->num_splits,
                    attn::kMaxCtas);
    if (!(a->scale == a->scale) || isinf(a->scale)) return fail(ATTN_ERR_SHAPE, "scale must be finite");
    if (a->workspace && !aligned16(a->workspace)) return fail(ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (((uintptr_t)a->out_lse & 3u) != 0) return fail(ATTN_ERR_ALIGN, "out_lse must be 4-byte aligned");

    int log2_bs = 0;
    if (a->block_table) {
        if (a->kv_stride != 0) return fail(ATTN_ERR_SHAPE, "kv_stride must be 0 with a block table");
        if (a->block_size < 16 || (a->block_size & (a->block_size - 1)))
            return fail(ATTN_ERR_UNSUPPORTED, "block_size=%d (supported: powers of two >= 16)", a->block_size);
        if (a->max_blocks_per_seq <= 0 || a->num_blocks <= 0)
            return fail(ATTN_ERR_SHAPE, "max_blocks_per_seq and num_blocks must be positive");
        if (((uintptr_t)a->block_table & 3u) != 0) return fail(ATTN_ERR_ALIGN, "block_table must be 4-byte aligned");
        while ((1 << log2_bs) < a->block_size) ++log2_bs;
    } else if (a->block_size != 0 || a->max_blocks_per_seq != 0 || a->num_blocks != 0) {
        return fail(ATTN_ERR_SHAPE, "block_size, max_blocks_per_seq and num_blocks need a block table");
    }

    const int G = a->Hq / a->KH;
    int64_t stride = a->kv_stride;
    if (a->block_table) {
        stride = (int64_t)a->max_blocks_per_seq * a->block_size;  // the longest context a table row can map
    } else if (stride == 0) {
        for (int b = 0; b < a->B; ++b) stride = a->seqlens[b] > stride ? a->seqlens[b] : stride;
    }
    const int T = a->tile_keys > 0 ? a->tile_keys : attn::decode_tile_keys(a->Hsz, G * qlen);

    attn::DecodeParams p;
    if (dev_sl) {
        // only the shape is known here; the device fills in L_b, the prefix and N
        const int64_t nmax = (stride + T - 1) / T;  // tiles of the longest possible context
        if ((int64_t)a->B * a->KH * nmax > 0x7fffffffLL)
            return fail(ATTN_ERR_UNSUPPORTED, "B*KH*ceil(kv_stride/T)=%lld LeanTiles exceed 2^31; raise tile_keys",
                        (long long)a->B * a->KH * nmax);
        p.plan = LeanPlan{};
        p.plan.B = a->B;
        p.plan.KH = a->KH;
        p.plan.T = T;
        for (int b = 0; b <= a->B; ++b) p.plan.tile_prefix[b] = (int32_t)((int64_t)b * a->KH * nmax);  // upper bounds
        p.plan.N = (int64_t)a->B * a->KH * nmax;
        p.plan.mode = kPlanStreamK;
        p.plan.splits = 1;
    } else {
        st = build_plan(a->seqlens, a->B, a->KH, T, stride, &p.plan);
        if (st != ATTN_OK) return st;
    }
    p.seqlens_dev = nullptr;
    p.wide_count = nullptr;
    p.wide_list = nullptr;
    p.q = static_cast<const uint16_t *>(a->q);
    p.k = static_cast<const uint16_t *>(a->k_cache);
    p.v = static_cast<const uint16_t *>(a->v_cache);
    p.out = a->out;
    p.lse = a->out_lse;
    p.ws = nullptr;
    p.kv_stride = stride;
    p.Hq = a->Hq;
    p.G = G;
    p.qlen = qlen;
    p.NC = G * qlen;
    p.slot_floats = attn::decode_slot_floats(p.NC, a->Hsz);
    const float scale = a->scale > 0.f ? a->scale : 1.0f / sqrtf((float)a->Hsz);
    const bool fp8 = a->kv_dtype == ATTN_KV_FP8_E4M3;
    const float k_scale = fp8 && a->k_scale > 0.f ? a->k_scale : 1.f;
    p.scale_log2 = scale * k_scale * 1.4426950408889634f;
    p.v_scale = fp8 && a->v_scale > 0.f ? a->v_scale : 1.f;
    p.block_table = a->block_table;
    p.max_blocks_per_seq = a->max_blocks_per_seq;
    p.log2_block_size = log2_bs;
    p.num_blocks = a->num_blocks;

    // ---- the schedule and the CTA count.  The device is queried only when
    // the caller leaves the count to the library, so that with an explicit
    // stream-K count every argument error (the workspace size included) is
    // still reported before the first HIP call. ----
    int resident = 0;
    auto query_resident = [&]() -> int {
        return resident > 0 ? ATTN_OK : device_default_ctas(a->Hsz, p.NC, &resident);
    };
    // The selector (the digest's runtime selection policy: stream-K tiles for
    // long, few-head or ragged work; no split when the batch alone fills every
    // resident slot evenly) runs one CTA per segment when that finishes no later
    // than stream-K's even share, ceil(N / resident) tiles (so no partial
    // states at all), and stream-K otherwise.  With device seqlens the host
    // cannot see the lengths, and stream-K is the choice that never leaves a
    // long context to one CTA.
    int P = a->num_ctas;
    int schedule = a->schedule;
    if (schedule == ATTN_SCHEDULE_AUTO) {
        schedule = ATTN_SCHEDULE_STREAM_K;
        if (!dev_sl && a->num_ctas == 0 && p.plan.N > 0) {
            if ((st = query_resident()) != ATTN_OK) return st;
            int64_t heap[attn::kMaxCtas];  // the selector's min-heap, one entry per resident slot
            const int R = resident < attn::kMaxCtas ? resident : attn::kMaxCtas;
            const int64_t even = (p.plan.N + R - 1) / R;
            if (plan_whole_segments_makespan(p.plan, R, heap) <= even)
                schedule = ATTN_SCHEDULE_FIXED_SPLIT;
        }
    }
    if (schedule == ATTN_SCHEDULE_FIXED_SPLIT) {
        int S = a->num_splits;
        if (S == 0) {
            if (a->schedule == ATTN_SCHEDULE_AUTO) {
                S = 1;
            } else {
                if ((st = query_resident()) != ATTN_OK) return st;
                S = default_splits(p.plan, resident);
            }
        }
        p.plan.mode = kPlanFixedSplit;
        p.plan.splits = S;
        P = a->B * a->KH * S;
    } else {
        if (P == 0) {
            if ((st = query_resident()) != ATTN_OK) return st;
            P = stream_k_default_ctas((int64_t)a->B * a->KH, resident);
        }
        // no empty CTA; one CTA zeroes an all-empty batch (with device seqlens the device clamps P)
        if (!dev_sl && P > p.plan.N) P = p.plan.N > 0 ? (int)p.plan.N : 1;
    }
    p.plan.P = P;
    p.counters = nullptr;

    attn::WideMergeParams wide;
    wide.count = 0;
    wide.count_dev = nullptr;
    wide.head_dev = nullptr;
    bool split = dev_sl;  // with device seqlens the host cannot tell: always bring the workspace
    if (!dev_sl && p.plan.N > 0 && !scan_segments(p.plan, &split, &wide))
        return fail(ATTN_ERR_UNSUPPORTED, "more than %d heads split over more than %d workgroups", attn::kMaxWideHeads,
                    attn::kMergeFanIn);
    const size_t need = split ? attn::decode_workspace_bytes(P, p.NC, a->Hsz) : 0;
    if (split && src == WorkspaceSource::Caller && a->workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace_bytes=%zu < %zu needed for %d workgroups", a->workspace_bytes, need, P);
    if (split && src == WorkspaceSource::Scratch && need > kScratchBytes)
        return fail(ATTN_ERR_WORKSPACE, "this call needs %zu bytes of partial-state workspace; attn_decode_noalloc "
                    "holds at most %zu (ATTN_NOALLOC_SCRATCH_BYTES)", need, kScratchBytes);

    // ---- HIP calls from here on ----
    if (split) {
        char *w = nullptr;
        if (src == WorkspaceSource::Caller) {
            w = static_cast<char *>(a->workspace);
        } else if (src == WorkspaceSource::Scratch) {
            void *sp = nullptr;
            if ((st = scratch_pointer(&sp)) != ATTN_OK) return st;
            w = static_cast<char *>(sp);
            // The array keeps the last call's contents: clear the arrival counters
            // this call uses (a fill kernel rather than a memset, so a captured
            // graph replays it correctly).
            const hipError_t ez = attn::launch_zero_fill(w, (size_t)2 * P * sizeof(int), stream);
            if (ez != hipSuccess) return fail_hip(ez, "scratch counter fill");
        } else {
            void *lw = nullptr;
            if ((st = library_workspace(stream, need, &lw)) != ATTN_OK) return st;
            w = static_cast<char *>(lw);
        }
        p.counters = reinterpret_cast<int *>(w);
        p.ws = reinterpret_cast<float *>(w + attn::kCounterBytes + attn::kPlanAreaBytes);
        if (dev_sl) {
            // every CTA builds the plan from the device lengths; CTA 0 lists the wide
            // heads in the plan area for the merge kernel
            char *area = w + attn::kCounterBytes;
            p.seqlens_dev = a->seqlens;
            p.wide_count = reinterpret_cast<int *>(area + attn::kWideCountOffset);
            p.wide_list = reinterpret_cast<attn::WideHead *>(area + attn::kWideListOffset);
            wide.count_dev = p.wide_count;
            wide.head_dev = p.wide_list;
        }
    }

    hipError_t e;
    if (dev_sl) {
        // the most heads that can be split over more than kMergeFanIn CTAs
        const int64_t segs = (int64_t)a->B * a->KH;
        int64_t most = p.plan.mode == kPlanFixedSplit ? (p.plan.splits > attn::kMergeFanIn ? segs : 0)
                                                      : P / (attn::kMergeFanIn - 1);
        most = most < segs ? most : segs;
        wide.count = (int)(most < attn::kMaxWideHeads ? most : attn::kMaxWideHeads);
    }
    // The timing events are bound to the start of the tile kernel and to the end
    // of the last decode kernel of the call.
    const bool merge_follows = p.ws && wide.count > 0;
    e = attn::launch_decode_tiles(p, a->Hsz, fp8, stream, a->ev_tiles_begin, merge_follows ? nullptr : a->ev_tiles_end);
    if (e != hipSuccess) return fail_hip(e, "decode tile kernel launch");
    if (merge_follows) {
        wide.ws = p.ws;
        wide.out = p.out;
        wide.lse = p.lse;
        wide.slot_floats = p.slot_floats;
        wide.NC = p.NC;
        wide.G = p.G;
        wide.Hq = p.Hq;
        wide.qlen = p.qlen;
        wide.v_scale = p.v_scale;
        e = attn::launch_merge_wide(wide, a->Hsz, stream, a->ev_tiles_end);
        if (e != hipSuccess) return fail_hip(e, "wide merge kernel launch");
    }
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_ex(const attn_decode_args *a, hipStream_t stream) {
    g_last_error.clear();
    if (a && a->workspace) return decode_impl(a, stream, WorkspaceSource::Caller);
    return decode_impl(a, stream, WorkspaceSource::Library);
}

int attn_decode_noalloc(const attn_decode_args *a, hipStream_t stream) {
    g_last_error.clear();
    if (a && (a->workspace || a->workspace_bytes))
        return fail(ATTN_ERR_SHAPE, "attn_decode_noalloc uses the library's fixed scratch: workspace must be NULL and "
                    "workspace_bytes 0");
    return decode_impl(a, stream, WorkspaceSource::Scratch);
}

int attn_merge_shards(const float *outs, const float *lses, int S, int64_t rows, int Hsz, float *out, float *lse_out,
                      hipStream_t stream) {
    g_last_error.clear();
    if (!outs || !lses || !out) return fail(ATTN_ERR_NULL, "outs, lses and out must be non-NULL");
    if (S <= 0 || rows < 0) return fail(ATTN_ERR_SHAPE, "S=%d must be positive and rows=%lld non-negative", S, (long long)rows);
    if (Hsz <= 0 || Hsz % 4 != 0) return fail(ATTN_ERR_SHAPE, "Hsz=%d must be a positive multiple of 4", Hsz);
    if ((int64_t)S * rows * Hsz > ((int64_t)1 << 40)) return fail(ATTN_ERR_UNSUPPORTED, "S*rows*Hsz too large");
    if (!aligned16(outs) || !aligned16(out) || ((uintptr_t)lses & 3u) != 0 || ((uintptr_t)lse_out & 3u) != 0)
        return fail(ATTN_ERR_ALIGN, "outs and out must be 16-byte aligned, lses and lse_out 4-byte aligned");
    const hipError_t e = attn::launch_merge_shards(outs, lses, S, rows, Hsz, out, lse_out, stream);
    if (e != hipSuccess) return fail_hip(e, "shard merge kernel launch");
    return ATTN_OK;
}

int attn_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *seqlens, int B, int Hq,
                int KH, int Hsz, float *out, hipStream_t stream) {
    attn_decode_args a = {};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.seqlens = seqlens;
    a.out = out;
    a.B = B;
    a.Hq = Hq;
    a.KH = KH;
    a.Hsz = Hsz;
    return attn_decode_ex(&a, stream);
}

int attn_decode_plan(const int32_t *seqlens, int B, int KH, int tile_keys, int num_ctas, int64_t *N_out, int *P_out,
                     int64_t *cta_tile_begin, int64_t *seg_tile_begin) {
    g_last_error.clear();
    if (!seqlens || !N_out || !P_out) return fail(ATTN_ERR_NULL, "seqlens, N_out and P_out must be non-NULL");
    if (B <= 0 || KH <= 0) return fail(ATTN_ERR_SHAPE, "B and KH must be positive");
    if (B > ATTN_MAX_BATCH) return fail(ATTN_ERR_UNSUPPORTED, "B=%d exceeds %d", B, ATTN_MAX_BATCH);
    if (tile_keys <= 0 || num_ctas <= 0) return fail(ATTN_ERR_SHAPE, "tile_keys and num_ctas must be positive");
    if (num_ctas > attn::kMaxCtas) return fail(ATTN_ERR_UNSUPPORTED, "num_ctas=%d exceeds %d", num_ctas, attn::kMaxCtas);
    LeanPlan plan;
    int st = build_plan(seqlens, B, KH, tile_keys, -1, &plan);
    if (st != ATTN_OK) return st;
    int P = num_ctas;
    if (plan.N > 0 && P > plan.N) P = (int)plan.N;
    plan.P = P;
    *N_out = plan.N;
    *P_out = P;
    if (cta_tile_begin)
        for (int c = 0; c <= P; ++c) cta_tile_begin[c] = plan.N > 0 ? plan_cta_begin(plan, c) : 0;
    if (seg_tile_begin) {
        for (int b = 0; b < B; ++b) {
            const int nb = plan_tiles_per_segment(plan, b);
            for (int kh = 0; kh < KH; ++kh) seg_tile_begin[b * KH + kh] = plan.tile_prefix[b] + (int64_t)kh * nb;
        }
        seg_tile_begin[B * KH] = plan.N;
    }
    return ATTN_OK;
}

int attn_prefill_causal(const void *q, const void *k, const void *v, int B, int ISL, int Hq, int KH, int Hsz,
                        void *out, hipStream_t stream) {
    g_last_error.clear();
    if (!q || !k || !v || !out) return fail(ATTN_ERR_NULL, "q, k, v and out must be non-NULL");
    if (B <= 0 || ISL < 0 || Hq <= 0 || KH <= 0)
        return fail(ATTN_ERR_SHAPE, "B, Hq, KH must be positive and ISL non-negative");
    if (Hq % KH != 0) return fail(ATTN_ERR_SHAPE, "Hq=%d is not a multiple of KH=%d", Hq, KH);
    if (Hsz != 64 && Hsz != 128 && Hsz != 256)
        return fail(ATTN_ERR_UNSUPPORTED, "prefill supports Hsz=64, 128 and 256 (got %d)", Hsz);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(ATTN_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
    if (ISL == 0) return ATTN_OK;
    const float scale_log2 = (1.0f / sqrtf((float)Hsz)) * 1.4426950408889634f;
    hipError_t e = attn::launch_prefill_causal(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                                               static_cast<const uint16_t *>(v), static_cast<uint16_t *>(out), B,
                                               ISL, Hq, KH, Hsz, scale_log2, stream);
    if (e != hipSuccess) return fail_hip(e, "prefill kernel launch");
    return ATTN_OK;
}

int attn_hbm_copy_probe(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    g_last_error.clear();
    if (!src || !dst) return fail(ATTN_ERR_NULL, "src and dst must be non-NULL");
    if (bytes % 16 != 0) return fail(ATTN_ERR_SHAPE, "bytes=%zu is not a multiple of 16", bytes);
    if (!aligned16(src) || !aligned16(dst)) return fail(ATTN_ERR_ALIGN, "src and dst must be 16-byte aligned");
    hipError_t e = attn::launch_copy_probe(src, dst, bytes, stream);
    if (e != hipSuccess) return fail_hip(e, "copy probe launch");
    return ATTN_OK;
}

int attn_hbm_read_probe(const void *src, size_t bytes, void *sink, hipStream_t stream) {
    g_last_error.clear();
    if (!src || !sink) return fail(ATTN_ERR_NULL, "src and sink must be non-NULL");
    if (bytes % 16 != 0) return fail(ATTN_ERR_SHAPE, "bytes=%zu is not a multiple of 16", bytes);
    if (!aligned16(src) || !aligned16(sink)) return fail(ATTN_ERR_ALIGN, "src and sink must be 16-byte aligned");
    hipError_t e = attn::launch_read_probe(src, bytes, sink, stream);
    if (e != hipSuccess) return fail_hip(e, "read probe launch");
    return ATTN_OK;
}

int attn_device_info(int *num_cus, int *lds_bytes_per_cu) {
    g_last_error.clear();
    if (!num_cus || !lds_bytes_per_cu) return fail(ATTN_ERR_NULL, "outputs must be non-NULL");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    e = hipDeviceGetAttribute(num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute(MultiprocessorCount)");
    e = hipDeviceGetAttribute(lds_bytes_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute(MaxSharedMemoryPerMultiprocessor)");
    return ATTN_OK;
}

int attn_release(void) {
    g_last_error.clear();
    std::lock_guard<std::mutex> lock(g_mu);
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    int st = ATTN_OK;
    for (auto &kv : g_ws) {
        if (!kv.second.ptr) continue;
        if ((e = hipSetDevice(kv.first.first)) == hipSuccess) e = hipDeviceSynchronize();
        if (e == hipSuccess) e = hipFree(kv.second.ptr);
        if (e != hipSuccess) st = fail_hip(e, "releasing workspace");
        kv.second = Workspace();
    }
    g_ws.clear();
    (void)hipSetDevice(cur);
    return st;
}

}  // extern "C"
