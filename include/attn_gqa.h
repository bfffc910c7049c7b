/*
 * attn_gqa.h -- C ABI of the MI355X (gfx950) grouped-query attention library.
 *
 * The library computes exact softmax attention forward for grouped-query
 * attention (GQA): G = Hq / KH query heads share one K/V head, query head h
 * reads K/V head h / G (contiguous groups).  Sources, cited by page title and
 * section heading:
 *   - "장문 컨텍스트 추론을 위한 어텐션 공동 설계" (aitrends.kr, attention
 *     co-design), sections "프리필과 디코드의 차이" (decode reads the KV cache
 *     from HBM and is memory bound; prefill is a large matmul), "FlashAttention과
 *     GEMM 모양" (fused QK^T -> online softmax (running max and sum) -> PV over
 *     streamed K/V tiles) and "그룹 크기(G)의 영향";
 *   - "필수 LLM 최적화 기법(2)" (synabreu.github.io), section 1-1 (MHA, MQA,
 *     GQA; Llama-3 uses 32 query heads over 8 K/V heads);
 *   - "LeanAttention" digest (siliconandsystems.com), sections "조각별로 합칠 수
 *     있는 정확한 소프트맥스" (partial (max, sum, weighted V) states merged by
 *     rescaling to the common max) and "하드웨어에 맞춘 작업 단위" (tile count
 *     from total work and compute-unit count; resident CTAs take the next tile).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     memory) unless the argument says "host".  The caller owns every tensor;
 *     the library never frees caller memory.
 *   - bf16 means IEEE-754 binary32 truncated to its upper 16 bits (the
 *     bfloat16 storage format); tensors are dense and row-major in the stated
 *     dimension order.  Tensor pointers must be 16-byte aligned.
 *   - Calls are asynchronous on `stream` (0 = the null stream).  Argument
 *     errors are detected and returned synchronously before anything is
 *     enqueued; the call then has no effect.
 *   - Return value: ATTN_OK (0) or a negative ATTN_ERR_* code.  A readable
 *     message for the most recent failure on the calling thread is available
 *     from attn_last_error().  No C++ exception crosses this interface.
 *   - Numerics: bf16 inputs, fp32 accumulation; the softmax is evaluated with
 *     exp2 and the scale multiplied by log2(e).  Results do not depend on the
 *     work split beyond fp32 rounding.  NaN/Inf inputs are outside the contract.
 */
#ifndef ATTN_GQA_H
#define ATTN_GQA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,        /* a required pointer is NULL */
    ATTN_ERR_SHAPE = -2,       /* inconsistent sizes (B <= 0, Hq % KH != 0, L_b < 0 or > stride, ...) */
    ATTN_ERR_UNSUPPORTED = -3, /* valid but not implemented (Hsz not in {64,128,256}, too many query columns,
                                  B > 256, ...) */
    ATTN_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned */
    ATTN_ERR_WORKSPACE = -5,   /* caller workspace too small */
    ATTN_ERR_HIP = -6          /* a HIP runtime call failed; see attn_last_error() */
};

/* Largest batch the decode planner accepts (its plan travels in kernel arguments). */
#define ATTN_MAX_BATCH 256
/* Query columns one decode workgroup holds: the G = Hq / KH query heads of a kv
 * head times q_len drafted tokens.  G * q_len <= ATTN_MAX_COLUMNS, and
 * G * q_len * Hsz <= ATTN_MAX_COLUMN_ELEMS (64 columns at Hsz 64 or 128, 32 at
 * Hsz 256): every column's output accumulator stays in registers while K and V
 * stream past, so one pass over the cache serves all of them. */
#define ATTN_MAX_COLUMNS 64
#define ATTN_MAX_COLUMN_ELEMS 8192
/* Largest number of persistent decode workgroups (num_ctas). */
#define ATTN_MAX_CTAS 4096
/* Bytes at the start of a decode workspace that hold the merge counters
 * (one arrival counter per partial slot). */
#define ATTN_DECODE_COUNTER_BYTES 32768
/* Bytes after the counters that hold a plan built on the device (device seqlens). */
#define ATTN_DECODE_PLAN_BYTES 8192

/*
 * attn_decode -- one decode step of GQA attention (query length 1).
 *
 *   q        bf16 [B][Hq][Hsz]          query of the new token of each request
 *   k_cache  bf16 [B][KH][S][Hsz]       keys; request b uses rows 0..L_b-1
 *   v_cache  bf16 [B][KH][S][Hsz]       values, same layout
 *   seqlens  HOST int32 [B]             L_b, context length of request b
 *                                       (0 <= L_b; L_b = 0 yields a zero row)
 *   out      fp32 [B][Hq][Hsz]          softmax(q k^T / sqrt(Hsz)) v per head
 *   S (the cache capacity per (b, kv head)) is max_b L_b: the cache is packed
 *   to the longest request.  Use attn_decode_ex for any other capacity.
 *
 * The context of every (request, kv head) is cut into LeanTiles of T keys; the
 * tiles of the whole batch are numbered globally and split evenly over all
 * resident workgroups, each of which keeps the G query heads of a group
 * together.  A head split across workgroups leaves one partial (max, sum, O)
 * state per workgroup, merged by rescaling to the common max.  When a head is
 * split over at most 16 workgroups, the one that finishes last merges it
 * inside the same kernel; heads split over more (long contexts over few kv
 * heads) are merged by a second, short kernel on the same stream, which
 * spreads the reading of their partials over many workgroups.
 * The library owns the partial-state buffer (one per device and stream, grown
 * on demand with hipMalloc and zero-filled on the stream, freed by
 * attn_release); calls on the same stream are ordered, calls that share a
 * stream from several host threads at once are not supported.
 */
int attn_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *seqlens,
                int B, int Hq, int KH, int Hsz, float *out, hipStream_t stream);

/*
 * Work schedules of the decode kernel (attn_decode_args.schedule).
 *   ATTN_SCHEDULE_STREAM_K    LeanTiles numbered over the whole batch and split
 *                             evenly over num_ctas persistent workgroups (the
 *                             LeanAttention digest, "조각별로 합칠 수 있는 정확한
 *                             소프트맥스" and "하드웨어에 맞춘 작업 단위").
 *   ATTN_SCHEDULE_FIXED_SPLIT every (request, kv head) context cut into
 *                             num_splits near-equal chunks, one workgroup each
 *                             (the FlashDecoding-style baseline the digest compares
 *                             against, section "모양이 다른 프리필과 디코드");
 *                             num_splits = 0 fills every resident slot once.
 *   ATTN_SCHEDULE_AUTO        the selector: one workgroup per (request, kv head),
 *                             with no reduction, when running the segments whole
 *                             in launch order on the resident workgroups ends no
 *                             later than stream-K's even share of the tiles (many
 *                             segments of similar length); stream-K otherwise,
 *                             and always with device seqlens, whose lengths the
 *                             host cannot see (section "런타임 선택 정책").
 * All schedules compute the same function; results differ only by fp32 rounding.
 */
#define ATTN_SCHEDULE_AUTO 0
#define ATTN_SCHEDULE_STREAM_K 1
#define ATTN_SCHEDULE_FIXED_SPLIT 2

/*
 * Element types of the KV cache (attn_decode_args.kv_dtype).
 *   ATTN_KV_BF16      bf16 K and V, as in attn_decode.
 *   ATTN_KV_FP8_E4M3  one byte per element, OCP 8-bit float E4M3 (1 sign bit, 4
 *                     exponent bits with bias 7, 3 mantissa bits, exponent 0 =
 *                     subnormals, S.1111.111 = NaN, no infinity); the attended key
 *                     is k_scale * K and the value v_scale * V.  Halves the bytes a
 *                     decode step streams (co-design page: TL;DR and checklist, FP8
 *                     among the ways to shrink the KV state).  Every E4M3 value is
 *                     a bf16 value, so the kernel widens K and V exactly and the
 *                     rest of the computation is the bf16 path's.
 */
#define ATTN_KV_BF16 0
#define ATTN_KV_FP8_E4M3 1

/* Full-control decode.  Fields not listed keep the attn_decode meaning. */
typedef struct attn_decode_args {
    const void *q;            /* bf16 [B][Hq][Hsz] */
    const void *k_cache;      /* [B][KH][kv_stride][Hsz], element type kv_dtype */
    const void *v_cache;      /* same layout and type as k_cache */
    const int32_t *seqlens;   /* HOST int32 [B], 0 <= L_b <= kv_stride (DEVICE with seqlens_on_device) */
    float *out;               /* fp32 [B][Hq][Hsz] */
    int B, Hq, KH, Hsz;
    int64_t kv_stride;        /* cache capacity S per (b, kv head); 0 = max_b L_b */
    float scale;              /* softmax scale; <= 0 selects 1/sqrt(Hsz) */
    void *workspace;          /* optional device buffer for partial states (NULL = library-owned);
                                 its first ATTN_DECODE_COUNTER_BYTES bytes must be zero before its
                                 first use, and every completed call leaves them zero again.  One
                                 workspace serves one call at a time: calls that may overlap
                                 (different streams) need different workspaces. */
    size_t workspace_bytes;   /* its size; must be >= attn_decode_workspace_bytes(...) */
    int tile_keys;            /* LeanTile size T in keys; 0 = library default */
    int num_ctas;             /* stream-K: number of persistent workgroups P, <= ATTN_MAX_CTAS;
                                 0 = the library's choice: every resident slot once, or
                                 k times (k = floor(B*KH / slots), at most 4) when the
                                 (request, kv head) segments outnumber the slots at
                                 least twice.  Must be 0 for the fixed split. */
    hipEvent_t ev_tiles_begin;/* optional timing event, bound to the start of the decode tile
                                 kernel (launched through hipExtLaunchKernel, so no marker
                                 packet is added to the stream) */
    hipEvent_t ev_tiles_end;  /* optional timing event, bound to the end of the call's last decode
                                 kernel: the merge kernel of heads split over more than 16
                                 workgroups when one runs, the tile kernel otherwise.  With
                                 device seqlens the plan kernel in front is not included. */
    int schedule;             /* ATTN_SCHEDULE_*; 0 = AUTO */
    int num_splits;           /* fixed split: chunks per (request, kv head); 0 = fill the GPU once.
                                 With more than one split, B*KH*num_splits <= ATTN_MAX_CTAS. */
    int kv_dtype;             /* ATTN_KV_*; 0 = bf16 */
    float k_scale;            /* FP8 only: key scale (<= 0 selects 1); must be 0 or 1 for bf16 */
    float v_scale;            /* FP8 only: value scale (<= 0 selects 1); must be 0 or 1 for bf16 */
    /* Paged KV cache (block tables; "필수 LLM 최적화 기법(2)" section 3, PagedAttention).
     * With a table, k_cache/v_cache are pools [num_blocks][KH][block_size][Hsz] and
     * row j of request b lives in block block_table[b][j / block_size] at in-block row
     * j % block_size; kv_stride must be 0 and every L_b <= max_blocks_per_seq *
     * block_size.  Entries past a request's last block are never read; ids outside
     * [0, num_blocks) are clamped into the pool (wrong numbers, never a bad access). */
    const int32_t *block_table; /* DEVICE int32 [B][max_blocks_per_seq], or NULL = contiguous cache */
    int block_size;           /* tokens per block: a power of two >= 16 */
    int max_blocks_per_seq;   /* row stride of block_table */
    int num_blocks;           /* blocks in each pool */
    /* Multi-token decode (speculative verification; lecture page "추론 최적화", section 5:
     * the target model checks gamma drafted tokens at once).  With q_len = gamma > 1, q
     * and out are [B][Hq][gamma][Hsz], the cache already holds the drafted tokens as
     * the last gamma of each context, and query t attends keys 0 .. L_b - gamma + t.
     * Needs G * gamma within the column limits (ATTN_MAX_COLUMNS, ATTN_MAX_COLUMN_ELEMS)
     * and L_b = 0 or L_b >= gamma. */
    int q_len;                /* 0 or 1 = one query token per request */
    /* Device seqlens.  Nonzero: `seqlens` is a DEVICE int32 [B] that the call never
     * reads on the host.  A one-workgroup kernel builds the LeanTile plan on the
     * device in front of the decode kernel, so the call needs no synchronisation
     * and can be captured in a graph whose replays see new lengths.  kv_stride must
     * then be given (> 0) unless a block table is; each L_b is clamped into
     * [0, kv_stride] (or the table's capacity) on the device, and a nonzero L_b below
     * q_len gives undefined rows for that request.  Such a call always needs the
     * workspace, and with num_ctas = 0 it launches the default workgroup count (those
     * beyond the tile count exit at once).  A caller-owned workspace makes the call
     * allocation-free. */
    int seqlens_on_device;
    /* Optional DEVICE fp32 [B][Hq][q_len] (NULL = none): log2 of each output row's softmax
     * denominator, sum_j 2^(s_j), with s_j the score in log2 units (scale * k_scale * log2 e
     * times q.k_j); -inf for a row that sees no key.  With it, decodes over disjoint key
     * ranges of the same rows (the KV sequence split across devices) merge exactly through
     * attn_merge_shards. */
    float *out_lse;
} attn_decode_args;

int attn_decode_ex(const attn_decode_args *args, hipStream_t stream);

/*
 * attn_decode_noalloc -- attn_decode_ex for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It calls no hipMalloc, hipFree or other allocating routine.
 *
 *   args   as for attn_decode_ex, except that workspace must be NULL and
 *          workspace_bytes 0 (ATTN_ERR_SHAPE otherwise): the partial states,
 *          merge counters and device-built plan live in a fixed device array of
 *          ATTN_NOALLOC_SCRATCH_BYTES inside the library, one copy per device,
 *          held from the library's load until the process ends.
 *   stream as for attn_decode_ex; the same kernels run, plus one small kernel
 *          that clears the counters the call uses.
 * Returns ATTN_ERR_WORKSPACE, before anything is enqueued, when the call needs
 * more partial-state memory than the array holds (attn_decode_multi_workspace_bytes
 * gives the need); calls that split no head need none.  All calls on one device
 * share its array: calls that may overlap on one device (different streams, or
 * several host threads on one stream) race and give wrong results; calls
 * ordered on one stream do not.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_decode_noalloc(const attn_decode_args *args, hipStream_t stream);

/*
 * Bytes of workspace attn_decode_ex needs for these sizes when it runs with
 * `num_ctas` workgroups: ATTN_DECODE_COUNTER_BYTES of merge counters,
 * ATTN_DECODE_PLAN_BYTES for a plan built on the device, then 2 partial slots
 * per workgroup of (G*Hsz + 2G) floats rounded up to 16 bytes.
 *   num_ctas > 0   exactly that many workgroups: a stream-K call with that
 *                  num_ctas, or a fixed split with num_ctas = B*KH*num_splits.
 *   num_ctas = 0   enough for every call that leaves the count to the library on
 *                  the current device (this query initialises the HIP runtime):
 *                  the larger of the stream-K default and the fixed split's
 *                  default, so any schedule (AUTO included) with num_ctas = 0 and
 *                  num_splits = 0 fits.
 * Returns 0 for unsupported sizes (and when the device query fails).
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int KH, int Hsz, int num_ctas);

/* The same for multi-token decode with q_len query tokens per request (slots hold
 * G * q_len states); q_len <= 1 gives attn_decode_workspace_bytes. */
size_t attn_decode_multi_workspace_bytes(int B, int Hq, int KH, int Hsz, int q_len, int num_ctas);

/*
 * attn_merge_shards -- merges S decode outputs of the same rows computed over
 * disjoint key ranges (the KV sequence split across devices or calls, each run
 * with out_lse):
 *   outs     DEVICE fp32 [S][rows][Hsz]   normalised rows of each shard
 *   lses     DEVICE fp32 [S][rows]        their out_lse (-inf: the shard saw no key)
 *   out      DEVICE fp32 [rows][Hsz]      sum_s outs[s] 2^(lses[s] - M) / sum_s 2^(lses[s] - M),
 *                                         M = max_s lses[s]; zero when every lse is -inf
 *   lse_out  optional DEVICE fp32 [rows]  the merged lse, for a further merge
 * The rescale-and-sum of the LeanAttention digest's section "조각별로 합칠 수
 * 있는 정확한 소프트맥스", over shard outputs instead of partial states.  Hsz is
 * a multiple of 4; outs and out 16-byte aligned.
 */
int attn_merge_shards(const float *outs, const float *lses, int S, int64_t rows, int Hsz, float *out, float *lse_out,
                      hipStream_t stream);

/*
 * attn_prefill_causal -- causal GQA attention over a whole prompt.
 *
 *   q    bf16 [B][Hq][ISL][Hsz]
 *   k    bf16 [B][KH][ISL][Hsz]   (the decode cache layout, capacity ISL)
 *   v    bf16 [B][KH][ISL][Hsz]
 *   out  bf16 [B][Hq][ISL][Hsz]   row i = softmax over keys 0..i (top-left
 *                                 causal mask), scale 1/sqrt(Hsz), fp32
 *                                 accumulation, rounded to bf16 once at the end
 * QK^T runs on bf16 MFMA; the PV product runs on fp16 MFMA with V converted
 * bf16 -> fp16 and
 * the softmax weights rounded to fp16.  The conversion of V is exact for bf16 values
 * in fp16's normal range (2^-14 <= |v| < 65504) and for zero; smaller nonzero |v| lose
 * mantissa bits (an absolute error below 2^-24 per element); |v| >= 65504 is outside
 * the contract.
 * Source: co-design page, sections "프리필과 디코드의 차이" and "FlashAttention과
 * GEMM 모양" (prefill is the large, compute-bound matmul form of the same
 * fused kernel).  Hsz must be 64, 128 or 256 (ATTN_ERR_UNSUPPORTED otherwise).
 */
int attn_prefill_causal(const void *q, const void *k, const void *v, int B, int ISL, int Hq, int KH,
                        int Hsz, void *out, hipStream_t stream);

/*
 * attn_decode_plan -- the host half of the LeanTile planner, exposed for
 * inspection (no GPU use).  For the given HOST seqlens it returns the number
 * of tiles N and, if the arrays are non-NULL:
 *   cta_tile_begin  int64 [P+1]   CTA c owns global tiles [begin[c], begin[c+1])
 *   seg_tile_begin  int64 [B*KH+1] segment s = b*KH + kh owns tiles
 *                                  [seg_tile_begin[s], seg_tile_begin[s+1])
 * `num_ctas` must be in [1, ATTN_MAX_CTAS] here; the effective P is
 * min(num_ctas, N) and is written to *P_out.
 */
int attn_decode_plan(const int32_t *seqlens, int B, int KH, int tile_keys, int num_ctas,
                     int64_t *N_out, int *P_out, int64_t *cta_tile_begin, int64_t *seg_tile_begin);

/*
 * attn_hbm_copy_probe -- plain device-to-device copy of `bytes` (a multiple of
 * 16) from src to dst with 16-byte vector loads and stores.  A measurement
 * reference of known traffic: it calibrates the HBM byte counters and gives
 * the practical streaming ceiling next to the 8 TB/s peak.
 */
int attn_hbm_copy_probe(const void *src, void *dst, size_t bytes, hipStream_t stream);

/*
 * attn_hbm_read_probe -- reads `bytes` (a multiple of 16) from src once with
 * 16-byte vector loads and folds them into a value that is written to the
 * 4-byte device word `sink` only when it equals a fixed sentinel.  Its time
 * is the practical streaming read rate, the ceiling the decode kernel chases.
 */
int attn_hbm_read_probe(const void *src, size_t bytes, void *sink, hipStream_t stream);

/* Compute units and LDS bytes per compute unit of the current device. */
int attn_device_info(int *num_cus, int *lds_bytes_per_cu);

/* Frees every library-owned workspace on every device (synchronises them). */
int attn_release(void);

/* Static description of a status code. */
const char *attn_status_string(int status);

/* Message for the most recent failure on the calling thread ("" if none). */
const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_GQA_H */
