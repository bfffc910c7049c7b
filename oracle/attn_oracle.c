/*
 * attn_oracle.c -- plain fp64 CPU reference for exact grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the test-suite, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or helper with the HIP path.
 *
 * What it computes (sources cited by page title and section heading; the
 * pages are Korean, headings are given as printed with an English gloss):
 *  - Attention is the exact (not approximate) softmax of scaled query-key
 *    scores applied to the values: page "장문 컨텍스트 추론을 위한 어텐션 공동
 *    설계" (aitrends.kr, "attention co-design"), section "FlashAttention과 GEMM
 *    모양" and glossary "용어 해설"; page "추론 최적화" (base.kaita.kr,
 *    "inference optimisation" lecture), section 6 "FlashAttention은 어디에
 *    들어가나" (exact, not approximate attention).
 *  - Grouped-query attention: G = Hq / KH query heads share one K/V head
 *    (page "필수 LLM 최적화 기법(2)" (synabreu.github.io), section 1-1;
 *    co-design page, section "그룹 크기(G)의 영향").  The pages do not say
 *    which query heads form a group; the reading used here is contiguous
 *    groups, kv head = h / G.
 *  - Decode: one query token per request attends to that request's whole KV
 *    cache (L_b keys); prefill: causal mask, query row i sees keys 0..i
 *    (lecture section 1 "프리필과 디코드"; top-left alignment is a reading).
 *  - The pages print no formula for the softmax scale; the caller passes it
 *    (1/sqrt(Hsz) by default upstream), so a scaled variant needs no new code.
 *  - Partial state and merge: a slice of the context keeps its own maximum,
 *    normaliser and weighted value sum, and slices are merged by rescaling to
 *    the common maximum (page "LeanAttention" digest (siliconandsystems.com),
 *    section "조각별로 합칠 수 있는 정확한 소프트맥스", exactly mergeable
 *    softmax).  Here the state is kept in the natural-exponent domain.
 *
 * Arithmetic: inputs are bf16 bit patterns (uint16), decoded exactly to double;
 * every score, exponential, sum and quotient is fp64.  Two passes per output
 * row (max, then weights), no online update, no tiling.
 *
 *  - FP8 KV cache (co-design page, TL;DR and checklist "체크리스트": shrink
 *    the KV state; FP8 is named among the compression options): K and V are
 *    stored as OCP 8-bit floats E4M3 (1 sign, 4 exponent bits with bias 7, 3
 *    mantissa bits, exponent field 0 = subnormals, S.1111.111 = NaN, no
 *    infinity) with one scale per tensor: the attended key is k_scale * K and
 *    the value v_scale * V.  Decoded exactly to double.
 *
 *  - Multi-token decode (lecture page, section 5 "추측 디코딩": the target model
 *    checks the gamma drafted positions at once, like a short prefill, and
 *    since decode is memory bound this costs little more than one token):
 *    query t of gamma, at position L_b - gamma + t, attends to keys
 *    0 .. L_b - gamma + t (the cache already holds the drafted tokens; a causal
 *    mask aligned to the end of the context, which is the reading taken here).
 *
 * Pins (tests/test_oracle.py): closed forms for one and two keys, q = 0 gives
 * the mean of V, constant V, V = identity gives the weights (rows sum to 1,
 * matched to scipy's softmax), key permutation and common key shift
 * invariance, a planted score near 200, merge of arbitrary splits, GQA equal
 * to MHA with repeated K/V, torch CPU scaled_dot_product_attention in fp64,
 * prefill row 0 = v_0; the E4M3 decoder on all 256 codes against torch's
 * float8_e4m3fn, and the FP8 decode against the bf16 decode on the same values.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the parallel loops below will use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* bf16 is the upper half of an IEEE-754 binary32; widening is exact. */
double oracle_bf16_to_f64(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

void oracle_bf16_decode(const uint16_t *src, double *dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_bf16_to_f64(src[i]);
}

/* score of query row qrow against key row krow, both Hsz long */
static double dot_scaled(const uint16_t *qrow, const uint16_t *krow, int Hsz, double scale) {
    double acc = 0.0;
    for (int d = 0; d < Hsz; ++d) acc += oracle_bf16_to_f64(qrow[d]) * oracle_bf16_to_f64(krow[d]);
    return scale * acc;
}

/*
 * softmax(scores) . V over keys [j0, j1) of one (b, kv-head) cache, written to
 * dst[Hsz].  Empty ranges give zeros.  Also returns (m, l) through the
 * optional pointers: m = max score, l = sum_j exp(s_j - m).
 */
static void attend_rows(const uint16_t *qrow, const uint16_t *kbase, const uint16_t *vbase,
                        int64_t j0, int64_t j1, int Hsz, double scale, int normalise,
                        double *dst, double *m_out, double *l_out) {
    for (int d = 0; d < Hsz; ++d) dst[d] = 0.0;
    if (j1 <= j0) {
        if (m_out) *m_out = -INFINITY;
        if (l_out) *l_out = 0.0;
        return;
    }
    int64_t n = j1 - j0;
    double *s = (double *)malloc((size_t)n * sizeof(double));
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = dot_scaled(qrow, kbase + (j0 + j) * Hsz, Hsz, scale);
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double w = exp(s[j] - m);
        l += w;
        const uint16_t *vrow = vbase + (j0 + j) * Hsz;
        for (int d = 0; d < Hsz; ++d) dst[d] += w * oracle_bf16_to_f64(vrow[d]);
    }
    if (normalise)
        for (int d = 0; d < Hsz; ++d) dst[d] /= l;
    free(s);
    if (m_out) *m_out = m;
    if (l_out) *l_out = l;
}

static int dims_ok(int B, int Hq, int KH, int Hsz) {
    return B > 0 && Hq > 0 && KH > 0 && Hsz > 0 && Hq % KH == 0;
}

/*
 * Decode attention.  q [B][Hq][Hsz], k/v [B][KH][S][Hsz] (bf16 bits),
 * seqlens[B] (each 0 <= L_b <= S), out [B][Hq][Hsz] fp64.
 * rows: optional list of flat (b*Hq + h) indices to compute (NULL = all);
 * rows not listed are left untouched.  Returns 0, or -1 on bad arguments.
 */
int oracle_decode_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const int32_t *seqlens, int B, int Hq, int KH, int Hsz, int64_t S,
                      double scale, const int64_t *rows, int64_t nrows, double *out) {
    if (!q || !k || !v || !seqlens || !out || !dims_ok(B, Hq, KH, Hsz) || S < 0) return -1;
    for (int b = 0; b < B; ++b)
        if (seqlens[b] < 0 || seqlens[b] > S) return -1;
    int G = Hq / KH;
    int64_t total = rows ? nrows : (int64_t)B * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < total; ++r) {
        int64_t bh = rows ? rows[r] : r;
        int b = (int)(bh / Hq), h = (int)(bh % Hq);
        int kh = h / G;
        const uint16_t *kb = k + ((int64_t)b * KH + kh) * S * Hsz;
        const uint16_t *vb = v + ((int64_t)b * KH + kh) * S * Hsz;
        attend_rows(q + bh * Hsz, kb, vb, 0, seqlens[b], Hsz, scale, 1, out + bh * Hsz, NULL, NULL);
    }
    return 0;
}

/*
 * Partial state of one (b, h) over keys [j0, j1): m = max score,
 * l = sum exp(s - m), o[Hsz] = sum exp(s - m) v (unnormalised).
 * Empty range: m = -inf, l = 0, o = 0.
 */
int oracle_partial_state_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             int B, int Hq, int KH, int Hsz, int64_t S, double scale,
                             int b, int h, int64_t j0, int64_t j1,
                             double *m, double *l, double *o) {
    if (!q || !k || !v || !m || !l || !o || !dims_ok(B, Hq, KH, Hsz)) return -1;
    if (b < 0 || b >= B || h < 0 || h >= Hq || j0 < 0 || j1 > S) return -1;
    int kh = h / (Hq / KH);
    const uint16_t *kb = k + ((int64_t)b * KH + kh) * S * Hsz;
    const uint16_t *vb = v + ((int64_t)b * KH + kh) * S * Hsz;
    attend_rows(q + ((int64_t)b * Hq + h) * Hsz, kb, vb, j0, j1, Hsz, scale, 0, o, m, l);
    return 0;
}

/*
 * Merge n partial states (m[i], l[i], o[i][Hsz]) of one output row:
 * M = max m_i, Lsum = sum l_i exp(m_i - M), out = sum o_i exp(m_i - M) / Lsum.
 * States with m = -inf contribute nothing; all empty gives zeros.
 */
int oracle_merge_states_f64(int n, const double *m, const double *l, const double *o,
                            int Hsz, double *out) {
    if (n < 0 || Hsz <= 0 || !out || (n > 0 && (!m || !l || !o))) return -1;
    double M = -INFINITY;
    for (int i = 0; i < n; ++i)
        if (m[i] > M) M = m[i];
    for (int d = 0; d < Hsz; ++d) out[d] = 0.0;
    if (M == -INFINITY) return 0;
    double Lsum = 0.0;
    for (int i = 0; i < n; ++i) {
        if (m[i] == -INFINITY) continue;
        double f = exp(m[i] - M);
        Lsum += l[i] * f;
        for (int d = 0; d < Hsz; ++d) out[d] += o[(int64_t)i * Hsz + d] * f;
    }
    for (int d = 0; d < Hsz; ++d) out[d] /= Lsum;
    return 0;
}

/*
 * Causal prefill.  q, out [B][Hq][ISL][Hsz]; k, v [B][KH][ISL][Hsz].
 * Row i of head h attends to keys 0..i of kv head h / G.
 * rows: optional list of flat ((b*Hq + h)*ISL + i) indices (NULL = all).
 */
int oracle_prefill_causal_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              int B, int ISL, int Hq, int KH, int Hsz, double scale,
                              const int64_t *rows, int64_t nrows, double *out) {
    if (!q || !k || !v || !out || !dims_ok(B, Hq, KH, Hsz) || ISL < 0) return -1;
    int G = Hq / KH;
    int64_t total = rows ? nrows : (int64_t)B * Hq * ISL;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < total; ++r) {
        int64_t idx = rows ? rows[r] : r;
        int64_t bh = idx / ISL;
        int64_t i = idx % ISL;
        int b = (int)(bh / Hq), h = (int)(bh % Hq);
        int kh = h / G;
        const uint16_t *kb = k + ((int64_t)b * KH + kh) * ISL * Hsz;
        const uint16_t *vb = v + ((int64_t)b * KH + kh) * ISL * Hsz;
        attend_rows(q + idx * Hsz, kb, vb, 0, i + 1, Hsz, scale, 1, out + idx * Hsz, NULL, NULL);
    }
    return 0;
}

/* OCP E4M3 (e4m3fn) code -> double, exactly. */
double oracle_fp8_e4m3_to_f64(uint8_t code) {
    int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);          /* subnormal: m/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7); /* normal: 1.m * 2^(e-7) */
    return sign ? -v : v;
}

/*
 * Decode attention over an FP8 E4M3 KV cache.  q [B][Hq][Hsz] bf16 bits;
 * k, v [B][KH][S][Hsz] E4M3 codes; key j of head kh is k_scale * decode(k),
 * value v_scale * decode(v).  Same two passes as oracle_decode_f64, on the
 * decoded values.  rows: optional list of flat (b*Hq + h) indices (NULL = all).
 */
int oracle_decode_fp8_f64(const uint16_t *q, const uint8_t *k, const uint8_t *v,
                          const int32_t *seqlens, int B, int Hq, int KH, int Hsz, int64_t S,
                          double scale, double k_scale, double v_scale,
                          const int64_t *rows, int64_t nrows, double *out) {
    if (!q || !k || !v || !seqlens || !out || !dims_ok(B, Hq, KH, Hsz) || S < 0) return -1;
    for (int b = 0; b < B; ++b)
        if (seqlens[b] < 0 || seqlens[b] > S) return -1;
    int G = Hq / KH;
    int64_t total = rows ? nrows : (int64_t)B * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < total; ++r) {
        int64_t bh = rows ? rows[r] : r;
        int b = (int)(bh / Hq), h = (int)(bh % Hq);
        int kh = h / G;
        int64_t L = seqlens[b];
        const uint8_t *kb = k + ((int64_t)b * KH + kh) * S * Hsz;
        const uint8_t *vb = v + ((int64_t)b * KH + kh) * S * Hsz;
        const uint16_t *qrow = q + bh * Hsz;
        double *dst = out + bh * Hsz;
        for (int d = 0; d < Hsz; ++d) dst[d] = 0.0;
        if (L == 0) continue;
        double *sc = (double *)malloc((size_t)L * sizeof(double));
        double m = -INFINITY;
        for (int64_t j = 0; j < L; ++j) {
            double acc = 0.0;
            for (int d = 0; d < Hsz; ++d)
                acc += oracle_bf16_to_f64(qrow[d]) * (k_scale * oracle_fp8_e4m3_to_f64(kb[j * Hsz + d]));
            sc[j] = scale * acc;
            if (sc[j] > m) m = sc[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < L; ++j) {
            double w = exp(sc[j] - m);
            l += w;
            for (int d = 0; d < Hsz; ++d) dst[d] += w * (v_scale * oracle_fp8_e4m3_to_f64(vb[j * Hsz + d]));
        }
        for (int d = 0; d < Hsz; ++d) dst[d] /= l;
        free(sc);
    }
    return 0;
}

/*
 * Multi-token decode.  q, out [B][Hq][gamma][Hsz]; k, v [B][KH][S][Hsz] (bf16 bits).
 * Row (b, h, t) attends keys 0 .. L_b - gamma + t of kv head h / G; a row whose
 * range is empty (L_b - gamma + t < 0, e.g. L_b = 0) is zero.
 * rows: optional list of flat ((b*Hq + h)*gamma + t) indices (NULL = all).
 */
int oracle_decode_multi_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const int32_t *seqlens, int B, int Hq, int KH, int Hsz, int64_t S,
                            int gamma, double scale, const int64_t *rows, int64_t nrows, double *out) {
    if (!q || !k || !v || !seqlens || !out || !dims_ok(B, Hq, KH, Hsz) || S < 0 || gamma < 1) return -1;
    for (int b = 0; b < B; ++b)
        if (seqlens[b] < 0 || seqlens[b] > S) return -1;
    int G = Hq / KH;
    int64_t total = rows ? nrows : (int64_t)B * Hq * gamma;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < total; ++r) {
        int64_t idx = rows ? rows[r] : r;
        int64_t bh = idx / gamma;
        int t = (int)(idx % gamma);
        int b = (int)(bh / Hq), h = (int)(bh % Hq);
        int kh = h / G;
        int64_t last = (int64_t)seqlens[b] - gamma + t;  /* last visible key */
        const uint16_t *kb = k + ((int64_t)b * KH + kh) * S * Hsz;
        const uint16_t *vb = v + ((int64_t)b * KH + kh) * S * Hsz;
        attend_rows(q + idx * Hsz, kb, vb, 0, last + 1 > 0 ? last + 1 : 0, Hsz, scale, 1, out + idx * Hsz,
                    NULL, NULL);
    }
    return 0;
}

