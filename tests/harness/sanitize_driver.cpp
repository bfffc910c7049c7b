// Host driver for the sanitizer build: runs the fp64 oracle (attn_oracle.c) and
// the LeanTile plan harness (plan_harness.cpp, which includes the kernels'
// plan header) over seeded small cases, including empty and one-key contexts,
// under AddressSanitizer and UndefinedBehaviorSanitizer.  It checks nothing
// numerically (the pytest pins do that): a clean exit means no out-of-bounds
// access, use of uninitialised heap memory or undefined arithmetic was hit.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <random>
#include <vector>

#include "plan_harness.cpp"

extern "C" {
int oracle_decode_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *seqlens, int B, int Hq,
                      int KH, int Hsz, int64_t S, double scale, const int64_t *rows, int64_t nrows, double *out);
int oracle_partial_state_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int Hq, int KH, int Hsz,
                             int64_t S, double scale, int b, int h, int64_t j0, int64_t j1, double *m, double *l,
                             double *o);
int oracle_merge_states_f64(int n, const double *m, const double *l, const double *o, int Hsz, double *out);
int oracle_prefill_causal_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int ISL, int Hq, int KH,
                              int Hsz, double scale, const int64_t *rows, int64_t nrows, double *out);
int oracle_decode_fp8_f64(const uint16_t *q, const uint8_t *k, const uint8_t *v, const int32_t *seqlens, int B, int Hq,
                          int KH, int Hsz, int64_t S, double scale, double k_scale, double v_scale,
                          const int64_t *rows, int64_t nrows, double *out);
int oracle_decode_multi_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *seqlens, int B,
                            int Hq, int KH, int Hsz, int64_t S, int gamma, double scale, const int64_t *rows,
                            int64_t nrows, double *out);
}

static std::vector<uint16_t> bf16_normal(size_t n, std::mt19937 &g) {
    std::normal_distribution<float> d(0.f, 1.f);
    std::vector<uint16_t> r(n);
    for (auto &x : r) {
        const float f = d(g);
        uint32_t w;
        memcpy(&w, &f, 4);
        x = (uint16_t)(w >> 16);
    }
    return r;
}

static int fail(const char *what) {
    fprintf(stderr, "%s returned an error\n", what);
    return 1;
}

int main() {
    std::mt19937 g(2024);
    const int B = 3, Hq = 8, KH = 2, Hsz = 64, S = 37, gamma = 3;
    const int32_t sl[B] = {0, 1, S};
    const double scale = 0.125;
    auto q = bf16_normal((size_t)B * Hq * Hsz, g);
    auto qm = bf16_normal((size_t)B * Hq * gamma * Hsz, g);
    auto k = bf16_normal((size_t)B * KH * S * Hsz, g), v = bf16_normal((size_t)B * KH * S * Hsz, g);
    std::vector<uint8_t> k8(k.size()), v8(v.size());
    for (size_t i = 0; i < k8.size(); ++i) k8[i] = (uint8_t)(g() & 0x7e), v8[i] = (uint8_t)(g() & 0xfe);
    std::vector<double> out((size_t)B * Hq * gamma * Hsz);
    if (oracle_decode_f64(q.data(), k.data(), v.data(), sl, B, Hq, KH, Hsz, S, scale, nullptr, 0, out.data()))
        return fail("oracle_decode_f64");
    const int64_t rows[3] = {0, 9, B * Hq - 1};
    if (oracle_decode_f64(q.data(), k.data(), v.data(), sl, B, Hq, KH, Hsz, S, scale, rows, 3, out.data()))
        return fail("oracle_decode_f64 (rows)");
    if (oracle_decode_fp8_f64(q.data(), k8.data(), v8.data(), sl, B, Hq, KH, Hsz, S, scale, 0.5, 2.0, nullptr, 0,
                              out.data()))
        return fail("oracle_decode_fp8_f64");
    const int32_t slm[B] = {gamma, gamma + 1, S};
    if (oracle_decode_multi_f64(qm.data(), k.data(), v.data(), slm, B, Hq, KH, Hsz, S, gamma, scale, nullptr, 0,
                                out.data()))
        return fail("oracle_decode_multi_f64");
    double m[4], l[4];
    std::vector<double> o(4 * Hsz), merged(Hsz);
    const int64_t cuts[5] = {0, 5, 6, 20, S};
    for (int i = 0; i < 4; ++i)
        if (oracle_partial_state_f64(q.data(), k.data(), v.data(), B, Hq, KH, Hsz, S, scale, 2, 5, cuts[i],
                                     cuts[i + 1], &m[i], &l[i], o.data() + i * Hsz))
            return fail("oracle_partial_state_f64");
    if (oracle_merge_states_f64(4, m, l, o.data(), Hsz, merged.data())) return fail("oracle_merge_states_f64");
    const int ISL = 29;
    auto qp = bf16_normal((size_t)Hq * ISL * Hsz, g);
    auto kp = bf16_normal((size_t)KH * ISL * Hsz, g), vp = bf16_normal((size_t)KH * ISL * Hsz, g);
    std::vector<double> op((size_t)Hq * ISL * Hsz);
    if (oracle_prefill_causal_f64(qp.data(), kp.data(), vp.data(), 1, ISL, Hq, KH, Hsz, scale, nullptr, 0, op.data()))
        return fail("oracle_prefill_causal_f64");

    // planner: random ragged batches, tile sizes, CTA counts and split counts
    for (int it = 0; it < 300; ++it) {
        const int b = 1 + g() % 40, kh = 1 + g() % 8, T = 16 << (g() % 5), P = 1 + g() % 300;
        const int splits = it % 3 == 0 ? 1 + g() % 5 : 0;
        std::vector<int32_t> lens(b);
        for (auto &x : lens) x = g() % 5 == 0 ? 0 : (int32_t)(g() % 5000);
        const int64_t n = harness_pieces(lens.data(), b, kh, T, P, splits, nullptr, 0);
        std::vector<int64_t> pieces(8 * (size_t)(n > 0 ? n : 1));
        harness_pieces(lens.data(), b, kh, T, P, splits, pieces.data(), n);
        std::vector<int32_t> lo((size_t)b * kh), cnt((size_t)b * kh), slots(4096);
        harness_segment_ctas(lens.data(), b, kh, T, P, splits, 16, lo.data(), cnt.data());
        for (int s = 0; s < b * kh; ++s) harness_merge_slots(lens.data(), b, kh, T, P, splits, s, slots.data(), 4096);
        harness_whole_segments_makespan(lens.data(), b, kh, T, 1 + (int)(g() % 600));
    }
    puts("sanitized oracle and planner runs: clean");
    return 0;
}
