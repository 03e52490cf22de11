// Host-only driver for the sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer): the scheduler of libmla_decode.so (plan.cpp,
// no HIP) and every function of the C oracle (mla_oracle.c) run on valid,
// edge-case and invalid inputs, with their invariants checked. The test
// suite compiles it with -fsanitize=address,undefined and expects a clean
// exit: no sanitizer report and every check passing.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../mla_latent_kv_bf16_amd/csrc/plan.h"
#include "../../include/mla_decode.h"

extern "C" {
float orc_bf16_to_f32(uint16_t h);
double orc_e4m3fn_decode(uint8_t c);
uint8_t orc_e4m3fn_encode(float x);
double orc_e2m1_decode(uint8_t nib);
uint8_t orc_e2m1_encode(double x);
double orc_e8m0_decode(uint8_t b);
void orc_e4m3fn_encode_f32(const float* x, size_t n, uint8_t* out);
void orc_e2m1_encode_f64(const double* x, size_t n, uint8_t* out);
float orc_fp8_absmax_scale(const uint16_t* x, size_t n);
float orc_fp8_static_scale(void);
void orc_fp8_quantize(const uint16_t* x, size_t n, float scale, uint8_t* out);
void orc_mxfp4_encode_rows(const uint16_t* x, size_t rows, size_t cols, uint8_t* packed,
                           uint8_t* scales);
void orc_mxfp4_dequant_rows(const uint8_t* packed, const uint8_t* scales, size_t rows,
                            size_t cols, double* out);
void orc_attend(const double* q, const double* kd, int n, double sm_scale, double* o,
                double* lse);
void orc_attend_cap(const double* q, const double* kd, int n, double sm_scale, double cap,
                    double* o, double* lse);
void orc_lse_merge(int nsplit, const double* o_s, const double* lse_s, double* o, double* lse);
long long orc_mla_decode(int kv_format, const uint8_t* q8, float q_scale, const uint8_t* kv,
                         const uint8_t* kv_scales, float kv_scale, const int32_t* qo_indptr,
                         const int32_t* kv_indptr, int batch, const int32_t* seqs, int nsel,
                         const int32_t* kv_lo, const int32_t* kv_hi, double sm_scale,
                         double* out, double* lse);
long long orc_mla_decode_bf16(const uint16_t* q, const uint16_t* kv, const int32_t* qo_indptr,
                              const int32_t* kv_indptr, int batch, const int32_t* seqs, int nsel,
                              const int32_t* kv_lo, const int32_t* kv_hi, double sm_scale,
                              double cap, double* out, double* lse);
int orc_num_threads(void);
}

static int g_failures = 0;
#define CHECK(cond)                                                            \
    do {                                                                       \
        if (!(cond)) {                                                         \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++g_failures;                                                      \
        }                                                                      \
    } while (0)

static uint32_t g_rng = 12345u;
static uint32_t next_u32() {  // xorshift32
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 17;
    g_rng ^= g_rng << 5;
    return g_rng;
}
static float uniform() { return (float)(next_u32() >> 8) * (1.0f / 16777216.0f); }
static uint16_t bf16_of(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------- scheduler

static std::vector<int32_t> prefix(const std::vector<int64_t>& lens) {
    std::vector<int32_t> p(lens.size() + 1, 0);
    for (size_t i = 0; i < lens.size(); i++) p[i + 1] = (int32_t)(p[i] + lens[i]);
    return p;
}

// Every cache row of every query row lies in exactly one item; slots and
// merge entries are consistent; items stay within the per-format row cap.
static void check_schedule(const std::vector<int32_t>& qo, const std::vector<int32_t>& kv,
                           int32_t fmt, int32_t num_cus, int32_t max_splits) {
    const int32_t batch = (int32_t)qo.size() - 1;
    int32_t counts[3] = {0, 0, 0};
    int st = mla_decode_plan_host(qo.data(), kv.data(), batch, 16, fmt, num_cus, max_splits,
                                  nullptr, 0, nullptr, 0, counts);
    CHECK(st == 0);
    if (st) return;
    std::vector<int32_t> items((size_t)counts[0] * 4 + 4), merges((size_t)counts[1] * 4 + 4);
    CHECK(mla_decode_plan_host(qo.data(), kv.data(), batch, 16, fmt, num_cus, max_splits,
                               items.data(), counts[0], merges.data(), counts[1], counts) == 0);
    // a too-small array is rejected, not overrun
    if (counts[0] > 0)
        CHECK(mla_decode_plan_host(qo.data(), kv.data(), batch, 16, fmt, num_cus, max_splits,
                                   items.data(), counts[0] - 1, merges.data(), counts[1],
                                   counts) == 1);
    const int64_t cap = mla::max_item_tokens(fmt);
    const int32_t rows = qo[batch];
    // per query row: its causal range and the items covering it
    std::vector<int32_t> seq_of_row((size_t)rows), rb((size_t)rows), re((size_t)rows);
    for (int32_t b = 0; b < batch; b++) {
        const int32_t R = qo[b + 1] - qo[b];
        for (int32_t i = 0; i < R; i++) {
            const int32_t r = qo[b] + i;
            seq_of_row[r] = b;
            rb[r] = kv[b];
            re[r] = std::max<int32_t>(kv[b], kv[b + 1] - (R - 1 - i));
        }
    }
    std::vector<std::vector<std::pair<int32_t, int32_t>>> cover((size_t)rows);
    std::vector<int32_t> slot_seen((size_t)counts[2], 0);
    for (int32_t i = 0; i < counts[0]; i++) {
        const int32_t r = items[4 * i], lo = items[4 * i + 1], hi = items[4 * i + 2];
        const int32_t slot = items[4 * i + 3];
        CHECK(r >= 0 && r < rows);
        if (r < 0 || r >= rows) continue;
        CHECK(hi > lo && lo >= rb[r] && hi <= re[r]);
        CHECK((int64_t)hi - lo <= cap);
        CHECK(slot >= -1 && slot < counts[2]);
        if (slot >= 0 && slot < counts[2]) slot_seen[slot]++;
        cover[r].push_back({lo, hi});
    }
    for (int32_t r = 0; r < rows; r++) {
        auto& c = cover[r];
        std::sort(c.begin(), c.end());
        int32_t at = rb[r];
        for (auto& iv : c) {
            CHECK(iv.first == at);
            at = iv.second;
        }
        CHECK(at == re[r]);
    }
    for (int32_t s = 0; s < counts[2]; s++) CHECK(slot_seen[s] == 1);
    for (int32_t m = 0; m < counts[1]; m++) {
        const int32_t r = merges[4 * m], first = merges[4 * m + 1], n = merges[4 * m + 2];
        CHECK(r >= 0 && r < rows);
        CHECK(n == 0 || (first >= 0 && first + n <= counts[2]));
    }
    // the shared-row schedule (FP8 or MXFP4, 1-4 rows per sequence)
    if (mla::use_rows_schedule(qo.data(), batch, fmt, false, (size_t)counts[0], num_cus)) {
        mla::RowsSchedule rs;
        mla::build_rows_schedule(qo.data(), kv.data(), batch, num_cus, max_splits, &rs);
        int64_t covered = 0;
        for (const auto& it : rs.items) {
            CHECK(it.kv_end > it.kv_begin && it.kv_end - it.kv_begin <= cap);
            covered += it.kv_end - it.kv_begin;
        }
        CHECK(covered == kv[batch]);
    }
}

static void scheduler_cases() {
    const int32_t fmts[3] = {MLA_KV_FP8_E4M3FN, MLA_KV_MXFP4, MLA_KV_BF16};
    const std::vector<std::vector<int64_t>> shapes = {
        {}, {0}, {1}, {31, 32, 33}, {1000, 0, 4097}, {5, 9000, 40, 700, 0, 3000},
        {4000000, 9000001, 33}, {8192, 8192, 8192, 8192}};
    const int32_t reqs[][2] = {{0, 0}, {256, 0}, {1, 0}, {256, 1}, {7, -3}, {256, -64},
                               {256, -2000}, {3, 5}};
    for (const auto& lens : shapes)
        for (int32_t fmt : fmts)
            for (const auto& rq : reqs) {
                std::vector<int32_t> qo(lens.size() + 1);
                for (size_t i = 0; i <= lens.size(); i++) qo[i] = (int32_t)i;
                check_schedule(qo, prefix(lens), fmt, rq[0], rq[1]);
            }
    // query rows: 1-4 per sequence (shared-row schedule) and more
    {
        const std::vector<int64_t> lens = {100, 3, 0, 2048, 7};
        const std::vector<int32_t> q_lens[] = {{1, 2, 3, 4, 1}, {5, 1, 1, 9, 2}, {1, 1, 1, 1, 1}};
        for (const auto& ql : q_lens) {
            std::vector<int32_t> qo(ql.size() + 1, 0);
            for (size_t i = 0; i < ql.size(); i++) qo[i + 1] = qo[i] + ql[i];
            for (int32_t fmt : fmts) check_schedule(qo, prefix(lens), fmt, 256, 0);
            check_schedule(qo, prefix(lens), MLA_KV_FP8_E4M3FN, 256, -3);
        }
    }
    // rejected inputs, with no output written
    int32_t counts[3] = {-7, -7, -7};
    const int32_t qo2[3] = {0, 1, 2}, kv_dec[3] = {0, 5, 3}, kv_bad0[3] = {1, 5, 9};
    const int32_t kv_ok[3] = {0, 5, 9}, qo_dec[3] = {0, 2, 1};
    CHECK(mla_decode_plan_host(qo2, kv_dec, 2, 16, 0, 0, 0, nullptr, 0, nullptr, 0, counts) == 1);
    CHECK(mla_decode_plan_host(qo2, kv_bad0, 2, 16, 0, 0, 0, nullptr, 0, nullptr, 0, counts) == 1);
    CHECK(mla_decode_plan_host(qo_dec, kv_ok, 2, 16, 0, 0, 0, nullptr, 0, nullptr, 0, counts) == 1);
    CHECK(mla_decode_plan_host(qo2, kv_ok, 2, 8, 0, 0, 0, nullptr, 0, nullptr, 0, counts) == 2);
    CHECK(mla_decode_plan_host(qo2, kv_ok, 2, 16, 3, 0, 0, nullptr, 0, nullptr, 0, counts) == 2);
    CHECK(mla_decode_plan_host(nullptr, kv_ok, 2, 16, 0, 0, 0, nullptr, 0, nullptr, 0, counts) == 1);
    CHECK(mla_decode_plan_host(qo2, kv_ok, -1, 16, 0, 0, 0, nullptr, 0, nullptr, 0, counts) == 1);
    CHECK(counts[0] == -7);
    // a bf16 range needing more than 512 items of 2^21 rows
    const int32_t qo1[2] = {0, 1}, kv_huge[2] = {0, (1 << 30) + 1};
    CHECK(mla_decode_plan_host(qo1, kv_huge, 1, 16, MLA_KV_BF16, 0, 0, nullptr, 0, nullptr, 0,
                               counts) == 2);
    CHECK(mla_decode_plan_host(qo1, kv_huge, 1, 16, MLA_KV_FP8_E4M3FN, 0, 1, nullptr, 0, nullptr,
                               0, counts) == 0);
    CHECK(counts[0] == 257);
}

// ------------------------------------------------------------------- oracle

static void oracle_cases() {
    CHECK(orc_num_threads() >= 1);
    // codecs over every bf16 value and every code
    std::vector<uint16_t> all(65536);
    for (uint32_t i = 0; i < 65536; i++) all[i] = (uint16_t)i;
    std::vector<float> allf(65536);
    for (uint32_t i = 0; i < 65536; i++) allf[i] = orc_bf16_to_f32(all[i]);
    std::vector<uint8_t> codes(65536);
    orc_e4m3fn_encode_f32(allf.data(), allf.size(), codes.data());
    for (uint32_t i = 0; i < 65536; i++) {
        if (std::isnan(allf[i])) CHECK(codes[i] == 0x7F);
        else CHECK((codes[i] & 0x7F) != 0x7F);
    }
    for (int c = 0; c < 256; c++) {
        const double v = orc_e4m3fn_decode((uint8_t)c);
        if ((c & 0x7F) == 0x7F) CHECK(std::isnan(v));
        else CHECK(orc_e4m3fn_encode((float)v) == (uint8_t)c);
        CHECK(std::isnan(orc_e8m0_decode((uint8_t)c)) == (c == 0xFF));
    }
    for (int c = 0; c < 16; c++) CHECK(orc_e2m1_encode(orc_e2m1_decode((uint8_t)c)) == c);
    std::vector<double> xs(1000);
    for (auto& x : xs) x = (uniform() - 0.5) * 20.0;
    std::vector<uint8_t> nib(xs.size());
    orc_e2m1_encode_f64(xs.data(), xs.size(), nib.data());
    for (size_t i = 0; i < xs.size(); i++) CHECK(nib[i] < 16);
    // quantiser: zero, finite, NaN and infinite tensors; empty tensor
    std::vector<uint16_t> x(3 * 16 * 576);
    for (auto& v : x) v = bf16_of((uniform() - 0.5f) * 6.0f);
    std::vector<uint8_t> q8(x.size());
    const float s = orc_fp8_absmax_scale(x.data(), x.size());
    CHECK(std::isfinite(s) && s > 0.0f);
    orc_fp8_quantize(x.data(), x.size(), s, q8.data());
    orc_fp8_quantize(x.data(), x.size(), orc_fp8_static_scale(), q8.data());
    CHECK(orc_fp8_absmax_scale(x.data(), 0) == 1e-12f / 448.0f);
    std::vector<uint16_t> xn = x;
    xn[77] = 0x7FC1;  // NaN
    CHECK(std::isnan(orc_fp8_absmax_scale(xn.data(), xn.size())));
    xn[77] = 0x7F80;  // +inf
    CHECK(std::isinf(orc_fp8_absmax_scale(xn.data(), xn.size())));
    // MXFP4 rows, with zero, NaN and infinite blocks
    std::vector<uint16_t> kvb(9 * 576);
    for (auto& v : kvb) v = bf16_of((uniform() - 0.5f) * 4.0f);
    for (int j = 0; j < 32; j++) kvb[32 + j] = 0;
    kvb[2 * 576 + 5] = 0x7FC0;
    kvb[3 * 576 + 600 % 576] = 0xFF80;
    std::vector<uint8_t> packed(9 * 288), scales(9 * 18);
    orc_mxfp4_encode_rows(kvb.data(), 9, 576, packed.data(), scales.data());
    CHECK(scales[1] == 0 && scales[2 * 18] == 0xFF && scales[3 * 18 + 0] == 0xFF);
    std::vector<double> dq(9 * 576);
    orc_mxfp4_dequant_rows(packed.data(), scales.data(), 9, 576, dq.data());
    CHECK(std::isnan(dq[2 * 576]) && std::isfinite(dq[0]));
    // attention and merge, including empty ranges and a soft cap
    std::vector<double> q(576), kd(40 * 576), o(512), o2(512);
    for (auto& v : q) v = uniform() - 0.5;
    for (auto& v : kd) v = uniform() - 0.5;
    double lse = 0, lse2 = 0;
    orc_attend(q.data(), kd.data(), 0, 1.0 / 24, o.data(), &lse);
    CHECK(lse == -INFINITY && o[0] == 0.0);
    orc_attend(q.data(), kd.data(), 40, 1.0 / 24, o.data(), &lse);
    orc_attend_cap(q.data(), kd.data(), 40, 1.0 / 24, 1e30, o2.data(), &lse2);
    CHECK(std::fabs(lse - lse2) < 1e-9);
    std::vector<double> os(3 * 512), ls(3);
    orc_attend(q.data(), kd.data(), 13, 1.0 / 24, os.data(), &ls[0]);
    orc_attend(q.data(), kd.data() + 13 * 576, 27, 1.0 / 24, os.data() + 512, &ls[1]);
    orc_attend(q.data(), kd.data(), 0, 1.0 / 24, os.data() + 1024, &ls[2]);
    orc_lse_merge(3, os.data(), ls.data(), o2.data(), &lse2);
    CHECK(std::fabs(lse - lse2) < 1e-12);
    for (int d = 0; d < 512; d++) CHECK(std::fabs(o[d] - o2[d]) < 1e-12);
    orc_lse_merge(0, os.data(), ls.data(), o2.data(), &lse2);
    CHECK(lse2 == -INFINITY);
    // full decodes: ragged sequences, query rows, selected sequences, split ranges
    const int32_t qo[5] = {0, 1, 3, 3, 7};
    const int32_t kvp[5] = {0, 50, 53, 53, 120};
    std::vector<uint16_t> qb(7 * 16 * 576);
    for (auto& v : qb) v = bf16_of(uniform() - 0.5f);
    std::vector<uint8_t> qc(qb.size());
    const float qs = orc_fp8_absmax_scale(qb.data(), qb.size());
    orc_fp8_quantize(qb.data(), qb.size(), qs, qc.data());
    std::vector<uint16_t> kb(120 * 576);
    for (auto& v : kb) v = bf16_of(uniform() - 0.5f);
    std::vector<uint8_t> kc(kb.size());
    const float ks = orc_fp8_absmax_scale(kb.data(), kb.size());
    orc_fp8_quantize(kb.data(), kb.size(), ks, kc.data());
    std::vector<uint8_t> kp(120 * 288), kscl(120 * 18);
    orc_mxfp4_encode_rows(kb.data(), 120, 576, kp.data(), kscl.data());
    std::vector<double> out(7 * 16 * 512), lo(7 * 16);
    CHECK(orc_mla_decode(0, qc.data(), qs, kc.data(), nullptr, ks, qo, kvp, 4, nullptr, 0,
                         nullptr, nullptr, 1.0 / 24, out.data(), lo.data()) == 7);
    CHECK(orc_mla_decode(1, qc.data(), qs, kp.data(), kscl.data(), 0.f, qo, kvp, 4, nullptr, 0,
                         nullptr, nullptr, 1.0 / 24, out.data(), lo.data()) == 7);
    const int32_t sel[2] = {3, 0}, klo[2] = {10, 0}, khi[2] = {60, 0};
    CHECK(orc_mla_decode(0, qc.data(), qs, kc.data(), nullptr, ks, qo, kvp, 4, sel, 2, klo, khi,
                         1.0 / 24, out.data(), lo.data()) == 5);
    const int32_t bad[1] = {9};
    CHECK(orc_mla_decode(0, qc.data(), qs, kc.data(), nullptr, ks, qo, kvp, 4, bad, 1, nullptr,
                         nullptr, 1.0 / 24, out.data(), lo.data()) == -1);
    CHECK(orc_mla_decode(2, qc.data(), qs, kc.data(), nullptr, ks, qo, kvp, 4, nullptr, 0,
                         nullptr, nullptr, 1.0 / 24, out.data(), lo.data()) == -1);
    CHECK(orc_mla_decode_bf16(qb.data(), kb.data(), qo, kvp, 4, nullptr, 0, nullptr, nullptr,
                              1.0 / 24, 30.0, out.data(), lo.data()) == 7);
}

int main() {
    scheduler_cases();
    oracle_cases();
    if (g_failures) {
        std::fprintf(stderr, "%d checks failed\n", g_failures);
        return 1;
    }
    std::printf("sanitizer driver: all checks passed\n");
    return 0;
}
