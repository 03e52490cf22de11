// A decode step driven through the C ABI alone (include/mla_decode.h and
// the HIP runtime, no Python): the caller's view of libmla_decode.so.
//
//   abi_decode <input file> <output file>
//
// Input (little-endian): int32 batch, int32 kv_format (0 FP8, 1 MXFP4),
// int32 q_scale_mode (0 static, 1 absmax), float sm_scale, int32 kv_len[batch],
// then the bf16 bits of Q (batch, 16, 576) and of the latent cache
// (sum kv_len, 576). One query row per sequence.
//
// The program encodes the cache on the GPU (per-tensor absmax FP8, or
// MXFP4), plans, prepares the workspace, runs mla_decode_run_fused once on
// its own stream and writes: the bf16 bits of O (batch, 16, 512), the fp32
// LSE (batch, 16), the Q codes (batch, 16, 576) and the fp32 Q scale.
// Any failed call prints its status and exits with status 1.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "mla_decode.h"

namespace {

int fail(const char* what, int status) {
    std::fprintf(stderr, "%s: %s (%d)\n", what, mla_status_string(status), status);
    return 1;
}

int hip_fail(const char* what, hipError_t e) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
}

template <class T>
bool read_n(std::FILE* f, T* dst, size_t n) {
    return std::fread(dst, sizeof(T), n, f) == n;
}

// Device buffer released at scope exit.
struct Dev {
    void* p = nullptr;
    ~Dev() {
        if (p) (void)hipFree(p);
    }
};

}  // namespace

int main(int argc, char** argv) {
    if (argc != 3) {
        std::fprintf(stderr, "usage: %s <input> <output>\n", argv[0]);
        return 2;
    }
    std::FILE* in = std::fopen(argv[1], "rb");
    if (!in) return hip_fail("open input", hipErrorInvalidValue);
    int32_t batch = 0, fmt = 0, mode = 0;
    float sm_scale = 0.f;
    bool ok = read_n(in, &batch, 1) && read_n(in, &fmt, 1) && read_n(in, &mode, 1) &&
              read_n(in, &sm_scale, 1) && batch > 0 && (fmt == 0 || fmt == 1);
    std::vector<int32_t> kv_len(ok ? (size_t)batch : 0);
    ok = ok && read_n(in, kv_len.data(), kv_len.size());
    std::vector<int32_t> qo((size_t)batch + 1), kvp((size_t)batch + 1, 0);
    for (int32_t b = 0; ok && b < batch; ++b) {
        qo[(size_t)b + 1] = b + 1;
        kvp[(size_t)b + 1] = kvp[(size_t)b] + kv_len[(size_t)b];
    }
    const size_t rows = (size_t)kvp[(size_t)batch];
    const size_t nq = (size_t)batch * MLA_NUM_HEADS * MLA_QK_DIM;
    std::vector<uint16_t> q(nq), kv(rows * MLA_QK_DIM);
    ok = ok && read_n(in, q.data(), q.size()) && read_n(in, kv.data(), kv.size());
    std::fclose(in);
    if (!ok) {
        std::fprintf(stderr, "malformed input\n");
        return 2;
    }

    hipStream_t st = nullptr;
    hipError_t e = hipStreamCreate(&st);
    if (e != hipSuccess) return hip_fail("hipStreamCreate", e);

    // inputs and outputs
    Dev dq, dkv, dcodes, dscales, dkscale, dq8, dqs, dout, dlse, dqws, dws;
    const size_t code_bytes = rows * (fmt == 0 ? MLA_QK_DIM : MLA_QK_DIM / 2);
    const size_t nout = (size_t)batch * MLA_NUM_HEADS * MLA_V_DIM;
    if ((e = hipMalloc(&dq.p, nq * 2)) != hipSuccess ||
        (e = hipMalloc(&dkv.p, kv.size() * 2 + 16)) != hipSuccess ||
        (e = hipMalloc(&dcodes.p, code_bytes + 16)) != hipSuccess ||
        (e = hipMalloc(&dscales.p, rows * (MLA_QK_DIM / 32) + 16)) != hipSuccess ||
        (e = hipMalloc(&dkscale.p, 4)) != hipSuccess ||
        (e = hipMalloc(&dq8.p, nq)) != hipSuccess ||
        (e = hipMalloc(&dqs.p, 4)) != hipSuccess ||
        (e = hipMalloc(&dout.p, nout * 2)) != hipSuccess ||
        (e = hipMalloc(&dlse.p, (size_t)batch * MLA_NUM_HEADS * 4)) != hipSuccess)
        return hip_fail("hipMalloc", e);
    if ((e = hipMemcpy(dq.p, q.data(), nq * 2, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(dkv.p, kv.data(), kv.size() * 2, hipMemcpyHostToDevice)) != hipSuccess)
        return hip_fail("hipMemcpy", e);

    // the cache as the library encodes it
    int s;
    if (fmt == 0) {
        size_t qwb = 0;
        if ((s = mla_quant_fp8_workspace_size(kv.size(), &qwb))) return fail("quant size", s);
        if ((e = hipMalloc(&dqws.p, qwb ? qwb : 256)) != hipSuccess) return hip_fail("hipMalloc", e);
        if ((s = mla_quant_fp8(dkv.p, kv.size(), MLA_Q_SCALE_ABSMAX, (float*)dkscale.p, dcodes.p,
                               dqws.p, qwb ? qwb : 256, st)))
            return fail("mla_quant_fp8", s);
    } else if (rows) {
        if ((s = mla_encode_mxfp4(dkv.p, rows, dcodes.p, dscales.p, st)))
            return fail("mla_encode_mxfp4", s);
    }

    // plan, workspace, one fused step
    mla_plan_t plan = nullptr;
    if ((s = mla_decode_plan(qo.data(), kvp.data(), batch, MLA_NUM_HEADS, fmt, 0, 0, st, &plan)))
        return fail("mla_decode_plan", s);
    size_t wsb = 0;
    if ((s = mla_decode_workspace_size(plan, &wsb))) return fail("workspace size", s);
    if ((e = hipMalloc(&dws.p, wsb ? wsb : 256)) != hipSuccess) return hip_fail("hipMalloc", e);
    if ((s = mla_decode_workspace_init(plan, dws.p, wsb ? wsb : 256, st)))
        return fail("mla_decode_workspace_init", s);
    if (mode == MLA_Q_SCALE_STATIC) {
        const float qs = 6.0f / 448.0f;
        if ((e = hipMemcpyAsync(dqs.p, &qs, 4, hipMemcpyHostToDevice, st)) != hipSuccess)
            return hip_fail("hipMemcpyAsync", e);
    }
    s = mla_decode_run_fused(plan, dq.p, dq8.p, (float*)dqs.p, mode, dcodes.p,
                             fmt == 1 ? dscales.p : nullptr,
                             fmt == 0 ? (const float*)dkscale.p : nullptr, sm_scale, 0.0f, dws.p,
                             wsb ? wsb : 256, dout.p, (float*)dlse.p, st);
    if (s) return fail("mla_decode_run_fused", s);
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail("hipStreamSynchronize", e);
    mla_decode_plan_destroy(plan);

    std::vector<uint16_t> out(nout);
    std::vector<float> lse((size_t)batch * MLA_NUM_HEADS);
    std::vector<uint8_t> q8(nq);
    float qscale = 0.f;
    if ((e = hipMemcpy(out.data(), dout.p, nout * 2, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(lse.data(), dlse.p, lse.size() * 4, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(q8.data(), dq8.p, nq, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(&qscale, dqs.p, 4, hipMemcpyDeviceToHost)) != hipSuccess)
        return hip_fail("hipMemcpy", e);
    (void)hipStreamDestroy(st);

    std::FILE* o = std::fopen(argv[2], "wb");
    if (!o) return hip_fail("open output", hipErrorInvalidValue);
    ok = std::fwrite(out.data(), 2, out.size(), o) == out.size() &&
         std::fwrite(lse.data(), 4, lse.size(), o) == lse.size() &&
         std::fwrite(q8.data(), 1, q8.size(), o) == q8.size() &&
         std::fwrite(&qscale, 4, 1, o) == 1;
    std::fclose(o);
    if (!ok) {
        std::fprintf(stderr, "short write\n");
        return 1;
    }
    std::printf("abi_decode: batch %d format %d mode %d done\n", batch, fmt, mode);
    return 0;
}
