// Measurement aid: the bf16 MFMA rate the matrix cores sustain with operands
// in registers and no memory traffic (gau_probe_mfma in gau_probe.h).  The
// layer's kernels are measured against the published peak and against this.
#include "../../include/gau_probe.h"
#include "gau_device.h"

namespace gau {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* out) {
    const int lane = threadIdx.x;
    // operands that differ per lane (values are irrelevant to the timing)
    bf16x8_t a, b;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        a[t] = (__bf16)(0.001f * (float)((lane + t) & 15));
        b[t] = (__bf16)(0.002f * (float)((lane * 3 + t) & 7));
    }
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    if (s == -1234567.0f) out[0] = s;  // never true for these operands
}

}  // namespace
}  // namespace gau

extern "C" gau_status gau_probe_mfma(int blocks, int iters, float* out, void* stream) {
    if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 20)) return GAU_ERR_SHAPE;
    // at most 2^22 block-iterations (about 4.4 PFLOP, a few seconds of the
    // whole chip), so that no call queues an effectively endless kernel
    if ((int64_t)blocks * iters > ((int64_t)1 << 22)) return GAU_ERR_SHAPE;
    if (!out) return GAU_ERR_NULL;
    if (((uintptr_t)out & 15) != 0) return GAU_ERR_ALIGN;
    hipLaunchKernelGGL(gau::mfma_probe_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
    return hipGetLastError() == hipSuccess ? GAU_OK : GAU_ERR_HIP;
}
