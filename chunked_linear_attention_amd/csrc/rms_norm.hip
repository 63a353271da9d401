// Pre-norm of the layer stack: xn = x / sqrt(mean(x^2) + eps) per token row,
// written in the layer's element type.  The listings apply a norm before every
// block and add the shortcut after it (wikillm, FLASH block pseudocode); the
// norm's body (Code 5, LayerNorm / ScaleNorm) is missing from the pages, and
// ScaleNorm with its gain fixed at sqrt(d) is this RMS norm.
//
// One 256-thread block per row; each thread reduces strided 16-byte vectors,
// then a wave shuffle and an LDS step give the row's sum of squares.
#include "gau_device.h"
#include "gau_launch.h"

namespace gau {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void rms_norm_kernel(NormParams p) {
    __shared__ float part[4];
    const int row = blockIdx.x;
    const f32x4_t* x = (const f32x4_t*)(p.x + (size_t)row * p.d);
    const int nv = p.d / 4;
    float ss = 0.f;
    for (int v = threadIdx.x; v < nv; v += 256) {
        const f32x4_t a = x[v];
        ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    }
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = part[0] + part[1] + part[2] + part[3];
    const float inv = 1.0f / sqrtf(tot / (float)p.d + p.eps);
    constexpr int EB = Elem<T>::kBytes;
    char* out = (char*)p.xn + (size_t)row * p.d * EB;
    for (int v = threadIdx.x; v < nv; v += 256) {
        const f32x4_t a = x[v] * inv;
        char* o = out + (size_t)v * 4 * EB;
        Elem<T>::put(o + 0 * EB, a.x);
        Elem<T>::put(o + 1 * EB, a.y);
        Elem<T>::put(o + 2 * EB, a.z);
        Elem<T>::put(o + 3 * EB, a.w);
    }
}

template <typename T>
hipError_t launch(const NormParams& p, hipStream_t st) {
    hipLaunchKernelGGL(rms_norm_kernel<T>, dim3(p.M), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rms_norm(const NormParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? launch<bf16>(p, st) : launch<float>(p, st);
}

}  // namespace gau
