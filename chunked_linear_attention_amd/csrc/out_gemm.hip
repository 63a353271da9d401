// Output projection O = Y W_o with Y = U * (V_quad + V_lin) from the chunk
// kernel (wikillm "Method" step 4: O_g = [U_g * (V_quad_g + V_lin_g)] W_o;
// Su's post, "Mixed Chunking", final equation).  With a residual pointer the
// epilogue also adds the layer's shortcut in fp32 (the skip connection the
// listings add after each block: wikillm, FLASH block pseudocode).
//
// An NT GEMM: A = Y [M, e], B = W_o^T [d, e], K = e.
#include "gau_device.h"
#include "gau_launch.h"

namespace gau {
namespace {

constexpr int BM = 128, BN = 128;

template <typename T>
__global__ __launch_bounds__(256) void out_gemm_kernel(OutParams p) {
    extern __shared__ __align__(16) char lds[];
    using G = GemmNT<T, BM, BN>;
    constexpr int EB = Elem<T>::kBytes;
    const int ntiles = p.d / BN;
    const int nt = blockIdx.x % ntiles;
    const int mt = blockIdx.x / ntiles;
    const int m0 = mt * BM, n0 = nt * BN;
    const size_t pitch = (size_t)p.e * EB;
    const int rows_a = min(BM, p.M - m0);

    f32x4_t acc[G::MB][G::NB];
    G::run(acc, (const char*)p.Y + (size_t)m0 * pitch, pitch, rows_a, (const char*)p.W_o + (size_t)n0 * pitch, pitch,
           BN, p.e, lds);

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave >> 1, wn = wave & 1;
    __syncthreads();
    if (p.residual == nullptr) {
        constexpr int PITCH = BN * EB + 16;
        for_each_acc(acc, lane, [&](int r, int c, float v) {
            Elem<T>::put(lds + (wm * (BM / 2) + r) * PITCH + (wn * (BN / 2) + c) * EB, v);
        });
        __syncthreads();
        constexpr int VPR = BN * EB / 16;
        char* O = (char*)p.O;
        for (int idx = tid; idx < BM * VPR; idx += 256) {
            const int row = idx / VPR, v = idx % VPR;
            if (m0 + row < p.M)
                *(u32x4_t*)(O + ((size_t)(m0 + row) * p.d + n0) * EB + v * 16) =
                    *(const u32x4_t*)(lds + row * PITCH + v * 16);
        }
    } else {
        constexpr int PITCH = BN * 4 + 16;
        for_each_acc(acc, lane, [&](int r, int c, float v) {
            *(float*)(lds + (wm * (BM / 2) + r) * PITCH + (wn * (BN / 2) + c) * 4) = v;
        });
        __syncthreads();
        constexpr int VPR = BN * 4 / 16;
        float* O = (float*)p.O;
        for (int idx = tid; idx < BM * VPR; idx += 256) {
            const int row = idx / VPR, v = idx % VPR;
            if (m0 + row < p.M) {
                const size_t off = (size_t)(m0 + row) * p.d + n0 + v * 4;
                f32x4_t x = *(const f32x4_t*)(p.residual + off);
                x += *(const f32x4_t*)(lds + row * PITCH + v * 16);
                *(f32x4_t*)(O + off) = x;
            }
        }
    }
}

template <typename T>
hipError_t launch(const OutParams& p, hipStream_t st) {
    using G = GemmNT<T, BM, BN>;
    constexpr int STAGE = BM * (BN * 4 + 16);
    constexpr int LDS = G::LDS_BYTES > STAGE ? G::LDS_BYTES : STAGE;
    const int blocks = (p.d / BN) * ((p.M + BM - 1) / BM);
    hipError_t e = allow_lds(out_gemm_kernel<T>, LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(out_gemm_kernel<T>, dim3(blocks), dim3(256), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_out_gemm(const OutParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? launch<bf16>(p, st) : launch<float>(p, st);
}

}  // namespace gau
