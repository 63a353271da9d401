// Output projection O = Y W_o with Y = U * (V_quad + V_lin) from the chunk
// kernel (wikillm "Method" step 4: O_g = [U_g * (V_quad_g + V_lin_g)] W_o;
// Su's post, "Mixed Chunking", final equation).  With a residual pointer the
// epilogue also adds the layer's shortcut in fp32 (the skip connection the
// listings add after each block: wikillm, FLASH block pseudocode).
//
// An NT GEMM on the shared core: A = Y [M, e], B = W_o^T [d, e], K = e,
// 256 x 256 output tiles (d need only be a multiple of 128: the last column
// tile may be half full).
#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {
namespace {

constexpr int BM = 256, BN = 256, WGM = 2, WGN = 4;

template <typename T>
struct OutTile {
    using G = GemmCore<T, BM, BN, WGM, WGN>;
    // fp32 staging (residual output or fp32 layer) in two passes of 128 rows
    static constexpr int STAGE = BM / WGM * (BN * 4 + 16);
    static constexpr int LDS = G::LDS_BYTES > STAGE ? G::LDS_BYTES : STAGE;
};

template <typename T>
__global__ __launch_bounds__(512) void out_gemm_kernel(OutParams p) {
    extern __shared__ __align__(16) char lds[];
    using G = typename OutTile<T>::G;
    constexpr int EB = Elem<T>::kBytes;
    const int ntiles = (p.d + BM - 1) / BM;  // feature tiles (acc rows)
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = bid % ntiles;
    const int mt = bid / ntiles;
    const int m0 = mt * BN, n0 = nt * BM;  // token offset, feature offset
    const size_t pitch = (size_t)p.e * EB;
    const int rows_y = min(BN, p.M - m0);
    const int rows_w = min(BM, p.d - n0);

    // acc = tile^T: rows = output features (W_o^T rows), columns = tokens, so
    // the packed epilogue writes run along the token-major rows of O.
    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    G::run(acc, (const char*)p.W_o + (size_t)n0 * pitch, pitch, rows_w, (const char*)p.Y + (size_t)m0 * pitch, pitch,
           rows_y, p.e, lds);

    constexpr int LDS = OutTile<T>::LDS;
    const int M = p.M, d = p.d;
    auto ident = [](int, int, float v) { return v; };
    if (p.residual == nullptr) {
        char* O = (char*)p.O;
        G::template store_packed<T>(acc, lds, LDS, ident, [&](int tok, int feat) -> char* {
            const int m = m0 + tok, n = n0 + feat;
            return (m < M && n < d) ? O + ((size_t)m * d + n) * EB : nullptr;
        });
    } else {
        // O = residual + Y W_o (fp32): stage the product, then add the residual
        // while storing (each 16-byte vector is read and written by one thread).
        float* O = (float*)p.O;
        const float* R = p.residual;
        G::template store_packed<float>(
            acc, lds, LDS, ident,
            [&](int tok, int feat) -> char* {
                const int m = m0 + tok, n = n0 + feat;
                return (m < M && n < d) ? (char*)(O + (size_t)m * d + n) : nullptr;
            },
            [&](char* dp, const u32x4_t& v) {
                const size_t off = (size_t)((float*)dp - O);
                f32x4_t x = *(const f32x4_t*)(R + off);
                x += __builtin_bit_cast(f32x4_t, v);
                *(f32x4_t*)dp = x;
            });
    }
}

template <typename T>
hipError_t launch(const OutParams& p, hipStream_t st) {
    constexpr int LDS = OutTile<T>::LDS;
    static_assert(LDS <= 160 * 1024, "output GEMM LDS over budget");
    const int blocks = ((p.d + BM - 1) / BM) * ((p.M + BN - 1) / BN);
    hipError_t e = allow_lds(out_gemm_kernel<T>, LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(out_gemm_kernel<T>, dim3(blocks), dim3(512), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_out_gemm(const OutParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? launch<bf16>(p, st) : launch<float>(p, st);
}

}  // namespace gau
