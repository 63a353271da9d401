// Fused input projection of the FLASH layer: H = X [W_u | W_v | W_z], then
// U = SiLU(H_u), V = SiLU(H_v), Z = SiLU(H_z) and the four per-dimension
// scale+offset heads of Z, all in the GEMM epilogue.
//
// Pages: one dense layer of width 2e+s followed by SiLU and a split into U, V
// and the shared base (wikillm, FLASH block pseudocode, the Code 8 rewrite);
// SiLU on U, V and Z (Su's post, "Gated Attention"; wikillm "Paper vs code");
// Q and K as per-dimension affine maps of Z (Su's post, "Weak Attention");
// four heads, quadratic and linear Q/K (wikillm "Method", mixed chunk
// attention; papercache 3.2 "Preparation").
//
// Layout written (see the workspace layout in gau.h):
//   U [M, e] row-major; Vt [B, e, T] (V transposed per sequence, so the chunk
//   kernels read tokens contiguously); Q_quad, K_quad, Q_lin [M, s] row-major;
//   K_lin_t [B, s, T] transposed.  M = B*T.
//
// One launch, two kinds of blocks on the shared MFMA core.  The first
// (s/128) * ceil(M/256) blocks each form a 128-feature x 256-token tile of Z
// and write its four heads; the rest form the 256 x 256 tiles of U and V (the
// e/256 tiles of each section side by side along N, so a block's columns lie
// in one section and its epilogue branch is uniform).  The Z blocks are
// dispatched first and cost half a U/V tile each, so the launch is about an
// eighth of a round longer than U and V alone instead of a second launch of
// small, latency-bound blocks.  U/V tiles are assigned to XCDs in contiguous
// ranges.
#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {

namespace {

constexpr int BM = 256, BN = 256, WGM = 2, WGN = 4;  // U/V tiles, wave grid
constexpr int ZF = 128, ZT = 256;                    // Z tiles: features x tokens

template <typename T>
struct ProjTile {
    using G = GemmCore<T, BM, BN, WGM, WGN>;
    using GZ = GemmCore<T, ZF, ZT, WGM, WGN>;
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int STAGE = (BM * (BN * EB + 16) > 160 * 1024 - 1024) ? BM / WGM * (BN * EB + 16)
                                                                           : BM * (BN * EB + 16);
    static constexpr int CORE = G::LDS_BYTES > GZ::LDS_BYTES ? G::LDS_BYTES : GZ::LDS_BYTES;
    static constexpr int LDS = CORE > STAGE ? CORE : STAGE;
};

// U and V: one 256 x 256 tile (logical index bid over the U/V tiles).
template <typename T>
__device__ __forceinline__ void uv_tile(const ProjParams& p, int bid, char* lds) {
    using G = typename ProjTile<T>::G;
    constexpr int EB = Elem<T>::kBytes;
    const int ntu = p.e / BN;  // tiles per section
    const int ntiles = 2 * ntu;
    const int nt = bid % ntiles;
    const int mt = bid / ntiles;
    const int m0 = mt * BM;
    const bool is_v = nt >= ntu;
    const int c0 = (is_v ? nt - ntu : nt) * BN;
    const size_t pitch = (size_t)p.d * EB;
    const int rows_x = min(BM, p.M - m0);
    const char* xt = (const char*)p.X + (size_t)m0 * pitch;
    const char* wt = (const char*)(is_v ? p.W_v : p.W_u) + (size_t)c0 * pitch;

    // Operand order per section, so that the accumulator's columns run along
    // the rows of the stored layout (packed epilogue writes): U is token-major,
    // so the weights are the A operand and the tokens the B operand
    // (acc = tile^T); Vt is feature-major, so the tokens are A.
    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    G::run(acc, is_v ? xt : wt, pitch, is_v ? rows_x : BN, is_v ? wt : xt, pitch, is_v ? BN : rows_x, p.d, lds);
    G::transform(acc, [](int, int, float v) { return silu(v); });

    constexpr int LDS = ProjTile<T>::LDS;
    const int M = p.M, T_ = p.T;
    auto ident = [](int, int, float v) { return v; };
    if (!is_v) {
        // acc rows = features, columns = tokens
        char* U = (char*)p.U;
        G::template store_packed<T>(acc, lds, LDS, ident, [&](int tok, int feat) -> char* {
            const int m = m0 + tok;
            return m < M ? U + ((size_t)m * p.e + c0 + feat) * EB : nullptr;
        });
    } else {
        // acc rows = tokens, columns = features
        char* Vt = (char*)p.Vt;
        G::template store_packed<T>(acc, lds, LDS, ident, [&](int feat, int tok) -> char* {
            const int m = m0 + tok;
            if (m >= M) return nullptr;
            const int b = m / T_, t = m - b * T_;
            return Vt + (((size_t)b * p.e + c0 + feat) * T_ + t) * EB;
        });
    }
}

// Z = SiLU(X W_z) for 128 features x 256 tokens (tile index zb), and its four
// heads h = Z * gamma[h] + beta[h]: Q_quad, K_quad, Q_lin token-major, K_lin
// feature-major.
template <typename T>
__device__ __forceinline__ void z_tile(const ProjParams& p, int zb, char* lds) {
    using G = typename ProjTile<T>::GZ;
    constexpr int EB = Elem<T>::kBytes;
    const int nf = p.s / ZF;
    const int ft = zb % nf;
    const int mt = zb / nf;
    const int m0 = mt * ZT, f0 = ft * ZF;
    const size_t pitch = (size_t)p.d * EB;
    const int rows_x = min(ZT, p.M - m0);

    // acc rows = features of Z, columns = tokens
    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    G::run(acc, (const char*)p.W_z + (size_t)f0 * pitch, pitch, ZF, (const char*)p.X + (size_t)m0 * pitch, pitch,
           rows_x, p.d, lds);
    G::transform(acc, [](int, int, float v) { return silu(v); });

    constexpr int LDS = ProjTile<T>::LDS;
    const int M = p.M, T_ = p.T, s = p.s;
    for (int h = 0; h < 4; ++h) {
        const float* gam = p.scale + h * s + f0;
        const float* bet = p.offset + h * s + f0;
        auto val = [&](int feat, int, float z) { return z * gam[feat] + bet[feat]; };
        if (h < 3) {
            char* dst = (char*)(h == 0 ? p.Qq : h == 1 ? p.Kq : p.Ql);
            G::template store_packed<T>(acc, lds, LDS, val, [&](int tok, int feat) -> char* {
                const int m = m0 + tok;
                return m < M ? dst + ((size_t)m * s + f0 + feat) * EB : nullptr;
            });
        } else {
            char* Klt = (char*)p.Klt;
            G::template store<T, false>(acc, lds, LDS, val, [&](int feat, int tok) -> char* {
                const int m = m0 + tok;
                if (m >= M) return nullptr;
                const int b = m / T_, t = m - b * T_;
                return Klt + (((size_t)b * s + f0 + feat) * T_ + t) * EB;
            });
        }
    }
}

template <typename T>
__global__ __launch_bounds__(512) void proj_kernel(ProjParams p) {
    extern __shared__ __align__(16) char lds[];
    const int nz = (p.s / ZF) * ((p.M + ZT - 1) / ZT);
    const int b = blockIdx.x;
    if (b < nz)
        z_tile<T>(p, b, lds);
    else
        uv_tile<T>(p, xcd_remap(b - nz, gridDim.x - nz), lds);
}

template <typename T>
hipError_t launch_t(const ProjParams& p, hipStream_t st) {
    constexpr int LDS = ProjTile<T>::LDS;
    static_assert(LDS <= 160 * 1024, "projection LDS over budget");
    const int mtiles = (p.M + BM - 1) / BM;
    const int blocks = (p.s / ZF) * ((p.M + ZT - 1) / ZT) + 2 * (p.e / BN) * mtiles;
    hipError_t e = allow_lds<proj_kernel<T>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(proj_kernel<T>, dim3(blocks), dim3(512), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_proj(const ProjParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? launch_t<bf16>(p, st) : launch_t<float>(p, st);
}

}  // namespace gau
