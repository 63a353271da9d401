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
// Two kernels on the shared MFMA core: U and V with 256 x 256 tiles (the
// e/256 tiles of each section side by side along N, so a block's columns lie
// in one section and its epilogue branch is uniform), and Z with its four
// heads with 128 x 64 tiles (s is small, and a separate launch keeps the U/V
// grid a whole number of rounds over the 256 CUs for the usual widths).
// Tiles are assigned to XCDs in contiguous ranges.
#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {

namespace {

constexpr int BM = 256, BN = 256, WGM = 2, WGN = 4;

template <typename T>
struct ProjTile {
    using G = GemmCore<T, BM, BN, WGM, WGN>;
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int STAGE = (BM * (BN * EB + 16) > 160 * 1024 - 1024) ? BM / WGM * (BN * EB + 16)
                                                                           : BM * (BN * EB + 16);
    static constexpr int LDS = G::LDS_BYTES > STAGE ? G::LDS_BYTES : STAGE;
};

// U and V: 256 x 256 tiles; the e/256 tiles of U and of V side by side.
template <typename T>
__global__ __launch_bounds__(512) void proj_uv_kernel(ProjParams p) {
    extern __shared__ __align__(16) char lds[];
    using G = typename ProjTile<T>::G;
    constexpr int EB = Elem<T>::kBytes;
    const int ntu = p.e / BN;  // tiles per section
    const int ntiles = 2 * ntu;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
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

// Z = SiLU(X W_z) and its four heads: 128 features x 64 tokens per block
// (B*T/64 blocks fill the CUs), with a 4-stage copy ring: the K loop over d
// is a dependent chain of d/64 chunk copies per block, so several must be in
// flight at once.
constexpr int ZF = 128, ZT = 64, ZNS = 4;

template <typename T>
struct ZTile {
    using G = GemmCore<T, ZF, ZT, 2, 2, ZNS>;
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int STAGE = ZT * (ZF * EB + 16) > ZF * (ZT * EB + 16) ? ZT * (ZF * EB + 16)
                                                                          : ZF * (ZT * EB + 16);
    static constexpr int LDS = G::LDS_BYTES > STAGE ? G::LDS_BYTES : STAGE;
};

template <typename T>
__global__ __launch_bounds__(256) void proj_z_kernel(ProjParams p) {
    extern __shared__ __align__(16) char lds[];
    using G = typename ZTile<T>::G;
    constexpr int EB = Elem<T>::kBytes;
    const int nf = p.s / ZF;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int ft = bid % nf;
    const int mt = bid / nf;
    const int m0 = mt * ZT, f0 = ft * ZF;
    const size_t pitch = (size_t)p.d * EB;
    const int rows_x = min(ZT, p.M - m0);

    // acc rows = features of Z, columns = tokens
    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    G::run(acc, (const char*)p.W_z + (size_t)f0 * pitch, pitch, ZF, (const char*)p.X + (size_t)m0 * pitch, pitch,
           rows_x, p.d, lds);
    G::transform(acc, [](int, int, float v) { return silu(v); });

    // head h = Z * gamma[h] + beta[h]; heads 0..2 token-major, head 3 (K_lin)
    // feature-major
    constexpr int LDS = ZTile<T>::LDS;
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
hipError_t launch_z(const ProjParams& p, hipStream_t st) {
    constexpr int LDS = ZTile<T>::LDS;
    static_assert(LDS <= 160 * 1024, "Z projection LDS over budget");
    const int blocks = (p.s / ZF) * ((p.M + ZT - 1) / ZT);
    hipError_t e = allow_lds<proj_z_kernel<T>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(proj_z_kernel<T>, dim3(blocks), dim3(256), LDS, st, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_uv(const ProjParams& p, hipStream_t st) {
    constexpr int LDS = ProjTile<T>::LDS;
    static_assert(LDS <= 160 * 1024, "projection GEMM LDS over budget");
    const int blocks = 2 * (p.e / BN) * ((p.M + BM - 1) / BM);
    hipError_t e = allow_lds<proj_uv_kernel<T>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(proj_uv_kernel<T>, dim3(blocks), dim3(512), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_proj_z(const ProjParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? launch_z<bf16>(p, st) : launch_z<float>(p, st);
}

hipError_t launch_proj_uv(const ProjParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? launch_uv<bf16>(p, st) : launch_uv<float>(p, st);
}

}  // namespace gau
