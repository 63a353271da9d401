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
// Tiling: 256 x 256 output tiles (GemmCore, 8 waves), the tiles of each
// section (U: e/256, V: e/256, Z: one tile of s <= 256 columns) laid side by
// side along N; tiles are assigned to XCDs in contiguous ranges.  A block's
// columns lie in exactly one section, so its epilogue branch is uniform.
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

template <typename T>
__global__ __launch_bounds__(512) void proj_gemm_kernel(ProjParams p) {
    extern __shared__ __align__(16) char lds[];
    using G = typename ProjTile<T>::G;
    constexpr int EB = Elem<T>::kBytes;
    const int ntu = p.e / BN;              // tiles per U or V section
    const int ntiles = 2 * ntu + 1;        // + one Z tile
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = bid % ntiles;
    const int mt = bid / ntiles;
    const int m0 = mt * BM;
    int section, c0, rows_b;
    const char* w;
    if (nt < ntu) {
        section = 0; c0 = nt * BN; w = (const char*)p.W_u; rows_b = BN;
    } else if (nt < 2 * ntu) {
        section = 1; c0 = (nt - ntu) * BN; w = (const char*)p.W_v; rows_b = BN;
    } else {
        section = 2; c0 = 0; w = (const char*)p.W_z; rows_b = p.s;
    }
    const size_t pitch = (size_t)p.d * EB;
    const int rows_x = min(BM, p.M - m0);
    const char* xt = (const char*)p.X + (size_t)m0 * pitch;
    const char* wt = w + (size_t)c0 * pitch;

    // Operand order per section, so that the accumulator's columns run along
    // the rows of the stored layout (packed epilogue writes): U and the heads
    // are token-major, so the weights are the A operand and the tokens the B
    // operand (acc = tile^T); Vt is feature-major, so the tokens are A.
    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    const bool tok_a = section == 1;
    G::run(acc, tok_a ? xt : wt, pitch, tok_a ? rows_x : rows_b, tok_a ? wt : xt, pitch, tok_a ? rows_b : rows_x,
           p.d, lds);
    G::transform(acc, [](int, int, float v) { return silu(v); });

    constexpr int LDS = ProjTile<T>::LDS;
    const int M = p.M, T_ = p.T;
    auto ident = [](int, int, float v) { return v; };
    if (section == 0) {
        // acc rows = features, columns = tokens
        char* U = (char*)p.U;
        G::template store_packed<T>(acc, lds, LDS, ident, [&](int tok, int feat) -> char* {
            const int m = m0 + tok;
            return m < M ? U + ((size_t)m * p.e + c0 + feat) * EB : nullptr;
        });
    } else if (section == 1) {
        // acc rows = tokens, columns = features
        char* Vt = (char*)p.Vt;
        G::template store_packed<T>(acc, lds, LDS, ident, [&](int feat, int tok) -> char* {
            const int m = m0 + tok;
            if (m >= M) return nullptr;
            const int b = m / T_, t = m - b * T_;
            return Vt + (((size_t)b * p.e + c0 + feat) * T_ + t) * EB;
        });
    } else {
        // acc rows = features of Z (s of them valid), columns = tokens.
        // head h = Z * gamma[h] + beta[h]; heads 0..2 token-major, head 3
        // (K_lin) feature-major.
        const int s = p.s;
        for (int h = 0; h < 4; ++h) {
            const float* gam = p.scale + h * s;
            const float* bet = p.offset + h * s;
            auto val = [&](int feat, int, float z) { return feat < s ? z * gam[feat] + bet[feat] : 0.f; };
            if (h < 3) {
                char* dst = (char*)(h == 0 ? p.Qq : h == 1 ? p.Kq : p.Ql);
                G::template store_packed<T>(acc, lds, LDS, val, [&](int tok, int feat) -> char* {
                    const int m = m0 + tok;
                    return (m < M && feat < s) ? dst + ((size_t)m * s + feat) * EB : nullptr;
                });
            } else {
                char* Klt = (char*)p.Klt;
                G::template store<T, false>(acc, lds, LDS, val, [&](int feat, int tok) -> char* {
                    const int m = m0 + tok;
                    if (m >= M || feat >= s) return nullptr;
                    const int b = m / T_, t = m - b * T_;
                    return Klt + (((size_t)b * s + feat) * T_ + t) * EB;
                });
            }
        }
    }
}

template <typename T>
hipError_t launch(const ProjParams& p, hipStream_t st) {
    constexpr int LDS = ProjTile<T>::LDS;
    static_assert(LDS <= 160 * 1024, "projection GEMM LDS over budget");
    const int ntiles = 2 * (p.e / BN) + 1;
    const int m_tiles = (p.M + BM - 1) / BM;
    hipError_t e = allow_lds(proj_gemm_kernel<T>, LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(proj_gemm_kernel<T>, dim3(ntiles * m_tiles), dim3(512), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_proj_gemm(const ProjParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? launch<bf16>(p, st) : launch<float>(p, st);
}

}  // namespace gau
