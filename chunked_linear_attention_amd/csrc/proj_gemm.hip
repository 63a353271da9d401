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
// small, latency-bound blocks.  U/V tiles are assigned to XCDs so that
// tiles sharing operand rows share an L2: at e = 1536 each XCD takes half of
// the column tiles for a quarter of the token tiles, at e = 2048 a quarter of
// them for half of the token tiles; otherwise contiguous ranges (the 2e/256
// column tiles of one token tile together).
#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {

namespace {

constexpr int BM = 256, BN = 256, WGM = 2, WGN = 4;  // U/V tiles, wave grid
constexpr int ZF = 128, ZT = 256;                    // Z tiles: features x tokens
constexpr int ZHOSTS = 4;                            // U tiles that carry a Z slice

// ZR = 0: Z in tiles of its own; ZR = s / ZHOSTS: each of the first ZHOSTS U
// tiles of a token tile also forms ZR features of Z (the GEMM core's side
// product, sharing the tile's X chunks and B fragments).
template <typename T, int ZR>
struct ProjTile {
    using G = GemmCore<T, BM, BN, WGM, WGN, 2, ZR>;
    using GZ = GemmCore<T, ZF, ZT, WGM, WGN>;
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int STAGE = (BM * (BN * EB + 16) > 160 * 1024 - 1024) ? BM / WGM * (BN * EB + 16)
                                                                           : BM * (BN * EB + 16);
    static constexpr int CORE = G::LDS_BYTES > GZ::LDS_BYTES ? G::LDS_BYTES : GZ::LDS_BYTES;
    static constexpr int LDS = CORE > STAGE ? CORE : STAGE;
};

// Epilogue of a Z slice formed as a side product: ZR features f0.. of Z for the
// 256 tokens m0.. .  Applies SiLU and the four heads and stores Q_quad, K_quad,
// Q_lin (token-major) and K_lin_t (feature-major) through LDS, all four heads
// in one staging pass when they fit, else one head per pass.
template <typename T, int ZR, typename Side>
__device__ __forceinline__ void z_side_epilogue(const ProjParams& p, Side& sd, int m0, int f0, char* lds,
                                                int lds_bytes) {
    constexpr int EB = Elem<T>::kBytes;
    constexpr int ZMB = ZR / 32;
    constexpr int NT = WGM * WGN * kWave;
    constexpr int TP = ZR * EB + 16;  // token-major staging pitch
    constexpr int FP = BN * EB + 16;  // feature-major staging pitch
    constexpr int HEAD_T = BN * TP;   // bytes of one token-major head
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int wm = wave / WGN, wn = wave % WGN;
    const int c = lane & 31, h = lane >> 5;
    const int tok = wn * 64 + wm * 32 + c;  // B-tile column this lane's side outputs belong to
    const int M = p.M, T_ = p.T, s = p.s;
    const bool one_pass = 3 * HEAD_T + ZR * FP <= lds_bytes;
#pragma unroll
    for (int i = 0; i < ZMB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) sd.acc[i][r] = silu(sd.acc[i][r]);

    // stage head hd (token-major heads at hd * HEAD_T when one_pass, else at 0;
    // K_lin after the three token-major heads, or at 0)
    auto stage_head = [&](int hd, char* base) {
        const f32x4_t* gam = (const f32x4_t*)(p.scale + hd * s + f0);
        const f32x4_t* bet = (const f32x4_t*)(p.offset + hd * s + f0);
#pragma unroll
        for (int i = 0; i < ZMB; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int zr0 = i * 32 + 8 * g4 + 4 * h;  // four consecutive Z features
                const f32x4_t gm = gam[zr0 / 4], bt = bet[zr0 / 4];
                const float v0 = sd.acc[i][4 * g4 + 0] * gm.x + bt.x, v1 = sd.acc[i][4 * g4 + 1] * gm.y + bt.y;
                const float v2 = sd.acc[i][4 * g4 + 2] * gm.z + bt.z, v3 = sd.acc[i][4 * g4 + 3] * gm.w + bt.w;
                if (hd < 3) {
                    char* q = base + tok * TP + zr0 * EB;
                    if constexpr (EB == 2) {
                        *(u32x2_t*)q = u32x2_t{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                    } else {
                        *(f32x4_t*)q = f32x4_t{v0, v1, v2, v3};
                    }
                } else {
                    char* q = base + zr0 * FP + tok * EB;
                    Elem<T>::put(q, v0);
                    Elem<T>::put(q + FP, v1);
                    Elem<T>::put(q + 2 * FP, v2);
                    Elem<T>::put(q + 3 * FP, v3);
                }
            }
    };
    auto store_head = [&](int hd, const char* base) {
        if (hd < 3) {
            char* dst = (char*)(hd == 0 ? p.Qq : hd == 1 ? p.Kq : p.Ql);
            constexpr int VPR = ZR * EB / 16;  // 16-byte vectors per token row
            for (int idx = threadIdx.x; idx < BN * VPR; idx += NT) {
                const int t = idx / VPR, v = idx - t * VPR;
                const int m = m0 + t;
                if (m < M)
                    *(u32x4_t*)(dst + ((size_t)m * s + f0) * EB + v * 16) = *(const u32x4_t*)(base + t * TP + v * 16);
            }
        } else {
            char* Klt = (char*)p.Klt;
            constexpr int VPR = BN * EB / 16;  // 16-byte vectors per feature row
            constexpr int TPV = 16 / EB;       // tokens per vector
            for (int idx = threadIdx.x; idx < ZR * VPR; idx += NT) {
                const int zr = idx / VPR, v = idx - zr * VPR;
                const int m = m0 + v * TPV;
                if (m < M) {
                    const int b = m / T_, t = m - b * T_;
                    *(u32x4_t*)(Klt + (((size_t)b * s + f0 + zr) * T_ + t) * EB) =
                        *(const u32x4_t*)(base + zr * FP + v * 16);
                }
            }
        }
    };
    if (one_pass) {
        __syncthreads();
        for (int hd = 0; hd < 4; ++hd) stage_head(hd, lds + hd * HEAD_T);
        __syncthreads();
        for (int hd = 0; hd < 4; ++hd) store_head(hd, lds + hd * HEAD_T);
    } else {
        for (int hd = 0; hd < 4; ++hd) {
            __syncthreads();
            stage_head(hd, lds);
            __syncthreads();
            store_head(hd, lds);
        }
    }
}

// U and V: one 256 x 256 tile (logical index bid over the U/V tiles); with
// ZR > 0 the first ZHOSTS U tiles of each token tile also form a Z slice.
template <typename T, int ZR>
__device__ __forceinline__ void uv_tile(const ProjParams& p, int bid, char* lds) {
    using G = typename ProjTile<T, ZR>::G;
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
    typename G::Side sd;
    const bool side = ZR > 0 && !is_v && nt < ZHOSTS;
    bool ran = false;
    if constexpr (ZR > 0) {
        if (side) {  // block-uniform: the side product has a main loop of its own
            G::run_with_side(acc, sd, wt, pitch, BN, xt, pitch, rows_x, p.d,
                             (const char*)p.W_z + (size_t)(nt * ZR) * pitch, pitch, true, lds);
            ran = true;
        }
    }
    if (!ran)
        G::run(acc, is_v ? xt : wt, pitch, is_v ? rows_x : BN, is_v ? wt : xt, pitch, is_v ? BN : rows_x, p.d, lds);
    G::transform(acc, [](int, int, float v) { return silu(v); });

    constexpr int LDS = ProjTile<T, ZR>::LDS;
    const int M = p.M, T_ = p.T;
    auto ident = [](int, int, float v) { return v; };
    if (!is_v) {
        // acc rows = features, columns = tokens
        char* U = (char*)p.U;
        G::template store_packed<T>(acc, lds, LDS, ident, [&](int tok, int feat) -> char* {
            const int m = m0 + tok;
            return m < M ? U + ((size_t)m * p.e + c0 + feat) * EB : nullptr;
        });
        if constexpr (ZR > 0) {
            if (side) z_side_epilogue<T, ZR>(p, sd, m0, nt * ZR, lds, LDS);
        }
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
    using G = typename ProjTile<T, 0>::GZ;
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

    constexpr int LDS = ProjTile<T, 0>::LDS;
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

template <typename T, int ZR>
__global__ __launch_bounds__(512) void proj_kernel(ProjParams p) {
    extern __shared__ __align__(16) char lds[];
    const int nz = ZR > 0 ? 0 : (p.s / ZF) * ((p.M + ZT - 1) / ZT);
    const int b = blockIdx.x;
    if (b < nz) {
        z_tile<T>(p, b, lds);
        return;
    }
    const int ntiles = 2 * (p.e / BN);
    const int mtiles = (p.M + BM - 1) / BM;
    if (ZR > 0 && ntiles == 12 && mtiles % 4 == 0) {
        // XCD x (dispatch index % 8) takes half of the column tiles (each half
        // with two of the four tiles that carry a Z slice) and a quarter of
        // the token tiles: its six weight tiles (2.4 MB at d = 768) stay in
        // its 4 MB L2 while its token tiles stream through, where a range of
        // whole token tiles would cycle all twelve weight tiles through it
        // every round (165 -> 113 MB fetched per launch at B*T = 16384).
        // Inside an XCD the Z-carrying tiles (the slower ones) are dispatched
        // first, so the last round holds only plain tiles.
        constexpr int kHost[2][2] = {{0, 1}, {2, 3}}, kRest[2][4] = {{4, 6, 7, 8}, {5, 9, 10, 11}};
        const int u = b - nz;
        const int x = u & 7, j = u >> 3, h = x & 1;
        const int tq = mtiles / 4, nh = 2 * tq;  // token tiles and Z-carrying tiles per XCD
        const int t = (x >> 1) * tq + (j < nh ? j / 2 : (j - nh) / 4);
        const int col = j < nh ? kHost[h][j % 2] : kRest[h][(j - nh) % 4];
        uv_tile<T, ZR>(p, t * ntiles + col, lds);
    } else if (ZR > 0 && ntiles == 16 && mtiles % 2 == 0) {
        // e = 2048: XCD x takes a quarter of the column tiles (g, g+4, g+8,
        // g+12 with g = x % 4: one Z-carrying tile each) for half of the token
        // tiles (its weight tiles: 2 MB at d = 1024), the Z-carrying tiles first
        const int u = b - nz;
        const int x = u & 7, j = u >> 3, gq = x & 3;
        const int th = mtiles / 2;  // token tiles per XCD (= its Z-carrying tiles)
        const int t = (x >> 2) * th + (j < th ? j : (j - th) / 3);
        const int col = j < th ? gq : gq + 4 * (1 + (j - th) % 3);
        uv_tile<T, ZR>(p, t * ntiles + col, lds);
    } else {
        uv_tile<T, ZR>(p, xcd_remap(b - nz, gridDim.x - nz), lds);
    }
}

template <typename T, int ZR>
hipError_t launch_t(const ProjParams& p, hipStream_t st) {
    constexpr int LDS = ProjTile<T, ZR>::LDS;
    static_assert(LDS <= 160 * 1024, "projection LDS over budget");
    const int mtiles = (p.M + BM - 1) / BM;
    const int nz = ZR > 0 ? 0 : (p.s / ZF) * ((p.M + ZT - 1) / ZT);
    const int blocks = nz + 2 * (p.e / BN) * mtiles;
    hipError_t e = allow_lds<proj_kernel<T, ZR>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((proj_kernel<T, ZR>), dim3(blocks), dim3(512), LDS, st, p);
    return hipGetLastError();
}

// Z as side products of U tiles when there are ZHOSTS U tiles per token tile,
// in tiles of its own otherwise.
template <typename T>
hipError_t dispatch(const ProjParams& p, hipStream_t st) {
    if (p.e / BN >= ZHOSTS) return p.s == 128 ? launch_t<T, 128 / ZHOSTS>(p, st) : launch_t<T, 256 / ZHOSTS>(p, st);
    return launch_t<T, 0>(p, st);
}

}  // namespace

hipError_t launch_proj(const ProjParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? dispatch<bf16>(p, st) : dispatch<float>(p, st);
}

}  // namespace gau
