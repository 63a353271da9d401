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
// With H non-null (the backward's recompute) the pre-activations X W_u,
// X W_v, X W_z are also stored, token-major with row pitch 2e + s, before
// the epilogue applies SiLU.
//
// Layout written (see the workspace layout in gau.h):
//   U [M, e] row-major; Vt [B, e, T] (V transposed per sequence, so the chunk
//   kernels read tokens contiguously); Q_quad, K_quad, Q_lin [M, s] row-major;
//   K_lin_t [B, s, T] transposed.  M = B*T.
//
// With rope = 1 the four heads are rotated by position in the same epilogue
// (the listing rotates them after the scale+offset, positions counted over
// the whole sequence: wikillm, FLASH block pseudocode and "Paper vs code";
// the pair (h_i, h_{i+s/2}) turns by t * 10000^(-i/(s/2)), the schedule and
// half-split layout of the printed sinusoid helper, papercache appendix D,
// _get_scaledsin).  Every Z slice is formed so that both members of each
// rotated pair lie in the same lane's registers, and the rotation is applied
// to the fp32 head values before their one rounding to the element type.
//
// One launch, two kinds of blocks on the shared MFMA core.  When e < 1024 the
// first ceil(M/256) blocks each form all s features of Z for 256 tokens and
// write its four heads; the rest form the 256 x 256 tiles of U and V (the
// e/256 tiles of each section side by side along N, so a block's columns lie
// in one section and its epilogue branch is uniform).  When e >= 1024 the
// first four U tiles of each token tile form Z as a side product instead
// (ZR = s/4 features each).  U/V tiles are assigned to XCDs so that
// tiles sharing operand rows share an L2: at e = 1536 each XCD takes half of
// the column tiles for a quarter of the token tiles, at e = 2048 a quarter of
// them for half of the token tiles; otherwise contiguous ranges (the 2e/256
// column tiles of one token tile together).
#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {

namespace {

constexpr int BM = 256, BN = 256, WGM = 2, WGN = 4;  // U/V tiles, wave grid
constexpr int ZT = 256;                              // Z tiles: all s features x 256 tokens
constexpr int ZHOSTS = 4;                            // U tiles that carry a Z slice
constexpr int THETA_BYTES = 1024;                    // rotary frequencies (fp64, s/2 <= 128) past the tiles' LDS

// Z tile of ZF = s features x ZT tokens: one wave row, eight wave columns, so
// every wave holds all ZF features of its 32 tokens (feature i and its
// rotary partner i + s/2 in one lane).
template <typename T, int ZF>
using ZCore = GemmCore<T, ZF, ZT, 1, 8>;

// ZR = 0: Z in tiles of its own; ZR = s / ZHOSTS: each of the first ZHOSTS U
// tiles of a token tile also forms ZR features of Z (the GEMM core's side
// product, sharing the tile's X chunks and B fragments).
template <typename T, int ZR>
struct ProjTile {
    using G = GemmCore<T, BM, BN, WGM, WGN, 2, ZR>;
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int STAGE = (BM * (BN * EB + 16) > 160 * 1024 - 1024) ? BM / WGM * (BN * EB + 16)
                                                                           : BM * (BN * EB + 16);
    static constexpr int ZC = ZCore<T, 256>::LDS_BYTES > ZCore<T, 128>::LDS_BYTES ? ZCore<T, 256>::LDS_BYTES
                                                                                   : ZCore<T, 128>::LDS_BYTES;
    static constexpr int CORE = G::LDS_BYTES > ZC ? G::LDS_BYTES : ZC;
    static constexpr int LDS = CORE > STAGE ? CORE : STAGE;  // tiles and staging; the frequencies follow
};

// The rotary frequencies theta_i = 10000^(-i/(s/2)) of the block, fp64, in
// LDS past the tiles (read after the K loop's barriers).
__device__ __forceinline__ void fill_theta(double* theta, int half) {
    for (int i = threadIdx.x; i < half; i += blockDim.x) theta[i] = rope_theta(i, half);
}

// Epilogue of a Z slice formed as a side product: ZR features of Z for the
// 256 tokens m0.. .  Slice rows r < ZR/2 are features hb + r, rows r >= ZR/2
// features s/2 + hb + r - ZR/2, so rotary pair (hb + r, s/2 + hb + r) lies in
// one lane (ZR = 32: registers q and q + 8 of a block; ZR = 64: register q of
// blocks 0 and 1).  Applies SiLU, the four heads (and with ROPE their
// rotation by position m mod T) and stores Q_quad, K_quad, Q_lin
// (token-major) and K_lin_t (feature-major) through LDS, all four heads in
// one staging pass when they fit, else one head per pass.
template <typename T, int ZR, bool ROPE, typename Side>
__device__ __forceinline__ void z_side_epilogue(const ProjParams& p, Side& sd, int m0, int hb, char* lds,
                                                int lds_bytes, const double* theta) {
    constexpr int EB = Elem<T>::kBytes;
    constexpr int ZMB = ZR / 32;
    constexpr int ZH = ZR / 2;         // rotary pairs in the slice
    constexpr int DI = ZH / 32;        // partner of (block i, register q): (i + DI, q + DQ)
    constexpr int DQ = (ZH % 32) / 2;
    constexpr int NT = WGM * WGN * kWave;
    constexpr int TP = ZR * EB + 16;  // token-major staging pitch
    constexpr int FP = BN * EB + 16;  // feature-major staging pitch
    constexpr int HEAD_T = BN * TP;   // bytes of one token-major head
    static_assert(ZH % 8 == 0, "a 16-byte vector of the slice lies in one half");
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int wm = wave / WGN, wn = wave % WGN;
    const int c = lane & 31, h = lane >> 5;
    const int tok = wn * 64 + wm * 32 + c;  // B-tile column this lane's side outputs belong to
    const int M = p.M, T_ = p.T, s = p.s, half = p.s / 2;
    const bool one_pass = 3 * HEAD_T + ZR * FP <= lds_bytes;
    auto feat = [&](int zr) { return zr < ZH ? hb + zr : half + hb + (zr - ZH); };
    if (p.H) {  // the slice's pre-activations, token-major at column 2e + feature
        __syncthreads();
#pragma unroll
        for (int i = 0; i < ZMB; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                char* q = lds + tok * TP + (i * 32 + 8 * g4 + 4 * h) * EB;
                const float x[4] = {sd.acc[i][4 * g4], sd.acc[i][4 * g4 + 1], sd.acc[i][4 * g4 + 2],
                                    sd.acc[i][4 * g4 + 3]};
                if constexpr (EB == 2) {
                    *(u32x2_t*)q = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                } else {
                    *(f32x4_t*)q = f32x4_t{x[0], x[1], x[2], x[3]};
                }
            }
        __syncthreads();
        constexpr int VPR = ZR * EB / 16;
        const size_t hrp = (size_t)(2 * p.e + s);
        for (int idx = threadIdx.x; idx < BN * VPR; idx += NT) {
            const int t = idx / VPR, v = idx - t * VPR;
            const int m = m0 + t;
            if (m < M)
                *(u32x4_t*)((char*)p.H + ((size_t)m * hrp + 2 * p.e + feat(v * (16 / EB))) * EB) =
                    *(const u32x4_t*)(lds + t * TP + v * 16);
        }
    }
#pragma unroll
    for (int i = 0; i < ZMB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) sd.acc[i][r] = silu(sd.acc[i][r]);

    // rotation of the lane's pairs (first-half rows i*32 + 8*(q/4) + 4h + q%4 < ZH)
    float cs[ZMB][16], sn[ZMB][16];
    if constexpr (ROPE) {
        const int m = m0 + tok;
        const double pos = (double)((m < M ? m : 0) % T_);
#pragma unroll
        for (int i = 0; i < ZMB; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (i * 32 + 8 * (q >> 2) < ZH) {
                    const int zr = i * 32 + 8 * (q >> 2) + 4 * h + (q & 3);
                    rope_cos_sin(pos, theta[hb + zr], cs[i][q], sn[i][q]);
                }
    }

    // head hd's values (z * gamma + beta, rotated with ROPE), staged at base
    // (token-major heads at hd * HEAD_T when one_pass, else at 0; K_lin after
    // the three token-major heads, or at 0)
    auto stage_head = [&](int hd, char* base) {
        float v[ZMB][16];
#pragma unroll
        for (int i = 0; i < ZMB; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int f0 = feat(i * 32 + 8 * g4 + 4 * h);  // four consecutive features
                const f32x4_t gm = *(const f32x4_t*)(p.scale + hd * s + f0);
                const f32x4_t bt = *(const f32x4_t*)(p.offset + hd * s + f0);
                v[i][4 * g4 + 0] = sd.acc[i][4 * g4 + 0] * gm.x + bt.x;
                v[i][4 * g4 + 1] = sd.acc[i][4 * g4 + 1] * gm.y + bt.y;
                v[i][4 * g4 + 2] = sd.acc[i][4 * g4 + 2] * gm.z + bt.z;
                v[i][4 * g4 + 3] = sd.acc[i][4 * g4 + 3] * gm.w + bt.w;
            }
        if constexpr (ROPE) {
#pragma unroll
            for (int i = 0; i < ZMB; ++i)
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (i * 32 + 8 * (q >> 2) < ZH) {
                        const float lo = v[i][q], hi = v[i + DI][q + DQ];
                        v[i][q] = lo * cs[i][q] - hi * sn[i][q];
                        v[i + DI][q + DQ] = hi * cs[i][q] + lo * sn[i][q];
                    }
        }
#pragma unroll
        for (int i = 0; i < ZMB; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int zr0 = i * 32 + 8 * g4 + 4 * h;  // four consecutive slice rows
                const float v0 = v[i][4 * g4 + 0], v1 = v[i][4 * g4 + 1];
                const float v2 = v[i][4 * g4 + 2], v3 = v[i][4 * g4 + 3];
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
                    *(u32x4_t*)(dst + ((size_t)m * s + feat(v * (16 / EB))) * EB) =
                        *(const u32x4_t*)(base + t * TP + v * 16);
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
                    *(u32x4_t*)(Klt + (((size_t)b * s + feat(zr)) * T_ + t) * EB) =
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
template <typename T, int ZR, bool ROPE>
__device__ __forceinline__ void uv_tile(const ProjParams& p, int bid, char* lds, const double* theta) {
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
            // slice nt: features hb.. and s/2 + hb.. (ZR/2 each), hb = nt * ZR/2
            const int hb = nt * (ZR / 2);
            G::run_with_side(acc, sd, wt, pitch, BN, xt, pitch, rows_x, p.d, (const char*)p.W_z + (size_t)hb * pitch,
                             (const char*)p.W_z + (size_t)(p.s / 2 + hb) * pitch, ZR / 2, pitch, true, lds);
            ran = true;
        }
    }
    if (!ran)
        G::run(acc, is_v ? xt : wt, pitch, is_v ? rows_x : BN, is_v ? wt : xt, pitch, is_v ? BN : rows_x, p.d, lds);

    constexpr int LDS = ProjTile<T, ZR>::LDS;
    const int M = p.M, T_ = p.T;
    auto ident = [](int, int, float v) { return v; };
    if (p.H) {  // pre-activations, token-major, columns c0.. of the U or V section
        char* Hb = (char*)p.H + (size_t)((is_v ? p.e : 0) + c0) * EB;
        const size_t hrp = (size_t)(2 * p.e + p.s);
        if (!is_v)  // acc rows = features, columns = tokens
            G::template store_packed<T>(acc, lds, LDS, ident, [&](int tok, int feat) -> char* {
                const int m = m0 + tok;
                return m < M ? Hb + ((size_t)m * hrp + feat) * EB : nullptr;
            });
        else  // acc rows = tokens, columns = features
            G::template store<T, false>(acc, lds, LDS, ident, [&](int tok, int feat) -> char* {
                const int m = m0 + tok;
                return m < M ? Hb + ((size_t)m * hrp + feat) * EB : nullptr;
            });
    }
    // SiLU, then the stores: in two column passes over two LDS buffers
    // (store_packed_cols: the first pass's stores overlap the second's SiLU)
    // when they fit, else SiLU on the whole tile and one store_packed
    auto act = [](int, int, float v) { return silu(v); };
    constexpr bool cols = G::template kColsFit<T, LDS>;
    if constexpr (!cols) G::transform(acc, act);
    auto store_act = [&](auto&& dst) {
        if constexpr (cols)
            G::template store_packed_cols<T, LDS>(acc, lds, act, dst);
        else
            G::template store_packed<T>(acc, lds, LDS, ident, dst);
    };
    if (!is_v) {
        // acc rows = features, columns = tokens (U is not stored when the
        // pre-activations are: the backward forms U = SiLU(X W_u) from them)
        char* U = (char*)p.U;
        if (!p.H)
            store_act([&](int tok, int feat) -> char* {
                const int m = m0 + tok;
                return m < M ? U + ((size_t)m * p.e + c0 + feat) * EB : nullptr;
            });
        if constexpr (ZR > 0) {
            if (side) z_side_epilogue<T, ZR, ROPE>(p, sd, m0, nt * (ZR / 2), lds, LDS, theta);
        }
    } else {
        // acc rows = tokens, columns = features
        char* Vt = (char*)p.Vt;
        store_act([&](int feat, int tok) -> char* {
            const int m = m0 + tok;
            if (m >= M) return nullptr;
            const int b = m / T_, t = m - b * T_;
            return Vt + (((size_t)b * p.e + c0 + feat) * T_ + t) * EB;
        });
    }
}

// Z = SiLU(X W_z) for all ZF = s features of the 256 tokens of token tile
// zb, and its four heads h = Z * gamma[h] + beta[h] (rotated by position with
// ROPE): Q_quad, K_quad, Q_lin token-major, K_lin feature-major.  Every wave
// holds all features of its 32 tokens (rows i*32 + 8*(q/4) + 4*(l/32) + q%4 of
// accumulator block i, lane l, register q; column = the wave's token), so
// rotary pairs (f, f + s/2) are blocks i and i + MB/2 of one lane, and the
// heads are stored from registers (4 consecutive features per 8- or 16-byte
// store; K_lin_t one element per store).  This path serves the layers with
// e < 1024 only.
template <typename T, int ZF, bool ROPE>
__device__ __forceinline__ void z_tile(const ProjParams& p, int zb, char* lds, const double* theta) {
    using G = ZCore<T, ZF>;
    constexpr int EB = Elem<T>::kBytes;
    constexpr int MB = G::MB;
    static_assert(G::NB == 1 && MB % 2 == 0, "Z tile layout");
    const int m0 = zb * ZT;
    const size_t pitch = (size_t)p.d * EB;
    const int rows_x = min(ZT, p.M - m0);

    f32x16_t acc[MB][1];
    G::zero(acc);
    G::run(acc, (const char*)p.W_z, pitch, ZF, (const char*)p.X + (size_t)m0 * pitch, pitch, rows_x, p.d, lds);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int c = lane & 31, h = lane >> 5;
    const int m = m0 + wave * 32 + c;  // this lane's token
    if (m >= p.M) return;              // (no barrier follows)
    if (p.H) {  // pre-activations X W_z, token-major at column 2e
        char* row = (char*)p.H + ((size_t)m * (2 * p.e + p.s) + 2 * p.e) * EB;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                char* q = row + (size_t)(i * 32 + 8 * g4 + 4 * h) * EB;
                const float x[4] = {acc[i][0][4 * g4], acc[i][0][4 * g4 + 1], acc[i][0][4 * g4 + 2],
                                    acc[i][0][4 * g4 + 3]};
                if constexpr (EB == 2) {
                    *(u32x2_t*)q = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                } else {
                    *(f32x4_t*)q = f32x4_t{x[0], x[1], x[2], x[3]};
                }
            }
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][0][r] = silu(acc[i][0][r]);
    const int T_ = p.T, s = p.s, half = p.s / 2;
    const int b = m / T_, t = m - b * T_;
    char* Klt = (char*)p.Klt + ((size_t)b * s * T_ + t) * EB;
    // features f0 .. f0+3 (block i) and their rotary partners f0 + s/2 ..
    // (block i + MB/2), all four heads
#pragma unroll
    for (int i = 0; i < MB / 2; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int f0 = i * 32 + 8 * g4 + 4 * h;
            float cs[4], sn[4];
            if constexpr (ROPE) {
#pragma unroll
                for (int k = 0; k < 4; ++k) rope_cos_sin((double)t, theta[f0 + k], cs[k], sn[k]);
            }
            for (int hd = 0; hd < 4; ++hd) {
                const f32x4_t gl = *(const f32x4_t*)(p.scale + hd * s + f0);
                const f32x4_t bl = *(const f32x4_t*)(p.offset + hd * s + f0);
                const f32x4_t gh = *(const f32x4_t*)(p.scale + hd * s + half + f0);
                const f32x4_t bh = *(const f32x4_t*)(p.offset + hd * s + half + f0);
                float lo[4], hi[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    lo[k] = acc[i][0][4 * g4 + k] * gl[k] + bl[k];
                    hi[k] = acc[i + MB / 2][0][4 * g4 + k] * gh[k] + bh[k];
                }
                if constexpr (ROPE) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float a = lo[k], z = hi[k];
                        lo[k] = a * cs[k] - z * sn[k];
                        hi[k] = z * cs[k] + a * sn[k];
                    }
                }
                if (hd < 3) {
                    char* row = (char*)(hd == 0 ? p.Qq : hd == 1 ? p.Kq : p.Ql) + (size_t)m * s * EB;
                    char* ql = row + (size_t)f0 * EB;
                    char* qh = row + (size_t)(half + f0) * EB;
                    if constexpr (EB == 2) {
                        *(u32x2_t*)ql = u32x2_t{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3])};
                        *(u32x2_t*)qh = u32x2_t{pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
                    } else {
                        *(f32x4_t*)ql = f32x4_t{lo[0], lo[1], lo[2], lo[3]};
                        *(f32x4_t*)qh = f32x4_t{hi[0], hi[1], hi[2], hi[3]};
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        Elem<T>::put(Klt + (size_t)(f0 + k) * T_ * EB, lo[k]);
                        Elem<T>::put(Klt + (size_t)(half + f0 + k) * T_ * EB, hi[k]);
                    }
                }
            }
        }
}

template <typename T, int ZR, bool ROPE>
__global__ __launch_bounds__(512) void proj_kernel(ProjParams p) {
    extern __shared__ __align__(16) char lds[];
    double* theta = (double*)(lds + ProjTile<T, ZR>::LDS);
    if constexpr (ROPE) fill_theta(theta, p.s / 2);
    const int nz = ZR > 0 ? 0 : (p.M + ZT - 1) / ZT;
    const int b = blockIdx.x;
    if (b < nz) {
        if (p.s == 128)
            z_tile<T, 128, ROPE>(p, b, lds, theta);
        else
            z_tile<T, 256, ROPE>(p, b, lds, theta);
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
        uv_tile<T, ZR, ROPE>(p, t * ntiles + col, lds, theta);
    } else if (ZR > 0 && ntiles == 16 && mtiles % 2 == 0) {
        // e = 2048: XCD x takes a quarter of the column tiles (g, g+4, g+8,
        // g+12 with g = x % 4: one Z-carrying tile each) for half of the token
        // tiles (its weight tiles: 2 MB at d = 1024), the Z-carrying tiles first
        const int u = b - nz;
        const int x = u & 7, j = u >> 3, gq = x & 3;
        const int th = mtiles / 2;  // token tiles per XCD (= its Z-carrying tiles)
        const int t = (x >> 2) * th + (j < th ? j : (j - th) / 3);
        const int col = j < th ? gq : gq + 4 * (1 + (j - th) % 3);
        uv_tile<T, ZR, ROPE>(p, t * ntiles + col, lds, theta);
    } else {
        uv_tile<T, ZR, ROPE>(p, xcd_remap(b - nz, gridDim.x - nz), lds, theta);
    }
}

template <typename T, int ZR, bool ROPE>
hipError_t launch_t(const ProjParams& p, hipStream_t st) {
    constexpr int LDS = ProjTile<T, ZR>::LDS + (ROPE ? THETA_BYTES : 0);
    static_assert(LDS <= 160 * 1024, "projection LDS over budget");
    const int mtiles = (p.M + BM - 1) / BM;
    const int nz = ZR > 0 ? 0 : (p.M + ZT - 1) / ZT;
    const int blocks = nz + 2 * (p.e / BN) * mtiles;
    hipError_t e = allow_lds<proj_kernel<T, ZR, ROPE>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((proj_kernel<T, ZR, ROPE>), dim3(blocks), dim3(512), LDS, st, p);
    return hipGetLastError();
}

template <typename T, int ZR>
hipError_t launch_r(const ProjParams& p, hipStream_t st) {
    return p.rope ? launch_t<T, ZR, true>(p, st) : launch_t<T, ZR, false>(p, st);
}

// Z as side products of U tiles when there are ZHOSTS U tiles per token tile,
// in tiles of its own otherwise.
template <typename T>
hipError_t dispatch(const ProjParams& p, hipStream_t st) {
    if (p.e / BN >= ZHOSTS) return p.s == 128 ? launch_r<T, 128 / ZHOSTS>(p, st) : launch_r<T, 256 / ZHOSTS>(p, st);
    return launch_r<T, 0>(p, st);
}

}  // namespace

hipError_t launch_proj(const ProjParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? dispatch<bf16>(p, st) : dispatch<float>(p, st);
}

}  // namespace gau
