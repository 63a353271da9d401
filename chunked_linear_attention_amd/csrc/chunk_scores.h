// Per-chunk attention weights of the local (quadratic) part:
//   A_g[i][j] = relu^2(quad_scale * q_quad_i . k_quad_j + Bias[i][j]),
//   Bias[i][j] = w[C-1 + j - i];  causal: A_g[i][j] = 0 for j > i (diagonal kept).
// Pages: relu^2(Q K^T + b) inside each chunk (wikillm "Method" step 1 and
// eq. 5; Su's post "Weak Attention" and "Mixed Chunking"); the bias as a
// Toeplitz matrix of a 2C-1 vector (papercache, appendix D, Code 4, n < 512);
// the listing scales Q K^T by 1/C before adding the bias and masks after
// relu^2 (wikillm, FLASH block pseudocode), which quad_scale carries.
//
// A batched GEMM over chunks on the shared MFMA core: each block forms one
// TS x TS (query x key) tile from Q_quad and K_quad rows (K = s), applies
// bias, relu^2 and the mask in the epilogue and stores A_g query-major in the
// layer's element type, the precision the attention GEMM reads it in.  Causal
// chunks compute only the tiles at or below the diagonal.
#pragma once

#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {

template <typename T, int TS>
struct ScoresTile {
    using G = GemmCore<T, TS, TS, 2, 2>;
    static constexpr int STAGE = TS * (TS * Elem<T>::kBytes + 16);
    static constexpr int LDS = G::LDS_BYTES > STAGE ? G::LDS_BYTES : STAGE;
};

// Query x key tile width: 128, or 64 for C = 64.
inline int scores_tile_width(int C) { return C >= 128 ? 128 : 64; }

// Tiles of the launch: the lower-triangle tile pairs (causal) or all pairs,
// for every chunk.
inline int scores_blocks(const ScoresParams& p) {
    const int nt = p.C / scores_tile_width(p.C);
    const int npairs = p.causal ? nt * (nt + 1) / 2 : nt * nt;
    return npairs * p.B * (p.T / p.C);
}

// One TS x TS tile (logical index bid over all the tiles of all chunks).
template <typename T, int TS>
__device__ __forceinline__ void scores_tile(const ScoresParams& p, int bid, char* lds) {
    using G = typename ScoresTile<T, TS>::G;
    constexpr int EB = Elem<T>::kBytes;
    const int nt = p.C / TS;
    const int npairs = p.causal ? nt * (nt + 1) / 2 : nt * nt;
    const int pair = bid % npairs;
    const int chunk = bid / npairs;
    int qt, kt;
    if (p.causal) {  // pair -> (qt, kt) with kt <= qt, row-major over the lower triangle
        qt = 0;
        while ((qt + 1) * (qt + 2) / 2 <= pair) ++qt;
        kt = pair - qt * (qt + 1) / 2;
    } else {
        qt = pair / nt;
        kt = pair % nt;
    }
    const int q0 = qt * TS, k0 = kt * TS;
    const int G_ = p.T / p.C;
    const int b = chunk / G_, g = chunk - b * G_;
    const size_t tok0 = (size_t)b * p.T + (size_t)g * p.C;
    const size_t pitch = (size_t)p.s * EB;

    // acc rows = keys (A operand K_quad), columns = queries: the packed store
    // then runs along the query-major rows of A_g.
    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    G::run(acc, (const char*)p.Kq + (tok0 + k0) * pitch, pitch, TS, (const char*)p.Qq + (tok0 + q0) * pitch, pitch,
           TS, p.s, lds);

    const float qs = p.quad_scale;
    const float* w = p.relpos + (p.C - 1);
    const bool diag = p.causal && qt == kt;
    auto val = [&](int kr, int qc, float v) {
        const int i = q0 + qc, j = k0 + kr;  // query and key positions in the chunk
        float x = v * qs + w[j - i];
        x = x > 0.f ? x * x : 0.f;
        return (diag && j > i) ? 0.f : x;
    };
    char* A = (char*)p.A + ((size_t)chunk * p.C + q0) * p.C * EB + (size_t)k0 * EB;
    const int C = p.C;
    G::template store_packed<T>(acc, lds, ScoresTile<T, TS>::LDS, val,
                                [&](int q, int k) -> char* { return A + ((size_t)q * C + k) * EB; });
}

}  // namespace gau
