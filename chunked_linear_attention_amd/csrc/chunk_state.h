// Per-chunk linear-attention state: S_g = lin_scale * K_lin_g^T V_g (s x e),
// accumulated in fp32 and stored transposed as S_g^T ([e, s]) in the layer's
// element type: the prefix sums over chunks are formed in fp32 and handed to
// an MFMA in that same element type, so a wider store would only add traffic.
//
// Pages: the chunk summary K_lin_h^T V_h that the global (linear) part sums
// over chunks (wikillm "Method", eq. 7 and 8; Su's post, "Mixed Chunking");
// the listing divides the summary by C (wikillm, FLASH block pseudocode,
// "summaries"), which lin_scale carries.
//
// A batched GEMM over the B*G chunks on the shared MFMA core, K = the chunk's
// C tokens: A operand = K_lin_t rows (state dimensions), B operand = Vt rows
// (features), both token-contiguous.  The accumulator's columns are features,
// so the packed epilogue store runs along the rows of S_g^T, which is the
// layout the chunk kernel reads P_g in (K = s contiguous).
#pragma once

#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {

constexpr int BS = 128, BE = 128;  // state dims x features per block

template <typename T>
struct StateTile {
    using G = GemmCore<T, BS, BE, 2, 2>;
    static constexpr int STAGE = BE * (BS * Elem<T>::kBytes + 16);
    static constexpr int LDS = G::LDS_BYTES > STAGE ? G::LDS_BYTES : STAGE;
};

// Tiles of the launch: (s / BS) x (e / BE) per chunk.
inline int state_blocks(const StateParams& p) { return (p.e / BE) * (p.s / BS) * p.B * (p.T / p.C); }

// One BS x BE tile of one chunk's state (logical index bid over all tiles).
template <typename T>
__device__ __forceinline__ void state_tile(const StateParams& p, int bid, char* lds) {
    using G = typename StateTile<T>::G;
    constexpr int EB = Elem<T>::kBytes;
    const int G_ = p.T / p.C;
    const int ST = p.s / BS, ET = p.e / BE;
    const int et = bid % ET;
    const int st = (bid / ET) % ST;
    const int chunk = bid / (ET * ST);  // b * G + g
    const int b = chunk / G_, g = chunk - b * G_;
    const int e0 = et * BE, s0 = st * BS;
    const size_t pitch = (size_t)p.T * EB;
    const char* kl = (const char*)p.Klt + (((size_t)b * p.s + s0) * p.T + (size_t)g * p.C) * EB;
    const char* vt = (const char*)p.Vt + (((size_t)b * p.e + e0) * p.T + (size_t)g * p.C) * EB;

    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    G::run(acc, kl, pitch, BS, vt, pitch, BE, p.C, lds);

    const float ls = p.lin_scale;
    char* S = (char*)p.S + (((size_t)chunk * p.e + e0) * p.s + s0) * EB;
    const int s = p.s;
    G::template store_packed<T>(acc, lds, StateTile<T>::LDS, [&](int, int, float v) { return v * ls; },
                                [&](int f, int k) -> char* { return S + ((size_t)f * s + k) * EB; });
}

}  // namespace gau
