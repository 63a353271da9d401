// Per-chunk attention of the FLASH layer, fused with the linear term and the
// U gate:
//   Y_g = U_g * (A_g V_g + Q_lin_g P_g)
// with A_g the chunk's masked relu^2 attention weights (chunk_scores) and P_g
// the chunk's prefix state (chunk_scan).  Pages: local part A_g V_g inside
// each chunk and global part Q_lin_g (sum of earlier chunk summaries), summed
// and gated by U (wikillm "Method" steps 1-4 and the FLASH block pseudocode;
// Su's post "Mixed Chunking", V_quad, V_lin and the output equation).
//
// Both products are one GEMM per chunk on the shared MFMA core: the K axis is
// the chunk's keys followed by the s state dimensions,
//   A operand (rows = features): [ Vt_g (keys) | P_g^T (s) ]
//   B operand (rows = queries) : [ A_g  (keys) | Q_lin_g (s) ]
// so the local and global terms accumulate into the same registers.  A causal
// query tile reads only the keys up to its last query (later keys are masked
// to zero).  The gate multiplies the fp32 accumulator by U in the epilogue,
// which stores Y token-major; the block's U values are loaded into registers
// before the main loop, so their latency overlaps the chunk copies instead of
// adding one more round trip after them.  Y may be U itself (the forward
// gates in place): a block writes exactly the elements of Y whose gate values
// it has already read, and no other block reads them.
#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {
namespace {

constexpr int BF = 128;         // features per block (accumulator rows)
constexpr int WGM = 2, WGN = 2;  // wave grid

template <typename T, int BQ>
struct AttnTile {
    using G = GemmCore<T, BF, BQ, WGM, WGN>;
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int STAGE = BQ * (BF * EB + 16);
    static constexpr int LDS = G::LDS_BYTES > STAGE ? G::LDS_BYTES : STAGE;
};

// The gate values of one lane: for each accumulator block (i, j) and group
// g4 of four rows, four consecutive features of one token of U.
template <typename T>
struct GateVec;
template <>
struct GateVec<bf16> {
    using type = u32x2_t;
};
template <>
struct GateVec<float> {
    using type = f32x4_t;
};

template <typename T, int BQ, bool GATED>
__global__ __launch_bounds__(WGM * WGN * kWave) void chunk_attn_kernel(AttnParams p) {
    extern __shared__ __align__(16) char lds[];
    using G = typename AttnTile<T, BQ>::G;
    constexpr int EB = Elem<T>::kBytes;
    constexpr int KELEMS = G::KELEMS;
    const int FT = p.e / BF;
    const int QT = p.C / BQ;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int ft = bid % FT;
    const int qt = (bid / FT) % QT;
    const int chunk = bid / (FT * QT);  // b * G + g
    const int G_ = p.T / p.C;
    const int b = chunk / G_, g = chunk - b * G_;
    const int f0 = ft * BF, q0 = qt * BQ;
    const size_t tok0 = (size_t)b * p.T + (size_t)g * p.C;
    const int keys = p.causal ? q0 + BQ : p.C;
    const size_t pidx = (p.causal || p.p_chunked) ? (size_t)chunk : (size_t)b;

    const KSeg a0{(const char*)p.Vt + (((size_t)b * p.e + f0) * p.T + (size_t)g * p.C) * EB, (size_t)p.T * EB,
                  p.local ? keys / KELEMS : 0};
    const KSeg a1{(const char*)p.P + (pidx * p.e + f0) * p.s * EB, (size_t)p.s * EB, p.global ? p.s / KELEMS : 0};
    const KSeg b0{(const char*)p.A + ((size_t)chunk * p.C + q0) * p.C * EB, (size_t)p.C * EB,
                  p.local ? keys / KELEMS : 0};
    const KSeg b1{(const char*)p.Ql + (tok0 + q0) * p.s * EB, (size_t)p.s * EB, p.global ? p.s / KELEMS : 0};

    // gate: acc rows are features f0 + row, columns are queries q0 + col; the
    // four rows a lane holds are four consecutive features of one token of U
    // (the accumulator layout of the MFMA core, as in transform4)
    // (GATED false: U == nullptr, Y = the attention output itself; a template
    // parameter so that the gated kernel's code is that of the gate alone)
    const char* U = (const char*)p.U + ((tok0 + q0) * p.e + f0) * EB;
    const size_t pitch_e = (size_t)p.e * EB;
    using GV = typename GateVec<T>::type;
    GV gate[G::MB][G::NB][4];
    if constexpr (GATED) {
        const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
        const int wm = wave / WGN, wn = wave % WGN;
        const int c = lane & 31, h = lane >> 5;
#pragma unroll
        for (int i = 0; i < G::MB; ++i)
#pragma unroll
            for (int j = 0; j < G::NB; ++j)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int row0 = wm * G::WTM + i * 32 + 8 * g4 + 4 * h;
                    const int col = wn * G::WTN + j * 32 + c;
                    gate[i][j][g4] = *(const GV*)(U + (size_t)col * pitch_e + (size_t)row0 * EB);
                }
    }

    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    G::run_segs(acc, a0, a1, BF, b0, b1, BQ, lds);

    if constexpr (GATED)
#pragma unroll
    for (int i = 0; i < G::MB; ++i)
#pragma unroll
        for (int j = 0; j < G::NB; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const GV w = gate[i][j][g4];
                if constexpr (EB == 2) {
                    acc[i][j][4 * g4 + 0] *= __uint_as_float(w.x << 16);
                    acc[i][j][4 * g4 + 1] *= __uint_as_float(w.x & 0xFFFF0000u);
                    acc[i][j][4 * g4 + 2] *= __uint_as_float(w.y << 16);
                    acc[i][j][4 * g4 + 3] *= __uint_as_float(w.y & 0xFFFF0000u);
                } else {
                    acc[i][j][4 * g4 + 0] *= w.x;
                    acc[i][j][4 * g4 + 1] *= w.y;
                    acc[i][j][4 * g4 + 2] *= w.z;
                    acc[i][j][4 * g4 + 3] *= w.w;
                }
            }

    char* Y = (char*)p.Y + ((tok0 + q0) * p.e + f0) * EB;
    auto ident = [](int, int, float v) { return v; };
    G::template store_packed<T>(acc, lds, AttnTile<T, BQ>::LDS, ident,
                                [&](int q, int f) -> char* { return Y + (size_t)q * pitch_e + (size_t)f * EB; });
}

template <typename T, int BQ, bool GATED>
hipError_t launch_t(const AttnParams& p, hipStream_t st) {
    constexpr int LDS = AttnTile<T, BQ>::LDS;
    static_assert(LDS <= 160 * 1024, "chunk kernel LDS over budget");
    const int blocks = (p.e / BF) * (p.C / BQ) * p.B * (p.T / p.C);
    hipError_t e = allow_lds<chunk_attn_kernel<T, BQ, GATED>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_attn_kernel<T, BQ, GATED>), dim3(blocks), dim3(WGM * WGN * kWave), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_attn(const AttnParams& p, bool bf16_storage, hipStream_t st) {
    const bool g = p.U != nullptr;
    if (bf16_storage) {
        if (p.C >= 128) return g ? launch_t<bf16, 128, true>(p, st) : launch_t<bf16, 128, false>(p, st);
        return g ? launch_t<bf16, 64, true>(p, st) : launch_t<bf16, 64, false>(p, st);
    }
    if (p.C >= 128) return g ? launch_t<float, 128, true>(p, st) : launch_t<float, 128, false>(p, st);
    return g ? launch_t<float, 64, true>(p, st) : launch_t<float, 64, false>(p, st);
}

}  // namespace gau
