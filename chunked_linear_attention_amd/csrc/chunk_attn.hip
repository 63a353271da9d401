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
// which stores Y token-major.
#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {
namespace {

constexpr int BF = 128;  // features per block (accumulator rows)

template <typename T, int BQ>
struct AttnTile {
    using G = GemmCore<T, BF, BQ, 2, 2>;
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int STAGE = BQ * (BF * EB + 16);
    static constexpr int LDS = G::LDS_BYTES > STAGE ? G::LDS_BYTES : STAGE;
};

template <typename T, int BQ>
__global__ __launch_bounds__(256) void chunk_attn_kernel(AttnParams p) {
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
    const size_t pidx = p.causal ? (size_t)chunk : (size_t)b;

    const KSeg a0{(const char*)p.Vt + (((size_t)b * p.e + f0) * p.T + (size_t)g * p.C) * EB, (size_t)p.T * EB,
                  keys / KELEMS};
    const KSeg a1{(const char*)p.P + (pidx * p.e + f0) * p.s * EB, (size_t)p.s * EB, p.s / KELEMS};
    const KSeg b0{(const char*)p.A + ((size_t)chunk * p.C + q0) * p.C * EB, (size_t)p.C * EB, keys / KELEMS};
    const KSeg b1{(const char*)p.Ql + (tok0 + q0) * p.s * EB, (size_t)p.s * EB, p.s / KELEMS};

    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    G::run_segs(acc, a0, a1, BF, b0, b1, BQ, lds);

    // gate: acc rows are features f0 + row, columns are queries q0 + col; the
    // four rows a lane holds are four consecutive features of one token of U
    const char* U = (const char*)p.U + ((tok0 + q0) * p.e + f0) * EB;
    const size_t pitch_e = (size_t)p.e * EB;
    G::transform4(acc, [&](int row0, int col, float (&v)[4]) {
        const char* u = U + (size_t)col * pitch_e + (size_t)row0 * EB;
        if constexpr (EB == 2) {
            const u32x2_t w = *(const u32x2_t*)u;
            v[0] *= __uint_as_float(w.x << 16);
            v[1] *= __uint_as_float(w.x & 0xFFFF0000u);
            v[2] *= __uint_as_float(w.y << 16);
            v[3] *= __uint_as_float(w.y & 0xFFFF0000u);
        } else {
            const f32x4_t w = *(const f32x4_t*)u;
            v[0] *= w.x;
            v[1] *= w.y;
            v[2] *= w.z;
            v[3] *= w.w;
        }
    });

    char* Y = (char*)p.Y + ((tok0 + q0) * p.e + f0) * EB;
    auto ident = [](int, int, float v) { return v; };
    G::template store_packed<T>(acc, lds, AttnTile<T, BQ>::LDS, ident,
                                [&](int q, int f) -> char* { return Y + (size_t)q * pitch_e + (size_t)f * EB; });
}

template <typename T, int BQ>
hipError_t launch_t(const AttnParams& p, hipStream_t st) {
    constexpr int LDS = AttnTile<T, BQ>::LDS;
    static_assert(LDS <= 160 * 1024, "chunk kernel LDS over budget");
    const int blocks = (p.e / BF) * (p.C / BQ) * p.B * (p.T / p.C);
    hipError_t e = allow_lds<chunk_attn_kernel<T, BQ>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_attn_kernel<T, BQ>), dim3(blocks), dim3(256), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_attn(const AttnParams& p, bool bf16_storage, hipStream_t st) {
    if (bf16_storage) return p.C >= 128 ? launch_t<bf16, 128>(p, st) : launch_t<bf16, 64>(p, st);
    return p.C >= 128 ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

}  // namespace gau
