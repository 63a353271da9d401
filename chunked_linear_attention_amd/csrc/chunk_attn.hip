// Per-chunk attention of the FLASH layer, fused with the linear term and the
// U gate:
//   A_g   = relu^2(quad_scale * Q_quad_g K_quad_g^T + Bias), Bias[i][j] = w[C-1+j-i]
//           causal: A_g[i][j] = 0 for j > i (diagonal kept), applied after relu^2
//   Y_g   = U_g * (A_g V_g + Q_lin_g P_g)
// Pages: local part relu^2(Q K^T + b) V inside each chunk (wikillm "Method"
// step 1; Su's post "Mixed Chunking", the V_quad equation; the upper triangle
// is masked for a decoder); relu^2 activation and the relative-position bias
// of eq. 5 (wikillm "Method"; Su's post "Weak Attention"); the bias as a
// Toeplitz matrix of a 2C-1 vector (papercache, appendix D, Code 4);
// linear term Q_lin_g P_g and the gate U_g * (V_quad + V_lin) (wikillm
// "Method" steps 2-4, the FLASH block pseudocode).
//
// One block computes a 64-query x NE-feature tile of one chunk.  The C x C
// score matrix never leaves the chip: for each 64-key block the scores are
// formed by MFMA from LDS tiles of Q_quad and K_quad, passed through the bias,
// relu^2 and mask, written to LDS in the element type, and multiplied into the
// output accumulator against the matching V tile.  The linear term is one more
// MFMA contraction over s (Q_lin against the chunk's prefix state P_g, stored
// [e, s]) into the same accumulator, and the gate multiplies by U in the
// epilogue.  Causal blocks skip key blocks that lie wholly above the diagonal.
#include "gau_device.h"
#include "gau_launch.h"

namespace gau {
namespace {

constexpr int MQ = 64;      // query rows per block
constexpr int KB = 64;      // keys per key block
constexpr int SL = 128;     // s-elements per slice of the contraction over s

template <typename T, int NE>
struct AttnLayout {
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int SB = SL * EB;                 // bytes per slice row
    static constexpr int P_S = SB + 16;                // pitch of Q/K/P slices
    static constexpr int P_SC = KB * EB + 16;          // pitch of the score tile
    static constexpr int P_V = KB * EB + 16;           // pitch of the V tile (rows = features)
    static constexpr int P_U = NE * EB + 16;           // pitch of the U / Y tile
    // phase 1
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_K = OFF_Q + MQ * P_S;
    static constexpr int OFF_SC = OFF_K + KB * P_S;
    static constexpr int OFF_V = OFF_SC + MQ * P_SC;
    static constexpr int END1 = OFF_V + NE * P_V;
    // phase 2
    static constexpr int OFF_QL = 0;
    static constexpr int OFF_P = OFF_QL + MQ * P_S;
    static constexpr int END2 = OFF_P + NE * P_S;
    // epilogue
    static constexpr int END3 = MQ * P_U;
    static constexpr int BYTES = END1 > END2 ? (END1 > END3 ? END1 : END3) : (END2 > END3 ? END2 : END3);
};

template <typename T, int NE, int SD>
__global__ __launch_bounds__(256) void chunk_attn_kernel(AttnParams p) {
    extern __shared__ __align__(16) char lds[];
    using L = AttnLayout<T, NE>;
    constexpr int EB = L::EB;
    constexpr int NSL = SD / SL;
    constexpr int NB_O = NE / 2 / 16;  // 16-wide column blocks per wave in the output tile

    const int ET = p.e / NE;
    const int QT = p.C / MQ;
    int bid = blockIdx.x;
    const int et = bid % ET; bid /= ET;
    const int qt = bid % QT; bid /= QT;
    const int chunk = bid;  // b * G + g
    const int G_ = p.T / p.C;
    const int b = chunk / G_, g = chunk - b * G_;
    const int q0 = qt * MQ, e0 = et * NE;
    const size_t tok0 = (size_t)b * p.T + (size_t)g * p.C;  // first token row of the chunk

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave >> 1, wn = wave & 1;

    const size_t pitch_s = (size_t)p.s * EB;
    const size_t pitch_t = (size_t)p.T * EB;
    const char* Qq = (const char*)p.Qq + (tok0 + q0) * pitch_s;
    const char* Kq = (const char*)p.Kq + tok0 * pitch_s;
    const char* Vt = (const char*)p.Vt + (((size_t)b * p.e + e0) * p.T + (size_t)g * p.C) * EB;

    f32x4_t acc[2][NB_O];
    zero_acc(acc);

    // ---------------- local part: relu^2 scores times V, one key block at a time
    const int nkb = p.causal ? qt + 1 : p.C / KB;
    const float qs = p.quad_scale;
    const float* w = p.relpos + (p.C - 1);
    for (int kb = 0; kb < nkb; ++kb) {
        f32x4_t sacc[2][2];
        zero_acc(sacc);
        for (int sl = 0; sl < NSL; ++sl) {
            TileCopy<MQ, L::SB, 256> cq;
            TileCopy<KB, L::SB, 256> ck;
            TileCopy<NE, KB * EB, 256> cv;
            const bool load_q = (NSL > 1) || (kb == 0);
            if (load_q) cq.load(Qq + sl * L::SB, pitch_s, MQ, tid);
            ck.load(Kq + (size_t)kb * KB * pitch_s + sl * L::SB, pitch_s, KB, tid);
            if (sl == 0) cv.load(Vt + (size_t)kb * KB * EB, pitch_t, NE, tid);
            __syncthreads();  // previous users of the Q/K/score/V tiles are done
            if (load_q) cq.store(lds + L::OFF_Q, tid);
            ck.store(lds + L::OFF_K, tid);
            if (sl == 0) cv.store(lds + L::OFF_V, tid);
            __syncthreads();
            wave_mma<T, 2, 2, L::SB / 64>(sacc, lds + L::OFF_Q + wm * 32 * L::P_S, L::P_S,
                                          lds + L::OFF_K + wn * 32 * L::P_S, L::P_S, lane);
        }
        // bias, relu^2, causal mask -> score tile in LDS (element type)
        const bool diag = p.causal && (kb == qt);
        for_each_acc(sacc, lane, [&](int r, int c, float v) {
            const int i = q0 + wm * 32 + r;  // query position in the chunk
            const int j = kb * KB + wn * 32 + c;  // key position in the chunk
            float x = v * qs + w[j - i];
            x = x > 0.f ? x * x : 0.f;
            if (diag && j > i) x = 0.f;
            Elem<T>::put(lds + L::OFF_SC + (wm * 32 + r) * L::P_SC + (wn * 32 + c) * EB, x);
        });
        __syncthreads();
        wave_mma<T, 2, NB_O, KB * EB / 64>(acc, lds + L::OFF_SC + wm * 32 * L::P_SC, L::P_SC,
                                           lds + L::OFF_V + wn * (NE / 2) * L::P_V, L::P_V, lane);
    }

    // ---------------- global part: Q_lin_g P_g (P stored [e, s] per chunk)
    {
        const size_t pidx = p.causal ? (size_t)chunk : (size_t)b;
        const char* Ql = (const char*)p.Ql + (tok0 + q0) * pitch_s;
        const char* P = (const char*)p.P + (pidx * p.e + e0) * pitch_s;
        for (int sl = 0; sl < NSL; ++sl) {
            TileCopy<MQ, L::SB, 256> cq;
            TileCopy<NE, L::SB, 256> cp;
            cq.load(Ql + sl * L::SB, pitch_s, MQ, tid);
            cp.load(P + sl * L::SB, pitch_s, NE, tid);
            __syncthreads();
            cq.store(lds + L::OFF_QL, tid);
            cp.store(lds + L::OFF_P, tid);
            __syncthreads();
            wave_mma<T, 2, NB_O, L::SB / 64>(acc, lds + L::OFF_QL + wm * 32 * L::P_S, L::P_S,
                                             lds + L::OFF_P + wn * (NE / 2) * L::P_S, L::P_S, lane);
        }
    }

    // ---------------- gate: Y = U * (quad + lin)
    const size_t pitch_e = (size_t)p.e * EB;
    const char* U = (const char*)p.U + (tok0 + q0) * pitch_e + (size_t)e0 * EB;
    {
        TileCopy<MQ, NE * EB, 256> cu;
        cu.load(U, pitch_e, MQ, tid);
        __syncthreads();
        cu.store(lds, tid);
        __syncthreads();
    }
    for_each_acc(acc, lane, [&](int r, int c, float v) {
        char* a = lds + (wm * 32 + r) * L::P_U + (wn * (NE / 2) + c) * EB;
        Elem<T>::put(a, Elem<T>::get(a) * v);
    });
    __syncthreads();
    char* Y = (char*)p.Y + (tok0 + q0) * pitch_e + (size_t)e0 * EB;
    constexpr int VPR = NE * EB / 16;
    for (int idx = tid; idx < MQ * VPR; idx += 256) {
        const int row = idx / VPR, v = idx % VPR;
        *(u32x4_t*)(Y + (size_t)row * pitch_e + v * 16) = *(const u32x4_t*)(lds + row * L::P_U + v * 16);
    }
}

template <typename T, int NE, int SD>
hipError_t launch_t(const AttnParams& p, hipStream_t st) {
    constexpr int LDS = AttnLayout<T, NE>::BYTES;
    static_assert(LDS <= 160 * 1024, "chunk kernel LDS over budget");
    const int blocks = (p.e / NE) * (p.C / MQ) * p.B * (p.T / p.C);
    hipError_t e = allow_lds(chunk_attn_kernel<T, NE, SD>, LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_attn_kernel<T, NE, SD>), dim3(blocks), dim3(256), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_attn(const AttnParams& p, bool bf16_storage, hipStream_t st) {
    if (bf16_storage)
        return p.s == 128 ? launch_t<bf16, 256, 128>(p, st) : launch_t<bf16, 256, 256>(p, st);
    return p.s == 128 ? launch_t<float, 128, 128>(p, st) : launch_t<float, 128, 256>(p, st);
}

}  // namespace gau
