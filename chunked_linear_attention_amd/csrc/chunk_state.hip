// Per-chunk linear-attention state: S_g = lin_scale * K_lin_g^T V_g (s x e),
// stored transposed as S_g^T = lin_scale * V_g^T K_lin_g ([e, s], fp32).
//
// Pages: the chunk summary K_lin_h^T V_h that the global (linear) part sums
// over chunks (wikillm "Method", eq. 7 and 8; Su's post, "Mixed Chunking");
// the listing divides the summary by C (wikillm, FLASH block pseudocode,
// "summaries"), which lin_scale carries.
//
// A batched NT GEMM over the B*G chunks: A = Vt[b, e-rows, chunk tokens] and
// B = K_lin_t[b, s-rows, chunk tokens], both token-contiguous, K = C.  The
// transposed storage [e, s] is what the consumer (Q_lin P_g in the chunk
// kernel) reads as its K-contiguous B operand.
#include "gau_device.h"
#include "gau_launch.h"

namespace gau {
namespace {

constexpr int BM = 128, BN = 128;

template <typename T>
__global__ __launch_bounds__(256) void chunk_state_kernel(StateParams p) {
    extern __shared__ __align__(16) char lds[];
    using G = GemmNT<T, BM, BN>;
    constexpr int EB = Elem<T>::kBytes;
    const int G_ = p.T / p.C;
    const int mtiles = p.e / BM, ntiles = p.s / BN;
    int bid = blockIdx.x;
    const int nt = bid % ntiles; bid /= ntiles;
    const int mt = bid % mtiles; bid /= mtiles;
    const int chunk = bid;               // b * G + g
    const int b = chunk / G_, g = chunk - b * G_;
    const size_t pitch = (size_t)p.T * EB;
    const char* a = (const char*)p.Vt + (((size_t)b * p.e + mt * BM) * p.T + (size_t)g * p.C) * EB;
    const char* w = (const char*)p.Klt + (((size_t)b * p.s + nt * BN) * p.T + (size_t)g * p.C) * EB;

    f32x4_t acc[G::MB][G::NB];
    G::run(acc, a, pitch, BM, w, pitch, BN, p.C, lds);

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave >> 1, wn = wave & 1;
    constexpr int PITCH = BN * 4 + 16;
    __syncthreads();
    const float ls = p.lin_scale;
    for_each_acc(acc, lane, [&](int r, int c, float v) {
        *(float*)(lds + (wm * (BM / 2) + r) * PITCH + (wn * (BN / 2) + c) * 4) = v * ls;
    });
    __syncthreads();
    float* S = p.S + ((size_t)chunk * p.e + mt * BM) * p.s + nt * BN;
    constexpr int VPR = BN * 4 / 16;
    for (int idx = tid; idx < BM * VPR; idx += 256) {
        const int row = idx / VPR, v = idx % VPR;
        *(u32x4_t*)(S + (size_t)row * p.s + v * 4) = *(const u32x4_t*)(lds + row * PITCH + v * 16);
    }
}

template <typename T>
hipError_t launch(const StateParams& p, hipStream_t st) {
    using G = GemmNT<T, BM, BN>;
    constexpr int STAGE = BM * (BN * 4 + 16);
    constexpr int LDS = G::LDS_BYTES > STAGE ? G::LDS_BYTES : STAGE;
    const int blocks = (p.e / BM) * (p.s / BN) * p.B * (p.T / p.C);
    hipError_t e = allow_lds(chunk_state_kernel<T>, LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_state_kernel<T>, dim3(blocks), dim3(256), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_state(const StateParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? launch<bf16>(p, st) : launch<float>(p, st);
}

}  // namespace gau
