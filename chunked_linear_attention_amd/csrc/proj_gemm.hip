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
// Grid: one block per (128 rows) x (128 columns of the concatenated 2e+s
// outputs).  e and s are multiples of 128, so a block's columns lie in exactly
// one of the U, V and Z sections and its epilogue branch is uniform.
#include "gau_device.h"
#include "gau_launch.h"

namespace gau {

namespace {

constexpr int BM = 128, BN = 128;

// Stage a BM x BN tile (values from `val(row, col)`) into LDS and store it to
// global memory, row-major (rows = tokens) or transposed (rows = features).
template <typename T, bool TRANSPOSED, typename V, typename D>
__device__ __forceinline__ void stage_and_store(char* lds, V&& val, D&& dst_row, const f32x4_t (&acc)[BM / 32][BN / 32],
                                                int wm, int wn, int lane, int tid) {
    constexpr int EB = Elem<T>::kBytes;
    constexpr int ROWS = TRANSPOSED ? BN : BM;
    constexpr int COLS = TRANSPOSED ? BM : BN;
    constexpr int PITCH = COLS * EB + 16;
    __syncthreads();
    for_each_acc(acc, lane, [&](int r, int c, float v) {
        const int row = wm * (BM / 2) + r;
        const int col = wn * (BN / 2) + c;
        const float x = val(row, col, v);
        if (TRANSPOSED)
            Elem<T>::put(lds + col * PITCH + row * EB, x);
        else
            Elem<T>::put(lds + row * PITCH + col * EB, x);
    });
    __syncthreads();
    constexpr int VPR = COLS * EB / 16;  // 16-byte vectors per staged row
    for (int idx = tid; idx < ROWS * VPR; idx += 256) {
        const int row = idx / VPR;
        const int v = idx % VPR;
        char* d = dst_row(row, v * 16 / EB);
        if (d) *(u32x4_t*)d = *(const u32x4_t*)(lds + row * PITCH + v * 16);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void proj_gemm_kernel(ProjParams p) {
    extern __shared__ __align__(16) char lds[];
    using G = GemmNT<T, BM, BN>;
    const int n_tiles = (2 * p.e + p.s) / BN;
    const int nt = blockIdx.x % n_tiles;
    const int mt = blockIdx.x / n_tiles;
    const int m0 = mt * BM;
    const int n0 = nt * BN;
    int section, c0;
    const char* w;
    if (n0 < p.e) {
        section = 0; c0 = n0; w = (const char*)p.W_u;
    } else if (n0 < 2 * p.e) {
        section = 1; c0 = n0 - p.e; w = (const char*)p.W_v;
    } else {
        section = 2; c0 = n0 - 2 * p.e; w = (const char*)p.W_z;
    }
    constexpr int EB = Elem<T>::kBytes;
    const size_t pitch = (size_t)p.d * EB;
    const int rows_a = min(BM, p.M - m0);

    f32x4_t acc[G::MB][G::NB];
    G::run(acc, (const char*)p.X + (size_t)m0 * pitch, pitch, rows_a, w + (size_t)c0 * pitch, pitch, BN, p.d, lds);

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = p.M, T_ = p.T;

    if (section == 0) {
        char* U = (char*)p.U;
        stage_and_store<T, false>(
            lds, [&](int, int, float v) { return silu(v); },
            [&](int row, int col) -> char* {
                const int m = m0 + row;
                return m < M ? U + ((size_t)m * p.e + c0 + col) * EB : nullptr;
            },
            acc, wm, wn, lane, tid);
    } else if (section == 1) {
        char* Vt = (char*)p.Vt;
        stage_and_store<T, true>(
            lds, [&](int, int, float v) { return silu(v); },
            [&](int frow, int tcol) -> char* {
                const int m = m0 + tcol;
                if (m >= M) return nullptr;
                const int b = m / T_, t = m - b * T_;
                return Vt + (((size_t)b * p.e + c0 + frow) * T_ + t) * EB;
            },
            acc, wm, wn, lane, tid);
    } else {
        // Z = SiLU(H_z); head h = Z * gamma[h] + beta[h].  Heads 0..2 are
        // stored row-major, head 3 (K_lin) transposed.
        for (int h = 0; h < 4; ++h) {
            const float* gam = p.scale + h * p.s + c0;
            const float* bet = p.offset + h * p.s + c0;
            auto val = [&](int, int col, float v) { return silu(v) * gam[col] + bet[col]; };
            if (h < 3) {
                char* dst = (char*)(h == 0 ? p.Qq : h == 1 ? p.Kq : p.Ql);
                stage_and_store<T, false>(
                    lds, val,
                    [&](int row, int col) -> char* {
                        const int m = m0 + row;
                        return m < M ? dst + ((size_t)m * p.s + c0 + col) * EB : nullptr;
                    },
                    acc, wm, wn, lane, tid);
            } else {
                char* Klt = (char*)p.Klt;
                stage_and_store<T, true>(
                    lds, val,
                    [&](int frow, int tcol) -> char* {
                        const int m = m0 + tcol;
                        if (m >= M) return nullptr;
                        const int b = m / T_, t = m - b * T_;
                        return Klt + (((size_t)b * p.s + c0 + frow) * T_ + t) * EB;
                    },
                    acc, wm, wn, lane, tid);
            }
        }
    }
}

template <typename T>
hipError_t launch(const ProjParams& p, hipStream_t st) {
    using G = GemmNT<T, BM, BN>;
    constexpr int EB = Elem<T>::kBytes;
    constexpr int STAGE_T = BN * (BM * EB + 16);  // transposed staging (largest)
    constexpr int STAGE_R = BM * (BN * EB + 16);
    constexpr int LDS = G::LDS_BYTES > STAGE_T ? (G::LDS_BYTES > STAGE_R ? G::LDS_BYTES : STAGE_R)
                                               : (STAGE_T > STAGE_R ? STAGE_T : STAGE_R);
    const int n_tiles = (2 * p.e + p.s) / BN;
    const int m_tiles = (p.M + BM - 1) / BM;
    hipError_t e = allow_lds(proj_gemm_kernel<T>, LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(proj_gemm_kernel<T>, dim3(n_tiles * m_tiles), dim3(256), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_proj_gemm(const ProjParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? launch<bf16>(p, st) : launch<float>(p, st);
}

}  // namespace gau
