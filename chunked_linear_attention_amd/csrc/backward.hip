// Kernels of the layer's backward pass (gradients of <dO, O>): a batched NT
// GEMM on the shared MFMA core, a batched transpose that makes every product's
// operands K-major, and the elementwise and reduction steps of the chain rule
// through the forward's steps (the derivative of each product written out;
// the forward's steps as the pages give them: wikillm "Method" and the FLASH
// block pseudocode; Su's post, "Gated Attention" and "Mixed Chunking").  The
// order of the launches and the buffers they use are in gau_api.hip.
//
// Every reduction runs in a fixed order (two-stage sums, no atomics), so the
// gradients are bitwise reproducible.
#include "gau_device.h"
#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {
namespace {

template <typename T>
__device__ __forceinline__ float ld(const void* p, size_t i);
template <>
__device__ __forceinline__ float ld<bf16>(const void* p, size_t i) {
    return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
}
template <>
__device__ __forceinline__ float ld<float>(const void* p, size_t i) {
    return ((const float*)p)[i];
}

template <typename T>
__device__ __forceinline__ void st(void* p, size_t i, float v) {
    Elem<T>::put((char*)p + i * Elem<T>::kBytes, v);
}

template <int N> struct Bits;
template <> struct Bits<2> { using type = uint16_t; };
template <> struct Bits<4> { using type = float; };

// C[z] = alpha * A[z] B[z]^T: 64 x 64 tiles, K in chunks; operand z of a
// batch is at base + (z / div) * batch stride.
template <typename T>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmNTParams q) {
    extern __shared__ __align__(16) char lds[];
    using G = GemmCore<T, 64, 64, 2, 2>;
    constexpr int EB = Elem<T>::kBytes;
    // block -> (batch, row tile, column tile), column tiles fastest
    const int tiles = q.tm * q.tn;
    const int z = blockIdx.x / tiles, t = blockIdx.x - z * tiles;
    const int m0 = (t / q.tn) * 64, n0 = (t % q.tn) * 64;
    const char* a = (const char*)q.A + ((int64_t)(z / q.a_div) * q.a_bs + (int64_t)m0 * q.a_rp) * EB;
    const char* b = (const char*)q.B + ((int64_t)(z / q.b_div) * q.b_bs + (int64_t)n0 * q.b_rp) * EB;
    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    G::run(acc, a, (size_t)q.a_rp * EB, 64, b, (size_t)q.b_rp * EB, 64, q.K, lds);
    const int64_t cb = (int64_t)z * q.c_bs + (int64_t)m0 * q.c_rp + n0;
    const float alpha = q.alpha;
    G::for_each(acc, [&](int r, int c, float v) {
        const int64_t i = cb + (int64_t)r * q.c_rp + c;
        if (q.c_f32)
            ((float*)q.C)[i] = alpha * v;
        else
            st<T>(q.C, i, alpha * v);
    });
}

// out[z][c][r] = in[z][r][c] for 64 x 64 tiles (R, Cc multiples of 64).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(TransposeParams q) {
    using S = typename Bits<Elem<T>::kBytes>::type;
    constexpr int TP = 65;  // padded tile row
    constexpr int TILE = 64 * TP;
    __shared__ S tile[TILE];
    const int tiles = q.tr * q.tc;
    const int z = blockIdx.x / tiles, t = blockIdx.x - z * tiles;
    const int r0 = (t / q.tc) * 64, c0 = (t % q.tc) * 64;
    const S* in = (const S*)q.in + (size_t)z * q.in_bs;
    S* out = (S*)q.out + (size_t)z * q.out_bs;
    for (int k = threadIdx.x; k < 64 * 64; k += 256) {
        const int rr = k / 64, cc = k % 64;
        tile[rr * TP + cc] = in[(size_t)(r0 + rr) * q.in_rp + c0 + cc];
    }
    __syncthreads();
    for (int k = threadIdx.x; k < 64 * 64; k += 256) {
        const int cc = k / 64, rr = k % 64;
        out[(size_t)(c0 + cc) * q.out_rp + r0 + rr] = tile[rr * TP + cc];
    }
}

// dU = dY * Wq (fp32), dWq = dY * U (element type), Y = U * Wq (element type),
// with Wq = A V + Q_lin P the attention before the gate.
template <typename T>
__global__ __launch_bounds__(256) void gate_bwd_kernel(BwdElemParams q) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= q.n) return;
    const float dy = q.f1[i], w = ld<T>(q.b, i), u = ld<T>(q.c, i);
    q.f0[i] = dy * w;
    st<T>(q.o0, i, dy * u);
    st<T>(q.o1, i, u * w);
}

// dSc = 2 relu(Sc) dA * mask with relu(Sc) = sqrt(A) (A = relu(Sc)^2 as the
// forward stored it); fp32 copy for the bias gradient, element type for the
// products.  One thread per entry of the [B*G, C, C] scores.
template <typename T>
__global__ __launch_bounds__(256) void scores_bwd_kernel(BwdElemParams q) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= q.n) return;
    const int C = q.C;
    const int r = (int)((i / C) % C), c = (int)(i % C);  // query, key
    float v = 0.f;
    if (!q.causal || c <= r) v = 2.f * sqrtf(fmaxf(ld<T>(q.b, i), 0.f)) * q.f1[i];
    q.f0[i] = v;
    st<T>(q.o0, i, v);
}

// Bias gradient, stage 1: per chunk, the sums of dSc along each diagonal
// (key - query = k - (C-1)), one thread per diagonal.
__global__ __launch_bounds__(256) void relpos_partial_kernel(const float* dsc, float* part, int C) {
    const int k = blockIdx.y * 256 + threadIdx.x;
    if (k >= 2 * C - 1) return;
    const size_t z = blockIdx.x;
    const float* m = dsc + z * C * C;
    const int dd = k - (C - 1);
    float acc = 0.f;
    for (int i = 0; i < C; ++i) {
        const int j = i + dd;
        if (j >= 0 && j < C) acc += m[(size_t)i * C + j];
    }
    part[z * (2 * C - 1) + k] = acc;
}

// Column sums of a [rows, cols] fp32 array whose rows are `pitch` apart, in
// row order: out[c] = sum_r in[r * pitch + c].
__global__ __launch_bounds__(256) void colsum_kernel(const float* in, int pitch, float* out, int rows, int cols) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= cols) return;
    float acc = 0.f;
    for (int r = 0; r < rows; ++r) acc += in[(size_t)r * pitch + c];
    out[c] = acc;
}

// dS from dP (fp32 [B, G, s*e]): causal dS_h = sum_{g > h} dP_g (a reverse
// exclusive sum, walked g = G-1 .. 0), non-causal dS_h = sum_g dP_g.  Element
// type output (an MFMA operand).  One thread per state entry.
template <typename T>
__global__ __launch_bounds__(256) void scan_bwd_kernel(BwdScanParams q) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)q.B * q.es) return;
    const size_t b = idx / q.es, v = idx - b * q.es;
    const float* dp = q.dP + b * q.G * q.es + v;
    if (q.causal) {
        float run = 0.f;
        for (int g = q.G - 1; g >= 0; --g) {
            st<T>(q.dS, (b * q.G + g) * q.es + v, run);
            run += dp[(size_t)g * q.es];
        }
    } else {
        float tot = 0.f;
        for (int g = 0; g < q.G; ++g) tot += dp[(size_t)g * q.es];
        for (int g = 0; g < q.G; ++g) st<T>(q.dS, (b * q.G + g) * q.es + v, tot);
    }
}

// dZ = sum_k gamma_k dh_k over the four heads; per block of 64 tokens the
// partial sums of dh_k * Z and dh_k (for gamma and beta).  Thread per feature
// i (s threads), tokens in order.
template <typename T>
__global__ __launch_bounds__(256) void heads_bwd_kernel(BwdHeadsParams q) {
    const int i = threadIdx.x;
    if (i >= q.s) return;
    const int m0 = blockIdx.x * 64;
    float pg[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f};
    for (int m = m0; m < m0 + 64 && m < q.M; ++m) {
        const size_t o = (size_t)m * q.s + i;
        const float z = silu(ld<T>(q.Hz, (size_t)m * q.hpitch + i));
        float dz = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float dh = q.dh[k][o];
            dz += q.scale[k * q.s + i] * dh;
            pg[k] += dh * z;
            pb[k] += dh;
        }
        q.dZ[o] = dz;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        q.part[((size_t)blockIdx.x * 8 + k) * q.s + i] = pg[k];
        q.part[((size_t)blockIdx.x * 8 + 4 + k) * q.s + i] = pb[k];
    }
}

// dH = [dU | dV_local + dV_lin | dZ] * SiLU'(H), element type [M, 2e+s].
template <typename T>
__global__ __launch_bounds__(256) void silu_bwd_kernel(BwdSiluParams q) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const int W = 2 * q.e + q.s;
    if (i >= (size_t)q.M * W) return;
    const size_t m = i / W;
    const int f = (int)(i - m * W);
    float g;
    if (f < q.e)
        g = q.dU[m * q.e + f];
    else if (f < 2 * q.e)
        g = (q.dVl ? q.dVl[m * q.e + f - q.e] : 0.f) + (q.dVg ? q.dVg[m * q.e + f - q.e] : 0.f);
    else
        g = q.dZ[m * q.s + f - 2 * q.e];
    const float h = ld<T>(q.H, i);
    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-h));
    st<T>(q.dH, i, g * sg * (1.0f + h * (1.0f - sg)));
}

template <typename T>
__global__ __launch_bounds__(256) void fill_one_kernel(void* x, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) st<T>(x, i, 1.0f);
}

template <typename P>
hipError_t go(void (*k)(P), unsigned blocks, const P& p, hipStream_t st) {
    hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nt(const GemmNTParams& q0, int M, int N, int nb, bool bf, hipStream_t st) {
    GemmNTParams q = q0;
    q.tm = M / 64;
    q.tn = N / 64;
    const int64_t blocks = (int64_t)nb * q.tm * q.tn;
    if (blocks <= 0 || blocks > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    if (bf) {
        constexpr int LDS = GemmCore<bf16, 64, 64, 2, 2>::LDS_BYTES;
        hipLaunchKernelGGL(gemm_nt_kernel<bf16>, grid, dim3(256), LDS, st, q);
    } else {
        constexpr int LDS = GemmCore<float, 64, 64, 2, 2>::LDS_BYTES;
        hipLaunchKernelGGL(gemm_nt_kernel<float>, grid, dim3(256), LDS, st, q);
    }
    return hipGetLastError();
}

hipError_t launch_transpose(const TransposeParams& q0, int R, int Cc, int nb, bool bf, hipStream_t st) {
    TransposeParams q = q0;
    q.tr = R / 64;
    q.tc = Cc / 64;
    const int64_t blocks = (int64_t)nb * q.tr * q.tc;
    if (blocks <= 0 || blocks > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    if (bf)
        hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, st, q);
    else
        hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, st, q);
    return hipGetLastError();
}

hipError_t launch_fill_one(void* x, size_t n, bool bf, hipStream_t st) {
    const unsigned b = (unsigned)((n + 255) / 256);
    if (bf)
        hipLaunchKernelGGL(fill_one_kernel<bf16>, dim3(b), dim3(256), 0, st, x, n);
    else
        hipLaunchKernelGGL(fill_one_kernel<float>, dim3(b), dim3(256), 0, st, x, n);
    return hipGetLastError();
}

hipError_t launch_gate_bwd(const BwdElemParams& q, bool bf, hipStream_t st) {
    const unsigned b = (unsigned)((q.n + 255) / 256);
    return bf ? go(gate_bwd_kernel<bf16>, b, q, st) : go(gate_bwd_kernel<float>, b, q, st);
}

hipError_t launch_scores_bwd(const BwdElemParams& q, bool bf, hipStream_t st) {
    const unsigned b = (unsigned)((q.n + 255) / 256);
    return bf ? go(scores_bwd_kernel<bf16>, b, q, st) : go(scores_bwd_kernel<float>, b, q, st);
}

hipError_t launch_relpos_bwd(const float* dsc, float* part, float* drelpos, int nchunks, int C, hipStream_t st) {
    hipLaunchKernelGGL(relpos_partial_kernel, dim3(nchunks, (2 * C - 1 + 255) / 256), dim3(256), 0, st, dsc, part, C);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(colsum_kernel, dim3((2 * C - 1 + 255) / 256), dim3(256), 0, st, part, 2 * C - 1, drelpos,
                       nchunks, 2 * C - 1);
    return hipGetLastError();
}

hipError_t launch_scan_bwd(const BwdScanParams& q, bool bf, hipStream_t st) {
    const unsigned b = (unsigned)(((size_t)q.B * q.es + 255) / 256);
    return bf ? go(scan_bwd_kernel<bf16>, b, q, st) : go(scan_bwd_kernel<float>, b, q, st);
}

hipError_t launch_heads_bwd(const BwdHeadsParams& q, float* dscale, float* doffset, bool bf, hipStream_t st) {
    const int nblk = (q.M + 63) / 64;
    hipError_t e = bf ? go(heads_bwd_kernel<bf16>, (unsigned)nblk, q, st) : go(heads_bwd_kernel<float>, (unsigned)nblk, q, st);
    if (e != hipSuccess) return e;
    // part is [nblk, 8, s]: the gamma sums in rows 0..3, the beta sums in rows 4..7
    const dim3 g((4 * q.s + 255) / 256);
    hipLaunchKernelGGL(colsum_kernel, g, dim3(256), 0, st, q.part, 8 * q.s, dscale, nblk, 4 * q.s);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(colsum_kernel, g, dim3(256), 0, st, q.part + 4 * q.s, 8 * q.s, doffset, nblk, 4 * q.s);
    return hipGetLastError();
}

hipError_t launch_silu_bwd(const BwdSiluParams& q, bool bf, hipStream_t st) {
    const unsigned b = (unsigned)(((size_t)q.M * (2 * q.e + q.s) + 255) / 256);
    return bf ? go(silu_bwd_kernel<bf16>, b, q, st) : go(silu_bwd_kernel<float>, b, q, st);
}

}  // namespace gau
