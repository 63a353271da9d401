// Rotary position embedding of the four heads, in place after the projection,
// and the RoPE-built relative-position bias vector.
//
// Pages: the listing rotates the queries and keys after the scale+offset,
// over positions counted through the whole sequence, not restarted per chunk
// (wikillm, FLASH block pseudocode and "Paper vs code"); Su's post notes that
// every FLASH model in the paper uses RoPE.  The rotation itself is not
// printed; the reading here takes the frequency schedule and half-split
// layout of the sinusoid helper the pages print (papercache, appendix D,
// _get_scaledsin): the pair (h_i, h_{i+s/2}) of a head vector at position t
// turns by t * theta_i, theta_i = 10000^(-i/(s/2)).
//
// The bias: for chunk lengths of 512 and more, Code 4 (papercache, appendix D)
// builds the Toeplitz matrix as rope(a)_m . rope(b)_n from two learned
// vectors; the product depends only on n - m, so one 2n-1 vector w with
// w[n-1 + d] = a . rope(b, d) carries it, and the layer takes it as its
// relpos argument unchanged.
//
// Angles t * theta_i reach about 10^4 rad at the sequence lengths here, where
// an fp32 product would lose 4 decimal digits: they are formed in fp64 and
// reduced to [-pi, pi] there, and only the reduced angle's cosine and sine
// are fp32.  The heads are read and written in the layer's element type: two
// memory-bound passes, one over the three token-major heads and one over
// K_lin_t, each with coalesced 4-element vectors.
#include "gau_device.h"
#include "gau_launch.h"

namespace gau {
namespace {

template <typename T>
__device__ __forceinline__ void get4(const char* p, double (&v)[4]);
template <>
__device__ __forceinline__ void get4<bf16>(const char* p, double (&v)[4]) {
    const u32x2_t w = *(const u32x2_t*)p;
    v[0] = __uint_as_float(w.x << 16);
    v[1] = __uint_as_float(w.x & 0xFFFF0000u);
    v[2] = __uint_as_float(w.y << 16);
    v[3] = __uint_as_float(w.y & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void get4<float>(const char* p, double (&v)[4]) {
    const f32x4_t w = *(const f32x4_t*)p;
    v[0] = w.x, v[1] = w.y, v[2] = w.z, v[3] = w.w;
}

template <typename T>
__device__ __forceinline__ void put4(char* p, const double (&v)[4]);
template <>
__device__ __forceinline__ void put4<bf16>(char* p, const double (&v)[4]) {
    *(u32x2_t*)p = u32x2_t{pack_bf16x2((float)v[0], (float)v[1]), pack_bf16x2((float)v[2], (float)v[3])};
}
template <>
__device__ __forceinline__ void put4<float>(char* p, const double (&v)[4]) {
    *(f32x4_t*)p = f32x4_t{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// (lo, hi) <- (lo cos - hi sin, hi cos + lo sin), element-wise
__device__ __forceinline__ void turn(double (&lo)[4], double (&hi)[4], const double (&c)[4], const double (&s)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const double a = lo[k], b = hi[k];
        lo[k] = a * c[k] - b * s[k];
        hi[k] = b * c[k] + a * s[k];
    }
}

// cos and sin of t * theta: the angle formed in fp64 and reduced to
// [-pi, pi] there, the reduced angle's cosine and sine in fp32 (about 1 ulp).
__device__ __forceinline__ void turn_cs(double t, double theta, double& c, double& s) {
    constexpr double kTwoPi = 6.283185307179586476925287;
    const double a = t * theta;
    const float r = (float)(a - kTwoPi * rint(a / kTwoPi));
    float sf, cf;
    sincosf(r, &sf, &cf);
    c = cf;
    s = sf;
}

// Token-major heads Q_quad, K_quad, Q_lin [M, s]: one thread per token and
// four consecutive pair indices i0 .. i0+3 (consecutive threads along the
// row).  The block's pair frequencies come from an LDS table (fp64).
template <typename T>
__global__ __launch_bounds__(256) void rope_rows_kernel(RopeParams p) {
    constexpr int EB = Elem<T>::kBytes;
    __shared__ double theta[128];
    const int half = p.s / 2;
    for (int i = threadIdx.x; i < half; i += 256) theta[i] = rope_theta(i, half);
    __syncthreads();
    const int groups = half / 4;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)p.M * groups) return;
    const int m = (int)(idx / groups);
    const int i0 = (int)(idx - (long)m * groups) * 4;
    const double t = (double)(m % p.T);
    double c[4], s[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) turn_cs(t, theta[i0 + k], c[k], s[k]);
    void* heads[3] = {p.Qq, p.Kq, p.Ql};
#pragma unroll
    for (int h = 0; h < 3; ++h) {
        char* row = (char*)heads[h] + (size_t)m * p.s * EB;
        double lo[4], hi[4];
        get4<T>(row + (size_t)i0 * EB, lo);
        get4<T>(row + (size_t)(i0 + half) * EB, hi);
        turn(lo, hi, c, s);
        put4<T>(row + (size_t)i0 * EB, lo);
        put4<T>(row + (size_t)(i0 + half) * EB, hi);
    }
}

// K_lin_t [B, s, T]: one thread per sequence, pair index i and four
// consecutive tokens t0 .. t0+3 (consecutive threads along the tokens).
template <typename T>
__global__ __launch_bounds__(256) void rope_cols_kernel(RopeParams p) {
    constexpr int EB = Elem<T>::kBytes;
    const int half = p.s / 2;
    const int tg = p.T / 4;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)p.B * half * tg) return;
    const int b = (int)(idx / ((long)half * tg));
    const long r = idx - (long)b * half * tg;
    const int i = (int)(r / tg);
    const int t0 = (int)(r - (long)i * tg) * 4;
    const double th = rope_theta(i, half);  // uniform over most of the block
    double c[4], s[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) turn_cs((double)(t0 + k), th, c[k], s[k]);
    char* base = (char*)p.Klt + ((size_t)b * p.s * p.T + t0) * EB;
    char* lo_p = base + (size_t)i * p.T * EB;
    char* hi_p = base + (size_t)(i + half) * p.T * EB;
    double lo[4], hi[4];
    get4<T>(lo_p, lo);
    get4<T>(hi_p, hi);
    turn(lo, hi, c, s);
    put4<T>(lo_p, lo);
    put4<T>(hi_p, hi);
}

// w[n-1 + d] = sum_i a_i (b_i cos - b_{i+h} sin) + a_{i+h} (b_{i+h} cos + b_i sin),
// angle d * theta_i, for d = -(n-1) .. n-1.
__global__ __launch_bounds__(256) void rope_relpos_kernel(const float* a, const float* b, int n, int dim,
                                                         float* w) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= 2 * n - 1) return;
    const int half = dim / 2;
    const double d = (double)(k - (n - 1));
    double acc = 0.0;
    for (int i = 0; i < half; ++i) {
        double sn, cs;
        sincos(d * rope_theta(i, half), &sn, &cs);
        const double ai = a[i], ah = a[i + half], bi = b[i], bh = b[i + half];
        acc += cs * (ai * bi + ah * bh) + sn * (ah * bi - ai * bh);
    }
    w[k] = (float)acc;
}

template <typename T>
hipError_t launch(const RopeParams& p, hipStream_t st) {
    const long rows = (long)p.M * (p.s / 8);
    hipLaunchKernelGGL(rope_rows_kernel<T>, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long cols = (long)p.B * (p.s / 2) * (p.T / 4);
    hipLaunchKernelGGL(rope_cols_kernel<T>, dim3((unsigned)((cols + 255) / 256)), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_heads(const RopeParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? launch<bf16>(p, st) : launch<float>(p, st);
}

hipError_t launch_rope_relpos(const float* a, const float* b, int n, int dim, float* relpos, hipStream_t st) {
    hipLaunchKernelGGL(rope_relpos_kernel, dim3((unsigned)((2 * n - 1 + 255) / 256)), dim3(256), 0, st, a, b, n,
                       dim, relpos);
    return hipGetLastError();
}

}  // namespace gau
