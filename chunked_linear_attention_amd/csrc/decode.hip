// Incremental causal decoding: one new token of each of B sequences per call,
// with a constant-size state per sequence.
//
// Pages: the chunk-level recurrence of the causal layer (wikillm, "Method"
// steps 2-4), the decoder's linear part as a cumulative sum over chunks (Su's
// post, "Mixed Chunking") and the incremental form of linear attention
// (papercache 3.1).  The state: P, the sum of the summaries
// lin_scale * K_lin^T V of the chunks already completed (s x e, fp32), and
// the current chunk's K_quad, V and K_lin rows (C slots, the layer's element
// type).  Token t at slot j = t mod C:
//   u, v, z = SiLU(x W_u), SiLU(x W_v), SiLU(x W_z); four heads from z
//   (rotated by t with RoPE on); K_quad, V, K_lin stored in slot j;
//   quad = sum_{tau <= j} relu^2(q_quad . k_quad_tau * quad_scale + w[C-1 + tau - j]) v_tau
//   y = u * (quad + q_lin P);  o = y W_o
// and at j = C-1 the chunk's summary is added to P.
//
// Three launches per step (a fourth at a chunk's end).  Up to MFMA_MIN_B - 1
// tokens the projection and output products are GEMVs that read every
// weight once (one half wave per weight row, 16-byte loads); from
// MFMA_MIN_B on they run on the shared MFMA core as GEMMs with 64-token
// tiles.  The attention kernel reads the chunk's cached rows and P in the
// layer's element type: the fp32 state is rounded into that copy once per
// chunk, at its update (for bf16 this halves the state bytes every step
// reads, the bulk of a step's traffic at large batch, and matches the
// forward, whose prefix states are rounded to the element type too).
#include "gau_device.h"
#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {
namespace {

constexpr int BT = 8;           // tokens per pass over a weight row (GEMV)
constexpr int MFMA_MIN_B = 9;   // batch from which the products use the MFMA core (measured)

template <typename T>
__device__ __forceinline__ float ld1(const char* p);
template <>
__device__ __forceinline__ float ld1<bf16>(const char* p) {
    return __uint_as_float((uint32_t)(*(const uint16_t*)p) << 16);
}
template <>
__device__ __forceinline__ float ld1<float>(const char* p) {
    return *(const float*)p;
}

// Eight consecutive elements (16-byte aligned) as floats, and back (bf16:
// round to nearest even, as Elem<bf16>::put).
template <typename T>
__device__ __forceinline__ void ld8(const char* p, float (&v)[8]);
template <>
__device__ __forceinline__ void ld8<bf16>(const char* p, float (&v)[8]) {
    const u32x4_t w = *(const u32x4_t*)p;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
}
template <>
__device__ __forceinline__ void ld8<float>(const char* p, float (&v)[8]) {
    const f32x4_t a = *(const f32x4_t*)p, c = *(const f32x4_t*)(p + 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[k] = a[k];
        v[4 + k] = c[k];
    }
}
template <typename T>
__device__ __forceinline__ void st8(char* p, const float (&v)[8]);
template <>
__device__ __forceinline__ void st8<bf16>(char* p, const float (&v)[8]) {
    u32x4_t w;
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
    *(u32x4_t*)p = w;
}
template <>
__device__ __forceinline__ void st8<float>(char* p, const float (&v)[8]) {
    *(f32x4_t*)p = f32x4_t{v[0], v[1], v[2], v[3]};
    *(f32x4_t*)(p + 16) = f32x4_t{v[4], v[5], v[6], v[7]};
}

// Sum over the 32 lanes of a half wave.
__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

constexpr int RL = 32;  // lanes per weight row

// The elements of one 16-byte vector as floats (8 for bf16, 4 for fp32).
template <typename T>
__device__ __forceinline__ void unpack16(const u32x4_t& w, float (&v)[16 / Elem<T>::kBytes]) {
    if constexpr (Elem<T>::kBytes == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = __uint_as_float(w[k]);
    }
}

// acc[bb] = row . x[b0 + bb] for the tokens of one tile.  row: K elements,
// x: B rows of K elements, both of type T, 16-byte aligned (K is a multiple
// of 64).  The row is read in 16-byte vectors strided over the RL lanes of
// its half wave, up to U vectors per lane in flight (one pass for K <= 2048
// in bf16), each multiplied with the same vector of every token's x.
template <typename T>
__device__ __forceinline__ void row_dots(const char* row, const char* x, int K, int B, int b0, int rl,
                                         float (&acc)[BT]) {
    constexpr int EB = Elem<T>::kBytes, VE = 16 / EB;
    constexpr int U = 8;
#pragma unroll
    for (int bb = 0; bb < BT; ++bb) acc[bb] = 0.f;
    const int nv = K / VE;
    for (int v0 = rl; v0 < nv; v0 += RL * U) {
        u32x4_t w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int vi = v0 + u * RL;
            w[u] = vi < nv ? *(const u32x4_t*)(row + (size_t)vi * 16) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int bb = 0; bb < BT; ++bb) {
            if (b0 + bb >= B) break;
            const char* xb = x + (size_t)(b0 + bb) * K * EB;
            u32x4_t xv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int vi = v0 + u * RL;
                xv[u] = vi < nv ? *(const u32x4_t*)(xb + (size_t)vi * 16) : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (v0 + u * RL < nv) {
                    float a[VE], c[VE];
                    unpack16<T>(w[u], a);
                    unpack16<T>(xv[u], c);
#pragma unroll
                    for (int k = 0; k < VE; ++k) acc[bb] += a[k] * c[k];
                }
            }
        }
    }
#pragma unroll
    for (int bb = 0; bb < BT; ++bb) acc[bb] = half_sum(acc[bb]);
}

// u, v (into the cache slot) and z: one half wave per row of W_u | W_v | W_z.
template <typename T>
__global__ __launch_bounds__(256) void decode_proj_kernel(DecodeParams p) {
    constexpr int EB = Elem<T>::kBytes;
    const int lane = threadIdx.x % RL;
    const int f = blockIdx.x * 8 + threadIdx.x / RL;
    const int N = 2 * p.e + p.s;
    if (f >= N) return;
    const size_t pitch = (size_t)p.d * EB;
    const char* row = f < p.e       ? (const char*)p.W_u + (size_t)f * pitch
                      : f < 2 * p.e ? (const char*)p.W_v + (size_t)(f - p.e) * pitch
                                    : (const char*)p.W_z + (size_t)(f - 2 * p.e) * pitch;
    for (int b0 = 0; b0 < p.B; b0 += BT) {
        float acc[BT];
        row_dots<T>(row, (const char*)p.x, p.d, p.B, b0, lane, acc);
        if (lane != 0) continue;
#pragma unroll
        for (int bb = 0; bb < BT; ++bb) {
            const int b = b0 + bb;
            if (b >= p.B) break;
            const float h = silu(acc[bb]);
            if (f < p.e)
                p.u[(size_t)b * p.e + f] = h;
            else if (f < 2 * p.e)
                Elem<T>::put((char*)p.V + (((size_t)b * p.C + p.j) * p.e + (f - p.e)) * EB, h);
            else
                p.z[(size_t)b * p.s + (f - 2 * p.e)] = h;
        }
    }
}

// The value x takes once stored in T (the cache holds the heads in the
// layer's element type, as the forward's workspace does).
template <typename T>
__device__ __forceinline__ float as_stored(float x);
template <>
__device__ __forceinline__ float as_stored<bf16>(float x) {
    return __uint_as_float((uint32_t)f32_to_bf16(x) << 16);
}
template <>
__device__ __forceinline__ float as_stored<float>(float x) {
    return x;
}

// FV consecutive elements as floats, and back.
template <typename T, int FV>
__device__ __forceinline__ void ldn(const char* p, float (&v)[FV]) {
    if constexpr (FV == 8) {
        ld8<T>(p, v);
    } else {
        static_assert(FV == 1, "1 or 8 features per thread");
        v[0] = ld1<T>(p);
    }
}
template <typename T, int FV>
__device__ __forceinline__ void stn(char* p, const float (&v)[FV]) {
    if constexpr (FV == 8) {
        st8<T>(p, v);
    } else {
#pragma unroll
        for (int k = 0; k < FV; ++k) Elem<T>::put(p + k * Elem<T>::kBytes, v[k]);
    }
}

// The token's four heads, and y = u * (quad + q_lin P) for 64 * FV of its
// features.  Every block of the token forms the heads from z (s/2 pairs,
// turned by position t with RoPE on) into LDS, uses its own K_quad for the
// score of slot j, and the first block writes K_quad and K_lin into the
// cache slot.  The 256 threads then form 4 groups of 64 that split the sums
// over the chunk slots and the state rows; a thread owns FV consecutive
// features, read as one vector per slot or state row.  More features per
// block (FV = 8: 16-byte loads, e/512 blocks per token) cut the score work,
// which every block of a token repeats, and the load instructions; fewer
// (FV = 1: e/64 blocks per token) spread a small batch over more CUs.
// Measured per step at d=768, e=1536, C=256, bf16 (FV = 1 / 8): B=1 21.8 /
// 24.3 us, B=32 37.1 / 38.9, B=128 67.5 / 48.9.
template <typename T, int FV>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeParams p) {
    constexpr int EB = Elem<T>::kBytes;
    constexpr int FT = 64 * FV;            // features per block
    constexpr int RIF = FV == 1 ? 8 : 4;   // rows in flight per thread
    constexpr int PARTS = 2 * 4 * FT;      // [quad | lin][group][feature]
    __shared__ float alpha[512];
    __shared__ float qq[256];
    __shared__ float ql[256];
    __shared__ float kq[256];
    __shared__ float part[PARTS];
    const int ftiles = (p.e + FT - 1) / FT;
    const int b = blockIdx.x / ftiles;
    const int ft = blockIdx.x - b * ftiles;
    const int f0 = ft * FT;
    const int tid = threadIdx.x;
    const int j = p.j;
    const int half = p.s / 2;
    for (int i = tid; i < half; i += 256) {
        const float zl = p.z[(size_t)b * p.s + i], zh = p.z[(size_t)b * p.s + i + half];
        double c = 1.0, sn = 0.0;
        if (p.rope) sincos((double)p.t * rope_theta(i, half), &sn, &c);
        for (int h = 0; h < 4; ++h) {
            const float* g = p.scale + h * p.s;
            const float* o = p.offset + h * p.s;
            const double lo = (double)(zl * g[i] + o[i]), hi = (double)(zh * g[i + half] + o[i + half]);
            const float rl = as_stored<T>((float)(lo * c - hi * sn)), rh = as_stored<T>((float)(hi * c + lo * sn));
            float* dst = h == 0 ? qq : h == 1 ? kq : h == 2 ? ql : nullptr;
            if (dst) {
                dst[i] = rl;
                dst[i + half] = rh;
            }
            if (ft == 0 && (h == 1 || h == 3)) {
                char* k = (char*)(h == 1 ? p.Kq : p.Kl) + (((size_t)b * p.C + j) * p.s) * EB;
                Elem<T>::put(k + (size_t)i * EB, rl);
                Elem<T>::put(k + (size_t)(i + half) * EB, rh);
            }
        }
    }
    __syncthreads();
    // scores of the chunk's slots 0 .. j (slot j from this block's own K_quad):
    // one thread per slot, its K_quad row read as 16-byte vectors all in
    // flight, each batch's query values read from LDS as 16-byte vectors
    // before its products (one wait per batch instead of one per vector)
    for (int tau = tid; tau <= (p.local ? j : -1); tau += 256) {
        float acc = 0.f;
        const float rpos = p.relpos[p.C - 1 + tau - j];
        if (tau == j) {
            for (int i = 0; i < p.s; ++i) acc += qq[i] * kq[i];
        } else {
            const char* k = (const char*)p.Kq + (((size_t)b * p.C + tau) * p.s) * EB;
            constexpr int VE = 16 / EB;  // elements per vector
            for (int i0 = 0; i0 < p.s; i0 += 8 * VE) {  // s is a multiple of 128
                u32x4_t w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) w[u] = *(const u32x4_t*)(k + (size_t)(i0 + u * VE) * EB);
                float qv[8 * VE];
#pragma unroll
                for (int x = 0; x < 2 * VE; ++x) {
                    const f32x4_t q4 = *(const f32x4_t*)(qq + i0 + 4 * x);
                    qv[4 * x] = q4.x, qv[4 * x + 1] = q4.y, qv[4 * x + 2] = q4.z, qv[4 * x + 3] = q4.w;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = u * VE;
                    if constexpr (EB == 2) {
                        const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc += qv[i + 2 * q] * __uint_as_float(ww[q] << 16) +
                                   qv[i + 2 * q + 1] * __uint_as_float(ww[q] & 0xFFFF0000u);
                    } else {
                        acc += qv[i] * __uint_as_float(w[u].x) + qv[i + 1] * __uint_as_float(w[u].y) +
                               qv[i + 2] * __uint_as_float(w[u].z) + qv[i + 3] * __uint_as_float(w[u].w);
                    }
                }
            }
        }
        const float x = acc * p.qs + rpos;
        alpha[tau] = x > 0.f ? x * x : 0.f;
    }
    __syncthreads();
    const int g = tid / 64, fl = tid % 64;  // group, thread inside the group
    const int f = f0 + fl * FV;             // first of this thread's 8 features
    float quad[FV] = {}, lin[FV] = {};
    if (f < p.e) {
        const char* V = (const char*)p.V + ((size_t)b * p.C * p.e + f) * EB;
        const size_t vs = (size_t)p.e * EB;
        const int jl = p.local ? j : -1;  // last slot of the local term
        int tau = g;
        for (; tau + 4 * (RIF - 1) <= jl; tau += 4 * RIF) {  // RIF rows in flight
            float v[RIF][FV];
#pragma unroll
            for (int u = 0; u < RIF; ++u) ldn<T, FV>(V + (size_t)(tau + 4 * u) * vs, v[u]);
#pragma unroll
            for (int u = 0; u < RIF; ++u)
#pragma unroll
                for (int k = 0; k < FV; ++k) quad[k] += alpha[tau + 4 * u] * v[u][k];
        }
        for (; tau <= jl; tau += 4) {
            float v[FV];
            ldn<T, FV>(V + (size_t)tau * vs, v);
#pragma unroll
            for (int k = 0; k < FV; ++k) quad[k] += alpha[tau] * v[k];
        }
        // the state in the element type (the copy rounded at each chunk end)
        const char* P = (const char*)p.Pr + ((size_t)b * p.s * p.e + f) * EB;
        for (int i = g; i < (p.global ? p.s : 0); i += 4 * RIF) {  // s is a multiple of 128
            float w[RIF][FV];
#pragma unroll
            for (int u = 0; u < RIF; ++u) ldn<T, FV>(P + (size_t)(i + 4 * u) * p.e * EB, w[u]);
#pragma unroll
            for (int u = 0; u < RIF; ++u)
#pragma unroll
                for (int k = 0; k < FV; ++k) lin[k] += ql[i + 4 * u] * w[u][k];
        }
    }
#pragma unroll
    for (int k = 0; k < FV; ++k) {
        part[g * FT + fl * FV + k] = quad[k];
        part[4 * FT + g * FT + fl * FV + k] = lin[k];
    }
    __syncthreads();
    if (g == 0 && f < p.e) {
        float y[FV];
#pragma unroll
        for (int k = 0; k < FV; ++k) {
            float q = 0.f, l = 0.f;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {  // fixed order: 0, 1, 2, 3
                q += part[gg * FT + fl * FV + k];
                l += part[4 * FT + gg * FT + fl * FV + k];
            }
            y[k] = p.u[(size_t)b * p.e + f + k] * (q + l);
        }
        stn<T, FV>((char*)p.y + ((size_t)b * p.e + f) * EB, y);
    }
}

// o = y W_o: one half wave per row of W_o^T ([d, e], row n contiguous over e).
template <typename T>
__global__ __launch_bounds__(256) void decode_out_kernel(DecodeParams p) {
    constexpr int EB = Elem<T>::kBytes;
    const int lane = threadIdx.x % RL;
    const int n = blockIdx.x * 8 + threadIdx.x / RL;
    if (n >= p.d) return;
    const char* row = (const char*)p.W_o + (size_t)n * p.e * EB;
    for (int b0 = 0; b0 < p.B; b0 += BT) {
        float acc[BT];
        row_dots<T>(row, (const char*)p.y, p.e, p.B, b0, lane, acc);
        if (lane != 0) continue;
#pragma unroll
        for (int bb = 0; bb < BT; ++bb) {
            if (b0 + bb >= p.B) break;
            Elem<T>::put((char*)p.o + ((size_t)(b0 + bb) * p.d + n) * EB, acc[bb]);
        }
    }
}

// P += lin_scale * sum_tau k_lin_tau v_tau^T over the completed chunk's C
// slots: a 64 x 64 tile of (state row i, feature f) per block, the slots in
// steps of 16 staged through LDS, each thread 4 x 4 entries (rows ty + 16 r,
// features tx + 16 c), slots summed in order.
template <typename T>
__global__ __launch_bounds__(256) void decode_state_kernel(DecodeParams p) {
    constexpr int EB = Elem<T>::kBytes;
    constexpr int TI = 64, TF = 64, TK = 16;
    constexpr int KT = TK * TI, VT = TK * TF;
    __shared__ float kt[KT];
    __shared__ float vt[VT];
    const int itiles = p.s / TI, ftiles = (p.e + TF - 1) / TF;
    const int blk = blockIdx.x;
    const int b = blk / (itiles * ftiles);
    const int r = blk - b * itiles * ftiles;
    const int i0 = (r / ftiles) * TI, f0 = (r % ftiles) * TF;
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    const char* kl = (const char*)p.Kl + (size_t)b * p.C * p.s * EB;
    const char* v = (const char*)p.V + (size_t)b * p.C * p.e * EB;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < p.C; k0 += TK) {
        __syncthreads();
        for (int x = tid; x < KT; x += 256) {  // [slot][row]
            const int kk = x / TI, ii = x % TI;
            kt[x] = ld1<T>(kl + ((size_t)(k0 + kk) * p.s + i0 + ii) * EB);
        }
        for (int x = tid; x < VT; x += 256) {  // [slot][feature]
            const int kk = x / TF, ff = x % TF;
            vt[x] = f0 + ff < p.e ? ld1<T>(v + ((size_t)(k0 + kk) * p.e + f0 + ff) * EB) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) acc[rr][cc] += kt[kk * TI + ty + 16 * rr] * vt[kk * TF + tx + 16 * cc];
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int f = f0 + tx + 16 * cc;
            if (f < p.e) {
                const size_t k = ((size_t)b * p.s + i0 + ty + 16 * rr) * p.e + f;
                const float x = p.P[k] + p.ls * acc[rr][cc];
                p.P[k] = x;
                if constexpr (EB == 2) Elem<T>::put((char*)p.Pr + k * EB, x);  // the copy the steps read
            }
        }
}

// The projection as a GEMM for larger batches: 64 rows of W_u | W_v | W_z
// (the tile lies in one of them: e and s are multiples of 64) times 64
// tokens, K = d; epilogue as decode_proj_kernel.
template <typename T>
__global__ __launch_bounds__(256) void decode_proj_mfma_kernel(DecodeParams p) {
    extern __shared__ __align__(16) char lds[];
    using G = GemmCore<T, 64, 64, 2, 2>;
    constexpr int EB = Elem<T>::kBytes;
    const int ntiles = (2 * p.e + p.s) / 64;
    const int nt = blockIdx.x % ntiles, bt = blockIdx.x / ntiles;
    const int f0 = nt * 64, b0 = bt * 64;
    const size_t pitch = (size_t)p.d * EB;
    const char* w = f0 < p.e       ? (const char*)p.W_u + (size_t)f0 * pitch
                    : f0 < 2 * p.e ? (const char*)p.W_v + (size_t)(f0 - p.e) * pitch
                                   : (const char*)p.W_z + (size_t)(f0 - 2 * p.e) * pitch;
    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    G::run(acc, w, pitch, 64, (const char*)p.x + (size_t)b0 * pitch, pitch, min(64, p.B - b0), p.d, lds);
    G::for_each(acc, [&](int row, int col, float v) {
        const int f = f0 + row, b = b0 + col;
        if (b >= p.B) return;
        const float h = silu(v);
        if (f < p.e)
            p.u[(size_t)b * p.e + f] = h;
        else if (f < 2 * p.e)
            Elem<T>::put((char*)p.V + (((size_t)b * p.C + p.j) * p.e + (f - p.e)) * EB, h);
        else
            p.z[(size_t)b * p.s + (f - 2 * p.e)] = h;
    });
}

// o = y W_o as a GEMM for larger batches: 32 rows of W_o^T times 64 tokens,
// K = e (two waves).
template <typename T>
__global__ __launch_bounds__(128) void decode_out_mfma_kernel(DecodeParams p) {
    extern __shared__ __align__(16) char lds[];
    using G = GemmCore<T, 32, 64, 1, 2>;
    constexpr int EB = Elem<T>::kBytes;
    const int ntiles = p.d / 32;
    const int nt = blockIdx.x % ntiles, bt = blockIdx.x / ntiles;
    const int n0 = nt * 32, b0 = bt * 64;
    const size_t pitch = (size_t)p.e * EB;
    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    G::run(acc, (const char*)p.W_o + (size_t)n0 * pitch, pitch, 32, (const char*)p.y + (size_t)b0 * pitch, pitch,
           min(64, p.B - b0), p.e, lds);
    G::for_each(acc, [&](int row, int col, float v) {
        const int b = b0 + col;
        if (b < p.B) Elem<T>::put((char*)p.o + ((size_t)b * p.d + n0 + row) * EB, v);
    });
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* x, size_t n) {
    const size_t k = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (k < n) x[k] = 0.f;
}

// 8 features per thread in the attention kernel once that grid (B * e / 512
// blocks) still gives every one of the 256 CUs a block.
bool attn_wide(int B, int e) { return (long)B * ((e + 511) / 512) >= 256; }

template <typename T>
hipError_t step(const DecodeParams& p, hipStream_t st) {
    const bool mfma = p.B >= MFMA_MIN_B;
    const unsigned btiles = (unsigned)((p.B + 63) / 64);
    if (mfma) {
        constexpr int LDS = GemmCore<T, 64, 64, 2, 2>::LDS_BYTES;
        hipLaunchKernelGGL(decode_proj_mfma_kernel<T>, dim3((unsigned)((2 * p.e + p.s) / 64) * btiles), dim3(256),
                           LDS, st, p);
    } else {
        hipLaunchKernelGGL(decode_proj_kernel<T>, dim3((unsigned)((2 * p.e + p.s + 7) / 8)), dim3(256), 0, st, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (attn_wide(p.B, p.e))
        hipLaunchKernelGGL((decode_attn_kernel<T, 8>), dim3((unsigned)(p.B * ((p.e + 511) / 512))), dim3(256), 0, st,
                           p);
    else
        hipLaunchKernelGGL((decode_attn_kernel<T, 1>), dim3((unsigned)(p.B * ((p.e + 63) / 64))), dim3(256), 0, st,
                           p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (mfma) {
        constexpr int LDS = GemmCore<T, 32, 64, 1, 2>::LDS_BYTES;
        hipLaunchKernelGGL(decode_out_mfma_kernel<T>, dim3((unsigned)(p.d / 32) * btiles), dim3(128), LDS, st, p);
    } else {
        hipLaunchKernelGGL(decode_out_kernel<T>, dim3((unsigned)((p.d + 7) / 8)), dim3(256), 0, st, p);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.j == p.C - 1 && p.global) {
        hipLaunchKernelGGL(decode_state_kernel<T>, dim3((unsigned)(p.B * (p.s / 64) * ((p.e + 63) / 64))), dim3(256),
                           0, st, p);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

hipError_t launch_decode_step(const DecodeParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? step<bf16>(p, st) : step<float>(p, st);
}

hipError_t launch_fill_zero(float* x, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, n);
    return hipGetLastError();
}

}  // namespace gau
