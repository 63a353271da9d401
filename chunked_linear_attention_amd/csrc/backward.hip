// Kernels of the layer's backward pass (gradients of <dO, O>): a batched NT
// GEMM on the shared MFMA core (its operands K-major or MN-major, optionally
// over two K segments, with a fused SiLU-derivative epilogue), a batched
// transpose for the few small tensors still made K-major, and the
// elementwise and reduction
// steps of the chain rule through the forward's steps (the derivative of each
// product written out; the forward's steps as the pages give them: wikillm
// "Method" and the FLASH block pseudocode; Su's post, "Gated Attention" and
// "Mixed Chunking").  The order of the launches and the buffers they use are
// in gau_api.hip.
//
// Every reduction runs in a fixed order (split sums written to scratch and
// added in index order; no atomics), so the gradients are bitwise
// reproducible.
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

// Eight consecutive elements at index i (a multiple of 8, 16-byte aligned).
template <typename T>
__device__ __forceinline__ void load8(const void* p, int64_t i, float (&v)[8]) {
    if constexpr (Elem<T>::kBytes == 2) {
        const u32x4_t x = *(const u32x4_t*)((const uint16_t*)p + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(x[k] << 16);
            v[2 * k + 1] = __uint_as_float(x[k] & 0xFFFF0000u);
        }
    } else {
        const f32x4_t a = *(const f32x4_t*)((const float*)p + i);
        const f32x4_t b = *(const f32x4_t*)((const float*)p + i + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = a[k];
            v[4 + k] = b[k];
        }
    }
}

// Eight consecutive elements as loaded (one 16-byte vector for bf16, two for
// fp32), and as floats.
template <typename T> struct Raw8 { u32x4_t x; };
template <> struct Raw8<float> { f32x4_t a, b; };
template <typename T>
__device__ __forceinline__ void load8raw(const void* p, int64_t i, Raw8<T>& r) {
    if constexpr (Elem<T>::kBytes == 2) {
        r.x = *(const u32x4_t*)((const uint16_t*)p + i);
    } else {
        r.a = *(const f32x4_t*)((const float*)p + i);
        r.b = *(const f32x4_t*)((const float*)p + i + 4);
    }
}
template <typename T>
__device__ __forceinline__ void unpack8(const Raw8<T>& r, float (&v)[8]) {
    if constexpr (Elem<T>::kBytes == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(r.x[k] << 16);
            v[2 * k + 1] = __uint_as_float(r.x[k] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = r.a[k];
            v[4 + k] = r.b[k];
        }
    }
}

template <typename T>
__device__ __forceinline__ void store8(void* p, int64_t i, const float (&v)[8]) {
    if constexpr (Elem<T>::kBytes == 2) {
        u32x4_t x;
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = (uint32_t)f32_to_bf16(v[2 * k]) | ((uint32_t)f32_to_bf16(v[2 * k + 1]) << 16);
        *(u32x4_t*)((uint16_t*)p + i) = x;
    } else {
        *(f32x4_t*)((float*)p + i) = f32x4_t{v[0], v[1], v[2], v[3]};
        *(f32x4_t*)((float*)p + i + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
    }
}

// C[z] = alpha * (A[z] B[z]^T + A2[z] B2[z]^T) on BT x BT tiles, then the
// epilogue EPI (GemmNTParams).  TA, TB: MN-major A, B in the first segment;
// TA2, TB2 in the second (its own K loop into the same accumulators).
template <typename T, int BT, int EPI, bool TA, bool TB, bool TA2, bool TB2>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmNTParams q) {
    extern __shared__ __align__(16) char lds[];
    using G = GemmCore<T, BT, BT, 2, 2, 2, 0, 2, TA, TB>;
    using G2 = GemmCore<T, BT, BT, 2, 2, 2, 0, 2, TA2, TB2>;
    constexpr int EB = Elem<T>::kBytes;
    // block -> (batch, row tile, column tile), column tiles fastest, the
    // logical order spread over the XCDs in contiguous ranges (the tiles of
    // one batch entry share their operands in one L2)
    const int tiles = q.tm * q.tn;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int z = bid / tiles, t = bid - z * tiles;
    const int m0 = (t / q.tn) * BT, n0 = (t % q.tn) * BT;
    if (q.skip_upper && n0 >= m0 + BT) return;  // wholly above the diagonal: never read
    const int64_t zs = z / q.zg, zc = z - zs * q.zg;
    // first element of an operand's tile: row r0 of a K-major operand, column
    // r0 of an MN-major one
    auto tile = [&](const void* base, int64_t bsq, int64_t bs, int rp, bool mn_major, int r0) {
        return (const char*)base + (zs * bsq + zc * bs + (mn_major ? (int64_t)r0 : (int64_t)r0 * rp)) * EB;
    };
    const int64_t cb = (int64_t)z * q.c_bs + (int64_t)m0 * q.c_rp + n0;
    // SiLU-derivative epilogue: each thread takes ITERS runs of 8 consecutive
    // columns; their pre-activations are loaded before the K loop, so that
    // the memory latency overlaps it
    constexpr int PER_ROW = BT / 8, ITERS = BT * PER_ROW / 256;
    Raw8<T> hr[EPI == EPI_SILU ? ITERS : 1];
    if constexpr (EPI == EPI_SILU) {
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int k = threadIdx.x + it * 256, r = k / PER_ROW, c = (k % PER_ROW) * 8;
            load8raw<T>(q.H, cb + (int64_t)r * q.c_rp + c, hr[it]);
        }
    }
    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    // first K index of segment 1 (a K row of an MN-major operand, an element
    // of a K-major one's rows)
    const int k0 = q.k_from_row ? m0 : 0;
    G::run(acc, tile(q.A, q.a_bsq, q.a_bs, q.a_rp, TA, m0) + (TA ? (int64_t)k0 * q.a_rp : k0) * EB,
           (size_t)q.a_rp * EB, BT, tile(q.B, q.b_bsq, q.b_bs, q.b_rp, TB, n0) + (TB ? (int64_t)k0 * q.b_rp : k0) * EB,
           (size_t)q.b_rp * EB, BT, q.K - k0, lds);
    if (q.K2 > 0)
        G2::run(acc, tile(q.A2, q.a2_bsq, q.a2_bs, q.a2_rp, TA2, m0), (size_t)q.a2_rp * EB, BT,
                tile(q.B2, q.b2_bsq, q.b2_bs, q.b2_rp, TB2, n0), (size_t)q.b2_rp * EB, BT, q.K2, lds);
    const float alpha = q.alpha;
    if constexpr (EPI == EPI_STORE) {
        G::for_each(acc, [&](int r, int c, float v) {
            const int64_t i = cb + (int64_t)r * q.c_rp + c;
            if (q.c_f32)
                ((float*)q.C)[i] = alpha * v;
            else
                st<T>(q.C, i, alpha * v);
        });
    } else {
        // the tile (times alpha) through LDS, then 8 consecutive columns per
        // thread: 16-byte loads of the inputs and stores of the outputs
        float* tile = (float*)lds;
        G::for_each(acc, [&](int r, int c, float v) { tile[r * BT + c] = alpha * v; });
        __syncthreads();
        static_assert(BT * PER_ROW % 256 == 0, "whole runs per thread");
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int k = threadIdx.x + it * 256, r = k / PER_ROW, c = (k % PER_ROW) * 8;
            float v[8], h[8];
            const f32x4_t v0 = *(const f32x4_t*)(tile + r * BT + c);
            const f32x4_t v1 = *(const f32x4_t*)(tile + r * BT + c + 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                v[u] = v0[u];
                v[4 + u] = v1[u];
            }
            const int64_t i = cb + (int64_t)r * q.c_rp + c;
            unpack8<T>(hr[it], h);
            float o[8];
            static_assert(EPI == EPI_SILU, "epilogues: store, SiLU derivative");
#pragma unroll
            for (int u = 0; u < 8; ++u) o[u] = v[u] * silu_grad(h[u]);
            store8<T>(q.C, i, o);
        }
    }
}

// out[z][c][r] = in[z][r][c] on 64 x 64 tiles (R, Cc multiples of 64), rows
// read and written as 16-byte vectors, the tile turned in LDS.  bf16: each
// thread reads 8 columns of two adjacent rows and writes the 8 (even row, odd
// row) pairs as 32-bit words to LDS, column-major, so that an output vector
// (8 rows of one column) is one 16-byte LDS read.
template <typename T>
__device__ __forceinline__ void transpose_block(const TransposeParams& q, int bid) {
    const int tiles = q.tr * q.tc;
    const int z = bid / tiles, t = bid - z * tiles;
    const int r0 = (t / q.tc) * 64, c0 = (t % q.tc) * 64;
    if constexpr (Elem<T>::kBytes == 2) {
        constexpr int WP = 36;          // LDS words per column (32 row pairs + pad)
        constexpr int TILE = 64 * WP;
        __shared__ uint32_t tile[TILE];
        const uint16_t* in = (const uint16_t*)q.in + (size_t)z * q.in_bs;
        uint16_t* out = (uint16_t*)q.out + (size_t)z * q.out_bs;
        const int rp = threadIdx.x / 8, cg = (threadIdx.x % 8) * 8;
        const u32x4_t a = *(const u32x4_t*)(in + (size_t)(r0 + 2 * rp) * q.in_rp + c0 + cg);
        const u32x4_t b = *(const u32x4_t*)(in + (size_t)(r0 + 2 * rp + 1) * q.in_rp + c0 + cg);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            tile[(cg + 2 * k) * WP + rp] = (a[k] & 0xFFFFu) | (b[k] << 16);
            tile[(cg + 2 * k + 1) * WP + rp] = (a[k] >> 16) | (b[k] & 0xFFFF0000u);
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 64; p += 32) {
            const int c = p + threadIdx.x / 8, part = threadIdx.x % 8;
            const u32x4_t y = *(const u32x4_t*)(tile + c * WP + part * 4);
            *(u32x4_t*)(out + (size_t)(c0 + c) * q.out_rp + r0 + part * 8) = y;
        }
    } else {
        constexpr int TP = 64 + 4;  // padded LDS row (floats)
        constexpr int TILE = 64 * TP;
        __shared__ float tile[TILE];
        const float* in = (const float*)q.in + (size_t)z * q.in_bs;
        float* out = (float*)q.out + (size_t)z * q.out_bs;
        const int vr = threadIdx.x / 16, vc = (threadIdx.x % 16) * 4;
#pragma unroll
        for (int p = 0; p < 64; p += 16) {
            const f32x4_t x = *(const f32x4_t*)(in + (size_t)(r0 + p + vr) * q.in_rp + c0 + vc);
#pragma unroll
            for (int k = 0; k < 4; ++k) tile[(vc + k) * TP + p + vr] = x[k];
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 64; p += 16) {
            const int c = p + vr;
            const f32x4_t y = *(const f32x4_t*)(tile + c * TP + vc);
            *(f32x4_t*)(out + (size_t)(c0 + c) * q.out_rp + r0 + vc) = y;
        }
    }
}

// Several independent transposes in one launch: block b runs job j with
// start[j] <= b < start[j+1] (their tiles are small; apart they cost a launch
// ramp each).
template <typename T>
__global__ __launch_bounds__(256) void transpose_batch_kernel(TransposeBatch b) {
    int j = 0;
    while (j + 1 < b.n && (int)blockIdx.x >= b.start[j + 1]) ++j;
    transpose_block<T>(b.job[j], (int)blockIdx.x - b.start[j]);
}

// dSc = 2 relu(Sc) dA * mask with relu(Sc) = sqrt(A) (A = relu(Sc)^2 as the
// forward stored it), stored in the element type for the products, and the
// bias gradient's first stage: per chunk and slab of 32 query rows, the sums
// of dSc along each diagonal (key - query = k - (C-1)), rows in order.  One
// block per slab: its 32 x C entries (eight consecutive ones per thread and
// step) are kept in LDS in fp32 for the diagonal sums, one thread per
// diagonal.
template <typename T>
__global__ __launch_bounds__(256) void scores_bwd_kernel(BwdElemParams q, float* part) {
    extern __shared__ __align__(16) char lds[];
    float* slab = (float*)lds;  // [32, C]
    const int C = q.C, slabs = C / 32;
    const size_t z = blockIdx.x / slabs;
    const int i0 = (blockIdx.x % slabs) * 32;
#pragma unroll 4
    for (int t8 = threadIdx.x; t8 < 4 * C; t8 += 256) {
        const int t = 8 * t8, r = i0 + t / C, c = t % C;  // query, first key of eight
        const size_t i = (z * C + r) * C + c;
        float a[8], v[8];
        load8<T>(q.b, (int64_t)i, a);
        const f32x4_t d0 = *(const f32x4_t*)(q.f1 + i), d1 = *(const f32x4_t*)(q.f1 + i + 4);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float dk = k < 4 ? d0[k] : d1[k - 4];
            v[k] = (!q.causal || c + k <= r) ? 2.f * sqrtf(fmaxf(a[k], 0.f)) * dk : 0.f;
        }
        store8<T>(q.o0, (int64_t)i, v);
        *(f32x4_t*)(slab + t) = f32x4_t{v[0], v[1], v[2], v[3]};
        *(f32x4_t*)(slab + t + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
    }
    __syncthreads();
    for (int k = threadIdx.x; k < 2 * C - 1; k += 256) {
        const int dd = k - (C - 1);
        float acc = 0.f;
#pragma unroll 8
        for (int ii = 0; ii < 32; ++ii) {
            const int j = i0 + ii + dd;
            if (j >= 0 && j < C) acc += slab[ii * C + j];
        }
        part[(size_t)blockIdx.x * (2 * C - 1) + k] = acc;
    }
}

// Column sums of a [rows, cols] fp32 array whose rows are `pitch` apart:
// column c < split goes to out0[c], column c >= split to out1[c - split].
// Block of 16 columns x 64 row groups; row group g adds rows g, g+64, ... in
// order (eight loads in flight), then the 64 group sums are added in group
// order.
__global__ __launch_bounds__(1024) void colsum_kernel(const float* in, int pitch, float* out0, float* out1, int split,
                                                      int rows, int cols) {
    constexpr int CW = 16, NG = 64, NL = 8;
    constexpr int RED = NG * CW;
    __shared__ float red[RED];
    const int cl = threadIdx.x % CW, g = threadIdx.x / CW;
    const int c = blockIdx.x * CW + cl;
    float acc = 0.f;
    if (c < cols) {
        int r = g;
        for (; r + (NL - 1) * NG < rows; r += NL * NG) {
            float v[NL];
#pragma unroll
            for (int k = 0; k < NL; ++k) v[k] = in[(size_t)(r + k * NG) * pitch + c];
#pragma unroll
            for (int k = 0; k < NL; ++k) acc += v[k];
        }
        for (; r < rows; r += NG) acc += in[(size_t)r * pitch + c];
    }
    red[g * CW + cl] = acc;
    __syncthreads();
    if (g == 0 && c < cols) {
        float s = 0.f;
        for (int k = 0; k < NG; ++k) s += red[k * CW + cl];
        if (c < split)
            out0[c] = s;
        else
            out1[c - split] = s;
    }
}

// out[i] = sum over z = 0..S-1 (in order) of part[z * stride + i], four
// entries per thread (n a multiple of 4), for up to kSplitJobs jobs: job j
// takes blocks start[j] .. start[j+1]-1.
constexpr int kSplitJobs = 4;
struct SplitJobs {
    const float* part[kSplitJobs];
    float* out[kSplitJobs];
    int64_t n[kSplitJobs];
    int start[kSplitJobs + 1];
    int64_t stride;
    int S, jobs;
};

__global__ __launch_bounds__(256) void split_reduce_kernel(SplitJobs q) {
    int j = 0;
    while (j + 1 < q.jobs && (int)blockIdx.x >= q.start[j + 1]) ++j;
    const int64_t i = ((int64_t)(blockIdx.x - q.start[j]) * 256 + threadIdx.x) * 4;
    if (i >= q.n[j]) return;
    const float* part = q.part[j];
    f32x4_t acc = *(const f32x4_t*)(part + i);
    for (int z = 1; z < q.S; ++z) acc += *(const f32x4_t*)(part + z * q.stride + i);
    *(f32x4_t*)(q.out[j] + i) = acc;
}

// dS from dP (fp32 [B, G, s*e]): causal dS_h = sum_{g > h} dP_g (a reverse
// exclusive sum, walked g = G-1 .. 0), non-causal dS_h = sum_g dP_g; stored
// times `scale` (lin_scale, which both of dS's products carry), element type.
// With segment ids (runs of equal consecutive ids, chunks a .. z-1) the
// transpose of the forward's averaging: causal dS_h = sum_{h < g < z}
// dP_g / (g - a), non-causal dS_h = sum_{a <= g < z} dP_g / (z - a).
template <typename T>
__global__ __launch_bounds__(256) void scan_bwd_kernel(BwdScanParams q) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)q.B * q.es) return;
    const size_t b = idx / q.es, v = idx - b * q.es;
    const float* dp = q.dP + b * q.G * q.es + v;
    if (q.seg) {
        const int32_t* sg = q.seg + b * q.G;
        for (int z = q.G; z > 0;) {
            int a = z - 1;  // the segment is chunks a .. z-1
            while (a > 0 && sg[a - 1] == sg[z - 1]) --a;
            if (q.causal) {
                float run = 0.f;
                for (int g = z - 1; g >= a; --g) {
                    st<T>(q.dS, (b * q.G + g) * q.es + v, q.scale * run);
                    if (g > a) run += dp[(size_t)g * q.es] * (1.0f / (float)(g - a));
                }
            } else {
                float tot = 0.f;
                for (int g = a; g < z; ++g) tot += dp[(size_t)g * q.es];
                const float avg = tot * (1.0f / (float)(z - a));
                for (int g = a; g < z; ++g) st<T>(q.dS, (b * q.G + g) * q.es + v, q.scale * avg);
            }
            z = a;
        }
    } else if (q.causal) {
        float run = 0.f;
        for (int g = q.G - 1; g >= 0; --g) {
            st<T>(q.dS, (b * q.G + g) * q.es + v, q.scale * run);
            run += dp[(size_t)g * q.es];
        }
    } else {
        float tot = 0.f;
        for (int g = 0; g < q.G; ++g) tot += dp[(size_t)g * q.es];
        for (int g = 0; g < q.G; ++g) st<T>(q.dS, (b * q.G + g) * q.es + v, q.scale * tot);
    }
}

// dZ = sum_k gamma_k dh_k over the four heads, stored as its pre-activation
// gradient dZ * SiLU'(H_z); per block of kHeadsBwdTokens tokens the partial sums of
// dh_k * Z and dh_k (for gamma and beta).  Thread per feature i (s threads),
// tokens in order.  With rope the dh_k given are those of the rotated heads:
// each goes back through the transposed rotation of its pair (i, i +- s/2)
// at the token's position (dlo = dlo' c + dhi' sin, dhi = dhi' c - dlo' sin).
template <typename T, bool ROPE>
__global__ __launch_bounds__(256) void heads_bwd_kernel(BwdHeadsParams q) {
    const int i = threadIdx.x;
    if (i >= q.s) return;
    const int half = q.s / 2;
    const bool lo = i < half;
    const int partner = lo ? i + half : i - half;
    const double theta = ROPE ? rope_theta(lo ? i : partner, half) : 0.0;
    const int m0 = blockIdx.x * kHeadsBwdTokens;
    float pg[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f};
    float gk[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) gk[k] = q.scale[k * q.s + i];
    // groups of U tokens: every load of a group in flight together, then the
    // arithmetic in token order (the sums keep that order)
    constexpr int U = 4;
    static_assert(kHeadsBwdTokens % U == 0, "whole groups");
    for (int m1 = m0; m1 < m0 + kHeadsBwdTokens; m1 += U) {
        float hv[U], dv[U][4], pv[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int m = min(m1 + u, q.M - 1);  // (a token past the end is loaded, not used)
            hv[u] = ld<T>(q.Hz, (size_t)m * q.hpitch + i);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                dv[u][k] = q.dh[k][(size_t)m * q.s + i];
                if constexpr (ROPE) pv[u][k] = q.dh[k][(size_t)m * q.s + partner];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int m = m1 + u;
            if (m >= q.M) break;
            const float h = hv[u];
            const float z = silu(h);
            float dhk[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) dhk[k] = dv[u][k];
            if constexpr (ROPE) {
                float c, sn;
                rope_cos_sin((double)(m % q.T), theta, c, sn);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float pk = pv[u][k];
                    dhk[k] = lo ? dhk[k] * c + pk * sn : dhk[k] * c - pk * sn;
                }
            }
            float dz = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float dh = dhk[k];
                dz += gk[k] * dh;
                pg[k] += dh * z;
                pb[k] += dh;
            }
            st<T>(q.dHz, (size_t)m * q.hpitch + i, dz * silu_grad(h));
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        q.part[((size_t)blockIdx.x * 8 + k) * q.s + i] = pg[k];
        q.part[((size_t)blockIdx.x * 8 + 4 + k) * q.s + i] = pb[k];
    }
}

template <typename P>
hipError_t go(void (*k)(P), unsigned blocks, const P& p, hipStream_t st) {
    hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, st, p);
    return hipGetLastError();
}

template <typename T, int BT, int EPI, bool TA, bool TB, bool TA2, bool TB2>
hipError_t gemm_go1(const GemmNTParams& q, unsigned blocks, hipStream_t st) {
    constexpr int LDS = GemmCore<T, BT, BT, 2, 2>::LDS_BYTES;  // the same for every operand layout
    const hipError_t e = allow_lds<gemm_nt_kernel<T, BT, EPI, TA, TB, TA2, TB2>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_nt_kernel<T, BT, EPI, TA, TB, TA2, TB2>), dim3(blocks), dim3(256), LDS, st, q);
    return hipGetLastError();
}

template <typename T, int BT>
hipError_t gemm_go(const GemmNTParams& q, unsigned blocks, hipStream_t st) {
    const bool two = q.K2 > 0;
    const int a2 = two ? q.a2_t : q.a_t, b2 = two ? q.b2_t : q.b_t;
    const int key = (q.a_t ? 8 : 0) | (q.b_t ? 4 : 0) | (a2 ? 2 : 0) | (b2 ? 1 : 0);
    if (q.epi == EPI_STORE) {
        switch (key) {
            case 0x0: return gemm_go1<T, BT, EPI_STORE, false, false, false, false>(q, blocks, st);
            case 0x5: return gemm_go1<T, BT, EPI_STORE, false, true, false, true>(q, blocks, st);
            case 0xF: return gemm_go1<T, BT, EPI_STORE, true, true, true, true>(q, blocks, st);
            default: return hipErrorInvalidValue;
        }
    }
    if (q.epi == EPI_SILU) {
        switch (key) {
            case 0x0: return gemm_go1<T, BT, EPI_SILU, false, false, false, false>(q, blocks, st);
            case 0xC: return gemm_go1<T, BT, EPI_SILU, true, true, false, false>(q, blocks, st);
            case 0xF: return gemm_go1<T, BT, EPI_SILU, true, true, true, true>(q, blocks, st);
            default: return hipErrorInvalidValue;
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_nt(const GemmNTParams& q0, int M, int N, int nb, bool bf, hipStream_t st) {
    GemmNTParams q = q0;
    // 128 x 128 tiles when they divide the output and still give every CU work
    if (q.bt != 0 && q.bt != 64 && !(q.bt == 128 && M % 128 == 0 && N % 128 == 0)) return hipErrorInvalidValue;
    if (q.k_from_row && (M > q.K || q.K % 64 != 0)) return hipErrorInvalidValue;
    const bool big = q.bt ? q.bt == 128 : M % 128 == 0 && N % 128 == 0 && (int64_t)nb * (M / 128) * (N / 128) >= 512;
    const int bt = big ? 128 : 64;
    q.tm = M / bt;
    q.tn = N / bt;
    const int64_t blocks = (int64_t)nb * q.tm * q.tn;
    if (blocks <= 0 || blocks > INT32_MAX) return hipErrorInvalidValue;
    if (bf) return big ? gemm_go<bf16, 128>(q, (unsigned)blocks, st) : gemm_go<bf16, 64>(q, (unsigned)blocks, st);
    return big ? gemm_go<float, 128>(q, (unsigned)blocks, st) : gemm_go<float, 64>(q, (unsigned)blocks, st);
}

hipError_t launch_transpose_batch(const TransposeParams* jobs, const int* R, const int* Cc, const int* nb, int n,
                                  bool bf, hipStream_t st) {
    if (n < 1 || n > kTransposeBatch) return hipErrorInvalidValue;
    TransposeBatch b{};
    b.n = n;
    int64_t total = 0;
    for (int j = 0; j < n; ++j) {
        b.job[j] = jobs[j];
        b.job[j].tr = R[j] / 64;
        b.job[j].tc = Cc[j] / 64;
        b.start[j] = (int)total;
        total += (int64_t)nb[j] * b.job[j].tr * b.job[j].tc;
        if (total > INT32_MAX) return hipErrorInvalidValue;
    }
    b.start[n] = (int)total;
    if (total <= 0) return hipErrorInvalidValue;
    if (bf)
        hipLaunchKernelGGL(transpose_batch_kernel<bf16>, dim3((unsigned)total), dim3(256), 0, st, b);
    else
        hipLaunchKernelGGL(transpose_batch_kernel<float>, dim3((unsigned)total), dim3(256), 0, st, b);
    return hipGetLastError();
}

hipError_t launch_scores_bwd(const BwdElemParams& q, float* part, float* drelpos, bool bf, hipStream_t st) {
    const int C = q.C;
    if (C % 32 != 0 || q.n % ((size_t)C * C) != 0) return hipErrorInvalidValue;
    const int nchunks = (int)(q.n / ((size_t)C * C)), rows = nchunks * (C / 32);
    const int lds = 32 * C * 4;
    hipError_t e = bf ? allow_lds<scores_bwd_kernel<bf16>>(lds) : allow_lds<scores_bwd_kernel<float>>(lds);
    if (e != hipSuccess) return e;
    if (bf)
        hipLaunchKernelGGL(scores_bwd_kernel<bf16>, dim3(rows), dim3(256), lds, st, q, part);
    else
        hipLaunchKernelGGL(scores_bwd_kernel<float>, dim3(rows), dim3(256), lds, st, q, part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(colsum_kernel, dim3((2 * C - 1 + 15) / 16), dim3(1024), 0, st, part, 2 * C - 1, drelpos,
                       drelpos, 2 * C - 1, rows, 2 * C - 1);
    return hipGetLastError();
}

hipError_t launch_split_reduce(const float* const* parts, float* const* outs, const int64_t* ns, int jobs,
                               int64_t stride, int S, hipStream_t st) {
    if (jobs < 1 || jobs > kSplitJobs || stride % 4 != 0 || S < 1) return hipErrorInvalidValue;
    SplitJobs q{};
    q.stride = stride;
    q.S = S;
    q.jobs = jobs;
    int64_t blocks = 0;
    for (int j = 0; j < jobs; ++j) {
        if (ns[j] % 4 != 0 || ns[j] > stride) return hipErrorInvalidValue;
        q.part[j] = parts[j];
        q.out[j] = outs[j];
        q.n[j] = ns[j];
        q.start[j] = (int)blocks;
        blocks += (ns[j] / 4 + 255) / 256;
        if (blocks > INT32_MAX) return hipErrorInvalidValue;
    }
    q.start[jobs] = (int)blocks;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, q);
    return hipGetLastError();
}

hipError_t launch_scan_bwd(const BwdScanParams& q, bool bf, hipStream_t st) {
    const unsigned b = (unsigned)(((size_t)q.B * q.es + 255) / 256);
    return bf ? go(scan_bwd_kernel<bf16>, b, q, st) : go(scan_bwd_kernel<float>, b, q, st);
}

hipError_t launch_heads_bwd(const BwdHeadsParams& q, float* dscale, float* doffset, bool bf, hipStream_t st) {
    const int nblk = (q.M + kHeadsBwdTokens - 1) / kHeadsBwdTokens;
    hipError_t e = bf ? (q.rope ? go(heads_bwd_kernel<bf16, true>, (unsigned)nblk, q, st)
                                : go(heads_bwd_kernel<bf16, false>, (unsigned)nblk, q, st))
                      : (q.rope ? go(heads_bwd_kernel<float, true>, (unsigned)nblk, q, st)
                                : go(heads_bwd_kernel<float, false>, (unsigned)nblk, q, st));
    if (e != hipSuccess) return e;
    // part is [nblk, 8, s]: the gamma sums in rows 0..3, the beta sums in rows
    // 4..7, i.e. columns [0, 4s) and [4s, 8s) of an [nblk, 8s] array
    hipLaunchKernelGGL(colsum_kernel, dim3((8 * q.s + 15) / 16), dim3(1024), 0, st, q.part, 8 * q.s, dscale, doffset,
                       4 * q.s, nblk, 8 * q.s);
    return hipGetLastError();
}

}  // namespace gau
