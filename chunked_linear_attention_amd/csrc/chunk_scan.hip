// Chunk-level sum of the linear-attention states.
//   causal:     P_g = sum_{h<g} S_h  (exclusive prefix, eq. 8: h = 1..g-1)
//   non-causal: P   = sum_h S_h      (eq. 7, one total per sequence)
// Pages: wikillm "Method" steps 2-3 and the FLASH block pseudocode
// (exclusive_cumsum over the chunk axis, or sum); Su's post, "Mixed
// Chunking" (cumulative-sum form for the decoder).  The chunking reduces the
// sequential dependency from T token steps to G chunk steps (wikillm
// "Method" step 4; papercache 3.2.1).
//
// Every one of the B * e * s state entries is an independent G-step sum.  A
// thread owns four consecutive entries (one 16-byte vector) and walks the G
// chunks in order g = 0..G-1, so each output is a true exclusive prefix summed
// in a fixed order (never an inclusive sum minus the own term), which keeps the
// causal outputs independent of later chunks bit for bit.  S and P are in the
// layer's element type (P's consumer is an MFMA operand of that type); the
// sums are fp32.  HBM bound: it reads S once and writes P once.  In the
// causal case P may be S itself (the forward runs the scan in place): a
// thread reads each of its entries of S_g before it writes the same entries
// of P_g, and no other thread touches them, so S and P are not restrict.
//
// With segment ids (packed sequences; wikillm "Paper vs code" and
// "Pitfalls", segment masks: the listing's chunk mask, each row divided by
// its sum, applied to the summaries) a segment is a run of consecutive
// chunks with equal ids, and P_g is the average of the summaries visible
// from chunk g: causal, S_h for the h < g of g's segment (0 when there is
// none); non-causal, every S_h of the segment.  One state per chunk in
// both cases; the non-causal pass reads a whole segment's S before it writes
// its P, so it too may run in place.
#include "gau_device.h"
#include "gau_launch.h"

namespace gau {
namespace {

template <typename T>
__device__ __forceinline__ f32x4_t get4(const void* src);
template <>
__device__ __forceinline__ f32x4_t get4<float>(const void* src) {
    return *(const f32x4_t*)src;
}
template <>
__device__ __forceinline__ f32x4_t get4<bf16>(const void* src) {
    const u32x2_t w = *(const u32x2_t*)src;
    return f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                   __uint_as_float(w.y & 0xFFFF0000u)};
}

template <typename T>
__device__ __forceinline__ void put4(void* dst, const f32x4_t& v);
template <>
__device__ __forceinline__ void put4<float>(void* dst, const f32x4_t& v) {
    *(f32x4_t*)dst = v;
}
template <>
__device__ __forceinline__ void put4<bf16>(void* dst, const f32x4_t& v) {
    u32x2_t w;
    w.x = pack_bf16x2(v.x, v.y);
    w.y = pack_bf16x2(v.z, v.w);
    *(u32x2_t*)dst = w;
}

template <typename T>
__global__ __launch_bounds__(256) void chunk_scan_kernel(ScanParams p) {
    // 64-bit lane index: B * e * s / 4 lanes may exceed 2^31 (check_config
    // bounds it below 2^31 so that the grid fits, but no product here wraps)
    const int64_t per_b = p.es / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= per_b * p.B) return;
    const int64_t b = idx / per_b;
    const int64_t v = idx - b * per_b;
    const size_t stride = (size_t)p.es;  // elements between consecutive chunks
    constexpr int EB = Elem<T>::kBytes;
    const char* S = (const char*)p.S + ((size_t)b * p.G * stride + (size_t)v * 4) * EB;
    char* P = (char*)p.P;
    const size_t cstride = stride * EB;  // bytes between consecutive chunks
    f32x4_t run = {0.f, 0.f, 0.f, 0.f};
    if (p.seg) {
        const int32_t* sg = p.seg + b * p.G;
        char* out = P + ((size_t)b * p.G * stride + (size_t)v * 4) * EB;
        if (p.causal) {
            int start = 0;  // first chunk of the current segment
            for (int g = 0; g < p.G; ++g) {
                if (g > 0 && sg[g] != sg[g - 1]) {
                    run = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    start = g;
                }
                const f32x4_t s0 = get4<T>(S + (size_t)g * cstride);
                const int n = g - start;  // chunks visible from g
                put4<T>(out + (size_t)g * cstride, n > 0 ? run * (1.0f / (float)n) : run);
                run += s0;
            }
        } else {
            for (int a = 0; a < p.G;) {
                int z = a + 1;  // the segment is chunks a .. z-1
                while (z < p.G && sg[z] == sg[a]) ++z;
                for (int g = a; g < z; ++g) run += get4<T>(S + (size_t)g * cstride);
                const f32x4_t avg = run * (1.0f / (float)(z - a));
                for (int g = a; g < z; ++g) put4<T>(out + (size_t)g * cstride, avg);
                run = f32x4_t{0.f, 0.f, 0.f, 0.f};
                a = z;
            }
        }
    } else if (p.causal) {
        char* out = P + ((size_t)b * p.G * stride + (size_t)v * 4) * EB;
        int g = 0;
        // U chunks' loads in flight at once (a long sequence has few lanes
        // per chunk step and many steps: its loads must overlap), then their
        // stores and sums in chunk order
        constexpr int U = 16;
        for (; g + U <= p.G; g += U) {
            f32x4_t sv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) sv[u] = get4<T>(S + (size_t)(g + u) * cstride);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                put4<T>(out + (size_t)(g + u) * cstride, run);
                run += sv[u];
            }
        }
        for (; g < p.G; ++g) {
            const f32x4_t s0 = get4<T>(S + (size_t)g * cstride);
            put4<T>(out + (size_t)g * cstride, run);
            run += s0;
        }
    } else {
        for (int g = 0; g < p.G; ++g) run += get4<T>(S + (size_t)g * cstride);
        put4<T>(P + ((size_t)b * stride + (size_t)v * 4) * EB, run);
    }
}

template <typename T>
hipError_t launch(const ScanParams& p, hipStream_t st) {
    const int64_t threads = (int64_t)p.B * (p.es / 4);
    const int blocks = (int)((threads + 255) / 256);
    hipLaunchKernelGGL(chunk_scan_kernel<T>, dim3(blocks), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_scan(const ScanParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? launch<bf16>(p, st) : launch<float>(p, st);
}

}  // namespace gau
