// Device-side building blocks shared by the libgau kernels (gfx950 only).
//
// Element types: `bf16` (storage of bfloat16 bits; MFMA v_mfma_f32_16x16x32_bf16
// with fp32 accumulation) and `float` (fp32 storage; four v_mfma_f32_16x16x4_f32
// per 16-byte fragment).  Both are handled by one code path: every MFMA operand
// fragment is 16 bytes per lane, taken along the contraction (K) dimension, so
// LDS tiles are laid out and read identically for the two types; only the
// number of K elements per 16 bytes differs.
//
// Fragment layout of a 16x16 MFMA block (lane l, 64 lanes; verified on gfx950):
//   operand A: row (l % 16), 16 bytes of K starting at byte 16 * (l / 16) of a
//              64-byte K step; operand B: column (l % 16), same K bytes.
//   accumulator (4 floats): column (l % 16), rows 4 * (l / 16) + r, r = 0..3.
// For fp32 the four floats of a fragment feed four K=4 MFMAs, slot t of lane
// group q standing for K index 4q + t; A and B use the same assignment, so the
// sum over K is complete and exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gau {

struct bf16 {
    uint16_t bits;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ scalars

// fp32 -> bf16, round to nearest, ties to even (finite values).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename T> struct Elem;
template <> struct Elem<bf16> {
    static constexpr int kBytes = 2;
    __device__ static __forceinline__ void put(void* p, float v) { *(uint16_t*)p = f32_to_bf16(v); }
    __device__ static __forceinline__ float get(const void* p) { return bf16_to_f32(*(const uint16_t*)p); }
};
template <> struct Elem<float> {
    static constexpr int kBytes = 4;
    __device__ static __forceinline__ void put(void* p, float v) { *(float*)p = v; }
    __device__ static __forceinline__ float get(const void* p) { return *(const float*)p; }
};

// SiLU(x) = x * sigmoid(x) = x / (1 + exp(-x)), evaluated in fp32 with the
// hardware exponential and reciprocal (v_exp_f32, v_rcp_f32; about 1 ulp
// each).  For x below about -88, exp(-x) overflows to +inf and the result is
// x * 0 = -0, the correctly rounded limit.
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// ------------------------------------------------------------------ MFMA

__device__ __forceinline__ void mma16(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b, bf16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b, float) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// ------------------------------------------------------------------ tiles
//
// An LDS tile holds ROWS rows of KBYTES bytes each, rows padded by 16 bytes
// (pitch KBYTES + 16) so that the 16 rows read by one MFMA fragment load fall
// in distinct LDS banks.

template <int KBYTES> struct LdsPitch { static constexpr int value = KBYTES + 16; };

// Global -> registers -> LDS copy of a ROWS x KBYTES tile by NT threads.
// Rows at or beyond `rows_valid` re-read row rows_valid-1 (in bounds; the
// results they feed are never stored).
template <int ROWS, int KBYTES, int NT>
struct TileCopy {
    static constexpr int kVecPerRow = KBYTES / 16;
    static constexpr int kTotal = ROWS * kVecPerRow;
    static constexpr int kPerThread = kTotal / NT;
    static_assert(kTotal % NT == 0, "tile not divisible among threads");
    static constexpr int kPitch = LdsPitch<KBYTES>::value;
    u32x4_t r[kPerThread];

    __device__ __forceinline__ void load(const char* __restrict__ g, size_t gpitch, int rows_valid, int tid) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int idx = tid + i * NT;
            int row = idx / kVecPerRow;
            const int c = idx % kVecPerRow;
            row = row < rows_valid ? row : rows_valid - 1;
            r[i] = *(const u32x4_t*)(g + (size_t)row * gpitch + c * 16);
        }
    }
    __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int idx = tid + i * NT;
            const int row = idx / kVecPerRow;
            const int c = idx % kVecPerRow;
            *(u32x4_t*)(lds + row * kPitch + c * 16) = r[i];
        }
    }
};

// One wave's MFMA work on an LDS stage: acc[MB][NB] (16x16 blocks) +=
// A[MB*16 rows] . B[NB*16 rows]^T over KSTEPS 64-byte K steps.  `a` and `b`
// point at the wave's first row in LDS.
template <typename T, int MB, int NB, int KSTEPS>
__device__ __forceinline__ void wave_mma(f32x4_t (&acc)[MB][NB], const char* a, int pitch_a,
                                         const char* b, int pitch_b, int lane) {
    const int r = lane & 15;
    const int q = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        u32x4_t fa[MB], fb[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) fa[i] = *(const u32x4_t*)(a + (i * 16 + r) * pitch_a + ks * 64 + q * 16);
#pragma unroll
        for (int j = 0; j < NB; ++j) fb[j] = *(const u32x4_t*)(b + (j * 16 + r) * pitch_b + ks * 64 + q * 16);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) mma16(acc[i][j], fa[i], fb[j], T());
    }
}

template <int MB, int NB>
__device__ __forceinline__ void zero_acc(f32x4_t (&acc)[MB][NB]) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// ------------------------------------------------------------------ NT GEMM
//
// Block-level C[BM x BN] = A[BM x K] . B[BN x K]^T with A and B row-major and
// K contiguous (both operands "K-major").  256 threads = 4 waves in a 2 x 2
// grid, each wave owning a (BM/2) x (BN/2) sub-tile.  K is walked in steps of
// 128 bytes with a double-buffered LDS stage: the next step's global loads are
// in flight while the current one is multiplied.
//
// LDS use: 2 * (BM + BN) * 144 bytes.

template <typename T, int BM, int BN>
struct GemmNT {
    static constexpr int NT = 256;
    static constexpr int KBYTES = 128;
    static constexpr int KELEMS = KBYTES / Elem<T>::kBytes;
    static constexpr int PITCH = LdsPitch<KBYTES>::value;
    static constexpr int MB = BM / 2 / 16;
    static constexpr int NB = BN / 2 / 16;
    static constexpr int STAGE_BYTES = (BM + BN) * PITCH;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;

    // a, b: first row of the block's tile; pitches in bytes; K in elements
    // (a multiple of KELEMS).  rows_a / rows_b: rows that exist (clamped).
    __device__ static __forceinline__ void run(f32x4_t (&acc)[MB][NB], const char* __restrict__ a, size_t pitch_a,
                                               int rows_a, const char* __restrict__ b, size_t pitch_b, int rows_b,
                                               int K, char* lds) {
        const int tid = threadIdx.x;
        const int wave = tid / kWave;
        const int lane = tid % kWave;
        const int wm = wave >> 1, wn = wave & 1;
        TileCopy<BM, KBYTES, NT> ca;
        TileCopy<BN, KBYTES, NT> cb;
        zero_acc(acc);
        const int ksteps = K / KELEMS;
        ca.load(a, pitch_a, rows_a, tid);
        cb.load(b, pitch_b, rows_b, tid);
        ca.store(lds, tid);
        cb.store(lds + BM * PITCH, tid);
        __syncthreads();
        for (int kt = 0; kt < ksteps; ++kt) {
            char* cur = lds + (kt & 1) * STAGE_BYTES;
            char* nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;
            const bool more = kt + 1 < ksteps;
            if (more) {
                ca.load(a + (size_t)(kt + 1) * KBYTES, pitch_a, rows_a, tid);
                cb.load(b + (size_t)(kt + 1) * KBYTES, pitch_b, rows_b, tid);
            }
            wave_mma<T, MB, NB, KBYTES / 64>(acc, cur + wm * (BM / 2) * PITCH, PITCH,
                                             cur + BM * PITCH + wn * (BN / 2) * PITCH, PITCH, lane);
            if (more) {
                ca.store(nxt, tid);
                cb.store(nxt + BM * PITCH, tid);
            }
            __syncthreads();
        }
    }
};

// Walk every element of a wave's accumulator tile: f(row, col, value) with
// row/col relative to the wave's sub-tile origin.
template <int MB, int NB, typename F>
__device__ __forceinline__ void for_each_acc(const f32x4_t (&acc)[MB][NB], int lane, F&& f) {
    const int c = lane & 15;
    const int q = lane >> 4;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) f(i * 16 + 4 * q + r, j * 16 + c, acc[i][j][r]);
}

// Allow kernel `Kernel` more than the default dynamic LDS (the attribute is set
// once per kernel).
template <auto Kernel>
inline hipError_t allow_lds(int bytes) {
    static const hipError_t err =
        hipFuncSetAttribute((const void*)Kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return err;
}

}  // namespace gau
