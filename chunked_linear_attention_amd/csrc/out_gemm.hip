// Output projection O = Y W_o with Y = U * (V_quad + V_lin) from the chunk
// kernel (wikillm "Method" step 4: O_g = [U_g * (V_quad_g + V_lin_g)] W_o;
// Su's post, "Mixed Chunking", final equation).  With a residual pointer the
// epilogue also adds the layer's shortcut in fp32 (the skip connection the
// listings add after each block: wikillm, FLASH block pseudocode).
//
// An NT GEMM on the shared core, K = e: A operand = W_o^T rows (output
// features), B operand = Y rows (tokens).  Tiles are BF features x 256 tokens
// with BF chosen per d (256, 192 or 128, dividing d) so that the grid is as
// close as possible to whole rounds over the 256 CUs: d = 768 takes 192, which
// gives 4 x 64 = 256 blocks at B*T = 16384.
#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {
namespace {

// Four consecutive elements (aligned to four) as loaded, as floats, and back.
template <typename T> struct Raw4 { using type = f32x4_t; };
template <> struct Raw4<bf16> { using type = u32x2_t; };

__device__ __forceinline__ void unpack4(const u32x2_t& w, float (&v)[4]) {
    v[0] = __uint_as_float(w.x << 16);
    v[1] = __uint_as_float(w.x & 0xFFFF0000u);
    v[2] = __uint_as_float(w.y << 16);
    v[3] = __uint_as_float(w.y & 0xFFFF0000u);
}
__device__ __forceinline__ void unpack4(const f32x4_t& w, float (&v)[4]) {
    v[0] = w.x;
    v[1] = w.y;
    v[2] = w.z;
    v[3] = w.w;
}
template <typename T>
__device__ __forceinline__ void put4(char* p, const float (&v)[4]) {
    if constexpr (Elem<T>::kBytes == 2)
        *(u32x2_t*)p = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    else
        *(f32x4_t*)p = f32x4_t{v[0], v[1], v[2], v[3]};
}

constexpr int BN = 256, WGM = 2, WGN = 4;  // tokens per tile, wave grid

template <typename T, int BM, bool TN = false>
struct OutTile {
    // Y (the B operand) streams from HBM: a third B stage keeps two of its
    // chunks in flight; W_o (A) stays in L2 with two stages.  MN-major
    // operands (TN) take the plain two-stage ring.
    using G = typename PickT<TN, GemmCore<T, BM, BN, WGM, WGN, 2, 0, 2, true, true>,
                             GemmCore<T, BM, BN, WGM, WGN, 2, 0, 3>>::type;
    // staging of one pass of the epilogue in the worst case (fp32, WGN passes)
    static constexpr int STAGE = BN / WGN * (BM * 4 + 16);
    static constexpr int LDS = G::LDS_BYTES > STAGE ? G::LDS_BYTES : STAGE;
};

// Epilogue kinds, each a kernel of its own so that the others carry none of
// its prefetch registers: plain stores, the backward's gate (p.gH set), the
// residual add (p.residual set).
enum { kEpPlain = 0, kEpGate = 1, kEpResid = 2 };

template <typename T, int BM, bool TN, int EP>
__global__ __launch_bounds__(512) void out_gemm_kernel(OutParams p) {
    extern __shared__ __align__(16) char lds[];
    using G = typename OutTile<T, BM, TN>::G;
    constexpr int EB = Elem<T>::kBytes;
    const int ntiles = (p.d + BM - 1) / BM;  // feature tiles (acc rows)
    const int tiles = ntiles * ((p.M + BN - 1) / BN);
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int z = bid / tiles, tt = bid - z * tiles;  // K split, tile
    const int nt = tt % ntiles;
    const int mt = tt / ntiles;
    const int m0 = mt * BN, n0 = nt * BM;  // token offset, feature offset
    const size_t pitch = (size_t)(p.k_rp > 0 ? p.k_rp : p.e) * EB;
    const int rows_y = min(BN, p.M - m0);
    const int rows_w = min(BM, p.d - n0);
    // this block's K chunks (one range unless split)
    const int S = p.ksplit > 1 ? p.ksplit : 1;
    const int nk = p.e / G::KELEMS, kbase = nk / S, krem = nk % S;
    const int kc0 = z * kbase + min(z, krem), nkz = kbase + (z < krem ? 1 : 0);

    const int M = p.M, d = p.d;
    const size_t orp = p.o_rp > 0 ? (size_t)p.o_rp : (size_t)d;  // output row pitch

    // Inputs of the gate epilogue (the OutParams gate fields) and of the
    // residual add, processed in NPASS passes of PROWS tokens; each thread
    // takes NV 4-element vectors (features n..n+3 of token m) per pass.  bf16:
    // the first pass's inputs are loaded before the K loop, so that their
    // memory latency overlaps it, each later pass's at the start of the pass
    // before it (two register buffers).  fp32 (vectors twice as wide, no
    // registers to spare in the K loop): one buffer, the first pass's loaded
    // after the K loop, each later pass's at the end of the pass before it.
    constexpr int NPASS = WGN, PROWS = BN / NPASS;
    constexpr int VPR = BM / 4;              // 4-element vectors per token row of the tile
    constexpr int NV = PROWS * VPR / G::NT;  // vectors per thread per pass
    using Raw = typename Raw4<T>::type;
    constexpr int NBUF = EB == 2 ? 2 : 1;
    constexpr bool gate = !TN && EP == kEpGate, resid = !TN && EP == kEpResid;
    Raw hb[gate ? NBUF : 1][NV], wb[gate ? NBUF : 1][NV];
    f32x4_t rb[resid ? NBUF : 1][NV];
    const size_t grp = (size_t)p.g_rp;
    auto gload = [&](int pass, Raw (&h)[NV], Raw (&w)[NV]) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + i * G::NT;
            const int m = m0 + pass * PROWS + idx / VPR, n = n0 + (idx % VPR) * 4;
            if (m < M && n < d) {
                h[i] = *(const Raw*)((const char*)p.gH + ((size_t)m * orp + n) * EB);
                w[i] = *(const Raw*)((const char*)p.gW + ((size_t)m * grp + n) * EB);
            }
        }
    };
    auto rload = [&](int pass, f32x4_t (&r)[NV]) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + i * G::NT;
            const int m = m0 + pass * PROWS + idx / VPR, n = n0 + (idx % VPR) * 4;
            if (m < M && n < d) r[i] = *(const f32x4_t*)(p.residual + (size_t)m * orp + n);
        }
    };
    if constexpr (NBUF == 2 && gate) gload(0, hb[0], wb[0]);
    if constexpr (NBUF == 2 && resid) rload(0, rb[0]);

    // acc = tile^T: rows = output features (W_o^T rows), columns = tokens, so
    // the packed epilogue writes run along the token-major rows of O.
    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    if constexpr (TN) {
        // tiles start at column n0 (m0) of their first K row
        const size_t wp = (size_t)p.w_rp * EB, yp = (size_t)p.k_rp * EB;
        G::run(acc, (const char*)p.W_o + (size_t)n0 * EB + (size_t)kc0 * G::KELEMS * wp, wp, rows_w,
               (const char*)p.Y + (size_t)m0 * EB + (size_t)kc0 * G::KELEMS * yp, yp, rows_y, nkz * G::KELEMS, lds);
    } else {
        G::run(acc, (const char*)p.W_o + (size_t)n0 * pitch + (size_t)kc0 * 128, pitch, rows_w,
               (const char*)p.Y + (size_t)m0 * pitch + (size_t)kc0 * 128, pitch, rows_y, nkz * G::KELEMS, lds);
    }

    constexpr int LDS = OutTile<T, BM, TN>::LDS;
    auto ident = [](int, int, float v) { return v; };
    if constexpr (TN) {
        // fp32 O = Y W_o (split z: its partial product at O + z * o_bs)
        float* O = (float*)p.O + (size_t)z * p.o_bs;
        G::template store_packed<float>(acc, lds, LDS, ident, [&](int tok, int feat) -> char* {
            const int m = m0 + tok, n = n0 + feat;
            return (m < M && n < d) ? (char*)(O + (size_t)m * orp + n) : nullptr;
        });
    } else if constexpr (gate) {
        // gate epilogue: the product staged in fp32 (staged rows = tokens),
        // one pass at a time; the pass's inputs were loaded one pass ahead
        constexpr int PITCH = BM * 4 + 16;  // fp32 staging row
        static_assert(PROWS * VPR % G::NT == 0 && PROWS * PITCH <= LDS, "gate epilogue passes");
        if constexpr (NBUF == 1) gload(0, hb[0], wb[0]);
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
            const int cur = NBUF == 2 ? (pass & 1) : 0;
            if constexpr (NBUF == 2) {
                if (pass + 1 < NPASS) gload(pass + 1, hb[cur ^ 1], wb[cur ^ 1]);  // in flight across this pass
            }
            __syncthreads();
            G::template stage_packed<float>(acc, lds, pass, PROWS, NPASS, ident);
            __syncthreads();
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int idx = threadIdx.x + i * G::NT;
                const int srow = idx / VPR, n = n0 + (idx % VPR) * 4;
                const size_t m = (size_t)(m0 + pass * PROWS + srow);
                if ((int)m >= M || n >= d) continue;
                const u32x4_t v = *(const u32x4_t*)(lds + srow * PITCH + (idx % VPR) * 16);
                float hv[4], wv[4], a[4], y[4], o[4];
                unpack4(hb[cur][i], hv);
                unpack4(wb[cur][i], wv);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float dy = __uint_as_float(v[k]), h = hv[k], w = wv[k];
                    // U = h sigma(h); SiLU'(h) = sigma(h) (1 + h (1 - sigma(h)))
                    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-h));
                    const float u = h * sg;
                    a[k] = dy * u;
                    y[k] = u * w;
                    o[k] = dy * w * (sg * (1.0f + h * (1.0f - sg)));
                }
                const size_t j = m * grp + n;
                put4<T>((char*)p.gDWq + j * EB, a);
                put4<T>((char*)p.gY + j * EB, y);
                put4<T>((char*)p.O + (m * orp + n) * EB, o);
            }
            if constexpr (NBUF == 1) {
                if (pass + 1 < NPASS) gload(pass + 1, hb[0], wb[0]);  // in flight across the next pass's staging
            }
        }
    } else if constexpr (resid) {
        // O = residual + Y W_o (fp32), in place allowed: each output vector is
        // read from the residual and written by the same thread
        constexpr int PITCH = BM * 4 + 16;  // fp32 staging row
        static_assert(PROWS * VPR % G::NT == 0 && PROWS * PITCH <= LDS, "residual epilogue passes");
        float* O = (float*)p.O;
        if constexpr (NBUF == 1) rload(0, rb[0]);
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
            const int cur = NBUF == 2 ? (pass & 1) : 0;
            if constexpr (NBUF == 2) {
                if (pass + 1 < NPASS) rload(pass + 1, rb[cur ^ 1]);  // in flight across this pass
            }
            __syncthreads();
            G::template stage_packed<float>(acc, lds, pass, PROWS, NPASS, ident);
            __syncthreads();
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int idx = threadIdx.x + i * G::NT;
                const int srow = idx / VPR, n = n0 + (idx % VPR) * 4;
                const int m = m0 + pass * PROWS + srow;
                if (m >= M || n >= d) continue;
                f32x4_t x = *(const f32x4_t*)(lds + srow * PITCH + (idx % VPR) * 16);
                x += rb[cur][i];
                *(f32x4_t*)(O + (size_t)m * orp + n) = x;
            }
            if constexpr (NBUF == 1) {
                if (pass + 1 < NPASS) rload(pass + 1, rb[0]);  // in flight across the next pass's staging
            }
        }
    } else if (p.residual == nullptr && !p.f32_out) {
        char* O = (char*)p.O;
        G::template store_packed<T>(acc, lds, LDS, ident, [&](int tok, int feat) -> char* {
            const int m = m0 + tok, n = n0 + feat;
            return (m < M && n < d) ? O + ((size_t)m * orp + n) * EB : nullptr;
        });
    } else {
        // fp32 O = Y W_o (split z: its partial product at O + z * o_bs)
        float* O = (float*)p.O + (size_t)z * p.o_bs;
        G::template store_packed<float>(acc, lds, LDS, ident, [&](int tok, int feat) -> char* {
            const int m = m0 + tok, n = n0 + feat;
            return (m < M && n < d) ? (char*)(O + (size_t)m * orp + n) : nullptr;
        });
    }
}

template <typename T, int BM, bool TN = false, int EP = kEpPlain>
hipError_t launch(const OutParams& p, hipStream_t st) {
    constexpr int LDS = OutTile<T, BM, TN>::LDS;
    static_assert(LDS <= 160 * 1024, "output GEMM LDS over budget");
    const int S = p.ksplit > 1 ? p.ksplit : 1;
    if (S > 1 && (p.residual != nullptr || p.gH != nullptr || !p.f32_out)) return hipErrorInvalidValue;
    if (TN && (p.residual != nullptr || p.gH != nullptr || !p.f32_out || p.M % 64 != 0 || p.d % 64 != 0))
        return hipErrorInvalidValue;
    if (S > p.e / OutTile<T, BM, TN>::G::KELEMS) return hipErrorInvalidValue;
    const int blocks = ((p.d + BM - 1) / BM) * ((p.M + BN - 1) / BN) * S;
    if ((EP == kEpGate) != (p.gH != nullptr) || (EP == kEpResid) != (p.residual != nullptr))
        return hipErrorInvalidValue;
    hipError_t e = allow_lds<out_gemm_kernel<T, BM, TN, EP>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((out_gemm_kernel<T, BM, TN, EP>), dim3(blocks), dim3(512), LDS, st, p);
    return hipGetLastError();
}

// Feature-tile width for d: the candidate (dividing d) with the least
// rounds-times-tile-width over 256 CUs, the larger tile on ties.
int feature_tile(int d, int M) {
    const int cand[3] = {256, 192, 128};
    int best = 128;
    long best_cost = -1;
    const int mt = (M + BN - 1) / BN;
    for (int bf : cand) {
        if (d % bf) continue;
        const long blocks = (long)(d / bf) * mt;
        const long cost = (blocks + 255) / 256 * bf;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = bf;
        }
    }
    return best;
}

template <typename T, int BM>
hipError_t launch_ep(const OutParams& p, hipStream_t st) {
    if (p.gH != nullptr) return launch<T, BM, false, kEpGate>(p, st);
    if (p.residual != nullptr) return launch<T, BM, false, kEpResid>(p, st);
    return launch<T, BM>(p, st);
}

template <typename T>
hipError_t dispatch(const OutParams& p, hipStream_t st) {
    if (p.tn) return p.bm == 256 ? launch<T, 256, true>(p, st) : hipErrorInvalidValue;
    switch (p.bm > 0 ? p.bm : feature_tile(p.d, p.M)) {
        case 256: return launch_ep<T, 256>(p, st);
        case 192: return launch_ep<T, 192>(p, st);
        default: return launch_ep<T, 128>(p, st);
    }
}

}  // namespace

int out_gemm_tiles(int d, int M, int bm) {
    const int b = bm > 0 ? bm : feature_tile(d, M);
    return ((d + b - 1) / b) * ((M + BN - 1) / BN);
}

hipError_t launch_out_gemm(const OutParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? dispatch<bf16>(p, st) : dispatch<float>(p, st);
}

}  // namespace gau
