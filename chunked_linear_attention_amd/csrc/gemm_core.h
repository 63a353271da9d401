// Block-level NT GEMM core for gfx950:  C[BM x BN] += A[BM x K] . B[BN x K]^T
// with A and B K-major (row-major, K contiguous), or either one MN-major (K
// rows of contiguous M or N elements: TA, TB; see DmaOperandT and frag_t).
// Used by the layer's GEMM-shaped kernels, forward and backward.
//
// Design (MI355X / CDNA4):
//  * 32x32x16 bf16 MFMA (v_mfma_f32_32x32x16_bf16; fp32: four
//    v_mfma_f32_32x32x2_f32 per 16-byte fragment), fp32 accumulation.  Each of
//    the WGM x WGN waves owns a (BM/WGM) x (BN/WGN) sub-tile.
//  * K advances in chunks of 128 bytes (64 bf16 / 32 fp32).  Global memory is
//    copied straight into LDS (no VGPR staging: buffer_load_dwordx4 ... lds
//    for bf16 K-major operands, global_load_lds_dwordx4 otherwise; see
//    DmaOperand), through a ring of NS stages (NS = 2 for the large tiles, more for small
//    tiles whose blocks would otherwise wait on one copy at a time): the
//    copies of the next NS-1 chunks are in flight while one chunk is
//    multiplied, and one barrier per chunk separates them.
//  * LDS rows are 128 bytes without padding; the eight 16-byte pieces of row r
//    are stored XOR-permuted by ((r >> 1) & 7).  The LDS serves a 16-byte
//    read for 16 lanes per cycle (a 256-byte bank window, two rows), so the
//    16 rows a fragment load touches per cycle must fall in distinct bank
//    groups: the pair of rows sharing a window differs in r & 1, and the
//    eight pairs differ in (r >> 1) & 7 (measured on gfx950: 188 B/clk/CU
//    against 117 for an (r & 7) permutation).  Every wave's direct copy still
//    writes 1 KiB of consecutive LDS (the permutation is applied to the global
//    addresses instead).
//
// Fragment layout of v_mfma_f32_32x32x16_bf16 (lane l; verified on gfx950):
//   A: row l % 32, 16 bytes of K at byte 16 * (l / 32) of a 32-byte K step;
//   B: column l % 32, same K bytes; accumulator (16 floats): column l % 32,
//   row 8 * (r / 4) + 4 * (l / 32) + r % 4.
// For fp32 the fragment's four floats feed four K=2 MFMAs (slot t of lane
// group h stands for K index 4h + t in both operands).
#pragma once

#include "gau_device.h"

namespace gau {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void mma32(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b, bf16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b, float) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* glb_ptr_t;

// Wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima so they do not wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// One segment of a K-major operand: `chunks` K chunks of 128 bytes starting at
// `base` (first row of the tile), rows `pitch` bytes apart.
struct KSeg {
    const char* base;
    size_t pitch;
    int chunks;
};

// Direct global -> LDS copy of one 128-byte K chunk of a ROWS-row operand
// tile whose K axis is the concatenation of two segments (the second may be
// empty).  The tile is moved as 1 KiB wave pieces (8 rows); wave w of NW takes
// pieces w, w + NW, ...  Each lane's source (row clamped to the rows that
// exist, piece XOR-permuted by the row) is computed once; a chunk only adds
// its K offset.
//   BUF = false: 64-bit source pointers per lane, global_load_lds_dwordx4.
//   BUF = true: a raw buffer resource per segment (its tile base, in SGPRs;
//     no range limit) and 32-bit byte offsets per lane, the chunk's K offset
//     as the scalar offset: buffer_load_dwordx4 ... lds.  Fewer address
//     registers and instructions per copy (the bf16 operands: projection -1.2
//     us, output GEMM -1.1 us).  A segment's rows must lie within 2 GiB of its
//     base (the tiles here span at most 256 rows of a few KiB).
template <int ROWS, int NW, bool BUF = false>
struct DmaOperand {
    static constexpr int kLoads = ROWS / 8 / NW;
    static_assert(ROWS % (8 * NW) == 0, "pieces must split evenly over the waves");
    const char* src0[BUF ? 1 : kLoads];
    const char* src1[BUF ? 1 : kLoads];
    __amdgpu_buffer_rsrc_t r0, r1;
    int off0[BUF ? kLoads : 1];
    int off1[BUF ? kLoads : 1];
    int n0;

    __device__ __forceinline__ void init(const KSeg& s0, const KSeg& s1, int rows_valid, int wave, int lane) {
        const int sub = lane >> 3;  // row inside the 8-row piece
        n0 = s0.chunks;
        if constexpr (BUF) {
            // raw buffers (stride 0), no range limit; word 3 as for untyped dword loads
            r0 = __builtin_amdgcn_make_buffer_rsrc((void*)s0.base, (short)0, -1, 0x00020000);
            r1 = __builtin_amdgcn_make_buffer_rsrc((void*)s1.base, (short)0, -1, 0x00020000);
        }
#pragma unroll
        for (int jj = 0; jj < kLoads; ++jj) {
            const int row = (wave + jj * NW) * 8 + sub;
            const int piece = (lane & 7) ^ ((row >> 1) & 7);  // logical 16-byte piece this lane fetches
            const int r = row < rows_valid ? row : rows_valid - 1;
            if constexpr (BUF) {
                off0[jj] = r * (int)s0.pitch + piece * 16;
                off1[jj] = r * (int)s1.pitch + piece * 16;
            } else {
                src0[jj] = s0.base + (size_t)r * s0.pitch + piece * 16;
                src1[jj] = s1.base + (size_t)r * s1.pitch + piece * 16;
            }
        }
    }
    // Issue the copy of K chunk `kc` into `lds_tile`.
    __device__ __forceinline__ void issue(char* lds_tile, int kc, int wave) const {
        const bool first = kc < n0;
        const int kb = (first ? kc : kc - n0) * 128;
#pragma unroll
        for (int jj = 0; jj < kLoads; ++jj) {
            lds_ptr_t dst = (lds_ptr_t)(lds_tile + (wave + jj * NW) * 1024);
            if constexpr (BUF)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(first ? r0 : r1, dst, 16, first ? off0[jj] : off1[jj], kb, 0,
                                                         0);
            else
                __builtin_amdgcn_global_load_lds((glb_ptr_t)((first ? src0[jj] : src1[jj]) + kb), dst, 16, 0, 0);
        }
    }
};

// Piece permutation of an MN-major operand tile in LDS (one row per K index,
// PPR 16-byte pieces of consecutive MN elements per row): logical piece c of
// row k sits at c ^ tsw<PPR>(k).  It spreads the transposed fragment reads
// over the banks: a bf16 read touches K rows k0..k0+3 (32 bytes of each per
// 16 lanes) in both halves of the wave; fp32 reads touch row k in one half of
// the wave and k + 4 in the other.  With PPR >= 16 (a row covers every bank)
// 4 (k & 3) separates the four rows and 8 ((k >> 2) & 1) the fp32 halves;
// with PPR = 8 consecutive rows already alternate between the two halves of
// the banks and 4 ((k >> 1) & 1) separates the pairs.
template <int PPR>
__device__ __forceinline__ int tsw(int k) {
    if constexpr (PPR >= 16)
        return (4 * (k & 3)) ^ (8 * ((k >> 2) & 1));
    else
        return 4 * ((k >> 1) & 1);
}

// Direct global -> LDS copy of one K chunk (KE = 128 / EB K indices) of an
// MN-major operand tile: the segment's K rows are `pitch` bytes apart and hold
// the tile's ROWS MN elements contiguously from `base`.  In LDS row k of the
// chunk lies at k * RB bytes (RB = ROWS * EB), its pieces permuted by tsw;
// each 1 KiB wave copy moves 1024 / RB whole rows, so a chunk is ROWS / 8
// copies as for a K-major tile.  Pieces past the rows_valid MN elements
// (rows_valid a multiple of 16 / EB) read the last valid piece instead.
template <int ROWS, int NW, int EB>
struct DmaOperandT {
    static constexpr int RB = ROWS * EB;
    static constexpr int PPR = RB / 16;
    static constexpr int KE = 128 / EB;
    static constexpr int kLoads = ROWS / 8 / NW;
    static_assert(ROWS % (8 * NW) == 0 && PPR >= 8 && 64 % PPR == 0, "MN-major tile shape");
    const char* src0[kLoads];
    const char* src1[kLoads];
    size_t step0, step1;  // bytes per chunk (KE rows) in each segment
    int n0;

    __device__ __forceinline__ void init(const KSeg& s0, const KSeg& s1, int rows_valid, int wave, int lane) {
        n0 = s0.chunks;
        step0 = (size_t)KE * s0.pitch;
        step1 = (size_t)KE * s1.pitch;
        const int last = rows_valid * EB / 16 - 1;
#pragma unroll
        for (int jj = 0; jj < kLoads; ++jj) {
            const int pc = (wave + jj * NW) * 64 + lane;  // LDS piece of the chunk this lane fills
            const int k = pc / PPR;
            int c = (pc % PPR) ^ tsw<PPR>(k);  // logical piece held there
            c = c <= last ? c : last;
            src0[jj] = s0.base + (size_t)k * s0.pitch + c * 16;
            src1[jj] = s1.base + (size_t)k * s1.pitch + c * 16;
        }
    }
    // Issue the copy of K chunk `kc` into `lds_tile`.
    __device__ __forceinline__ void issue(char* lds_tile, int kc, int wave) const {
        const bool first = kc < n0;
        const size_t off = first ? (size_t)kc * step0 : (size_t)(kc - n0) * step1;
#pragma unroll
        for (int jj = 0; jj < kLoads; ++jj)
            __builtin_amdgcn_global_load_lds((glb_ptr_t)((first ? src0[jj] : src1[jj]) + off),
                                             (lds_ptr_t)(lds_tile + (wave + jj * NW) * 1024), 16, 0, 0);
    }
};

// Transposed LDS read of 16-bit elements (ds_read_b64_tr_b16, gfx950).  In
// each group of 16 lanes, lane 4j + r passes the address of four consecutive
// elements; lane i of the group receives, as its element jj, element i % 4 of
// the four that lane 4jj + i / 4 addressed (measured on gfx950).  So when
// lanes 4j .. 4j+3 address 16 consecutive MN elements of K row j, lane i
// receives MN element i of K rows 0..3.
__device__ __forceinline__ u32x2_t lds_read_tr16(const char* p) {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)p);
    return __builtin_bit_cast(u32x2_t, v);
}

template <bool C, typename X, typename Y> struct PickT { using type = X; };
template <typename X, typename Y> struct PickT<false, X, Y> { using type = Y; };

// The hardware dispatches workgroup b to XCD b % 8, and each XCD has its own
// L2.  xcd_remap turns the dispatch index into a logical tile index such that
// each XCD receives a contiguous range of logical tiles (so neighbouring tiles,
// which share operand rows, share one L2).  Bijective for any count.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
    constexpr int kXcd = 8;
    const int x = b % kXcd, q = nb / kXcd, r = nb % kXcd;
    return x * q + (x < r ? x : r) + b / kXcd;
}

// LDS byte offset of logical 16-byte piece c of row r in a swizzled tile.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// GemmCore<T, BM, BN, WGM, WGN, NS, ZR>: with ZR > 0 the core can also form a
// side product: ZR more rows of A-type operand (K-major like A, copied into
// each stage after B) times the B tile, accumulated per wave into ZR x 32
// outputs (run_with_side).  Wave (wm, wn) multiplies the side rows by its own
// B fragment wm, so the 2 x WGN waves cover the B tile's columns once.
//
// NSB > NS (only NS = 2, NSB = 3): the B operand gets a ring of its own with
// one more stage, so two of its chunks are in flight while one is multiplied
// (for a B operand streamed from HBM beside an A operand that stays in L2).
// The A stages then lie at [0, NS * A_BYTES) and the B stages after them, and
// the per-chunk barrier waits only for LDS reads and the copies it needs.
template <typename T, int BM, int BN, int WGM, int WGN, int NS = 2, int ZR = 0, int NSB = NS, bool TA = false,
          bool TB = false>
struct GemmCore {
    static constexpr int NW = WGM * WGN;
    static constexpr int NT = NW * kWave;
    static constexpr int WTM = BM / WGM;  // wave tile
    static constexpr int WTN = BN / WGN;
    static constexpr int MB = WTM / 32;
    static constexpr int NB = WTN / 32;
    static constexpr int KELEMS = 128 / Elem<T>::kBytes;  // K elements per chunk
    static constexpr int A_BYTES = BM * 128;
    static constexpr int Z_OFF = (BM + BN) * 128;  // side rows inside a stage
    static constexpr int STAGE_BYTES = (BM + BN + ZR) * 128;
    static constexpr int B_BYTES = BN * 128;
    static constexpr bool kAsym = NSB != NS;
    static constexpr int LDS_BYTES = kAsym ? NS * A_BYTES + NSB * B_BYTES : NS * STAGE_BYTES;
    static constexpr int LOADS = (BM / 8) / NW + (BN / 8) / NW;  // DMA loads per wave per chunk
    static constexpr int ZMB = ZR > 0 ? ZR / 32 : 1;  // side row blocks per wave
    static constexpr int ZPIECES = ZR / 8;            // 1 KiB wave pieces of the side rows
    // NS = 2: every wait is for all of a wave's copies, so the waves that copy
    // a side piece may issue one more load per chunk than the others.
    static_assert(ZR == 0 || (ZR % 32 == 0 && WGM == 2 && WTN == 64 && NS == 2 && ZPIECES <= NW),
                  "side operand layout");
    static_assert(NS >= 2 && (NS - 2) * LOADS < 64, "stages / vmcnt range");
    static_assert(!kAsym || (NS == 2 && NSB == 3 && ZR == 0), "split ring: NS = 2, NSB = 3, no side rows");
    static_assert(!(TA || TB) || (!kAsym && ZR == 0), "MN-major operands: plain ring, no side rows");
    // copy engines of the two operands (K-major or MN-major tiles)
    // K-major copies through buffer resources for bf16 (for fp32 the global
    // form: the compiler's register allocation of the fp32 kernels fares
    // worse with the resources)
    static constexpr bool kBuf = Elem<T>::kBytes == 2;
    using DKA = DmaOperand<BM, NW, kBuf>;
    using DKB = DmaOperand<BN, NW, kBuf>;
    using DA = typename PickT<TA, DmaOperandT<BM, NW, Elem<T>::kBytes>, DKA>::type;
    using DB = typename PickT<TB, DmaOperandT<BN, NW, Elem<T>::kBytes>, DKB>::type;
    static_assert(BM % (32 * WGM) == 0 && BN % (32 * WGN) == 0, "tile shape");
    static_assert(BM % 8 == 0 && BN % 8 == 0, "tile rows");
    static_assert((BM / 8) % NW == 0 && (BN / 8) % NW == 0, "pieces must split evenly over waves");

    __device__ static __forceinline__ void zero(f32x16_t (&acc)[MB][NB]) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }

    // Fragment of the 32 MN rows mn .. mn+31 of an MN-major tile of ROWS
    // rows for K step ks: the same lane layout as a K-major fragment (lane
    // l: row l % 32, K indices 8 (l / 32) .. +7 for bf16; 4 (l / 32) + t for
    // fp32's four K=2 steps).  bf16: two transposed reads of four K rows each;
    // fp32: four 4-byte reads (32 consecutive MN elements per half wave).
    template <int ROWS>
    __device__ static __forceinline__ u32x4_t frag_t(const char* tile, int mn, int ks) {
        constexpr int EB = Elem<T>::kBytes, RB = ROWS * EB, PPR = RB / 16;
        const int lane = threadIdx.x % kWave;
        if constexpr (EB == 2) {
            const int g = lane & 15, q = lane >> 4, j = g >> 2, r = g & 3;
            const int m = mn + 16 * (q & 1) + 4 * r;
            const int k0 = 16 * ks + 8 * (q >> 1) + j;
            const u32x2_t lo = lds_read_tr16(tile + k0 * RB + (((m >> 3) ^ tsw<PPR>(k0)) << 4) + 8 * (r & 1));
            const int k1 = k0 + 4;
            const u32x2_t hi = lds_read_tr16(tile + k1 * RB + (((m >> 3) ^ tsw<PPR>(k1)) << 4) + 8 * (r & 1));
            return u32x4_t{lo.x, lo.y, hi.x, hi.y};
        } else {
            const int h = lane >> 5, m = mn + (lane & 31);
            u32x4_t v;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int k = 8 * ks + 4 * h + t;
                v[t] = *(const uint32_t*)(tile + k * RB + (((m >> 2) ^ tsw<PPR>(k)) << 4) + 4 * (m & 3));
            }
            return v;
        }
    }

    // Fragments of one 32-byte K step (ks = 0..3 inside a 128-byte chunk).
    // K-major operands: ta / tb point at the wave's first row of the tile;
    // MN-major operands: at the tile (the wave's rows are found here).
    __device__ static __forceinline__ void load_frags(u32x4_t (&fa)[MB], u32x4_t (&fb)[NB], const char* ta,
                                                      const char* tb, int ks, int fr, int fh) {
        const int wave = threadIdx.x / kWave;
        if constexpr (TA) {
#pragma unroll
            for (int i = 0; i < MB; ++i) fa[i] = frag_t<BM>(ta, (wave / WGN) * WTM + i * 32, ks);
        } else {
#pragma unroll
            for (int i = 0; i < MB; ++i) fa[i] = *(const u32x4_t*)(ta + swz(i * 32 + fr, 2 * ks + fh));
        }
        if constexpr (TB) {
#pragma unroll
            for (int j = 0; j < NB; ++j) fb[j] = frag_t<BN>(tb, (wave % WGN) * WTN + j * 32, ks);
        } else {
#pragma unroll
            for (int j = 0; j < NB; ++j) fb[j] = *(const u32x4_t*)(tb + swz(j * 32 + fr, 2 * ks + fh));
        }
    }

    __device__ static __forceinline__ void mma_step(f32x16_t (&acc)[MB][NB], const u32x4_t (&fa)[MB],
                                                    const u32x4_t (&fb)[NB]) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) mma32(acc[i][j], fa[i], fb[j], T());
    }

    // Scheduling pattern for one K step: NMFMA MFMAs, each followed by one LDS
    // read while any remain (NREAD) and one DMA load while any remain (NVMEM).
    template <int NMFMA, int NREAD, int NVMEM>
    __device__ static __forceinline__ void sched_step() {
        constexpr int n0 = NREAD > NVMEM ? NREAD : NVMEM;
        constexpr int n = n0 < NMFMA ? n0 : NMFMA;
#pragma unroll
        for (int x = 0; x < n; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
            if (x < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            if (x < NVMEM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // DMA load
        }
        if constexpr (NMFMA > n) __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - n, 0);
    }

    // Side product state of one wave (used when ZR > 0 and `on`): the side
    // accumulators, their double-buffered fragments, and this lane's copy
    // source (waves below ZPIECES each copy one 1 KiB piece of the side rows).
    struct Side {
        f32x16_t acc[ZMB];
        u32x4_t fz[2][ZMB];
        const char* src;
        int wm;
        bool on;
    };

    __device__ static __forceinline__ void load_side(Side& sd, int buf, const char* tz, int ks, int fr, int fh) {
#pragma unroll
        for (int i = 0; i < ZMB; ++i) sd.fz[buf][i] = *(const u32x4_t*)(tz + swz(i * 32 + fr, 2 * ks + fh));
    }

    // Copy side rows of K chunk kc into the stage at `stage_base`: wave w <
    // ZPIECES copies rows 8w .. 8w+7 of the ZR x 128-byte side tile.
    __device__ static __forceinline__ void issue_side(const Side& sd, char* stage_base, int kc, int wave, int) {
        if (wave < ZPIECES)
            __builtin_amdgcn_global_load_lds((glb_ptr_t)(sd.src + (size_t)kc * 128),
                                             (lds_ptr_t)(stage_base + Z_OFF + wave * 1024), 16, 0, 0);
    }

    // One K step of a chunk: read the fragments of step KS+1 (if any), issue
    // the next chunk's DMA (ISSUE, step 0 only), multiply step KS.  SIDE adds
    // the side product (fragments from tz) when sd.on.
    template <int KS, bool ISSUE, bool SIDE>
    __device__ static __forceinline__ void step(f32x16_t (&acc)[MB][NB], u32x4_t (&fa)[2][MB],
                                                u32x4_t (&fb)[2][NB], const char* ta, const char* tb,
                                                const DA& da, const DB& db, char* nxt, int kc_next, int wave,
                                                int fr, int fh, Side& sd, const char* tz, int lane) {
        constexpr int NL = DA::kLoads + DB::kLoads;
        if constexpr (KS < 3) load_frags(fa[(KS + 1) & 1], fb[(KS + 1) & 1], ta, tb, KS + 1, fr, fh);
        if constexpr (SIDE && KS < 3) {
            if (sd.on) load_side(sd, (KS + 1) & 1, tz, KS + 1, fr, fh);
        }
        if constexpr (ISSUE && KS == 0) {
            da.issue(nxt, kc_next, wave);
            db.issue(nxt + A_BYTES, kc_next, wave);
            if constexpr (SIDE) {
                if (sd.on) issue_side(sd, nxt, kc_next, wave, lane);
            }
        }
        mma_step(acc, fa[KS & 1], fb[KS & 1]);
        if constexpr (SIDE) {
            if (sd.on) {
                const u32x4_t& bsel = sd.wm == 0 ? fb[KS & 1][0] : fb[KS & 1][1];
#pragma unroll
                for (int i = 0; i < ZMB; ++i) mma32(sd.acc[i], sd.fz[KS & 1][i], bsel, T());
            }
        }
        sched_step<MB * NB, (KS < 3 ? MB + NB : 0), ((ISSUE && KS == 0) ? NL : 0)>();
    }

    // One 128-byte K chunk from LDS (four K steps; fragments double-buffered
    // in registers).  With ISSUE the DMA copy of the next chunk is spread over
    // the first step's MFMAs.
    template <bool ISSUE, bool SIDE>
    __device__ static __forceinline__ void chunk(f32x16_t (&acc)[MB][NB], u32x4_t (&fa)[2][MB],
                                                 u32x4_t (&fb)[2][NB], const char* ta, const char* tb,
                                                 const DA& da, const DB& db, char* nxt, int kc_next, int wave,
                                                 int fr, int fh, Side& sd, const char* tz, int lane) {
        step<0, ISSUE, SIDE>(acc, fa, fb, ta, tb, da, db, nxt, kc_next, wave, fr, fh, sd, tz, lane);
        step<1, ISSUE, SIDE>(acc, fa, fb, ta, tb, da, db, nxt, kc_next, wave, fr, fh, sd, tz, lane);
        step<2, ISSUE, SIDE>(acc, fa, fb, ta, tb, da, db, nxt, kc_next, wave, fr, fh, sd, tz, lane);
        step<3, ISSUE, SIDE>(acc, fa, fb, ta, tb, da, db, nxt, kc_next, wave, fr, fh, sd, tz, lane);
    }

    // Wait until this wave's copy of the current chunk has landed, given that
    // the copies of `ahead` later chunks (issued after it) may be in flight.
    __device__ static __forceinline__ void wait_chunk(int ahead) {
        switch (ahead) {
            case 0: wait_vmcnt<0>(); break;
            case 1: wait_vmcnt<(NS > 2 ? 1 : 0) * LOADS>(); break;
            case 2: wait_vmcnt<(NS > 3 ? 2 : 0) * LOADS>(); break;
            case 3: wait_vmcnt<(NS > 4 ? 3 : 0) * LOADS>(); break;
            default: wait_vmcnt<(NS > 5 ? 4 : 0) * LOADS>(); break;
        }
    }

    // acc += A . B^T where A's and B's K axes are the concatenations
    // a0|a1 and b0|b1 (a0.chunks == b0.chunks, a1.chunks == b1.chunks); with
    // SIDE and sd.on also the side product.
    //
    // A ring of NS LDS stages, NS-1 chunk copies in flight.  Iteration kt:
    // issue the copy of chunk kt+NS-1 into the stage chunk kt-1 used (free
    // since the barrier that ended iteration kt-1), spread over the first K
    // step's MFMAs; multiply chunk kt (fragments register-double-buffered);
    // then wait for this wave's copy of chunk kt+1 (the later ones may still
    // fly), barrier, and read chunk kt+1's first fragments.  Ends with a
    // barrier (LDS free for the epilogue).
    template <bool SIDE>
    __device__ static __forceinline__ void run_impl(f32x16_t (&acc)[MB][NB], const KSeg& a0, const KSeg& a1,
                                                    int rows_a, const KSeg& b0, const KSeg& b1, int rows_b,
                                                    char* lds, Side& sd) {
        const int tid = threadIdx.x;
        const int wave = tid / kWave;
        const int lane = tid % kWave;
        const int wm = wave / WGN, wn = wave % WGN;
        const int nk = a0.chunks + a1.chunks;
        const int fr = lane & 31;  // fragment row
        const int fh = lane >> 5;  // fragment K half

        DA da;
        DB db;
        da.init(a0, a1, rows_a, wave, lane);
        db.init(b0, b1, rows_b, wave, lane);
#pragma unroll
        for (int c = 0; c < NS - 1; ++c)
            if (c < nk) {
                da.issue(lds + c * STAGE_BYTES, c, wave);
                db.issue(lds + c * STAGE_BYTES + A_BYTES, c, wave);
                if constexpr (SIDE) {
                    if (sd.on) issue_side(sd, lds + c * STAGE_BYTES, c, wave, lane);
                }
            }
        wait_chunk(min(NS - 2, nk - 1));
        __syncthreads();

        u32x4_t fa[2][MB], fb[2][NB];
        const int oa = TA ? 0 : (wm * WTM) * 128, ob = A_BYTES + (TB ? 0 : (wn * WTN) * 128);
        load_frags(fa[0], fb[0], lds + oa, lds + ob, 0, fr, fh);
        if constexpr (SIDE) {
            if (sd.on) load_side(sd, 0, lds + Z_OFF, 0, fr, fh);
        }

        // main loop: chunks whose iteration still issues a copy
        int stage = 0;
        int kt = 0;
        for (; kt + NS - 1 < nk; ++kt) {
            char* cur = lds + stage * STAGE_BYTES;
            char* dst = lds + (stage == 0 ? NS - 1 : stage - 1) * STAGE_BYTES;
            chunk<true, SIDE>(acc, fa, fb, cur + oa, cur + ob, da, db, dst, kt + NS - 1, wave, fr, fh, sd,
                              cur + Z_OFF, lane);
            wait_chunk(min(NS - 2, nk - 2 - kt));
            __syncthreads();
            stage = stage + 1 == NS ? 0 : stage + 1;
            char* n = lds + stage * STAGE_BYTES;
            load_frags(fa[0], fb[0], n + oa, n + ob, 0, fr, fh);
            if constexpr (SIDE) {
                if (sd.on) load_side(sd, 0, n + Z_OFF, 0, fr, fh);
            }
        }
        // tail: the last NS-1 chunks (all copies issued)
        for (; kt < nk; ++kt) {
            char* cur = lds + stage * STAGE_BYTES;
            chunk<false, SIDE>(acc, fa, fb, cur + oa, cur + ob, da, db, nullptr, 0, wave, fr, fh, sd, cur + Z_OFF,
                               lane);
            if (kt + 1 < nk) {
                wait_chunk(min(NS - 2, nk - 2 - kt));
                __syncthreads();
                stage = stage + 1 == NS ? 0 : stage + 1;
                char* n = lds + stage * STAGE_BYTES;
                load_frags(fa[0], fb[0], n + oa, n + ob, 0, fr, fh);
                if constexpr (SIDE) {
                    if (sd.on) load_side(sd, 0, n + Z_OFF, 0, fr, fh);
                }
            }
        }
        __syncthreads();  // LDS free for the epilogue
    }

    // One chunk kt of the split ring.  MORE_A: chunk kt+1 exists (copy A(kt+1),
    // then barrier and read chunk kt+1's first fragments); MORE_B: chunk kt+2
    // exists (copy B(kt+2), which may stay in flight across the barrier).
    template <bool MORE_A, bool MORE_B>
    __device__ static __forceinline__ void split_chunk(f32x16_t (&acc)[MB][NB], u32x4_t (&fa)[2][MB],
                                                       u32x4_t (&fb)[2][NB], char* la, char* lb,
                                                       const DKA& da, const DKB& db,
                                                       int& sa, int& sb, int kt, int wave, int fr, int fh, int oa,
                                                       int ob) {
        constexpr int LB = DKB::kLoads;
        const char* ca = la + sa * A_BYTES + oa;
        const char* cb = lb + sb * B_BYTES + ob;
        const int na = sa ^ 1;                    // A stage of chunk kt+1
        const int nb1 = sb == 2 ? 0 : sb + 1;     // B stage of chunk kt+1
        const int nb2 = nb1 == 2 ? 0 : nb1 + 1;   // B stage of chunk kt+2
        if constexpr (MORE_A) da.issue(la + na * A_BYTES, kt + 1, wave);
        if constexpr (MORE_B) db.issue(lb + nb2 * B_BYTES, kt + 2, wave);
        Side none;
        none.on = false;
        step<0, false, false>(acc, fa, fb, ca, cb, da, db, nullptr, 0, wave, fr, fh, none, nullptr, 0);
        step<1, false, false>(acc, fa, fb, ca, cb, da, db, nullptr, 0, wave, fr, fh, none, nullptr, 0);
        step<2, false, false>(acc, fa, fb, ca, cb, da, db, nullptr, 0, wave, fr, fh, none, nullptr, 0);
        step<3, false, false>(acc, fa, fb, ca, cb, da, db, nullptr, 0, wave, fr, fh, none, nullptr, 0);
        if constexpr (MORE_A) {
            ring_barrier<MORE_B ? LB : 0>();
            sa = na;
            sb = nb1;
            load_frags(fa[0], fb[0], la + sa * A_BYTES + oa, lb + sb * B_BYTES + ob, 0, fr, fh);
        }
    }

    // Workgroup barrier for the split ring: waits for this wave's LDS reads
    // (its fragments of the chunk just multiplied) and for all but the NOUT
    // most recent vector-memory operations (its copies of the next chunk);
    // unlike __syncthreads it does not wait for every copy in flight.  The
    // signal fences (no instructions) keep the compiler from moving memory
    // accesses across it.
    template <int NOUT>
    __device__ static __forceinline__ void ring_barrier() {
        static_assert(NOUT >= 0 && NOUT < 64, "vmcnt out of range");
        __builtin_amdgcn_s_waitcnt((NOUT & 0xF) | ((NOUT >> 4) << 14) | 0x70);  // lgkmcnt(0), vmcnt(NOUT)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }

    // acc += A . B^T with the split ring (NS = 2 A stages, NSB = 3 B stages).
    // Copy order: A(0), B(0), B(1), then iteration kt issues A(kt+1) and
    // B(kt+2).  Vector-memory loads complete in issue order, so chunk kt+1 is
    // complete (A(kt+1) and the earlier B(kt+1)) once at most B(kt+2)'s loads
    // are outstanding.  A stage kt%2 and B stage kt%3 are rewritten only in
    // iteration kt+1, after the barrier that ends iteration kt.
    __device__ static __forceinline__ void run_split(f32x16_t (&acc)[MB][NB], const KSeg& a0, const KSeg& a1,
                                                     int rows_a, const KSeg& b0, const KSeg& b1, int rows_b,
                                                     char* lds) {
        static_assert(kAsym, "split ring only");
        constexpr int LB = DKB::kLoads;
        const int tid = threadIdx.x;
        const int wave = tid / kWave;
        const int lane = tid % kWave;
        const int wm = wave / WGN, wn = wave % WGN;
        const int nk = a0.chunks + a1.chunks;
        const int fr = lane & 31;
        const int fh = lane >> 5;
        char* const la = lds;                  // A stages
        char* const lb = lds + NS * A_BYTES;   // B stages

        DKA da;
        DKB db;
        da.init(a0, a1, rows_a, wave, lane);
        db.init(b0, b1, rows_b, wave, lane);
        if (nk > 0) {
            da.issue(la, 0, wave);
            db.issue(lb, 0, wave);
        }
        if (nk > 1) {
            db.issue(lb + B_BYTES, 1, wave);
            ring_barrier<LB>();
        } else {
            ring_barrier<0>();
        }

        u32x4_t fa[2][MB], fb[2][NB];
        const int oa = (wm * WTM) * 128, ob = (wn * WTN) * 128;
        load_frags(fa[0], fb[0], la + oa, lb + ob, 0, fr, fh);

        int sa = 0, sb = 0;  // stages of chunk kt
        int kt = 0;
        for (; kt + 2 < nk; ++kt) split_chunk<true, true>(acc, fa, fb, la, lb, da, db, sa, sb, kt, wave, fr, fh, oa, ob);
        if (kt + 1 < nk) {
            split_chunk<true, false>(acc, fa, fb, la, lb, da, db, sa, sb, kt, wave, fr, fh, oa, ob);
            ++kt;
        }
        if (kt < nk) split_chunk<false, false>(acc, fa, fb, la, lb, da, db, sa, sb, kt, wave, fr, fh, oa, ob);
        __syncthreads();  // LDS free for the epilogue
    }

    __device__ static __forceinline__ void run_segs(f32x16_t (&acc)[MB][NB], const KSeg& a0, const KSeg& a1,
                                                    int rows_a, const KSeg& b0, const KSeg& b1, int rows_b,
                                                    char* lds) {
        if constexpr (kAsym) {
            run_split(acc, a0, a1, rows_a, b0, b1, rows_b, lds);
        } else {
            Side none;
            none.on = false;
            run_impl<false>(acc, a0, a1, rows_a, b0, b1, rows_b, lds, none);
        }
    }

    // acc += A . B^T over K elements (a multiple of KELEMS), one segment each.
    __device__ static __forceinline__ void run(f32x16_t (&acc)[MB][NB], const char* a, size_t pitch_a, int rows_a,
                                               const char* b, size_t pitch_b, int rows_b, int K, char* lds) {
        const int nk = K / KELEMS;
        run_segs(acc, KSeg{a, pitch_a, nk}, KSeg{a, pitch_a, 0}, rows_a, KSeg{b, pitch_b, nk}, KSeg{b, pitch_b, 0},
                 rows_b, lds);
    }

    // As run(), plus (when `on`, block-uniform) the side product of ZR rows
    // (K-major, rows z_pitch bytes apart, all present) with the B tile: side
    // row r < zsplit is row r at z, side row r >= zsplit is row r - zsplit at
    // z2 (zsplit a multiple of 8, so each 8-row copy piece lies in one part).
    // sd.acc[i] (16 floats per lane) holds side rows i*32 + 8*(r/4) + 4*(l/32)
    // + r%4 (lane l, register r) times B-tile column wn*64 + wm*32 + l%32.
    __device__ static __forceinline__ void run_with_side(f32x16_t (&acc)[MB][NB], Side& sd, const char* a,
                                                         size_t pitch_a, int rows_a, const char* b, size_t pitch_b,
                                                         int rows_b, int K, const char* z, const char* z2,
                                                         int zsplit, size_t z_pitch, bool on, char* lds) {
        static_assert(ZR > 0, "core without side rows");
        const int nk = K / KELEMS;
        const int wave = threadIdx.x / kWave;
        const int lane = threadIdx.x % kWave;
        sd.on = on;
        sd.wm = wave / WGN;
#pragma unroll
        for (int i = 0; i < ZMB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) sd.acc[i][r] = 0.f;
        // lane's 16-byte piece: row 8*wave + lane/8 (waves below ZPIECES),
        // physical piece lane % 8, logical piece (lane % 8) ^ perm(row)
        const int row = (wave < ZPIECES ? wave : 0) * 8 + (lane >> 3);
        const char* zrow = row < zsplit ? z + (size_t)row * z_pitch : z2 + (size_t)(row - zsplit) * z_pitch;
        sd.src = zrow + (((lane & 7) ^ ((row >> 1) & 7)) << 4);
        run_impl<true>(acc, KSeg{a, pitch_a, nk}, KSeg{a, pitch_a, 0}, rows_a, KSeg{b, pitch_b, nk},
                       KSeg{b, pitch_b, 0}, rows_b, lds, sd);
    }

    // Apply f4(row0, col, v) to groups of four consecutive accumulator rows of
    // one column (the elements a lane holds together); v is modified in place.
    template <typename F>
    __device__ static __forceinline__ void transform4(f32x16_t (&acc)[MB][NB], F&& f4) {
        const int wave = threadIdx.x / kWave;
        const int lane = threadIdx.x % kWave;
        const int wm = wave / WGN, wn = wave % WGN;
        const int c = lane & 31;
        const int h = lane >> 5;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    float v[4] = {acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                                  acc[i][j][4 * g4 + 3]};
                    f4(wm * WTM + i * 32 + 8 * g4 + 4 * h, wn * WTN + j * 32 + c, v);
#pragma unroll
                    for (int t = 0; t < 4; ++t) acc[i][j][4 * g4 + t] = v[t];
                }
    }

    // Apply f to every accumulator element in place: acc = f(row, col, acc).
    template <typename F>
    __device__ static __forceinline__ void transform(f32x16_t (&acc)[MB][NB], F&& f) {
        const int wave = threadIdx.x / kWave;
        const int lane = threadIdx.x % kWave;
        const int wm = wave / WGN, wn = wave % WGN;
        const int c = lane & 31;
        const int h = lane >> 5;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = f(wm * WTM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3), wn * WTN + j * 32 + c,
                                     acc[i][j][r]);
    }

    // Store the block tile through LDS with 16-byte global stores.
    //   TRANSPOSED = false: staged rows are tile rows; dst(row, col) gives the
    //     global address of element (row, col..col+V-1) or nullptr to skip.
    //   TRANSPOSED = true: staged rows are tile columns; dst(col, row) gives
    //     the address of elements (row..row+V-1, col).
    // val(row, col, acc) gives the value stored (in OutT); emit(d, v) writes
    // one staged 16-byte vector v to d (a plain store by default).  When the staged
    // tile does not fit in LDS at once it is staged in passes of one wave row
    // (or column) of the wave grid.  Begins and ends with a barrier.
    struct PlainEmit {
        __device__ __forceinline__ void operator()(char* d, const u32x4_t& v) const { *(u32x4_t*)d = v; }
    };

    template <typename OutT, bool TRANSPOSED, typename V, typename D, typename E = PlainEmit>
    __device__ static __forceinline__ void store(const f32x16_t (&acc)[MB][NB], char* lds, int lds_bytes, V&& val,
                                                 D&& dst, E&& emit = E()) {
        constexpr int EB = Elem<OutT>::kBytes;
        constexpr int SROWS = TRANSPOSED ? BN : BM;  // staged rows
        constexpr int SCOLS = TRANSPOSED ? BM : BN;  // elements per staged row
        constexpr int PITCH = SCOLS * EB + 16;
        constexpr int NG = TRANSPOSED ? WGN : WGM;   // wave groups along the staged rows
        const int npass = SROWS * PITCH <= lds_bytes ? 1 : NG;
        const int prows = SROWS / npass;
        const int wave = threadIdx.x / kWave;
        const int lane = threadIdx.x % kWave;
        const int wm = wave / WGN, wn = wave % WGN;
        const int c = lane & 31;
        const int h = lane >> 5;
        const int mygroup = TRANSPOSED ? wn : wm;
        constexpr int VPR = SCOLS * EB / 16;  // 16-byte vectors per staged row
        for (int pass = 0; pass < npass; ++pass) {
            __syncthreads();
            if (npass == 1 || mygroup == pass) {
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int row = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                            const int col = wn * WTN + j * 32 + c;
                            const float x = val(row, col, acc[i][j][r]);
                            if (TRANSPOSED)
                                Elem<OutT>::put(lds + (col - pass * prows) * PITCH + row * EB, x);
                            else
                                Elem<OutT>::put(lds + (row - pass * prows) * PITCH + col * EB, x);
                        }
            }
            __syncthreads();
            for (int idx = threadIdx.x; idx < prows * VPR; idx += NT) {
                const int srow = idx / VPR;
                const int v = idx % VPR;
                char* d = dst(pass * prows + srow, v * (16 / EB));
                if (d) emit(d, *(const u32x4_t*)(lds + srow * PITCH + v * 16));
            }
        }
    }

    // The LDS writes of one pass of store_packed: staged element (col - pass
    // prows, row) = val(row, col, acc) for the waves of wave column `pass`
    // (all waves when npass == 1), rows BM * EB + 16 bytes apart.  Each lane
    // holds four consecutive accumulator rows of one column, so every write is
    // one packed 4-element store (8 bytes for bf16).
    template <typename OutT, typename V>
    __device__ static __forceinline__ void stage_packed(const f32x16_t (&acc)[MB][NB], char* lds, int pass, int prows,
                                                        int npass, V&& val) {
        constexpr int EB = Elem<OutT>::kBytes;
        constexpr int PITCH = BM * EB + 16;
        const int wave = threadIdx.x / kWave;
        const int lane = threadIdx.x % kWave;
        const int wm = wave / WGN, wn = wave % WGN;
        const int c = lane & 31;
        const int h = lane >> 5;
        if (npass == 1 || wn == pass) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int row0 = wm * WTM + i * 32 + 8 * g4 + 4 * h;
                        const int col = wn * WTN + j * 32 + c;
                        float x[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) x[t] = val(row0 + t, col, acc[i][j][4 * g4 + t]);
                        char* q = lds + (col - pass * prows) * PITCH + row0 * EB;
                        if constexpr (EB == 2) {
                            u32x2_t w;
                            w.x = pack_bf16x2(x[0], x[1]);
                            w.y = pack_bf16x2(x[2], x[3]);
                            *(u32x2_t*)q = w;
                        } else {
                            *(f32x4_t*)q = f32x4_t{x[0], x[1], x[2], x[3]};
                        }
                    }
        }
    }

    // Store the block tile through LDS with the accumulator's column index as
    // the staged row: staged element (col, row) = val(row, col, acc) (written
    // by stage_packed).  dst(srow, scol) gives the global address of staged
    // elements (srow, scol..scol+V-1) or nullptr; the caller picks the operand
    // order so that the staged rows are the rows of the global layout.
    // Passes as in store().
    template <typename OutT, typename V, typename D, typename E = PlainEmit>
    __device__ static __forceinline__ void store_packed(const f32x16_t (&acc)[MB][NB], char* lds, int lds_bytes,
                                                        V&& val, D&& dst, E&& emit = E()) {
        constexpr int EB = Elem<OutT>::kBytes;
        constexpr int SROWS = BN, SCOLS = BM;
        constexpr int PITCH = SCOLS * EB + 16;
        const int npass = SROWS * PITCH <= lds_bytes ? 1 : WGN;
        const int prows = SROWS / npass;
        constexpr int VPR = SCOLS * EB / 16;
        for (int pass = 0; pass < npass; ++pass) {
            __syncthreads();
            stage_packed<OutT>(acc, lds, pass, prows, npass, val);
            __syncthreads();
            for (int idx = threadIdx.x; idx < prows * VPR; idx += NT) {
                const int srow = idx / VPR;
                const int v = idx % VPR;
                char* d = dst(pass * prows + srow, v * (16 / EB));
                if (d) emit(d, *(const u32x4_t*)(lds + srow * PITCH + v * 16));
            }
        }
    }

    // Whether store_packed_cols fits (two buffers of WGN * 32 staged rows of
    // OutT in LDS_BYTES).
    template <typename OutT, int LDS_BYTES>
    static constexpr bool kColsFit = 2 * WGN * 32 * (BM * Elem<OutT>::kBytes + 16) <= LDS_BYTES;

    // store_packed with an elementwise f applied on the way, in NB passes of
    // one accumulator block column each (every wave's block column j: the
    // staged rows wn * WTN + j * 32 + c, WGN * 32 of them).  Pass j applies f
    // to acc[.][j], stages the result and stores it; the passes alternate
    // between two LDS buffers, so one barrier per pass suffices and the
    // global stores of pass j are in flight while pass j + 1 computes.
    // Requires kColsFit.  Begins with a barrier.
    template <typename OutT, int LDS_BYTES, typename F, typename D>
    __device__ static __forceinline__ void store_packed_cols(f32x16_t (&acc)[MB][NB], char* lds, F&& f, D&& dst) {
        constexpr int EB = Elem<OutT>::kBytes;
        constexpr int PITCH = BM * EB + 16;
        constexpr int SROWS = WGN * 32;  // staged rows per pass
        constexpr int BUF = SROWS * PITCH;
        constexpr int VPR = BM * EB / 16;
        static_assert(kColsFit<OutT, LDS_BYTES>, "two column-pass buffers must fit");
        const int wave = threadIdx.x / kWave;
        const int lane = threadIdx.x % kWave;
        const int wm = wave / WGN, wn = wave % WGN;
        const int c = lane & 31;
        const int h = lane >> 5;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            char* buf = lds + (j & 1) * BUF;
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int row0 = wm * WTM + i * 32 + 8 * g4 + 4 * h;
                    const int col = wn * WTN + j * 32 + c;
                    float x[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) x[t] = f(row0 + t, col, acc[i][j][4 * g4 + t]);
                    char* q = buf + (wn * 32 + c) * PITCH + row0 * EB;
                    if constexpr (EB == 2) {
                        *(u32x2_t*)q = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                    } else {
                        *(f32x4_t*)q = f32x4_t{x[0], x[1], x[2], x[3]};
                    }
                }
            __syncthreads();
            for (int idx = threadIdx.x; idx < SROWS * VPR; idx += NT) {
                const int srow = idx / VPR;
                const int v = idx % VPR;
                char* d = dst((srow >> 5) * WTN + j * 32 + (srow & 31), v * (16 / EB));
                if (d) *(u32x4_t*)d = *(const u32x4_t*)(buf + srow * PITCH + v * 16);
            }
        }
    }

    // f(row, col, value) for every accumulator element; row/col relative to
    // the block tile.
    template <typename F>
    __device__ static __forceinline__ void for_each(const f32x16_t (&acc)[MB][NB], F&& f) {
        const int wave = threadIdx.x / kWave;
        const int lane = threadIdx.x % kWave;
        const int wm = wave / WGN, wn = wave % WGN;
        const int c = lane & 31;
        const int h = lane >> 5;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    f(wm * WTM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3), wn * WTN + j * 32 + c, acc[i][j][r]);
    }
};

}  // namespace gau
