// Host-side launch interface between the C ABI (gau_api.hip) and the kernel
// translation units.  Internal to libgau; not exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gau {

// Fused projection + SiLU + scale/offset heads.
struct ProjParams {
    const void* X;      // [M, d]
    const void* W_u;    // [e, d]  (W_u transposed)
    const void* W_v;    // [e, d]
    const void* W_z;    // [s, d]
    const float* scale;   // [4, s]
    const float* offset;  // [4, s]
    void* U;    // [M, e]
    void* Vt;   // [B, e, T]
    void* Qq;   // [M, s]
    void* Kq;   // [M, s]
    void* Ql;   // [M, s]
    void* Klt;  // [B, s, T]
    int M, T, d, e, s;
    int rope;   // 1: the four heads rotated by position t = m mod T (in the epilogue)
    void* H;    // [M, 2e+s] token-major pre-activations X [W_u | W_v | W_z] (row pitch 2e+s),
                // written when non-null (the backward's recompute), instead of U and besides
                // the other activated outputs
};

// Per-chunk state S_g^T = lin_scale * V_g^T K_lin_g, [B, G, e, s] in the
// layer's element type (fp32 accumulation).
struct StateParams {
    const void* Vt;   // [B, e, T]
    const void* Klt;  // [B, s, T]
    void* S;          // [B, G, e, s]
    int B, T, e, s, C;
    float lin_scale;
};

// Exclusive prefix over chunks (causal) or the total (non-causal); with
// segment ids, the average over the chunks visible in the chunk's segment.
struct ScanParams {
    const void* S;   // [B, G, e, s], element type of the layer
    void* P;         // [B, G, e, s] causal or segmented (may be S: scanned in place), [B, 1, e, s] otherwise
    int B, G, es;    // es = e * s
    int causal;
    const int32_t* seg;  // [B, G] chunk segment ids, or nullptr (no segments)
};

// Per-chunk attention weights A_g = relu^2(quad_scale Q_quad K_quad^T + Bias),
// causal-masked, [B*G, C, C] (query-major); causal: only the key tiles at or
// below the diagonal are written (the consumer reads no others).
struct ScoresParams {
    const void* Qq;   // [M, s]
    const void* Kq;   // [M, s]
    const float* relpos;  // [2C-1]
    void* A;          // [B*G, C, C]
    int B, T, s, C;
    int causal;
    float quad_scale;
};

// Per chunk: Y = U * (A_g V_g + Q_lin_g P_g), one GEMM with K = keys then s.
struct AttnParams {
    const void* A;    // [B*G, C, C]
    const void* Ql;   // [M, s]
    const void* Vt;   // [B, e, T]
    const void* P;    // [B, G or 1, e, s]
    const void* U;    // [M, e], or nullptr: no gate (Y = A_g V_g + Q_lin P_g)
    void* Y;          // [M, e]; may be U (gated in place)
    int B, T, e, s, C;
    int causal;
    int local, global;  // which terms enter Y (the LocalOnly / GlobalOnly variants)
    int p_chunked;      // P holds one state per chunk also when non-causal (segments)
};

// Output projection O = Y W_o (optionally O = residual + Y W_o in fp32).
struct OutParams {
    const void* Y;     // [M, e]
    const void* W_o;   // [d, e]  (W_o transposed)
    void* O;           // [M, d]  element type of the layer, or fp32 when residual or f32_out
    const float* residual;  // [M, d] fp32 or nullptr
    int M, d, e;
    int f32_out;       // O in fp32 without a residual (the backward's dX = dH W^T)
    int o_rp;          // elements between rows of O (and of residual); 0: d
    // gate epilogue of the backward (when gH != nullptr), with v = the product
    // (dY) in fp32, h = gH[m, n] and U = SiLU(h) (formed from h, with the
    // sigmoid SiLU' needs), per element at row m, column n (gate index
    // j = m g_rp + n):
    //   gDWq[j] = v U, gY[j] = U Wq, O[m, n] = v Wq SiLU'(h), element type
    const void* gH;    // pre-activations X W_u, pitch o_rp
    const void* gW;    // Wq (ungated attention output)
    void* gDWq;
    void* gY;
    int g_rp;
    // split-K (fp32 output without residual or gate only): block z of ksplit
    // takes K chunks [z*(nk/ksplit) + min(z, nk%ksplit), ...) of the nk = e/64
    // (bf16) and writes its partial product at O + z * o_bs elements
    int ksplit;        // 0 or 1: one K range
    int64_t o_bs;
    int k_rp;          // elements between rows of W_o and Y (their K pitch); 0: e
    int bm;            // feature-tile width (256, 192 or 128); 0: chosen from d and M
    // MN-major operands (tn = 1; 256-feature tiles, fp32 output without
    // residual or gate only): K row k of Y holds its M elements contiguously
    // from Y + k * k_rp, K row k of W_o its d elements from W_o + k * w_rp
    int tn;
    int w_rp;
};

// Blocks of a split-K output GEMM of d x M outputs with feature tiles of bm.
int out_gemm_tiles(int d, int M, int bm);

// Row RMS normalisation for the layer stack: Xn = bf16(x / sqrt(mean(x^2) + eps)).
struct NormParams {
    const float* x;  // [M, d]
    void* xn;        // [M, d] layer element type
    int M, d;
    float eps;
};

hipError_t launch_proj(const ProjParams& p, bool bf16_storage, hipStream_t st);  // U, Vt, Z heads (+ RoPE)

// One incremental decoding step (causal): token t, chunk slot j = t mod C.
struct DecodeParams {
    const void* x;      // [B, d]  the new tokens
    const void* W_u;    // [e, d]
    const void* W_v;    // [e, d]
    const void* W_z;    // [s, d]
    const void* W_o;    // [d, e]
    const float* scale;   // [4, s]
    const float* offset;  // [4, s]
    const float* relpos;  // [2C-1]
    void* o;            // [B, d]
    float* P;           // [B, s, e] fp32 state: completed chunks' summaries
    void* Pr;           // [B, s, e] the state in the element type, as the steps read it
                        // (bf16: rounded from P at each chunk end; fp32: P itself)
    void* Kq;           // [B, C, s] chunk cache
    void* V;            // [B, C, e]
    void* Kl;           // [B, C, s]
    float *u, *z;       // [B, e], [B, s] fp32 scratch
    void* y;            // [B, e] element type scratch (the gated attention output)
    int B, d, e, s, C, t, j, rope;
    float qs, ls;
    int local, global;  // which terms enter y (the LocalOnly / GlobalOnly variants)
};

hipError_t launch_decode_step(const DecodeParams& p, bool bf16_storage, hipStream_t st);
hipError_t launch_fill_zero(float* x, size_t n, hipStream_t st);
// w[n-1 + d] = a . rope(b, d), d = -(n-1) .. n-1 (a, b: [dim] fp32; w: [2n-1])
hipError_t launch_rope_relpos(const float* a, const float* b, int n, int dim, float* relpos, hipStream_t st);
hipError_t launch_chunk_state(const StateParams& p, bool bf16_storage, hipStream_t st);
hipError_t launch_chunk_scan(const ScanParams& p, bool bf16_storage, hipStream_t st);
hipError_t launch_chunk_scores(const ScoresParams& p, bool bf16_storage, hipStream_t st);
// Scores and states in one launch (the forward pass's stages 1 and 2).
hipError_t launch_chunk_scores_state(const ScoresParams& ps, const StateParams& pt, bool bf16_storage,
                                     hipStream_t st);
hipError_t launch_chunk_attn(const AttnParams& p, bool bf16_storage, hipStream_t st);
hipError_t launch_out_gemm(const OutParams& p, bool bf16_storage, hipStream_t st);
hipError_t launch_rms_norm(const NormParams& p, bool bf16_storage, hipStream_t st);

// ---- backward pass -------------------------------------------------------

// Epilogues of the backward GEMM (value v = alpha * accumulator at (row, col),
// i its index in C).
enum { EPI_STORE = 0,  // C[i] = v (fp32 when c_f32, else the element type)
       EPI_SILU = 1 }; // C[i] = v * SiLU'(H[i])

// Batched C[z] = alpha * (A[z] B[z]^T + A2[z] B2[z]^T) on the MFMA core, 64 x 64
// or 128 x 128 output tiles.  Each operand is K-major (*_t = 0: row r of its
// M or N axis holds its K elements contiguously, rows *_rp elements apart) or
// MN-major (*_t = 1: K index k holds its M or N elements contiguously, K rows
// *_rp elements apart).  Batch entry z is chunk z % zg of sequence z / zg; an
// operand's entry starts at (z / zg) * *_bsq + (z % zg) * *_bs elements, C's
// at z * c_bs, C's rows c_rp elements apart.  K and K2 are multiples of 64,
// every dimension a multiple of 64.  The second segment is used when K2 > 0.
// Layouts implemented: (a_t, b_t) = (0, 0), (0, 1), (1, 1) (the SiLU epilogue:
// (0, 0), (1, 1)); with a second segment and the SiLU epilogue (1, 1) then
// (a2_t, b2_t) = (0, 0).
struct GemmNTParams {
    const void* A;
    const void* B;
    void* C;
    int64_t a_bs, b_bs, c_bs;
    int64_t a_bsq, b_bsq;
    int a_rp, b_rp, c_rp;
    int zg;
    int K;
    int c_f32;
    float alpha;
    int tm, tn;  // row / column tiles per batch entry (set by the launcher)
    const void* A2;
    const void* B2;
    int64_t a2_bs, b2_bs, a2_bsq, b2_bsq;
    int a2_rp, b2_rp;
    int K2;
    int epi;
    const void* H;              // EPI_SILU
    int skip_upper;  // skip output tiles wholly above the diagonal (never read)
    int a_t, b_t, a2_t, b2_t;
    int bt;          // tile size 64 or 128; 0: 128 when it divides M and N and gives >= 512 blocks
    int k_from_row;  // the first segment's K range starts at the tile's first row m0 (A[z][r][k]
                     // = 0 for k < r, e.g. the transposed causal scores)
};

// out[z][c][r] = in[z][r][c], element type, R and Cc multiples of 64.
struct TransposeParams {
    const void* in;
    void* out;
    int64_t in_bs, out_bs;
    int in_rp, out_rp;
    int tr, tc;  // row / column tiles per batch entry (set by the launcher)
};

// The scores' elementwise step (see backward.hip).
struct BwdElemParams {
    const float* f1;   // dA, fp32
    const void* b;     // A, element type
    void* o0;          // dSc, element type
    size_t n;          // entries: chunks * C * C
    int C, causal;
};

struct BwdScanParams {
    const float* dP;  // [B, G, es] fp32
    void* dS;         // [B, G, es] element type, times scale
    int B, G, es, causal;
    float scale;
    const int32_t* seg;  // [B, G] chunk segment ids, or nullptr (no segments)
};

constexpr int kHeadsBwdTokens = 16;  // tokens per block of the heads' backward step

struct BwdHeadsParams {
    const float* dh[4];  // gradients of Q_quad, K_quad, Q_lin, K_lin, [M, s] fp32
    const void* Hz;      // pre-activation of Z: row m at Hz + m * hpitch elements
    int hpitch;
    const float* scale;  // [4, s]
    void* dHz;           // its gradient, same layout as Hz
    float* part;         // [ceil(M / kHeadsBwdTokens), 8, s] per-block sums
    int M, s;
    int rope, T;         // rope: the heads were rotated by position m mod T
};

hipError_t launch_gemm_nt(const GemmNTParams& q, int M, int N, int nb, bool bf16_storage, hipStream_t st);

// Up to kTransposeBatch independent transposes (job j: R[j] x Cc[j], nb[j]
// batch entries) in one launch.
constexpr int kTransposeBatch = 16;
struct TransposeBatch {
    TransposeParams job[kTransposeBatch];
    int start[kTransposeBatch + 1];
    int n;
};
hipError_t launch_transpose_batch(const TransposeParams* jobs, const int* R, const int* Cc, const int* nb, int n,
                                  bool bf16_storage, hipStream_t st);
// dSc from dA (element type) and the bias gradient: per chunk and 32-row slab
// the diagonal sums into part [chunks * C / 32, 2C-1], then their column sums
// into drelpos [2C-1].
hipError_t launch_scores_bwd(const BwdElemParams& q, float* part, float* drelpos, bool bf, hipStream_t st);
// For each job j < jobs (at most 4), in one launch:
// outs[j][i] = sum_{z < S} parts[j][z * stride + i], i < ns[j]
// (ns[j] <= stride, both multiples of 4)
hipError_t launch_split_reduce(const float* const* parts, float* const* outs, const int64_t* ns, int jobs,
                               int64_t stride, int S, hipStream_t st);
hipError_t launch_scan_bwd(const BwdScanParams& q, bool bf16_storage, hipStream_t st);
hipError_t launch_heads_bwd(const BwdHeadsParams& q, float* dscale, float* doffset, bool bf16_storage,
                            hipStream_t st);

}  // namespace gau
