/*
 * gau.h -- C ABI of libgau, the forward pass of the FLASH gated attention unit
 * (GAU) with mixed chunk attention, for AMD Instinct MI355X (gfx950).
 *
 * What is computed ("Transformer Quality in Linear Time", Hua, Dai, Liu, Le;
 * equations as summarised on the wikillm page, section "Method", and in Su
 * Jianlin's post "FLASH: Possibly the Most Interesting Efficient Transformer
 * Design in Recent Times", sections "Gated Attention" and "Mixed Chunking"):
 *
 *   U = SiLU(X W_u),  V = SiLU(X W_v),  Z = SiLU(X W_z)        (GAU, eq. 1-4)
 *   Q_quad, K_quad, Q_lin, K_lin = Z * gamma_h + beta_h, h = 0..3
 *   per chunk g of C tokens (G = T / C chunks):
 *     V_quad_g = relu^2(quad_scale * Q_quad_g K_quad_g^T + Bias) V_g
 *                Bias[i][j] = relpos[C-1 + j - i]   (papercache page,
 *                appendix D, Code 4, branch n < 512); causal: entries with
 *                key j > query i are zeroed after relu^2
 *     S_g      = lin_scale * K_lin_g^T V_g                      (s x e)
 *     P_g      = sum_{h<g} S_h   (causal, eq. 8)
 *              = sum_{h}   S_h   (non-causal, eq. 7)
 *     V_lin_g  = Q_lin_g P_g
 *   O_g = [U_g * (V_quad_g + V_lin_g)] W_o         (display after eq. 8)
 *
 * The listing (Code 8 as rewritten on the wikillm page) divides Q K^T by C and
 * each chunk summary by C; the equations use no factor.  Both factors are
 * arguments here (gau_config.quad_scale, gau_config.lin_scale); the listing's
 * reading is quad_scale = lin_scale = 1/C.  No dense-layer biases.
 *
 * Optional rotary position embedding (gau_config.rope = 1): the listing rotates
 * the four heads after the scale+offset, by each token's position in its
 * sequence (0 .. T-1, not restarted per chunk; wikillm, FLASH block
 * pseudocode and "Paper vs code").  The rotation is not printed on the pages;
 * here the pair (h_i, h_{i+s/2}) at position t turns by t * theta_i with
 * theta_i = 10000^(-i/(s/2)), the frequency schedule and half-split layout of
 * the sinusoid helper the pages do print (papercache, appendix D,
 * _get_scaledsin).
 *
 * Conventions for every entry point:
 *  - Every pointer is caller-owned device memory (HBM of the current HIP
 *    device) unless stated otherwise.  The library allocates nothing and may
 *    be called from several host threads at once; its only global state is
 *    the scratch array of gau_forward_noalloc (below) and that array's
 *    address per device.
 *  - Work is queued on `stream` (a hipStream_t; NULL is the default stream)
 *    and the call returns without synchronising.
 *  - Arguments are checked before anything is queued.  A non-OK status means
 *    nothing was queued and no output was touched, except GAU_ERR_HIP, which
 *    reports a failed launch (outputs then are unspecified).
 *  - All pointers must be 16-byte aligned.  Outputs must not alias inputs.
 *  - Matrix layouts are row-major.  Weight matrices W in R^{in x out} (the
 *    pages' orientation, X W) are passed output-major: element (i, o) of W at
 *    offset o * in + i, i.e. an out x in row-major array (W transposed).
 */
#ifndef GAU_H
#define GAU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GAU_OK = 0,
    GAU_ERR_NULL = 1,       /* a required pointer is NULL                        */
    GAU_ERR_SHAPE = 2,      /* unsupported shape (see gau_config)                */
    GAU_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned                  */
    GAU_ERR_DTYPE = 4,      /* dtype is not GAU_F32 or GAU_BF16                  */
    GAU_ERR_WORKSPACE = 5,  /* workspace smaller than gau_workspace_bytes()      */
    GAU_ERR_HIP = 6         /* a kernel launch failed                            */
} gau_status;

typedef enum {
    GAU_F32 = 0,   /* fp32 storage, fp32 MFMA arithmetic                         */
    GAU_BF16 = 1   /* bf16 storage, bf16 MFMA with fp32 accumulation             */
} gau_dtype;

/*
 * Layer shape and options.
 *   B batch, T tokens per sequence, d model width, e expanded width,
 *   s shared (attention) width, C chunk length; G = T / C.
 * Supported: B, T >= 0 (B*T == 0 is a no-op); T % C == 0 (the chunking splits
 *   the sequence into whole chunks, wikillm "Method", papercache 3.2);
 *   C in {64, 128, 256, 512}; d % 128 == 0; e % 256 == 0; s in {128, 256};
 *   B*T <= 2^30, d, e <= 65536, B*T*max(d, e) <= 2^40 and B*e*s < 2^33 (the
 *   kernels' grids and index arithmetic); in bf16 also T <= 2^22 (32-bit
 *   offsets of the operand tiles the matrix cores copy, whose rows are
 *   T-element token runs).  Otherwise GAU_ERR_SHAPE.
 */
typedef struct {
    int64_t B, T, d, e, s, C;
    int32_t causal;      /* 1: lower-triangular in-chunk mask and exclusive chunk
                            prefix (eq. 8); 0: full in-chunk attention and the
                            sum over all chunks (eq. 7)                          */
    int32_t dtype;       /* gau_dtype of X, W_*, O and the stored intermediates  */
    float quad_scale;    /* multiplies Q_quad K_quad^T before the bias is added  */
    float lin_scale;     /* multiplies every chunk summary K_lin^T V             */
    int32_t rope;        /* 1: rotate the four heads by position (see above);
                            0: no rotation; anything else is GAU_ERR_SHAPE      */
    int32_t ablation;    /* GAU_FULL (0): the layer as above; GAU_LOCAL_ONLY:
                            V_lin = 0; GAU_GLOBAL_ONLY: V_quad = 0 (the
                            LocalOnly / GlobalOnly variants, wikillm "Ablation
                            variants"); anything else is GAU_ERR_SHAPE          */
} gau_config;

enum { GAU_FULL = 0, GAU_LOCAL_ONLY = 1, GAU_GLOBAL_ONLY = 2 };

/*
 * Byte offsets, inside the workspace, of the intermediates gau_forward leaves
 * there (valid after the stream has reached the end of the call).  "dt" is the
 * element type selected by gau_config.dtype.
 *   U       [B*T, e]      dt    SiLU(X W_u)
 *   Vt      [B, e, T]     dt    SiLU(X W_v), transposed per sequence
 *   Q_quad  [B*T, s]      dt
 *   K_quad  [B*T, s]      dt
 *   Q_lin   [B*T, s]      dt
 *   K_lin_t [B, s, T]     dt    K_lin transposed per sequence
 *   S       [B, G, e, s]  dt    S_g transposed (element (b,g,c,k) = S_g[k][c])
 *   P       [B, G', e, s] dt    P_g transposed; G' = G if causal, else 1
 *   A       [B*G, C, C]   dt    per-chunk attention weights
 *                               relu^2(quad_scale Q_quad K_quad^T + Bias), masked,
 *                               query-major; causal: key blocks above the diagonal
 *                               (128 wide, 64 when C = 64) are not written
 *   Y       [B*T, e]      dt    U * (V_quad + V_lin)
 *   total   bytes needed (== gau_workspace_bytes)
 * Two regions are reused in place, so that the layer's intermediates fit the
 * last-level cache at the benchmark sizes: Y == U (the attention stage
 * overwrites each element of U with the gated output at the same index), and
 * when causal P == S (the scan overwrites S_g with P_g).  After a whole
 * forward those regions hold Y and P; U and S can be read after a
 * gau_forward_stages range that ends before the attention stage (U) or
 * before the scan (S).
 */
typedef struct {
    size_t U, Vt, Q_quad, K_quad, Q_lin, K_lin_t, S, P, A, Y, total;
} gau_ws_layout;

/* Workspace bytes gau_forward needs for cfg (0 if cfg is invalid). */
size_t gau_workspace_bytes(const gau_config* cfg);

/* Fills *out with the workspace layout for cfg.  GAU_ERR_NULL / _SHAPE /
 * _DTYPE as gau_forward. */
gau_status gau_workspace_layout(const gau_config* cfg, gau_ws_layout* out);

/*
 * One FLASH layer forward: O = GAU(X).
 *   X       [B, T, d]   dt   input activations
 *   W_u     [e, d]      dt   W_u transposed (output-major, see above)
 *   W_v     [e, d]      dt
 *   W_z     [s, d]      dt
 *   W_o     [d, e]      dt   W_o transposed
 *   scale   [4, s]      fp32 gamma of Q_quad, K_quad, Q_lin, K_lin (in order)
 *   offset  [4, s]      fp32 beta, same order
 *   relpos  [2C-1]      fp32 relative-position vector, Bias[i][j] = relpos[C-1+j-i]
 *   O       [B, T, d]   dt   output
 *   workspace, workspace_bytes: device scratch of at least gau_workspace_bytes
 *   stream  hipStream_t (may be NULL)
 */
gau_status gau_forward(const gau_config* cfg,
                       const void* X, const void* W_u, const void* W_v,
                       const void* W_z, const void* W_o,
                       const float* scale, const float* offset, const float* relpos,
                       void* O, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The layer over packed sequences: gau_forward with a segment mask on the
 * linear (cross-chunk) term.  The listing's Code 7 builds a chunk-level mask
 * and divides each row by its sum (divide_no_nan), and Code 8 applies it to
 * the chunk summaries, so the linear term becomes an average over the visible
 * chunks; the local (in-chunk) part has no segment mask (wikillm, "Paper vs
 * code" and "Pitfalls", segment masks).  Here:
 *   chunk_segments [B, G] int32 device array, one id per chunk (documents
 *     packed along a sequence start on chunk boundaries).  A segment is a run
 *     of consecutive chunks with equal ids (an id that comes back after
 *     another starts a new segment).  Chunk h is visible from chunk g when
 *     both lie in one segment and, causal, h < g (non-causal: every chunk of
 *     the segment, g included).
 *   V_lin_g = Q_lin_g P_g with P_g = (1/n_g) sum of the visible S_h (n_g of
 *     them; P_g = 0 when n_g = 0, e.g. the first chunk of a causal segment).
 * Everything else (arguments, checks, status codes, the workspace size) as
 * gau_forward; chunk_segments must be non-NULL and 16-byte aligned.  In the
 * workspace, the P region is S's (the states are averaged in place, one per
 * chunk, also when non-causal).
 */
gau_status gau_forward_segmented(const gau_config* cfg, const int32_t* chunk_segments,
                                 const void* X, const void* W_u, const void* W_v,
                                 const void* W_z, const void* W_o,
                                 const float* scale, const float* offset, const float* relpos,
                                 void* O, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gau_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace lives in a device array of the
 * library of GAU_NOALLOC_SCRATCH_BYTES bytes (64 MiB; every device the library
 * runs on holds one until the process ends); the call itself allocates
 * nothing.  Arguments, outputs and results as gau_forward (the same kernels in
 * the same order: O is bitwise equal to gau_forward's).
 *   GAU_ERR_WORKSPACE if gau_workspace_bytes(cfg) > GAU_NOALLOC_SCRATCH_BYTES
 *   (at d = 768, e = 1536, s = 128, C = 256, bf16: B*T up to 7168 tokens),
 *   nothing queued.  GAU_ERR_HIP if the array's device address cannot be
 *   looked up (done once per device, on the first call with it current).
 * All calls on one device share its array, which keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap on one
 * device (other streams, other host threads) race and give undefined results;
 * calls queued in order on one stream do not.
 */
#define GAU_NOALLOC_SCRATCH_BYTES (64u << 20)

gau_status gau_forward_noalloc(const gau_config* cfg,
                               const void* X, const void* W_u, const void* W_v,
                               const void* W_z, const void* W_o,
                               const float* scale, const float* offset, const float* relpos,
                               void* O, void* stream);

/*
 * The six kernels gau_forward queues, in order.  gau_forward_stages runs a
 * contiguous range of them (for stage-wise tests and per-kernel timing); the
 * stages communicate only through the workspace.
 *   GAU_STAGE_PROJ   U = SiLU(X W_u), Vt = SiLU(X W_v)^T (Su's post "Gated Attention"),
 *                    Z = SiLU(X W_z) and its four scale+offset heads Q_quad, K_quad,
 *                    Q_lin, K_lin_t (Su's post "Weak Attention"; wikillm "Method")
 *   GAU_STAGE_SCORES A_g = relu^2(quad_scale Q_quad K_quad^T + Bias), causal-masked,
 *                    per chunk (wikillm "Method" step 1, eq. 5; papercache appendix D, Code 4)
 *   GAU_STAGE_STATE  S_g = lin_scale * K_lin_g^T V_g for every chunk (eq. 7-8)
 *   GAU_STAGE_SCAN   P_g = exclusive prefix over chunks (causal, eq. 8) or total (eq. 7)
 *   GAU_STAGE_ATTN   Y = U * (A_g V_g + Q_lin P_g) per chunk (wikillm "Method" steps 2-4)
 *   GAU_STAGE_OUT    O = Y W_o
 * With GAU_LOCAL_ONLY the state and scan stages queue nothing (P is not
 * read); with GAU_GLOBAL_ONLY the scores stage queues nothing (A is not read).
 * Arguments, checks and status codes as gau_forward (every pointer is
 * checked, also those the selected stages do not read).  A stage reads the
 * workspace regions earlier stages wrote, so a range that does not start at
 * GAU_STAGE_PROJ needs them there already.  first > last or a stage number
 * outside 0..5 gives GAU_ERR_SHAPE.
 */
enum {
    GAU_STAGE_PROJ = 0,
    GAU_STAGE_SCORES = 1,
    GAU_STAGE_STATE = 2,
    GAU_STAGE_SCAN = 3,
    GAU_STAGE_ATTN = 4,
    GAU_STAGE_OUT = 5
};

gau_status gau_forward_stages(const gau_config* cfg, int first_stage, int last_stage,
                              const void* X, const void* W_u, const void* W_v,
                              const void* W_z, const void* W_o,
                              const float* scale, const float* offset, const float* relpos,
                              void* O, void* workspace, size_t workspace_bytes, void* stream);

/*
 * A stack of n_layers FLASH layers with pre-norm and residual adds, the block
 * structure of the listings (wikillm, FLASH block pseudocode: norm, block,
 * add the shortcut):
 *   for l in 0..n_layers-1:  X <- X + gau_forward(rms_norm(X); layer l)
 * rms_norm(x) = x / sqrt(mean(x^2) + 1e-6) per token row; the norm's body
 * (Code 5) is missing from the pages, and this is ScaleNorm with its gain fixed
 * at sqrt(d).  The normalised activations are stored in cfg->dtype; the
 * residual stream stays fp32.
 *   X        [B, T, d] fp32, updated in place
 *   W_u .. relpos: host arrays of n_layers device pointers, each as for
 *            gau_forward
 *   workspace: at least gau_stack_workspace_bytes(cfg) bytes
 * Every layer uses cfg (quad_scale, lin_scale, causal, dtype).
 */
size_t gau_stack_workspace_bytes(const gau_config* cfg);

gau_status gau_stack_forward(const gau_config* cfg, int n_layers, float* X,
                             const void* const* W_u, const void* const* W_v,
                             const void* const* W_z, const void* const* W_o,
                             const float* const* scale, const float* const* offset,
                             const float* const* relpos,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gradients of the layer (training).  Given dO = dL/dO for the outputs of
 * gau_forward(cfg, X, ...), writes dL/dX and dL/d(every parameter): the
 * chain rule through the forward's steps (the equations at the top of this
 * file) taken in reverse.  The intermediates are recomputed from X inside the
 * call (nothing is kept between gau_forward and gau_backward).  The products
 * whose derivatives it takes, per chunk:
 *   dY = dO W_o^T, dW_o = Y^T dO;  dU = dY * (V_quad + V_lin), dWq = dY * U
 *   dA = dWq V^T;  dSc = dA * 2 relu(Sc) * mask  (Sc the pre-activation scores)
 *   dQ_quad = quad_scale dSc K_quad,  dK_quad = quad_scale dSc^T Q_quad,
 *   drelpos[C-1+j-i] += dSc[i][j]
 *   dQ_lin = dWq P^T,  dP = Q_lin^T dWq,
 *   dS_h = sum_{g>h} dP_g (causal) or sum_g dP_g (non-causal)
 *   dV = A^T dWq + lin_scale K_lin dS,  dK_lin = lin_scale V dS^T
 *   with rope = 1 the dh_h of the rotated heads first go back through the
 *   transposed rotation (the rotation by the opposite angle) at each token's
 *   position;
 *   dZ = sum_h gamma_h dh_h, dgamma_h = sum Z * dh_h, dbeta_h = sum dh_h
 *   d(pre-activations) = [dU | dV | dZ] * SiLU'(X W);  dX, dW_* from X W.
 *
 * cfg: as gau_forward (rope 0 or 1, any ablation: with GAU_LOCAL_ONLY the
 *   gradients of the Q_lin and K_lin heads' scale and offset are zero, with
 *   GAU_GLOBAL_ONLY those of Q_quad, K_quad and drelpos).  With rope, drelpos
 *   is the gradient with respect to the relpos vector passed in (for a bias
 *   built by gau_rope_relpos, the caller chains it to a and b).
 * X .. relpos: as gau_forward.   dO [B, T, d] cfg->dtype.
 * Outputs (fp32, written, not accumulated):
 *   dX [B, T, d];  dW_u, dW_v [e, d], dW_z [s, d], dW_o [d, e] (the layout in
 *   which the weights are passed: output-major);  dscale, doffset [4, s];
 *   drelpos [2C-1].
 * workspace: at least gau_backward_workspace_bytes(cfg) bytes of device
 *   memory.  Its start holds the forward's intermediates on return, at the
 *   offsets gau_workspace_layout gives for Vt, the heads, S and A (U is not
 *   stored: the backward forms SiLU(X W_u) from the pre-activations); Y and
 *   P are kept in regions of their own there (the backward needs Y, S and P
 *   at once), so they are not at the offsets gau_workspace_layout gives.
 * Sums over tokens run in a fixed order: the results are bitwise
 * reproducible for a given cfg and inputs.  B * T == 0: the parameter
 * gradients are set to zero (X, the weights, scale, offset, relpos, dO, dX and
 * workspace are not read and may be NULL).  Checks and
 * status codes otherwise as gau_forward; gau_backward_workspace_bytes gives 0
 * for a cfg gau_backward rejects.
 */
size_t gau_backward_workspace_bytes(const gau_config* cfg);

gau_status gau_backward(const gau_config* cfg, const void* X,
                        const void* W_u, const void* W_v, const void* W_z, const void* W_o,
                        const float* scale, const float* offset, const float* relpos, const void* dO,
                        float* dX, float* dW_u, float* dW_v, float* dW_z, float* dW_o,
                        float* dscale, float* doffset, float* drelpos,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * gau_backward for the segment-masked layer of gau_forward_segmented (packed
 * sequences; wikillm "Paper vs code" and "Pitfalls", segment masks): the same
 * arguments plus chunk_segments [B, T/C] int32 (16-byte aligned), the ids
 * gau_forward_segmented took.  The summaries reach P through the
 * row-normalised chunk mask M (P_g = sum_h M[g][h] S_h), so the reverse sum
 * becomes dS_h = sum_g M[g][h] dP_g: causal, sum over the later chunks g of
 * h's segment of dP_g / (chunks visible from g); non-causal, the segment's
 * sum of dP_g over its length.  Any rope and ablation.  Checks and status
 * codes as gau_backward (NULL chunk_segments: GAU_ERR_NULL); the workspace
 * is gau_backward_workspace_bytes(cfg).
 */
gau_status gau_backward_segmented(const gau_config* cfg, const int32_t* chunk_segments, const void* X,
                                  const void* W_u, const void* W_v, const void* W_z, const void* W_o,
                                  const float* scale, const float* offset, const float* relpos, const void* dO,
                                  float* dX, float* dW_u, float* dW_v, float* dW_z, float* dW_o,
                                  float* dscale, float* doffset, float* drelpos,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Incremental causal decoding: one new token of each of the B sequences per
 * call, with a constant-size state per sequence (the chunk-level recurrence
 * of the causal layer: wikillm, "Method" steps 2-4; Su's post, "Mixed
 * Chunking", the decoder's cumulative sum over chunks; papercache 3.1, the
 * incremental form of linear attention).  Token t at slot j = t mod C of its
 * chunk:
 *   u, v, z = SiLU(x W_u), SiLU(x W_v), SiLU(x W_z); the four heads of z
 *     (rotated by position t when cfg->rope = 1)
 *   quad = sum_{tau = 0..j} relu^2(quad_scale q_quad . k_quad_tau + relpos[C-1 + tau - j]) v_tau
 *   o_t  = [u * (quad + q_lin P)] W_o
 * over the current chunk's cached k_quad, v, k_lin rows, where P is the sum of
 * lin_scale * K_lin^T V over the chunks already completed; when j = C-1 the
 * chunk's summary is added to P.  Calling it for t = 0, 1, 2, ... gives the
 * causal gau_forward's outputs token by token.
 *
 * cfg: as gau_forward with causal = 1 (else GAU_ERR_SHAPE); cfg->T bounds the
 *   positions (0 <= t < T); B is the number of sequences decoded together.
 * workspace: at least gau_decode_workspace_bytes(cfg) bytes of device memory
 *   holding the state (P as [B, s, e] fp32, and for bf16 its copy rounded to
 *   bf16 at each chunk end, which the steps read; the chunk's K_quad and K_lin
 *   rows [B, C, s] and V rows [B, C, e] in cfg->dtype) and per-step scratch.  It
 *   must be reset (gau_decode_reset) before t = 0, and each call must follow
 *   the call for t - 1 on the same workspace (not checked: the library keeps
 *   no position).
 *   x  [B, d] dt  the tokens at position t;  o [B, d] dt  their outputs.
 *   W_u .. relpos as gau_forward.
 * Checks and status codes as gau_forward; 0 is returned for an invalid cfg by
 * gau_decode_workspace_bytes.  B == 0 is a no-op.
 */
size_t gau_decode_workspace_bytes(const gau_config* cfg);

gau_status gau_decode_reset(const gau_config* cfg, void* workspace, size_t workspace_bytes, void* stream);

gau_status gau_decode_step(const gau_config* cfg, int64_t t, const void* x,
                           const void* W_u, const void* W_v, const void* W_z, const void* W_o,
                           const float* scale, const float* offset, const float* relpos,
                           void* o, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The relative-position bias of chunk length n built from RoPE-rotated vectors
 * (the n >= 512 branch of papercache, appendix D, Code 4): the Toeplitz matrix
 * rope(a)_m . rope(b)_k depends only on k - m, so it is carried by
 *   relpos[n-1 + d] = a . rope(b, d),   d = -(n-1) .. n-1,
 * the vector gau_forward takes as `relpos` (Bias[i][j] = relpos[C-1+j-i]).
 * rope(b, d) turns the pairs (b_i, b_{i+dim/2}) by d * 10000^(-i/(dim/2)).
 *   a, b    [dim] fp32 device arrays (Code 4 uses dim = 128)
 *   relpos  [2n-1] fp32 device array, written
 * n >= 1, dim even and > 0 (else GAU_ERR_SHAPE); NULL pointers GAU_ERR_NULL;
 * pointers 16-byte aligned (GAU_ERR_ALIGN).  Queued on `stream`.
 */
gau_status gau_rope_relpos(const float* a, const float* b, int64_t n, int64_t dim, float* relpos, void* stream);

/* Static description of a status code. */
const char* gau_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GAU_H */
