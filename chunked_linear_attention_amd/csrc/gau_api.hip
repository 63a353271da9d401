// C ABI of libgau: argument checks, workspace layout and the launch sequence
// of the FLASH layer forward.  Declarations and the meaning of every argument
// are in include/gau.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gau.h"
#include "gau_launch.h"

// Scratch of gau_forward_noalloc: the forward's workspace, at most
// GAU_NOALLOC_SCRATCH_BYTES, in a device array of this library.  Each device
// the library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, not the device copy: its device
// address is taken once per device with hipGetSymbolAddress (noalloc_scratch
// below), and only that address is passed to kernels.
static __device__ __align__(256) char scratch[GAU_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t elem_bytes(int32_t dtype) { return dtype == GAU_BF16 ? 2 : 4; }

gau_status check_config(const gau_config* c) {
    if (!c) return GAU_ERR_NULL;
    if (c->dtype != GAU_F32 && c->dtype != GAU_BF16) return GAU_ERR_DTYPE;
    if (c->B < 0 || c->T < 0) return GAU_ERR_SHAPE;
    if (!(c->C == 64 || c->C == 128 || c->C == 256 || c->C == 512)) return GAU_ERR_SHAPE;
    if (c->T % c->C != 0) return GAU_ERR_SHAPE;
    if (c->d <= 0 || c->d % 128 != 0) return GAU_ERR_SHAPE;
    if (c->e <= 0 || c->e % 256 != 0) return GAU_ERR_SHAPE;
    if (!(c->s == 128 || c->s == 256)) return GAU_ERR_SHAPE;
    if (c->rope != 0 && c->rope != 1) return GAU_ERR_SHAPE;
    if (c->ablation != GAU_FULL && c->ablation != GAU_LOCAL_ONLY && c->ablation != GAU_GLOBAL_ONLY)
        return GAU_ERR_SHAPE;
    // 32-bit index arithmetic inside the kernels
    const int64_t M = c->B * c->T;
    if (M > (int64_t)1 << 30 || c->d > 65536 || c->e > 65536) return GAU_ERR_SHAPE;
    if (M * (c->e > c->d ? c->e : c->d) > ((int64_t)1 << 40)) return GAU_ERR_SHAPE;
    // the chunk scan's grid: one lane per four of the B * e * s state
    // entries, fewer than 2^31 lanes
    if (c->B * c->e * c->s >= ((int64_t)1 << 33)) return GAU_ERR_SHAPE;
    // bf16: the MFMA core copies K-major operand tiles through buffer
    // resources with 32-bit signed row offsets (up to 255 rows of the
    // operand's pitch); the token-major operands (V and K_lin transposed per
    // sequence) have a pitch of T elements, so 255 * 2 T bytes must stay
    // below 2^31
    if (c->dtype == GAU_BF16 && c->T > ((int64_t)1 << 22)) return GAU_ERR_SHAPE;
    return GAU_OK;
}

// Workspace regions.  With `shared` (the forward's layout) two regions are
// reused in place, which keeps the layer's working set small enough to stay
// in the 256 MB last-level cache at the benchmark size: Y overwrites U (each
// element of Y = U * (...) is written by the block that read that element of U
// as its gate), and in the causal case P overwrites S (each lane of the scan
// reads an entry of S_g before it writes the same entry of P_g).  The
// backward keeps every region separate (shared = false): it needs U, Y, S and
// P together.
void layout(const gau_config* c, gau_ws_layout* L, bool shared = true) {
    const size_t eb = elem_bytes(c->dtype);
    const size_t M = (size_t)(c->B * c->T);
    const size_t G = c->T / c->C;
    const size_t Gp = c->causal ? G : 1;
    const size_t es = (size_t)c->e * c->s;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    L->U = take(M * c->e * eb);
    L->Vt = take(M * c->e * eb);
    L->Q_quad = take(M * c->s * eb);
    L->K_quad = take(M * c->s * eb);
    L->Q_lin = take(M * c->s * eb);
    L->K_lin_t = take(M * c->s * eb);
    L->S = take((size_t)c->B * G * es * eb);
    L->A = take(M * (size_t)c->C * eb);
    // the regions that may be shared come last, so that every other region
    // has the same offset in both layouts
    L->P = (shared && c->causal) ? L->S : take((size_t)c->B * Gp * es * eb);
    L->Y = shared ? L->U : take(M * c->e * eb);
    L->total = off;
}


struct LayerPtrs {
    const void *X, *W_u, *W_v, *W_z, *W_o;
    const float *scale, *offset, *relpos;
};

gau_status check_layer_ptrs(const LayerPtrs& a) {
    const void* ptrs[] = {a.X, a.W_u, a.W_v, a.W_z, a.W_o, a.scale, a.offset, a.relpos};
    for (const void* q : ptrs)
        if (!q) return GAU_ERR_NULL;
    for (const void* q : ptrs)
        if (!aligned16(q)) return GAU_ERR_ALIGN;
    return GAU_OK;
}

// Decoding workspace: the state (P fp32, the chunk cache in the element type)
// and the per-step fp32 scratch.
struct DecodeLayout {
    size_t P, Pr, Kq, V, Kl, u, z, y, total;
};

void decode_layout(const gau_config* c, DecodeLayout* D) {
    const size_t eb = elem_bytes(c->dtype);
    const size_t B = (size_t)c->B, C = (size_t)c->C, e = (size_t)c->e, s = (size_t)c->s;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    D->P = take(B * s * e * 4);
    D->Pr = eb == 4 ? D->P : take(B * s * e * eb);  // the copy the steps read
    D->Kq = take(B * C * s * eb);
    D->V = take(B * C * e * eb);
    D->Kl = take(B * C * s * eb);
    D->u = take(B * e * 4);
    D->z = take(B * s * 4);
    D->y = take(B * e * eb);
    D->total = off;
}

gau::StateParams state_params(const gau_config* c, const gau_ws_layout& L, char* ws) {
    return gau::StateParams{ws + L.Vt, ws + L.K_lin_t, ws + L.S, (int)c->B, (int)c->T,
                            (int)c->e, (int)c->s, (int)c->C, c->lin_scale};
}

// Stages first..last of one layer.  `residual` != nullptr makes the output
// stage write O = residual + Y W_o in fp32.  `seg` != nullptr ([B, G] chunk
// segment ids): the scan forms one averaged state per chunk, in place over S
// (also when non-causal), and the attention stage reads it per chunk.
gau_status run_stages(const gau_config* c, int first, int last, const LayerPtrs& a, void* O, const float* residual,
                      char* ws, hipStream_t st, bool shared = true, const int32_t* seg = nullptr,
                      void* preact = nullptr) {
    gau_ws_layout L;
    layout(c, &L, shared);
    if (seg) L.P = L.S;
    const bool bf = c->dtype == GAU_BF16;
    const int M = (int)(c->B * c->T);
    const int G = (int)(c->T / c->C);
    const bool local = c->ablation != GAU_GLOBAL_ONLY, global = c->ablation != GAU_LOCAL_ONLY;
    for (int stage = first; stage <= last; ++stage) {
        hipError_t e = hipSuccess;
        switch (stage) {
            case GAU_STAGE_PROJ: {
                gau::ProjParams p{a.X, a.W_u, a.W_v, a.W_z, a.scale, a.offset, ws + L.U, ws + L.Vt,
                                  ws + L.Q_quad, ws + L.K_quad, ws + L.Q_lin, ws + L.K_lin_t,
                                  M, (int)c->T, (int)c->d, (int)c->e, (int)c->s, c->rope, preact};
                e = gau::launch_proj(p, bf, st);
                break;
            }
            case GAU_STAGE_STATE: {
                if (global) e = gau::launch_chunk_state(state_params(c, L, ws), bf, st);
                break;
            }
            case GAU_STAGE_SCAN: {
                if (!global) break;
                gau::ScanParams p{ws + L.S, ws + L.P, (int)c->B, G, (int)(c->e * c->s),
                                  c->causal ? 1 : 0, seg};
                e = gau::launch_chunk_scan(p, bf, st);
                break;
            }
            case GAU_STAGE_SCORES: {
                const gau::ScoresParams p{ws + L.Q_quad, ws + L.K_quad, a.relpos, ws + L.A, (int)c->B, (int)c->T,
                                          (int)c->s, (int)c->C, c->causal ? 1 : 0, c->quad_scale};
                if (last >= GAU_STAGE_STATE && local && global) {  // one launch, the state stage done with it
                    e = gau::launch_chunk_scores_state(p, state_params(c, L, ws), bf, st);
                    ++stage;
                } else if (local) {
                    e = gau::launch_chunk_scores(p, bf, st);
                }
                break;
            }
            case GAU_STAGE_ATTN: {
                gau::AttnParams p{ws + L.A, ws + L.Q_lin, ws + L.Vt, ws + L.P, ws + L.U, ws + L.Y, (int)c->B,
                                  (int)c->T, (int)c->e, (int)c->s, (int)c->C, c->causal ? 1 : 0,
                                  local ? 1 : 0, global ? 1 : 0, seg ? 1 : 0};
                e = gau::launch_chunk_attn(p, bf, st);
                break;
            }
            case GAU_STAGE_OUT: {
                gau::OutParams p{ws + L.Y, a.W_o, O, residual, M, (int)c->d, (int)c->e, 0, 0,
                                 nullptr, nullptr, nullptr, nullptr, 0};
                e = gau::launch_out_gemm(p, bf, st);
                break;
            }
            default:
                return GAU_ERR_SHAPE;
        }
        if (e != hipSuccess) return GAU_ERR_HIP;
    }
    return GAU_OK;
}

// Backward workspace: the forward's regions, then the backward's own.
struct BwdLayout {
    size_t H, dWq, Yb, WoT, dA, dScE;
    size_t dQq, dKq, dQl, dKl, dP, dSst, Kl, rpart, hpart, dH, Wt, wpart, total;
    int split_o, split_w;  // K splits of the weight-gradient products
};

// K splits of a weight-gradient product (K = M tokens, 64 per chunk) on the
// output GEMM's 256 x 256 tiles: as many as fill one round of the 256 CUs,
// at most one per chunk.
int weight_splits(int64_t M, int tiles) {
    int S = tiles >= 256 ? 1 : 256 / tiles;
    const int64_t chunks = M / 64;
    if (S > chunks) S = (int)(chunks > 0 ? chunks : 1);
    return S;
}

void bwd_layout(const gau_config* c, BwdLayout* L) {
    gau_ws_layout F;
    layout(c, &F, false);
    const size_t eb = elem_bytes(c->dtype);
    const size_t M = (size_t)(c->B * c->T), d = c->d, e = c->e, s = c->s, C = c->C;
    const size_t G = c->T / c->C, Z = (size_t)c->B * G;
    const size_t W3 = 2 * e + s;
    // dW_o: feature tiles over e, token tiles over d; [dW_u|dW_v|dW_z]: over d and 2e + s
    L->split_o = weight_splits((int64_t)M, gau::out_gemm_tiles((int)e, (int)d, 256));
    L->split_w = weight_splits((int64_t)M, gau::out_gemm_tiles((int)d, (int)W3, 256));
    size_t off = F.total;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    L->H = take(M * W3 * eb);
    L->dWq = take(M * e * eb);
    L->Yb = take(M * e * eb);
    L->WoT = take(e * d * eb);
    L->dA = take(Z * C * C * 4);
    L->dScE = take(Z * C * C * eb);
    L->dQq = take(M * s * 4);
    L->dKq = take(M * s * 4);
    L->dQl = take(M * s * 4);
    L->dKl = take(M * s * 4);
    L->dP = take(Z * e * s * 4);
    L->dSst = take(Z * e * s * eb);
    L->Kl = take(M * s * eb);
    L->rpart = take(M / 32 * (2 * C - 1) * 4);
    L->hpart = take((M + gau::kHeadsBwdTokens - 1) / gau::kHeadsBwdTokens * 8 * s * 4);
    L->dH = take(M * W3 * eb);
    L->Wt = take(d * W3 * eb);
    const size_t po = (size_t)L->split_o * d * e, pw = (size_t)L->split_w * W3 * d;
    L->wpart = take((po > pw ? po : pw) * 4);
    L->total = off;
}

// One operand of a batched NT product (GemmNTParams): entry z (chunk z % zg
// of sequence z / zg) at (z / zg) * bsq + (z % zg) * bs elements.
struct NtOp {
    const void* p;
    int64_t bs, bsq;
    int rp;
    int mn_major;
};
// K-major, rows rp elements apart, entries bs elements apart throughout
NtOp kmaj(const void* p, int64_t bs, int rp, int zg) { return NtOp{p, bs, bs * zg, rp, 0}; }
// MN-major, K rows rp elements apart, chunks bs and sequences bsq apart
NtOp mnmaj(const void* p, int64_t bs, int64_t bsq, int rp) { return NtOp{p, bs, bsq, rp, 1}; }

gau::GemmNTParams nt(const NtOp& a, const NtOp& b, void* C, int64_t c_bs, int c_rp, int K, bool c_f32, int zg,
                     float alpha = 1.f) {
    gau::GemmNTParams q{};
    q.A = a.p;
    q.B = b.p;
    q.C = C;
    q.a_bs = a.bs;
    q.a_bsq = a.bsq;
    q.a_rp = a.rp;
    q.a_t = a.mn_major;
    q.b_bs = b.bs;
    q.b_bsq = b.bsq;
    q.b_rp = b.rp;
    q.b_t = b.mn_major;
    q.c_bs = c_bs;
    q.c_rp = c_rp;
    q.zg = zg;
    q.K = K;
    q.c_f32 = c_f32 ? 1 : 0;
    q.alpha = alpha;
    q.epi = gau::EPI_STORE;
    return q;
}

gau::TransposeParams tp(const void* in, int64_t in_bs, int in_rp, void* out, int64_t out_bs, int out_rp) {
    return gau::TransposeParams{in, out, in_bs, out_bs, in_rp, out_rp, 0, 0};
}

// The backward pass: recompute the forward's intermediates, then the chain
// rule through its steps in reverse (the launch order below).
gau_status run_backward(const gau_config* c, const LayerPtrs& a, const void* dO, float* dX, float* dW_u,
                        float* dW_v, float* dW_z, float* dW_o, float* dscale, float* doffset, float* drelpos,
                        char* ws, hipStream_t st, const int32_t* seg = nullptr) {
    gau_ws_layout F;
    layout(c, &F, false);
    BwdLayout L;
    bwd_layout(c, &L);
    const bool bf = c->dtype == GAU_BF16;
    const size_t eb = elem_bytes(c->dtype);
    const int M = (int)(c->B * c->T), d = (int)c->d, e = (int)c->e, s = (int)c->s, C = (int)c->C;
    const int T = (int)c->T, Bn = (int)c->B, G = T / C, Z = Bn * G, W3 = 2 * e + s;
    const int64_t CC = (int64_t)C * C, Ce = (int64_t)C * e, Cs = (int64_t)C * s, es = (int64_t)e * s;
    auto W = [&](size_t off) { return (void*)(ws + off); };
    auto Wc = [&](size_t off, size_t elems) { return (void*)(ws + off + elems * eb); };
    hipError_t err = hipSuccess;  // the first failed launch
    auto ok = [&](hipError_t x) {
        if (err == hipSuccess) err = x;
    };
    auto gemm = [&](const gau::GemmNTParams& q, int m, int n, int nb) { ok(gau::launch_gemm_nt(q, m, n, nb, bf, st)); };
    // independent transposes queued together and run as one launch
    struct Batch {
        gau::TransposeParams q[gau::kTransposeBatch];
        int r[gau::kTransposeBatch], cc[gau::kTransposeBatch], nb[gau::kTransposeBatch];
        int n = 0;
    } batch;
    auto add = [&](const gau::TransposeParams& q, int r, int cc, int nb) {
        batch.q[batch.n] = q;
        batch.r[batch.n] = r;
        batch.cc[batch.n] = cc;
        batch.nb[batch.n] = nb;
        ++batch.n;
    };
    auto flush = [&]() {
        if (batch.n) ok(gau::launch_transpose_batch(batch.q, batch.r, batch.cc, batch.nb, batch.n, bf, st));
        batch.n = 0;
    };

    // which terms reach Y (the LocalOnly / GlobalOnly layers keep one)
    const bool local = c->ablation != GAU_GLOBAL_ONLY, global = c->ablation != GAU_LOCAL_ONLY;
    // forward intermediates: heads, states, prefix, weights (the causal
    // weight tiles above the diagonal stay unwritten: the attention and dV
    // products never read them, and the scores' derivative selects zero
    // there without using what it loaded)
    // (the projection also stores the pre-activations H = X [W_u | W_v | W_z],
    // which the SiLU derivatives below read)
    // (with segments the scan leaves one averaged state per chunk in place
    // of S)
    gau_status sres = run_stages(c, GAU_STAGE_PROJ, GAU_STAGE_SCAN, a, nullptr, nullptr, ws, st, false, seg,
                                 W(L.H));
    const size_t Poff = seg ? F.S : F.P;
    if (sres != GAU_OK) return sres;
    // Wq = A V + Q_lin P, or the kept term (into the forward's Y region): the
    // attention stage without the gate
    {
        gau::AttnParams p{W(F.A), W(F.Q_lin), W(F.Vt), W(Poff), nullptr, W(F.Y), Bn, T, e, s, C,
                          c->causal ? 1 : 0, local ? 1 : 0, global ? 1 : 0, seg ? 1 : 0};
        ok(gau::launch_chunk_attn(p, bf, st));
    }
    // the transposes left, in one launch: W_o^T (dY), the weights (dX) and
    // token-major K_lin (dV); every other product reads its operands where
    // they lie, K-major or MN-major
    add(tp(a.W_o, 0, e, W(L.WoT), 0, d), d, e, 1);
    add(tp(W(F.K_lin_t), (int64_t)s * T, T, W(L.Kl), (int64_t)T * s, s), s, T, Bn);
    add(tp(a.W_u, 0, d, W(L.Wt), 0, W3), e, d, 1);
    add(tp(a.W_v, 0, d, Wc(L.Wt, e), 0, W3), e, d, 1);
    add(tp(a.W_z, 0, d, Wc(L.Wt, 2 * e), 0, W3), s, d, 1);
    flush();
    // O = Y W_o and the gate Y = U * Wq: dY = dO W_o^T, fused with
    // dWq = dY * U, Y, and dH_u = dY * Wq * SiLU'(H_u)
    // (on the output GEMM's tiles: rows of dO times rows of W_o, K = d, with
    // the gate epilogue)
    ok(gau::launch_out_gemm(gau::OutParams{dO, W(L.WoT), W(L.dH), nullptr, M, e, d, 0, W3, W(L.H), W(F.Y),
                                           W(L.dWq), W(L.Yb), e},
                            bf, st));

    // operands per chunk z (chunk z % G of sequence z / G): dWq, the heads
    // and A token-major ([C, e], [C, s], [C, C]); V from Vt and P, dS as
    // [e, s] (feature-major)
    const NtOp dWq_k = kmaj(W(L.dWq), Ce, e, G);                       // rows q, K = f
    const NtOp dWq_m = mnmaj(W(L.dWq), Ce, (int64_t)G * Ce, e);        // K = q, MN = f
    const NtOp V_m = mnmaj(W(F.Vt), C, (int64_t)e * T, T);             // K = f, MN = keys
    const NtOp dS_m = mnmaj(W(L.dSst), es, (int64_t)G * es, s);        // K = f, MN = j
    auto heads_m = [&](size_t off) { return mnmaj(W(off), Cs, (int64_t)G * Cs, s); };  // K = tokens, MN = j

    // a term the layer drops: its head gradients (and the bias's) are zero
    auto zero = [&](float* x, size_t n) { ok(gau::launch_fill_zero(x, n, st)); };
    if (!local) {
        zero((float*)W(L.dQq), (size_t)M * s);
        zero((float*)W(L.dKq), (size_t)M * s);
        zero(drelpos, (size_t)(2 * C - 1));
    }
    if (!global) {
        zero((float*)W(L.dQl), (size_t)M * s);
        zero((float*)W(L.dKl), (size_t)M * s);
    }

    // local part: dA = dWq V^T, dSc = dA * 2 relu(Sc) * mask,
    // dQ_quad = qs dSc K_quad, dK_quad = qs dSc^T Q_quad, dBias
    if (local) {
        {
            gau::GemmNTParams q = nt(dWq_k, V_m, W(L.dA), CC, C, e, true, G);
            q.skip_upper = c->causal ? 1 : 0;
            q.bt = C % 128 == 0 ? 128 : 64;  // K = e is long: the larger tile's operand reuse pays
            gemm(q, C, C, Z);
        }
        {
            gau::BwdElemParams p{(const float*)W(L.dA), W(F.A), W(L.dScE), (size_t)Z * CC, C, c->causal ? 1 : 0};
            ok(gau::launch_scores_bwd(p, (float*)W(L.rpart), drelpos, bf, st));
        }
        gemm(nt(kmaj(W(L.dScE), CC, C, G), heads_m(F.K_quad), W(L.dQq), Cs, s, C, true, G, c->quad_scale), C, s, Z);
        gemm(nt(mnmaj(W(L.dScE), CC, (int64_t)G * CC, C), heads_m(F.Q_quad), W(L.dKq), Cs, s, C, true, G,
                c->quad_scale),
             C, s, Z);
    }

    // global part: dQ_lin = dWq P^T, dP = Q_lin^T dWq (per chunk, stored [e, s]),
    // dS = ls * (reverse exclusive sum of dP, or the total when non-causal),
    // dK_lin = V dS^T
    if (global) {
        {
            const NtOp P_m = (c->causal || seg) ? mnmaj(W(Poff), es, (int64_t)G * es, s) : mnmaj(W(Poff), 0, es, s);
            gemm(nt(dWq_k, P_m, W(L.dQl), Cs, s, e, true, G), C, s, Z);
        }
        gemm(nt(dWq_m, heads_m(F.Q_lin), W(L.dP), es, s, C, true, G), e, s, Z);
        {
            gau::BwdScanParams p{(const float*)W(L.dP), W(L.dSst), Bn, G, (int)es, c->causal ? 1 : 0,
                                 c->lin_scale, seg};
            ok(gau::launch_scan_bwd(p, bf, st));
        }
        gemm(nt(V_m, dS_m, W(L.dKl), Cs, s, e, true, G), C, s, Z);
    }

    // dV = A^T dWq + K_lin dS (two K segments; one when the layer keeps one
    // term), stored as dH_v = dV * SiLU'(H_v)
    {
        const NtOp Kl_k = kmaj(W(L.Kl), Cs, s, G), dS_k = kmaj(W(L.dSst), es, s, G);
        gau::GemmNTParams q = local ? nt(mnmaj(W(F.A), CC, (int64_t)G * CC, C), dWq_m, Wc(L.dH, e), (int64_t)C * W3,
                                         W3, C, false, G)
                                    : nt(Kl_k, dS_k, Wc(L.dH, e), (int64_t)C * W3, W3, s, false, G);
        if (local && global) {
            q.A2 = Kl_k.p;
            q.a2_bs = Kl_k.bs;
            q.a2_bsq = Kl_k.bsq;
            q.a2_rp = Kl_k.rp;
            q.B2 = dS_k.p;
            q.b2_bs = dS_k.bs;
            q.b2_bsq = dS_k.bsq;
            q.b2_rp = dS_k.rp;
            q.K2 = s;
        }
        q.k_from_row = local && c->causal ? 1 : 0;  // A[q][k] = 0 for queries q < k
        q.epi = gau::EPI_SILU;
        q.H = Wc(L.H, e);
        gemm(q, C, e, Z);
    }
    // heads h_k = Z gamma_k + beta_k: dZ (stored as dH_z), dgamma, dbeta
    {
        gau::BwdHeadsParams p{{(const float*)W(L.dQq), (const float*)W(L.dKq), (const float*)W(L.dQl),
                               (const float*)W(L.dKl)},
                              Wc(L.H, 2 * e), W3, a.scale, Wc(L.dH, 2 * e), (float*)W(L.hpart), M, s,
                              c->rope ? 1 : 0, T};
        ok(gau::launch_heads_bwd(p, dscale, doffset, bf, st));
    }
    // X W: dX = dH W^T
    // (the output GEMM's form: rows of dH times rows of W^T, K = 2e + s)
    ok(gau::launch_out_gemm(gau::OutParams{W(L.dH), W(L.Wt), dX, nullptr, M, d, W3, 1, 0, nullptr, nullptr,
                                           nullptr, nullptr, 0},
                            bf, st));

    // weight gradients, K = M split L.split_* ways into fp32 partials added in
    // split order: dW_o (stored [d, e]) = dO^T Y, [dW_u | dW_v | dW_z] = dH^T X,
    // on the output GEMM's 256 x 256 tiles with MN-major operands (the
    // token-major tensors as they lie: K = tokens)
    float* wp = (float*)W(L.wpart);
    // (Y's e features as the feature side, dO's d as the token side: the
    // product is [d, e])
    {
        const int S = L.split_o;
        gau::OutParams q{dO, W(L.Yb), wp, nullptr, d, e, M, 1, e, nullptr, nullptr, nullptr, nullptr,
                         0, S, (int64_t)d * e, d, 256, 1, e};
        ok(gau::launch_out_gemm(q, bf, st));
        const float* parts[1] = {wp};
        float* outs[1] = {dW_o};
        const int64_t ns[1] = {(int64_t)d * e};
        ok(gau::launch_split_reduce(parts, outs, ns, 1, (int64_t)d * e, S, st));
    }
    // (X's d features as the feature side, dH's 2e + s as the token side: the
    // product is [2e + s, d])
    {
        const int S = L.split_w;
        const int64_t stride = (int64_t)W3 * d;
        gau::OutParams q{W(L.dH), a.X, wp, nullptr, W3, d, M, 1, d, nullptr, nullptr, nullptr, nullptr,
                         0, S, stride, W3, 256, 1, d};
        ok(gau::launch_out_gemm(q, bf, st));
        const float* parts[3] = {wp, wp + (size_t)e * d, wp + (size_t)2 * e * d};
        float* outs[3] = {dW_u, dW_v, dW_z};
        const int64_t ns[3] = {(int64_t)e * d, (int64_t)e * d, (int64_t)s * d};
        ok(gau::launch_split_reduce(parts, outs, ns, 3, stride, S, st));
    }
    return err == hipSuccess ? GAU_OK : GAU_ERR_HIP;
}

}  // namespace

extern "C" {

size_t gau_workspace_bytes(const gau_config* cfg) {
    if (check_config(cfg) != GAU_OK) return 0;
    gau_ws_layout L;
    layout(cfg, &L);
    return L.total;
}

gau_status gau_workspace_layout(const gau_config* cfg, gau_ws_layout* out) {
    if (!out) return GAU_ERR_NULL;
    const gau_status s = check_config(cfg);
    if (s != GAU_OK) return s;
    layout(cfg, out);
    return GAU_OK;
}

gau_status gau_forward_stages(const gau_config* cfg, int first_stage, int last_stage, const void* X,
                              const void* W_u, const void* W_v, const void* W_z, const void* W_o,
                              const float* scale, const float* offset, const float* relpos, void* O,
                              void* workspace, size_t workspace_bytes, void* stream) {
    gau_status s = check_config(cfg);
    if (s != GAU_OK) return s;
    if (first_stage < GAU_STAGE_PROJ || last_stage > GAU_STAGE_OUT || first_stage > last_stage) return GAU_ERR_SHAPE;
    if (cfg->B * cfg->T == 0) return GAU_OK;
    const LayerPtrs a{X, W_u, W_v, W_z, W_o, scale, offset, relpos};
    if ((s = check_layer_ptrs(a)) != GAU_OK) return s;
    if (!O || !workspace) return GAU_ERR_NULL;
    if (!aligned16(O) || !aligned16(workspace)) return GAU_ERR_ALIGN;
    if (workspace_bytes < gau_workspace_bytes(cfg)) return GAU_ERR_WORKSPACE;
    return run_stages(cfg, first_stage, last_stage, a, O, nullptr, (char*)workspace, (hipStream_t)stream);
}

gau_status gau_forward(const gau_config* cfg, const void* X, const void* W_u, const void* W_v, const void* W_z,
                       const void* W_o, const float* scale, const float* offset, const float* relpos, void* O,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return gau_forward_stages(cfg, GAU_STAGE_PROJ, GAU_STAGE_OUT, X, W_u, W_v, W_z, W_o, scale, offset, relpos, O,
                              workspace, workspace_bytes, stream);
}

gau_status gau_forward_segmented(const gau_config* cfg, const int32_t* chunk_segments, const void* X,
                                 const void* W_u, const void* W_v, const void* W_z, const void* W_o,
                                 const float* scale, const float* offset, const float* relpos, void* O,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    gau_status s = check_config(cfg);
    if (s != GAU_OK) return s;
    if (cfg->B * cfg->T == 0) return GAU_OK;
    const LayerPtrs a{X, W_u, W_v, W_z, W_o, scale, offset, relpos};
    if ((s = check_layer_ptrs(a)) != GAU_OK) return s;
    if (!chunk_segments || !O || !workspace) return GAU_ERR_NULL;
    if (!aligned16(chunk_segments) || !aligned16(O) || !aligned16(workspace)) return GAU_ERR_ALIGN;
    if (workspace_bytes < gau_workspace_bytes(cfg)) return GAU_ERR_WORKSPACE;
    return run_stages(cfg, GAU_STAGE_PROJ, GAU_STAGE_OUT, a, O, nullptr, (char*)workspace, (hipStream_t)stream,
                      true, chunk_segments);
}

size_t gau_stack_workspace_bytes(const gau_config* cfg) {
    if (check_config(cfg) != GAU_OK) return 0;
    gau_ws_layout L;
    layout(cfg, &L);
    return L.total + align_up((size_t)(cfg->B * cfg->T) * cfg->d * elem_bytes(cfg->dtype));
}

gau_status gau_stack_forward(const gau_config* cfg, int n_layers, float* X, const void* const* W_u,
                             const void* const* W_v, const void* const* W_z, const void* const* W_o,
                             const float* const* scale, const float* const* offset, const float* const* relpos,
                             void* workspace, size_t workspace_bytes, void* stream) {
    gau_status s = check_config(cfg);
    if (s != GAU_OK) return s;
    if (n_layers < 0) return GAU_ERR_SHAPE;
    if (cfg->B * cfg->T == 0 || n_layers == 0) return GAU_OK;
    if (!X || !workspace || !W_u || !W_v || !W_z || !W_o || !scale || !offset || !relpos) return GAU_ERR_NULL;
    if (!aligned16(X) || !aligned16(workspace)) return GAU_ERR_ALIGN;
    if (workspace_bytes < gau_stack_workspace_bytes(cfg)) return GAU_ERR_WORKSPACE;
    char* ws = (char*)workspace;
    gau_ws_layout L;
    layout(cfg, &L);
    void* xn = ws + L.total;
    for (int l = 0; l < n_layers; ++l) {
        const LayerPtrs a{xn, W_u[l], W_v[l], W_z[l], W_o[l], scale[l], offset[l], relpos[l]};
        if ((s = check_layer_ptrs(a)) != GAU_OK) return s;
    }
    hipStream_t st = (hipStream_t)stream;
    const bool bf = cfg->dtype == GAU_BF16;
    for (int l = 0; l < n_layers; ++l) {
        gau::NormParams np{X, xn, (int)(cfg->B * cfg->T), (int)cfg->d, 1e-6f};
        if (gau::launch_rms_norm(np, bf, st) != hipSuccess) return GAU_ERR_HIP;
        const LayerPtrs a{xn, W_u[l], W_v[l], W_z[l], W_o[l], scale[l], offset[l], relpos[l]};
        if ((s = run_stages(cfg, GAU_STAGE_PROJ, GAU_STAGE_OUT, a, X, X, ws, st)) != GAU_OK) return s;
    }
    return GAU_OK;
}

// What gau_backward takes beyond check_config: at most 2^38 pre-activation
// entries (one-dimensional grids of 256-thread blocks).
static gau_status check_backward(const gau_config* c) {
    gau_status s = check_config(c);
    if (s != GAU_OK) return s;
    if (c->B * c->T * (2 * c->e + c->s) > ((int64_t)1 << 38)) return GAU_ERR_SHAPE;
    return GAU_OK;
}

size_t gau_backward_workspace_bytes(const gau_config* cfg) {
    if (check_backward(cfg) != GAU_OK) return 0;
    BwdLayout L;
    bwd_layout(cfg, &L);
    return L.total;
}

}  // extern "C"

namespace {

gau_status backward_entry(const gau_config* cfg, const int32_t* seg, bool segmented, const void* X,
                          const void* W_u, const void* W_v, const void* W_z, const void* W_o, const float* scale,
                          const float* offset, const float* relpos, const void* dO, float* dX, float* dW_u,
                          float* dW_v, float* dW_z, float* dW_o, float* dscale, float* doffset, float* drelpos,
                          void* workspace, size_t workspace_bytes, void* stream) {
    gau_status s = check_backward(cfg);
    if (s != GAU_OK) return s;
    float* outs[] = {dW_u, dW_v, dW_z, dW_o, dscale, doffset, drelpos};
    for (float* q : outs)
        if (!q) return GAU_ERR_NULL;
    for (float* q : outs)
        if (!aligned16(q)) return GAU_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    if (cfg->B * cfg->T == 0) {  // no tokens: every parameter gradient is zero
        const size_t n[] = {(size_t)(cfg->e * cfg->d), (size_t)(cfg->e * cfg->d), (size_t)(cfg->s * cfg->d),
                            (size_t)(cfg->d * cfg->e), (size_t)(4 * cfg->s), (size_t)(4 * cfg->s),
                            (size_t)(2 * cfg->C - 1)};
        for (int i = 0; i < 7; ++i)
            if (gau::launch_fill_zero(outs[i], n[i], st) != hipSuccess) return GAU_ERR_HIP;
        return GAU_OK;
    }
    const LayerPtrs a{X, W_u, W_v, W_z, W_o, scale, offset, relpos};
    if ((s = check_layer_ptrs(a)) != GAU_OK) return s;
    if (!dO || !dX || !workspace || (segmented && !seg)) return GAU_ERR_NULL;
    if (!aligned16(dO) || !aligned16(dX) || !aligned16(workspace) || (segmented && !aligned16(seg)))
        return GAU_ERR_ALIGN;
    if (workspace_bytes < gau_backward_workspace_bytes(cfg)) return GAU_ERR_WORKSPACE;
    return run_backward(cfg, a, dO, dX, dW_u, dW_v, dW_z, dW_o, dscale, doffset, drelpos, (char*)workspace, st,
                        segmented ? seg : nullptr);
}

}  // namespace

extern "C" {

gau_status gau_backward(const gau_config* cfg, const void* X, const void* W_u, const void* W_v, const void* W_z,
                        const void* W_o, const float* scale, const float* offset, const float* relpos,
                        const void* dO, float* dX, float* dW_u, float* dW_v, float* dW_z, float* dW_o,
                        float* dscale, float* doffset, float* drelpos, void* workspace, size_t workspace_bytes,
                        void* stream) {
    return backward_entry(cfg, nullptr, false, X, W_u, W_v, W_z, W_o, scale, offset, relpos, dO, dX, dW_u, dW_v,
                          dW_z, dW_o, dscale, doffset, drelpos, workspace, workspace_bytes, stream);
}

gau_status gau_backward_segmented(const gau_config* cfg, const int32_t* chunk_segments, const void* X,
                                  const void* W_u, const void* W_v, const void* W_z, const void* W_o,
                                  const float* scale, const float* offset, const float* relpos, const void* dO,
                                  float* dX, float* dW_u, float* dW_v, float* dW_z, float* dW_o, float* dscale,
                                  float* doffset, float* drelpos, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    return backward_entry(cfg, chunk_segments, true, X, W_u, W_v, W_z, W_o, scale, offset, relpos, dO, dX, dW_u,
                          dW_v, dW_z, dW_o, dscale, doffset, drelpos, workspace, workspace_bytes, stream);
}

size_t gau_decode_workspace_bytes(const gau_config* cfg) {
    if (check_config(cfg) != GAU_OK || !cfg->causal) return 0;
    DecodeLayout D;
    decode_layout(cfg, &D);
    return D.total;
}

gau_status gau_decode_reset(const gau_config* cfg, void* workspace, size_t workspace_bytes, void* stream) {
    gau_status s = check_config(cfg);
    if (s != GAU_OK) return s;
    if (!cfg->causal) return GAU_ERR_SHAPE;
    if (cfg->B == 0) return GAU_OK;
    if (!workspace) return GAU_ERR_NULL;
    if (!aligned16(workspace)) return GAU_ERR_ALIGN;
    DecodeLayout D;
    decode_layout(cfg, &D);
    if (workspace_bytes < D.total) return GAU_ERR_WORKSPACE;
    const size_t n = (size_t)cfg->B * cfg->s * cfg->e;
    if (gau::launch_fill_zero((float*)((char*)workspace + D.P), n, (hipStream_t)stream) != hipSuccess)
        return GAU_ERR_HIP;
    if (D.Pr != D.P &&  // the element-type copy (2-byte elements: n / 2 words, s * e is even)
        gau::launch_fill_zero((float*)((char*)workspace + D.Pr), n * elem_bytes(cfg->dtype) / 4,
                              (hipStream_t)stream) != hipSuccess)
        return GAU_ERR_HIP;
    return GAU_OK;
}

gau_status gau_decode_step(const gau_config* cfg, int64_t t, const void* x, const void* W_u, const void* W_v,
                           const void* W_z, const void* W_o, const float* scale, const float* offset,
                           const float* relpos, void* o, void* workspace, size_t workspace_bytes, void* stream) {
    gau_status s = check_config(cfg);
    if (s != GAU_OK) return s;
    if (!cfg->causal || t < 0 || t >= cfg->T) return GAU_ERR_SHAPE;
    if (cfg->B == 0) return GAU_OK;
    const LayerPtrs a{x, W_u, W_v, W_z, W_o, scale, offset, relpos};
    if ((s = check_layer_ptrs(a)) != GAU_OK) return s;
    if (!o || !workspace) return GAU_ERR_NULL;
    if (!aligned16(o) || !aligned16(workspace)) return GAU_ERR_ALIGN;
    DecodeLayout D;
    decode_layout(cfg, &D);
    if (workspace_bytes < D.total) return GAU_ERR_WORKSPACE;
    char* ws = (char*)workspace;
    const gau::DecodeParams p{x, W_u, W_v, W_z, W_o, scale, offset, relpos, o,
                              (float*)(ws + D.P), ws + D.Pr, ws + D.Kq, ws + D.V, ws + D.Kl,
                              (float*)(ws + D.u), (float*)(ws + D.z), ws + D.y, (int)cfg->B, (int)cfg->d, (int)cfg->e, (int)cfg->s, (int)cfg->C,
                              (int)t, (int)(t % cfg->C), cfg->rope, cfg->quad_scale, cfg->lin_scale,
                              cfg->ablation != GAU_GLOBAL_ONLY, cfg->ablation != GAU_LOCAL_ONLY};
    if (gau::launch_decode_step(p, cfg->dtype == GAU_BF16, (hipStream_t)stream) != hipSuccess) return GAU_ERR_HIP;
    return GAU_OK;
}

gau_status gau_rope_relpos(const float* a, const float* b, int64_t n, int64_t dim, float* relpos, void* stream) {
    if (!a || !b || !relpos) return GAU_ERR_NULL;
    if (n < 1 || n > (1 << 20) || dim <= 0 || dim % 2 != 0 || dim > 65536) return GAU_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(b) || !aligned16(relpos)) return GAU_ERR_ALIGN;
    if (gau::launch_rope_relpos(a, b, (int)n, (int)dim, relpos, (hipStream_t)stream) != hipSuccess)
        return GAU_ERR_HIP;
    return GAU_OK;
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up on the
// first call for that device (with it current) and kept for later calls.
gau_status noalloc_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GAU_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GAU_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GAU_OK;
}

}  // namespace

extern "C" {

gau_status gau_forward_noalloc(const gau_config* cfg, const void* X, const void* W_u, const void* W_v,
                               const void* W_z, const void* W_o, const float* scale, const float* offset,
                               const float* relpos, void* O, void* stream) {
    gau_status s = check_config(cfg);
    if (s != GAU_OK) return s;
    if (cfg->B * cfg->T == 0) return GAU_OK;
    const LayerPtrs a{X, W_u, W_v, W_z, W_o, scale, offset, relpos};
    if ((s = check_layer_ptrs(a)) != GAU_OK) return s;
    if (!O) return GAU_ERR_NULL;
    if (!aligned16(O)) return GAU_ERR_ALIGN;
    const size_t need = gau_workspace_bytes(cfg);
    if (need > (size_t)GAU_NOALLOC_SCRATCH_BYTES) return GAU_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((s = noalloc_scratch(&ws)) != GAU_OK) return s;
    // the forward writes every workspace entry it reads (nothing needs to
    // start at zero), so the previous call's contents do not matter
    return run_stages(cfg, GAU_STAGE_PROJ, GAU_STAGE_OUT, a, O, nullptr, (char*)ws, (hipStream_t)stream);
}

const char* gau_status_string(int status) {
    switch (status) {
        case GAU_OK: return "ok";
        case GAU_ERR_NULL: return "a required pointer is NULL";
        case GAU_ERR_SHAPE: return "unsupported shape or argument";
        case GAU_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case GAU_ERR_DTYPE: return "unsupported dtype";
        case GAU_ERR_WORKSPACE: return "workspace too small";
        case GAU_ERR_HIP: return "a HIP kernel launch failed";
        default: return "unknown status";
    }
}

}  // extern "C"
