// C ABI of libgau: argument checks, workspace layout and the launch sequence
// of the FLASH layer forward.  Declarations and the meaning of every argument
// are in include/gau.h.
#include <hip/hip_runtime.h>

#include "../../include/gau.h"
#include "gau_launch.h"

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
    return GAU_OK;
}

void layout(const gau_config* c, gau_ws_layout* L) {
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
    L->P = take((size_t)c->B * Gp * es * eb);
    L->A = take(M * (size_t)c->C * eb);
    L->Y = take(M * c->e * eb);
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
    size_t P, Kq, V, Kl, u, z, y, total;
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
// stage write O = residual + Y W_o in fp32.
gau_status run_stages(const gau_config* c, int first, int last, const LayerPtrs& a, void* O, const float* residual,
                      char* ws, hipStream_t st) {
    gau_ws_layout L;
    layout(c, &L);
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
                                  M, (int)c->T, (int)c->d, (int)c->e, (int)c->s};
                e = gau::launch_proj(p, bf, st);
                if (e == hipSuccess && c->rope) {
                    const gau::RopeParams r{ws + L.Q_quad, ws + L.K_quad, ws + L.Q_lin, ws + L.K_lin_t, (int)c->B,
                                            (int)c->T, M, (int)c->s};
                    e = gau::launch_rope_heads(r, bf, st);
                }
                break;
            }
            case GAU_STAGE_STATE: {
                if (global) e = gau::launch_chunk_state(state_params(c, L, ws), bf, st);
                break;
            }
            case GAU_STAGE_SCAN: {
                if (!global) break;
                gau::ScanParams p{ws + L.S, ws + L.P, (int)c->B, G, (int)(c->e * c->s),
                                  c->causal ? 1 : 0};
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
                                  local ? 1 : 0, global ? 1 : 0};
                e = gau::launch_chunk_attn(p, bf, st);
                break;
            }
            case GAU_STAGE_OUT: {
                gau::OutParams p{ws + L.Y, a.W_o, O, residual, M, (int)c->d, (int)c->e};
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
                              (float*)(ws + D.P), ws + D.Kq, ws + D.V, ws + D.Kl,
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
