// Bounds check of every kernel launch of the library on the CPU emulation:
// each operand in its own exact-size heap buffer (AddressSanitizer reports any
// access outside), for the shapes the tests and the benchmark use.
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "gau.h"
#include "gau_launch.h"

using namespace gau;

static void* buf(size_t n) {
    void* p = malloc(n ? n : 1);
    memset(p, 0, n ? n : 1);
    return p;
}

struct Cfg {
    int B, T, d, e, s, C;
    bool bf;
    bool causal;
};

static double now() {
    return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

#define CHECK(x)                                                        \
    do {                                                                \
        if ((x) != hipSuccess) {                                        \
            fprintf(stderr, "launch failed: %s\n", #x);                 \
            exit(1);                                                    \
        }                                                               \
    } while (0)

static void run(const Cfg& c, const std::string& only) {
    const size_t eb = c.bf ? 2 : 4;
    const size_t M = (size_t)c.B * c.T;
    const int G = c.T / c.C;
    const int Gp = c.causal ? G : 1;
    fprintf(stderr, "config B%d T%d d%d e%d s%d C%d %s %s\n", c.B, c.T, c.d, c.e, c.s, c.C, c.bf ? "bf16" : "f32",
            c.causal ? "causal" : "full");
    void* X = buf(M * c.d * eb);
    void* Wu = buf((size_t)c.e * c.d * eb);
    void* Wv = buf((size_t)c.e * c.d * eb);
    void* Wz = buf((size_t)c.s * c.d * eb);
    void* Wo = buf((size_t)c.d * c.e * eb);
    float* sc = (float*)buf(4 * c.s * 4);
    float* of = (float*)buf(4 * c.s * 4);
    float* rp = (float*)buf((2 * c.C - 1) * 4);
    void* U = buf(M * c.e * eb);
    void* Vt = buf(M * c.e * eb);
    void* Qq = buf(M * c.s * eb);
    void* Kq = buf(M * c.s * eb);
    void* Ql = buf(M * c.s * eb);
    void* Klt = buf(M * c.s * eb);
    void* S = buf((size_t)c.B * G * c.e * c.s * eb);
    void* P = buf((size_t)c.B * Gp * c.e * c.s * eb);
    void* A = buf(M * c.C * eb);
    void* Y = buf(M * c.e * eb);
    void* O = buf(M * c.d * eb);
    float* Of = (float*)buf(M * c.d * 4);
    auto t = [&](const char* name, auto fn) {
        if (!only.empty() && std::string(name).compare(0, only.size(), only) != 0) return;  // prefix match
        double t0 = now();
        fn();
        fprintf(stderr, "  %-12s ok (%.1f s)\n", name, now() - t0);
    };
    ProjParams pp{X, Wu, Wv, Wz, sc, of, U, Vt, Qq, Kq, Ql, Klt, (int)M, c.T, c.d, c.e, c.s, 0, nullptr};
    t("proj", [&] { CHECK(launch_proj(pp, c.bf, nullptr)); });
    ProjParams ppr = pp;
    ppr.rope = 1;  // the heads rotated in the epilogue
    t("proj_rope", [&] { CHECK(launch_proj(ppr, c.bf, nullptr)); });
    void* Hpre = buf(M * (2 * c.e + c.s) * eb);
    ProjParams pph = pp;
    pph.H = Hpre;  // the pre-activations stored too (the backward's recompute)
    t("proj_preact", [&] { CHECK(launch_proj(pph, c.bf, nullptr)); });
    free(Hpre);
    float* ra = (float*)buf(128 * 4);
    float* rb = (float*)buf(128 * 4);
    float* rw = (float*)buf((2 * c.C - 1) * 4);
    t("rope_relpos", [&] { CHECK(launch_rope_relpos(ra, rb, c.C, 128, rw, nullptr)); });
    // one decoding step at the first slot of a chunk and one at its last
    // (which also adds the chunk's summary to the state)
    void* dx = buf((size_t)c.B * c.d * eb);
    void* dO = buf((size_t)c.B * c.d * eb);
    float* dP = (float*)buf((size_t)c.B * c.s * c.e * 4);
    void* dPr = c.bf ? buf((size_t)c.B * c.s * c.e * eb) : (void*)dP;  // the copy the steps read
    void* dKq = buf((size_t)c.B * c.C * c.s * eb);
    void* dV = buf((size_t)c.B * c.C * c.e * eb);
    void* dKl = buf((size_t)c.B * c.C * c.s * eb);
    float* du = (float*)buf((size_t)c.B * c.e * 4);
    float* dz = (float*)buf((size_t)c.B * c.s * 4);
    void* dy = buf((size_t)c.B * c.e * eb);
    if (c.causal) {
        for (int pos : {0, c.C - 1}) {
            DecodeParams dp{dx, Wu, Wv, Wz, Wo, sc, of, rp, dO, dP, dPr, dKq, dV, dKl, du, dz, dy,
                            c.B, c.d, c.e, c.s, c.C, pos, pos % c.C, 1, 1.0f / c.C, 1.0f / c.C, 1, 1};
            t(pos == 0 ? "decode_step_j0" : "decode_step_jlast",
              [&] { CHECK(launch_decode_step(dp, c.bf, nullptr)); });
        }
        t("fill_zero", [&] { CHECK(launch_fill_zero(dP, (size_t)c.B * c.s * c.e, nullptr)); });
    }
    ScoresParams sp{Qq, Kq, rp, A, c.B, c.T, c.s, c.C, c.causal ? 1 : 0, 1.0f / c.C};
    t("chunk_scores", [&] { CHECK(launch_chunk_scores(sp, c.bf, nullptr)); });
    StateParams stp{Vt, Klt, S, c.B, c.T, c.e, c.s, c.C, 1.0f / c.C};
    t("chunk_state", [&] { CHECK(launch_chunk_state(stp, c.bf, nullptr)); });
    t("chunk_scores_state", [&] { CHECK(launch_chunk_scores_state(sp, stp, c.bf, nullptr)); });
    ScanParams scp{S, P, c.B, G, c.e * c.s, c.causal ? 1 : 0, nullptr};
    t("chunk_scan", [&] { CHECK(launch_chunk_scan(scp, c.bf, nullptr)); });
    // segmented: one state per chunk (in place over S), ids in an exact-size array
    int32_t* seg = (int32_t*)buf((size_t)c.B * G * 4);
    for (int i = 0; i < c.B * G; ++i) seg[i] = (i / 2) % 3;
    ScanParams scs{S, S, c.B, G, c.e * c.s, c.causal ? 1 : 0, seg};
    t("chunk_scan_segmented", [&] { CHECK(launch_chunk_scan(scs, c.bf, nullptr)); });
    AttnParams aps{A, Ql, Vt, S, U, Y, c.B, c.T, c.e, c.s, c.C, c.causal ? 1 : 0, 1, 1, 1};
    t("chunk_attn_segmented", [&] { CHECK(launch_chunk_attn(aps, c.bf, nullptr)); });
    AttnParams ap{A, Ql, Vt, P, U, Y, c.B, c.T, c.e, c.s, c.C, c.causal ? 1 : 0, 1, 1, 0};
    t("chunk_attn", [&] { CHECK(launch_chunk_attn(ap, c.bf, nullptr)); });
    AttnParams apu = ap;
    apu.U = nullptr;  // no gate (the backward's recompute of the attention output)
    t("chunk_attn_ungated", [&] { CHECK(launch_chunk_attn(apu, c.bf, nullptr)); });
    OutParams op{Y, Wo, O, nullptr, (int)M, c.d, c.e};
    t("out_gemm", [&] { CHECK(launch_out_gemm(op, c.bf, nullptr)); });
    OutParams opr{Y, Wo, Of, Of, (int)M, c.d, c.e};
    t("out_residual", [&] { CHECK(launch_out_gemm(opr, c.bf, nullptr)); });
    // the backward's dY product with its gate epilogue (K = d, e outputs per
    // token)
    t("out_gate", [&] {
        const int W3 = 2 * c.e + c.s;
        void* WoT = buf((size_t)c.e * c.d * eb);
        void* gO = buf(M * c.d * eb);
        void* dH = buf(M * W3 * eb);
        void* gH = buf(M * W3 * eb);
        void* gW = buf(M * c.e * eb);
        void* gD = buf(M * c.e * eb);
        void* gY = buf(M * c.e * eb);
        OutParams og{gO, WoT, dH, nullptr, (int)M, c.e, c.d, 0, W3, gH, gW, gD, gY, c.e};
        CHECK(launch_out_gemm(og, c.bf, nullptr));
        for (void* q : {WoT, gO, dH, gH, gW, gD, gY}) free(q);
    });
    NormParams np{Of, X, (int)M, c.d, 1e-6f};
    t("rms_norm", [&] { CHECK(launch_rms_norm(np, c.bf, nullptr)); });
    // the whole layer through the C ABI, one workspace
    t("gau_forward", [&] {
        gau_config cfg{c.B, c.T, c.d, c.e, c.s, c.C, c.causal ? 1 : 0, c.bf ? GAU_BF16 : GAU_F32, 1.0f / c.C,
                       1.0f / c.C};
        const size_t wsb = gau_workspace_bytes(&cfg);
        void* ws = buf(wsb);
        int st = gau_forward(&cfg, X, Wu, Wv, Wz, Wo, sc, of, rp, O, ws, wsb, nullptr);
        if (st != GAU_OK) {
            fprintf(stderr, "gau_forward status %d\n", st);
            exit(1);
        }
        free(ws);
    });
    t("gau_forward_segmented", [&] {
        gau_config cfg{c.B, c.T, c.d, c.e, c.s, c.C, c.causal ? 1 : 0, c.bf ? GAU_BF16 : GAU_F32, 1.0f / c.C,
                       1.0f / c.C};
        const size_t wsb = gau_workspace_bytes(&cfg);
        void* ws = buf(wsb);
        int st = gau_forward_segmented(&cfg, seg, X, Wu, Wv, Wz, Wo, sc, of, rp, O, ws, wsb, nullptr);
        if (st != GAU_OK) {
            fprintf(stderr, "gau_forward_segmented status %d\n", st);
            exit(1);
        }
        free(ws);
    });
    // the backward pass through the C ABI: exact-size inputs, outputs and
    // workspace, for the full layer, with RoPE, for each partial layer and
    // with segment ids
    for (int variant = 0; variant < 5; ++variant)
    if (M <= 4096) t(variant == 0 ? "gau_backward" : variant == 1 ? "gau_backward_rope"
                     : variant == 2 ? "gau_backward_local" : variant == 3 ? "gau_backward_global"
                     : "gau_backward_segmented", [&] {
        gau_config cfg{c.B, c.T, c.d, c.e, c.s, c.C, c.causal ? 1 : 0, c.bf ? GAU_BF16 : GAU_F32, 1.0f / c.C,
                       1.0f / c.C, variant == 1 ? 1 : 0,
                       variant == 2 ? GAU_LOCAL_ONLY : variant == 3 ? GAU_GLOBAL_ONLY : GAU_FULL};
        const size_t wsb = gau_backward_workspace_bytes(&cfg);
        void* ws = buf(wsb);
        void* gO = buf(M * c.d * eb);
        float* gX = (float*)buf(M * c.d * 4);
        float* gu = (float*)buf((size_t)c.e * c.d * 4);
        float* gv = (float*)buf((size_t)c.e * c.d * 4);
        float* gz = (float*)buf((size_t)c.s * c.d * 4);
        float* go = (float*)buf((size_t)c.d * c.e * 4);
        float* gs = (float*)buf(4 * c.s * 4);
        float* gb = (float*)buf(4 * c.s * 4);
        float* gr = (float*)buf((2 * c.C - 1) * 4);
        int st = variant == 4 ? gau_backward_segmented(&cfg, seg, X, Wu, Wv, Wz, Wo, sc, of, rp, gO, gX, gu, gv, gz,
                                                       go, gs, gb, gr, ws, wsb, nullptr)
                              : gau_backward(&cfg, X, Wu, Wv, Wz, Wo, sc, of, rp, gO, gX, gu, gv, gz, go, gs, gb, gr,
                                             ws, wsb, nullptr);
        if (st != GAU_OK) {
            fprintf(stderr, "gau_backward status %d\n", st);
            exit(1);
        }
        for (void* p : {ws, gO, (void*)gX, (void*)gu, (void*)gv, (void*)gz, (void*)go, (void*)gs, (void*)gb,
                        (void*)gr})
            free(p);
    });
    for (void* p : {X, Wu, Wv, Wz, Wo, (void*)sc, (void*)of, (void*)rp, U, Vt, Qq, Kq, Ql, Klt, (void*)S, P, A, Y, O,
                    (void*)Of, (void*)ra, (void*)rb, (void*)rw, dx, dO, (void*)dP, dKq, dV, dKl, (void*)du,
                    (void*)dz, dy, (void*)seg})
        free(p);
}

int main(int argc, char** argv) {
    // B, T, d, e, s, C, bf16, causal
    std::vector<Cfg> small = {
        {1, 256, 128, 256, 128, 64, false, true},   {1, 256, 128, 256, 128, 64, false, false},
        {2, 512, 256, 512, 128, 128, true, true},   {2, 512, 256, 512, 128, 128, true, false},
        {1, 320, 128, 256, 128, 64, true, true},    {1, 320, 128, 256, 128, 64, false, true},
        {1, 1024, 256, 512, 128, 512, true, true},  {1, 1024, 256, 512, 128, 512, true, false},
        {1, 512, 256, 512, 256, 256, true, true},   {1, 256, 128, 256, 256, 128, false, false},
        {3, 128, 128, 256, 128, 128, true, true},   {2, 192, 384, 768, 128, 64, true, true},
        {1, 1024, 256, 512, 128, 256, true, true},  {2, 512, 1024, 2048, 128, 256, true, true},
        {1, 64, 128, 256, 128, 64, true, true},     {1, 64, 128, 256, 128, 64, false, false},
        {1, 256, 128, 1024, 128, 64, false, true},  {1, 512, 256, 1024, 256, 128, true, true},
        {1, 320, 128, 1024, 256, 64, false, false}, {2, 256, 128, 1280, 128, 128, true, true},
        // batches that decode on the MFMA core (one ragged and two token tiles)
        {17, 64, 128, 256, 128, 64, true, true},     {70, 64, 128, 512, 256, 64, false, true},
    };
    // batches whose decoding attention takes 8 features per thread (decoding
    // launches only)
    std::vector<Cfg> decode_wide = {
        {96, 64, 128, 1536, 128, 64, false, true}, {176, 64, 128, 1536, 128, 64, true, true},
    };
    std::vector<Cfg> full = {
        {8, 1024, 768, 1536, 128, 256, true, true}, {4, 4096, 768, 1536, 128, 256, true, true},
        {4, 4096, 768, 1536, 128, 256, true, false}, {2, 8192, 768, 1536, 128, 512, true, true},
        {2, 8192, 768, 1536, 128, 256, true, true},
    };
    const std::string which = argc > 1 ? argv[1] : "small";
    const std::string only = argc > 2 ? argv[2] : "";
    if (which == "small" || which == "all") {
        for (auto& c : small) run(c, only);
        if (only.empty() || only.compare(0, 6, "decode") == 0)
            for (auto& c : decode_wide) run(c, only.empty() ? "decode" : only);
    }
    if (which == "full" || which == "all")
        for (auto& c : full) run(c, only);
    if (which == "headline") run(full.back(), only);
    fprintf(stderr, "all launches in bounds\n");
    return 0;
}
