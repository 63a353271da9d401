// CPU emulation runtime for libgau's kernels (test infrastructure only; the
// library never uses it).
//
// FAST mode: every lane of every block runs to completion one after another;
// barriers are no-ops, MFMA returns its accumulator, shuffles return the own
// value.  Addresses do not depend on data in these kernels, so this visits
// every global and LDS access; built with AddressSanitizer and exact-size
// buffers it reports any out-of-bounds access with the source line.
//
// FULL mode: the lanes of a block run as fibers.  __syncthreads is a block
// barrier, MFMA and shuffles are wave-wide exchanges with the hardware's
// operand layouts, and LDS DMA writes land either at issue (EMU_DMA_LATE=0)
// or only when an s_waitcnt requires them (late), so both a missing wait and
// a write into a stage still being read change the results.  The mode is set
// with emu_set_mode() or the EMU_MODE=full / EMU_DMA_LATE=1 environment.
#include "hip/hip_runtime.h"

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <deque>
#include <map>
#include <sys/mman.h>
#include <vector>

extern "C" void emu_switch(void** from_sp, void* to_sp);
asm(R"(
.text
.globl emu_switch
.type emu_switch,@function
emu_switch:
    pushq %rbp
    pushq %rbx
    pushq %r12
    pushq %r13
    pushq %r14
    pushq %r15
    movq %rsp, (%rdi)
    movq %rsi, %rsp
    popq %r15
    popq %r14
    popq %r13
    popq %r12
    popq %rbx
    popq %rbp
    ret
.size emu_switch, .-emu_switch
)");

namespace emu {

namespace {

enum State { READY, AT_BARRIER, AT_WAVE, DONE };
enum WaveOp { OP_NONE, OP_M32_BF16, OP_M32_F32, OP_M16_BF16, OP_M16_F32, OP_SHFL, OP_TR16 };

struct DmaEntry {
    char* dst;
    uint8_t data[16];
};

struct Lane {
    dim3 tid;
    int lin = 0, lane = 0, wave = 0;
    State state = READY;
    void* sp = nullptr;
    char* stack = nullptr;
    std::deque<DmaEntry> q;
    size_t dma_count = 0;
    WaveOp op = OP_NONE;
    int op_arg = 0;
    float a[8], b[8], c[16], r[16];
    const char* tr_ptr = nullptr;  // OP_TR16: this lane's LDS address
    uint16_t tr_out[4];
};

struct Wave {
    std::vector<char*> dma_lds;
};

bool g_full = false;
bool g_late = false;
bool g_mode_set = false;
bool g_verbose = false;
const char* g_name = "";
dim3 g_grid, g_block, g_bid;
char* g_lds = nullptr;
size_t g_lds_bytes = 0;
std::map<int, char*> g_static;
std::vector<Lane> g_lanes;
std::vector<Wave> g_waves;
Lane* g_cur = nullptr;
void (*g_tramp)(void*) = nullptr;
void* g_ctx = nullptr;
void* g_sched_sp = nullptr;
std::map<const void*, int> g_attr;
constexpr size_t kStack = 256 * 1024;
long long g_launches = 0;

[[noreturn]] void fail(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    fprintf(stderr, "EMU ERROR in %s block (%u,%u,%u)", g_name, g_bid.x, g_bid.y, g_bid.z);
    if (g_cur) fprintf(stderr, " thread %d (wave %d lane %d)", g_cur->lin, g_cur->wave, g_cur->lane);
    fprintf(stderr, ": ");
    vfprintf(stderr, fmt, ap);
    fprintf(stderr, "\n");
    va_end(ap);
    abort();
}

void flush(Lane* l, size_t keep) {
    while (l->q.size() > keep) {
        DmaEntry& e = l->q.front();
        memcpy(e.dst, e.data, 16);
        l->q.pop_front();
    }
}

void yield_to_sched() { emu_switch(&g_cur->sp, g_sched_sp); }

void fiber_main() {
    g_tramp(g_ctx);
    flush(g_cur, 0);
    g_cur->state = DONE;
    yield_to_sched();
    __builtin_unreachable();
}

void init_fiber(Lane& l) {
    if (!l.stack) {
        void* m = mmap(nullptr, kStack + 4096, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS, -1, 0);
        if (m == MAP_FAILED) fail("mmap stack");
        mprotect(m, 4096, PROT_NONE);  // guard page below the stack
        l.stack = (char*)m + 4096;
    }
    uintptr_t top = ((uintptr_t)l.stack + kStack) & ~(uintptr_t)15;
    void** s = (void**)top;
    *--s = nullptr;                 // fake return address of fiber_main
    *--s = (void*)&fiber_main;      // popped by emu_switch's ret
    for (int i = 0; i < 6; ++i) *--s = nullptr;  // rbp rbx r12 r13 r14 r15
    l.sp = s;
}

void resume(Lane* l) {
    g_cur = l;
    emu_switch(&g_sched_sp, l->sp);
    g_cur = nullptr;
}

float bf2f(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

// Execute the wave op all lanes of wave w are waiting at.
void run_wave_op(int w, int first, int n) {
    Lane* L = &g_lanes[first];
    const WaveOp op = L[0].op;
    const int arg = L[0].op_arg;
    for (int i = 0; i < n; ++i)
        if (L[i].op != op || L[i].op_arg != arg) fail("wave %d: lanes wait at different wave ops", w);
    if (op == OP_TR16) {
        // ds_read_b64_tr_b16: per group of 16 lanes, lane i receives as its
        // element jj element i % 4 of the 8 bytes lane 4 jj + i / 4 addressed
        if (n != 64) fail("transposed LDS read in a partial wave");
        for (int i = 0; i < n; ++i) {
            const char* q = L[i].tr_ptr;
            if (q < g_lds || q + 8 > g_lds + g_lds_bytes)
                fail("transposed read of LDS [%td, %td) outside the %zu-byte allocation", q - g_lds, q + 8 - g_lds,
                     g_lds_bytes);
            if (((q - g_lds) & 7) != 0) fail("transposed read address not 8-byte aligned");
        }
        for (int l = 0; l < 64; ++l) {
            const int g = l % 16, base = l - g;
            for (int jj = 0; jj < 4; ++jj)
                memcpy(&L[l].tr_out[jj], L[base + 4 * jj + g / 4].tr_ptr + 2 * (g % 4), 2);
        }
        return;
    }
    if (op == OP_SHFL) {
        for (int i = 0; i < n; ++i) {
            const int src = i ^ arg;
            if (src >= n) fail("shuffle source lane %d outside the wave", src);
            L[i].r[0] = L[src].c[0];
        }
        return;
    }
    if (n != 64) fail("MFMA in a partial wave");
    if (op == OP_M32_BF16 || op == OP_M32_F32) {
        const int kpl = op == OP_M32_BF16 ? 8 : 1;
        const int K = 2 * kpl;
        for (int l = 0; l < 64; ++l) {
            const int j = l % 32, h = l / 32;
            for (int r = 0; r < 16; ++r) {
                const int i = 8 * (r / 4) + 4 * h + (r % 4);
                double s = L[l].c[r];
                for (int k = 0; k < K; ++k)
                    s += (double)L[i + 32 * (k / kpl)].a[k % kpl] * (double)L[j + 32 * (k / kpl)].b[k % kpl];
                L[l].r[r] = (float)s;
            }
        }
    } else {
        const int kpl = op == OP_M16_BF16 ? 8 : 1;
        const int K = 4 * kpl;
        for (int l = 0; l < 64; ++l) {
            const int j = l % 16;
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * (l / 16) + r;
                double s = L[l].c[r];
                for (int k = 0; k < K; ++k)
                    s += (double)L[i + 16 * (k / kpl)].a[k % kpl] * (double)L[j + 16 * (k / kpl)].b[k % kpl];
                L[l].r[r] = (float)s;
            }
        }
    }
}

void run_block_full(int nt) {
    for (int t = 0; t < nt; ++t) {
        g_lanes[t].state = READY;
        init_fiber(g_lanes[t]);
    }
    const int nw = (nt + 63) / 64;
    for (;;) {
        for (int w = 0; w < nw; ++w) {
            const int first = 64 * w, n = std::min(64, nt - first);
            for (;;) {
                for (int i = 0; i < n; ++i)
                    if (g_lanes[first + i].state == READY) resume(&g_lanes[first + i]);
                int at_wave = 0, done = 0;
                for (int i = 0; i < n; ++i) {
                    at_wave += g_lanes[first + i].state == AT_WAVE;
                    done += g_lanes[first + i].state == DONE;
                }
                if (at_wave == 0) break;
                if (at_wave != n) fail("wave %d: %d lanes at a wave op, %d done, the rest at a barrier", w, at_wave, done);
                run_wave_op(w, first, n);
                for (int i = 0; i < n; ++i) g_lanes[first + i].state = READY;
            }
        }
        int done = 0, bar = 0;
        for (int t = 0; t < nt; ++t) {
            done += g_lanes[t].state == DONE;
            bar += g_lanes[t].state == AT_BARRIER;
        }
        if (done == nt) break;
        if (done + bar != nt) fail("scheduler: lanes neither done nor at the barrier");
        // every wave must pass the same number of barriers: a lane that has
        // finished while others wait at a barrier means the counts differ
        if (done != 0) fail("barrier count mismatch: %d lanes done, %d at a barrier", done, bar);
        for (int t = 0; t < nt; ++t)
            if (g_lanes[t].state == AT_BARRIER) g_lanes[t].state = READY;
    }
}

void wave_op(WaveOp op, int arg) {
    g_cur->op = op;
    g_cur->op_arg = arg;
    g_cur->state = AT_WAVE;
    yield_to_sched();
}

}  // namespace

const dim3& thread_idx() { return g_cur->tid; }
const dim3& block_idx() { return g_bid; }
const dim3& grid_dim() { return g_grid; }
const dim3& block_dim() { return g_block; }

void syncthreads() {
    if (!g_full) return;
    g_cur->state = AT_BARRIER;
    yield_to_sched();
}

char* lds_base() { return g_lds; }

void* static_shared(int key, size_t bytes) {
    auto it = g_static.find(key);
    if (it != g_static.end()) return it->second;
    char* p = (char*)malloc(bytes);
    memset(p, 0xFF, bytes);
    g_static[key] = p;
    return p;
}

void global_load_lds(const void* g, void* l, int size, int offset, int aux) {
    if (size != 16 || offset != 0 || aux != 0) fail("global_load_lds form not emulated");
    Lane* L = g_cur;
    Wave& W = g_waves[L->wave];
    const size_t k = L->dma_count++;
    if (k >= W.dma_lds.size())
        W.dma_lds.push_back((char*)l);
    else if (W.dma_lds[k] != (char*)l)
        fail("LDS base of DMA #%zu differs across the wave (%td vs %td)", k, (char*)l - g_lds, W.dma_lds[k] - g_lds);
    if (((uintptr_t)g & 15) != 0) fail("DMA source not 16-byte aligned");
    char* dst = (char*)l + 16 * L->lane;
    if (dst < g_lds || dst + 16 > g_lds + g_lds_bytes)
        fail("DMA writes LDS [%td, %td) outside the %zu-byte allocation", dst - g_lds, dst + 16 - g_lds, g_lds_bytes);
    DmaEntry e;
    memcpy(e.data, g, 16);
    if (!g_full || !g_late) {
        memcpy(dst, e.data, 16);
    } else {
        e.dst = dst;
        L->q.push_back(e);
    }
}

BufRsrc make_buffer_rsrc(const void* base, int stride, int num_records, int flags) {
    if (stride != 0 || flags != 0x00020000) fail("buffer resource form not emulated");
    return BufRsrc{(const char*)base, (uint32_t)num_records};
}

// buffer_load_dwordx4 ... lds (offen): the lane's bytes at base + voffset +
// soffset + offset; an offset at or past num_records reads zeros (the raw
// buffer's range check), otherwise the same copy as global_load_lds.
void buffer_load_lds(const BufRsrc& r, void* l, int size, int voffset, int soffset, int offset, int aux) {
    if (size != 16 || offset != 0 || aux != 0) fail("buffer_load_lds form not emulated");
    if (voffset < 0 || soffset < 0) fail("negative buffer offset (%d, %d)", voffset, soffset);
    const uint64_t off = (uint64_t)voffset + (uint64_t)soffset;
    if (off + 16 > r.num_records) {
        alignas(16) static const char zeros[16] = {};
        global_load_lds(zeros, l, 16, 0, 0);
        return;
    }
    global_load_lds(r.base + off, l, 16, 0, 0);
}

void s_waitcnt(int imm) {
    const int vm = (imm & 0xF) | (((imm >> 14) & 3) << 4);
    flush(g_cur, (size_t)vm);
}

f32x16_t mfma_32x32x16_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    if (!g_full) return c;
    uint16_t ua[8], ub[8];
    memcpy(ua, &a, 16);
    memcpy(ub, &b, 16);
    for (int t = 0; t < 8; ++t) {
        g_cur->a[t] = bf2f(ua[t]);
        g_cur->b[t] = bf2f(ub[t]);
    }
    for (int r = 0; r < 16; ++r) g_cur->c[r] = c[r];
    wave_op(OP_M32_BF16, 0);
    f32x16_t d;
    for (int r = 0; r < 16; ++r) d[r] = g_cur->r[r];
    return d;
}

f32x16_t mfma_32x32x2_f32(float a, float b, f32x16_t c) {
    if (!g_full) return c;
    g_cur->a[0] = a;
    g_cur->b[0] = b;
    for (int r = 0; r < 16; ++r) g_cur->c[r] = c[r];
    wave_op(OP_M32_F32, 0);
    f32x16_t d;
    for (int r = 0; r < 16; ++r) d[r] = g_cur->r[r];
    return d;
}

f32x4_t mfma_16x16x32_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    if (!g_full) return c;
    uint16_t ua[8], ub[8];
    memcpy(ua, &a, 16);
    memcpy(ub, &b, 16);
    for (int t = 0; t < 8; ++t) {
        g_cur->a[t] = bf2f(ua[t]);
        g_cur->b[t] = bf2f(ub[t]);
    }
    for (int r = 0; r < 4; ++r) g_cur->c[r] = c[r];
    wave_op(OP_M16_BF16, 0);
    f32x4_t d;
    for (int r = 0; r < 4; ++r) d[r] = g_cur->r[r];
    return d;
}

f32x4_t mfma_16x16x4_f32(float a, float b, f32x4_t c) {
    if (!g_full) return c;
    g_cur->a[0] = a;
    g_cur->b[0] = b;
    for (int r = 0; r < 4; ++r) g_cur->c[r] = c[r];
    wave_op(OP_M16_F32, 0);
    f32x4_t d;
    for (int r = 0; r < 4; ++r) d[r] = g_cur->r[r];
    return d;
}

s16x4_t ds_read_tr16(const void* p) {
    const char* q = (const char*)p;
    s16x4_t out;
    if (!g_full) {
        // addresses only: the lane's own 8 bytes (in bounds, aligned)
        if (q < g_lds || q + 8 > g_lds + g_lds_bytes)
            fail("transposed read of LDS [%td, %td) outside the %zu-byte allocation", q - g_lds, q + 8 - g_lds,
                 g_lds_bytes);
        if (((q - g_lds) & 7) != 0) fail("transposed read address not 8-byte aligned");
        memcpy(&out, q, 8);
        return out;
    }
    g_cur->tr_ptr = q;
    wave_op(OP_TR16, 0);
    memcpy(&out, g_cur->tr_out, 8);
    return out;
}

float shfl_xor(float v, int mask) {
    if (!g_full) return v;
    g_cur->c[0] = v;
    wave_op(OP_SHFL, mask);
    return g_cur->r[0];
}

hipError_t func_set_attr(const void* f, int attr, int value) {
    if (attr == hipFuncAttributeMaxDynamicSharedMemorySize) g_attr[f] = value;
    return hipSuccess;
}

hipError_t last_error() { return hipSuccess; }

void launch_impl(const char* name, const void* fn, void (*tramp)(void*), void* ctx, dim3 grid, dim3 block,
                 size_t lds, hipStream_t) {
    static bool init = false;
    if (!init) {
        init = true;
        if (!g_mode_set) {
            const char* m = getenv("EMU_MODE");
            g_full = m && !strcmp(m, "full");
            const char* d = getenv("EMU_DMA_LATE");
            g_late = d && !strcmp(d, "1");
        }
        g_verbose = getenv("EMU_VERBOSE") != nullptr;
    }
    g_name = name;
    g_cur = nullptr;
    ++g_launches;
    const long long nblocks = (long long)grid.x * grid.y * grid.z;
    const int nt = (int)(block.x * block.y * block.z);
    if (nblocks <= 0 || nt <= 0) fail("empty launch (grid %u,%u,%u block %u,%u,%u)", grid.x, grid.y, grid.z, block.x, block.y, block.z);
    if (nt > 1024) fail("block of %d threads", nt);
    if (grid.x > 0x7fffffffu) fail("grid too large");
    if (lds > 160 * 1024) fail("%zu bytes of dynamic LDS", lds);
    if (lds > 64 * 1024) {
        auto it = g_attr.find(fn);
        if (it == g_attr.end() || (size_t)it->second < lds) fail("%zu bytes of dynamic LDS without the attribute", lds);
    }
    if (g_verbose) fprintf(stderr, "emu launch %s grid %lld x %d lds %zu\n", name, nblocks, nt, lds);
    g_grid = grid;
    g_block = block;
    g_tramp = tramp;
    g_ctx = ctx;
    g_lanes.resize(std::max<size_t>(g_lanes.size(), nt));
    g_waves.assign((nt + 63) / 64, Wave());
    for (unsigned bz = 0; bz < grid.z; ++bz)
        for (unsigned by = 0; by < grid.y; ++by)
            for (unsigned bx = 0; bx < grid.x; ++bx) {
                g_bid = dim3(bx, by, bz);
                g_lds_bytes = lds;
                g_lds = (char*)malloc(lds ? lds : 1);
                memset(g_lds, 0xFF, lds ? lds : 1);  // unwritten LDS reads as NaN
                for (auto& w : g_waves) w.dma_lds.clear();
                for (int t = 0; t < nt; ++t) {
                    Lane& l = g_lanes[t];
                    l.lin = t;
                    l.tid = dim3(t % block.x, (t / block.x) % block.y, t / (block.x * block.y));
                    l.lane = t % 64;
                    l.wave = t / 64;
                    l.q.clear();
                    l.dma_count = 0;
                }
                if (g_full) {
                    run_block_full(nt);
                } else {
                    for (int t = 0; t < nt; ++t) {
                        g_cur = &g_lanes[t];
                        tramp(ctx);
                        flush(g_cur, 0);
                    }
                    g_cur = nullptr;
                }
                free(g_lds);
                g_lds = nullptr;
                for (auto& kv : g_static) free(kv.second);
                g_static.clear();
            }
}

}  // namespace emu

// Select FULL (full != 0) or FAST emulation, and for FULL whether LDS DMA
// writes land late (at the wait that requires them) or at issue.
extern "C" void emu_set_mode(int full, int late) {
    emu::g_mode_set = true;
    emu::g_full = full != 0;
    emu::g_late = late != 0;
}
