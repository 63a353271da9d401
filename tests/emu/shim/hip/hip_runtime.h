// CPU emulation shim: lets the library's kernel sources compile for the host.
// Kernels run on the CPU, one lane at a time (FAST: addresses only) or as
// fibers with wave-level MFMA / shuffle and block barriers (FULL).
#pragma once
#include <cstdint>
#include <cstddef>
#include <cmath>
#include <cstring>
#include <algorithm>

#define __device__
#define __host__
#define __global__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __align__(n) __attribute__((aligned(n)))
#define __restrict__ __restrict

typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorLaunchFailure = 719 };
typedef void* hipStream_t;
typedef int hipFuncAttribute;
enum { hipFuncAttributeMaxDynamicSharedMemorySize = 8 };
struct dim3 {
    unsigned x, y, z;
    dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};

namespace emu {
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
const dim3& thread_idx();
const dim3& block_idx();
const dim3& grid_dim();
const dim3& block_dim();
void syncthreads();
char* lds_base();
void* static_shared(int key, size_t bytes);
void global_load_lds(const void* g, void* l, int size, int offset, int aux);
// A raw buffer resource (stride 0): its base and the byte count past which
// loads read zeros.
struct BufRsrc {
    const char* base;
    uint32_t num_records;
};
BufRsrc make_buffer_rsrc(const void* base, int stride, int num_records, int flags);
void buffer_load_lds(const BufRsrc& r, void* l, int size, int voffset, int soffset, int offset, int aux);
void s_waitcnt(int imm);
f32x16_t mfma_32x32x16_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c);
f32x16_t mfma_32x32x2_f32(float a, float b, f32x16_t c);
f32x4_t mfma_16x16x32_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c);
f32x4_t mfma_16x16x4_f32(float a, float b, f32x4_t c);
float shfl_xor(float v, int mask);
s16x4_t ds_read_tr16(const void* p);
hipError_t func_set_attr(const void* f, int attr, int value);
void launch_impl(const char* name, const void* fn, void (*tramp)(void*), void* ctx, dim3 grid, dim3 block,
                 size_t lds, hipStream_t st);
template <typename F>
void launch(const char* name, const void* fn, F&& f, dim3 grid, dim3 block, size_t lds, hipStream_t st) {
    launch_impl(name, fn, [](void* c) { (*(F*)c)(); }, (void*)&f, grid, block, lds, st);
}
hipError_t last_error();
}  // namespace emu

#define threadIdx (::emu::thread_idx())
#define blockIdx (::emu::block_idx())
#define gridDim (::emu::grid_dim())
#define blockDim (::emu::block_dim())
inline void __syncthreads() { ::emu::syncthreads(); }
inline float __uint_as_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
inline uint32_t __float_as_uint(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
inline float __expf(float x) { return expf(x); }
inline float __shfl_xor(float v, int mask) { return ::emu::shfl_xor(v, mask); }
using std::max;
using std::min;

#define __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, x, y, z) ::emu::mfma_32x32x16_bf16(a, b, c)
#define __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, x, y, z) ::emu::mfma_32x32x2_f32(a, b, c)
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, x, y, z) ::emu::mfma_16x16x32_bf16(a, b, c)
#define __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, x, y, z) ::emu::mfma_16x16x4_f32(a, b, c)
#define __builtin_amdgcn_global_load_lds(g, l, sz, off, aux) \
    ::emu::global_load_lds((const void*)(g), (void*)(l), sz, off, aux)
typedef ::emu::BufRsrc __amdgpu_buffer_rsrc_t;
#define __builtin_amdgcn_make_buffer_rsrc(p, stride, n, flags) ::emu::make_buffer_rsrc((const void*)(p), stride, n, flags)
#define __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, sz, voff, soff, off, aux) \
    ::emu::buffer_load_lds(r, (void*)(l), sz, voff, soff, off, aux)
#define __builtin_amdgcn_s_waitcnt(imm) ::emu::s_waitcnt(imm)
#define __builtin_amdgcn_ds_read_tr16_b64_v4i16(p) ::emu::ds_read_tr16((const void*)(p))
#define __builtin_amdgcn_sched_group_barrier(a, b, c) ((void)0)
#define __builtin_amdgcn_s_barrier() ::emu::syncthreads()
#define __builtin_amdgcn_sched_barrier(m) ((void)0)
#define __builtin_amdgcn_rcpf(x) (1.0f / (x))

#define hipFuncSetAttribute(f, attr, v) ::emu::func_set_attr((const void*)(f), attr, v)
#define hipGetLastError() ::emu::last_error()
#define hipLaunchKernelGGL(kernel, grid, block, lds, stream, ...) \
    ::emu::launch(#kernel, (const void*)(kernel), [=]() { kernel(__VA_ARGS__); }, dim3(grid), dim3(block), (lds), (stream))

// Device symbols: on the host emulation a __device__ array is an ordinary
// host array, so its "device address" is its address; one device (0).
#define HIP_SYMBOL(x) ((const void*)&(x))
inline hipError_t hipGetDevice(int* dev) {
    *dev = 0;
    return hipSuccess;
}
inline hipError_t hipGetSymbolAddress(void** p, const void* sym) {
    *p = const_cast<void*>(sym);
    return hipSuccess;
}
