// The RoPE-built relative-position bias vector.  (The rotation of the four
// heads runs in the projection's epilogue, proj_gemm.hip.)
//
// The rotation is not printed on the pages; the reading here takes the
// frequency schedule and half-split layout of the sinusoid helper the pages
// print (papercache, appendix D, _get_scaledsin): the pair (h_i, h_{i+dim/2})
// turns by d * theta_i, theta_i = 10000^(-i/(dim/2)).
//
// The bias: for chunk lengths of 512 and more, Code 4 (papercache, appendix D)
// builds the Toeplitz matrix as rope(a)_m . rope(b)_n from two learned
// vectors; the product depends only on n - m, so one 2n-1 vector w with
// w[n-1 + d] = a . rope(b, d) carries it, and the layer takes it as its
// relpos argument unchanged.

#include "gau_device.h"
#include "gau_launch.h"

namespace gau {
namespace {

// w[n-1 + d] = sum_i a_i (b_i cos - b_{i+h} sin) + a_{i+h} (b_{i+h} cos + b_i sin),
// angle d * theta_i, for d = -(n-1) .. n-1.
__global__ __launch_bounds__(256) void rope_relpos_kernel(const float* a, const float* b, int n, int dim,
                                                         float* w) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= 2 * n - 1) return;
    const int half = dim / 2;
    const double d = (double)(k - (n - 1));
    double acc = 0.0;
    for (int i = 0; i < half; ++i) {
        double sn, cs;
        sincos(d * rope_theta(i, half), &sn, &cs);
        const double ai = a[i], ah = a[i + half], bi = b[i], bh = b[i + half];
        acc += cs * (ai * bi + ah * bh) + sn * (ah * bi - ai * bh);
    }
    w[k] = (float)acc;
}

}  // namespace

hipError_t launch_rope_relpos(const float* a, const float* b, int n, int dim, float* relpos, hipStream_t st) {
    hipLaunchKernelGGL(rope_relpos_kernel, dim3((unsigned)((2 * n - 1 + 255) / 256)), dim3(256), 0, st, a, b, n,
                       dim, relpos);
    return hipGetLastError();
}

}  // namespace gau
