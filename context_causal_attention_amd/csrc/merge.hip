// combine(): LSE-weighted merge of two partial attention results over disjoint
// key sets, in place into the accumulator (Accelerate concept guide, "So how
// does it work?", names combine() without a formula; this is the exact
// recombination of softmax over a union of key sets).
//
//   L = M + ln(e^(l1 - M) + e^(l2 - M)),  M = max(l1, l2)
//   O = e^(l1 - L) * O1 + e^(l2 - L) * O2
//
// (0, -inf) is the identity; two empty rows stay (0, -inf).  Every product and
// sum is rounded separately (no fused multiply-add) so that swapping the two
// operands gives the same bits.
//
// HBM-bound: each thread moves 16 bytes of each O operand per pass of a
// grid-stride loop; a row of d = 64 or 128 floats lies inside one wave (waves
// start on multiples of 64 vectors, and so does every pass, since the stride is
// a multiple of 256 vectors), so the thread that writes a row's new LSE does so
// after every lane of its wave has read the old one (same load instruction,
// data dependence of the store).
#include <hip/hip_runtime.h>

#include "internal.h"

namespace cpattn {
namespace {

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

__global__ __launch_bounds__(256) void merge_kernel(long long n4, int d4, f32x4* __restrict__ o_acc,
                                                    float* lse_acc, const f32x4* __restrict__ o_p,
                                                    const float* __restrict__ lse_p) {
#pragma clang fp contract(off)
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const long long row = i / d4;
    const float l1 = lse_acc[row];
    const float l2 = lse_p[row];
    const float M = fmaxf(l1, l2);
    f32x4 out;
    float L;
    if (M == -INFINITY) {
      out = f32x4{0.f, 0.f, 0.f, 0.f};
      L = -INFINITY;
    } else {
      L = M + logf(expf(l1 - M) + expf(l2 - M));
      const float w1 = expf(l1 - L);
      const float w2 = expf(l2 - L);
      const f32x4 a = o_acc[i];
      const f32x4 c = o_p[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = w1 * a[e];
        const float y = w2 * c[e];
        out[e] = x + y;
      }
    }
    o_acc[i] = out;
    if (i % d4 == 0) lse_acc[row] = L;
  }
}

}  // namespace

hipError_t launch_merge(int64_t rows, int32_t d, float* o_acc, float* lse_acc, const float* o_p,
                        const float* lse_p, hipStream_t stream) {
  const long long n4 = (long long)rows * d / 4;
  // One pass covers up to 2^30 vectors (2^25 rows at d = 128); larger inputs
  // loop, so the grid stays inside its 32-bit size limit for every row count.
  hipLaunchKernelGGL(merge_kernel, dim3(stride_blocks(n4)), dim3(256), 0, stream, n4, d / 4,
                     reinterpret_cast<f32x4*>(o_acc), lse_acc, reinterpret_cast<const f32x4*>(o_p), lse_p);
  return hipGetLastError();
}

}  // namespace cpattn
