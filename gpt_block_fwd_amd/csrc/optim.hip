// Adam update of fp32 master parameters, in place, with an optional bf16
// copy of the updated values for the forward pass.  One streaming pass over
// HBM: reads p, g, m, v and writes p, m, v (28 bytes per parameter, 30 with
// the copy); each thread moves 16-byte vectors, grid-stride.
#include <algorithm>

#include "kernels.h"

namespace {

DEV float adam_one(const AdamHyper &h, float &p, float g, float &m, float &v) {
  m = h.beta1 * m + h.one_minus_beta1 * g;
  v = h.beta2 * v + h.one_minus_beta2 * (g * g);
  p = p - h.lr * (m * h.corr1) / (sqrtf(v * h.corr2) + h.eps);
  return p;
}

__global__ __launch_bounds__(256) void adam_kernel(float *__restrict__ p, const float *__restrict__ g,
                                                   float *__restrict__ m, float *__restrict__ v,
                                                   bf16 *__restrict__ pb, long long n, AdamHyper h) {
  const long long n4 = n >> 2;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    f32x4 pp = ((const f32x4 *)p)[i];
    const f32x4 gg = ((const f32x4 *)g)[i];
    f32x4 mm = ((const f32x4 *)m)[i];
    f32x4 vv = ((const f32x4 *)v)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = pp[e], b = mm[e], c = vv[e];
      adam_one(h, a, gg[e], b, c);
      pp[e] = a;
      mm[e] = b;
      vv[e] = c;
    }
    ((f32x4 *)p)[i] = pp;
    ((f32x4 *)m)[i] = mm;
    ((f32x4 *)v)[i] = vv;
    if (pb) ((bf16x4 *)pb)[i] = (bf16x4){f2bf(pp[0]), f2bf(pp[1]), f2bf(pp[2]), f2bf(pp[3])};
  }
  // the last n % 4 parameters
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const long long i = (n4 << 2) + threadIdx.x;
    float a = p[i], b = m[i], c = v[i];
    adam_one(h, a, g[i], b, c);
    p[i] = a;
    m[i] = b;
    v[i] = c;
    if (pb) pb[i] = f2bf(a);
  }
}

}  // namespace

void launch_adam(float *p, const float *g, float *m, float *v, bf16 *pb, long long n, const AdamHyper &h,
                 hipStream_t s) {
  if (n <= 0) return;
  const long long n4 = n >> 2;
  // enough 256-thread workgroups to keep every CU streaming (8 per CU), at
  // least one for the tail
  const long long want = (n4 + 255) / 256;
  const unsigned blocks = (unsigned)std::max(1LL, std::min(want, 2048LL));
  adam_kernel<<<blocks, 256, 0, s>>>(p, g, m, v, pb, n, h);
}
