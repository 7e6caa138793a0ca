// Query transform q~ = T^{-T} q per query head (WUSH-KV digest, "method key points":
// the query side of the key transform is one d x d product per query, which keeps
// q~ . (T k) = q . k).  One workgroup per (batch row, query head); thread i forms
// output channel i from the row i of T^{-T} with four interleaved fp32 partial sums.
#include "wushkv_internal.h"

namespace wushkv {
namespace {

__global__ void __launch_bounds__(128) qtransform_kernel(QtArgs a) {
  __shared__ float qs[128];
  const int bh = blockIdx.x;
  const int h = bh % a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int i = threadIdx.x;
  if (i < a.d) qs[i] = load_in(a.q, a.q_dtype, (size_t)bh * a.d + i);
  __syncthreads();
  if (i >= a.d) return;
  const float *row = a.tinvt + ((size_t)g * a.d + i) * a.d;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  for (int j = 0; j < a.d; j += 4) {
    s0 = fmaf(row[j], qs[j], s0);
    s1 = fmaf(row[j + 1], qs[j + 1], s1);
    s2 = fmaf(row[j + 2], qs[j + 2], s2);
    s3 = fmaf(row[j + 3], qs[j + 3], s3);
  }
  a.qt[(size_t)bh * a.d + i] = (s0 + s1) + (s2 + s3);
}

}  // namespace

hipError_t launch_qtransform(const QtArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(qtransform_kernel, dim3(a.B * a.Hq), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace wushkv
