// Query transform q~ = T^{-T} q per query head (WUSH-KV digest, "method key points":
// the query side of the key transform is one d x d product per query, which keeps
// q~ . (T k) = q . k).
//
// One workgroup per (batch row, KV head): the head's T^{-T} is staged in LDS once
// (coalesced 16-byte loads) and serves all of its query heads.  Thread t forms output
// channel t % d of query head t / d (and the heads 256 / d further on), reading its row
// of T^{-T} from LDS with four interleaved fp32 partial sums.
#include "wushkv_internal.h"

namespace wushkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kHeadChunk = 16;   // query heads staged at a time

template <int D>
__global__ void __launch_bounds__(kThreads) qtransform_kernel(QtArgs a) {
  __shared__ float T[D][D + 4];            // +4: rows start in different banks
  __shared__ float qs[kHeadChunk][D];
  const int tid = threadIdx.x;
  const int bg = blockIdx.x;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const float *src = a.tinvt + (size_t)g * D * D;
  for (int i = tid; i < D * D / 4; i += kThreads) {
    const int r = i / (D / 4), c4 = i % (D / 4);
    *(f32x4 *)&T[r][4 * c4] = *(const f32x4 *)(src + (size_t)r * D + 4 * c4);
  }
  for (int h0 = 0; h0 < G; h0 += kHeadChunk) {
    const int nh = G - h0 < kHeadChunk ? G - h0 : kHeadChunk;
    const size_t qbase = ((size_t)b * a.Hq + (size_t)g * G + h0) * D;
    __syncthreads();   // T staged; the previous chunk's qs reads are done
    for (int i = tid; i < nh * D; i += kThreads) qs[i / D][i % D] = load_in(a.q, a.q_dtype, qbase + i);
    __syncthreads();
    for (int o = tid; o < nh * D; o += kThreads) {
      const int h = o / D, i = o % D;
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int j = 0; j < D; j += 4) {
        const f32x4 t = *(const f32x4 *)&T[i][j];
        const f32x4 x = *(const f32x4 *)&qs[h][j];
        s[0] = fmaf(t[0], x[0], s[0]);
        s[1] = fmaf(t[1], x[1], s[1]);
        s[2] = fmaf(t[2], x[2], s[2]);
        s[3] = fmaf(t[3], x[3], s[3]);
      }
      a.qt[qbase + o] = (s[0] + s[1]) + (s[2] + s[3]);
    }
  }
}

}  // namespace

hipError_t launch_qtransform(const QtArgs &a, hipStream_t s) {
  if (a.d == 128)
    hipLaunchKernelGGL(qtransform_kernel<128>, dim3(a.B * a.Hkv), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(qtransform_kernel<64>, dim3(a.B * a.Hkv), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace wushkv
