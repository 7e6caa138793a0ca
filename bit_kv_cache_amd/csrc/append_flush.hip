// Append + flush kernels of the WUSH-KV cache on gfx950.
//
// Append writes new tokens' fp16 values into the sink window or the ring of the
// recent window.  Flush quantizes tokens leaving the recent window (WUSH-KV digest,
// "takeaways" / "method key points": FP16 sink and recent windows, chunked flush;
// the key transform after RoPE, one d x d product per token).
//
// Flush, per workgroup: one (batch row, KV head, 64-token V set).
//   1. stage the rows' fp16 K and V in LDS (from the ring or the new input);
//   2. x = T_K k16 on MFMA (v_mfma_f32_16x16x32_f16: fp16 x fp16 products are exact,
//      accumulation fp32 in four 32-term steps);
//   3. per-token parameters from LDS: sum of squares (QuEST) or the few smallest /
//      largest values (percentile-clipped affine), reduced across 4 lanes per row;
//   4. codes into LDS, then packed: K rows token-major, V words in the set layout
//      (read-modify-write when the flush covers only part of a set).
#include "wushkv_internal.h"

namespace wushkv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// ------------------------------------------------------------------ append

__global__ void __launch_bounds__(kThreads) append_kernel(AppendArgs a) {
  // one thread per (token, 8-channel group); blockIdx.y = b * Hkv + g
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int groups = a.d / 8;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.n_new * groups) return;
  const int64_t t = idx / groups;
  const int j0 = (int)(idx % groups) * 8;
  const int64_t p = a.n_before + t;
  _Float16 *dk, *dv;
  if (p < a.S) {
    dk = (_Float16 *)((char *)a.sink_k + bg * a.sink_bytes) + p * a.d;
    dv = (_Float16 *)((char *)a.sink_v + bg * a.sink_bytes) + p * a.d;
  } else if (p >= a.S + a.q_after) {
    const int64_t slot = (p - a.S) % (a.R + a.C);
    dk = (_Float16 *)((char *)a.ring_k + bg * a.ring_bytes) + slot * a.d;
    dv = (_Float16 *)((char *)a.ring_v + bg * a.ring_bytes) + slot * a.d;
  } else {
    return;  // flushed straight from the input by the flush kernel
  }
  const size_t src = (((size_t)b * a.Hkv + g) * a.n_new + t) * a.d + j0;
  half8 hk, hv;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hk[e] = (_Float16)load_in(a.k_new, a.in_dtype, src + e);
    hv[e] = (_Float16)load_in(a.v_new, a.in_dtype, src + e);
  }
  *(half8 *)(dk + j0) = hk;
  *(half8 *)(dv + j0) = hv;
}

// ------------------------------------------------------------------ flush

template <int D>
struct FlushSmem {
  static constexpr int KP = D + 8;         // fp16 row pitch (16 B pad)
  static constexpr int XP = D + 4;         // fp32 row pitch
  _Float16 k16[kSet][KP];
  _Float16 v16[kSet][KP];
  float x[kSet][XP];                       // transformed keys
  uint8_t ck[kSet][D];                     // K codes
  uint8_t cv[kSet][D];                     // V codes
  float stat[kSet][4][2 * kMaxOrderStats]; // per row, per quarter: smallest / largest
  float par[2][kSet][2];                   // [K|V][row][scale, zero]
};

__device__ __forceinline__ void insert_lo(float *lo, int n, float v) {
  // keep lo[0..n) ascending: the n smallest values seen
  if (v >= lo[n - 1]) return;
  int i = n - 1;
  while (i > 0 && lo[i - 1] > v) { lo[i] = lo[i - 1]; --i; }
  lo[i] = v;
}

__device__ __forceinline__ void insert_hi(float *hi, int n, float v) {
  // keep hi[0..n) descending: the n largest values seen
  if (v <= hi[n - 1]) return;
  int i = n - 1;
  while (i > 0 && hi[i - 1] < v) { hi[i] = hi[i - 1]; --i; }
  hi[i] = v;
}

// Per-row quantizer parameters from the row's values in LDS (4 threads per row).
// Returns (scale, zero) in fp32 holding fp16-rounded values; QuEST puts the step
// in scale and leaves zero unused.
template <int D, bool KEYS>
__device__ __forceinline__ float row_val(const FlushSmem<D> &sm, int r, int j) {
  if constexpr (KEYS) return sm.x[r][j];
  else return (float)sm.v16[r][j];
}

template <int D, bool KEYS>
__device__ void row_params(const FlushArgs &a, FlushSmem<D> &sm, int row, int part, int quant, int bits) {
  const int which = KEYS ? 0 : 1;
  constexpr int Q = D / 4;
  const int j0 = part * Q;
  const int L = 1 << bits;
  if (quant == WUSHKV_Q_QUEST) {
    // pairwise: 4 partial sums of Q/4 terms per thread, then across the 4 threads
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      float v = row_val<D, KEYS>(sm, row, j0 + j);
      s[j & 3] = fmaf(v, v, s[j & 3]);
    }
    float ss = (s[0] + s[1]) + (s[2] + s[3]);
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    if (part == 0) {
      float r = sqrtf(ss / (float)D);
      float step = (float)(_Float16)(2.0f * a.clip * r / (float)L);
      sm.par[which][row][0] = step;
      sm.par[which][row][1] = 0.f;
    }
  } else {
    float lo[kMaxOrderStats], hi[kMaxOrderStats];
#pragma unroll
    for (int i = 0; i < kMaxOrderStats; ++i) { lo[i] = INFINITY; hi[i] = -INFINITY; }
    const int nl = a.need_lo, nh = a.need_hi;
    for (int j = 0; j < Q; ++j) {
      float v = row_val<D, KEYS>(sm, row, j0 + j);
      insert_lo(lo, nl, v);
      insert_hi(hi, nh, v);
    }
    for (int i = 0; i < nl; ++i) sm.stat[row][part][i] = lo[i];
    for (int i = 0; i < nh; ++i) sm.stat[row][part][kMaxOrderStats + i] = hi[i];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (part == 0) {
      for (int p = 1; p < 4; ++p) {
        for (int i = 0; i < nl; ++i) insert_lo(lo, nl, sm.stat[row][p][i]);
        for (int i = 0; i < nh; ++i) insert_hi(hi, nh, sm.stat[row][p][kMaxOrderStats + i]);
      }
      // sorted ascending xs: xs[k] = lo[k] for small k, xs[D-1-k] = hi[k]
      float x0 = lo[a.lo_i], x1 = (a.lo_i + 1 < D) ? lo[a.lo_i + 1] : x0;
      float vlo = (a.lo_i + 1 < D) ? x0 + a.lo_t * (x1 - x0) : x0;
      int hk = D - 1 - a.hi_i;  // index of xs[hi_i] in hi[]
      float y0 = hi[hk], y1 = (hk >= 1) ? hi[hk - 1] : y0;
      float vhi = (a.hi_i + 1 < D) ? y0 + a.hi_t * (y1 - y0) : y0;
      float scale = (float)(_Float16)((vhi - vlo) / (float)(L - 1));
      float zero = (float)(_Float16)vlo;
      sm.par[which][row][0] = scale;
      sm.par[which][row][1] = zero;
    }
  }
}

// The exact quantizer input: the transformed key sum_m T[j][m] k16[m] in fp64
// (fp16 x fp16 products are exact in fp64), or the value's fp16 itself.
template <int D, bool KEYS>
__device__ __noinline__ double exact_val(const FlushArgs &a, const FlushSmem<D> &sm, int g, int row, int j) {
  if constexpr (KEYS) {
    const _Float16 *T = a.tk + ((size_t)g * D + j) * D;
    double s = 0.0;
    for (int m = 0; m < D; ++m) s = fma((double)T[m], (double)sm.k16[row][m], s);
    return s;
  } else {
    return (double)sm.v16[row][j];
  }
}

// Codes from the fp32 value; an element whose scaled value lies within kEdge bins
// of a decision boundary is decided again from the exact input in fp64, so the
// code is that of the exact transformed key whatever the fp32 rounding did.
constexpr float kEdge = 2e-4f;

template <int D, bool KEYS>
__device__ void quantize_row_part(const FlushArgs &a, FlushSmem<D> &sm, int g, int row, int part, int quant, int bits) {
  const int which = KEYS ? 0 : 1;
  uint8_t (*codes)[D] = KEYS ? sm.ck : sm.cv;
  constexpr int Q = D / 4;
  const int L = 1 << bits;
  const float sc = sm.par[which][row][0], z = sm.par[which][row][1];
  if (quant == WUSHKV_Q_QUEST) {
    if (sc == 0.f) {
      for (int j = 0; j < Q; ++j) codes[row][part * Q + j] = (uint8_t)(L / 2);
      return;
    }
    const float inv = 1.0f / sc;
    for (int j = 0; j < Q; ++j) {
      float v = row_val<D, KEYS>(sm, row, part * Q + j);
      float t = fmaf(v, inv, (float)(L / 2));
      float c = floorf(t);
      if (t - c < kEdge || c + 1.0f - t < kEdge) {
        double td = exact_val<D, KEYS>(a, sm, g, row, part * Q + j) / (double)sc + (double)(L / 2);
        c = (float)floor(td);
      }
      c = fminf(fmaxf(c, 0.f), (float)(L - 1));
      codes[row][part * Q + j] = (uint8_t)c;
    }
  } else {
    if (sc == 0.f) {
      for (int j = 0; j < Q; ++j) codes[row][part * Q + j] = 0;
      return;
    }
    const float inv = 1.0f / sc;
    for (int j = 0; j < Q; ++j) {
      float v = row_val<D, KEYS>(sm, row, part * Q + j);
      float t = (v - z) * inv;
      float c = rintf(t);
      if (fabsf(t - floorf(t) - 0.5f) < kEdge) {
        double td = (exact_val<D, KEYS>(a, sm, g, row, part * Q + j) - (double)z) / (double)sc;
        c = (float)rint(td);
      }
      c = fminf(fmaxf(c, 0.f), (float)(L - 1));
      codes[row][part * Q + j] = (uint8_t)c;
    }
  }
}

template <int D>
__global__ void __launch_bounds__(kThreads) flush_kernel(FlushArgs a) {
  __shared__ FlushSmem<D> sm;
  const int tid = threadIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int64_t set = a.u0 / kSet + blockIdx.x;
  const int64_t base = set * kSet;                  // body index of row 0
  const int64_t r0 = a.u0 > base ? a.u0 - base : 0; // rows [r0, r1) of this set are flushed
  const int64_t r1 = (a.u1 < base + kSet) ? a.u1 - base : kSet;

  // 1. stage fp16 K and V rows
  for (int idx = tid; idx < kSet * D; idx += kThreads) {
    const int r = idx / D, j = idx % D;
    _Float16 hk = (_Float16)0.f, hv = (_Float16)0.f;
    if (r >= r0 && r < r1) {
      const int64_t p = a.S + base + r;
      if (p < a.n_before) {
        const int64_t slot = (p - a.S) % (a.R + a.C);
        hk = ((const _Float16 *)((const char *)a.ring_k + bg * a.ring_bytes))[slot * D + j];
        hv = ((const _Float16 *)((const char *)a.ring_v + bg * a.ring_bytes))[slot * D + j];
      } else {
        const size_t src = (((size_t)b * a.Hkv + g) * a.n_new + (p - a.n_before)) * D + j;
        hk = (_Float16)load_in(a.k_new, a.in_dtype, src);
        hv = (_Float16)load_in(a.v_new, a.in_dtype, src);
      }
    }
    sm.k16[r][j] = hk;
    sm.v16[r][j] = hv;
  }
  __syncthreads();

  // 2. x = k16 T^T on MFMA: tiles of 16 rows x 16 output channels, K = D
  {
    const int wave = tid / 64, lane = tid % 64;
    const int lq = lane / 16, lr = lane % 16;
    const _Float16 *T = a.tk + (size_t)g * D * D;
    constexpr int CT = D / 16;
    for (int tile = wave; tile < 4 * CT; tile += 4) {
      const int rt = tile / CT, ct = tile % CT;
      float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        half8 av = *(const half8 *)&sm.k16[rt * 16 + lr][32 * s + 8 * lq];
        half8 bv = *(const half8 *)&T[(size_t)(ct * 16 + lr) * D + 32 * s + 8 * lq];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.x[rt * 16 + 4 * lq + i][ct * 16 + lr] = acc[i];
    }
  }
  __syncthreads();

  // 3. parameters: 4 threads per row (adjacent lanes)
  const int row = tid / 4, part = tid % 4;
  row_params<D, true>(a, sm, row, part, a.quant_k, a.bits_k);
  row_params<D, false>(a, sm, row, part, a.quant_v, a.bits_v);
  __syncthreads();

  // 4. codes
  quantize_row_part<D, true>(a, sm, g, row, part, a.quant_k, a.bits_k);
  quantize_row_part<D, false>(a, sm, g, row, part, a.quant_v, a.bits_v);
  __syncthreads();

  // 5a. parameters out
  if (tid < kSet && tid >= r0 && tid < r1) {
    const int64_t u = base + tid;
    _Float16 *pk = (_Float16 *)((char *)a.par_k + bg * a.kpar_bytes) + u * a.kpar_n;
    _Float16 *pv = (_Float16 *)((char *)a.par_v + bg * a.vpar_bytes) + u * a.vpar_n;
    pk[0] = (_Float16)sm.par[0][tid][0];
    if (a.kpar_n == 2) pk[1] = (_Float16)sm.par[0][tid][1];
    pv[0] = (_Float16)sm.par[1][tid][0];
    if (a.vpar_n == 2) pv[1] = (_Float16)sm.par[1][tid][1];
  }

  // 5b. K rows: plane 0 words (16 channels), then plane 1
  {
    constexpr int W0 = D / 16;
    const int w1n = a.bits_k == 3 ? D / 32 : (a.bits_k == 4 ? D / 16 : 0);
    const int wrow = W0 + w1n;
    uint8_t *kb = a.codes_k + bg * a.kcode_bytes;
    for (int idx = tid; idx < kSet * wrow; idx += kThreads) {
      const int r = idx / wrow, w = idx % wrow;
      if (r < r0 || r >= r1) continue;
      unsigned word = 0;
      if (w < W0) {
        for (int f = 0; f < 16; ++f) word |= (unsigned)(sm.ck[r][16 * w + f] & 3) << (2 * f);
      } else if (a.bits_k == 3) {
        const int ww = w - W0;
        for (int f = 0; f < 32; ++f) word |= (unsigned)((sm.ck[r][32 * ww + f] >> 2) & 1) << f;
      } else {
        const int ww = w - W0;
        for (int f = 0; f < 16; ++f) word |= (unsigned)((sm.ck[r][16 * ww + f] >> 2) & 3) << (2 * f);
      }
      *(unsigned *)(kb + (size_t)(base + r) * a.kcode_row + 4 * w) = word;
    }
  }

  // 5c. V set words: lane = 16c + m, word t; field f = 4a + e <-> token 16a + 4c + e,
  //     2-bit field at bit 2(f>>1) + 16(f&1), 1-bit field at bit (f>>1) + 8(f&1)
  {
    constexpr int NT = D / 16;
    uint8_t *vb = a.codes_v + bg * a.vcode_bytes + (size_t)set * a.vset_bytes;
    const bool full = (r0 == 0 && r1 == kSet);
    for (int idx = tid; idx < 64 * NT; idx += kThreads) {
      const int lanei = idx / NT, t = idx % NT;
      const int c = lanei / 16, m = lanei % 16;
      const int j = 16 * t + m;
      unsigned w0 = full ? 0u : ((unsigned *)vb)[idx];
      unsigned w1 = 0;
      if (a.bits_v == 4) w1 = full ? 0u : ((unsigned *)(vb + 64 * NT * 4))[idx];
      if (a.bits_v == 3) w1 = full ? 0u : ((unsigned short *)(vb + 64 * NT * 4))[idx];
      for (int f = 0; f < 16; ++f) {
        const int r = 16 * (f / 4) + 4 * c + (f % 4);
        if (r < r0 || r >= r1) continue;
        const unsigned code = sm.cv[r][j];
        const int b2 = 2 * (f >> 1) + 16 * (f & 1), b1 = (f >> 1) + 8 * (f & 1);
        w0 = (w0 & ~(3u << b2)) | ((code & 3u) << b2);
        if (a.bits_v == 3) w1 = (w1 & ~(1u << b1)) | (((code >> 2) & 1u) << b1);
        if (a.bits_v == 4) w1 = (w1 & ~(3u << b2)) | (((code >> 2) & 3u) << b2);
      }
      ((unsigned *)vb)[idx] = w0;
      if (a.bits_v == 4) ((unsigned *)(vb + 64 * NT * 4))[idx] = w1;
      if (a.bits_v == 3) ((unsigned short *)(vb + 64 * NT * 4))[idx] = (unsigned short)w1;
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  const int64_t work = a.n_new * (a.d / 8);
  dim3 grid((unsigned)((work + kThreads - 1) / kThreads), a.B * a.Hkv);
  hipLaunchKernelGGL(append_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_flush(const FlushArgs &a, hipStream_t s) {
  const int64_t s0 = a.u0 / kSet, s1 = (a.u1 + kSet - 1) / kSet;
  dim3 grid((unsigned)(s1 - s0), a.B * a.Hkv);
  if (a.d == 128)
    hipLaunchKernelGGL(flush_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(flush_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace wushkv
