// Generic GQA decode attention over the mixed-precision cache (all shapes the ABI
// accepts).  It favours plain indexing over speed; decode_fast.hip holds the
// MFMA kernel used for the common shapes.
//
// Grid (P + 1, B * Hkv): workgroups 0..P-1 take contiguous ranges of 64-token body
// sets, workgroup P takes the FP16 tokens (sink + recent window).  Each computes
// scores for the G query heads of its KV head (raw q on FP16 keys, q~ = T^{-T} q on
// transformed body keys; WUSH-KV digest, "method key points"), an online softmax
// in the exp2 domain, and the weighted value sum, and writes a partial
// (m, l, o); merge_kernel, launched next on the same stream, combines the P + 1
// partials of each (batch row, query head) in fixed order.
#include "wushkv_internal.h"

namespace wushkv {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxG = 16;
constexpr float kLog2e = 1.4426950408889634f;

struct GenSmem {
  float q[kMaxG][128];
  float qt[kMaxG][128];
  float sq[kMaxG];             // sum of q~ per head
  float s[kMaxG][kSet];        // scores, then probabilities
  float m[kMaxG], l[kMaxG], alpha[kMaxG];
  float pv[kSet][2];           // value parameters of the tile's tokens
};

__device__ __forceinline__ int k_code(const uint8_t *row, int d, int bits, int j) {
  const unsigned *w = (const unsigned *)row;
  int c = (w[j / 16] >> (2 * (j % 16))) & 3;
  if (bits == 3) {   // third bits: channel f of each 32 at bit 4 ((f >> 1) & 7) + (f & 1) + 2 (f >> 4)
    const int f = j % 32;
    c |= ((w[d / 16 + j / 32] >> (4 * ((f >> 1) & 7) + (f & 1) + 2 * (f >> 4))) & 1) << 2;
  }
  if (bits == 4) c |= ((w[d / 16 + j / 16] >> (2 * (j % 16))) & 3) << 2;
  return c;
}

__device__ __forceinline__ int v_code(const uint8_t *set, int d, int bits, int u, int j) {
  const int a = u / 16, c = (u / 4) % 4, e = u % 4;
  const int lane = 16 * c + (j % 16), t = j / 16;
  const int f = 4 * a + e;
  const int b2 = 2 * (f >> 1) + 16 * (f & 1), b1 = (f >> 1) + 8 * (f & 1);
  const int idx = lane * (d / 16) + t;
  int code = (((const unsigned *)set)[idx] >> b2) & 3;
  if (bits == 3) code |= ((((const unsigned short *)(set + 64 * (d / 16) * 4))[idx] >> b1) & 1) << 2;
  if (bits == 4) code |= ((((const unsigned *)(set + 64 * (d / 16) * 4))[idx] >> b2) & 3) << 2;
  return code;
}

__global__ void __launch_bounds__(kThreads) decode_generic_kernel(DecodeArgs a) {
  __shared__ GenSmem sm;  // one partial per workgroup; merge_kernel combines them
  const int tid = threadIdx.x;
  const int part = blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.G, d = a.d;
  const float qk_scale = kLog2e / sqrtf((float)d);
  const int h0 = g * G;  // first query head of this group
  const SeqLen sl = seq_len(a, b);   // this sequence's tokens and body tokens

  for (int i = tid; i < G * d; i += kThreads) {
    const int hh = i / d, j = i % d;
    const size_t off = ((size_t)b * a.Hq + h0 + hh) * d + j;
    sm.q[hh][j] = load_in(a.q, a.q_dtype, off);
    sm.qt[hh][j] = a.qt[off];
  }
  if (tid < G) { sm.m[tid] = -INFINITY; sm.l[tid] = 0.f; }
  __syncthreads();
  if (tid < G) {
    float s = 0.f;
    for (int j = 0; j < d; ++j) s += sm.qt[tid][j];
    sm.sq[tid] = s;
  }

  // token range of this workgroup
  const int64_t nsets = (sl.nq + kSet - 1) / kSet;
  const bool window = (part == a.P);
  int64_t t_begin, t_end;  // body indices, or window list indices
  const int64_t ns = sl.n < a.S ? sl.n : a.S;
  if (!window) {
    t_begin = nsets * part / a.P * kSet;
    t_end = nsets * (part + 1) / a.P * kSet;
    if (t_end > sl.nq) t_end = sl.nq;
  } else {
    t_begin = 0;
    t_end = ns + (sl.n - a.S - sl.nq > 0 ? sl.n - a.S - sl.nq : 0);
  }
  const int Lk = 1 << a.bits_k, Lv = 1 << a.bits_v;
  const _Float16 *sink_k = (const _Float16 *)((const char *)a.sink_k + bg * a.sink_bytes);
  const _Float16 *sink_v = (const _Float16 *)((const char *)a.sink_v + bg * a.sink_bytes);
  const _Float16 *ring_k = (const _Float16 *)((const char *)a.ring_k + bg * a.ring_bytes);
  const _Float16 *ring_v = (const _Float16 *)((const char *)a.ring_v + bg * a.ring_bytes);

  constexpr int kMaxOut = kMaxG * 128 / kThreads;
  float acc[kMaxOut];
#pragma unroll
  for (int i = 0; i < kMaxOut; ++i) acc[i] = 0.f;

  __syncthreads();
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kSet) {
    const int cnt = (int)((t_end - t0) < kSet ? (t_end - t0) : kSet);
    // body: this 64-token set's rows in each plane (t0 is a multiple of 64, and a set
    // lies within one page)
    const uint8_t *kset = nullptr, *vset = nullptr;
    const _Float16 *kpar = nullptr, *vpar = nullptr;
    if (!window) {
      kset = a.codes_k + body_read_offset(a.pg, a.Hkv, a.body_cap, b, g, t0, (int64_t)a.kcode_row);
      vset = a.codes_v + body_read_offset(a.pg, a.Hkv, a.body_cap, b, g, t0, (int64_t)(a.vset_bytes / kSet));
      kpar = (const _Float16 *)((const char *)a.par_k + body_read_offset(a.pg, a.Hkv, a.body_cap, b, g, t0, 2 * a.kpar_n));
      vpar = (const _Float16 *)((const char *)a.par_v + body_read_offset(a.pg, a.Hkv, a.body_cap, b, g, t0, 2 * a.vpar_n));
    }
    // scores: thread (token tt, head group hg)
    {
      const int tt = tid % kSet, hg = tid / kSet;
      if (tt < cnt) {
        const int64_t ti = t0 + tt;
        if (!window) {
          const uint8_t *row = kset + tt * a.kcode_row;
          float kp0 = (float)kpar[tt * a.kpar_n];
          float kp1 = a.kpar_n == 2 ? (float)kpar[tt * a.kpar_n + 1] : 0.f;
          for (int hh = hg; hh < G; hh += kThreads / kSet) {
            float dot = 0.f;
            for (int j = 0; j < d; ++j) dot = fmaf(sm.qt[hh][j], (float)k_code(row, d, a.bits_k, j), dot);
            float sc;
            if (a.quant_k == WUSHKV_Q_QUEST) sc = kp0 * (dot - 0.5f * (Lk - 1) * sm.sq[hh]);
            else sc = kp0 * dot + kp1 * sm.sq[hh];
            sm.s[hh][tt] = sc * qk_scale;
          }
          if (hg == 0) {
            sm.pv[tt][0] = (float)vpar[tt * a.vpar_n];
            sm.pv[tt][1] = a.vpar_n == 2 ? (float)vpar[tt * a.vpar_n + 1] : 0.f;
          }
        } else {
          const int64_t p = ti < ns ? ti : a.S + sl.nq + (ti - ns);
          const _Float16 *krow = p < a.S ? sink_k + p * d : ring_k + ((p - a.S) % (a.R + a.C)) * d;
          for (int hh = hg; hh < G; hh += kThreads / kSet) {
            float dot = 0.f;
            for (int j = 0; j < d; ++j) dot = fmaf(sm.q[hh][j], (float)krow[j], dot);
            sm.s[hh][tt] = dot * qk_scale;
          }
        }
      } else {
        for (int hh = hg; hh < G; hh += kThreads / kSet) sm.s[hh][tt] = -INFINITY;
      }
    }
    __syncthreads();
    if (tid < G) {
      float mx = sm.m[tid];
      for (int t = 0; t < cnt; ++t) mx = fmaxf(mx, sm.s[tid][t]);
      sm.alpha[tid] = __builtin_amdgcn_exp2f(sm.m[tid] - mx);
      sm.m[tid] = mx;
    }
    __syncthreads();
    {
      const int tt = tid % kSet, hg = tid / kSet;
      for (int hh = hg; hh < G; hh += kThreads / kSet)
        sm.s[hh][tt] = tt < cnt ? __builtin_amdgcn_exp2f(sm.s[hh][tt] - sm.m[hh]) : 0.f;
    }
    __syncthreads();
    if (tid < G) {
      float sum = 0.f;
      for (int t = 0; t < cnt; ++t) sum += sm.s[tid][t];
      sm.l[tid] = sm.l[tid] * sm.alpha[tid] + sum;
    }
    // weighted values: thread handles outputs o = tid + k*256 -> (head, channel)
#pragma unroll
    for (int k = 0; k < kMaxOut; ++k) {
      const int o = tid + k * kThreads;
      if (o >= G * d) break;
      const int hh = o / d, j = o % d;
      float s = 0.f;
      for (int t = 0; t < cnt; ++t) {
        const float p = sm.s[hh][t];
        float v;
        if (!window) {
          const int code = v_code(vset, d, a.bits_v, t, j);
          if (a.quant_v == WUSHKV_Q_QUEST) v = ((float)code - 0.5f * (Lv - 1)) * sm.pv[t][0];
          else v = fmaf((float)code, sm.pv[t][0], sm.pv[t][1]);
        } else {
          const int64_t ti = t0 + t;
          const int64_t p = ti < ns ? ti : a.S + sl.nq + (ti - ns);
          const _Float16 *vrow = p < a.S ? sink_v + p * d : ring_v + ((p - a.S) % (a.R + a.C)) * d;
          v = (float)vrow[j];
        }
        s = fmaf(p, v, s);
      }
      acc[k] = acc[k] * sm.alpha[hh] + s;
    }
    __syncthreads();
  }

  // partial out: [B][Hq][P+1][d], (m, l)
  const int P1 = a.P + 1;
#pragma unroll
  for (int k = 0; k < kMaxOut; ++k) {
    const int o = tid + k * kThreads;
    if (o >= G * d) break;
    const int hh = o / d, j = o % d;
    a.part_o[(((size_t)b * a.Hq + h0 + hh) * P1 + part) * d + j] = acc[k];
  }
  if (tid < G) {
    float *ml = a.part_ml + (((size_t)b * a.Hq + h0 + tid) * P1 + part) * 2;
    ml[0] = sm.m[tid];
    ml[1] = sm.l[tid];
  }
}

// Online-softmax merge of the nparts partials (m_p, l_p, o_p) of one (batch row, query
// head) row per workgroup: m* = max m_p, out = sum 2^{m_p - m*} o_p / sum 2^{m_p - m*} l_p
// over the partials with l_p > 0.  Thread (k, c) of the workgroup takes channels
// 4 c .. 4 c + 3 of the k-th of kMergeRanges contiguous ranges of partials, loading them
// all before it sums them in partition order; the ranges' sums are then added in range
// order, so the result does not depend on timing.  Every load is in bounds and
// unconditional (an empty partial's o_p is read but masked), so a range costs about one
// memory latency instead of one per partial.
constexpr int kMergeThreads = 256;
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(DecodeArgs a, int nparts) {
  __shared__ float red[kMergeThreads];
  __shared__ float4 rnum[kMergeThreads];
  __shared__ float rden[kMergeThreads];
  const int tid = threadIdx.x, bh = blockIdx.x;
  const int cpg = a.d / 4, ranges = kMergeThreads / cpg;    // channel quads, partial ranges
  const size_t row = (size_t)bh * (a.P + 1);
  const float2 *ml = reinterpret_cast<const float2 *>(a.part_ml) + row;
  // m*: the largest m_p of a non-empty partial (a max: the order does not matter)
  float mx = -INFINITY;
  for (int p = tid; p < nparts; p += kMergeThreads) {
    const float2 v = ml[p];
    if (v.y > 0.f) mx = fmaxf(mx, v.x);
  }
  red[tid] = mx;
  __syncthreads();
  for (int w = kMergeThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float mstar = red[0];
  const int k = tid / cpg, c = tid % cpg;
  const int p0 = (int)((int64_t)nparts * k / ranges), p1 = (int)((int64_t)nparts * (k + 1) / ranges);
  const float4 *o = reinterpret_cast<const float4 *>(a.part_o + row * a.d) + c;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  {
#pragma unroll 16
    for (int p = p0; p < p1; ++p) {
      const float2 v = ml[p];
      const float4 op = o[(size_t)p * cpg];
      const bool live = v.y > 0.f;
      const float f = live ? __builtin_amdgcn_exp2f(v.x - mstar) : 0.f;
      num.x = fmaf(f, live ? op.x : 0.f, num.x);
      num.y = fmaf(f, live ? op.y : 0.f, num.y);
      num.z = fmaf(f, live ? op.z : 0.f, num.z);
      num.w = fmaf(f, live ? op.w : 0.f, num.w);
      den = fmaf(f, live ? v.y : 0.f, den);
    }
  }
  rnum[tid] = num;
  rden[tid] = den;
  __syncthreads();
  if (tid >= cpg) return;
  float4 n = rnum[tid];
  float dd = rden[tid];
  for (int r = 1; r < ranges; ++r) {
    const float4 x = rnum[r * cpg + tid];
    n.x += x.x; n.y += x.y; n.z += x.z; n.w += x.w;
    dd += rden[r * cpg + tid];
  }
  reinterpret_cast<float4 *>(a.out + (size_t)bh * a.d)[tid] = make_float4(n.x / dd, n.y / dd, n.z / dd, n.w / dd);
}

}  // namespace

hipError_t launch_decode_generic(const DecodeArgs &a, hipStream_t s) {
  dim3 grid(a.P + 1, a.B * a.Hkv);
  hipLaunchKernelGGL(decode_generic_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a0, hipStream_t s) {
  hipError_t e;
  int nparts;
  DecodeArgs a = a0;
  if (a.tinvt && (!decode_fast_supported(a) || a.force_generic)) {
    // the fused query transform only lives in the MFMA kernel: form q~ first here
    QtArgs qa{a.tinvt, a.q, a.qt_out, a.q_dtype, a.B, a.Hq, a.Hkv, a.d};
    if ((e = launch_qtransform(qa, s)) != hipSuccess) return e;
    a.qt = a.qt_out;
    a.tinvt = nullptr;
  }
  if (decode_fast_supported(a) && !a.force_generic) {
    a.P = decode_fast_run_splits(a);   // (the workspace holds the requested count's partials)
    e = launch_decode_fast(a, s);
    if (e != hipSuccess || decode_fast_direct(a)) return e;
    nparts = decode_fast_partials(a);
  } else {
    e = launch_decode_generic(a, s);
    nparts = a.P + 1;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(a.B * a.Hq), dim3(kMergeThreads), 0, s, a, nparts);
  return hipGetLastError();
}

}  // namespace wushkv
