// Calibration statistics of WUSH-KV on gfx950: per KV head the second-order sums the
// transforms are built from (WUSH-KV digest, "method key points": the key transform's
// Hessian comes from the query heads that consume the key, sum Q Q^T, and the Gram
// matrices from the keys and values themselves; "takeaways": one calibration pass).
//
//   S_g = sum over rows x of x x^T,  rows = x[b][h][t][:] for every b, t and every h with
//   h / group == g   (group = 1: per-head Gram; group = G: the query heads of KV head g).
//
// A d x d sum over N rows is a contraction over the token axis, so it runs on
// v_mfma_f32_32x32x16_bf16 / _f16 with K = tokens.  Both operands of a 32 x 32 output
// tile (I, J) are "32 channels x 16 tokens" blocks of the same rows, and on this
// instruction A (row = channel) and B (column = channel) have the same lane layout, so
// one block read serves as A of tile (I, .) and B of tile (., I).  S is symmetric: the
// 10 tiles with I <= J of the 4 x 4 tiling at d = 128 are formed, the reduction mirrors them.
//
// Work: a workgroup takes one group (its heads) and a block of batch rows, streams their
// tokens in steps of 64 through LDS, transposed to channel-major on the way in (16-bit
// stores), and writes its 10 tiles as one partial; a second kernel sums a group's
// partials in a fixed order (the result does not depend on timing) and writes the full
// matrix.
#include "wushkv_internal.h"

namespace wushkv {
namespace {

constexpr int kCD = 128;              // head_dim of the MFMA path
constexpr int kStep = 64;             // tokens per LDS stage
constexpr int kPitch = kStep + 8;     // channel row pitch (16-bit elements) in LDS
constexpr int kTiles = 10;            // upper-triangle 32 x 32 tiles of a 128 x 128 sum
constexpr int kCalibThreads = 256;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Tile t of the upper triangle: (0,0) (0,1) (0,2) (0,3) (1,1) (1,2) (1,3) (2,2) (2,3) (3,3).
__host__ __device__ constexpr int tile_i(int t) { return t < 4 ? 0 : (t < 7 ? 1 : (t < 9 ? 2 : 3)); }
__host__ __device__ constexpr int tile_j(int t) {
  return t < 4 ? t : (t < 7 ? t - 3 : (t < 9 ? t - 5 : 3));
}

// One step of 64 rows: thread i takes row i % 64 and its 16-byte chunks (8 channels
// each) i / 64, i / 64 + 4, i / 64 + 8, i / 64 + 12; rows past the end read as zeros.
__device__ __forceinline__ void load_step(const uint8_t *rows, int64_t t0, int64_t T, int tid, u32x4 (&r)[4]) {
  const int64_t t = t0 + (tid & 63);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (u32x4){0u, 0u, 0u, 0u};
    if (t < T) r[i] = __builtin_nontemporal_load((const u32x4 *)(rows + (size_t)t * (kCD * 2)) + (tid >> 6) + 4 * i);
  }
}

// ... stored channel-major, lds[channel][row]: each 16-bit store instruction writes one
// channel of the wave's 64 rows, 128 contiguous bytes (no bank conflicts).
__device__ __forceinline__ void store_step(uint16_t *lds, int tid, const u32x4 (&r)[4]) {
  uint16_t *col = lds + (tid & 63);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch0 = 8 * ((tid >> 6) + 4 * i);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      col[(ch0 + 2 * k) * kPitch] = (uint16_t)(r[i][k] & 0xFFFFu);
      col[(ch0 + 2 * k + 1) * kPitch] = (uint16_t)(r[i][k] >> 16);
    }
  }
}

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// The MFMAs of wave WV on one 16-token chunk: tiles WV, WV + 4, WV + 8 (those below 10),
// with compile-time operand indices (the operands stay in registers).
template <bool BF16, int WV>
__device__ __forceinline__ void wave_tiles(f32x16 (&acc)[3], const u32x4 (&op)[4]) {
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    if (WV + 4 * k < kTiles) acc[k] = mfma32<BF16>(op[tile_i(WV + 4 * k)], op[tile_j(WV + 4 * k)], acc[k]);
  }
}

// Grid (batch blocks, groups): the workgroup sums the rows of its group's heads over its
// batch rows.  Wave w owns tiles w, w + 4, w + 8 (those below 10).
template <bool BF16>
__global__ void __launch_bounds__(kCalibThreads, 2) calib_partial_kernel(CalibArgs a) {
  __shared__ __align__(16) uint16_t stage[2][kCD * kPitch];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bc = blockIdx.x, g = blockIdx.y;
  const int b0 = bc * a.bpw, b1 = b0 + a.bpw < a.B ? b0 + a.bpw : a.B;
  const int64_t steps_per_row = (a.T + kStep - 1) / kStep;
  const int64_t nsteps = (int64_t)(b1 - b0) * a.group * steps_per_row;
  // step s: row block s / steps_per_row = (batch row, head of the group), tokens from
  // (s % steps_per_row) * 64
  auto rows_of = [&](int64_t s) {
    const int64_t hb = s / steps_per_row;
    const int b = b0 + (int)(hb / a.group), h = g * a.group + (int)(hb % a.group);
    return (const uint8_t *)a.x + ((size_t)b * a.H + h) * (size_t)a.T * (kCD * 2);
  };
  constexpr int NT = 3;
  f32x16 acc[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[k][v] = 0.f;

  u32x4 r[4];
  if (nsteps > 0) {
    load_step(rows_of(0), 0, a.T, tid, r);
    store_step(stage[0], tid, r);
  }
  __syncthreads();
  // operand of lane l for channel block I and 16-token chunk kc: channel 32 I + l % 32,
  // tokens 16 kc + 8 (l / 32) .. + 7
  const int orow = lane & 31, ocol = 8 * (lane >> 5);
  for (int64_t s = 0; s < nsteps; ++s) {
    const bool more = s + 1 < nsteps;
    if (more) {
      const int64_t sn = s + 1;
      load_step(rows_of(sn), (sn % steps_per_row) * kStep, a.T, tid, r);
    }
    const uint16_t *st = stage[s & 1];
#pragma unroll
    for (int kc = 0; kc < kStep / 16; ++kc) {
      u32x4 op[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) op[I] = *(const u32x4 *)(st + (32 * I + orow) * kPitch + 16 * kc + ocol);
      switch (wave) {   // wave-uniform
        case 0: wave_tiles<BF16, 0>(acc, op); break;
        case 1: wave_tiles<BF16, 1>(acc, op); break;
        case 2: wave_tiles<BF16, 2>(acc, op); break;
        default: wave_tiles<BF16, 3>(acc, op); break;
      }
    }
    if (more) store_step(stage[(s + 1) & 1], tid, r);
    __syncthreads();
  }
  // partial (g, bc), tile-major 32 x 32 blocks
  float *part = a.partials + ((size_t)g * a.nparts + bc) * (kTiles * 1024);
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    const int t = wave + 4 * k;
    if (t >= kTiles) continue;
    // D layout of the 32 x 32 MFMA: item v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4,
    // column l % 32
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), j = lane & 31;
      part[t * 1024 + i * 32 + j] = acc[k][v];
    }
  }
}

// Grid (groups, tiles, 4): one thread per element of a tile; the group's partials are
// summed in index order and the sum written to the full symmetric matrix (tile (I, J)
// and its mirror).
__global__ void __launch_bounds__(kCalibThreads) calib_reduce_kernel(CalibArgs a) {
  const int g = blockIdx.x, t = blockIdx.y, e = blockIdx.z * kCalibThreads + threadIdx.x;
  const int I = tile_i(t), J = tile_j(t);
  const float *part = a.partials + (size_t)g * a.nparts * (kTiles * 1024) + t * 1024 + e;
  float sum = 0.f;
#pragma unroll 8
  for (int p = 0; p < a.nparts; ++p) sum += part[(size_t)p * (kTiles * 1024)];
  float *out = a.out + (size_t)g * kCD * kCD;
  const int i = 32 * I + e / 32, j = 32 * J + e % 32;
  out[i * kCD + j] = sum;
  if (I != J) out[j * kCD + i] = sum;
}

}  // namespace

// Batch rows per workgroup: enough workgroups for about two rounds of two per CU.
int calib_batch_per_wg(int B, int groups) {
  const int want_blocks = (1024 + groups - 1) / groups;
  const int blocks = want_blocks < B ? want_blocks : B;
  return (B + blocks - 1) / blocks;
}

size_t calib_partial_floats(int B, int H, int group) {
  const int groups = H / group;
  const int bpw = calib_batch_per_wg(B, groups);
  const int nb = (B + bpw - 1) / bpw;
  return (size_t)groups * nb * (kTiles * 1024);
}

hipError_t launch_calib(const CalibArgs &a0, hipStream_t s) {
  CalibArgs a = a0;
  const int nb = (a.B + a.bpw - 1) / a.bpw;
  a.nparts = nb;
  dim3 grid(nb, a.H / a.group);
  if (a.dtype == WUSHKV_DT_BF16) hipLaunchKernelGGL(calib_partial_kernel<true>, grid, dim3(kCalibThreads), 0, s, a);
  else hipLaunchKernelGGL(calib_partial_kernel<false>, grid, dim3(kCalibThreads), 0, s, a);
  hipLaunchKernelGGL(calib_reduce_kernel, dim3(a.H / a.group, kTiles, 1024 / kCalibThreads), dim3(kCalibThreads), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace wushkv
