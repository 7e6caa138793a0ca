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
// tokens in steps of 64 (loaded two steps ahead into registers) through LDS, transposed to
// channel-major on the way in (16-bit stores), and writes its 10 tiles as one partial; a second kernel sums a group's
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

// LDS holds a step channel-major, lds[channel][token], with the 8-token chunks of a
// channel row permuted: token t of channel c sits at column
//   ((t / 8) xor ((c / 16) mod 8)) * 8 + t mod 8.
// A 16-byte operand read (8 consecutive tokens of one channel) stays contiguous, the 16
// lanes of a read pass (16 consecutive channels) share the permutation and hit distinct
// banks through the row pitch, and the 16-bit stores below (16 channel groups x 4
// tokens per instruction) are spread over all banks by it.
__device__ __forceinline__ int lds_col(int c, int t) { return (((t >> 3) ^ ((c >> 4) & 7)) << 3) | (t & 7); }

// One step of 64 rows, loaded contiguously: 16-byte chunk i of the step's 16 KB goes to
// thread i % 256 (row i / 16, channels 8 (i % 16) .. + 7), so one load instruction reads
// four whole rows.  The loads are unconditional (a row past the end re-reads the last
// row and is zeroed at the store), so the compiler counts the loads in flight exactly
// instead of draining them.
__device__ __forceinline__ void load_step(const uint8_t *rows, int64_t t0, int64_t T, int tid, u32x4 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kCalibThreads * i;
    const int64_t t = t0 + c / 16;
    r[i] = __builtin_nontemporal_load((const u32x4 *)(rows + (size_t)(t < T ? t : T - 1) * (kCD * 2)) + (c % 16));
  }
}

// ... stored channel-major (16-bit stores, element by element).
__device__ __forceinline__ void store_step(uint16_t *lds, int tid, int64_t t0, int64_t T, const u32x4 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kCalibThreads * i;
    const int row = c / 16, ch0 = 8 * (c % 16);
    const bool valid = t0 + row < T;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned w = valid ? r[i][k] : 0u;
      const int c0 = ch0 + 2 * k, c1 = c0 + 1;
      lds[c0 * kPitch + lds_col(c0, row)] = (uint16_t)(w & 0xFFFFu);
      lds[c1 * kPitch + lds_col(c1, row)] = (uint16_t)(w >> 16);
    }
  }
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations complete, then
// s_barrier.  (__syncthreads also waits for every outstanding global load, which would
// drain the prefetched rows at each step.)  The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

  // Rows of step s are loaded into registers during step s - 2 and stored to LDS (stage
  // s % 2) during step s - 1, so every load has two steps of work to land in.  Two
  // register sets alternate; the loop body is written for both orders.
  u32x4 ra[4], rb[4];
  // step s's token offset, and whether this thread's row of it exists
  auto t0_of = [&](int64_t s) { return (s % steps_per_row) * kStep; };
  // a step past the last re-reads the last one (branch-free loads; never stored)
  auto clamp = [&](int64_t s) { return s < nsteps ? s : nsteps - 1; };
  if (nsteps > 0) {
    load_step(rows_of(0), 0, a.T, tid, ra);
    load_step(rows_of(clamp(1)), t0_of(clamp(1)), a.T, tid, rb);
    store_step(stage[0], tid, 0, a.T, ra);
  }
  lds_barrier();
  // operand of lane l for channel block I and 16-token chunk kc: channel 32 I + l % 32,
  // tokens 16 kc + 8 (l / 32) .. + 7
  const int orow = lane & 31, ocol = 8 * (lane >> 5);
  auto step = [&](int64_t s, u32x4 (&rload)[4], u32x4 (&rstore)[4]) {
    const int64_t sl = clamp(s + 2);
    load_step(rows_of(sl), t0_of(sl), a.T, tid, rload);
    const uint16_t *st = stage[s & 1];
#pragma unroll
    for (int kc = 0; kc < kStep / 16; ++kc) {
      u32x4 op[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int c = 32 * I + orow;
        op[I] = *(const u32x4 *)(st + c * kPitch + lds_col(c, 16 * kc + ocol));
      }
      switch (wave) {   // wave-uniform
        case 0: wave_tiles<BF16, 0>(acc, op); break;
        case 1: wave_tiles<BF16, 1>(acc, op); break;
        case 2: wave_tiles<BF16, 2>(acc, op); break;
        default: wave_tiles<BF16, 3>(acc, op); break;
      }
    }
    if (s + 1 < nsteps) store_step(stage[(s + 1) & 1], tid, t0_of(s + 1), a.T, rstore);
    lds_barrier();
  };
  for (int64_t s = 0; s < nsteps; s += 2) {
    step(s, ra, rb);                       // loads step s + 2 into ra, stores step s + 1 from rb
    if (s + 1 < nsteps) step(s + 1, rb, ra);
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
