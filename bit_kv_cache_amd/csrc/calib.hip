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
// Work: a workgroup takes one group (its heads) and a block of batch rows (about one
// resident round of workgroups in all), streams their tokens in steps of 64 (loaded two
// steps ahead into registers) through LDS, transposed to channel-major on the way in
// (16-bit stores); each of its four waves forms all 10 tiles over its own 16 tokens of a
// step, and the waves' sums are added into one partial.  A second kernel sums a group's
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
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
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

// One step of 64 rows: thread t takes rows 4 (t / 16) .. + 3 and the 16-byte chunk t mod 16
// of each (channels 8 (t mod 16) .. + 7), so one load instruction reads four whole rows.
// The loads are unconditional (a row past the end re-reads the last row, which the
// cache still holds, and is zeroed at the store), so the compiler counts the loads in
// flight exactly instead of draining them.
__device__ __forceinline__ void load_step(const uint8_t *rows, int64_t t0, int64_t T, int tid, u32x4 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + 4 * (tid >> 4) + i;
    r[i] = *((const u32x4 *)(rows + (size_t)(t < T ? t : T - 1) * (kCD * 2)) + (tid & 15));
  }
}

// ... stored channel-major: for each of its 8 channels the thread packs its four
// consecutive tokens into 8 bytes (two byte permutes) and writes them with one 64-bit
// store, which stays inside one 8-token chunk of the permuted row.
__device__ __forceinline__ void store_step(uint16_t *lds, int tid, int64_t t0, int64_t T, const u32x4 (&r)[4]) {
  const int tq = 4 * (tid >> 4), ch0 = 8 * (tid & 15);
  u32x4 x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool valid = t0 + tq + i < T;
    x[i] = valid ? r[i] : (u32x4){0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const unsigned sel = (m & 1) ? 0x07060302u : 0x05040100u;   // the high or low halves
    const unsigned lo = __builtin_amdgcn_perm(x[1][m >> 1], x[0][m >> 1], sel);
    const unsigned hi = __builtin_amdgcn_perm(x[3][m >> 1], x[2][m >> 1], sel);
    const int c = ch0 + m;
    *(u32x2 *)(lds + c * kPitch + lds_col(c, tq)) = (u32x2){lo, hi};
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

// Grid (batch blocks, groups): the workgroup sums the rows of its group's heads over its
// batch rows.  Wave w takes tokens 16 w .. 16 w + 15 of every step for all 10 tiles, so
// each staged element is read from LDS once; the four waves' sums are added in wave
// order at the end.
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
  f32x16 acc[kTiles];
#pragma unroll
  for (int k = 0; k < kTiles; ++k)
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
  // operand of lane l for channel block I: channel 32 I + l % 32, tokens
  // 16 wave + 8 (l / 32) .. + 7 of the step
  const int orow = lane & 31, ocol = 16 * wave + 8 * (lane >> 5);
  auto step = [&](int64_t s, u32x4 (&rload)[4], u32x4 (&rstore)[4]) {
    const int64_t sl = clamp(s + 2);
    load_step(rows_of(sl), t0_of(sl), a.T, tid, rload);
    const uint16_t *st = stage[s & 1];
    u32x4 op[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const int c = 32 * I + orow;
      op[I] = *(const u32x4 *)(st + c * kPitch + lds_col(c, ocol));
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t) acc[t] = mfma32<BF16>(op[tile_i(t)], op[tile_j(t)], acc[t]);
    if (s + 1 < nsteps) store_step(stage[(s + 1) & 1], tid, t0_of(s + 1), a.T, rstore);
    lds_barrier();
  };
  for (int64_t s = 0; s < nsteps; s += 2) {
    step(s, ra, rb);                       // loads step s + 2 into ra, stores step s + 1 from rb
    if (s + 1 < nsteps) step(s + 1, rb, ra);
  }
  // partial (g, bc): the 10 tiles, each 1024 floats in the MFMA's D order (item v of
  // lane l at v * 64 + l).  The waves' sums are added in wave order through LDS, two
  // tiles at a time (the last step's barrier has retired every operand read).
  float *red = reinterpret_cast<float *>(&stage[0][0]);   // [2 tiles][4 waves][1024]
  float *part = a.partials + ((size_t)g * a.nparts + bc) * (kTiles * 1024);
#pragma unroll
  for (int t0 = 0; t0 < kTiles; t0 += 2) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((tt * 4 + wave) * 16 + v) * 64 + lane] = acc[t0 + tt][v];
    lds_barrier();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = 4 * tid + 1024 * k;                   // 4 consecutive elements of tile t0 + k
      const float4 *r = reinterpret_cast<const float4 *>(red + k * 4096 + (e & 1023));
      const float4 sum = ((r[0] + r[256]) + r[512]) + r[768];
      *reinterpret_cast<float4 *>(part + (t0 + k) * 1024 + (e & 1023)) = sum;
    }
    lds_barrier();
  }
}

// Grid (groups, tiles, 4): a workgroup sums 256 elements of one tile over the group's
// partials.  Wave q takes 4 consecutive elements per lane over the q-th quarter of the
// partials, in index order; the quarters are then added in order q = 0, 1, 2, 3 (the
// result does not depend on timing) and written to the full symmetric matrix (tile
// (I, J) and its mirror).
__global__ void __launch_bounds__(kCalibThreads) calib_reduce_kernel(CalibArgs a) {
  __shared__ float4 quarter[3][64];
  const int g = blockIdx.x, t = blockIdx.y, lane = threadIdx.x & 63;
  const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e4 = blockIdx.z * 64 + lane;            // float4 index within the tile
  const int per = (a.nparts + 3) / 4;
  const int p0 = q * per, p1 = p0 + per < a.nparts ? p0 + per : a.nparts;
  const float4 *part = (const float4 *)(a.partials + (size_t)g * a.nparts * (kTiles * 1024) + t * 1024) + e4;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int p = p0; p < p1; ++p) sum += part[(size_t)p * (kTiles * 256)];
  if (q > 0) quarter[q - 1][lane] = sum;
  __syncthreads();
  if (q != 0) return;
  sum = ((sum + quarter[0][lane]) + quarter[1][lane]) + quarter[2][lane];
  // element 4 e4 of the tile in D order: item v = e / 64 of lane l = e % 64 is row
  // 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32 (the four elements are columns j .. j + 3)
  const int I = tile_i(t), J = tile_j(t);
  float *out = a.out + (size_t)g * kCD * kCD;
  const int v = (4 * e4) >> 6, l = (4 * e4) & 63;
  const int i = 32 * I + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3), j = 32 * J + (l & 31);
  *(float4 *)(out + i * kCD + j) = sum;
  if (I != J) {
    out[(j + 0) * kCD + i] = sum.x;
    out[(j + 1) * kCD + i] = sum.y;
    out[(j + 2) * kCD + i] = sum.z;
    out[(j + 3) * kCD + i] = sum.w;
  }
}

}  // namespace

// Batch rows per workgroup: about one round of two workgroups per CU (256 CUs), so
// that each workgroup streams many steps and the group has few partials to sum.
constexpr int kCalibTargetBlocks = 512;
int calib_batch_per_wg(int B, int groups) {
  const int want_blocks = (kCalibTargetBlocks + groups - 1) / groups;
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
