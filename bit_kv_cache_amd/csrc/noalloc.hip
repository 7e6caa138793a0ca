// wushkv_decode_attention_noalloc: the decode with its split-K partials in a fixed
// device array of this library instead of a caller workspace, for callers that cannot
// allocate device memory (code under graph capture, serving loops that forbid it).
//
// The array is a file-scope __device__ symbol.  Its host-side name is only a stand-in
// for the device address, so each device's address is looked up once, with that device
// current, through hipGetSymbolAddress, and only that address is ever handed to a
// kernel.  Each GPU holds its own copy of the array until the process ends.
#include <mutex>

#include "wushkv_internal.h"

namespace wushkv {
namespace {

// Maximum partials the array holds: fp32 [batch][num_q_heads][splits + 1][head_dim + 2],
// e.g. 8 sequences x 64 query heads x 129 partitions at head_dim 128 (34.3 MB).
constexpr size_t kScratchBytes = WUSHKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // per device: the array's device address, once looked up

// The device the call's work runs on: the stream's, or the current one for the null stream.
int stream_device(void *stream, int *dev) {
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = s ? hipStreamGetDevice(s, dev) : hipGetDevice(dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return WUSHKV_ERR_HIP;
  }
  return (*dev >= 0 && *dev < kMaxDevices) ? WUSHKV_OK : WUSHKV_ERR_UNSUPPORTED;
}

// Device address of `scratch` on `dev`: hipGetSymbolAddress with that device current,
// on the first call for the device, then the kept value.
int scratch_address(int dev, void **ptr) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
      (void)hipGetLastError();
      return WUSHKV_ERR_HIP;
    }
    if (cur != dev && hipSetDevice(dev) != hipSuccess) {
      (void)hipGetLastError();
      return WUSHKV_ERR_HIP;
    }
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return WUSHKV_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return WUSHKV_OK;
}

}  // namespace
}  // namespace wushkv

extern "C" {

int wushkv_decode_attention_noalloc(const wushkv_cache *c, int64_t n_tokens, const void *q, int32_t q_dtype,
                                    const float *q_t, int32_t num_q_heads, int32_t num_splits, float *out,
                                    void *stream) {
  using namespace wushkv;
  // every argument check first, on the host, with a stand-in workspace of the array's size
  const size_t need = wushkv_decode_workspace_bytes(c, n_tokens, num_q_heads, num_splits);
  if (need > kScratchBytes) return WUSHKV_ERR_WORKSPACE;
  int st = decode_attention_checked(c, n_tokens, q, q_dtype, q_t, num_q_heads, num_splits,
                                    reinterpret_cast<void *>((uintptr_t)256), kScratchBytes, out, stream, true);
  if (st != WUSHKV_OK) return st;
  int dev = 0;
  if ((st = stream_device(stream, &dev)) != WUSHKV_OK) return st;
  void *ptr = nullptr;
  if ((st = scratch_address(dev, &ptr)) != WUSHKV_OK) return st;
  // the partials need no clearing: the merge reads only slots this call writes
  return decode_attention_checked(c, n_tokens, q, q_dtype, q_t, num_q_heads, num_splits, ptr, kScratchBytes, out,
                                  stream, false);
}

}  // extern "C"
