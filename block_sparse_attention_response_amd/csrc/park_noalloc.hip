// park_retrieve_blocks_noalloc: park_retrieve_blocks for callers that cannot allocate device
// memory.  Its scratch (the centroid operands of the fused PAMA kernel) lives in a file-scope
// device array, one copy per GPU, instead of a caller workspace; the call allocates nothing.
#include <math.h>

#include <atomic>
#include <mutex>

#include "../../include/park.h"
#include "park_internal.h"

namespace {

// The library's fixed scratch: PARK_NOALLOC_SCRATCH_BYTES on every GPU the library runs on,
// held until the process ends.  In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) unsigned char scratch[PARK_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];
std::mutex scratch_mtx;

// Device address of the current device's copy of `scratch` (looked up on the first call on
// that device, with the device current); nullptr if the lookup fails.
void* device_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(scratch_mtx);
  p = scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" {

size_t park_noalloc_scratch_bytes(int B, int H, int N, int d, int n_clusters) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128) || n_clusters < 1 || n_clusters > N ||
      n_clusters > PARK_MAX_CLUSTERS || (long long)B * H > (1 << 20))
    return 0;
  park::Shape s;
  s.BH = B * H; s.N = N; s.d = d; s.nk = n_clusters; s.dtype = PARK_BF16;
  return park::retrieve_workspace(s, false);
}

int park_retrieve_blocks_noalloc(const void* Q, int dtype, int B, int H, int N, int d, const float* centroids,
                                 const int32_t* counts, int n_clusters, int q_block, float top_p, int top_k,
                                 float scale, float* scores, uint8_t* mask, int32_t* block_list,
                                 int32_t* block_count, void* stream) {
  if (dtype != PARK_F32 && dtype != PARK_BF16) return PARK_ERR_INVALID;
  if (B < 1 || H < 1 || N < 1 || n_clusters < 1 || n_clusters > N) return PARK_ERR_INVALID;
  if (!Q || !centroids || !counts || !scores || !mask || !block_list || !block_count) return PARK_ERR_INVALID;
  if (!isfinite(top_p) || top_p < 0.0f || top_p > 1.0f || top_k < 0 || !isfinite(scale)) return PARK_ERR_INVALID;
  if ((d != 64 && d != 128) || n_clusters > PARK_MAX_CLUSTERS || q_block != PARK_QUERY_BLOCK)
    return PARK_ERR_UNSUPPORTED;
  long long elems = B;
  for (const int f : {H, N, d}) {
    elems *= f;
    if (elems >= (1LL << 31)) return PARK_ERR_UNSUPPORTED;
  }
  park::Shape s;
  s.BH = B * H; s.N = N; s.d = d; s.nk = n_clusters; s.dtype = dtype;
  if (park::retrieve_workspace(s, false) > PARK_NOALLOC_SCRATCH_BYTES) return PARK_ERR_WORKSPACE;
  // the scratch is the current device's: the stream must run on that device
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PARK_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return PARK_ERR_HIP;
    if (sdev != dev) return PARK_ERR_INVALID;
  }
  void* ws = device_scratch(dev);
  if (!ws) return PARK_ERR_HIP;
  if (scale <= 0.0f) scale = 1.0f / sqrtf((float)d);
  const hipError_t e = park::launch_retrieve(s, Q, centroids, counts, scale, top_p, top_k, false, scores, mask,
                                             block_list, block_count, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PARK_OK : PARK_ERR_HIP;
}

}  // extern "C"
