// kvsel_gather_decode_noalloc: kvsel_gather_decode with its scratch memory
// (the (m, s, o) partials of every key split, merged at the end) in a
// fixed-size array of the library's own device memory, for callers that must
// not allocate: code under HIP graph capture, serving loops, harnesses that
// forbid hipMalloc.  The call allocates nothing.  Every call on one GPU shares
// that GPU's array, so calls that overlap on one GPU (different streams, or
// host threads) race; one call at a time per GPU is the contract.  The
// partials are written before they are read, so nothing needs clearing.
#include <mutex>

#include "internal.h"
#include "kvsel.h"

namespace kvsel {
void set_error(const char* fmt, ...);
}

namespace {

constexpr size_t kScratchBytes = size_t{128} << 20;
constexpr int kMaxDevices = 64;

// The scratch array.  In host code this name stands for the array, it is not
// its device address: host code uses the address looked up per device below.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    kvsel::set_error("kvsel_gather_decode_noalloc: no current device");
    return KVSEL_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      kvsel::set_error("kvsel_gather_decode_noalloc: scratch address: %s", hipGetErrorString(e));
      return KVSEL_ERR_HIP;
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return KVSEL_OK;
}

}  // namespace

extern "C" {

size_t kvsel_noalloc_scratch_bytes(void) { return kScratchBytes; }

int kvsel_gather_decode_noalloc(const void* q, int64_t T, int64_t Hq, float scale,
                                const void* k_src, const void* v_src, kvsel_cache kc,
                                int64_t unit_len, const int32_t* idx, int64_t k,
                                int64_t idx_group, void* k_dst, void* v_dst,
                                const kvsel_segment* extra, int32_t n_extra, float* out,
                                float* lse, hipStream_t stream) {
  const size_t need = kvsel_gather_decode_workspace(T, Hq, kc, unit_len, k, extra, n_extra);
  if (need > kScratchBytes) {
    kvsel::set_error("kvsel_gather_decode_noalloc: needs %zu bytes of scratch, the library "
                     "holds %zu", need, kScratchBytes);
    return KVSEL_ERR_WORKSPACE;
  }
  if (stream != nullptr) {  // the scratch is the current device's
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess) {
      (void)hipGetLastError();
      kvsel::set_error("kvsel_gather_decode_noalloc: device of the stream unknown");
      return KVSEL_ERR_HIP;
    }
    if (sdev != cur) {
      kvsel::set_error("kvsel_gather_decode_noalloc: stream on device %d, current device %d",
                       sdev, cur);
      return KVSEL_ERR_UNSUPPORTED;
    }
  }
  void* ws = nullptr;
  const int rc = scratch_ptr(&ws);
  if (rc != KVSEL_OK) return rc;
  return kvsel_gather_decode(q, T, Hq, scale, k_src, v_src, kc, unit_len, idx, k, idx_group,
                             k_dst, v_dst, extra, n_extra, out, lse, ws, kScratchBytes, stream);
}

}  // extern "C"
