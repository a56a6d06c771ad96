// The forward without a caller-provided workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation). Its workspace lives in a file-scope
// device array of kScratchBytes that every GPU the library runs on holds until
// the process ends; all calls on one GPU share it, so calls on one GPU that
// overlap in time (other streams, other host threads) race.
#include <mutex>

#include "../../include/hstu_attn.h"
#include "internal.h"

namespace {

// Enough for the forward's per-sequence metadata, rebased timestamps and
// work lists of about 3.5 million tokens.
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_scratch[kMaxDevices];     // device address of `scratch` on each device

}  // namespace

// The array itself. In host code its name is only a stand-in for the symbol:
// kernels and copies get the device address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with it current) and kept.
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

hstu_status hstu_attn_fwd_noalloc(const hstu_attn_desc* desc, const int64_t* seq_offsets,
                                  const int64_t* num_targets, const int64_t* timestamps,
                                  const float* rab_pos, const float* rab_time, const void* q,
                                  const void* k, const void* v, const void* u, void* o,
                                  float* a_saved, void* stream) {
  size_t need = 0;
  hstu_status st = hstu_attn_fwd_workspace_size(desc, &need);
  if (st != HSTU_OK) return st;
  if (need > kScratchBytes)
    return (hstu_status)hstu::set_error(HSTU_EWORKSPACE,
                                        "hstu_attn_fwd_noalloc: this shape needs %zu bytes of "
                                        "workspace, above the library's fixed %zu",
                                        need, kScratchBytes);
  void* ws = nullptr;
  if (hipError_t e = scratch_on_current_device(&ws); e != hipSuccess)
    return (hstu_status)hstu::set_error(HSTU_EHIP, "hstu_attn_fwd_noalloc: scratch address: %s",
                                        hipGetErrorString(e));
  return hstu_attn_fwd(desc, seq_offsets, num_targets, timestamps, rab_pos, rab_time, q, k, v, u,
                       o, a_saved, ws, kScratchBytes, stream);
}

}  // extern "C"
