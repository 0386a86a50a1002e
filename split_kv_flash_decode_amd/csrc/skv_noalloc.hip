// The allocation-free split-KV call: skv_attention_decode_paged_splitkv with
// its partial records in a static device buffer of the library instead of
// caller-owned buffers, for callers that cannot allocate device memory.
//
// The buffer is a file-scope __device__ array; each GPU the library runs on
// holds its own copy at its own address. Host code never uses the array's
// name as an address (on the host that name is only a stand-in): the first
// call on a device, with that device current, asks the runtime for the
// device address once (hipGetSymbolAddress) and keeps it per device; the
// kernels receive that address exactly as they receive caller buffers.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "skv.h"
#include "skv_internal.h"

namespace {

constexpr size_t kScratchBytes = SKV_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, once looked up

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Device address of this device's scratch (looked up on its first use).
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SKV_ERR_LAUNCH;
  std::lock_guard<std::mutex> hold(g_lock);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();   // leave no error behind for the next launch check
      return SKV_ERR_LAUNCH;
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SKV_OK;
}

}  // namespace

extern "C" int skv_attention_decode_paged_splitkv_noalloc(const skv_desc* d, const skv_args* a,
                                                          int32_t num_splits, void* stream) {
  int rc = skv::check_split_call(d, a, 1, num_splits);
  if (rc) return rc;
  const int64_t slots = skv_uniform_slots(d, num_splits);
  size_t mb = 0, lb = 0, ab = 0;
  rc = skv_workspace_size(d, slots, &mb, &lb, &ab);
  if (rc) return rc;
  const size_t m_off = 0, l_off = round256(mb), acc_off = l_off + round256(lb);
  if (acc_off + round256(ab) > kScratchBytes) return SKV_ERR_SCRATCH;
  void* base = nullptr;
  rc = scratch_on_current_device(&base);
  if (rc) return rc;
  char* c = static_cast<char*>(base);
  skv_partials p;
  p.m = reinterpret_cast<float*>(c + m_off);
  p.l = reinterpret_cast<float*>(c + l_off);
  p.acc = c + acc_off;
  p.capacity_slots = slots;
  return skv_attention_decode_paged_splitkv(d, a, num_splits, &p, stream);
}
