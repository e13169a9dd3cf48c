// Allocation-free draft block: the pass of dflash_draft_block with its
// workspace in a static device array of the library instead of a caller's
// buffer, for callers that cannot allocate device memory.
//
// The array below is a device symbol. In host code its name stands for a
// host-side shadow, not for device memory, so host code never passes it to a
// kernel or a copy: the device address comes from hipGetSymbolAddress, once per
// device (with that device current), and only that address is used.
#include <dflash.h>
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

static __device__ __align__(256) unsigned char scratch[DFLASH_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of the array, resolved on the
// first call on that device.
dflash_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DFLASH_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DFLASH_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFLASH_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DFLASH_OK;
}

}  // namespace

extern "C" dflash_status dflash_draft_block_noalloc(const dflash_model* m, dflash_kv* kv, const int32_t* anchor,
                                                     int32_t* draft, float* dbg_logits, float* dbg_hidden,
                                                     void* stream) {
  size_t need = 0;
  dflash_status s = dfl::draft_block_check(m, kv, anchor, draft, &need);
  if (s != DFLASH_OK) return s;
  if (need > DFLASH_NOALLOC_SCRATCH_BYTES) return DFLASH_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != DFLASH_OK) return s;
  // the pass reads no workspace byte that it has not written earlier in the
  // same call, so the contents left by an earlier call need no clearing
  return dfl::draft_block_run(m, kv, anchor, draft, dbg_logits, dbg_hidden, ws, DFLASH_NOALLOC_SCRATCH_BYTES,
                              stream, true);
}
