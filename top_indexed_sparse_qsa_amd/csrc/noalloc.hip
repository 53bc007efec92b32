// Allocation-free variant of qsa_indexer_decode.  For callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc), the decode indexer's workspace -- the
// fp32 score row of each sequence -- comes from a file-scope device array
// that the library holds on every GPU it runs on until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is handed to the kernels.  Every
// call on one GPU uses that GPU's array; calls that overlap on one GPU race.
// The kernels write every score they read in the same call, so the array
// needs no clearing between calls.
#include <hip/hip_runtime.h>

#include <atomic>

#include "libqsa.h"
#include "qsa_launch.h"

namespace {

constexpr size_t kScratchBytes = QSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (nullptr on failure).
// Two threads may both look it up the first time; they store the same value.
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

extern "C" qsa_status qsa_indexer_decode_noalloc(const qsa_indexer_decode_params *p) {
  if (!p) return QSA_ERR_NULL_POINTER;
  qsa_indexer_decode_params q = *p;
  // validate first, against the scratch size, with a stand-in address that
  // passes the alignment check; no HIP call happens before this
  q.workspace = reinterpret_cast<void *>(static_cast<uintptr_t>(256));
  q.workspace_bytes = kScratchBytes;
  if (qsa_status st = qsa::check_indexer_decode(&q)) return st;
  void *ptr = scratch_on_current_device();
  if (ptr == nullptr) return QSA_ERR_LAUNCH;
  q.workspace = ptr;
  return qsa_indexer_decode(&q);
}
