// noalloc.hip -- sanatan_prefill_chunked_noalloc: the chunked prefill with its workspace in a fixed device
// array of the library instead of a caller buffer, for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ object: every GPU the library runs on holds its own copy, at its own
// address, for the life of the process.  In host code the name `scratch` is only a host-side stand-in, so it
// is never passed to a kernel; its device address is looked up once per device with hipGetSymbolAddress
// (that device current) and kept in a per-device table.  The prefill writes every workspace byte it reads
// (the position table, then each piece's boundary state before any other piece reads it), so the array
// needs no clearing between calls.  Calls on one GPU share the array: calls that overlap in time on that
// GPU (different streams, or threads without ordering) race on it.
#include <mutex>

#include "launchers.h"
#include "sanatan.h"
#include "sanatan_device.h"

namespace sanatan {

// 48 MiB: enough for the prefill of 96 sequences of 2048 tokens, or of 12 sequences of 32768 tokens, at one
// workgroup per compute unit on a 256-CU device.
constexpr size_t kNoallocScratchBytes = (size_t)48 << 20;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of this device's scratch array (looked up on the first call on each device); null on error.
static void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

size_t noalloc_scratch_bytes() { return kNoallocScratchBytes; }

void* noalloc_scratch() { return device_scratch(); }

}  // namespace sanatan
