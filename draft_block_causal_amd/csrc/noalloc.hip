// domino_draft_block_noalloc: the draft call with its scratch in a fixed,
// file-scope device array instead of a caller-provided workspace, for callers
// that cannot allocate device memory (code under stream capture, serving loops
// that forbid allocation).
//
// The array `scratch` is kScratchBytes long and lives on every device the
// library runs on until the process ends.  In host code its name is only a
// stand-in for the symbol, not a device address: the device address is looked
// up once per device with hipGetSymbolAddress (on the entry point's first call
// with that device current) and kept in a per-device table; only that address
// reaches the kernels.  Every call on a device shares the device's array, so
// calls that overlap on one device race; each call's first launch clears the
// words that must start at zero (argmax keys, status and exchange words).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "validate.h"

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;  // covers 32 blocks of a Qwen3-8B-shaped head
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the current device (looked up once per
// device); nullptr and the HIP error on failure.
void* scratch_address(hipError_t& err) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  err = hipGetDevice(&dev);
  if (err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return nullptr;
    if ((reinterpret_cast<uintptr_t>(p) & 255u) != 0) {
      err = hipErrorInvalidValue;
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" int domino_draft_block_noalloc(const domino_head* h, int32_t batch, const void* hidden,
                                          const float* base_logits, const int32_t* x_t, const int32_t* teacher,
                                          float temperature, uint64_t seed, uint32_t offset, int32_t* tokens,
                                          float* logits, float* gru_states, void* stream) {
  int st = domino::check_draft_io(h, batch, hidden, base_logits, x_t, temperature, tokens, logits, gru_states);
  if (st != DOMINO_OK || batch == 0) return st;
  if (domino::workspace_layout(h, batch).total > kScratchBytes) return DOMINO_ERR_UNSUPPORTED;
  hipError_t e = hipSuccess;
  void* ws = scratch_address(e);
  if (!ws) return DOMINO_ERR_HIP;
  return domino::enqueue_draft_block(h, batch, hidden, base_logits, x_t, teacher, temperature, seed, offset, tokens,
                                     logits, gru_states, ws, stream);
}
