// dfa_decode_attn_noalloc: dual-flow decode attention for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops and
// harnesses that forbid hipMalloc). It runs exactly dfa_decode_attn -- the same
// split plan and kernels -- with the split records in a file-scope device
// array instead of a caller workspace.
//
// The array (`scratch`) has a fixed size, DFA_NOALLOC_SCRATCH_BYTES; each GPU
// the library runs on holds its own copy until the process ends. Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in): the first call on a device, with that device current, looks up
// the device address of that device's copy once (hipGetSymbolAddress) and
// keeps it; every call then hands that address to dfa_decode_attn as the
// workspace. Nothing in the array must start at zero: every split writes its
// record (an empty record past the end of its sequence) before the combine
// reads it. Calls that overlap in time on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string>

#include "../../include/dfa.h"
#include "dfa_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[DFA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_init_mu;

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device. A stream of another device is refused: its
// kernels would read this device's copy.
dfa_status scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dfa::report_error(DFA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return dfa::report_error(DFA_ERR_UNSUPPORTED, "device index above 63");
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return dfa::report_error(DFA_ERR_HIP, std::string("hipStreamGetDevice: ") + hipGetErrorString(e));
    if (sdev != dev)
      return dfa::report_error(DFA_ERR_UNSUPPORTED, "dfa_decode_attn_noalloc: the stream belongs to another device "
                                                    "than the current one");
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_init_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return dfa::report_error(DFA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                                  (e != hipSuccess ? hipGetErrorString(e) : "null address"));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return DFA_OK;
}

}  // namespace

extern "C" dfa_status dfa_decode_attn_noalloc(const dfa_attn_desc* desc, const void* q1, const void* q2,
                                              const float* a, const void* k_cache, const void* v_cache,
                                              const int32_t* block_table, const int32_t* ctx_lens, float* o1,
                                              float* o2, void* stream) {
  try {
    int32_t splits = 0;
    const dfa_status valid =
        dfa::attn_host_checks(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens, o1, o2, &splits);
    if (valid != DFA_OK) return valid;
    // one split per sequence: no records, so no workspace
    if (splits == 1)
      return dfa_decode_attn(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens, nullptr, 0, o1, o2, stream);
    const size_t need = dfa_decode_attn_workspace_size(desc);
    if (need > DFA_NOALLOC_SCRATCH_BYTES)
      return dfa::report_error(DFA_ERR_WORKSPACE,
                               "dfa_decode_attn_noalloc: the split records need " + std::to_string(need) +
                                   " bytes, more than the library's fixed scratch of " +
                                   std::to_string(DFA_NOALLOC_SCRATCH_BYTES) +
                                   " bytes; use dfa_decode_attn with a workspace");
    void* ws = nullptr;
    const dfa_status st = scratch_of_current_device(static_cast<hipStream_t>(stream), &ws);
    if (st != DFA_OK) return st;
    return dfa_decode_attn(desc, q1, q2, a, k_cache, v_cache, block_table, ctx_lens, ws, DFA_NOALLOC_SCRATCH_BYTES,
                           o1, o2, stream);
  } catch (...) {
    return dfa::report_error(DFA_ERR_HIP, "unexpected host exception");
  }
}
