// ttt_layer_forward_noalloc: the layer's prefill with its workspace in a
// static device array instead of a caller buffer, for callers that cannot
// allocate device memory (code under graph capture, serving loops that
// forbid hipMalloc). Contract in include/ttt.h.
//
// `scratch` lives in the library's code object: the loader reserves it on
// every device the library runs on, for the life of the process. In host
// code its name is only a stand-in for the symbol, not a device address, so
// the host never passes it to a kernel or copy: the device address of each
// GPU's copy is looked up once per device with hipGetSymbolAddress (with
// that device current) and kept.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>
#include <vector>

#include "ttt.h"

namespace {

constexpr size_t kScratchBytes = TTT_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // by device ordinal; null until looked up

// The device address of the current device's copy of `scratch`, looked up on
// the first call on that device. Returns null (and the HIP error in *err) if
// the lookup fails.
void* scratch_for_current_device(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

// Records the reason of a failure in the library's thread-local error
// record (ttt_last_error) and returns s; defined in ttt_api.cpp.
namespace tttk_api {
ttt_status set_error(ttt_status s, const std::string& msg);
}

extern "C" {

ttt_status ttt_layer_forward_noalloc(const ttt_desc* desc, const void* H, const void* X0,
                                     const void* Wg, const void* Wu, const void* W_down0,
                                     const void* conv_taps, const void* W_target, float eta,
                                     int32_t chunk, void* O, float* W_down_final, void* stream) {
  size_t need = 0;
  const ttt_status st = ttt_workspace_size(desc, chunk, &need);
  if (st != TTT_OK) return st;
  if (need > kScratchBytes)
    return tttk_api::set_error(
        TTT_ERR_WORKSPACE,
        "this problem needs " + std::to_string(need) + " bytes of workspace; the static scratch "
        "of ttt_layer_forward_noalloc holds " + std::to_string(kScratchBytes) +
        " (call ttt_layer_forward with a caller workspace instead)");
  hipError_t err = hipSuccess;
  void* ws = scratch_for_current_device(&err);
  if (ws == nullptr)
    return tttk_api::set_error(TTT_ERR_HIP, std::string("looking up the static scratch: ") +
                                                hipGetErrorString(err));
  return ttt_layer_forward(desc, H, X0, Wg, Wu, W_down0, conv_taps, W_target, eta, chunk, O,
                           W_down_final, ws, kScratchBytes, stream);
}

}  // extern "C"
