// moe_layer_forward without a caller workspace, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid it).
//
// The workspace is a file-scope device array of kScratchBytes, one copy per
// GPU the library runs on, held until the process ends.  Host code never uses
// the array's name as an address (on the host it is only a stand-in): its
// device address is looked up once per device with that device current
// (hipGetSymbolAddress) and kept in g_scratch; kernels receive that address.
// Calls on one GPU share its array and must not overlap in time.
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <mutex>

#include "launch.h"
#include "moe.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

namespace {

void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch of the current device.  The first time a device's scratch is
// handed out, its status word (the first 4 bytes of any workspace, see
// moe_workspace_init) is cleared by a kernel on `stream`; nothing else in a
// workspace needs to start at zero.
moe_status scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    fprintf(stderr, "libmoe: moe_layer_forward_noalloc: no usable current device\n");
    return MOE_ELAUNCH;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      fprintf(stderr, "libmoe: moe_layer_forward_noalloc: scratch lookup failed: %s\n", hipGetErrorString(e));
      return MOE_ELAUNCH;
    }
    qmoe::clear_last_error();
    if (qmoe::launch_zero_words(static_cast<uint32_t*>(ptr), 1, stream) != hipSuccess) {
      fprintf(stderr, "libmoe: moe_layer_forward_noalloc: clearing the scratch status word failed\n");
      return MOE_ELAUNCH;
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

MOE_API moe_status moe_layer_forward_noalloc(const moe_config* cfg, int32_t T, const void* x_dev,
                                             const float* gate_w_dev, const float* sel_bias_dev,
                                             const void* arena_dev, const void* shared_dev, float* out_dev,
                                             int32_t* topk_ids_out_dev, float* topk_w_out_dev, hipStream_t stream) {
  const moe_status cs = moe_check_config(cfg);
  if (cs != MOE_OK) return cs;
  if (T < 0) return MOE_EUNSUPPORTED;
  const size_t need_bytes = moe_workspace_bytes(cfg, T);
  if (need_bytes == 0) return MOE_EUNSUPPORTED;  // T above the supported maximum
  if (need_bytes > kScratchBytes) {
    fprintf(stderr, "libmoe: moe_layer_forward_noalloc: T=%d needs %zu bytes of scratch, above its %zu\n", (int)T,
            need_bytes, kScratchBytes);
    return MOE_EWORKSPACE;
  }
  if (T == 0) return MOE_OK;
  // the argument rules of moe_layer_forward, checked before anything is enqueued
  auto bad = [](const void* p, bool required) {
    if (!p) return required ? MOE_EINVAL : MOE_OK;
    return (reinterpret_cast<uintptr_t>(p) & 15u) ? MOE_EALIGN : MOE_OK;
  };
  const void* args[] = {x_dev, gate_w_dev, sel_bias_dev, arena_dev, shared_dev, out_dev, topk_ids_out_dev,
                        topk_w_out_dev};
  const bool routed = cfg->n_experts > 0;  // a dense block reads no router weight or arena
  const bool required[] = {true, routed, false, routed, cfg->n_shared != 0, true, false, false};
  for (int i = 0; i < 8; i++) {
    const moe_status s = bad(args[i], required[i]);
    if (s != MOE_OK) return s;
  }
  void* ws = nullptr;
  const moe_status ss = scratch_of_current_device(stream, &ws);
  if (ss != MOE_OK) return ss;
  return moe_layer_forward(cfg, T, x_dev, gate_w_dev, sel_bias_dev, arena_dev, shared_dev, out_dev,
                           topk_ids_out_dev, topk_w_out_dev, ws, kScratchBytes, stream);
}
