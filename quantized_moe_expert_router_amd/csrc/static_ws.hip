// moeq_moe_layer_noalloc: the whole-layer call for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its workspace is a file-scope device
// array of fixed size instead of a caller buffer.
//
// The array lives in the code object: every GPU the library is loaded on
// holds its own copy, kStaticWsBytes large, until the process ends.  In host
// code `scratch` is only a stand-in symbol; the device address of the
// current GPU's copy comes from hipGetSymbolAddress, looked up once per device
// (on the first call made with that device current) and kept.  Every call on
// a GPU uses that GPU's copy, which keeps the last call's contents: the layer
// kernels ignore workspace contents on entry (everything they read from it
// they wrote earlier in the same call), so nothing needs clearing.  Calls on
// one GPU whose work overlaps in time race on the copy; the caller orders
// them (one stream, or events).
#include <mutex>

#include "../../include/moeq.h"
#include "common.hpp"

namespace {

constexpr size_t kStaticWsBytes = MOEQ_NOALLOC_MAX_BYTES;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kStaticWsBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of this GPU's `scratch`, or nullptr if the lookup failed.
void* scratch_of_device(int dev) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moeq_moe_layer_noalloc(const moeq_route_desc* r, const moeq_ffn_desc* f, const float* x, const float* w_router,
                           const float* bias, double* logits, int32_t* topk_ids, float* topk_w,
                           int32_t* expert_offsets, int32_t* pairs, int32_t* active, const float* shared_scale,
                           float* y, void* stream) {
  const size_t need = moeq_moe_layer_workspace(r, f);
  if (need == 0) return MOEQ_E_INVALID;                 // the descriptors fail the layer call's checks
  if (need > kStaticWsBytes) return MOEQ_E_STATIC_LIMIT;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOEQ_E_HIP;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return MOEQ_E_HIP;
    if ((int)sdev != dev) return MOEQ_E_INVALID;        // the stream must belong to the current device
  }
  void* ws = scratch_of_device(dev);
  if (ws == nullptr) return MOEQ_E_HIP;
  return moeq_moe_layer(r, f, x, w_router, bias, logits, topk_ids, topk_w, expert_offsets, pairs, active,
                        shared_scale, y, ws, kStaticWsBytes, stream);
}

}  // extern "C"
