// gqa_decode_noalloc: gqa_decode with its split partials in a static device
// array instead of a caller workspace, for callers that cannot allocate
// device memory (code under graph capture, tight serving loops).
//
// The array lives in the library's code object, one copy per GPU, for as long
// as the process runs.  Its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and kept; host code only
// ever passes that address on, never the array's own name (in host code the
// name is a host-side stand-in, not a device address).  Every call on a GPU
// uses that GPU's one array: calls that overlap in time on one GPU (two
// streams, two threads) race on it.  gqa_decode reads nothing of its
// workspace that it has not written in the same call, so nothing is cleared.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/gha.h"
#include "kernels.hpp"

namespace {

// 16 MiB: the streaming decode's partials for up to ~1400 (sequence, KV head)
// units at d = 128 and 16 padded rows (the decode workload at batch 64 with
// 8 KV heads needs 6.3 MB)
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // scratch's device address, per device

}  // namespace

extern "C" {

size_t gqa_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

gha_status gqa_decode_noalloc(const gha_tensor* q, const gha_tensor* k_cache, const gha_tensor* v_cache,
                              const int32_t* seqlens_k, const gha_tensor* o, float* lse, int B, int h_q,
                              int h_kv, int s_q, int L_cap, int L_max_hint, int d, gha_dtype in_dtype,
                              gha_dtype out_dtype, float scale, void* stream) {
  // the workspace of the kernel these cache views take
  const size_t need = gha::gqa_decode_path_workspace(k_cache, v_cache, B, h_q, h_kv, s_q, L_cap, L_max_hint, d);
  if (need > kScratchBytes) {
    // the sizes themselves are checked by gqa_decode below (need is 0 for
    // sizes it rejects); here only the scratch limit
    char msg[160];
    snprintf(msg, sizeof(msg), "gqa_decode_noalloc: these sizes need %zu bytes of scratch, above its %zu", need,
             kScratchBytes);
    gha::set_last_error(msg);
    return GHA_ERR_WORKSPACE;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    gha::set_last_error("gqa_decode_noalloc: no usable HIP device");
    return GHA_ERR_HIP;
  }
  void* ptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) {
        char msg[160];
        snprintf(msg, sizeof(msg), "gqa_decode_noalloc: hipGetSymbolAddress failed: %s", hipGetErrorString(e));
        gha::set_last_error(msg);
        return GHA_ERR_HIP;
      }
      g_ptr[dev] = p;
    }
    ptr = g_ptr[dev];
  }
  return gqa_decode(q, k_cache, v_cache, seqlens_k, o, lse, B, h_q, h_kv, s_q, L_cap, L_max_hint, d, in_dtype,
                    out_dtype, scale, ptr, kScratchBytes, stream);
}

}  // extern "C"
