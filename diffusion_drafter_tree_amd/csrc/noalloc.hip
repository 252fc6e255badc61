// dartree_build_round_noalloc: the round with its scratch in a file-scope
// device array instead of a caller workspace, for callers that cannot
// allocate device memory.
//
// The scratch of a round is the scan launch's sorted slice lists, the fp16
// copy of A for the block-decoding tree kernel (16 MiB at 64 requests, K =
// 512; 160 KiB at one request, K = 64) and, when it fits, the split general
// kernel's exchange area (its flags are cleared by the round's scan launch);
// when it does not fit, the round runs the general kernel with one workgroup
// a request, which gives the same bits. Each kernel writes its part of the
// scratch before any kernel reads it, so nothing in it has to start at zero. Every GPU the library runs on holds its own copy of
// the array (kNoAllocScratchBytes) until the process ends; host code reaches
// it only through the address hipGetSymbolAddress gives for that device.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/dartree.h"
#include "api_internal.h"

namespace {

constexpr size_t kNoAllocScratchBytes = DARTREE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// This device's address of `scratch`, looked up once per device (with the
// device current) and kept.
dartree_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  char msg[256];
  if (e != hipSuccess) {
    snprintf(msg, sizeof(msg), "hipGetDevice: %s", hipGetErrorString(e));
    return dartree::set_error(DARTREE_ERR_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(msg, sizeof(msg), "device %d beyond the %d devices the scratch table holds", dev, kMaxDevices);
    return dartree::set_error(DARTREE_ERR_UNSUPPORTED, msg);
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return dartree::set_error(DARTREE_ERR_HIP, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DARTREE_OK;
}

}  // namespace

extern "C" dartree_status dartree_build_round_noalloc(const dartree_dims* dims, const dartree_head* head,
                                                      const void* logits, const void* H_or_h, int32_t* cand_ids,
                                                      float* cand_logit, float* h, dartree_supertree* st,
                                                      int32_t* n_sel, int32_t* tok, int32_t* depth, int32_t* parent,
                                                      float* score, int32_t* slot, uint64_t* mask, void* stream) {
  dartree::set_error(DARTREE_OK, "");
  dartree_status s = dartree::check_round_dims(dims);
  if (s != DARTREE_OK) return s;
  // the split tree kernel's exchange area when it fits, else one workgroup a request
  const bool split = dartree::round_workspace_bytes(dims, true) <= kNoAllocScratchBytes;
  const size_t need = dartree::round_workspace_bytes(dims, split);
  if (need > kNoAllocScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "these sizes need %zu bytes of round scratch; the allocation-free entry point holds %zu "
             "(use dartree_build_round with a workspace)",
             need, kNoAllocScratchBytes);
    return dartree::set_error(DARTREE_ERR_UNSUPPORTED, msg);
  }
  void* ws = nullptr;
  s = scratch_for_current_device(&ws);
  if (s != DARTREE_OK) return s;
  return dartree::build_round_impl(dims, head, logits, H_or_h, cand_ids, cand_logit, h, st, n_sel, tok, depth, parent,
                                   score, slot, mask, ws, kNoAllocScratchBytes, stream, split);
}
