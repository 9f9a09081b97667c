// The decode step for callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid device allocation): paged_decode_step with its workspace -- the
// split-K partials and the vector engine's q copy -- in a file-scope device array instead of a
// caller buffer.  Each device holds its own copy of the array, from the first call on that device
// until the process ends; host code reaches it only through the address hipGetSymbolAddress gives
// for the current device (the array's name on the host is a stand-in, not a device address).
#include "../../include/kvq.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kernels.hpp"

static_assert(KVQ_NOALLOC_WORKSPACE_BYTES % 256 == 0, "whole 256-byte units");

static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};          // scratch's device address, per device

// scratch's address on the current device, looked up once per device; nullptr with the error set
void* device_scratch(int* code) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    char buf[160];
    snprintf(buf, sizeof buf, "paged_decode_step_noalloc: no usable current device (%s)",
             e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
    *code = kvq::set_error(KVQ_ERR_HIP, buf);
    return nullptr;
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      char buf[160];
      snprintf(buf, sizeof buf, "paged_decode_step_noalloc: hipGetSymbolAddress of the scratch array: %s",
               hipGetErrorString(e));
      *code = kvq::set_error(KVQ_ERR_HIP, buf);
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int paged_decode_step_noalloc(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                                         kvq_pool* pool, const int32_t* block_table, const int32_t* lengths,
                                         float scale, const kvq_decode_shape* shape, void* out, void* stream) {
  // the size check first: a shape that does not fit is refused before the device is touched
  const size_t need = paged_decode_workspace_bytes(pool, shape);
  if (need == 0)   // invalid shape: the checks of the allocating entry point report it
    return paged_decode_step(q, k_new, v_new, pool, block_table, lengths, scale, shape, nullptr, 0, out, stream);
  if (need > KVQ_NOALLOC_WORKSPACE_BYTES) {
    char buf[200];
    snprintf(buf, sizeof buf,
             "paged_decode_step_noalloc: this shape needs %zu bytes of workspace; the built-in scratch holds %zu "
             "(KVQ_NOALLOC_WORKSPACE_BYTES)", need, (size_t)KVQ_NOALLOC_WORKSPACE_BYTES);
    return kvq::set_error(KVQ_ERR_WORKSPACE, buf);
  }
  if (!q || !k_new || !v_new || !block_table || !lengths || !out)
    return kvq::set_error(KVQ_ERR_INVALID, "paged_decode_step_noalloc: q, k_new, v_new, block_table, lengths and "
                                           "out must be device pointers");
  int code = KVQ_OK;
  void* ws = device_scratch(&code);
  if (!ws) return code;
  return paged_decode_step(q, k_new, v_new, pool, block_table, lengths, scale, shape, ws,
                           (size_t)KVQ_NOALLOC_WORKSPACE_BYTES, out, stream);
}
