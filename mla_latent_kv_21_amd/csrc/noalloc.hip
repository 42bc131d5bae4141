// mla_decode_noalloc: mla_decode for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The split-K
// partials, log-sum-exps, recompute flags and split plan that mla_decode keeps in the caller's
// workspace live here in one file-scope device array instead, of a fixed size.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address is
// looked up once per device with hipGetSymbolAddress (with that device current) and only that
// address is ever passed to kernels. Each GPU holds its own copy until the process ends. Calls
// on one GPU share its copy, so calls that overlap on one GPU (two streams, two threads) race.
// Nothing in the array has to start at zero: every call's split kernel writes each partial,
// flag and plan entry that its merge then reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

// Device address of the current device's copy of `scratch`, or null (with *err set).
void* scratch_of_current_device(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    g_lookup[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_lookup[dev] == hipSuccess ? p : nullptr;
  });
  *err = g_lookup[dev];
  return g_scratch[dev];
}

}  // namespace

extern "C" mla_status mla_decode_noalloc(const mla_dims* dims, int32_t batch, int32_t s_q,
                                         const void* q_abs, const void* latent_cache,
                                         int32_t num_blocks, const int32_t* block_table,
                                         int32_t max_blocks, const int32_t* seq_lens,
                                         const void* w_uv, int32_t n_split, void* out,
                                         float* lse, hipStream_t stream) {
  // nothing to enqueue, or arguments mla_decode rejects before it looks at a workspace
  if (dims == nullptr || batch <= 0)
    return mla_decode(dims, batch, s_q, q_abs, latent_cache, num_blocks, block_table,
                      max_blocks, seq_lens, w_uv, n_split, nullptr, 0, out, lse, stream);
  // the workspace mla_decode would need; 0 means invalid arguments, which mla_decode itself
  // reports with the matching status before it looks at a workspace
  const size_t need = mla_decode_workspace_bytes(dims, batch, s_q, n_split, max_blocks);
  if (need == 0)
    return mla_decode(dims, batch, s_q, q_abs, latent_cache, num_blocks, block_table,
                      max_blocks, seq_lens, w_uv, n_split, nullptr, 0, out, lse, stream);
  if (need > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  hipError_t e = hipSuccess;
  void* ws = scratch_of_current_device(&e);
  if (ws == nullptr) return MLA_ERR_HIP;
  return mla_decode(dims, batch, s_q, q_abs, latent_cache, num_blocks, block_table, max_blocks,
                    seq_lens, w_uv, n_split, ws, MLA_NOALLOC_SCRATCH_BYTES, out, lse, stream);
}
