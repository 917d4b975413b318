// fi_noalloc.hip -- paged decode for callers that cannot allocate device
// memory: the plan's int32 sections and its fp32 partial states live in one
// static device array of this library instead of a caller workspace.
//
// The array, `scratch`, is a file-scope __device__ object: each GPU the
// library runs on holds its own copy, at its own address, from the first call
// on that GPU until the process ends. Host code never passes the array's name
// to a kernel (on the host it is a stand-in, not a device address); the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and is what the kernels, the copy and the merge get.
// Every call on a GPU reuses that GPU's array and leaves the last call's
// contents there: calls that overlap on one GPU (two streams, or two threads)
// race on it. Each call uploads every plan section the kernels read (the
// fused merge's arrival counts among them, as zeros), and the attention
// kernel writes every partial row before it is merged, both ordered on the
// call's stream.

#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

#include "fi_host.h"

namespace {

constexpr size_t kScratchBytes = (size_t)FI_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch array, looked up on the
// first call on that device.
fi_status scratch_for_current_device(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fi::set_error(FI_ERR_HIP, "fi_paged_decode_noalloc: hipGetDevice: %s",
                         hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fi::set_error(FI_ERR_UNSUPPORTED, "fi_paged_decode_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fi::set_error(FI_ERR_HIP, "fi_paged_decode_noalloc: scratch address: %s",
                           hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = (char*)g_scratch_ptr[dev];
  return FI_OK;
}

}  // namespace

extern "C" fi_status fi_paged_decode_noalloc(const fi_plan_t* p, const void* q,
                                             const void* k_cache, const void* v_cache,
                                             const int32_t* kv_indices, float sm_scale, void* o,
                                             float* lse, void* stream) {
  using namespace fi;
  clear_error();
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return set_error(FI_ERR_INVALID_ARG,
                     "fi_paged_decode_noalloc: sm_scale must be finite and > 0, got %g",
                     (double)sm_scale);
  if (!p) return set_error(FI_ERR_PLAN_MISMATCH, "fi_paged_decode_noalloc: plan is NULL");
  if (p->hp.desc.kind != FI_KIND_DECODE)
    return set_error(FI_ERR_PLAN_MISMATCH, "fi_paged_decode_noalloc: plan was built for kind %d",
                     p->hp.desc.kind);
  if (p->on_device || p->host_blob.size() != p->lay.blob_bytes)
    return set_error(FI_ERR_PLAN_MISMATCH,
                     "fi_paged_decode_noalloc: needs a host-only plan (built without a device "
                     "workspace)");
  if (p->lay.dev_bytes > kScratchBytes)
    return set_error(FI_ERR_WORKSPACE,
                     "fi_paged_decode_noalloc: the plan needs %zu bytes of device workspace, "
                     "the static scratch holds %zu",
                     p->lay.dev_bytes, kScratchBytes);
  if (p->hp.desc.batch > 0 && (!q || !k_cache || !v_cache || !kv_indices || !o))
    return set_error(FI_ERR_INVALID_ARG, "fi_paged_decode_noalloc: NULL tensor pointer");
  char* base = nullptr;
  fi_status st = scratch_for_current_device(&base);
  if (st != FI_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(base, p->host_blob.data(), p->lay.blob_bytes,
                                hipMemcpyHostToDevice, s);
  if (e != hipSuccess)
    return set_error(FI_ERR_HIP, "fi_paged_decode_noalloc: plan upload: %s",
                     hipGetErrorString(e));
  const AttnArgs a =
      plan_attn_args(p, base, 0, q, k_cache, v_cache, kv_indices, nullptr, sm_scale, o, lse);
  TimerScope t(s);
  e = plan_launch_level(p, 0, a, s);
  t.done();
  if (e != hipSuccess)
    return set_error(FI_ERR_HIP, "fi_paged_decode_noalloc: attention launch: %s",
                     hipGetErrorString(e));
  if (!p->hp.fused) e = plan_launch_merge(p, base, o, lse, s);
  if (e != hipSuccess)
    return set_error(FI_ERR_HIP, "fi_paged_decode_noalloc: merge launch: %s",
                     hipGetErrorString(e));
  return FI_OK;
}
