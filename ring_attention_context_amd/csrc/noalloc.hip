// ra_ring_fwd_noalloc: the ring forward of ra_ring_fwd for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation). Its workspace is a file-scope device
// array of RA_NOALLOC_SCRATCH_BYTES that every call on a GPU shares; the
// chunk transfers run on the caller's one stream (RA_RING_SERIALIZE), so no
// second stream and no event is needed either.
#include <mutex>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr size_t SCRATCH_BYTES = RA_NOALLOC_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;

// Each GPU the library runs on holds its own copy until the process ends. In
// host code `scratch` names a host-side stand-in, not a device address: only
// the pointer hipGetSymbolAddress returns for the current device is used.
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex scratch_mu;
void *scratch_dev[MAX_DEVICES] = {};

// Device address of `scratch` on the current device, looked up once per device.
ra_status scratch_ptr(void **out) {
  int dev = 0;
  ra_status st = hip_check(hipGetDevice(&dev), "ra_ring_fwd_noalloc: hipGetDevice");
  if (st != RA_OK) return st;
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(RA_ERR_UNSUPPORTED, "ra_ring_fwd_noalloc: device %d beyond %d", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void *p = nullptr;
    st = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                   "ra_ring_fwd_noalloc: hipGetSymbolAddress(scratch)");
    if (st != RA_OK) return st;
    if (!p) return fail(RA_ERR_HIP, "ra_ring_fwd_noalloc: no device address for the scratch");
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return RA_OK;
}

}  // namespace
}  // namespace ra

extern "C" ra_status ra_ring_fwd_noalloc(const ra_ring_desc *desc, const void *q,
                                         const void *k_chunks, const void *v_chunks, float *o,
                                         float *lse, void *stream) {
  ra::clear_error();
  size_t need = 0;
  ra_status st = ra_ring_workspace_bytes(desc, &need);
  if (st != RA_OK) return st;
  if (need > ra::SCRATCH_BYTES)
    return ra::fail(RA_ERR_INVALID_ARG,
                    "ra_ring_fwd_noalloc: this ring needs %zu bytes of workspace; the static "
                    "scratch holds %zu (use ra_ring_fwd with a caller workspace)",
                    need, ra::SCRATCH_BYTES);
  void *ws = nullptr;
  st = ra::scratch_ptr(&ws);
  if (st != RA_OK) return st;
  // The same call as ra_ring_fwd with the scratch as workspace and the copies
  // on the compute stream. The ring writes every workspace byte it reads
  // before reading it, so nothing needs clearing between calls.
  return ra_ring_fwd(desc, q, k_chunks, v_chunks, o, lse, ws, ra::SCRATCH_BYTES, stream, stream);
}
