// Decode attention that allocates nothing: tq_attn_decode with its workspace in a device array of
// fixed size that the library owns, for callers that cannot allocate device memory.
#include <mutex>

#include "tq_internal.h"

namespace {

// The workspace of every call on a device: query images, per-split partial records and merged rows.
// One copy per GPU (each holds its own), kept until the process ends.
__device__ __align__(256) unsigned char scratch[TQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};  // device address of `scratch` per device (null until the first call there)

// The address of this device's copy of `scratch`.  In host code the array's name is only a stand-in
// for the device symbol, so the address is looked up once per device, with that device current.
int scratch_ptr(int dev, void **out) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return tq::hip_fail(e);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TQ_OK;
}

}  // namespace

extern "C" int tq_attn_decode_noalloc(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B,
                                      int Hq, int Hkv, const uint8_t *kcodes, const uint16_t *knorms,
                                      const uint16_t *kgammas, const uint8_t *vcodes, const uint16_t *vnorms,
                                      const uint16_t *vgammas, int vlayout, int64_t Tstride, const int32_t *seq_len,
                                      float scale, float *out, void *stream) {
  if (!kq || !vq) return TQ_ERR_INVALID;
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return tq::hip_fail(e);
  if (dev != kq->device || dev < 0 || dev >= kMaxDevices) return TQ_ERR_INVALID;
  // the size check comes first: a call that does not fit launches nothing
  if (tq_attn_decode_ws_bytes(kq, B, Hq, Hkv, Tstride, vlayout) > (size_t)TQ_NOALLOC_SCRATCH_BYTES)
    return TQ_ERR_WORKSPACE;
  void *ws = nullptr;
  const int rc = scratch_ptr(dev, &ws);
  if (rc != TQ_OK) return rc;
  return tq_attn_decode(kq, vq, q, qt, B, Hq, Hkv, kcodes, knorms, kgammas, vcodes, vnorms, vgammas, vlayout,
                        Tstride, seq_len, scale, out, ws, (size_t)TQ_NOALLOC_SCRATCH_BYTES, stream);
}
