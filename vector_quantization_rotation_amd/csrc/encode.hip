// Host side of the fused encode (kernels in encode.cuh): the bf16 pieces of the
// per-shape matrices, the supported shapes and the dispatch.
#include "encode.cuh"

namespace tq {

// pieces [3][d][d] of a fp32 matrix (piece-major, rows unchanged): exact split as in encode.cuh
__global__ void split3_kernel(const float *src, int64_t n, uint16_t *dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float p[3];
  split_exact<3>(src[i], p);
  dst[i] = (uint16_t)(__float_as_uint(p[0]) >> 16);
  dst[n + i] = (uint16_t)(__float_as_uint(p[1]) >> 16);
  dst[2 * n + i] = (uint16_t)(__float_as_uint(p[2]) >> 16);
}

int make_pieces(const float *src, int64_t n, uint16_t *dst, hipStream_t st) {
  hipLaunchKernelGGL(split3_kernel, dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st, src, n, dst);
  return launch_check();
}

// pieces [2][n] of src 2^k as fp16 hi + lo, each rounded to nearest (|src| 2^k below 2^14)
__global__ void split2h_kernel(const float *src, int64_t n, int k, uint16_t *dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  split_f16(__builtin_amdgcn_ldexpf(src[i], k), dst[i], dst[n + i]);
}

int make_pieces_f16(const float *src, int64_t n, int k, uint16_t *dst, hipStream_t st) {
  hipLaunchKernelGGL(split2h_kernel, dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st, src, n, k, dst);
  return launch_check();
}

// compute units of the current device (cached per device)
int device_cus() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] > 0) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  cache[dev] = cus;
  return cus;
}

bool encode_fused_supported(const tq_quantizer *q) {
  return (q->d == 64 || q->d == 128) && q->pi3 && q->pih && q->bmse >= 1 && q->bmse <= 4 &&
         (q->mode != TQ_PROD || (q->m3 && q->mh));
}

int run_encode_fused(const tq_quantizer *q, const void *x, int xt, int64_t n, int64_t ldx, uint8_t *codes,
                     uint16_t *norms, uint16_t *gammas, hipStream_t st) {
  return run_encode_fused_cache(q, x, xt, 1, n, ldx, 0, n, TQ_LAYOUT_ROWS, codes, norms, gammas, st);
}

int run_encode_fused_cache(const tq_quantizer *q, const void *x, int xt, int64_t nseq, int64_t T, int64_t ldx,
                           int64_t t0, int64_t Tstride, int layout, void *codes, uint16_t *norms, uint16_t *gammas,
                           hipStream_t st) {
  if (nseq == 0 || T == 0) return TQ_OK;
  EncArgs ea{};
  ea.x = x; ea.ldx = ldx; ea.T = T; ea.tps = cdiv64(T, EB); ea.ntiles = nseq * ea.tps; ea.t0 = t0;
  ea.Tstride = Tstride; ea.pi3 = q->pi3; ea.m3 = q->m3;
  ea.pih = q->pih; ea.mh = q->mh; ea.kp = q->kp; ea.km = q->km;
  if (layout == TQ_LAYOUT_TILE32) ea.tiles = static_cast<uint32_t *>(codes);
  else ea.codes = static_cast<uint8_t *>(codes);
  ea.code_bytes = (int64_t)q->code_bytes; ea.ntile32 = cdiv64(Tstride, 32);
  ea.norms = norms; ea.gammas = gammas; ea.cb = q->cb;
  ProfScope ps(q->mode == TQ_PROD ? "encode_prod" : "encode_mse", st);
  if (q->mode == TQ_PROD) launch_encode_prod(xt, q->d, q->bmse, ea, st);
  else launch_encode_mse(xt, q->d, q->bmse, ea, st);
  return launch_check();
}

}  // namespace tq
