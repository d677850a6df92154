// Internal declarations shared by the host entry points and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

constexpr int kMaxCentroids = 16;  // 4-bit Algorithm-1 codebook at most

// Codebook passed to kernels by value (kernel-argument memory).
struct Codebook {
  int L;                          // number of centroids (2^bmse)
  float c[kMaxCentroids];         // ascending centroids (unit-sphere coordinate domain)
  float t[kMaxCentroids - 1];     // boundaries (midpoints)
};

constexpr int APPEND_DMAX_HOST = 512;  // head dims the decode-step append handles

// Decode-step append (the new token's key and value encoded into the cache by the step's query
// preparation kernel): one side (key or value) of the encoding.
struct AppendSide {
  int bm;            // index bits (0 for the 1-bit sign mode)
  int prod;          // Algorithm 2: a sign plane and a gamma follow the index planes
  const float *piT;  // Pi^T (y = Pi x reads it column-wise, coalesced)
  const float *pi;   // Pi (z = Pi^T c reads it column-wise)
  const float *sT;   // S^T (Algorithm 2)
  double t[kMaxCentroids - 1];
  double c[kMaxCentroids];
};

// everything the append reads and writes
struct AppendArgs {
  int on;                      // 0: a plain decode step
  const void *k_new, *v_new;   // [B, Hkv, d] of type xt
  int xt, d, Hkv;
  int vlayout;                 // TQ_LAYOUT_ROWS or TQ_LAYOUT_TILE32
  int64_t Tstride;
  const int32_t *seq_len;      // position of the new token (tokens already cached)
  uint8_t *kcodes;
  uint16_t *knorms, *kgammas;  // kgammas for Algorithm-2 keys
  uint8_t *vcodes;             // rows, or uint32 tile words (TQ_LAYOUT_TILE32)
  uint16_t *vnorms, *vgammas;
  AppendSide k, v;
};

}  // namespace tq

struct tq_quantizer {
  int d;
  int bits;        // bits per coordinate of a record (incl. the sign bit for TQ_PROD)
  int mode;        // TQ_MSE / TQ_PROD
  int bmse;        // bits of the Algorithm-1 index (bits or bits-1)
  int planes;      // bit planes per record
  size_t code_bytes;
  int device;
  double c64[tq::kMaxCentroids];
  double t64[tq::kMaxCentroids - 1];
  tq::Codebook cb;
  float qjl_scale;  // sqrt(pi/2)/d
  // device fp32 d*d row-major matrices
  float *pi = nullptr;   // Pi
  float *piT = nullptr;  // Pi^T
  float *s = nullptr;    // S            (TQ_PROD)
  float *sT = nullptr;   // S^T          (TQ_PROD)
  float *m = nullptr;    // S Pi^T       (TQ_PROD): S r = M (Pi x - n_hat c[idx]) up to Pi's fp32 orthogonality
  // bf16 pieces [3][d][d] (hi, mid, lo; exact splits of the fp32 entries) for the bf16 matrix cores
  uint16_t *pi3 = nullptr;  // of Pi
  uint16_t *m3 = nullptr;   // of S Pi^T (TQ_PROD)
  uint16_t *pit3 = nullptr; // of Pi^T (decode, head dims up to 128)
  uint16_t *st3 = nullptr;  // of S^T (decode, TQ_PROD, head dims up to 128)
  // fp16 pieces [2][d][d] (hi, lo) of Pi 2^kp (head dims up to 512) and S Pi^T 2^km (up to 128) for bf16 /
  // fp16 rows; the exponents put the largest entry (Pi) or a bound on it (S Pi^T) just under 2^14
  uint16_t *pih = nullptr;
  uint16_t *mh = nullptr;
  int kp = 0, km = 0;
};

namespace tq {

// optional event timing of launches (profile.cpp)
bool profiling();
void *prof_begin(const char *name, hipStream_t st);
void prof_end(void *tok, hipStream_t st);
// events that the launch itself stamps (hipExtLaunchKernel): they time the dispatch alone, not the packets
// around it; both null when the name is not recorded
void prof_kernel_events(const char *name, hipEvent_t *start, hipEvent_t *stop);
struct ProfKernel {
  hipEvent_t start, stop;
  explicit ProfKernel(const char *name) { prof_kernel_events(name, &start, &stop); }
};
struct ProfScope {
  void *tok;
  hipStream_t st;
  ProfScope(const char *name, hipStream_t s) : tok(prof_begin(name, s)), st(s) {}
  ~ProfScope() { prof_end(tok, st); }
};

// status helpers (tq_host.cpp)
int hip_fail(hipError_t e);
int launch_check();

// kernel launchers (defined in the .hip files); all return a tq_status
int run_encode(const tq_quantizer *q, const void *x, int xt, int64_t n, int64_t ldx, uint8_t *codes,
               uint16_t *norms, uint16_t *gammas, hipStream_t st);
int run_decode(const tq_quantizer *q, const uint8_t *codes, const uint16_t *norms, const uint16_t *gammas,
               int64_t n, float *out, int64_t ldo, hipStream_t st);
size_t score_ws_bytes(const tq_quantizer *q, int64_t m, int64_t n, int k);
int run_score(const tq_quantizer *q, const float *queries, int64_t m, int64_t ldq, const uint8_t *codes,
              const uint16_t *norms, const uint16_t *gammas, int64_t n, int k, float *scores, int64_t *idx,
              void *ws, size_t ws_bytes, hipStream_t st);
size_t attn_ws_bytes(const tq_quantizer *kq, int B, int Hq, int Hkv, int64_t Tstride, int vlayout);
int run_attn_decode(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int Hq,
                    int Hkv, const uint8_t *kcodes, const uint16_t *knorms, const uint16_t *kgammas,
                    const uint8_t *vcodes, const uint16_t *vnorms, const uint16_t *vgammas, int vlayout,
                    int64_t Tstride, const int32_t *seq_len, float scale, float *out, void *ws, size_t ws_bytes,
                    const AppendArgs *app, hipStream_t st);
size_t attn_prefill_ws_bytes(const tq_quantizer *kq, int B, int M, int Hq, int Hkv, int64_t Tstride, int vlayout);
int run_attn_prefill(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int M, int Hq,
                     int Hkv, const uint8_t *kcodes, const uint16_t *knorms, const uint16_t *kgammas,
                     const uint8_t *vcodes, const uint16_t *vnorms, const uint16_t *vgammas, int vlayout,
                     int64_t Tstride, const int32_t *q_pos, float scale, float *out, void *ws, hipStream_t st);
int run_tile_records(const tq_quantizer *q, const uint8_t *codes, int64_t nseq, int64_t T, uint32_t *tiles,
                     hipStream_t st);
int make_pieces(const float *src, int64_t n, uint16_t *dst, hipStream_t st);
int make_pieces_f16(const float *src, int64_t n, int k, uint16_t *dst, hipStream_t st);
bool encode_fused_supported(const tq_quantizer *q);
int run_encode_fused(const tq_quantizer *q, const void *x, int xt, int64_t n, int64_t ldx, uint8_t *codes,
                     uint16_t *norms, uint16_t *gammas, hipStream_t st);
// encode into a cache: nseq x T rows of x to positions t0.. of each sequence (layout TQ_LAYOUT_ROWS:
// records [nseq][Tstride][code_bytes]; TQ_LAYOUT_TILE32: words [nseq][ceil(Tstride/32)][planes][d])
int run_encode_fused_cache(const tq_quantizer *q, const void *x, int xt, int64_t nseq, int64_t T, int64_t ldx,
                           int64_t t0, int64_t Tstride, int layout, void *codes, uint16_t *norms, uint16_t *gammas,
                           hipStream_t st);
int run_encode_cache(const tq_quantizer *q, const void *x, int xt, int64_t nseq, int64_t T, int64_t ldx, int64_t t0,
                     int64_t Tstride, int layout, void *codes, uint16_t *norms, uint16_t *gammas, hipStream_t st);
int run_tile_records_at(const tq_quantizer *q, const uint8_t *codes, int64_t nseq, int64_t T, int64_t toff,
                        int64_t ntile_dst, uint32_t *tiles, hipStream_t st);
int compute_sPiT(int d, const float *s, const float *pi, float *m, hipStream_t st);
int rotate_back(const float *merged, int64_t rows, int d, const float *piT, const float *sT, float *out, bool split1,
                hipStream_t st);
int device_cus();  // compute units of the current device (cached)
bool decode_fused_supported(const tq_quantizer *q);
int run_decode_fused(const tq_quantizer *q, const uint8_t *codes, const uint16_t *norms, const uint16_t *gammas,
                     int64_t n, float *out, int64_t ldo, hipStream_t st);
// Walsh coefficients beta_S of a symmetric 2^bits-level codebook over the odd-size subsets of the index
// bits (enumeration order of walsh_planes): c[idx] = sum_S beta_S prod_{p in S} (2 bit_p - 1)
void walsh_coeffs(const double *c, int bits, double *beta);

}  // namespace tq
