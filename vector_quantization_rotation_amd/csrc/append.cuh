// Decode-step append: the new key and value of one (batch, kv-head) encoded into the cache at position
// seq_len[b], by one work-group of 256 threads, inside the step's query-preparation kernel (so the
// append costs no launch of its own and the attention that follows covers the new token).
//
// Algorithm 1 for the key (or Algorithm 2 for Algorithm-2 keys) and Algorithm 2 for the value, as the
// ai-navigate-news Gemma 4 post assigns them (section "仕組み（技術的）"), one vector at a time: the
// rotations and the QJL projection are fp64 sums of fp32 products (a handful of vectors per step, so
// precision costs nothing here), the cell index counts the boundaries t_k ||x|| below (Pi x)_j, the
// residual is taken in the original domain against n_hat Pi^T c[idx], and the sign is [(S r)_i >= 0].
#pragma once

#include "common.cuh"

namespace tq {

constexpr int APPEND_DMAX = APPEND_DMAX_HOST;  // head dims the append handles
constexpr int APPEND_THREADS = 256;

struct AppendShared {
  double x[APPEND_DMAX], y[APPEND_DMAX], r[APPEND_DMAX];
  double part[APPEND_THREADS / 64][APPEND_DMAX];  // per-wave partial sums of a matrix-vector product
  int idx[APPEND_DMAX];
  uint8_t bits[5][APPEND_DMAX];  // [plane][coordinate]
  double red[APPEND_THREADS / 64];
};

__device__ __forceinline__ double append_block_sum(double v, AppendShared &sh) {
  const int tid = threadIdx.x;
  v = wave_sum_f64(v);
  __syncthreads();  // earlier readers of sh.red are done
  if ((tid & 63) == 0) sh.red[tid >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < APPEND_THREADS / 64; ++w) s += sh.red[w];
  return s;
}

// one pass of append_matvec over NB column blocks of 64 starting at c0: every load is unconditional (the
// block count is uniform), so a batch of RB rows x NB columns is in flight at once
template <int NB>
__device__ inline void append_matvec_pass(const float *A, const double *v, int d, int c0, AppendShared &sh) {
  constexpr int RB = NB <= 2 ? 16 : 8;  // rows per batch (a wave's row count d / 4 is a multiple of 16)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rows = d / 4, r0 = w * rows;
  double acc[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) acc[cb] = 0.0;
  for (int r = r0; r < r0 + rows; r += RB) {
    float a[RB][NB];
#pragma unroll
    for (int u = 0; u < RB; ++u)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) a[u][cb] = A[(int64_t)(r + u) * d + c0 + 64 * cb + lane];
#pragma unroll
    for (int u = 0; u < RB; ++u)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) acc[cb] = fma((double)a[u][cb], v[r + u], acc[cb]);
  }
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) sh.part[w][c0 + 64 * cb + lane] = acc[cb];
}

// y[col] = sum_row A[row d + col] v[row] in fp64 (A a d x d fp32 matrix in global memory, d a multiple of
// 64; v and y in LDS): wave w sums the rows w d/4 .. (w+1) d/4 for every column, each lane 64 columns
// apart, up to four column blocks per pass; the four partial sums are added through LDS.  Ends with a
// barrier.
__device__ inline void append_matvec(const float *A, const double *v, double *y, int d, AppendShared &sh) {
  const int nb = d / 64;
  for (int c0 = 0; c0 < d; c0 += 4 * 64) {
    const int cnt = nb - c0 / 64 < 4 ? nb - c0 / 64 : 4;  // uniform across the work-group
    if (cnt == 1) append_matvec_pass<1>(A, v, d, c0, sh);
    else if (cnt == 2) append_matvec_pass<2>(A, v, d, c0, sh);
    else if (cnt == 3) append_matvec_pass<3>(A, v, d, c0, sh);
    else append_matvec_pass<4>(A, v, d, c0, sh);
  }
  __syncthreads();
  for (int col = threadIdx.x; col < d; col += APPEND_THREADS)
    y[col] = (sh.part[0][col] + sh.part[1][col]) + (sh.part[2][col] + sh.part[3][col]);
  __syncthreads();
}

// one vector (already in sh.x, d coordinates): its plane bits into sh.bits, its fp16 norm and gamma
__device__ inline void append_encode(const AppendSide &sd, int d, AppendShared &sh, uint16_t &nh_out,
                                     uint16_t &gm_out) {
  const int tid = threadIdx.x;
  double ss = 0.0;
  for (int j = tid; j < d; j += APPEND_THREADS) ss = fma(sh.x[j], sh.x[j], ss);
  const double n = sqrt(append_block_sum(ss, sh));
  const int L = 1 << sd.bm;
  // y_j = (Pi x)_j = sum_k Pi^T[k][j] x_k
  append_matvec(sd.piT, sh.x, sh.y, d, sh);
  for (int j = tid; j < d; j += APPEND_THREADS) {
    // idx_j = #{k : t_k n < y_j}; the zero vector compares y = 0 against t_k
    const double yy = n > 0.0 ? sh.y[j] : 0.0, nn = n > 0.0 ? n : 1.0;
    int idx = 0;
    for (int k = 0; k + 1 < L; ++k) idx += (sd.t[k] * nn < yy) ? 1 : 0;
    sh.idx[j] = idx;
    for (int p = 0; p < sd.bm; ++p) sh.bits[p][j] = (uint8_t)((idx >> p) & 1);
  }
  const uint16_t nh = f64_to_f16_rne_sat(n);
  nh_out = nh;
  gm_out = 0;
  if (!sd.prod) return;
  __syncthreads();  // every index is in sh.idx
  const double nhd = (double)f16_to_f32(nh);
  // r = x - n_hat Pi^T c[idx]:  (Pi^T c)_k = sum_j Pi[j][k] c[idx_j]  (c[idx_j] staged in sh.r)
  for (int j = tid; j < d; j += APPEND_THREADS) sh.r[j] = sd.c[sh.idx[j]];
  __syncthreads();
  append_matvec(sd.pi, sh.r, sh.y, d, sh);
  double rs = 0.0;
  for (int k = tid; k < d; k += APPEND_THREADS) {
    const double r = sh.x[k] - nhd * sh.y[k];
    sh.r[k] = r;
    rs = fma(r, r, rs);
  }
  const double rn = sqrt(append_block_sum(rs, sh));  // (the block sum's barriers order the sh.r writes)
  gm_out = f64_to_f16_rne_sat(rn);
  // sign bit i = [(S r)_i >= 0]:  (S r)_i = sum_k S^T[k][i] r_k
  append_matvec(sd.sT, sh.r, sh.y, d, sh);
  for (int i = tid; i < d; i += APPEND_THREADS) sh.bits[sd.bm][i] = sh.y[i] >= 0.0 ? 1 : 0;
}

__device__ inline void append_load(const void *src, int xt, int64_t off, int d, AppendShared &sh) {
  for (int j = threadIdx.x; j < d; j += APPEND_THREADS) {
    float v;
    if (xt == TQ_F32) v = static_cast<const float *>(src)[off + j];
    else if (xt == TQ_BF16) v = bf16_to_f32(static_cast<const uint16_t *>(src)[off + j]);
    else v = f16_to_f32(static_cast<const uint16_t *>(src)[off + j]);
    sh.x[j] = (double)v;
  }
  __syncthreads();
}

// row record of `planes` planes: byte e = bits 8 (e % (d/8)) .. +7 of plane e / (d/8)
__device__ inline void append_write_row(uint8_t *rec, int planes, int d, const AppendShared &sh) {
  const int wb = d / 8;
  for (int e = threadIdx.x; e < planes * wb; e += APPEND_THREADS) {
    const int p = e / wb, j0 = 8 * (e % wb);
    uint32_t byte = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) byte |= (uint32_t)sh.bits[p][j0 + i] << i;
    rec[e] = (uint8_t)byte;
  }
}

// token-tiled words of the sequence: bit (t % 32) of word [t / 32][p][j] set to the plane bit (one
// writer per sequence in a step, so a plain read-modify-write)
__device__ inline void append_write_tiles(uint32_t *seq_tiles, int64_t t, int planes, int d,
                                          const AppendShared &sh) {
  uint32_t *tile = seq_tiles + (t >> 5) * (int64_t)planes * d;
  const uint32_t bit = 1u << (t & 31);
  for (int e = threadIdx.x; e < planes * d; e += APPEND_THREADS) {
    const int p = e / d, j = e % d;
    const uint32_t w = tile[e];
    tile[e] = sh.bits[p][j] ? (w | bit) : (w & ~bit);
  }
}

// the new key (which = 0) or value (which = 1) of (b, g) into the cache at t = seq_len[b] (nothing when
// t is outside [0, Tstride)); the two are encoded by different work-groups of the same launch
__device__ inline void append_token(const AppendArgs &a, int b, int g, int which, AppendShared &sh) {
  const int64_t t = a.seq_len[b];
  if (t < 0 || t >= a.Tstride) return;
  const int d = a.d;
  const int64_t seq = (int64_t)b * a.Hkv + g;
  const int64_t row = seq * a.Tstride + t;
  uint16_t nh, gm;
  if (which == 0) {
    append_load(a.k_new, a.xt, seq * d, d, sh);
    append_encode(a.k, d, sh, nh, gm);
    __syncthreads();
    const int kplanes = a.k.bm + a.k.prod;
    append_write_row(a.kcodes + row * (int64_t)(kplanes * d / 8), kplanes, d, sh);
    if (threadIdx.x == 0) {
      a.knorms[row] = nh;
      if (a.k.prod) a.kgammas[row] = gm;
    }
    return;
  }
  append_load(a.v_new, a.xt, seq * d, d, sh);
  append_encode(a.v, d, sh, nh, gm);
  __syncthreads();
  const int vplanes = a.v.bm + 1;
  if (a.vlayout == TQ_LAYOUT_TILE32) {
    const int64_t ntile = (a.Tstride + 31) / 32;
    append_write_tiles(reinterpret_cast<uint32_t *>(a.vcodes) + seq * ntile * vplanes * d, t, vplanes, d, sh);
  } else {
    append_write_row(a.vcodes + row * (int64_t)(vplanes * d / 8), vplanes, d, sh);
  }
  if (threadIdx.x == 0) {
    a.vnorms[row] = nh;
    a.vgammas[row] = gm;
  }
}

}  // namespace tq
