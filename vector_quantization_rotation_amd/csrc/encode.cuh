// Fused encode for head dims 64 and 128 on the bf16 matrix cores.
//
// Algorithm 1 (TurboQuant_mse) and Algorithm 2 (TurboQuant_prod) as on the
// ai-navigate-news Gemma 4 post, section "仕組み（技術的）": the norm, the
// rotation y = Pi x, the Lloyd-Max cell index of every coordinate packed into
// bit planes, and for Algorithm 2 the residual (taken in the rotated domain,
// r_rot = y - n_hat c[idx]), the signs of S r = (S Pi^T) r_rot and ||r||.
//
// Precision: the codes are compared against the fp64 definition with a tie zone
// of 1e-5 of the coordinate scale, so the contractions must be fp32-accurate.
// Every operand is split exactly into bf16 pieces (truncation: hi keeps the top
// 8 significant bits, mid the next 8, lo the rest, so x = hi + mid + lo holds
// exactly for fp32, x = hi + lo for fp16, and bf16 is one piece).  Products of
// pieces are exact in fp32, so the result carries fp32 accumulation error only:
//   bf16 x:  x Pi_hi + x Pi_mid + x Pi_lo                              (3 MFMAs)
//   fp16 x:  x_hi (Pi_hi + Pi_mid + Pi_lo) + x_lo (Pi_hi + Pi_mid)      (5 MFMAs)
//   fp32 a:  a_hi b_hi + a_hi b_mid + a_mid b_hi + a_hi b_lo +
//            a_lo b_hi + a_mid b_mid                                    (6 MFMAs)
// (the dropped cross terms are below 2^-23 of the product).
//
// Work split.  A persistent work-group of NW waves (4; 8 for Algorithm 2 at
// d = 128) walks 64-row tiles.  Wave w owns output columns [w d/NW, (w+1) d/NW):
// its pieces of Pi (and of S Pi^T) stay in registers for the whole launch, so
// the matrices cross L2 once per work-group.  The row tile is staged whole in
// LDS (NW threads per row, fp64 norm on the way, the next tile's loads in
// flight behind the contraction).
// The quantizer runs with lane = row over the wave's own columns: the cell index
// is a binary search over the scaled boundaries, its bits are shifted into one
// 32-bit word per plane (add-with-carry, no cross-lane traffic), and the words
// go straight to the record.  The Algorithm 2 residual is split into its pieces
// once, in LDS, as the operand of the second contraction; its squared norm is
// accumulated in fp32 (the fp16 gamma tolerates 1e-5 relative), the vector norm
// in fp64 (the fp16 norm must round exactly as the fp64 value does).
#pragma once

#include "common.cuh"

namespace tq {

constexpr int EB = 64;  // rows per tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct EncArgs {
  const void *x;
  int64_t ldx, n, ntiles;
  const uint16_t *pi3;  // [3][D][D] pieces of Pi (row j, column k)
  const uint16_t *m3;   // [3][D][D] pieces of S Pi^T (Algorithm 2)
  uint8_t *codes;
  int64_t code_bytes;
  uint16_t *norms, *gammas;
  Codebook cb;
};

template <int XT>
struct EncIn {
  static constexpr int NPA = XT == TQ_BF16 ? 1 : (XT == TQ_F16 ? 2 : 3);  // bf16 pieces per element
  static constexpr int ESZ = XT == TQ_F32 ? 4 : 2;
};

// 16-byte alignment lets every fragment access be one ds_read/ds_write_b128 (8 lanes a cycle, conflict-free
// at the padded strides below) instead of b64 pairs (16 lanes a cycle, two-way conflicts)
// waves per work-group: Algorithm 2 at d = 128 splits the columns over 8 waves (16 each), which halves
// the register-resident matrix pieces and lets two waves share each SIMD (one wave's quantizer overlaps
// the other's matrix-core work); otherwise 4 waves
__host__ __device__ constexpr int enc_waves(int D, bool PROD) { return PROD && D == 128 ? 8 : 4; }

template <int D, int NPA, bool PROD>
struct __attribute__((aligned(16))) EncLds {
  static constexpr int NW = enc_waves(D, PROD);
  static constexpr int CW = D / NW;
  uint16_t a[NPA][EB][D + 8];          // row pieces of the tile
  float cw[NW][EB][CW + 4];            // per-wave transpose: MFMA layout -> lane = row
  uint16_t rp[PROD ? 3 : 1][PROD ? EB : 1][D + 16];  // residual pieces (Algorithm 2; this stride measured 5 % faster than D + 8)
  float gpart[PROD ? NW : 1][EB];      // per-wave partial ||r||^2
  float n32[2][EB], nh[2][EB];         // norms by tile parity
};

__device__ __forceinline__ float trunc_bf16(float x) { return __uint_as_float(__float_as_uint(x) & 0xFFFF0000u); }

// exact pieces of x (see the header): p[0] + p[1] + p[2] == x
template <int NP>
__device__ __forceinline__ void split_exact(float x, float (&p)[3]) {
  p[0] = trunc_bf16(x);
  const float r1 = x - p[0];
  if (NP == 2) {
    p[1] = r1;
    p[2] = 0.f;
  } else {
    p[1] = trunc_bf16(r1);
    p[2] = r1 - p[1];
  }
}

// upper halves (bf16 bits) of two exact-bf16 floats into one dword: lo element first
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// the exact-piece products (A piece, B piece), smallest terms first
template <int NPA>
struct PieceTerms;
template <>
struct PieceTerms<1> {
  static constexpr int N = 3;
  static constexpr int A[N] = {0, 0, 0}, B[N] = {2, 1, 0};
};
template <>
struct PieceTerms<2> {
  static constexpr int N = 5;
  static constexpr int A[N] = {1, 0, 1, 0, 0}, B[N] = {1, 2, 0, 1, 0};
};
template <>
struct PieceTerms<3> {
  static constexpr int N = 6;
  static constexpr int A[N] = {1, 2, 0, 1, 0, 0}, B[N] = {1, 0, 2, 0, 1, 0};
};

// acc[rt][ct] += A rows (16 rt ..) x B columns (16 ct ..) over one 32-deep k-step,
// term-major so that consecutive MFMAs write different accumulators
template <int NPA, int NCT>
__device__ __forceinline__ void contract_kstep(const bf16x8 (&af)[4][3], const bf16x8 (&bf)[NCT][3],
                                               floatx4 (&acc)[4][NCT]) {
  using TT = PieceTerms<NPA>;
#pragma unroll
  for (int t = 0; t < TT::N; ++t)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = mfma_bf16(af[rt][TT::A[t]], bf[ct][TT::B[t]], acc[rt][ct]);
}

// all of this work-group's LDS traffic done, then the work-group meets (no wait on global loads)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// keeps the compiler from moving LDS accesses across (the LDS runs one wave's accesses in order)
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

// Lloyd-Max cell index idx = #{k : t_k n < y} of one coordinate by binary
// search over the scaled boundaries T[k-1] = t_k n (non-decreasing in k), its
// bits shifted into the plane words (P[s] = 2 P[s] + bit s of idx, columns
// visited high to low) and, for Algorithm 2, the centroid c[idx] selected on the
// way.  Each level compares against the one boundary its decided bits leave,
// then narrows every lower level's candidates (and the centroids) by that bit;
// the compare mask lives in VCC only, and add-with-carry does the shift.
template <int BM, bool CENT>
__device__ __forceinline__ void quant_coord(float y, const float (&T)[(1 << BM) - 1], const float (&C)[1 << BM],
                                            uint32_t (&P)[BM], float &cv) {
  if constexpr (BM == 1) {
    if constexpr (CENT) {
      asm volatile(
          "v_cmp_gt_f32_e32 vcc, %[y], %[t0]\n\t"
          "v_cndmask_b32_e32 %[cv], %[c0], %[c1], vcc\n\t"
          "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
          : [p0] "+v"(P[0]), [cv] "=&v"(cv)
          : [y] "v"(y), [t0] "v"(T[0]), [c0] "v"(C[0]), [c1] "v"(C[1])
          : "vcc");
    } else {
      asm volatile(
          "v_cmp_gt_f32_e32 vcc, %[y], %[t0]\n\t"
          "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
          : [p0] "+v"(P[0])
          : [y] "v"(y), [t0] "v"(T[0])
          : "vcc");
    }
  } else if constexpr (BM == 2) {
    float th;
    if constexpr (CENT) {
      float ca, cb;
      asm volatile(
          "v_cmp_gt_f32_e32 vcc, %[y], %[t1]\n\t"
          "v_cndmask_b32_e32 %[th], %[t0], %[t2], vcc\n\t"
          "v_cndmask_b32_e32 %[ca], %[c0], %[c2], vcc\n\t"
          "v_cndmask_b32_e32 %[cb], %[c1], %[c3], vcc\n\t"
          "v_addc_co_u32_e32 %[p1], vcc, %[p1], %[p1], vcc\n\t"
          "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
          "v_cndmask_b32_e32 %[cv], %[ca], %[cb], vcc\n\t"
          "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
          : [p0] "+v"(P[0]), [p1] "+v"(P[1]), [th] "=&v"(th), [ca] "=&v"(ca), [cb] "=&v"(cb), [cv] "=&v"(cv)
          : [y] "v"(y), [t0] "v"(T[0]), [t1] "v"(T[1]), [t2] "v"(T[2]), [c0] "v"(C[0]), [c1] "v"(C[1]),
            [c2] "v"(C[2]), [c3] "v"(C[3])
          : "vcc");
    } else {
      asm volatile(
          "v_cmp_gt_f32_e32 vcc, %[y], %[t1]\n\t"
          "v_cndmask_b32_e32 %[th], %[t0], %[t2], vcc\n\t"
          "v_addc_co_u32_e32 %[p1], vcc, %[p1], %[p1], vcc\n\t"
          "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
          "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
          : [p0] "+v"(P[0]), [p1] "+v"(P[1]), [th] "=&v"(th)
          : [y] "v"(y), [t0] "v"(T[0]), [t1] "v"(T[1]), [t2] "v"(T[2])
          : "vcc");
    }
  } else if constexpr (BM == 3) {
    float th, ta, tb;
    asm volatile(
        "v_cmp_gt_f32_e32 vcc, %[y], %[t3]\n\t"
        "v_cndmask_b32_e32 %[th], %[t1], %[t5], vcc\n\t"
        "v_cndmask_b32_e32 %[ta], %[t0], %[t4], vcc\n\t"
        "v_cndmask_b32_e32 %[tb], %[t2], %[t6], vcc\n\t"
        "v_addc_co_u32_e32 %[p2], vcc, %[p2], %[p2], vcc\n\t"
        "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
        "v_cndmask_b32_e32 %[th], %[ta], %[tb], vcc\n\t"
        "v_addc_co_u32_e32 %[p1], vcc, %[p1], %[p1], vcc\n\t"
        "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
        "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
        : [p0] "+v"(P[0]), [p1] "+v"(P[1]), [p2] "+v"(P[2]), [th] "=&v"(th), [ta] "=&v"(ta), [tb] "=&v"(tb)
        : [y] "v"(y), [t0] "v"(T[0]), [t1] "v"(T[1]), [t2] "v"(T[2]), [t3] "v"(T[3]), [t4] "v"(T[4]),
          [t5] "v"(T[5]), [t6] "v"(T[6])
        : "vcc");
    if constexpr (CENT) {
      // c[idx] from the finished words' low bits (idx = 4 b2 + 2 b1 + b0)
      const int idx = (int)((P[0] & 1u) | ((P[1] & 1u) << 1) | ((P[2] & 1u) << 2));
      float v = C[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) v = idx == i ? C[i] : v;
      cv = v;
    }
  } else {
    static_assert(BM == 4 && !CENT, "4-bit cells: Algorithm 1 only");
    float th, u0, u1, w0, w1, w2, w3;
    asm volatile(
        "v_cmp_gt_f32_e32 vcc, %[y], %[t7]\n\t"
        "v_cndmask_b32_e32 %[th], %[t3], %[t11], vcc\n\t"
        "v_cndmask_b32_e32 %[u0], %[t1], %[t9], vcc\n\t"
        "v_cndmask_b32_e32 %[u1], %[t5], %[t13], vcc\n\t"
        "v_cndmask_b32_e32 %[w0], %[t0], %[t8], vcc\n\t"
        "v_cndmask_b32_e32 %[w1], %[t2], %[t10], vcc\n\t"
        "v_cndmask_b32_e32 %[w2], %[t4], %[t12], vcc\n\t"
        "v_cndmask_b32_e32 %[w3], %[t6], %[t14], vcc\n\t"
        "v_addc_co_u32_e32 %[p3], vcc, %[p3], %[p3], vcc\n\t"
        "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
        "v_cndmask_b32_e32 %[th], %[u0], %[u1], vcc\n\t"
        "v_cndmask_b32_e32 %[w0], %[w0], %[w2], vcc\n\t"
        "v_cndmask_b32_e32 %[w1], %[w1], %[w3], vcc\n\t"
        "v_addc_co_u32_e32 %[p2], vcc, %[p2], %[p2], vcc\n\t"
        "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
        "v_cndmask_b32_e32 %[th], %[w0], %[w1], vcc\n\t"
        "v_addc_co_u32_e32 %[p1], vcc, %[p1], %[p1], vcc\n\t"
        "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
        "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
        : [p0] "+v"(P[0]), [p1] "+v"(P[1]), [p2] "+v"(P[2]), [p3] "+v"(P[3]), [th] "=&v"(th), [u0] "=&v"(u0),
          [u1] "=&v"(u1), [w0] "=&v"(w0), [w1] "=&v"(w1), [w2] "=&v"(w2), [w3] "=&v"(w3)
        : [y] "v"(y), [t0] "v"(T[0]), [t1] "v"(T[1]), [t2] "v"(T[2]), [t3] "v"(T[3]), [t4] "v"(T[4]),
          [t5] "v"(T[5]), [t6] "v"(T[6]), [t7] "v"(T[7]), [t8] "v"(T[8]), [t9] "v"(T[9]), [t10] "v"(T[10]),
          [t11] "v"(T[11]), [t12] "v"(T[12]), [t13] "v"(T[13]), [t14] "v"(T[14])
        : "vcc");
  }
}

// w = 2 w + b: the next-lower column's bit shifted in (columns visited high to low)
__device__ __forceinline__ uint32_t shift_in(uint32_t w, bool b) { return (w << 1) | (b ? 1u : 0u); }

template <int XT, int D, bool PROD, int BM>
__global__ __launch_bounds__(enc_waves(D, PROD) * 64) void encode_kernel(EncArgs a) {
  constexpr int NPA = EncIn<XT>::NPA, ESZ = EncIn<XT>::ESZ;
  constexpr int NW = enc_waves(D, PROD);
  constexpr int CW = D / NW;       // columns per wave
  constexpr int NCT = CW / 16;     // 16-column MFMA tiles per wave
  constexpr int NKS = D / 32;      // 32-deep k-steps
  constexpr int L = 1 << BM;
  constexpr int PER = D / NW;      // staged elements per thread (NW threads per row)
  constexpr int RAW = PER * ESZ / 16;
  static_assert(RAW >= 1, "tile staging");
  __shared__ EncLds<D, NPA, PROD> sh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j16 = lane & 15, g4 = lane >> 4;

  // ---- register-resident matrix pieces of this wave's columns ----
  bf16x8 bpi[NKS][NCT][3];
  bf16x8 bmq[PROD ? NKS : 1][NCT][3];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const int64_t off = ((int64_t)p * D + CW * wave + 16 * ct + j16) * D + 32 * ks + 8 * g4;
        bpi[ks][ct][p] = *reinterpret_cast<const bf16x8 *>(a.pi3 + off);
        if (PROD) bmq[ks][ct][p] = *reinterpret_cast<const bf16x8 *>(a.m3 + off);
      }
  float tb[L - 1], cc[L];
#pragma unroll
  for (int k = 0; k < L - 1; ++k) tb[k] = a.cb.t[k];
#pragma unroll
  for (int k = 0; k < L; ++k) cc[k] = a.cb.c[k];

  // ---- staging geometry: row sr, elements [sk, sk + PER) ----
  const int sr = tid / NW, sk = (tid % NW) * PER;
  uint4 raw[RAW];
  auto load_raw = [&](int64_t tile) {
    const int64_t row = tile * EB + sr;
    if (row < a.n) {
      const uint4 *src =
          reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(a.x) + (row * a.ldx + sk) * ESZ);
#pragma unroll
      for (int i = 0; i < RAW; ++i) raw[i] = src[i];
    } else {
#pragma unroll
      for (int i = 0; i < RAW; ++i) raw[i] = uint4{0u, 0u, 0u, 0u};
    }
  };

  int64_t tile = blockIdx.x;
  if (tile < a.ntiles) load_raw(tile);
  for (int it = 0; tile < a.ntiles; ++it, tile += gridDim.x) {
    const int64_t row0 = tile * EB;
    const int rows = (int)imin64(EB, a.n - row0);
    const int buf = it & 1;

    // ---- stage the tile: pieces into LDS, fp64 norm ----
    {
      float v[PER];
#pragma unroll
      for (int i = 0; i < RAW; ++i) {
        const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (XT == TQ_F32) {
            v[4 * i + q] = __uint_as_float(w[q]);
          } else if (XT == TQ_BF16) {
            v[8 * i + 2 * q] = bf16_to_f32((uint16_t)(w[q] & 0xFFFF));
            v[8 * i + 2 * q + 1] = bf16_to_f32((uint16_t)(w[q] >> 16));
          } else {
            v[8 * i + 2 * q] = f16_to_f32((uint16_t)(w[q] & 0xFFFF));
            v[8 * i + 2 * q + 1] = f16_to_f32((uint16_t)(w[q] >> 16));
          }
        }
      }
      double ssq = 0.0;
#pragma unroll
      for (int i = 0; i < PER; ++i) ssq = fma((double)v[i], (double)v[i], ssq);
      if (XT == TQ_BF16) {
#pragma unroll
        for (int i = 0; i < RAW; ++i) *reinterpret_cast<uint4 *>(&sh.a[0][sr][sk + 8 * i]) = raw[i];
      } else {
#pragma unroll
        for (int i = 0; i < PER; i += 8) {
          uint32_t pk[3][4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float p0[3], p1[3];
            split_exact<NPA>(v[i + 2 * q], p0);
            split_exact<NPA>(v[i + 2 * q + 1], p1);
#pragma unroll
            for (int p = 0; p < 3; ++p) pk[p][q] = pack_bf16x2(p0[p], p1[p]);
          }
#pragma unroll
          for (int p = 0; p < NPA; ++p)
            *reinterpret_cast<uint4 *>(&sh.a[p][sr][sk + i]) = uint4{pk[p][0], pk[p][1], pk[p][2], pk[p][3]};
        }
      }
#pragma unroll
      for (int o = 1; o < NW; o <<= 1) ssq += __shfl_xor(ssq, o, 64);
      if (tid % NW == 0) {
        const double nn = sqrt(ssq);
        const uint16_t h = f64_to_f16_rne_sat(nn);
        sh.n32[buf][sr] = (float)nn;
        sh.nh[buf][sr] = f16_to_f32(h);
        if (sr < rows) a.norms[row0 + sr] = h;
      }
    }
    lds_barrier();  // tile and norms staged

    // next tile's rows in flight behind this tile's work
    if (tile + gridDim.x < a.ntiles) load_raw(tile + gridDim.x);
    const float n = sh.n32[buf][lane], nhat = sh.nh[buf][lane];

    // ---- y = Pi x for this wave's columns ----
    floatx4 acc[4][NCT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 af[4][3];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int p = 0; p < 3; ++p)
          af[rt][p] = p < NPA ? *reinterpret_cast<const bf16x8 *>(&sh.a[p][16 * rt + j16][32 * ks + 8 * g4]) : af[rt][0];
      contract_kstep<NPA, NCT>(af, bpi[ks], acc);
    }
    lds_barrier();  // row pieces consumed

    // ---- to lane = row ----
    float(*cw)[CW + 4] = sh.cw[wave];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) cw[16 * rt + 4 * g4 + e][16 * ct + j16] = acc[rt][ct][e];
    wave_lds_order();

    // ---- quantize row `lane` over this wave's columns ----
    float thr[L - 1];
#pragma unroll
    for (int k = 0; k < L - 1; ++k) thr[k] = tb[k] * n;
    uint32_t plane[BM];
#pragma unroll
    for (int p = 0; p < BM; ++p) plane[p] = 0u;
    float rs = 0.f;  // ||r||^2 over this wave's columns (fp32: gamma is checked to 1e-5 of a midpoint)
#pragma unroll
    for (int c8 = CW / 8 - 1; c8 >= 0; --c8) {
      const float4 y0 = *reinterpret_cast<const float4 *>(&cw[lane][8 * c8]);
      const float4 y1 = *reinterpret_cast<const float4 *>(&cw[lane][8 * c8 + 4]);
      const float ys[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
      float rv[8];
#pragma unroll
      for (int e = 7; e >= 0; --e) {
        float cv;
        quant_coord<BM, PROD>(ys[e], thr, cc, plane, cv);
        if (PROD) {
          rv[e] = fmaf(-nhat, cv, ys[e]);
          rs = fmaf(rv[e], rv[e], rs);
        }
      }
      if (PROD) {
        uint32_t pk[3][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float p0[3], p1[3];
          split_exact<3>(rv[2 * q], p0);
          split_exact<3>(rv[2 * q + 1], p1);
#pragma unroll
          for (int p = 0; p < 3; ++p) pk[p][q] = pack_bf16x2(p0[p], p1[p]);
        }
#pragma unroll
        for (int p = 0; p < 3; ++p)
          *reinterpret_cast<uint4 *>(&sh.rp[p][lane][CW * wave + 8 * c8]) = uint4{pk[p][0], pk[p][1], pk[p][2], pk[p][3]};
      }
    }
    if (n == 0.0f) {  // zero vector: every coordinate takes cell L/2 - 1
#pragma unroll
      for (int p = 0; p < BM; ++p) plane[p] = (((L / 2 - 1) >> p) & 1) ? 0xFFFFFFFFu : 0u;
    }
    uint8_t *rec = a.codes + (row0 + lane) * a.code_bytes + (CW / 8) * wave;
    if (lane < rows) {
#pragma unroll
      for (int p = 0; p < BM; ++p) {
        if (CW == 32) *reinterpret_cast<uint32_t *>(rec + p * (D / 8)) = plane[p];
        else *reinterpret_cast<uint16_t *>(rec + p * (D / 8)) = (uint16_t)plane[p];
      }
    }
    if (!PROD) continue;

    // ---- Algorithm 2: gamma, S r = (S Pi^T) r_rot, sign plane ----
    sh.gpart[wave][lane] = rs;
    lds_barrier();  // residual pieces and partial norms complete
    if (wave == 0 && lane < rows) {
      double g2 = 0.0;
#pragma unroll
      for (int w = 0; w < NW; ++w) g2 += (double)sh.gpart[w][lane];
      a.gammas[row0 + lane] = f64_to_f16_rne_sat(sqrt(g2));
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 af[4][3];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int p = 0; p < 3; ++p) af[rt][p] = *reinterpret_cast<const bf16x8 *>(&sh.rp[p][16 * rt + j16][32 * ks + 8 * g4]);
      contract_kstep<3, NCT>(af, bmq[ks], acc);
    }
    wave_lds_order();
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) cw[16 * rt + 4 * g4 + e][16 * ct + j16] = acc[rt][ct][e];
    wave_lds_order();
    uint32_t sg = 0u;
#pragma unroll
    for (int c4 = CW / 4 - 1; c4 >= 0; --c4) {
      const float4 s4 = *reinterpret_cast<const float4 *>(&cw[lane][4 * c4]);
      sg = shift_in(sg, s4.w >= 0.0f);
      sg = shift_in(sg, s4.z >= 0.0f);
      sg = shift_in(sg, s4.y >= 0.0f);
      sg = shift_in(sg, s4.x >= 0.0f);
    }
    if (lane < rows) {
      if (CW == 32) *reinterpret_cast<uint32_t *>(rec + BM * (D / 8)) = sg;
      else *reinterpret_cast<uint16_t *>(rec + BM * (D / 8)) = (uint16_t)sg;
    }
  }
}

// resident work-groups of encode_kernel<XT, D, PROD, BM> per CU (cached)
template <int XT, int D, bool PROD, int BM>
int enc_blocks_per_cu() {
  static int cache = 0;
  if (cache > 0) return cache;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, encode_kernel<XT, D, PROD, BM>, enc_waves(D, PROD) * 64,
                                                   0) != hipSuccess ||
      blocks <= 0)
    blocks = 1;
  cache = blocks;
  return blocks;
}



template <int XT, int D, bool PROD, int BM>
void launch_encode(EncArgs ea, hipStream_t st) {
  ea.ntiles = cdiv64(ea.n, EB);
  const int64_t slots = (int64_t)device_cus() * enc_blocks_per_cu<XT, D, PROD, BM>();
  const unsigned grid = (unsigned)imin64(ea.ntiles, slots);
  hipLaunchKernelGGL((encode_kernel<XT, D, PROD, BM>), dim3(grid), dim3(enc_waves(D, PROD) * 64), 0, st, ea);
}

// instantiated per (mode) in the encode translation units
void launch_encode_mse(int xt, int d, int bm, const EncArgs &ea, hipStream_t st);
void launch_encode_prod(int xt, int d, int bm, const EncArgs &ea, hipStream_t st);

}  // namespace tq
