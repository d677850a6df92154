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
// bf16 and fp16 rows take fp16 operands instead, two pieces where one is not
// exact: each row is scaled by a power of two 2^kx so that its norm lies in
// [2^13, 2^14) (then every coordinate converts to fp16 exactly; what falls below
// the fp16 normal range is below 2^-38 of the norm), and the matrices are held as
// hi + lo fp16 pieces of A 2^k (round to nearest, 2^-23 of each entry left out;
// k puts the largest entry, or a bound on it, just under 2^14):
//   rows:      x (Pi_hi + Pi_lo)                                       (2 MFMAs)
//   residual:  r_hi M_hi + r_hi M_lo + r_lo M_hi                       (3 MFMAs)
// Two rounded fp16 pieces hold an entry to 2^-22 of itself, so a coordinate of
// Pi x carries at most 2^-22 n of representation error (2.7e-6 of the
// coordinate scale n / sqrt(d) at d = 128) and a projection of S r at most
// 3 2^-22 ||S_i|| ||r|| (8.1e-6 ||r|| at d = 128 with ||S_i|| ~ sqrt(d)), both
// below the 1e-5 tie zone, beside the fp32 accumulation error of either form,
// with 5 MFMAs where the bf16 pieces take 9.  Every power-of-two scale is undone
// exactly: the cell boundaries and n_hat take the row's scale, gamma divides it
// out in fp64.
//
// Work split.  A persistent work-group of NW waves (4; 8 for Algorithm 2 at
// d = 128 on fp32 rows) walks 64-row tiles.  Wave w owns output columns [w d/NW, (w+1) d/NW):
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

#include <type_traits>

#include "common.cuh"
#include "quant.cuh"

namespace tq {

constexpr int EB = 64;  // rows per tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Rows of x are nseq sequences of T tokens (a plain encode: one sequence of n rows); token t of sequence s
// is written to position t0 + t of that sequence's cache row of Tstride positions: records (row layout)
// or, when `tiles` is set, the token-tiled words [s][t / 32][plane][coordinate], bit t % 32 (t0 a
// multiple of 32; every word holding a written position is written whole, positions past the last
// token as zero bits).  A 64-row tile never spans two sequences.
struct EncArgs {
  const void *x;
  int64_t ldx, ntiles;
  int64_t T, tps;        // tokens per sequence, 64-row tiles per sequence
  int64_t t0, Tstride;   // first cache position written, positions per sequence in the cache
  const uint16_t *pi3;   // [3][D][D] pieces of Pi (row j, column k)
  const uint16_t *m3;    // [3][D][D] pieces of S Pi^T (Algorithm 2)
  const uint16_t *pih;   // [2][D][D] fp16 pieces of Pi 2^kp (bf16 and fp16 rows)
  const uint16_t *mh;    // [2][D][D] fp16 pieces of S Pi^T 2^km (Algorithm 2)
  int kp, km;
  uint8_t *codes;        // row layout
  uint32_t *tiles;       // token-tiled layout (codes unused)
  int64_t code_bytes, ntile32;  // ntile32: 32-token words per sequence in the tiled cache
  uint16_t *norms, *gammas;
  Codebook cb;
};

// 32 x 32 bit-matrix transpose within each half-wave: on entry lane r of a half holds row r (bit c =
// column c), on exit lane c holds column c (bit r = row r).  Off-diagonal blocks of width 16, 8, 4, 2, 1
// are exchanged between lanes r and r ^ j: the lower lane keeps its bits in the low half of every
// 2j-bit block and takes the partner's low halves shifted up; the upper lane keeps its high halves and
// takes the partner's high halves shifted down.
__device__ __forceinline__ uint32_t transpose32_bits(uint32_t a, int lane) {
  uint32_t m = 0x0000FFFFu;
#pragma unroll
  for (int j = 16; j >= 1; j >>= 1) {
    const uint32_t p = (uint32_t)__shfl_xor((int)a, j, 64);
    const bool low = (lane & j) == 0;
    a = low ? ((a & m) | ((p << j) & ~m)) : ((a & ~m) | ((p >> j) & m));
    if (j > 1) m ^= m << (j >> 1);
  }
  return a;
}

template <int XT>
struct EncIn {
  static constexpr bool HP = XT != TQ_F32;                                // fp16 operands (one piece per row element)
  static constexpr int NPA = HP ? 1 : 3;                                  // pieces per row element
  static constexpr int NPB = HP ? 2 : 3;                                  // pieces per matrix entry
  static constexpr int NPR = HP ? 2 : 3;                                  // pieces per residual element
  static constexpr int ESZ = XT == TQ_F32 ? 4 : 2;
};

// 16-byte alignment lets every fragment access be one ds_read/ds_write_b128 (8 lanes a cycle, conflict-free
// at the padded strides below) instead of b64 pairs (16 lanes a cycle, two-way conflicts)
// waves per work-group: Algorithm 2 at d = 128 on the bf16 pieces (fp32 rows) splits the columns over
// 8 waves (16 each), which halves the register-resident matrix pieces so two waves share each SIMD;
// otherwise 4 waves (the fp16 pieces of both matrices fit one wave of 32 columns in 128 registers, and two
// work-groups share a CU, so the two waves on a SIMD come from different work-groups and are not held in
// step by barriers: one's quantizer overlaps the other's matrix-core work)
__host__ __device__ constexpr int enc_waves(int D, bool PROD, bool HP) { return PROD && D == 128 && !HP ? 8 : 4; }

// the tile's row pieces and the per-wave transpose area share storage when ALIAS (Algorithm 2 on fp16
// operands: 76 KB instead of 113 KB, two work-groups per CU); the next tile is then staged only after
// every wave has finished reading its transpose area
template <bool ALIAS, class A, class C>
struct EncAC;
template <class A, class C>
struct EncAC<true, A, C> {
  union {
    A a;
    C cw;
  };
};
template <class A, class C>
struct EncAC<false, A, C> {
  A a;
  C cw;
};

template <int D, int NPA, int NPR, bool PROD, bool HP>
struct __attribute__((aligned(16))) EncLds {
  static constexpr int NW = enc_waves(D, PROD, HP);
  static constexpr int CW = D / NW;
  static constexpr bool ALIAS = PROD && HP;
  // a: row pieces of the tile; cw: per-wave transpose, MFMA layout -> lane = row
  EncAC<ALIAS, uint16_t[NPA][EB][D + 8], float[NW][EB][CW + 4]> ac;
  uint16_t rp[PROD ? NPR : 1][PROD ? EB : 1][D + 16];  // residual pieces (Algorithm 2; this stride measured 5 % faster than D + 8)
  float gpart[PROD ? NW : 1][EB];      // per-wave partial ||r||^2
  float n32[2][EB], nh[2][EB];         // norms by tile parity (times the row's scale 2^(kx + kp) for fp16 operands)
  int ksc[2][EB];                      // kx + kp of the row (fp16 operands)
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
__device__ __forceinline__ floatx4 mfma_bf16(const f16x8 &a, const f16x8 &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// two fp32 values as packed fp16, truncating (exact for the scaled row elements, see the header)
__device__ __forceinline__ uint32_t pack_f16x2_rtz(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}
// x = hi + lo as fp16 pieces, each rounded to nearest
__device__ __forceinline__ void split_f16(float x, uint16_t &hi, uint16_t &lo) {
  const _Float16 h = (_Float16)x;
  const _Float16 l = (_Float16)(x - (float)h);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
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
// fp16 operands: one row piece against the matrix's two
struct PieceTermsH1 {
  static constexpr int N = 2;
  static constexpr int A[N] = {0, 0}, B[N] = {1, 0};
};
// fp16 operands: two residual pieces against the matrix's two (lo x lo left out)
struct PieceTermsH2 {
  static constexpr int N = 3;
  static constexpr int A[N] = {1, 0, 0}, B[N] = {0, 1, 0};
};

// acc[rt][ct] += A rows (16 rt ..) x B columns (16 ct ..) over one 32-deep k-step,
// term-major so that consecutive MFMAs write different accumulators
template <typename TT, int NCT, typename V, int NA, int NB>
__device__ __forceinline__ void contract_terms(const V (&af)[4][NA], const V (&bf)[NCT][NB], floatx4 (&acc)[4][NCT]) {
#pragma unroll
  for (int t = 0; t < TT::N; ++t)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = mfma_bf16(af[rt][TT::A[t]], bf[ct][TT::B[t]], acc[rt][ct]);
}

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

// w = 2 w + b: the next-lower column's bit shifted in (columns visited high to low)
__device__ __forceinline__ uint32_t shift_in(uint32_t w, bool b) { return (w << 1) | (b ? 1u : 0u); }

template <int XT, int D, bool PROD, int BM>
__global__ __launch_bounds__(enc_waves(D, PROD, XT != TQ_F32) * 64) __attribute__((amdgpu_waves_per_eu(2))) void
encode_kernel(EncArgs a) {
  constexpr bool HP = EncIn<XT>::HP;
  constexpr int NPA = EncIn<XT>::NPA, NPB = EncIn<XT>::NPB, NPR = EncIn<XT>::NPR, ESZ = EncIn<XT>::ESZ;
  using MT = std::conditional_t<HP, f16x8, bf16x8>;  // matrix-core operand type
  constexpr int NW = enc_waves(D, PROD, HP);
  constexpr int CW = D / NW;       // columns per wave
  constexpr int NCT = CW / 16;     // 16-column MFMA tiles per wave
  constexpr int NKS = D / 32;      // 32-deep k-steps
  constexpr int L = 1 << BM;
  constexpr int PER = D / NW;      // staged elements per thread (NW threads per row)
  constexpr int RAW = PER * ESZ / 16;
  static_assert(RAW >= 1, "tile staging");
  using Lds = EncLds<D, NPA, NPR, PROD, HP>;
  __shared__ Lds sh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j16 = lane & 15, g4 = lane >> 4;

  // ---- register-resident matrix pieces of this wave's columns ----
  MT bpi[NKS][NCT][NPB];
  MT bmq[PROD ? NKS : 1][NCT][NPB];
  const uint16_t *pisrc = HP ? a.pih : a.pi3, *msrc = HP ? a.mh : a.m3;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int p = 0; p < NPB; ++p) {
        const int64_t off = ((int64_t)p * D + CW * wave + 16 * ct + j16) * D + 32 * ks + 8 * g4;
        bpi[ks][ct][p] = *reinterpret_cast<const MT *>(pisrc + off);
        if (PROD) bmq[ks][ct][p] = *reinterpret_cast<const MT *>(msrc + off);
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
    const int64_t sq = tile / a.tps, tl = (tile - sq * a.tps) * EB + sr;
    if (tl < a.T) {
      const int64_t row = sq * a.T + tl;
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
    const int64_t sq = tile / a.tps, tl0 = (tile - sq * a.tps) * EB;  // sequence, first token of the tile
    const int rows = (int)imin64(EB, a.T - tl0);
    const int64_t row0 = sq * a.Tstride + a.t0 + tl0;  // cache position of the tile's first token
    const int buf = it & 1;

    // ---- stage the tile: pieces into LDS, fp64 norm ----
    if (Lds::ALIAS && it > 0) lds_barrier();  // every wave's reads of the shared transpose area done
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
      int kx = 0;  // the row's scale 2^kx (fp16 operands)
      if (HP) {
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) ssq += __shfl_xor(ssq, o, 64);
        const double nn = sqrt(ssq);
        // nn = m 2^E with m in [0.5, 1): nn 2^(14 - E) lies in [2^13, 2^14), and so does no |x_i| 2^kx exceed 2^14
        kx = nn > 0.0 ? 14 - ((int)((__double_as_longlong(nn) >> 52) & 0x7FF) - 1022) : 0;
#pragma unroll
        for (int i = 0; i < PER; i += 8) {
          uint32_t pk[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            pk[q] = pack_f16x2_rtz(__builtin_amdgcn_ldexpf(v[i + 2 * q], kx), __builtin_amdgcn_ldexpf(v[i + 2 * q + 1], kx));
          *reinterpret_cast<uint4 *>(&sh.ac.a[0][sr][sk + i]) = uint4{pk[0], pk[1], pk[2], pk[3]};
        }
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
            *reinterpret_cast<uint4 *>(&sh.ac.a[p][sr][sk + i]) = uint4{pk[p][0], pk[p][1], pk[p][2], pk[p][3]};
        }
      }
      if (!HP) {
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) ssq += __shfl_xor(ssq, o, 64);
      }
      if (tid % NW == 0) {
        const double nn = sqrt(ssq);
        const uint16_t h = f64_to_f16_rne_sat(nn);
        const int ks = HP ? kx + a.kp : 0;
        sh.n32[buf][sr] = __builtin_amdgcn_ldexpf((float)nn, ks);
        sh.nh[buf][sr] = __builtin_amdgcn_ldexpf(f16_to_f32(h), ks);
        sh.ksc[buf][sr] = ks;
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
      if constexpr (HP) {
        f16x8 af[4][1];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) af[rt][0] = *reinterpret_cast<const f16x8 *>(&sh.ac.a[0][16 * rt + j16][32 * ks + 8 * g4]);
        contract_terms<PieceTermsH1, NCT>(af, bpi[ks], acc);
      } else {
        bf16x8 af[4][3];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int p = 0; p < 3; ++p)
            af[rt][p] = p < NPA ? *reinterpret_cast<const bf16x8 *>(&sh.ac.a[p][16 * rt + j16][32 * ks + 8 * g4]) : af[rt][0];
        contract_kstep<NPA, NCT>(af, bpi[ks], acc);
      }
    }
    lds_barrier();  // row pieces consumed

    // ---- to lane = row ----
    float(*cw)[CW + 4] = sh.ac.cw[wave];
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
    const float rdn = HP ? __builtin_amdgcn_ldexpf(1.f, -a.kp) : 1.f;
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
      if (PROD && HP) {
        // r 2^(kx + kp) 2^-kp: at most 2^14 and a little (|r_i| <= max(|y_i|, n_hat |c|))
        uint32_t pk[2][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint16_t h0, l0, h1, l1;
          split_f16(rv[2 * q] * rdn, h0, l0);
          split_f16(rv[2 * q + 1] * rdn, h1, l1);
          pk[0][q] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          pk[1][q] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p)
          *reinterpret_cast<uint4 *>(&sh.rp[p][lane][CW * wave + 8 * c8]) = uint4{pk[p][0], pk[p][1], pk[p][2], pk[p][3]};
      } else if (PROD) {
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
    quant_fix_planes<BM>(plane, CW == 32 ? 0xFFFFFFFFu : (1u << CW) - 1u);
    if (n == 0.0f) {  // zero vector: every coordinate takes cell L/2 - 1
#pragma unroll
      for (int p = 0; p < BM; ++p) plane[p] = (((L / 2 - 1) >> p) & 1) ? 0xFFFFFFFFu : 0u;
    }
    uint8_t *rec = a.codes + (row0 + lane) * a.code_bytes + (CW / 8) * wave;
    // token-tiled words of this wave's columns: lane = (half hh, column c) after the transpose
    const int tc = lane & 31, thh = lane >> 5;
    const bool twr = tc < CW && tl0 + 32 * thh < a.T;
    uint32_t *tw = a.tiles + ((sq * a.ntile32 + (a.t0 + tl0) / 32 + thh) * (BM + (PROD ? 1 : 0))) * D + CW * wave + tc;
    if (a.tiles) {
#pragma unroll
      for (int p = 0; p < BM; ++p) {
        const uint32_t w = transpose32_bits(lane < rows ? plane[p] : 0u, lane);
        if (twr) tw[p * D] = w;
      }
    } else if (lane < rows) {
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
      if (HP) g2 = ldexp(g2, -2 * sh.ksc[buf][lane]);
      a.gammas[row0 + lane] = f64_to_f16_rne_sat(sqrt(g2));
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      MT af[4][NPR];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int p = 0; p < NPR; ++p) af[rt][p] = *reinterpret_cast<const MT *>(&sh.rp[p][16 * rt + j16][32 * ks + 8 * g4]);
      if constexpr (HP) contract_terms<PieceTermsH2, NCT>(af, bmq[ks], acc);
      else contract_kstep<3, NCT>(af, bmq[ks], acc);
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
    if (a.tiles) {
      const uint32_t w = transpose32_bits(lane < rows ? sg : 0u, lane);
      if (twr) tw[BM * D] = w;
    } else if (lane < rows) {
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
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, encode_kernel<XT, D, PROD, BM>,
                                                   enc_waves(D, PROD, XT != TQ_F32) * 64,
                                                   0) != hipSuccess ||
      blocks <= 0)
    blocks = 1;
  cache = blocks;
  return blocks;
}



template <int XT, int D, bool PROD, int BM>
void launch_encode(EncArgs ea, hipStream_t st) {
  const int64_t slots = (int64_t)device_cus() * enc_blocks_per_cu<XT, D, PROD, BM>();
  const unsigned grid = (unsigned)imin64(ea.ntiles, slots);
  hipLaunchKernelGGL((encode_kernel<XT, D, PROD, BM>), dim3(grid), dim3(enc_waves(D, PROD, XT != TQ_F32) * 64), 0, st,
                     ea);
}

// instantiated per (mode) in the encode translation units
void launch_encode_mse(int xt, int d, int bm, const EncArgs &ea, hipStream_t st);
void launch_encode_prod(int xt, int d, int bm, const EncArgs &ea, hipStream_t st);

}  // namespace tq
