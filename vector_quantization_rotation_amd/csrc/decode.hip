// Fused decode for head dims 64 and 128 on the bf16 matrix cores.
//
// Algorithm 1 and 2 decode as on the ai-navigate-news Gemma 4 post (section
// "仕組み（技術的）"):  x~ = n Pi^T c[idx]  (+ sqrt(pi/2)/d * gamma S^T (2 s - 1)
// for Algorithm 2).
//
// A persistent work-group of NW waves (4; 8 for Algorithm 2 at d = 128) walks
// 64-record tiles.  The tile's bits are expanded once into LDS: the centroid
// c[idx] of every coordinate as two
// bf16 pieces (hi keeps the top 8 significant bits, mid the next 8: c - hi - mid
// is below 2^-16 |c|) and, for Algorithm 2, the sign plane as +-1 (exact).
// Wave w owns output columns [w d/NW, (w+1) d/NW) and keeps two pieces of Pi^T
// (and of S^T) for them in registers for the whole launch.  Products:
// c_hi T_hi + c_hi T_mid + c_mid T_hi (and s T_hi + s T_mid), fp32 accumulate,
// so a reconstruction is within ~1e-5 of its fp64 value (the gate is 2e-3).  The
// norms multiply the accumulated rows: out = n acc_mse + qjl gamma acc_sign.
#include "common.cuh"

namespace tq {

constexpr int DB = 64;  // records per tile

typedef __bf16 dbf16x8 __attribute__((ext_vector_type(8)));

struct DecArgs {
  const uint8_t *codes;
  const uint16_t *norms, *gammas;
  float *out;
  int64_t ldo, n, ntiles, code_bytes;
  const uint16_t *pit3, *st3;  // [3][D][D] pieces of Pi^T and S^T (row j = output coordinate)
  float qjl;
  float c[16];                 // centroids
};

template <int D, bool PROD>
struct __attribute__((aligned(16))) DecLds {
  union {
    struct {
      uint16_t am[2][DB][D + 8];          // c[idx] pieces
      uint16_t aq[PROD ? DB : 1][D + 8];  // 2 s - 1
    } op;
    float ot[DB][D + 4];                  // the tile's output rows, staged for whole-row stores
  } u;
  float nh[DB], gq[DB];                   // n and qjl gamma per record
};

__device__ __forceinline__ uint32_t d_pack2(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// waves per work-group: Algorithm 2 at d = 128 holds the pieces of both matrices and two accumulator sets,
// so its columns are split over 8 waves (16 each: 64 matrix registers instead of 128), which lets several
// waves share a SIMD; otherwise 4 waves
__host__ __device__ constexpr int dec_waves(int D, bool PROD) { return PROD && D == 128 ? 8 : 4; }

template <int D, bool PROD, int BM>
__global__ __launch_bounds__(dec_waves(D, PROD) * 64) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(DecArgs a) {
  constexpr int NW = dec_waves(D, PROD);
  constexpr int CW = D / NW, NCT = CW / 16, NKS = D / 32, L = 1 << BM;
  constexpr int PER = D / NW;  // coordinates staged per thread (NW threads per record)
  static_assert(PER == 16 || PER == 32, "record bits are read as 16- or 32-bit words");
  constexpr int NPL = BM + (PROD ? 1 : 0);
  __shared__ DecLds<D, PROD> sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j16 = lane & 15, g4 = lane >> 4;

  dbf16x8 bpt[NKS][NCT][2], bst[PROD ? NKS : 1][NCT][2];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int64_t off = ((int64_t)p * D + CW * wave + 16 * ct + j16) * D + 32 * ks + 8 * g4;
        bpt[ks][ct][p] = *reinterpret_cast<const dbf16x8 *>(a.pit3 + off);
        if (PROD) bst[ks][ct][p] = *reinterpret_cast<const dbf16x8 *>(a.st3 + off);
      }
  float cc[L];
#pragma unroll
  for (int i = 0; i < L; ++i) cc[i] = a.c[i];
  // up to four centroids (BM <= 2): each bf16 piece of every centroid in a byte table of two words
  // (centroid k in bytes 2k, 2k + 1), so that one byte permute picks the pieces of two coordinates, with
  // the permute selectors of every pair of index values (and the +-1 pairs of the sign plane) in LDS
  __shared__ uint32_t s_sel[16 + 4];
  uint32_t lh_lo = 0u, lh_hi = 0u, lm_lo = 0u, lm_hi = 0u;
  if constexpr (BM <= 2) {
    uint32_t ph[4] = {0u, 0u, 0u, 0u}, pm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < L; ++k) {
      const float h = __uint_as_float(__float_as_uint(cc[k]) & 0xFFFF0000u);
      ph[k] = __float_as_uint(h) >> 16;
      pm[k] = __float_as_uint(cc[k] - h) >> 16;
    }
    lh_lo = ph[0] | (ph[1] << 16);
    lh_hi = ph[2] | (ph[3] << 16);
    lm_lo = pm[0] | (pm[1] << 16);
    lm_hi = pm[2] | (pm[3] << 16);
    // w = plane-0 bits of the pair | plane-1 bits << 2 (BM = 2), or the plane-0 bits (BM = 1)
    if (tid < 16) {
      const int w = tid;
      const int i0 = BM == 2 ? (w & 1) | ((w >> 1) & 2) : (w & 1);
      const int i1 = BM == 2 ? ((w >> 1) & 1) | ((w >> 2) & 2) : ((w >> 1) & 1);
      s_sel[w] = 0x01000100u + 0x0202u * (uint32_t)i0 + 0x02020000u * (uint32_t)i1;
    } else if (tid < 20) {
      const int sb = tid - 16;
      s_sel[tid] = ((sb & 1) ? 0x3F80u : 0xBF80u) | (((sb & 2) ? 0x3F80u : 0xBF80u) << 16);
    }
  }

  const int sr = tid / NW, sk = (tid % NW) * PER;
  uint32_t bits[NPL];
  float fn = 0.f, fg = 0.f;
  auto load_raw = [&](int64_t tile) {
    const int64_t r = tile * DB + sr;
    const bool ok = r < a.n;
    const uint8_t *rec = a.codes + (ok ? r : 0) * a.code_bytes + sk / 8;
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      if (PER == 32) bits[p] = ok ? *reinterpret_cast<const uint32_t *>(rec + p * (D / 8)) : 0u;
      else bits[p] = ok ? *reinterpret_cast<const uint16_t *>(rec + p * (D / 8)) : 0u;
    }
    fn = ok ? f16_to_f32(a.norms[r]) : 0.f;
    fg = (ok && PROD) ? a.qjl * f16_to_f32(a.gammas[r]) : 0.f;
  };

  int64_t tile = blockIdx.x;
  if (tile < a.ntiles) load_raw(tile);
  for (; tile < a.ntiles; tile += gridDim.x) {
    const int64_t row0 = tile * DB;
    __syncthreads();  // the previous tile's fragments and norms are consumed
    // ---- expand this tile's bits: c[idx] pieces and signs ----
#pragma unroll
    for (int i = 0; i < PER; i += 8) {
      uint32_t hi[4], mi[4], sg[4];
      if constexpr (BM <= 2) {  // (the tables are in LDS: the loop's first barrier has passed)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = i + 2 * q;
          uint32_t w = (bits[0] >> j) & 3u;
          if (BM == 2) w |= ((bits[1] >> j) & 3u) << 2;
          const uint32_t sel = s_sel[w];
          hi[q] = __builtin_amdgcn_perm(lh_hi, lh_lo, sel);
          mi[q] = __builtin_amdgcn_perm(lm_hi, lm_lo, sel);
          if (PROD) sg[q] = s_sel[16 + ((bits[BM] >> j) & 3u)];
        }
      } else
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float h2[2], m2[2];
        uint32_t s2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int j = i + 2 * q + t;
          // centroid by a select tree over the index bits
          float v[L];
#pragma unroll
          for (int u = 0; u < L; ++u) v[u] = cc[u];
#pragma unroll
          for (int p = 0, m = L; p < BM; ++p, m >>= 1) {
            const bool bp = (bits[p] >> j) & 1u;
#pragma unroll
            for (int u = 0; u < L / 2; ++u)
              if (u < m / 2) v[u] = bp ? v[2 * u + 1] : v[2 * u];
          }
          h2[t] = __uint_as_float(__float_as_uint(v[0]) & 0xFFFF0000u);
          m2[t] = __uint_as_float(__float_as_uint(v[0] - h2[t]) & 0xFFFF0000u);
          s2[t] = PROD && ((bits[BM] >> j) & 1u) ? 0x3F80u : 0xBF80u;  // +1 / -1 in bf16
        }
        hi[q] = d_pack2(h2[0], h2[1]);
        mi[q] = d_pack2(m2[0], m2[1]);
        sg[q] = s2[0] | (s2[1] << 16);
      }
      *reinterpret_cast<uint4 *>(&sh.u.op.am[0][sr][sk + i]) = uint4{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<uint4 *>(&sh.u.op.am[1][sr][sk + i]) = uint4{mi[0], mi[1], mi[2], mi[3]};
      if (PROD) *reinterpret_cast<uint4 *>(&sh.u.op.aq[sr][sk + i]) = uint4{sg[0], sg[1], sg[2], sg[3]};
    }
    if (tid % NW == 0) {
      sh.nh[sr] = fn;
      sh.gq[sr] = fg;
    }
    __syncthreads();
    if (tile + gridDim.x < a.ntiles) load_raw(tile + gridDim.x);

    // ---- contractions over k ----
    floatx4 accm[4][NCT], accq[PROD ? 4 : 1][NCT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        accm[rt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (PROD) accq[rt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int r = 16 * rt + j16, k = 32 * ks + 8 * g4;
        const dbf16x8 ah = *reinterpret_cast<const dbf16x8 *>(&sh.u.op.am[0][r][k]);
        const dbf16x8 am = *reinterpret_cast<const dbf16x8 *>(&sh.u.op.am[1][r][k]);
        dbf16x8 aq;
        if (PROD) aq = *reinterpret_cast<const dbf16x8 *>(&sh.u.op.aq[r][k]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          floatx4 c = accm[rt][ct];
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, bpt[ks][ct][0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bpt[ks][ct][1], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bpt[ks][ct][0], c, 0, 0, 0);
          accm[rt][ct] = c;
          if (PROD) {
            floatx4 e = accq[rt][ct];
            e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bst[ks][ct][1], e, 0, 0, 0);
            e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bst[ks][ct][0], e, 0, 0, 0);
            accq[rt][ct] = e;
          }
        }
      }
    }
    // ---- out = n acc_mse + qjl gamma acc_sign (lane: rows 16 rt + 4 g4 + e, column 16 ct + j16), staged in
    // LDS over the operands (every wave's reads of them done), then stored as whole rows: a wave's own
    // columns are only 16 or 32 floats of a row ----
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * g4 + e;
        const float nr = sh.nh[r], gr = PROD ? sh.gq[r] : 0.f;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          float v = nr * accm[rt][ct][e];
          if (PROD) v = fmaf(gr, accq[rt][ct][e], v);
          sh.u.ot[r][CW * wave + 16 * ct + j16] = v;
        }
      }
    __syncthreads();
    const int rows = (int)imin64(DB, a.n - row0);
    for (int i = tid; i < rows * (D / 4); i += NW * 64) {
      const int r = i / (D / 4), c4 = i % (D / 4);
      *reinterpret_cast<float4 *>(a.out + (row0 + r) * a.ldo + 4 * c4) =
          *reinterpret_cast<const float4 *>(&sh.u.ot[r][4 * c4]);
    }
  }
}

template <int D, bool PROD, int BM>
static void launch_decode(DecArgs da, hipStream_t st) {
  static int per_cu = 0;
  if (per_cu <= 0) {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, decode_kernel<D, PROD, BM>, dec_waves(D, PROD) * 64, 0) !=
            hipSuccess ||
        b <= 0)
      b = 1;
    per_cu = b;
  }
  da.ntiles = cdiv64(da.n, DB);
  const unsigned grid = (unsigned)imin64(da.ntiles, (int64_t)device_cus() * per_cu);
  hipLaunchKernelGGL((decode_kernel<D, PROD, BM>), dim3(grid), dim3(dec_waves(D, PROD) * 64), 0, st, da);
}

bool decode_fused_supported(const tq_quantizer *q) {
  return (q->d == 64 || q->d == 128) && q->bmse >= 1 && q->bmse <= 3 && q->pit3 &&
         (q->mode != TQ_PROD || q->st3);
}

int run_decode_fused(const tq_quantizer *q, const uint8_t *codes, const uint16_t *norms, const uint16_t *gammas,
                     int64_t n, float *out, int64_t ldo, hipStream_t st) {
  if (n == 0) return TQ_OK;
  DecArgs da{};
  da.codes = codes; da.norms = norms; da.gammas = gammas; da.out = out; da.ldo = ldo; da.n = n;
  da.code_bytes = (int64_t)q->code_bytes; da.pit3 = q->pit3; da.st3 = q->st3; da.qjl = q->qjl_scale;
  for (int i = 0; i < kMaxCentroids; ++i) da.c[i] = i < q->cb.L ? q->cb.c[i] : 0.f;
  const bool prod = q->mode == TQ_PROD;
  ProfScope ps("decode", st);
#define TQ_DEC(DD, PP, BB) \
  if (q->d == DD && prod == PP && q->bmse == BB) launch_decode<DD, PP, BB>(da, st);
  TQ_DEC(128, false, 1) TQ_DEC(128, false, 2) TQ_DEC(128, false, 3)
  TQ_DEC(128, true, 1) TQ_DEC(128, true, 2) TQ_DEC(128, true, 3)
  TQ_DEC(64, false, 1) TQ_DEC(64, false, 2) TQ_DEC(64, false, 3)
  TQ_DEC(64, true, 1) TQ_DEC(64, true, 2) TQ_DEC(64, true, 3)
#undef TQ_DEC
  return launch_check();
}

}  // namespace tq
