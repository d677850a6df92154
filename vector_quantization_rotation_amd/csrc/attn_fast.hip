// Fast decode attention on a TurboQuant cache: int8 matrix cores on bit planes.
//
// Method (ai-navigate-news Gemma 4 post, section "仕組み（技術的）"): keys are
// Algorithm-1 records, values Algorithm-2 records; scores use the rotated query
// q' = Pi_K q, values are aggregated in the rotated and sign domains and
// rotated back once per head by the combine kernel.
//
// Kernel design (gfx950):
// * A symmetric b-bit Lloyd-Max codebook is an odd function of the index bits,
//   so with s_p = 2 bit_p - 1 it expands exactly over the odd-size subsets S of
//   the bit planes:  c[idx] = sum_S beta_S prod_{p in S} s_p  (2^(b-1) terms;
//   for b = 3: planes b0, b1, b2 and the parity b0^b1^b2).  Each term is a 0/1
//   bit plane, so <q', c[idx]> = 2 sum_S beta_S <q', bits_S> - c[L-1] sum_j q'_j.
// * A 0/1 plane word w feeds v_mfma_i32_16x16x64_i8 directly: (w & 0x01010101 << k)
//   holds four bits as bytes of value 2^k (k = 7 reads as -128); the 2^-k (and
//   the sign for k = 7) is folded into the other operand.
// * The other operand (query or softmax weights) is split into four int8
//   terms (a1 + a2/2^7 + a3/2^14 + a4/2^21), one per MFMA row of a head, so
//   integer accumulation is exact and the only rounding is the split itself.
// * Keys stay in per-token records (their bits run along the contraction).
//   Values are read from the token-tiled layout (32 tokens per word) so that
//   the contraction over tokens also runs along the word bits.
// * Each work-group owns a (batch, kv-head, head group, sequence chunk); inside,
//   sub-chunks of 256 tokens are scored (pass K), their softmax weights split
//   to int8 in LDS, then aggregated (pass V) and folded into fp32 accumulators
//   with the running maximum (online softmax across sub-chunks).
#include <algorithm>

#include "common.cuh"

namespace tq {

constexpr int FA_THREADS = 256;
constexpr int FA_SUB = 256;     // tokens per sub-chunk
constexpr int FA_GMAX = 4;      // query heads per work-group (16 MFMA rows = 4 heads x 4 splits)

struct FastAttnArgs {
  const int *qimg;          // [units][KP*(D/128)*2][64 lanes][4] int32 query operand images
  const float *qinfo;       // [units][FA_GMAX][2]: 1/S_q, c[L-1]*sum(q')
  const uint8_t *kcodes;    // [B, Hkv, Tstride, kcb]
  const uint16_t *knorms;   // [B, Hkv, Tstride]
  const uint32_t *vtiles;   // [B, Hkv, ntile, VPL, D]
  const uint16_t *vnorms, *vgammas;
  const int32_t *seq_len;
  float *part;              // [B*Hq, nsplit, 2 + 2D]
  int64_t Tstride, ntile;
  int Hq, Hkv, G, nsub, chunk, nsplit;
  float scale_log2, vqjl;
  float vbeta[4];           // Walsh coefficients of the value codebook (odd subsets)
};

// Walsh subset masks (odd-size subsets of the index bits), enumeration order shared with the host
__host__ __device__ constexpr int walsh_count(int b) { return 1 << (b - 1); }

template <int B>
__device__ __forceinline__ void walsh_planes(const uint32_t *w, uint32_t *out) {
  if constexpr (B == 1) {
    out[0] = w[0];
  } else if constexpr (B == 2) {
    out[0] = w[0]; out[1] = w[1];
  } else if constexpr (B == 3) {
    out[0] = w[0]; out[1] = w[1]; out[2] = w[2]; out[3] = w[0] ^ w[1] ^ w[2];
  } else {
    out[0] = w[0]; out[1] = w[1]; out[2] = w[2]; out[3] = w[3];
    out[4] = w[0] ^ w[1] ^ w[2]; out[5] = w[0] ^ w[1] ^ w[3];
    out[6] = w[0] ^ w[2] ^ w[3]; out[7] = w[1] ^ w[2] ^ w[3];
  }
}

// v (|v| <= 127.5) as a1 + a2/2^7 + a3/2^14 + a4/2^21 with int8 terms (|a2..a4| <= 64)
__device__ __forceinline__ void split4(float v, int8_t *o) {
  const float a1 = rintf(v), r1 = (v - a1) * 128.f, a2 = rintf(r1), r2 = (r1 - a2) * 128.f, a3 = rintf(r2);
  const float a4 = rintf((r2 - a3) * 128.f);
  o[0] = (int8_t)(int)a1;
  o[1] = (int8_t)(int)a2;
  o[2] = (int8_t)(int)a3;
  o[3] = (int8_t)(int)a4;
}

__device__ __forceinline__ float rows16_max(float v) {
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float rows16_sum(float v) {
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// D: head dim; KB: key index bits; VB: value index bits (Algorithm-2 records hold VB+1 planes)
template <int D, int KB, int VB>
__global__ __launch_bounds__(FA_THREADS) void attn_fast_kernel(FastAttnArgs a) {
  constexpr int KP = walsh_count(KB);        // key Walsh planes
  constexpr int VMP = walsh_count(VB);       // value Walsh planes (index part)
  constexpr int VPL = VB + 1;                // stored value planes per tile
  constexpr int KW = D / 32;                 // 32-bit words per key plane
  constexpr int NINS = KP * (D / 128) * 2;   // key-side MFMAs per 16 tokens
  constexpr int NT = D / 16;                 // value column tiles
  constexpr int NT_W = NT / 4;               // column tiles per wave
  constexpr int KCB = KB * D / 8;            // key record bytes

  __shared__ float s_sc[FA_GMAX][FA_SUB];
  __shared__ float s_vn[FA_SUB], s_vg[FA_SUB];
  __shared__ __attribute__((aligned(16))) uint8_t s_w[2][FA_SUB / 64][16][64];  // int8 weight operands
  __shared__ float s_red[4][FA_GMAX][4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = blockIdx.x, split = blockIdx.y;
  const int sub = unit % a.nsub, bg = unit / a.nsub;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int h0 = g * a.G + sub * FA_GMAX;
  const int gw = min(FA_GMAX, a.G - sub * FA_GMAX);
  const int64_t T = min<int64_t>(max<int64_t>(a.seq_len[b], 0), a.Tstride);
  const int64_t c0 = (int64_t)split * a.chunk;
  const int64_t c1 = min<int64_t>(T, c0 + a.chunk);
  const int64_t seq = (int64_t)b * a.Hkv + g;

  // query operand image (constant over the chunk)
  intx4 qa[NINS];
  {
    const intx4 *img = reinterpret_cast<const intx4 *>(a.qimg) + (int64_t)unit * NINS * 64;
#pragma unroll
    for (int i = 0; i < NINS; ++i) qa[i] = img[i * 64 + lane];
  }
  const int hl = lane >> 4;  // head owned by this lane in score/accumulator layouts
  const float qinv = a.qinfo[((int64_t)unit * FA_GMAX + hl) * 2 + 0];
  const float qconst = a.qinfo[((int64_t)unit * FA_GMAX + hl) * 2 + 1];

  // zero the weight operand tiles once: unused rows stay zero
  for (int i = tid; i < (int)sizeof(s_w) / 4; i += FA_THREADS) reinterpret_cast<uint32_t *>(&s_w[0][0][0][0])[i] = 0u;

  // per-lane constants for the value B operand: k offset 0 or 4 by lane group parity
  const int kofs = ((lane >> 4) & 1) * 4;
  // fp32 accumulators: [plane (VMP mse + 1 sign)][column tile of this wave][split-combined]
  float acc[VMP + 1][NT_W];
#pragma unroll
  for (int p = 0; p <= VMP; ++p)
#pragma unroll
    for (int c = 0; c < NT_W; ++c) acc[p][c] = 0.f;
  float m_run[FA_GMAX];                       // running maxima, identical in every thread
#pragma unroll
  for (int h = 0; h < FA_GMAX; ++h) m_run[h] = -INFINITY;
  float l_run = 0.f, ym_run = 0.f, yq_run = 0.f;  // sums for head hl (this lane's head)

  const uint8_t *kbase = a.kcodes + seq * a.Tstride * KCB;
  const uint16_t *knb = a.knorms + seq * a.Tstride;
  const uint16_t *vnb = a.vnorms + seq * a.Tstride;
  const uint16_t *vgb = a.vgammas + seq * a.Tstride;
  const uint32_t *vtb = a.vtiles + seq * a.ntile * VPL * D;

  for (int64_t s0 = c0; s0 < c1; s0 += FA_SUB) {
    __syncthreads();  // previous sub-chunk fully consumed
    // ---------------- pass K: scores for FA_SUB tokens ----------------
    float lmax = -INFINITY, vnmax = 0.f, vgmax = 0.f;
    for (int grp = wave; grp < FA_SUB / 16; grp += 4) {
      const int tl = grp * 16 + (lane & 15);
      const int64_t t = s0 + tl;
      const bool valid = t < c1;
      uint32_t w[KB];
      const int gq = lane >> 4;  // lane group: which 32-coordinate words
#pragma unroll
      for (int p = 0; p < KB; ++p) w[p] = 0u;
      intx4 cacc = {0, 0, 0, 0};
#pragma unroll
      for (int wb = 0; wb < D / 128; ++wb) {
        if (valid) {
          const uint32_t *rec = reinterpret_cast<const uint32_t *>(kbase + t * KCB);
#pragma unroll
          for (int p = 0; p < KB; ++p) w[p] = rec[p * KW + wb * 4 + gq];
        }
        uint32_t wp[KP];
        walsh_planes<KB>(w, wp);
#pragma unroll
        for (int p = 0; p < KP; ++p) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            intx4 bb;
#pragma unroll
            for (int r = 0; r < 4; ++r) bb[r] = (int)(wp[p] & (0x01010101u << (4 * half + r)));
            cacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[(p * (D / 128) + wb) * 2 + half], bb, cacc, 0, 0, 0);
          }
        }
      }
      // lane (token tl, head hl) holds the four split partial sums in cacc[0..3]
      const float raw = (float)cacc[0] + (float)cacc[1] * (1.f / 128.f) + (float)cacc[2] * (1.f / 16384.f) +
                        (float)cacc[3] * (1.f / 2097152.f);
      float sc = -INFINITY;
      if (valid && hl < gw) sc = (raw * qinv - qconst) * f16_to_f32(knb[t]) * a.scale_log2;
      s_sc[hl][tl] = sc;
      lmax = fmaxf(lmax, sc);
      if (hl == 0) {
        const float vn = valid ? f16_to_f32(vnb[t]) : 0.f;
        s_vn[tl] = vn;
        vnmax = fmaxf(vnmax, vn);
      } else if (hl == 1) {
        const float vg = valid ? f16_to_f32(vgb[t]) : 0.f;
        s_vg[tl] = vg;
        vgmax = fmaxf(vgmax, vg);
      }
    }
    lmax = rows16_max(lmax);
    vnmax = wave_max_f32(vnmax);
    vgmax = wave_max_f32(vgmax);
    if ((lane & 15) == 0) s_red[wave][hl][0] = lmax;
    if (lane == 0) { s_red[wave][0][1] = vnmax; s_red[wave][0][2] = vgmax; }
    __syncthreads();
    float msub[FA_GMAX];
    float vnm = 0.f, vgm = 0.f;
#pragma unroll
    for (int h = 0; h < FA_GMAX; ++h)
      msub[h] = fmaxf(fmaxf(s_red[0][h][0], s_red[1][h][0]), fmaxf(s_red[2][h][0], s_red[3][h][0]));
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) { vnm = fmaxf(vnm, s_red[wv][0][1]); vgm = fmaxf(vgm, s_red[wv][0][2]); }
    // per-head int8 scales: the largest weight of the sub-chunk maps to 127
    // (p <= 2^(msub - mnew) and n <= vnm bound every weight of head h)
    float mnew[FA_GMAX], swm[FA_GMAX], swq[FA_GMAX];
#pragma unroll
    for (int h = 0; h < FA_GMAX; ++h) {
      mnew[h] = fmaxf(m_run[h], msub[h]);
      const float pm = msub[h] == -INFINITY ? 0.f : exp2f(msub[h] - mnew[h]);
      swm[h] = (pm * vnm > 0.f) ? 127.f / (pm * vnm) : 0.f;
      swq[h] = (pm * vgm > 0.f) ? 127.f / (pm * vgm) : 0.f;
    }

    // ---------------- weights: p, p*n, p*gamma -> four int8 splits each ----------------
    float psum[FA_GMAX], pmsum[FA_GMAX], pqsum[FA_GMAX];
#pragma unroll
    for (int h = 0; h < FA_GMAX; ++h) psum[h] = pmsum[h] = pqsum[h] = 0.f;
    {
      const int tl = tid;  // one token per thread (FA_SUB == FA_THREADS)
      const int within = tl & 31, blk = (tl >> 5) & 1, tile = tl >> 6;
      const int kbit = within & 7, ib = within >> 3;
      const int gpos = 2 * blk + (kbit >> 2);
      const int bpos = gpos * 16 + (kbit & 3) * 4 + ib;
      const float kscale = (kbit == 7) ? -1.f / 128.f : 1.f / (float)(1 << kbit);
      const float vn = s_vn[tl], vg = s_vg[tl];
#pragma unroll
      for (int h = 0; h < FA_GMAX; ++h) {
        if (h >= gw) break;
        const float p = exp2f(s_sc[h][tl] - mnew[h]);
        const float wm = p * vn, wq = p * vg;
        psum[h] = p; pmsum[h] = wm; pqsum[h] = wq;
        int8_t o[4];
        split4(wm * swm[h] * kscale, o);
#pragma unroll
        for (int sp = 0; sp < 4; ++sp) s_w[0][tile][4 * h + sp][bpos] = (uint8_t)o[sp];
        split4(wq * swq[h] * kscale, o);
#pragma unroll
        for (int sp = 0; sp < 4; ++sp) s_w[1][tile][4 * h + sp][bpos] = (uint8_t)o[sp];
      }
    }
    // block sums of p, p n, p gamma per head
#pragma unroll
    for (int h = 0; h < FA_GMAX; ++h) {
      psum[h] = wave_sum_f32(psum[h]);
      pmsum[h] = wave_sum_f32(pmsum[h]);
      pqsum[h] = wave_sum_f32(pqsum[h]);
    }
    __syncthreads();  // s_red maxima read by everyone; weights written
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < FA_GMAX; ++h) { s_red[wave][h][0] = psum[h]; s_red[wave][h][1] = pmsum[h]; s_red[wave][h][2] = pqsum[h]; }
    }

    // ---------------- pass V: int8 MFMA over token tiles ----------------
    intx4 vacc[VMP + 1][NT_W];
#pragma unroll
    for (int p = 0; p <= VMP; ++p)
#pragma unroll
      for (int c = 0; c < NT_W; ++c) vacc[p][c] = intx4{0, 0, 0, 0};
    const int64_t tile0 = s0 >> 5;
#pragma unroll
    for (int tt = 0; tt < FA_SUB / 64; ++tt) {
      const intx4 wa_m = *reinterpret_cast<const intx4 *>(&s_w[0][tt][lane & 15][16 * (lane >> 4)]);
      const intx4 wa_q = *reinterpret_cast<const intx4 *>(&s_w[1][tt][lane & 15][16 * (lane >> 4)]);
      const int64_t vt = tile0 + 2 * tt + ((lane >> 4) >> 1);
      const bool tvalid = vt < a.ntile && (vt << 5) < c1;
      const uint32_t *tp = vtb + vt * (VPL * D);
#pragma unroll
      for (int c = 0; c < NT_W; ++c) {
        const int col = (wave * NT_W + c) * 16 + (lane & 15);
        uint32_t wv[VPL];
#pragma unroll
        for (int p = 0; p < VPL; ++p) wv[p] = tvalid ? tp[p * D + col] : 0u;
        uint32_t wpl[VMP];
        walsh_planes<VB>(wv, wpl);
#pragma unroll
        for (int p = 0; p < VMP; ++p) {
          intx4 bb;
#pragma unroll
          for (int r = 0; r < 4; ++r) bb[r] = (int)(wpl[p] & (0x01010101u << (kofs + r)));
          vacc[p][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa_m, bb, vacc[p][c], 0, 0, 0);
        }
        intx4 bs;
#pragma unroll
        for (int r = 0; r < 4; ++r) bs[r] = (int)(wv[VB] & (0x01010101u << (kofs + r)));
        vacc[VMP][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa_q, bs, vacc[VMP][c], 0, 0, 0);
      }
    }
    __syncthreads();  // partial sums visible
    // ---------------- fold into fp32 (online softmax) ----------------
    {
      float ps = 0.f, pm = 0.f, pq = 0.f;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) { ps += s_red[wv][hl][0]; pm += s_red[wv][hl][1]; pq += s_red[wv][hl][2]; }
      float mr = m_run[0], mn = mnew[0];
#pragma unroll
      for (int h = 1; h < FA_GMAX; ++h)
        if (hl == h) { mr = m_run[h]; mn = mnew[h]; }
      const float alpha = (mr == -INFINITY) ? 0.f : exp2f(mr - mn);
      float sm = swm[0], sq = swq[0];
#pragma unroll
      for (int h = 1; h < FA_GMAX; ++h)
        if (hl == h) { sm = swm[h]; sq = swq[h]; }
      const float im = sm > 0.f ? 1.f / sm : 0.f, iq = sq > 0.f ? 1.f / sq : 0.f;
#pragma unroll
      for (int p = 0; p <= VMP; ++p) {
        const float isc = p < VMP ? im : iq;
#pragma unroll
        for (int c = 0; c < NT_W; ++c) {
          const float x = ((float)vacc[p][c][0] + (float)vacc[p][c][1] * (1.f / 128.f) +
                           (float)vacc[p][c][2] * (1.f / 16384.f) + (float)vacc[p][c][3] * (1.f / 2097152.f)) * isc;
          acc[p][c] = acc[p][c] * alpha + x;
        }
      }
      l_run = l_run * alpha + ps;
      ym_run = ym_run * alpha + pm;
      yq_run = yq_run * alpha + pq;
#pragma unroll
      for (int h = 0; h < FA_GMAX; ++h) m_run[h] = mnew[h];
    }
  }

  // ---------------- partial record: m, l, acc_mse[D], acc_qjl[D] ----------------
  if (hl < gw) {
    float *dst = a.part + (((int64_t)b * a.Hq + h0 + hl) * a.nsplit + split) * (2 + 2 * (int64_t)D);
    float mr = m_run[0];
#pragma unroll
    for (int h = 1; h < FA_GMAX; ++h)
      if (hl == h) mr = m_run[h];
    if (wave == 0 && (lane & 15) == 0) { dst[0] = mr; dst[1] = l_run; }
#pragma unroll
    for (int c = 0; c < NT_W; ++c) {
      const int col = (wave * NT_W + c) * 16 + (lane & 15);
      float am = 0.f;
#pragma unroll
      for (int p = 0; p < VMP; ++p) am += a.vbeta[p] * (2.f * acc[p][c] - ym_run);
      dst[2 + col] = am;
      dst[2 + D + col] = a.vqjl * (2.f * acc[VMP][c] - yq_run);
    }
  }
}

// ---------------------------------------------------------------------------
// query operand images: q' = Pi_K q, Walsh-weighted, 2^-k folded, three int8 splits
// ---------------------------------------------------------------------------
struct PrepArgs {
  const void *q;
  int qt, Hq, Hkv, G, nsub;
  const float *pi;
  float kbeta[8];
  float ctop;
  int *qimg;
  float *qinfo;
};

template <int D, int KB>
__global__ __launch_bounds__(256) void attn_fast_prep_kernel(PrepArgs a) {
  constexpr int KP = walsh_count(KB);
  constexpr int NINS = KP * (D / 128) * 2;
  __shared__ float qs[FA_GMAX][D];
  __shared__ float qp[FA_GMAX][D];
  __shared__ float red[FA_GMAX][2];
  const int unit = blockIdx.x;
  const int sub = unit % a.nsub, bg = unit / a.nsub;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int h0 = g * a.G + sub * FA_GMAX;
  const int gw = min(FA_GMAX, a.G - sub * FA_GMAX);
  for (int e = threadIdx.x; e < FA_GMAX * D; e += 256) {
    const int h = e / D, j = e % D;
    float v = 0.f;
    if (h < gw) {
      const int64_t off = ((int64_t)b * a.Hq + h0 + h) * D + j;
      if (a.qt == TQ_F32) v = static_cast<const float *>(a.q)[off];
      else if (a.qt == TQ_BF16) v = bf16_to_f32(static_cast<const uint16_t *>(a.q)[off]);
      else v = f16_to_f32(static_cast<const uint16_t *>(a.q)[off]);
    }
    qs[h][j] = v;
  }
  if (threadIdx.x < FA_GMAX * 2) red[threadIdx.x / 2][threadIdx.x % 2] = 0.f;
  __syncthreads();
  for (int e = threadIdx.x; e < FA_GMAX * D; e += 256) {
    const int h = e / D, j = e % D;
    float acc = 0.f;
    if (h < gw) {
      const float *row = a.pi + (int64_t)j * D;
      for (int k = 0; k < D; ++k) acc = fmaf(row[k], qs[h][k], acc);
    }
    qp[h][j] = acc;
  }
  __syncthreads();
  // per head: sum q' and max |q'_j 2^-k_j|
  {
    const int h = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float sm = 0.f, mx = 0.f;
    for (int j = lane; j < D; j += 64) {
      sm += qp[h][j];
      mx = fmaxf(mx, fabsf(qp[h][j]) / (float)(1 << (j & 7)));
    }
    sm = wave_sum_f32(sm);
    mx = wave_max_f32(mx);
    if (lane == 0) { red[h][0] = sm; red[h][1] = mx; }
  }
  __syncthreads();
  float bmax = 0.f;
#pragma unroll
  for (int p = 0; p < KP; ++p) bmax = fmaxf(bmax, fabsf(2.f * a.kbeta[p]));
  // image
  for (int e = threadIdx.x; e < NINS * 64 * 4; e += 256) {
    const int r = e & 3, lane = (e >> 2) & 63, ins = e >> 8;
    const int half = ins & 1, pw = ins >> 1, wb = pw % (D / 128), p = pw / (D / 128);
    const int m = lane & 15, h = m >> 2, sp = m & 3, gq = lane >> 4;
    uint32_t word = 0;
    if (h < gw) {
      const float mx = red[h][1] * bmax;
      const float sq = mx > 0.f ? 127.f / mx : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 32 * (4 * wb + gq) + 8 * i + 4 * half + r;
        const int kb = j & 7;
        const float ks = kb == 7 ? -1.f / 128.f : 1.f / (float)(1 << kb);
        int8_t o[4];
        split4(2.f * a.kbeta[p] * qp[h][j] * ks * sq, o);
        word |= (uint32_t)(uint8_t)o[sp] << (8 * i);
      }
    }
    a.qimg[(((int64_t)unit * NINS + ins) * 64 + lane) * 4 + r] = (int)word;
  }
  if (threadIdx.x < FA_GMAX) {
    const int h = threadIdx.x;
    const float mx = red[h][1] * bmax;
    const float sq = mx > 0.f ? 127.f / mx : 0.f;
    a.qinfo[((int64_t)unit * FA_GMAX + h) * 2 + 0] = (h < gw && sq > 0.f) ? 1.f / sq : 0.f;
    a.qinfo[((int64_t)unit * FA_GMAX + h) * 2 + 1] = h < gw ? a.ctop * red[h][0] : 0.f;
  }
}

// ---------------------------------------------------------------------------
// token-tiled layout: word [seq][tile][plane][coord] bit i = plane bit of token 32*tile + i
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void tile_records_kernel(const uint8_t *codes, int64_t cb, int planes, int D,
                                                          int64_t T, int64_t ntile, uint32_t *tiles) {
  const int lane = threadIdx.x;
  const int64_t seq = blockIdx.y;
  const int64_t tp = blockIdx.x;  // pair of tiles
  const int64_t t = tp * 64 + lane;
  const uint32_t *rec = reinterpret_cast<const uint32_t *>(codes + (seq * T + t) * cb);
  const int wpp = D / 32;
  for (int wi = 0; wi < planes * wpp; ++wi) {
    const uint32_t w = t < T ? rec[wi] : 0u;
    uint32_t lo = 0, hi = 0;
    for (int i = 0; i < 32; ++i) {
      const unsigned long long m = __ballot((w >> i) & 1u);
      if (lane == i) { lo = (uint32_t)m; hi = (uint32_t)(m >> 32); }
    }
    const int p = wi / wpp, j = (wi % wpp) * 32 + lane;
    if (lane < 32) {
      const int64_t t0 = 2 * tp, t1 = 2 * tp + 1;
      if (t0 < ntile) tiles[((seq * ntile + t0) * planes + p) * D + j] = lo;
      if (t1 < ntile) tiles[((seq * ntile + t1) * planes + p) * D + j] = hi;
    }
  }
}

int run_tile_records(const tq_quantizer *q, const uint8_t *codes, int64_t nseq, int64_t T, uint32_t *tiles,
                     hipStream_t st) {
  const int64_t ntile = (T + 31) / 32;
  if (nseq == 0 || ntile == 0) return TQ_OK;
  ProfScope ps("tile_records", st);
  dim3 grid((unsigned)((ntile + 1) / 2), (unsigned)nseq);
  hipLaunchKernelGGL(tile_records_kernel, grid, dim3(64), 0, st, codes, (int64_t)q->code_bytes, q->planes, q->d, T,
                     ntile, tiles);
  return launch_check();
}

// ---------------------------------------------------------------------------
// host dispatch
// ---------------------------------------------------------------------------
namespace {

// Walsh coefficients beta_S (odd subsets, enumeration order of walsh_planes) of a symmetric codebook
void walsh_coeffs(const double *c, int bits, double *beta) {
  static const int subs[4][8] = {{0x1}, {0x1, 0x2}, {0x1, 0x2, 0x4, 0x7}, {0x1, 0x2, 0x4, 0x8, 0x7, 0xB, 0xD, 0xE}};
  const int L = 1 << bits, n = 1 << (bits - 1);
  for (int s = 0; s < n; ++s) {
    double acc = 0.0;
    for (int idx = 0; idx < L; ++idx) {
      double sign = 1.0;
      for (int p = 0; p < bits; ++p)
        if (subs[bits - 1][s] >> p & 1) sign *= ((idx >> p) & 1) ? 1.0 : -1.0;
      acc += c[idx] * sign;
    }
    beta[s] = acc / L;
  }
}

struct FastPlan {
  int nsub, nsplit, chunk, nins;
  size_t img_off, info_off, part_off, total;
};

FastPlan fast_plan(int D, int KB, int B, int Hq, int Hkv, int64_t T) {
  FastPlan p{};
  const int G = Hq / Hkv;
  p.nsub = (G + FA_GMAX - 1) / FA_GMAX;
  p.nins = walsh_count(KB) * (D / 128) * 2;
  const int64_t units = (int64_t)B * Hkv * p.nsub;
  const int64_t want = std::max<int64_t>(1, 2048 / std::max<int64_t>(units, 1));
  int64_t chunk = (T + want - 1) / want;
  chunk = std::max<int64_t>(4 * FA_SUB, (chunk + FA_SUB - 1) / FA_SUB * FA_SUB);
  p.chunk = (int)std::min<int64_t>(chunk, 1 << 30);
  p.nsplit = (int)std::max<int64_t>(1, (T + p.chunk - 1) / p.chunk);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.img_off = 0;
  p.info_off = al((size_t)units * p.nins * 64 * 16);
  p.part_off = p.info_off + al((size_t)units * FA_GMAX * 2 * 4);
  p.total = p.part_off + (size_t)B * Hq * p.nsplit * (2 + 2 * (size_t)D) * 4;
  return p;
}

bool fast_supported(int D, int KB, int VB) {
  if (D != 128 && D != 256) return false;
  if (KB < 1 || KB > 4 || VB < 1 || VB > 3) return false;
  return walsh_count(KB) * (D / 128) * 2 <= 16;
}

template <int D, int KB, int VB>
int launch_fast(const FastPlan &fp, const FastAttnArgs &fa, const PrepArgs &pa, int units, hipStream_t st) {
  {
    ProfScope ps("attn_prep", st);
    hipLaunchKernelGGL((attn_fast_prep_kernel<D, KB>), dim3(units), dim3(256), 0, st, pa);
  }
  int rc = launch_check();
  if (rc != TQ_OK) return rc;
  ProfScope ps("attn_split", st);
  hipLaunchKernelGGL((attn_fast_kernel<D, KB, VB>), dim3(units, fp.nsplit), dim3(FA_THREADS), 0, st, fa);
  return launch_check();
}

}  // namespace

size_t attn_fast_ws_bytes(int D, int KB, int B, int Hq, int Hkv, int64_t T) {
  return fast_plan(D, KB, B, Hq, Hkv, T).total;
}

int attn_combine(const float *part, int BH, int nsplit, int d, const float *piT, const float *sT, float *out,
                 hipStream_t st);

int run_attn_fast(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int Hq, int Hkv,
                  const uint8_t *kcodes, const uint16_t *knorms, const uint32_t *vtiles, const uint16_t *vnorms,
                  const uint16_t *vgammas, int64_t Tstride, const int32_t *seq_len, float scale, float *out,
                  void *ws, hipStream_t st) {
  const int D = kq->d, KB = kq->bits, VB = vq->bmse;
  if (!fast_supported(D, KB, VB)) return TQ_ERR_UNSUPPORTED;
  FastPlan fp = fast_plan(D, KB, B, Hq, Hkv, Tstride);
  const int units = B * Hkv * fp.nsub;
  char *w = static_cast<char *>(ws);
  double kb64[8] = {0}, vb64[4] = {0};
  walsh_coeffs(kq->c64, KB, kb64);
  walsh_coeffs(vq->c64, VB, vb64);
  PrepArgs pa{};
  pa.q = q; pa.qt = qt; pa.Hq = Hq; pa.Hkv = Hkv; pa.G = Hq / Hkv; pa.nsub = fp.nsub; pa.pi = kq->pi;
  for (int i = 0; i < 8; ++i) pa.kbeta[i] = (float)kb64[i];
  pa.ctop = (float)kq->c64[(1 << KB) - 1];
  pa.qimg = reinterpret_cast<int *>(w + fp.img_off);
  pa.qinfo = reinterpret_cast<float *>(w + fp.info_off);
  FastAttnArgs fa{};
  fa.qimg = pa.qimg; fa.qinfo = pa.qinfo; fa.kcodes = kcodes; fa.knorms = knorms; fa.vtiles = vtiles;
  fa.vnorms = vnorms; fa.vgammas = vgammas; fa.seq_len = seq_len;
  fa.part = reinterpret_cast<float *>(w + fp.part_off);
  fa.Tstride = Tstride; fa.ntile = (Tstride + 31) / 32;
  fa.Hq = Hq; fa.Hkv = Hkv; fa.G = Hq / Hkv; fa.nsub = fp.nsub; fa.chunk = fp.chunk; fa.nsplit = fp.nsplit;
  fa.scale_log2 = scale * 1.4426950408889634f;
  fa.vqjl = vq->qjl_scale;
  for (int i = 0; i < 4; ++i) fa.vbeta[i] = (float)vb64[i];
  int rc = TQ_ERR_UNSUPPORTED;
#define TQ_FAST(DD, KK, VV) \
  if (D == DD && KB == KK && VB == VV) rc = launch_fast<DD, KK, VV>(fp, fa, pa, units, st);
  TQ_FAST(128, 1, 1) TQ_FAST(128, 2, 1) TQ_FAST(128, 3, 1) TQ_FAST(128, 4, 1)
  TQ_FAST(128, 1, 2) TQ_FAST(128, 2, 2) TQ_FAST(128, 3, 2) TQ_FAST(128, 4, 2)
  TQ_FAST(128, 1, 3) TQ_FAST(128, 2, 3) TQ_FAST(128, 3, 3) TQ_FAST(128, 4, 3)
  TQ_FAST(256, 1, 1) TQ_FAST(256, 2, 1) TQ_FAST(256, 3, 1)
  TQ_FAST(256, 1, 2) TQ_FAST(256, 2, 2) TQ_FAST(256, 3, 2)
  TQ_FAST(256, 1, 3) TQ_FAST(256, 2, 3) TQ_FAST(256, 3, 3)
#undef TQ_FAST
  if (rc != TQ_OK) return rc;
  return attn_combine(fa.part, B * Hq, fp.nsplit, D, vq->piT, vq->sT, out, st);
}

}  // namespace tq
