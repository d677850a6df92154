// Inner-product scoring of queries against packed records on the int8 matrix cores, and top-k.
//
// The estimate is the one of the ai-navigate-news Gemma 4 post (section
// "仕組み（技術的）"): for a record x with index planes, norm n and (Algorithm 2)
// sign plane s and residual norm gamma,
//     est(q, x) = n <Pi q, c[idx]> + sqrt(pi/2)/d * gamma <S q, 2 s - 1>,
// used for search as in the AiBoss overview (section "TurboQuantの応用事例").
//
// A symmetric codebook is an odd function of the index bits, so with the Walsh
// planes b_S (odd-size subsets of the index bits, XORed)
//     <q', c[idx]> = sum_S 2 beta_S <q', b_S> - c[L-1] sum_j q'_j,
//     <q'', 2 s - 1> = 2 <q'', s> - sum_j q''_j          (q' = Pi q, q'' = S q).
// Every term is a contraction of a query against a 0/1 bit plane, which the
// int8 matrix cores take directly: the database bits are spread to 0/1 bytes
// (B operand, 16 records x 64 coordinates per fragment), and the queries are
// int8 images 2 beta_S q' (and q'') scaled per query to 127 and split into two
// 7-bit digits, one MFMA row per (query, digit), so a 16-row fragment holds 8
// queries.  Integer accumulation is exact; the only rounding is the two-digit
// split (2^-15 of the query's largest image entry).
//
// Work split: a work-group takes 32 queries (4 fragments) x 256 records; each
// wave owns 64 records (4 fragments) and keeps the 4 x 4 accumulator tiles of
// the Algorithm-1 sum (all Walsh images accumulate into one, their beta folded
// into the images) and of the sign sum in registers.  The 64-coordinate query
// images of each step are staged in LDS (double-buffered) and shared by the
// four waves; each wave expands its records' bits once per step and feeds each
// expanded fragment to the four query fragments.
//
// Contraction order: the matrix cores sum over the 64 k-slots of a step in any
// order as long as both operands agree, so the coordinates are dealt to the
// slots by super-steps of SPS steps: lane group g owns 16 SPS contiguous
// coordinates of a super-step, which it reads as one 2 SPS-byte word per plane,
// prefetched a super-step ahead.  With whole 32-bit words (SPS >= 2) a step
// takes one nibble half of a word and each B register is that word ANDed with
// 0x01010101 << r: bytes of value 2^r (r < 4), whose 2^-r the query images
// carry (1 shift and 4 ANDs per fragment instead of spreading bits to bytes).
#include <algorithm>

#include "common.cuh"

namespace tq {

constexpr int SC_Q = 32;        // queries per work-group (4 fragments of 8 queries x 2 digits)
constexpr int SC_R = 256;       // records per work-group (4 waves x 64)
constexpr int SC_K = 64;        // coordinates per step (one v_mfma_i32_16x16x64_i8)

struct ScoreArgs {
  const int8_t *img;      // [groups][steps][nimg][4 fragments][64 lanes][16 B]
  const float *info;      // [m_pad][4]: 1/scale_mse, 1/scale_sign, c[L-1] sum q', sum q''
  const uint8_t *codes;   // [n][code_bytes]
  const uint16_t *norms, *gammas;
  float *scores;          // [m][ld]
  int64_t n, m, ld, code_bytes;
  int d, nsteps, ngroups;
  float qjl;
};

// 16 bits -> 16 bytes of 0/1 (byte i = bit i): a nibble times 0x204081 puts its bits at 0, 8, 16, 24
__device__ __forceinline__ intx4 spread_bits16(uint32_t h) {
  intx4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (int)((((h >> (4 * i)) & 0xFu) * 0x204081u) & 0x01010101u);
  return r;
}

// a lane's bits of one plane for a super-step of SPS steps (2 SPS bytes)
template <int SPS>
struct SuperBits;
template <>
struct SuperBits<1> {
  uint32_t w;
  __device__ __forceinline__ void load(const uint8_t *p) { w = *reinterpret_cast<const uint16_t *>(p); }
  __device__ __forceinline__ uint32_t step(int) const { return w; }
};
template <>
struct SuperBits<2> {
  uint32_t w;
  __device__ __forceinline__ void load(const uint8_t *p) { w = *reinterpret_cast<const uint32_t *>(p); }
  __device__ __forceinline__ uint32_t step(int u) const { return (w >> (16 * u)) & 0xFFFFu; }
  __device__ __forceinline__ uint32_t nib(int u) const { return w >> (4 * u); }
};
template <>
struct SuperBits<4> {
  uint32_t w0, w1;
  __device__ __forceinline__ void load(const uint8_t *p) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    w0 = v.x;
    w1 = v.y;
  }
  __device__ __forceinline__ uint32_t step(int u) const { return ((u < 2 ? w0 : w1) >> (16 * (u & 1))) & 0xFFFFu; }
  __device__ __forceinline__ uint32_t nib(int u) const { return (u < 2 ? w0 : w1) >> (4 * (u & 1)); }
};

template <bool PROD, int BM, int SPS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void score_scan_kernel(ScoreArgs a) {
  constexpr int KP = walsh_count(BM);          // Walsh images of the index part
  constexpr int NIMG = KP + (PROD ? 1 : 0);    // + the sign image
  constexpr int NPL = BM + (PROD ? 1 : 0);     // stored planes per record
  __shared__ __attribute__((aligned(16))) intx4 As[2][NIMG][4][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // query group fastest: consecutive work-groups (spread over the XCDs) share a record tile, and each XCD's
  // L2 holds the images of the few query groups dealt to it while the records stream past
  const int group = (int)(blockIdx.x % a.ngroups);
  const int64_t rec0 = (int64_t)(blockIdx.x / a.ngroups) * SC_R + 64 * wave;
  const int col = lane & 15, kq = lane >> 4;
  const int pb = a.d / 8;  // bytes per plane

  // record rows of this lane's four fragments (rows past the end read row 0, results dropped)
  const uint8_t *rec[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int64_t r = rec0 + 16 * rb + col;
    rec[rb] = a.codes + (r < a.n ? r : 0) * a.code_bytes + 2 * SPS * kq;
  }
  const intx4 *img = reinterpret_cast<const intx4 *>(a.img) + (int64_t)group * a.nsteps * NIMG * 4 * 64;

  intx4 accm[4][4], accq[PROD ? 4 : 1][4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      accm[qb][rb] = intx4{0, 0, 0, 0};
      if (PROD) accq[qb][rb] = intx4{0, 0, 0, 0};
    }

  // query images of a step: NIMG x 4 fragments x 64 lanes x 16 B, one 16 B piece per thread per pass
  intx4 ai[NIMG];
  auto load_a = [&](int st) {
#pragma unroll
    for (int s = 0; s < NIMG; ++s) ai[s] = img[((int64_t)st * NIMG + s) * 256 + tid];
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int s = 0; s < NIMG; ++s) As[buf][s][tid >> 6][tid & 63] = ai[s];
  };
  SuperBits<SPS> bcur[4][NPL], bnext[4][NPL];
  auto load_b = [&](SuperBits<SPS>(&bw)[4][NPL], int ss) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int p = 0; p < NPL; ++p) bw[rb][p].load(rec[rb] + p * pb + 8 * SPS * ss);
  };

  const int nss = a.nsteps / SPS;
  load_a(0);
  store_a(0);
  load_b(bcur, 0);
  __syncthreads();
  for (int ss = 0; ss < nss; ++ss) {
    if (ss + 1 < nss) load_b(bnext, ss + 1);  // a whole super-step ahead
#pragma unroll
    for (int u = 0; u < SPS; ++u) {
      const int st = ss * SPS + u, buf = st & 1;
      // this step's record bits: Walsh planes of the index bits, and the sign plane
      uint32_t wpl[4][NIMG];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        uint32_t w[NPL];
#pragma unroll
        for (int p = 0; p < NPL; ++p) {
          if constexpr (SPS == 1) w[p] = bcur[rb][p].step(u);
          else w[p] = bcur[rb][p].nib(u);
        }
        walsh_planes<BM>(w, wpl[rb]);
        if (PROD) wpl[rb][KP] = w[BM];
      }
      if (st + 1 < a.nsteps) load_a(st + 1);
#pragma unroll
      for (int s = 0; s < NIMG; ++s) {
        intx4 af[4];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) af[qb] = As[buf][s][qb][lane];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          // SPS >= 2: nibble position r of each byte of the lane's word (bytes 2^r; the images carry 2^-r)
          const uint32_t x = wpl[rb][s];
          const intx4 bf = SPS == 1 ? spread_bits16(x)
                                    : intx4{(int)(x & 0x01010101u), (int)(x & 0x02020202u), (int)(x & 0x04040404u),
                                            (int)(x & 0x08080808u)};
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) {
            if (PROD && s == KP) accq[qb][rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[qb], bf, accq[qb][rb], 0, 0, 0);
            else accm[qb][rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[qb], bf, accm[qb][rb], 0, 0, 0);
          }
        }
      }
      if (st + 1 < a.nsteps) {
        store_a(buf ^ 1);  // the other buffer was last read in the previous step, before its barrier
        __syncthreads();
      }
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int p = 0; p < NPL; ++p) bcur[rb][p] = bnext[rb][p];
  }

  // scores: lane holds MFMA rows 4 kq + e = (query 2 kq + e / 2, digit e % 2) of record col
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int64_t r = rec0 + 16 * rb + col;
    if (r >= a.n) continue;
    const float nh = f16_to_f32(a.norms[r]);
    const float gq = PROD ? a.qjl * f16_to_f32(a.gammas[r]) : 0.f;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t q = (int64_t)group * SC_Q + qb * 8 + 2 * kq + h;
        if (q >= a.m) continue;
        const float4 in = *reinterpret_cast<const float4 *>(a.info + 4 * q);
        const float vm = (float)accm[qb][rb][2 * h] + (float)accm[qb][rb][2 * h + 1] * (1.f / 128.f);
        float sc = nh * (vm * in.x - in.z);
        if (PROD) {
          const float vq = (float)accq[qb][rb][2 * h] + (float)accq[qb][rb][2 * h + 1] * (1.f / 128.f);
          sc += gq * (2.f * vq * in.y - in.w);
        }
        a.scores[q * a.ld + r] = sc;
      }
  }
}

// ---------------------------------------------------------------------------
// query images: one work-group per query (padding queries get zero images)
// ---------------------------------------------------------------------------
struct ScorePrepArgs {
  const float *qrot;      // [m][kq]: Pi q (d) then S q (d, Algorithm 2)
  int64_t m, kq;
  int d, nsteps, kp, prod, sps;
  float beta[8];          // Walsh coefficients of the codebook
  float ctop;
  int8_t *img;
  float *info;
};

__global__ __launch_bounds__(256) void score_prep_kernel(ScorePrepArgs a) {
  const int64_t q = blockIdx.x;
  const int nimg = a.kp + a.prod;
  __shared__ float red[4][4];
  const bool valid = q < a.m;
  const float *qp = a.qrot + (valid ? q : 0) * a.kq;
  // largest |2 beta_S q'_j| and |q''_j|, sums of q' and q''
  float bmax = 0.f;
  for (int s = 0; s < a.kp; ++s) bmax = fmaxf(bmax, fabsf(2.f * a.beta[s]));
  float mm = 0.f, mq = 0.f, sm = 0.f, sq = 0.f;
  for (int j = threadIdx.x; j < a.d; j += 256) {
    const float v = qp[j];
    mm = fmaxf(mm, fabsf(v) * bmax);
    sm += v;
    if (a.prod) {
      const float w = qp[a.d + j];
      mq = fmaxf(mq, fabsf(w));
      sq += w;
    }
  }
  mm = wave_max_f32(mm); mq = wave_max_f32(mq); sm = wave_sum_f32(sm); sq = wave_sum_f32(sq);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[w][0] = mm; red[w][1] = mq; red[w][2] = sm; red[w][3] = sq; }
  __syncthreads();
  mm = fmaxf(fmaxf(red[0][0], red[1][0]), fmaxf(red[2][0], red[3][0]));
  mq = fmaxf(fmaxf(red[0][1], red[1][1]), fmaxf(red[2][1], red[3][1]));
  sm = (red[0][2] + red[1][2]) + (red[2][2] + red[3][2]);
  sq = (red[0][3] + red[1][3]) + (red[2][3] + red[3][3]);
  const float scm = mm > 0.f ? 127.f / mm : 0.f, scq = mq > 0.f ? 127.f / mq : 0.f;
  if (threadIdx.x == 0) {
    a.info[4 * q + 0] = (valid && scm > 0.f) ? 1.f / scm : 0.f;
    a.info[4 * q + 1] = (valid && scq > 0.f) ? 1.f / scq : 0.f;
    a.info[4 * q + 2] = valid ? a.ctop * sm : 0.f;
    a.info[4 * q + 3] = valid ? sq : 0.f;
  }
  // image bytes: fragment row 2 qi + digit, lane = row + 16 (k / 16), byte k % 16
  const int64_t group = q / SC_Q;
  const int qb = (int)(q % SC_Q) / 8, qi = (int)(q % 8);
  for (int e = threadIdx.x; e < a.nsteps * nimg * SC_K; e += 256) {
    const int k = e % SC_K, s = (e / SC_K) % nimg, st = e / (SC_K * nimg);
    // coordinate of slot k of step st.  sps == 1: lane group g = k / 16 takes coordinates 16 g + (k % 16)
    // of the step, bytes 0/1.  sps >= 2: lane group g owns 16 sps coordinates of the super-step (sps / 2
    // words); step u reads nibble half u % 2 of word u / 2, and slot 4 r + j of the group (r, j < 4) holds
    // bit 8 j + r + 4 (u % 2) of that word as a byte of value 2^r, so its image carries 2^-r
    const int g = k / 16, i = k % 16, u = st % a.sps, r = a.sps == 1 ? 0 : i / 4;
    const int j = a.sps == 1 ? st * SC_K + 16 * g + i
                             : (st / a.sps) * SC_K * a.sps + 16 * a.sps * g + 32 * (u / 2) + 8 * (i % 4) + r + 4 * (u % 2);
    float v = 0.f;
    if (valid) v = (s < a.kp ? 2.f * a.beta[s] * qp[j] * scm : qp[a.d + j] * scq) * (1.f / (float)(1 << r));
    const float a1 = rintf(v), a2 = rintf((v - a1) * 128.f);
    int8_t *frag = a.img + ((((group * a.nsteps + st) * nimg + s) * 4 + qb) * 64) * 16;
    frag[(2 * qi + 0 + 16 * (k / 16)) * 16 + (k % 16)] = (int8_t)(int)a1;
    frag[(2 * qi + 1 + 16 * (k / 16)) * 16 + (k % 16)] = (int8_t)(int)a2;
  }
}

// ---------------------------------------------------------------------------
// top-k: per (query, chunk) the k best of a range, then per query the k best of the chunks' candidates
// ---------------------------------------------------------------------------
constexpr int TK_THREADS = 256;

__device__ __forceinline__ bool tk_better(float a, int64_t ia, float b, int64_t ib) {
  return a > b || (a == b && ia < ib);
}

// KM: list capacity (k <= KM); in_idx: indices of the inputs (nullptr: the position is the index)
template <int KM>
__global__ __launch_bounds__(TK_THREADS) void topk_chunk_kernel(const float *vals, const int64_t *in_idx, int64_t ld,
                                                                int64_t len, int64_t chunk, int k, float *out_v,
                                                                int64_t *out_i) {
  const int64_t qi = blockIdx.x, ci = blockIdx.y;
  const int64_t c0 = ci * chunk, c1 = imin64(len, c0 + chunk);
  const float *row = vals + qi * ld;
  const int64_t *irow = in_idx ? in_idx + qi * ld : nullptr;
  float lv[KM];
  int64_t li[KM];
#pragma unroll
  for (int i = 0; i < KM; ++i) { lv[i] = -INFINITY; li[i] = INT64_MAX; }
  auto insert = [&](float v, int64_t id) {
    if (!tk_better(v, id, lv[k - 1], li[k - 1])) return;
    // insert keeping lv descending (entries past k stay unused)
    bool placed = false;
#pragma unroll
    for (int i = KM - 1; i >= 0; --i) {
      if (i >= k || placed) continue;
      const bool up = i > 0 && tk_better(v, id, lv[i - 1], li[i - 1]);
      if (up) { lv[i] = lv[i - 1]; li[i] = li[i - 1]; }
      else { lv[i] = v; li[i] = id; placed = true; }
    }
  };
  // four loads in flight per thread; positions rise per thread, so equal values keep the lower index
  int64_t p = c0 + threadIdx.x;
  for (; p + 3 * TK_THREADS < c1; p += 4 * TK_THREADS) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = row[p + u * TK_THREADS];
#pragma unroll
    for (int u = 0; u < 4; ++u) insert(v[u], irow ? irow[p + u * TK_THREADS] : p + u * TK_THREADS);
  }
  for (; p < c1; p += TK_THREADS) insert(row[p], irow ? irow[p] : p);
  __shared__ float sv[TK_THREADS];
  __shared__ int64_t si[TK_THREADS];
  __shared__ int sw[TK_THREADS];
  int head = 0;
  for (int out = 0; out < k; ++out) {
    float hv = -INFINITY;
    int64_t hi = INT64_MAX;
#pragma unroll
    for (int i = 0; i < KM; ++i)
      if (i == head) { hv = lv[i]; hi = li[i]; }
    sv[threadIdx.x] = hv;
    si[threadIdx.x] = hi;
    sw[threadIdx.x] = threadIdx.x;
    __syncthreads();
    for (int s = TK_THREADS / 2; s > 0; s >>= 1) {
      if (threadIdx.x < s) {
        const int o = threadIdx.x + s;
        if (tk_better(sv[o], si[o], sv[threadIdx.x], si[threadIdx.x])) {
          sv[threadIdx.x] = sv[o];
          si[threadIdx.x] = si[o];
          sw[threadIdx.x] = sw[o];
        }
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) {
      out_v[(qi * gridDim.y + ci) * k + out] = sv[0];
      out_i[(qi * gridDim.y + ci) * k + out] = si[0];
    }
    if (threadIdx.x == sw[0]) ++head;
    __syncthreads();
  }
}

template <int KM>
static void launch_topk(const float *vals, const int64_t *in_idx, int64_t ld, int64_t len, int64_t m, int nchunk,
                        int k, float *ov, int64_t *oi, hipStream_t st) {
  const int64_t chunk = cdiv64(len, nchunk);
  hipLaunchKernelGGL((topk_chunk_kernel<KM>), dim3((unsigned)m, (unsigned)nchunk), dim3(TK_THREADS), 0, st, vals,
                     in_idx, ld, len, chunk, k, ov, oi);
}

static void topk_pass(const float *vals, const int64_t *in_idx, int64_t ld, int64_t len, int64_t m, int nchunk, int k,
                      float *ov, int64_t *oi, hipStream_t st) {
  if (k <= 16) launch_topk<16>(vals, in_idx, ld, len, m, nchunk, k, ov, oi, st);
  else launch_topk<64>(vals, in_idx, ld, len, m, nchunk, k, ov, oi, st);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

struct ScorePlan {
  int nsteps, nimg, kp, ngroups, nchunk;
  size_t qrot_off, img_off, info_off, scores_off, cand_v_off, cand_i_off, total;
};

int topk_chunks(int64_t m, int64_t n, int k) {
  if (k <= 0) return 0;
  int64_t c = std::max<int64_t>(1, 16384 / std::max<int64_t>(m, 1));
  c = std::min<int64_t>(c, std::max<int64_t>(1, n / std::max<int64_t>(4096, 4 * (int64_t)k)));
  return (int)std::min<int64_t>(c, 256);
}

ScorePlan score_plan(const tq_quantizer *q, int64_t m, int64_t n, int k) {
  ScorePlan p{};
  const bool prod = q->mode == TQ_PROD;
  p.kp = walsh_count(q->bmse);
  p.nimg = p.kp + (prod ? 1 : 0);
  p.nsteps = q->d / SC_K;
  p.ngroups = (int)cdiv64(m, SC_Q);
  p.nchunk = topk_chunks(m, n, k);
  const int kqd = prod ? 2 * q->d : q->d;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.qrot_off = 0;
  p.img_off = al((size_t)m * kqd * 4);
  p.info_off = p.img_off + al((size_t)p.ngroups * p.nsteps * p.nimg * 4 * 64 * 16);
  p.scores_off = p.info_off + al((size_t)p.ngroups * SC_Q * 4 * 4);
  p.total = p.scores_off;
  if (k > 0) {
    p.cand_v_off = p.scores_off + al((size_t)m * n * 4);
    p.cand_i_off = p.cand_v_off + al((size_t)m * p.nchunk * k * 4);
    p.total = p.cand_i_off + (size_t)m * p.nchunk * k * 8;
  }
  return p;
}

// steps per super-step: the largest of 4, 2, 1 that divides the step count
int score_sps(int d) { return (d / SC_K) % 4 == 0 ? 4 : (d / SC_K) % 2 == 0 ? 2 : 1; }

template <bool PROD, int BM>
void launch_scan(const ScoreArgs &sa, int64_t n, int ngroups, int sps, hipStream_t st) {
  const dim3 grid((unsigned)(cdiv64(n, SC_R) * ngroups));
  if (sps == 4) hipLaunchKernelGGL((score_scan_kernel<PROD, BM, 4>), grid, dim3(256), 0, st, sa);
  else if (sps == 2) hipLaunchKernelGGL((score_scan_kernel<PROD, BM, 2>), grid, dim3(256), 0, st, sa);
  else hipLaunchKernelGGL((score_scan_kernel<PROD, BM, 1>), grid, dim3(256), 0, st, sa);
}

}  // namespace

bool score_planes_supported(const tq_quantizer *q) { return q->d % SC_K == 0 && q->bmse >= 1 && q->bmse <= 3; }

size_t score_planes_ws_bytes(const tq_quantizer *q, int64_t m, int64_t n, int k) { return score_plan(q, m, n, k).total; }

int rotate_queries(const tq_quantizer *q, const float *queries, int64_t m, int64_t ldq, float *qrot, hipStream_t st);

int run_score_planes(const tq_quantizer *q, const float *queries, int64_t m, int64_t ldq, const uint8_t *codes,
                     const uint16_t *norms, const uint16_t *gammas, int64_t n, int k, float *scores, int64_t *idx,
                     void *ws, hipStream_t st) {
  if (m <= 0) return TQ_OK;
  const bool prod = q->mode == TQ_PROD;
  const ScorePlan p = score_plan(q, m, n, k);
  char *w = static_cast<char *>(ws);
  float *qrot = reinterpret_cast<float *>(w + p.qrot_off);
  int rc = rotate_queries(q, queries, m, ldq, qrot, st);
  if (rc != TQ_OK || n == 0) return rc;
  double b64[8] = {0};
  walsh_coeffs(q->c64, q->bmse, b64);
  ScorePrepArgs pa{};
  pa.qrot = qrot; pa.m = m; pa.kq = prod ? 2 * q->d : q->d; pa.d = q->d; pa.nsteps = p.nsteps; pa.kp = p.kp;
  pa.prod = prod ? 1 : 0;
  pa.sps = score_sps(q->d);
  for (int i = 0; i < 8; ++i) pa.beta[i] = (float)b64[i];
  pa.ctop = (float)q->c64[(1 << q->bmse) - 1];
  pa.img = reinterpret_cast<int8_t *>(w + p.img_off);
  pa.info = reinterpret_cast<float *>(w + p.info_off);
  {
    ProfScope ps("score_prep", st);
    hipLaunchKernelGGL(score_prep_kernel, dim3((unsigned)(p.ngroups * SC_Q)), dim3(256), 0, st, pa);
  }
  if ((rc = launch_check()) != TQ_OK) return rc;
  ScoreArgs sa{};
  sa.img = pa.img; sa.info = pa.info; sa.codes = codes; sa.norms = norms; sa.gammas = gammas;
  sa.scores = k > 0 ? reinterpret_cast<float *>(w + p.scores_off) : scores;
  sa.n = n; sa.m = m; sa.ld = n; sa.code_bytes = (int64_t)q->code_bytes; sa.d = q->d; sa.nsteps = p.nsteps;
  sa.qjl = q->qjl_scale;
  sa.ngroups = p.ngroups;
  {
    ProfScope ps("score_scan", st);
    if (prod) {
      if (q->bmse == 1) launch_scan<true, 1>(sa, n, p.ngroups, pa.sps, st);
      else if (q->bmse == 2) launch_scan<true, 2>(sa, n, p.ngroups, pa.sps, st);
      else launch_scan<true, 3>(sa, n, p.ngroups, pa.sps, st);
    } else {
      if (q->bmse == 1) launch_scan<false, 1>(sa, n, p.ngroups, pa.sps, st);
      else if (q->bmse == 2) launch_scan<false, 2>(sa, n, p.ngroups, pa.sps, st);
      else launch_scan<false, 3>(sa, n, p.ngroups, pa.sps, st);
    }
  }
  if ((rc = launch_check()) != TQ_OK || k == 0) return rc;
  float *cv = reinterpret_cast<float *>(w + p.cand_v_off);
  int64_t *ci = reinterpret_cast<int64_t *>(w + p.cand_i_off);
  ProfScope ps("topk", st);
  topk_pass(sa.scores, nullptr, n, n, m, p.nchunk, k, cv, ci, st);
  if ((rc = launch_check()) != TQ_OK) return rc;
  topk_pass(cv, ci, (int64_t)p.nchunk * k, (int64_t)p.nchunk * k, m, 1, k, scores, idx, st);
  return launch_check();
}

}  // namespace tq
