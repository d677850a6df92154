// Decode attention on a TurboQuant-compressed KV cache, split over the sequence.
//
// Keys are Algorithm-1 records and values Algorithm-2 records, the assignment
// made on the ai-navigate-news Gemma 4 post (section "仕組み（技術的）"): K~ for
// the scores, V~ (unbiased) for attn_weights . V.  Nothing is dequantized into
// the original domain: with q' = Pi_K q,
//     <q, K~_t> = n_t <q', c_K[idx_t]>,
//     sum_t p_t V~_t = Pi_V^T (sum_t p_t n_t c_V[idx_t]) + k_d S_V^T (sum_t p_t g_t s_t),
// so the kernels score in the rotated domain, accumulate in the rotated and the
// sign domains, and rotate back once per (batch, head) in the combine step.
//
// Generic path: one wavefront per (batch, kv head, head subgroup, sequence
// split); lane j owns coordinates j, j+64, ...; online softmax per head.
#include "append.cuh"
#include "common.cuh"

namespace tq {

namespace {

constexpr int kAttnChunkMin = 256;

struct AttnPlan {
  int G, GW, nsub, nsplit, chunk, CP;
};

int coords_per_lane_supported(int d) {
  const int cp = d / 64;
  return (cp == 1 || cp == 2 || cp == 4 || cp == 8 || cp == 16 || cp == 24 || cp == 32) ? cp : 0;
}

// heads per wave of attn_split_kernel: 32 query coordinates per lane, half that for Algorithm-2 keys
// (each head also holds S_K q)
constexpr int split_heads(int cp, bool kprod) {
  return kprod ? (32 / cp / 2 > 0 ? 32 / cp / 2 : 1) : (32 / cp > 0 ? 32 / cp : 1);
}

// M query tokens per sequence: M G query rows per (batch, kv-head) pair
AttnPlan make_plan(int d, int B, int Hq, int Hkv, int64_t T, bool kprod, int M = 1) {
  AttnPlan p{};
  p.CP = coords_per_lane_supported(d);
  p.G = Hq / Hkv;
  const int rows = M * p.G;
  p.GW = p.CP ? std::min(rows, split_heads(p.CP, kprod)) : 1;
  p.nsub = (rows + p.GW - 1) / p.GW;
  const int64_t units = (int64_t)B * Hkv * p.nsub;
  int64_t want = std::max<int64_t>(1, 4096 / std::max<int64_t>(units, 1));
  int64_t chunk = std::max<int64_t>(kAttnChunkMin, (T + want - 1) / std::max<int64_t>(want, 1));
  chunk = (chunk + 63) / 64 * 64;
  p.chunk = (int)std::min<int64_t>(chunk, 1 << 30);
  p.nsplit = (int)std::max<int64_t>(1, (T + p.chunk - 1) / p.chunk);
  return p;
}

size_t partial_floats(int d) { return 2 + 2 * (size_t)d; }

}  // namespace

// q'[b,h,:] = Pi_K q[b,h,:] into qrot[bh][0..d), and for Algorithm-2 keys (sT not null) also
// S_K q[b,h,:] into qrot[bh][d..2d); ld = d or 2d.  A decode step that appends a token (app.on) has its
// key and value encoded into the cache by the work-groups of the first two query heads of each kv head.
template <int QT>
__global__ __launch_bounds__(256) void attn_qrot_kernel(const void *q, int d, const float *piT, const float *sT,
                                                        int ld, float *qrot, int Hq, int G, AppendArgs app) {
  extern __shared__ float sq[];
  const int64_t bh = blockIdx.x;
  if (app.on && (bh % Hq) % G < 2) {  // the key by the group's first query head, the value by its second
    __shared__ AppendShared app_sh;
    const int b = (int)(bh / Hq), g = (int)((bh % Hq) / G), which = (int)((bh % Hq) % G);
    append_token(app, b, g, which, app_sh);
    if (G == 1) append_token(app, b, g, 1, app_sh);  // one head per kv head: this work-group does both
  }
  for (int j = threadIdx.x; j < d; j += 256) {
    float v;
    if (QT == TQ_F32) v = static_cast<const float *>(q)[bh * d + j];
    else if (QT == TQ_BF16) v = bf16_to_f32(static_cast<const uint16_t *>(q)[bh * d + j]);
    else v = f16_to_f32(static_cast<const uint16_t *>(q)[bh * d + j]);
    sq[j] = v;
  }
  __syncthreads();
  // q'_j = sum_k Pi[j][k] q_k = sum_k Pi^T[k][j] q_k: lanes read consecutive entries of row k of Pi^T
  for (int j = threadIdx.x; j < d; j += 256) {
    float acc = 0.f;
    for (int k = 0; k < d; ++k) acc = fmaf(piT[(int64_t)k * d + j], sq[k], acc);
    qrot[bh * ld + j] = acc;
  }
  if (sT)
    for (int j = threadIdx.x; j < d; j += 256) {
      float acc = 0.f;
      for (int k = 0; k < d; ++k) acc = fmaf(sT[(int64_t)k * d + j], sq[k], acc);
      qrot[bh * ld + d + j] = acc;
    }
}

// KPROD: Algorithm-2 keys (kbits index planes, then the sign plane; score adds kqjl gamma <S_K q, s>).
// The M query tokens of a sequence (M = 1 for a decode step) and the G query heads of a kv head form the
// M G query rows of a (batch, kv-head) pair, ordered token-major; a wave takes GW consecutive rows.  Row
// (m, h) is query row (b M + m) Hq + g G + h and attends the first min(len[b] + m + add, Tstride) tokens
// (a decode step: m = 0, add = 1 when it appended a token; a prefill chunk: add = 1, causal).
template <int CP, int GW, bool KPROD>
__global__ __launch_bounds__(64) void attn_split_kernel(
    const float *qrot, int Hq, int Hkv, int G, int M, int nsub, int d, const uint8_t *kcodes,
    const uint16_t *knorms, const uint16_t *kgammas, int64_t kcb, int kbits, float kqjl, const uint8_t *vcodes,
    const uint16_t *vnorms, const uint16_t *vgammas, int64_t vcb, int vbmse, int64_t Tstride, const int32_t *len,
    int add, float scale_log2, float vqjl, Codebook kc, Codebook vc, int chunk, int nsplit, float *part) {
  const int lane = threadIdx.x;
  const int unit = blockIdx.x;  // ((b * Hkv) + g) * nsub + sub
  const int split = blockIdx.y;
  const int sub = unit % nsub;
  const int bg = unit / nsub;
  const int g = bg % Hkv, b = bg / Hkv;
  const int r0 = sub * GW;                   // first row of this wave among the M G rows
  const int gw = imin32(GW, M * G - r0);
  const int64_t base_len = imax64(len[b], 0) + add;
  auto row_q = [&](int h) { const int r = r0 + h; return ((int64_t)b * M + r / G) * Hq + g * G + r % G; };
  auto row_T = [&](int h) { return imin64(base_len + (r0 + h) / G, Tstride); };
  const int64_t T = row_T(gw - 1);  // the rows are token-major: the last one sees the most tokens
  const int64_t t0 = (int64_t)split * chunk;
  const int64_t t1 = imin64(T, t0 + chunk);

  const int ldq = KPROD ? 2 * d : d;
  float qv[GW][CP], qs[KPROD ? GW : 1][CP];
#pragma unroll
  for (int h = 0; h < GW; ++h)
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      qv[h][c] = h < gw ? qrot[row_q(h) * ldq + lane + 64 * c] : 0.f;
      if (KPROD) qs[KPROD ? h : 0][c] = h < gw ? qrot[row_q(h) * ldq + d + lane + 64 * c] : 0.f;
    }
  float m[GW], l[GW], am[GW][CP], aq[GW][CP];
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int c = 0; c < CP; ++c) am[h][c] = aq[h][c] = 0.f;
  }
  const int64_t base = ((int64_t)b * Hkv + g) * Tstride;
  const int wbytes = d >> 3;
  for (int64_t t = t0; t < t1; ++t) {
    const uint8_t *kr = kcodes + (base + t) * kcb;
    const uint8_t *vr = vcodes + (base + t) * vcb;
    float kval[CP], ksg[CP], vm[CP], vs[CP];
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      int idx = 0;
      for (int p = 0; p < kbits; ++p) {
        unsigned long long w = *reinterpret_cast<const unsigned long long *>(kr + p * wbytes + 8 * c);
        idx |= (int)((w >> lane) & 1ull) << p;
      }
      kval[c] = kc.c[idx];
      if (KPROD) {
        unsigned long long w = *reinterpret_cast<const unsigned long long *>(kr + kbits * wbytes + 8 * c);
        ksg[c] = ((w >> lane) & 1ull) ? 1.f : -1.f;
      }
      int vi = 0;
      for (int p = 0; p < vbmse; ++p) {
        unsigned long long w = *reinterpret_cast<const unsigned long long *>(vr + p * wbytes + 8 * c);
        vi |= (int)((w >> lane) & 1ull) << p;
      }
      vm[c] = vc.c[vi];
      unsigned long long ws = *reinterpret_cast<const unsigned long long *>(vr + vbmse * wbytes + 8 * c);
      vs[c] = ((ws >> lane) & 1ull) ? 1.f : -1.f;
    }
    const float kn = f16_to_f32(knorms[base + t]) * scale_log2;
    const float kg = KPROD ? f16_to_f32(kgammas[base + t]) * kqjl * scale_log2 : 0.f;
    const float vn = f16_to_f32(vnorms[base + t]);
    const float vg = f16_to_f32(vgammas[base + t]) * vqjl;
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      if (h >= gw) break;
      if (t >= row_T(h)) continue;  // causal: this row's query token sees fewer tokens
      float part_s = 0.f, part_q = 0.f;
#pragma unroll
      for (int c = 0; c < CP; ++c) {
        part_s = fmaf(qv[h][c], kval[c], part_s);
        if (KPROD) part_q = fmaf(qs[KPROD ? h : 0][c], ksg[c], part_q);
      }
      // log2-domain score
      const float s = KPROD ? fmaf(wave_sum_f32(part_s), kn, wave_sum_f32(part_q) * kg) : wave_sum_f32(part_s) * kn;
      if (s > m[h]) {
        const float corr = exp2f(m[h] - s);
        l[h] *= corr;
#pragma unroll
        for (int c = 0; c < CP; ++c) { am[h][c] *= corr; aq[h][c] *= corr; }
        m[h] = s;
      }
      const float p = exp2f(s - m[h]);
      l[h] += p;
      const float pm = p * vn, pq = p * vg;
#pragma unroll
      for (int c = 0; c < CP; ++c) {
        am[h][c] = fmaf(pm, vm[c], am[h][c]);
        aq[h][c] = fmaf(pq, vs[c], aq[h][c]);
      }
    }
  }
  // partial record: [m (log2 domain), l, acc_mse[d], acc_qjl[d]]
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    if (h >= gw) break;
    float *dst = part + (row_q(h) * nsplit + split) * (2 + 2 * (int64_t)d);
    if (lane == 0) { dst[0] = m[h]; dst[1] = l[h]; }
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      dst[2 + lane + 64 * c] = am[h][c];
      dst[2 + d + lane + 64 * c] = aq[h][c];
    }
  }
}

// Finishing a (batch, head) row takes two short, latency-bound kernels with many threads each:
// (1) merge the row's sequence splits with their log-sum-exp weights,
//     A = [sum_s 2^(m_s - M) acc_mse_s, sum_s 2^(m_s - M) acc_qjl_s] / sum_s 2^(m_s - M) l_s
//     (one thread per entry of A; the split loads are issued together, FIN_CHUNK at a time);
// (2) rotate back once: out = Pi_V^T A_mse + S_V^T A_qjl, i.e. out_j = sum_k Pi[k][j] A_k + S[k][j] A_{d+k}
//     (a work-group takes 32 output columns of one row; eight k-slices of the 2d terms are summed
//     through LDS; consecutive threads read consecutive entries of a row of Pi or S).
constexpr int FIN_CHUNK = 16;

__global__ __launch_bounds__(256) void attn_merge_kernel(const float *part, int64_t BH, int nsplit, int d,
                                                         float *merged) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= BH * 2 * d) return;
  const int64_t bh = e / (2 * d);
  const int j = (int)(e % (2 * d));
  const int64_t rec = 2 + 2 * (int64_t)d;
  const float *pp = part + bh * nsplit * rec;
  if (nsplit == 1) {  // (a prefill chunk's rows: one split each) the general form below reduces to v / l
    const float l = pp[1], v = pp[2 + j];
    merged[e] = l > 0.f ? v / l : 0.f;
    return;
  }
  float M = -INFINITY;
  for (int q0 = 0; q0 < nsplit; q0 += FIN_CHUNK) {
    float m[FIN_CHUNK], l[FIN_CHUNK];
#pragma unroll
    for (int i = 0; i < FIN_CHUNK; ++i) {
      const int q = imin32(q0 + i, nsplit - 1);
      m[i] = pp[q * rec];
      l[i] = pp[q * rec + 1];
    }
#pragma unroll
    for (int i = 0; i < FIN_CHUNK; ++i)
      if (l[i] > 0.f) M = fmaxf(M, m[i]);
  }
  float L = 0.f, a = 0.f;
  for (int q0 = 0; q0 < nsplit; q0 += FIN_CHUNK) {
    float m[FIN_CHUNK], l[FIN_CHUNK], v[FIN_CHUNK];
#pragma unroll
    for (int i = 0; i < FIN_CHUNK; ++i) {
      const int q = imin32(q0 + i, nsplit - 1);
      m[i] = pp[q * rec];
      l[i] = q0 + i < nsplit ? pp[q * rec + 1] : 0.f;
      v[i] = pp[q * rec + 2 + j];
    }
#pragma unroll
    for (int i = 0; i < FIN_CHUNK; ++i) {
      const float f = l[i] > 0.f ? exp2f(m[i] - M) : 0.f;
      L = fmaf(l[i], f, L);
      a = fmaf(v[i], f, a);
    }
  }
  merged[e] = L > 0.f ? a / L : 0.f;
}

template <int PER>
__global__ __launch_bounds__(256) void attn_rotate_kernel(const float *merged, int64_t BH, int d, const float *pi,
                                                          const float *s, float *out) {
  constexpr int HB = 4;  // rows per work-group: each entry of Pi and S read serves all of them
  __shared__ float red[HB][8][33];
  const int64_t bh0 = (int64_t)blockIdx.x * HB;
  const int c = threadIdx.x & 31, sl = threadIdx.x >> 5;
  const int j = blockIdx.y * 32 + c;
  // slice sl covers terms t0 .. t0+PER-1 of the 2d (the first d pair with rows of Pi, the rest with rows of S)
  const int t0 = sl * PER;
  const float *mrow = t0 < d ? pi + (int64_t)t0 * d + j : s + (int64_t)(t0 - d) * d + j;
  float m[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) m[i] = mrow[(int64_t)i * d];
  float acc[HB];
#pragma unroll
  for (int h = 0; h < HB; ++h) {
    const float *A = merged + imin64(bh0 + h, BH - 1) * 2 * d + t0;
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) v = fmaf(m[i], A[i], v);
    acc[h] = v;
    red[h][sl][c] = v;
  }
  __syncthreads();
  if (sl == 0) {
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      float v = acc[h];
#pragma unroll
      for (int q = 1; q < 8; ++q) v += red[h][q][c];
      if (bh0 + h < BH) out[(bh0 + h) * d + j] = v;
    }
  }
}

// head dims above 256 (multiples of 256): HB rows per work-group, so that each entry of Pi and S read
// serves all of them; 512 threads = 16 slices of 2d / 16 terms (the first half pair with rows of Pi, the
// rest with rows of S) x 32 columns.  A thread loads its slice's matrix entries (coalesced across the 32
// columns) all at once, so one memory round trip covers them; the rows' terms are staged in LDS.
template <int HB>
__global__ __launch_bounds__(512) void attn_rotate_wide_kernel(const float *merged, int64_t BH, int d, const float *pi,
                                                               const float *s, float *out) {
  constexpr int NSL = 16, PER = 64;  // slices and terms per slice (2d = 1024 at head dim 512)
  extern __shared__ __attribute__((aligned(16))) float arows[];  // [HB][2d]
  __shared__ float red[HB][NSL][33];
  const int64_t bh0 = (int64_t)blockIdx.x * HB;
  const int tid = threadIdx.x, c = tid & 31, sl = tid >> 5;
  const int j = blockIdx.y * 32 + c;
  // the rows' terms into LDS, 16 unconditional loads per thread at a time (clamped indices)
  for (int e0 = 0; e0 < HB * 2 * d; e0 += 512 * 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = imin32(e0 + 512 * u + tid, HB * 2 * d - 1);
      v[u] = merged[imin64(bh0 + e / (2 * d), BH - 1) * 2 * d + e % (2 * d)];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (e0 + 512 * u + tid < HB * 2 * d) arows[e0 + 512 * u + tid] = v[u];
  }
  for (int t0 = sl * PER; t0 < 2 * d; t0 += NSL * PER) {  // one pass at head dim 512
    const float *mrow = t0 < d ? pi + (int64_t)t0 * d + j : s + (int64_t)(t0 - d) * d + j;
    float m[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) m[i] = mrow[(int64_t)i * d];
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first product
    __syncthreads();  // (first pass) the rows are staged
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      const float4 *A = reinterpret_cast<const float4 *>(arows + h * 2 * d + t0);
      float v = 0.f;
#pragma unroll
      for (int i = 0; i < PER / 4; ++i) {
        const float4 a4 = A[i];
        v = fmaf(m[4 * i], a4.x, v);
        v = fmaf(m[4 * i + 1], a4.y, v);
        v = fmaf(m[4 * i + 2], a4.z, v);
        v = fmaf(m[4 * i + 3], a4.w, v);
      }
      red[h][sl][c] = (t0 == sl * PER ? 0.f : red[h][sl][c]) + v;
    }
  }
  __syncthreads();
  if (sl == 0) {
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < NSL; ++q) v += red[h][q][c];
      if (bh0 + h < BH) out[(bh0 + h) * d + j] = v;
    }
  }
}

// Head dims up to 256: both steps in one kernel.  A work-group takes four rows and 32 output columns;
// its matrix entries are loaded first (in flight during the merge), each wave merges the splits' weights
// of one row (the largest split maximum M and the total weight L, then each split's factor
// 2^(m_s - M) / L into LDS), the four rows' entries of A are merged into LDS, and the rotation reads them
// there.  The merge is repeated by the d / 32 work-groups of a row group (its inputs are few kilobytes).
constexpr int CMB_SPLITS = 256;  // splits whose factors fit in LDS; beyond, the separate kernels run
template <int PER>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float *part, int64_t BH, int nsplit, int d,
                                                           const float *pi, const float *s, float *out) {
  constexpr int HB = 4;
  __shared__ float sf[HB][CMB_SPLITS];  // 2^(m_s - M) / L per row and split (0 for empty splits)
  __shared__ float sa[HB][8 * PER];     // the rows' A (2d = 8 PER entries)
  __shared__ float red[HB][8][33];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int64_t bh0 = (int64_t)blockIdx.x * HB;
  const int c = tid & 31, sl = tid >> 5;
  const int j = blockIdx.y * 32 + c;
  const int t0 = sl * PER;
  const float *mrow = t0 < d ? pi + (int64_t)t0 * d + j : s + (int64_t)(t0 - d) * d + j;
  float m[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) m[i] = mrow[(int64_t)i * d];
  const int64_t rec = 2 + 2 * (int64_t)d;
  {  // wave wv: the split factors of row bh0 + wv (each lane keeps its splits' m and l: 4 per lane here)
    const float *pp = part + imin64(bh0 + wv, BH - 1) * nsplit * rec;
    constexpr int QL = CMB_SPLITS / 64;
    float mq[QL], lq[QL];
#pragma unroll
    for (int k = 0; k < QL; ++k) {
      const int q = lane + 64 * k;
      mq[k] = q < nsplit ? pp[q * rec] : 0.f;
      lq[k] = q < nsplit ? pp[q * rec + 1] : 0.f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < QL; ++k)
      if (lq[k] > 0.f) M = fmaxf(M, mq[k]);
    M = wave_max_f32(M);
    float fq[QL], L = 0.f;
#pragma unroll
    for (int k = 0; k < QL; ++k) {
      fq[k] = lq[k] > 0.f ? exp2f(mq[k] - M) : 0.f;
      L = fmaf(lq[k], fq[k], L);
    }
    L = wave_sum_f32(L);
    const float il = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int k = 0; k < QL; ++k) sf[wv][lane + 64 * k] = fq[k] * il;
  }
  __syncthreads();
  {  // this thread's entries of A: e = tid + 256 i, every split's value loaded in one batch per chunk
    constexpr int EPT = HB * 8 * PER / 256;
    constexpr int QC = 64 / EPT < FIN_CHUNK ? 64 / EPT : FIN_CHUNK;
    float a[EPT];
    const float *pe[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid + 256 * i, h = e / (8 * PER), t = e % (8 * PER);
      pe[i] = part + imin64(bh0 + h, BH - 1) * nsplit * rec + 2 + t;
      a[i] = 0.f;
    }
    for (int q0 = 0; q0 < nsplit; q0 += QC) {
      float v[EPT][QC];
#pragma unroll
      for (int i = 0; i < EPT; ++i)
#pragma unroll
        for (int k = 0; k < QC; ++k) v[i][k] = pe[i][imin32(q0 + k, nsplit - 1) * rec];
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int h = (tid + 256 * i) / (8 * PER);
#pragma unroll
        for (int k = 0; k < QC; ++k)
          if (q0 + k < nsplit) a[i] = fmaf(v[i][k], sf[h][q0 + k], a[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid + 256 * i;
      sa[e / (8 * PER)][e % (8 * PER)] = a[i];
    }
  }
  __syncthreads();
  float acc[HB];
#pragma unroll
  for (int h = 0; h < HB; ++h) {
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) v = fmaf(m[i], sa[h][t0 + i], v);
    acc[h] = v;
    red[h][sl][c] = v;
  }
  __syncthreads();
  if (sl == 0) {
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      float v = acc[h];
#pragma unroll
      for (int q = 1; q < 8; ++q) v += red[h][q][c];
      if (bh0 + h < BH) out[(bh0 + h) * d + j] = v;
    }
  }
}

size_t attn_merge_ws_bytes(int BH, int d) { return (size_t)BH * 2 * d * sizeof(float); }

// rows from which the rotation back runs as one GEMM (a prefill chunk: one row per query token and head),
// after the merge kernel, or straight over the records when every row took one split.  Below, one fused
// launch whose work-groups each read the d x 2d matrix for four rows: fine for a decode step's few hundred
// rows, while the 16384 rows of a 512-token chunk made it read 512 MB from L2 (111 us; the GEMM 20 us)
constexpr int kCombineGemmRows = 4096;

int attn_combine(const float *part, int BH, int nsplit, int d, const tq_quantizer *vq, float *merged, float *out,
                 hipStream_t st) {
  if (BH == 0) return TQ_OK;
  ProfScope ps("attn_combine", st);
  const float *pi = vq->pi, *s = vq->s;
  if (BH >= kCombineGemmRows && vq->piT && vq->sT) {
    if (nsplit == 1) return rotate_back(part, BH, d, vq->piT, vq->sT, out, true, st);
    const int64_t n = (int64_t)BH * 2 * d;
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st, part, (int64_t)BH, nsplit,
                       d, merged);
    const int rc = launch_check();
    if (rc != TQ_OK) return rc;
    return rotate_back(merged, BH, d, vq->piT, vq->sT, out, false, st);
  }
  if (nsplit >= 1 && nsplit <= CMB_SPLITS && (d == 64 || d == 128 || d == 256)) {
    const dim3 grid((unsigned)cdiv64(BH, 4), (unsigned)(d / 32));
    if (d == 64) hipLaunchKernelGGL(attn_combine_kernel<16>, grid, dim3(256), 0, st, part, (int64_t)BH, nsplit, d, pi, s, out);
    if (d == 128) hipLaunchKernelGGL(attn_combine_kernel<32>, grid, dim3(256), 0, st, part, (int64_t)BH, nsplit, d, pi, s, out);
    if (d == 256) hipLaunchKernelGGL(attn_combine_kernel<64>, grid, dim3(256), 0, st, part, (int64_t)BH, nsplit, d, pi, s, out);
    return launch_check();
  }
  const int64_t n = (int64_t)BH * 2 * d;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st, part, (int64_t)BH, nsplit, d,
                     merged);
  int rc = launch_check();
  if (rc != TQ_OK) return rc;
  // eight slices of the 2d terms: 2d / 8 = d / 4 terms per thread
  const dim3 grid((unsigned)cdiv64(BH, 4), (unsigned)(d / 32));
  switch (d) {
    case 64: hipLaunchKernelGGL(attn_rotate_kernel<16>, grid, dim3(256), 0, st, merged, (int64_t)BH, d, pi, s, out); break;
    case 128: hipLaunchKernelGGL(attn_rotate_kernel<32>, grid, dim3(256), 0, st, merged, (int64_t)BH, d, pi, s, out); break;
    case 256: hipLaunchKernelGGL(attn_rotate_kernel<64>, grid, dim3(256), 0, st, merged, (int64_t)BH, d, pi, s, out); break;
    default: {
      // larger head dims (multiples of 256): eight rows per work-group
      if (d % 256 != 0) return TQ_ERR_UNSUPPORTED;
      hipLaunchKernelGGL(attn_rotate_wide_kernel<8>, dim3((unsigned)cdiv64(BH, 8), (unsigned)(d / 32)), dim3(512),
                         (size_t)8 * 2 * d * 4, st, merged, (int64_t)BH, d, pi, s, out);
    }
  }
  return launch_check();
}

size_t attn_fast_ws_bytes(int D, int KB, int B, int Hq, int Hkv, int64_t T);
int run_attn_fast(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int Hq, int Hkv,
                  const uint8_t *kcodes, const uint16_t *knorms, const uint32_t *vtiles, const uint16_t *vnorms,
                  const uint16_t *vgammas, int64_t Tstride, const int32_t *seq_len, int kv_div, float scale,
                  float *out, void *ws, const AppendArgs *app, hipStream_t st);

// workspace of the row-record path: rotated queries, split partials, merged rows (M query tokens per sequence)
size_t rows_ws_bytes(const tq_quantizer *kq, int B, int M, int Hq, int Hkv, int64_t Tstride) {
  const bool kprod = kq->mode == TQ_PROD;
  const int d = kq->d;
  const size_t BH = (size_t)B * M * Hq;
  AttnPlan p = make_plan(d, B, Hq, Hkv, Tstride, kprod, M);
  size_t qb = (BH * (kprod ? 2 : 1) * d * 4 + 255) & ~(size_t)255;
  return qb + ((BH * p.nsplit * partial_floats(d) * 4 + 255) & ~(size_t)255) + attn_merge_ws_bytes((int64_t)BH, d);
}

size_t attn_ws_bytes(const tq_quantizer *kq, int B, int Hq, int Hkv, int64_t Tstride, int vlayout) {
  const bool kprod = kq->mode == TQ_PROD;
  if (vlayout == TQ_LAYOUT_TILE32 && !kprod) return attn_fast_ws_bytes(kq->d, kq->bits, B, Hq, Hkv, Tstride);
  return rows_ws_bytes(kq, B, 1, Hq, Hkv, Tstride);
}

template <int CP>
static void launch_split(const AttnPlan &p, dim3 grid, hipStream_t st, const float *qrot, int Hq, int Hkv, int M,
                         int d, const tq_quantizer *kq, const tq_quantizer *vq, const uint8_t *kcodes,
                         const uint16_t *knorms, const uint16_t *kgammas, const uint8_t *vcodes,
                         const uint16_t *vnorms, const uint16_t *vgammas, int64_t Tstride, const int32_t *len,
                         int add, float scale_log2, float *part) {
  if (kq->mode == TQ_PROD)
    hipLaunchKernelGGL((attn_split_kernel<CP, split_heads(CP, true), true>), grid, dim3(64), 0, st, qrot, Hq, Hkv, p.G,
                       M, p.nsub, d, kcodes, knorms, kgammas, (int64_t)kq->code_bytes, kq->bmse, kq->qjl_scale,
                       vcodes, vnorms, vgammas, (int64_t)vq->code_bytes, vq->bmse, Tstride, len, add, scale_log2,
                       vq->qjl_scale, kq->cb, vq->cb, p.chunk, p.nsplit, part);
  else
    hipLaunchKernelGGL((attn_split_kernel<CP, split_heads(CP, false), false>), grid, dim3(64), 0, st, qrot, Hq, Hkv,
                       p.G, M, p.nsub, d, kcodes, knorms, kgammas, (int64_t)kq->code_bytes, kq->bmse, 0.f, vcodes,
                       vnorms, vgammas, (int64_t)vq->code_bytes, vq->bmse, Tstride, len, add, scale_log2,
                       vq->qjl_scale, kq->cb, vq->cb, p.chunk, p.nsplit, part);
}

// Row-record path for M query tokens per sequence: q [B, M, Hq, d] -> out [B, M, Hq, d]; query token m of
// sequence b attends the first min(len[b] + m + add, Tstride) tokens
static int run_attn_rows(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int M, int Hq,
                         int Hkv, const uint8_t *kcodes, const uint16_t *knorms, const uint16_t *kgammas,
                         const uint8_t *vcodes, const uint16_t *vnorms, const uint16_t *vgammas, int64_t Tstride,
                         const int32_t *len, int add, float scale, float *out, void *ws, const AppendArgs &ap,
                         hipStream_t st) {
  const bool kprod = kq->mode == TQ_PROD;
  const int d = kq->d;
  AttnPlan p = make_plan(d, B, Hq, Hkv, Tstride, kprod, M);
  if (!p.CP) return TQ_ERR_UNSUPPORTED;
  const int ldq = kprod ? 2 * d : d;
  const int64_t BH = (int64_t)B * M * Hq;
  float *qrot = static_cast<float *>(ws);
  float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + (((size_t)BH * ldq * 4 + 255) & ~(size_t)255));
  const size_t shq = (size_t)d * 4;
  const float *sT = kprod ? kq->sT : nullptr;
  const int G = Hq / Hkv;
  {
  ProfScope ps("attn_qrot", st);
  const dim3 qg((unsigned)BH);
  if (qt == TQ_F32) hipLaunchKernelGGL(attn_qrot_kernel<TQ_F32>, qg, dim3(256), shq, st, q, d, kq->piT, sT, ldq, qrot, Hq, G, ap);
  else if (qt == TQ_BF16) hipLaunchKernelGGL(attn_qrot_kernel<TQ_BF16>, qg, dim3(256), shq, st, q, d, kq->piT, sT, ldq, qrot, Hq, G, ap);
  else hipLaunchKernelGGL(attn_qrot_kernel<TQ_F16>, qg, dim3(256), shq, st, q, d, kq->piT, sT, ldq, qrot, Hq, G, ap);
  }
  int rc = launch_check();
  if (rc != TQ_OK) return rc;
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid((unsigned)(B * Hkv * p.nsub), (unsigned)p.nsplit);
  {
  ProfScope ps("attn_split", st);
#define TQ_SPLIT(CPV) launch_split<CPV>(p, grid, st, qrot, Hq, Hkv, M, d, kq, vq, kcodes, knorms, kgammas, vcodes, \
                                        vnorms, vgammas, Tstride, len, add, scale_log2, part)
  switch (p.CP) {
    case 1: TQ_SPLIT(1); break;
    case 2: TQ_SPLIT(2); break;
    case 4: TQ_SPLIT(4); break;
    case 8: TQ_SPLIT(8); break;
    case 16: TQ_SPLIT(16); break;
    case 24: TQ_SPLIT(24); break;
    default: TQ_SPLIT(32); break;
  }
#undef TQ_SPLIT
  }
  if ((rc = launch_check()) != TQ_OK) return rc;
  float *merged = reinterpret_cast<float *>(reinterpret_cast<char *>(part) +
                                            (((size_t)BH * p.nsplit * partial_floats(d) * 4 + 255) & ~(size_t)255));
  return attn_combine(part, (int)BH, p.nsplit, d, vq, merged, out, st);
}

int run_attn_decode(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int Hq, int Hkv,
                    const uint8_t *kcodes, const uint16_t *knorms, const uint16_t *kgammas, const uint8_t *vcodes,
                    const uint16_t *vnorms, const uint16_t *vgammas, int vlayout, int64_t Tstride,
                    const int32_t *seq_len, float scale, float *out, void *ws, size_t ws_bytes,
                    const AppendArgs *app, hipStream_t st) {
  const bool kprod = kq->mode == TQ_PROD;
  if (vlayout == TQ_LAYOUT_TILE32) {
    // the matrix-core kernels take Algorithm-1 keys and values with at least one index bit
    if (kprod || vq->bmse < 1) return TQ_ERR_UNSUPPORTED;
    return run_attn_fast(kq, vq, q, qt, B, Hq, Hkv, kcodes, knorms, reinterpret_cast<const uint32_t *>(vcodes), vnorms,
                         vgammas, Tstride, seq_len, 1, scale, out, ws, app, st);
  }
  AppendArgs ap{};
  if (app) ap = *app;
  return run_attn_rows(kq, vq, q, qt, B, 1, Hq, Hkv, kcodes, knorms, kgammas, vcodes, vnorms, vgammas, Tstride, seq_len,
                       ap.on ? 1 : 0, scale, out, ws, ap, st);
}

// token-tiled prefill: every query token is a row of its own (B * M rows, row b m of sequence b attending
// the tokens 0 .. q_pos[b] + m), all rows of a sequence reading its one cache row; the rows' lengths go
// after the decode kernels' workspace
static size_t prefill_tiled_lens_off(const tq_quantizer *kq, int B, int M, int Hq, int Hkv, int64_t Tstride) {
  return (attn_fast_ws_bytes(kq->d, kq->bits, B * M, Hq, Hkv, Tstride) + 255) & ~(size_t)255;
}

size_t attn_prefill_ws_bytes(const tq_quantizer *kq, int B, int M, int Hq, int Hkv, int64_t Tstride, int vlayout) {
  if (vlayout == TQ_LAYOUT_TILE32)
    return prefill_tiled_lens_off(kq, B, M, Hq, Hkv, Tstride) + (((size_t)B * M * 4 + 255) & ~(size_t)255);
  return rows_ws_bytes(kq, B, M, Hq, Hkv, Tstride);
}

__global__ void prefill_lens_kernel(const int32_t *q_pos, int B, int M, int64_t Tstride, int32_t *lens) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)B * M) return;
  const int64_t b = i / M, m = i - b * M;
  const int64_t pos = (int64_t)(q_pos[b] > 0 ? q_pos[b] : 0) + m + 1;
  lens[i] = (int32_t)(pos < Tstride ? pos : Tstride);
}

int run_attn_prefill(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int M, int Hq,
                     int Hkv, const uint8_t *kcodes, const uint16_t *knorms, const uint16_t *kgammas,
                     const uint8_t *vcodes, const uint16_t *vnorms, const uint16_t *vgammas, int vlayout,
                     int64_t Tstride, const int32_t *q_pos, float scale, float *out, void *ws, hipStream_t st) {
  if (vlayout == TQ_LAYOUT_TILE32) {
    // the decode kernels over B * M rows (the matrix-core kernels take Algorithm-1 keys and values with at
    // least one index bit)
    if (kq->mode == TQ_PROD || vq->bmse < 1) return TQ_ERR_UNSUPPORTED;
    int32_t *lens = reinterpret_cast<int32_t *>(static_cast<char *>(ws) +
                                                prefill_tiled_lens_off(kq, B, M, Hq, Hkv, Tstride));
    const int64_t rows = (int64_t)B * M;
    hipLaunchKernelGGL(prefill_lens_kernel, dim3((unsigned)cdiv64(rows, 256)), dim3(256), 0, st, q_pos, B, M, Tstride,
                       lens);
    int rc = launch_check();
    if (rc != TQ_OK) return rc;
    return run_attn_fast(kq, vq, q, qt, B * M, Hq, Hkv, kcodes, knorms, reinterpret_cast<const uint32_t *>(vcodes),
                         vnorms, vgammas, Tstride, lens, M, scale, out, ws, nullptr, st);
  }
  AppendArgs ap{};
  return run_attn_rows(kq, vq, q, qt, B, M, Hq, Hkv, kcodes, knorms, kgammas, vcodes, vnorms, vgammas, Tstride, q_pos,
                       1, scale, out, ws, ap, st);
}

}  // namespace tq
