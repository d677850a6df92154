// Rotations and projections as dense contractions on the fp32 matrix cores.
//
// One tiled kernel computes Z = A B^T (A: M x K, B: N x K, both read through
// operand loaders) with v_mfma_f32_16x16x4_f32 and hands the 64 x 64 output
// tile, staged in LDS, to an epilogue.  Loaders read dense fp32/bf16/fp16 rows
// or dequantize packed records on the fly; epilogues store fp32, quantize and
// pack index planes with wavefront ballots (Algorithm 1), or pack QJL sign bits
// (Algorithm 2).  Algorithm steps as on the ai-navigate-news Gemma 4 post,
// section "仕組み（技術的）".
//
// fp32 operands keep the rotated coordinates within ~1e-7 of their norm scale,
// far inside the 1e-5 tie zone the codes are checked against.
#include <algorithm>
#include <type_traits>

#include "common.cuh"

namespace tq {

constexpr int GBM = 64, GBN = 64, GBK = 16, GPAD = 16;

// ----------------------------------------------------------------------------
// operand loaders: fill v[0..3] with elements k..k+3 of row r (k % 4 == 0)
// ----------------------------------------------------------------------------
// Loaders: operator() gives four consecutive elements of row r from k as fp32; fetch / unpack split
// the same into the load (issued early, kept in registers) and the conversion.
struct LoadF32 {
  const float *p;
  int64_t ld;
  using Raw = float4;
  __device__ Raw fetch(int64_t r, int k) const { return *reinterpret_cast<const float4 *>(p + r * ld + k); }
  __device__ void unpack(const Raw &t, float *v) const { v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w; }
  __device__ void operator()(int64_t r, int k, float *v) const { unpack(fetch(r, k), v); }
};

struct LoadBF16 {
  const uint16_t *p;
  int64_t ld;
  using Raw = uint2;
  __device__ Raw fetch(int64_t r, int k) const { return *reinterpret_cast<const uint2 *>(p + r * ld + k); }
  __device__ void unpack(const Raw &t, float *v) const {
    v[0] = __uint_as_float(t.x << 16);
    v[1] = __uint_as_float(t.x & 0xFFFF0000u);
    v[2] = __uint_as_float(t.y << 16);
    v[3] = __uint_as_float(t.y & 0xFFFF0000u);
  }
  __device__ void operator()(int64_t r, int k, float *v) const { unpack(fetch(r, k), v); }
};

struct LoadF16 {
  const uint16_t *p;
  int64_t ld;
  using Raw = uint2;
  __device__ Raw fetch(int64_t r, int k) const { return *reinterpret_cast<const uint2 *>(p + r * ld + k); }
  __device__ void unpack(const Raw &t, float *v) const {
    v[0] = f16_to_f32(t.x & 0xFFFF);
    v[1] = f16_to_f32(t.x >> 16);
    v[2] = f16_to_f32(t.y & 0xFFFF);
    v[3] = f16_to_f32(t.y >> 16);
  }
  __device__ void operator()(int64_t r, int k, float *v) const { unpack(fetch(r, k), v); }
};

// rows [0, split) from a, rows [split, ...) from b (same row length ld)
struct LoadRows2 {
  const float *a, *b;
  int64_t split, ld;
  __device__ void operator()(int64_t r, int k, float *v) const {
    const float *p = r < split ? a + r * ld : b + (r - split) * ld;
    float4 t = *reinterpret_cast<const float4 *>(p + k);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  }
};

// columns [0, split) from a, [split, 2 split) from b (both row length split)
struct LoadCols2 {
  const float *a, *b;
  int split;
  __device__ void operator()(int64_t r, int k, float *v) const {
    const float *p = k < split ? a + r * split + k : b + r * split + (k - split);
    float4 t = *reinterpret_cast<const float4 *>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  }
};

// A record row dequantized to [n_hat c[idx] | qjl * gamma * (2 bit - 1)]
// (the second half only for Algorithm-2 records).
struct LoadDequant {
  const uint8_t *codes;
  const uint16_t *norms, *gammas;
  int64_t code_bytes;
  int d, bmse;
  float qjl;
  Codebook cb;
  __device__ void operator()(int64_t r, int k, float *v) const {
    const uint8_t *rec = codes + r * code_bytes;
    const int sh = k & 7;
    if (k < d) {
      int idx[4] = {0, 0, 0, 0};
      for (int p = 0; p < bmse; ++p) {
        int byte = rec[p * (d >> 3) + (k >> 3)] >> sh;
#pragma unroll
        for (int i = 0; i < 4; ++i) idx[i] |= ((byte >> i) & 1) << p;
      }
      float nh = f16_to_f32(norms[r]);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = cb.c[idx[i]] * nh;
    } else {
      int kk = k - d;
      int byte = rec[bmse * (d >> 3) + (kk >> 3)] >> sh;
      float g = qjl * f16_to_f32(gammas[r]);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = ((byte >> i) & 1) ? g : -g;
    }
  }
};

typedef float CTile[GBN + 1];

// ----------------------------------------------------------------------------
// epilogues (run by all 256 threads with the tile in LDS)
// ----------------------------------------------------------------------------
struct EpiStore {
  float *out;
  int64_t ldo;
  __device__ void operator()(const CTile *Cs, int64_t row0, int64_t col0, int64_t M, int64_t N) const {
    for (int e = threadIdx.x; e < GBM * GBN; e += 256) {
      int r = e / GBN, c = e % GBN;
      if (row0 + r < M && col0 + c < N) out[(row0 + r) * ldo + col0 + c] = Cs[r][c];
    }
  }
};

// Algorithm-1 index planes for 64 coordinates (one tile column block) per row.
// For Algorithm 2 also the rotated residual y - n_hat c[idx] and its squared norm over the block (fp32:
// the fp16 gamma tolerates 1e-5 relative), one partial per (row, block) so no atomics are needed.
// BM index bits; the cell index is a binary search over the row's scaled boundaries t_k n.
template <int BM>
struct EpiQuant {
  uint8_t *codes;
  int64_t code_bytes;
  int d;
  const float *n32;        // fp32 norms of the rows (chunk-relative)
  const uint16_t *nhat;    // fp16 norms (chunk-relative)
  float *resid;            // [rows, d] rotated residual, or null (Algorithm 1)
  float *rsq;              // [rows, d / 64] partial ||r||^2, or null
  Codebook cb;
  // rows rb..rb+15 of the tile by the calling wave (lane = column)
  __device__ void operator()(const CTile *Cs, int64_t row0, int64_t col0, int64_t M, int64_t N, int rb) const {
    constexpr int L = 1 << BM;
    const int lane = threadIdx.x & 63;
    // the 16 rows' norms: one load per lane, then uniform per row
    float nl = 0.f, hl = 0.f;
    if (lane < 16 && row0 + rb + lane < M) {
      nl = n32[row0 + rb + lane];
      hl = f16_to_f32(nhat[row0 + rb + lane]);
    }
    float tb[L - 1], cc[L];
#pragma unroll
    for (int k = 0; k < L - 1; ++k) tb[k] = cb.t[k];
#pragma unroll
    for (int k = 0; k < L; ++k) cc[k] = cb.c[k];
    const int nblk = d >> 6;
    float sq[16];  // r^2 of this lane's column, per row (summed over the block below)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      sq[rr] = 0.f;
      const int r = rb + rr;
      const int64_t row = row0 + r;
      if (row >= M) continue;
      const float y = Cs[r][lane];
      const float n = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(nl), rr));
      const float yq = n == 0.0f ? 0.0f : y, nq = n == 0.0f ? 1.0f : n;
      // binary search: bit s of idx decided against the one boundary the higher bits leave
      int idx = 0;
#pragma unroll
      for (int sbit = BM - 1; sbit >= 0; --sbit) {
        const int s = 1 << sbit;
        float t = tb[s - 1];
#pragma unroll
        for (int c = 1; c < L / (2 * s); ++c)
          if (idx == 2 * s * c) t = tb[2 * s * c + s - 1];
        idx += (yq > t * nq) ? s : 0;
      }
      uint8_t *dst = codes + row * code_bytes + (col0 >> 3);
#pragma unroll
      for (int p = 0; p < BM; ++p) {
        const unsigned long long m = __ballot(((idx >> p) & 1) != 0);
        if (lane == 0) *reinterpret_cast<unsigned long long *>(dst + p * (d >> 3)) = m;
      }
      if (resid) {
        float cv = cc[0];
#pragma unroll
        for (int k = 1; k < L; ++k) cv = idx == k ? cc[k] : cv;
        const float nh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hl), rr));
        const float rv = y - nh * cv;
        resid[row * d + col0 + lane] = rv;
        sq[rr] = rv * rv;
      }
    }
    if (resid) {
      // the 16 row sums over the lanes at once (independent shuffles in flight together)
#pragma unroll
      for (int o = 32; o > 0; o >>= 1)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sq[rr] += __shfl_xor(sq[rr], o, 64);
      float mine = sq[0];
#pragma unroll
      for (int rr = 1; rr < 16; ++rr) mine = (lane == rr) ? sq[rr] : mine;
      if (lane < 16 && row0 + rb + lane < M) rsq[(row0 + rb + lane) * nblk + (col0 >> 6)] = mine;
    }
  }
};

// QJL sign plane: bit = [(S r)_i >= 0]
struct EpiSign {
  uint8_t *codes;
  int64_t code_bytes;
  int d, plane;
  // rows rb..rb+15 of the tile by the calling wave (lane = column)
  __device__ void operator()(const CTile *Cs, int64_t row0, int64_t col0, int64_t M, int64_t N, int rb) const {
    const int lane = threadIdx.x & 63;
    for (int rr = 0; rr < 16; ++rr) {
      const int r = rb + rr;
      const int64_t row = row0 + r;
      if (row >= M) break;
      unsigned long long m = __ballot(Cs[r][lane] >= 0.0f);
      if (lane == 0)
        *reinterpret_cast<unsigned long long *>(codes + row * code_bytes + plane * (d >> 3) + (col0 >> 3)) = m;
    }
  }
};

// ----------------------------------------------------------------------------
// the tiled contraction
// ----------------------------------------------------------------------------
template <class LA, class LB, class EP>
__global__ __launch_bounds__(256) void gemm_kernel(LA la, LB lb, EP ep, int64_t M, int64_t N, int K) {
  __shared__ float As[GBK][GBM + GPAD];
  __shared__ float Bs[GBK][GBN + GPAD];
  __shared__ float Cs[GBM][GBN + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * GBM, col0 = (int64_t)blockIdx.y * GBN;
  const int wm = wave >> 1, wn = wave & 1;
  floatx4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int64_t ra = row0 + lr, rb = col0 + lr;
  for (int k0 = 0; k0 < K; k0 += GBK) {
    float va[4] = {0.f, 0.f, 0.f, 0.f}, vb[4] = {0.f, 0.f, 0.f, 0.f};
    if (ra < M) la(ra, k0 + lk, va);
    if (rb < N) lb(rb, k0 + lk, vb);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      As[lk + i][lr] = va[i];
      Bs[lk + i][lr] = vb[i];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kk = ks * 4 + (lane >> 4);
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = As[kk][wm * 32 + i * 16 + (lane & 15)];
        b[i] = Bs[kk][wn * 32 + i * 16 + (lane & 15)];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Cs[wm * 32 + i * 16 + 4 * (lane >> 4) + e][wn * 32 + j * 16 + (lane & 15)] = acc[i][j][e];
  __syncthreads();
  ep(Cs, row0, col0, M, N);
}

template <class LA, class LB, class EP>
static int gemm(const char *name, LA la, LB lb, EP ep, int64_t M, int64_t N, int K, hipStream_t st) {
  if (M <= 0 || N <= 0) return TQ_OK;
  dim3 grid((unsigned)cdiv64(M, GBM), (unsigned)cdiv64(N, GBN));
  ProfScope ps(name, st);
  hipLaunchKernelGGL((gemm_kernel<LA, LB, EP>), grid, dim3(256), 0, st, la, lb, ep, M, N, K);
  return launch_check();
}

// ----------------------------------------------------------------------------
// the tiled contraction on the bf16 matrix cores with exact pieces (encode at d > 128)
//
// C = A B^T with the fp32 A values (from a loader) split exactly into NPA bf16
// pieces on the fly (truncation: hi keeps 8 significant bits, mid the next 8,
// lo the rest; bf16 inputs are one piece, fp16 two) and B given as its three
// pre-split pieces [3][N][K].  Products of pieces are exact in fp32; the dropped
// cross terms are below 2^-23 of the product, so C is fp32-accurate (the codes
// are checked against the fp64 definition with a 1e-5 tie zone).  A 128 x 128
// tile per work-group, each wave a 64 x 64 quadrant (4 x 4 MFMA tiles), 32-deep
// k-steps staged in LDS with the next step's loads in registers; the epilogues
// of the fp32 kernel run once per quadrant.
// ----------------------------------------------------------------------------
constexpr int PBM = 128, PBN = 128, PBK = 32, PKP = 40;

typedef __bf16 gbf16x8 __attribute__((ext_vector_type(8)));

// upper halves of two exact-bf16 floats as one dword (lo element first)
__device__ __forceinline__ uint32_t g_pack2(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

template <int NPA>
__device__ __forceinline__ void g_split(float x, float (&p)[3]) {
  p[0] = __uint_as_float(__float_as_uint(x) & 0xFFFF0000u);
  const float r1 = x - p[0];
  p[1] = NPA == 2 ? r1 : __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
  p[2] = r1 - p[1];
}

template <int NPA>
__device__ __forceinline__ floatx4 g_terms(const gbf16x8 (&a)[3], const gbf16x8 (&b)[3], floatx4 c) {
#define TQ_MF(i, j) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], c, 0, 0, 0)
  if (NPA == 1) {
    TQ_MF(0, 2); TQ_MF(0, 1); TQ_MF(0, 0);
  } else if (NPA == 2) {
    TQ_MF(1, 1); TQ_MF(0, 2); TQ_MF(1, 0); TQ_MF(0, 1); TQ_MF(0, 0);
  } else {
    TQ_MF(1, 1); TQ_MF(2, 0); TQ_MF(0, 2); TQ_MF(1, 0); TQ_MF(0, 1); TQ_MF(0, 0);
  }
#undef TQ_MF
  return c;
}

template <int NPA, class LA, class EP>
__global__ __launch_bounds__(256) void gemm_pieces_kernel(LA la, const uint16_t *b3, EP ep, int64_t M, int64_t N,
                                                          int K) {
  // one buffer: the staged pieces during the contraction, then each wave's 64 x 64 result tile
  constexpr size_t AB = (size_t)(NPA + 3) * PBM * PKP * 2, CT = (size_t)4 * GBM * (GBN + 1) * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[AB > CT ? AB : CT];
  uint16_t(*As)[PBM][PKP] = reinterpret_cast<uint16_t(*)[PBM][PKP]>(lds);
  uint16_t(*Bs)[PBN][PKP] = reinterpret_cast<uint16_t(*)[PBN][PKP]>(lds + (size_t)NPA * PBM * PKP * 2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t row0 = (int64_t)blockIdx.x * PBM, col0 = (int64_t)blockIdx.y * PBN;
  const int ar = tid >> 1, ak = (tid & 1) * 16;  // A staging: row ar, k ak..ak+15
  const bool arow_ok = row0 + ar < M;
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // the next step's A and B elements are loaded into registers before this step's MFMAs and converted
  // to pieces only when they are stored, so the loads are in flight under the MFMAs
  typename LA::Raw rr[4];
  uint4 rb[6];
  auto gload = [&](int k0) {
    if (arow_ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) rr[i] = la.fetch(row0 + ar, k0 + ak + 4 * i);
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int e = tid + 256 * i, p = e >> 9, rem = e & 511, br = rem >> 2, kk = (rem & 3) * 8;
      const int64_t col = col0 + br;
      rb[i] = col < N ? *reinterpret_cast<const uint4 *>(b3 + ((int64_t)p * N + col) * K + k0 + kk)
                      : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&]() {
    float v[16];
    if (arow_ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) la.unpack(rr[i], v + 4 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w[3][4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float p0[3], p1[3];
        g_split<NPA>(v[8 * h + 2 * q], p0);
        g_split<NPA>(v[8 * h + 2 * q + 1], p1);
#pragma unroll
        for (int p = 0; p < 3; ++p) w[p][q] = g_pack2(p0[p], p1[p]);
      }
#pragma unroll
      for (int p = 0; p < NPA; ++p) *reinterpret_cast<uint4 *>(&As[p][ar][ak + 8 * h]) = uint4{w[p][0], w[p][1], w[p][2], w[p][3]};
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int e = tid + 256 * i, p = e >> 9, rem = e & 511, br = rem >> 2, kk = (rem & 3) * 8;
      *reinterpret_cast<uint4 *>(&Bs[p][br][kk]) = rb[i];
    }
  };

  const int fr = lane & 15, fk = 8 * (lane >> 4);
  gload(0);
  for (int k0 = 0; k0 < K; k0 += PBK) {
    __syncthreads();  // the previous step's fragments are consumed
    lstore();
    __syncthreads();
    if (k0 + PBK < K) gload(k0 + PBK);  // in flight during this step's MFMAs
    gbf16x8 af[4][3];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int p = 0; p < 3; ++p)
        af[rt][p] = p < NPA ? *reinterpret_cast<const gbf16x8 *>(&As[p][64 * wm + 16 * rt + fr][fk]) : af[rt][0];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      gbf16x8 bf[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) bf[p] = *reinterpret_cast<const gbf16x8 *>(&Bs[p][64 * wn + 16 * ct + fr][fk]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt][ct] = g_terms<NPA>(af[rt], bf, acc[rt][ct]);
    }
  }
  // every wave turns its own 64 x 64 quadrant to row-major in its part of the buffer and runs the
  // epilogue on it, 16 rows at a time (no work-group barrier after the first)
  __syncthreads();  // every read of the staged pieces done
  CTile *Cw = reinterpret_cast<CTile *>(lds + (size_t)wave * GBM * (GBN + 1) * 4);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) Cw[16 * rt + 4 * (lane >> 4) + e][16 * ct + fr] = acc[rt][ct][e];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int64_t qr0 = row0 + 64 * wm, qc0 = col0 + 64 * wn;
  if (qr0 < M && qc0 < N) {
#pragma unroll 1
    for (int rb = 0; rb < GBM; rb += 16) ep(Cw, qr0, qc0, M, N, rb);
  }
}

template <int NPA, class LA, class EP>
static int gemm_pieces(const char *name, LA la, const uint16_t *b3, EP ep, int64_t M, int64_t N, int K,
                       hipStream_t st) {
  if (M <= 0 || N <= 0) return TQ_OK;
  dim3 grid((unsigned)cdiv64(M, PBM), (unsigned)cdiv64(N, PBN));
  ProfScope ps(name, st);
  hipLaunchKernelGGL((gemm_pieces_kernel<NPA, LA, EP>), grid, dim3(256), 0, st, la, b3, ep, M, N, K);
  return launch_check();
}

// ----------------------------------------------------------------------------
// small kernels: norms, zero fill, gamma finalisation, M = S Pi^T
// ----------------------------------------------------------------------------
// one row per 16 lanes (16 rows per work-group): each lane sums the squares of 4 consecutive elements
// every 64, in fp64 (the fp16 norm must round as the exact value does), loads kept in flight together
template <int XT>
__global__ __launch_bounds__(256) void norm_kernel(const void *x, int64_t ldx, int d, int64_t n, uint16_t *nhat,
                                                   float *n32) {
  const int l16 = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  double s = 0.0;
  if (row < n) {
    for (int j0 = 4 * l16; j0 < d; j0 += 256) {
      float v[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + 64 * u;
        if (j >= d) {
          v[u][0] = v[u][1] = v[u][2] = v[u][3] = 0.f;
        } else if (XT == TQ_F32) {
          const float4 t = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + row * ldx + j);
          v[u][0] = t.x; v[u][1] = t.y; v[u][2] = t.z; v[u][3] = t.w;
        } else {
          const uint2 t = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + row * ldx + j);
          const uint16_t h[4] = {(uint16_t)(t.x & 0xFFFF), (uint16_t)(t.x >> 16), (uint16_t)(t.y & 0xFFFF),
                                 (uint16_t)(t.y >> 16)};
#pragma unroll
          for (int e = 0; e < 4; ++e) v[u][e] = XT == TQ_BF16 ? bf16_to_f32(h[e]) : f16_to_f32(h[e]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fma((double)v[u][e], (double)v[u][e], s);
    }
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (l16 == 0 && row < n) {
    const double nn = sqrt(s);
    nhat[row] = f64_to_f16_rne_sat(nn);
    n32[row] = (float)nn;
  }
}

// gamma = ||r|| from the rows' per-block partial squares (summed in fp64)
__global__ void gamma_kernel(const float *rsq, int nblk, int64_t n, uint16_t *gam) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  double s = 0.0;
  for (int b = 0; b < nblk; ++b) s += (double)rsq[i * nblk + b];
  gam[i] = f64_to_f16_rne_sat(sqrt(s));
}

// m[i][j] = sum_k s[i][k] pi[j][k] in fp64, rounded to fp32
__global__ void spit_kernel(int d, const float *s, const float *pi, float *m) {
  int i = blockIdx.y, j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= d) return;
  double acc = 0.0;
  for (int k = 0; k < d; ++k) acc += (double)s[(int64_t)i * d + k] * (double)pi[(int64_t)j * d + k];
  m[(int64_t)i * d + j] = (float)acc;
}

int compute_sPiT(int d, const float *s, const float *pi, float *m, hipStream_t st) {
  hipLaunchKernelGGL(spit_kernel, dim3((d + 127) / 128, d), dim3(128), 0, st, d, s, pi, m);
  return launch_check();
}

// ----------------------------------------------------------------------------
// encode / decode / score drivers
// ----------------------------------------------------------------------------
namespace {

struct Scratch {
  void *p = nullptr;
  hipStream_t st;
  explicit Scratch(hipStream_t s) : st(s) {}
  int alloc(size_t bytes) {
    hipError_t e = hipMallocAsync(&p, bytes, st);
    if (e != hipSuccess) { p = nullptr; return hip_fail(e); }
    return TQ_OK;
  }
  ~Scratch() { if (p) hipFreeAsync(p, st); }
};

template <class LX>
int encode_chunk(const tq_quantizer *q, LX lx, const void *x, int xt, int64_t ldx, int64_t cn, uint8_t *codes,
                 uint16_t *norms, uint16_t *gammas, float *n32, float *resid, float *rsq, hipStream_t st) {
  const int d = q->d;
  int rc;
  dim3 ng((unsigned)cdiv64(cn, 16));
  {
  ProfScope ps("encode_norm", st);
  if (xt == TQ_F32) hipLaunchKernelGGL(norm_kernel<TQ_F32>, ng, dim3(256), 0, st, x, ldx, d, cn, norms, n32);
  else if (xt == TQ_BF16) hipLaunchKernelGGL(norm_kernel<TQ_BF16>, ng, dim3(256), 0, st, x, ldx, d, cn, norms, n32);
  else hipLaunchKernelGGL(norm_kernel<TQ_F16>, ng, dim3(256), 0, st, x, ldx, d, cn, norms, n32);
  }
  if ((rc = launch_check()) != TQ_OK) return rc;
  const bool prod = q->mode == TQ_PROD;
  // exact bf16 pieces on the matrix cores: bf16 rows are one piece, fp16 two, fp32 three
  constexpr int NPA = std::is_same<LX, LoadBF16>::value ? 1 : std::is_same<LX, LoadF16>::value ? 2 : 3;
  auto rotate = [&](auto eq) { return gemm_pieces<NPA>("encode_rotate", lx, q->pi3, eq, cn, d, d, st); };
  float *rs = prod ? resid : nullptr, *rq = prod ? rsq : nullptr;
  const int64_t cbytes = (int64_t)q->code_bytes;
  switch (q->bmse) {
    case 1: rc = rotate(EpiQuant<1>{codes, cbytes, d, n32, norms, rs, rq, q->cb}); break;
    case 2: rc = rotate(EpiQuant<2>{codes, cbytes, d, n32, norms, rs, rq, q->cb}); break;
    case 3: rc = rotate(EpiQuant<3>{codes, cbytes, d, n32, norms, rs, rq, q->cb}); break;
    case 4: rc = rotate(EpiQuant<4>{codes, cbytes, d, n32, norms, rs, rq, q->cb}); break;
    default: rc = TQ_ERR_UNSUPPORTED;
  }
  if (rc != TQ_OK) return rc;
  if (!prod) return TQ_OK;
  LoadF32 lr{resid, d};
  EpiSign es{codes, (int64_t)q->code_bytes, d, q->planes - 1};
  if ((rc = gemm_pieces<3>("encode_qjl", lr, q->m3, es, cn, d, d, st)) != TQ_OK) return rc;
  hipLaunchKernelGGL(gamma_kernel, dim3((unsigned)cdiv64(cn, 256)), dim3(256), 0, st, rsq, d / 64, cn, gammas);
  return launch_check();
}

}  // namespace

int run_encode(const tq_quantizer *q, const void *x, int xt, int64_t n, int64_t ldx, uint8_t *codes, uint16_t *norms,
               uint16_t *gammas, hipStream_t st) {
  // head dims up to 128 with 16-byte aligned rows: one fused kernel on the bf16 matrix cores
  const size_t esz0 = xt == TQ_F32 ? 4 : 2;
  if (encode_fused_supported(q) && (reinterpret_cast<uintptr_t>(x) & 15) == 0 && (ldx * esz0) % 16 == 0)
    return run_encode_fused(q, x, xt, n, ldx, codes, norms, gammas, st);
  const int d = q->d;
  const bool prod = q->mode == TQ_PROD;
  const int64_t chunk = prod ? std::max<int64_t>(64, (int64_t(1) << 27) / d) : (int64_t(1) << 22);
  const int64_t cmax = std::min(n, chunk);
  size_t bytes = (size_t)cmax * 4 + 256;
  if (prod) bytes += (size_t)cmax * d * 4 + (size_t)cmax * (d / 64) * 4 + 256;
  Scratch sc(st);
  int rc = sc.alloc(bytes);
  if (rc != TQ_OK) return rc;
  char *base = static_cast<char *>(sc.p);
  float *n32 = reinterpret_cast<float *>(base);
  float *resid = nullptr, *rsq = nullptr;
  if (prod) {
    size_t off = ((size_t)cmax * 4 + 255) & ~(size_t)255;
    resid = reinterpret_cast<float *>(base + off);
    off += ((size_t)cmax * d * 4 + 255) & ~(size_t)255;
    rsq = reinterpret_cast<float *>(base + off);
  }
  const size_t esz = xt == TQ_F32 ? 4 : 2;
  for (int64_t r0 = 0; r0 < n; r0 += chunk) {
    const int64_t cn = std::min(chunk, n - r0);
    const void *xc = static_cast<const char *>(x) + (size_t)r0 * ldx * esz;
    uint8_t *cc = codes + (size_t)r0 * q->code_bytes;
    uint16_t *nc = norms + r0;
    uint16_t *gc = gammas ? gammas + r0 : nullptr;
    if (xt == TQ_F32) rc = encode_chunk(q, LoadF32{static_cast<const float *>(xc), ldx}, xc, xt, ldx, cn, cc, nc, gc, n32, resid, rsq, st);
    else if (xt == TQ_BF16) rc = encode_chunk(q, LoadBF16{static_cast<const uint16_t *>(xc), ldx}, xc, xt, ldx, cn, cc, nc, gc, n32, resid, rsq, st);
    else rc = encode_chunk(q, LoadF16{static_cast<const uint16_t *>(xc), ldx}, xc, xt, ldx, cn, cc, nc, gc, n32, resid, rsq, st);
    if (rc != TQ_OK) return rc;
  }
  return TQ_OK;
}

int run_decode(const tq_quantizer *q, const uint8_t *codes, const uint16_t *norms, const uint16_t *gammas, int64_t n,
               float *out, int64_t ldo, hipStream_t st) {
  // head dims up to 128: one fused kernel on the bf16 matrix cores
  if (decode_fused_supported(q) && (reinterpret_cast<uintptr_t>(codes) & 3) == 0)
    return run_decode_fused(q, codes, norms, gammas, n, out, ldo, st);
  const int d = q->d;
  const bool prod = q->mode == TQ_PROD;
  LoadDequant ld{codes, norms, gammas, (int64_t)q->code_bytes, d, q->bmse, q->qjl_scale, q->cb};
  LoadCols2 lb{q->piT, prod ? q->sT : q->piT, d};
  EpiStore es{out, ldo};
  return gemm("decode", ld, lb, es, n, d, prod ? 2 * d : d, st);
}


size_t score_planes_ws_bytes(const tq_quantizer *q, int64_t m, int64_t n, int k);
bool score_planes_supported(const tq_quantizer *q);
int run_score_planes(const tq_quantizer *q, const float *queries, int64_t m, int64_t ldq, const uint8_t *codes,
                     const uint16_t *norms, const uint16_t *gammas, int64_t n, int k, float *scores, int64_t *idx,
                     void *ws, hipStream_t st);

size_t score_ws_bytes(const tq_quantizer *q, int64_t m, int64_t n, int k) {
  if (score_planes_supported(q)) return score_planes_ws_bytes(q, m, n, k);
  const int kq = q->mode == TQ_PROD ? 2 * q->d : q->d;
  size_t b = (((size_t)m * kq * 4) + 255) & ~(size_t)255;
  if (k > 0) b += (size_t)m * n * 4;
  return b;
}

// rotated queries [Pi q | S q] (the second half for Algorithm 2 only), fp32 [m][kq]
int rotate_queries(const tq_quantizer *q, const float *queries, int64_t m, int64_t ldq, float *qrot, hipStream_t st) {
  const int d = q->d;
  const bool prod = q->mode == TQ_PROD;
  const int kq = prod ? 2 * d : d;
  return gemm("score_qrot", LoadF32{queries, ldq}, LoadRows2{q->pi, prod ? q->s : q->pi, d, d}, EpiStore{qrot, kq}, m,
              kq, d, st);
}

int run_topk(const float *scores, int64_t m, int64_t n, int k, float *vals, int64_t *idx, hipStream_t st);

int run_score(const tq_quantizer *q, const float *queries, int64_t m, int64_t ldq, const uint8_t *codes,
              const uint16_t *norms, const uint16_t *gammas, int64_t n, int k, float *scores, int64_t *idx, void *ws,
              size_t ws_bytes, hipStream_t st) {
  // bit planes on the int8 matrix cores where the shape allows; otherwise dequantizing fp32 GEMMs
  if (score_planes_supported(q))
    return run_score_planes(q, queries, m, ldq, codes, norms, gammas, n, k, scores, idx, ws, st);
  const int d = q->d;
  const bool prod = q->mode == TQ_PROD;
  const int kq = prod ? 2 * d : d;
  float *qrot = static_cast<float *>(ws);
  int rc;
  if ((rc = rotate_queries(q, queries, m, ldq, qrot, st)) != TQ_OK) return rc;
  if (n == 0) return TQ_OK;
  float *dst = scores;
  if (k > 0) dst = reinterpret_cast<float *>(static_cast<char *>(ws) + ((((size_t)m * kq * 4) + 255) & ~(size_t)255));
  LoadDequant lb{codes, norms, gammas, (int64_t)q->code_bytes, d, q->bmse, q->qjl_scale, q->cb};
  if ((rc = gemm("score_scan", LoadF32{qrot, kq}, lb, EpiStore{dst, n}, m, n, kq, st)) != TQ_OK) return rc;
  if (k == 0) return TQ_OK;
  return run_topk(dst, m, n, k, scores, idx, st);
}

}  // namespace tq
