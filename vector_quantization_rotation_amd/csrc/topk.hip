// Top-k selection over a dense score matrix: per query the k largest scores,
// ties broken toward the lower record index (the search reading of the AiBoss
// overview, section "TurboQuantの応用事例": inner-product retrieval).
#include "common.cuh"

namespace tq {

constexpr int kTopkThreads = 256;
constexpr int kTopkMax = 64;

__device__ __forceinline__ bool better(float a, int64_t ia, float b, int64_t ib) {
  return a > b || (a == b && ia < ib);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float *scores, int64_t n, int k, float *vals,
                                                            int64_t *idx) {
  const int64_t qi = blockIdx.x;
  const float *row = scores + qi * n;
  float lv[kTopkMax];
  int64_t li[kTopkMax];
  int cnt = 0;
  for (int64_t i = threadIdx.x; i < n; i += kTopkThreads) {
    float v = row[i];
    if (cnt == k && !better(v, i, lv[k - 1], li[k - 1])) continue;
    int pos = cnt < k ? cnt : k - 1;
    // shift smaller entries down (indices arrive in increasing order per thread)
    while (pos > 0 && better(v, i, lv[pos - 1], li[pos - 1])) {
      lv[pos] = lv[pos - 1];
      li[pos] = li[pos - 1];
      --pos;
    }
    lv[pos] = v;
    li[pos] = i;
    if (cnt < k) ++cnt;
  }
  __shared__ float sv[kTopkThreads];
  __shared__ int64_t si[kTopkThreads];
  __shared__ int sw[kTopkThreads];
  int head = 0;
  for (int out = 0; out < k; ++out) {
    float hv = head < cnt ? lv[head] : -INFINITY;
    int64_t hi = head < cnt ? li[head] : INT64_MAX;
    sv[threadIdx.x] = hv;
    si[threadIdx.x] = hi;
    sw[threadIdx.x] = threadIdx.x;
    __syncthreads();
    for (int s = kTopkThreads / 2; s > 0; s >>= 1) {
      if (threadIdx.x < s) {
        int o = threadIdx.x + s;
        if (better(sv[o], si[o], sv[threadIdx.x], si[threadIdx.x])) {
          sv[threadIdx.x] = sv[o];
          si[threadIdx.x] = si[o];
          sw[threadIdx.x] = sw[o];
        }
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) {
      vals[qi * k + out] = sv[0];
      idx[qi * k + out] = si[0];
    }
    if (threadIdx.x == sw[0]) ++head;
    __syncthreads();
  }
}

int run_topk(const float *scores, int64_t m, int64_t n, int k, float *vals, int64_t *idx, hipStream_t st) {
  ProfScope ps("topk", st);
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)m), dim3(kTopkThreads), 0, st, scores, n, k, vals, idx);
  return launch_check();
}

}  // namespace tq
