// Routing bias update of the K2 router (aux-loss-free load balancing).
//
// The router adds a per-expert correction bias to the sigmoid scores for the
// top-k choice only ("Kimi-K2-Base", Mixture of experts, Load balancing); the
// pages leave the rule that adjusts it undescribed.  The rule implemented is
// the published aux-loss-free balancing rule (Wang et al. 2024): with c_e the
// number of top-k choices of expert e over a training step and cbar their
// mean, b_e <- b_e + u * sign(cbar - c_e), decided on integers as
// sign(sum_e c_e - E * c_e), one fp32 addition per expert.
//
// Loads are integer counts, so they are the same whatever order the
// atomics land in: each workgroup counts its share of the choice array in an
// LDS histogram and adds its nonzero bins to the global counts.
#include <algorithm>

#include "k2_launch.h"

namespace k2 {

namespace {

constexpr int LOAD_THREADS = 256;
constexpr int LOAD_PER_THREAD = 8;     // choices per thread before the grid strides
constexpr int MAX_EXPERTS = 1024;

__global__ __launch_bounds__(LOAD_THREADS) void expert_load_kernel(int64_t n, int E,
                                                                   const int32_t* ids,
                                                                   int32_t* counts) {
  __shared__ int hist[MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += LOAD_THREADS) hist[e] = 0;
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * LOAD_THREADS;
  for (int64_t i = (int64_t)blockIdx.x * LOAD_THREADS + threadIdx.x; i < n; i += stride) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);   // other values: not an expert of this layer
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += LOAD_THREADS) {
    const int c = hist[e];
    if (c) atomicAdd(&counts[e], c);
  }
}

// one workgroup: the int64 total of the loads, then every expert's step
__global__ __launch_bounds__(MAX_EXPERTS) void bias_update_kernel(int E, const int32_t* counts,
                                                                  float speed, float* bias) {
  __shared__ long long wsum[MAX_EXPERTS / 64];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  const long long c = e < E ? (long long)counts[e] : 0;
  long long s = c;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) wsum[wave] = s;
  __syncthreads();
  long long total = 0;
#pragma unroll
  for (int w = 0; w < MAX_EXPERTS / 64; ++w) total += wsum[w];
  if (e < E) {
    const long long diff = total - (long long)E * c;   // sign(cbar - c_e)
    const float dir = diff > 0 ? 1.f : (diff < 0 ? -1.f : 0.f);
    bias[e] = __fadd_rn(bias[e], speed * dir);          // speed * dir is exact
  }
}

}  // namespace

hipError_t launch_expert_load(int64_t n, int E, const int32_t* ids, int32_t* counts,
                              hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t per_block = (int64_t)LOAD_THREADS * LOAD_PER_THREAD;
  const int grid = (int)std::min<int64_t>((n + per_block - 1) / per_block, 2048);
  expert_load_kernel<<<grid, LOAD_THREADS, 0, s>>>(n, E, ids, counts);
  return hipGetLastError();
}

hipError_t launch_bias_update(int E, const int32_t* counts, float speed, float* bias,
                              hipStream_t s) {
  bias_update_kernel<<<1, MAX_EXPERTS, 0, s>>>(E, counts, speed, bias);
  return hipGetLastError();
}

}  // namespace k2
