// fp32-format SwiGLU experts ("Kimi-K2-Base", Feed-forward:
// down_proj(act_fn(gate_proj(x)) * up_proj(x)), act_fn = SiLU, no biases).
// Used by the all-fp32 layer format, where nothing is quantised.  One thread
// per output element; the permuted rows of routed expert e are
// [offsets[e], offsets[e+1]) and the shared expert's rows follow at P + t.
#include "k2_common.h"
#include "k2_launch.h"

namespace k2 {

namespace {

// group and activation row (token) of permuted row `row`
__device__ __forceinline__ void row_group(int row, int P, int T, int E, int k,
                                          const int32_t* offsets, const int32_t* row_pair,
                                          int* grp, int* tok) {
  if (row >= P) {
    *grp = E;
    *tok = row - P;
    return;
  }
  int lo = 0, hi = E;  // offsets[lo] <= row < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= row) lo = mid; else hi = mid;
  }
  *grp = lo;
  *tok = min(max(row_pair[row] / k, 0), T - 1);
}

__global__ __launch_bounds__(256) void experts_f32_gateup_kernel(
    int T, int d, int I, int E, int k, int P, int nrows, const float* __restrict__ h,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row_pair,
    const float* __restrict__ packed, size_t ef, float* __restrict__ abuf) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)nrows * I) return;
  const int row = (int)(idx / I), i = (int)(idx - (long)row * I);
  int grp, tok;
  row_group(row, P, T, E, k, offsets, row_pair, &grp, &tok);
  const float* wg = packed + (size_t)grp * ef + (size_t)i * d;
  const float* wu = wg + (size_t)I * d;
  const float* hp = h + (size_t)tok * d;
  float gv = 0.f, uv = 0.f;
  for (int j = 0; j < d; ++j) {
    gv = fmaf(hp[j], wg[j], gv);
    uv = fmaf(hp[j], wu[j], uv);
  }
  abuf[idx] = gv / (1.0f + expf(-gv)) * uv;
}

__global__ __launch_bounds__(256) void experts_f32_down_kernel(
    int T, int d, int I, int E, int k, int P, int nrows, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ row_pair, const float* __restrict__ packed, size_t ef,
    const float* __restrict__ abuf, float* __restrict__ rows, float* __restrict__ shared_out,
    const float* __restrict__ topk_w, int weighted) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)nrows * d) return;
  const int row = (int)(idx / d), n = (int)(idx - (long)row * d);
  int grp, tok;
  row_group(row, P, T, E, k, offsets, row_pair, &grp, &tok);
  const float* wd = packed + (size_t)grp * ef + 2 * (size_t)I * d + (size_t)n * I;
  const float* ap = abuf + (size_t)row * I;
  float o = 0.f;
  for (int i = 0; i < I; ++i) o = fmaf(ap[i], wd[i], o);
  if (row >= P) {
    shared_out[(size_t)tok * d + n] = o;
  } else {
    if (weighted) o = o * topk_w[min(max(row_pair[row], 0), P - 1)];
    rows[(size_t)row * d + n] = o;
  }
}

}  // namespace

hipError_t launch_experts_f32(int T, int d, int I, int E, int k, int n_shared, const float* h,
                              const int32_t* offsets, const int32_t* row_pair,
                              const float* packed, size_t expert_floats, float* abuf,
                              float* rows, float* shared_out, const float* topk_w,
                              int weighted, hipStream_t s) {
  const int P = T * k;
  const int nrows = P + (n_shared ? T : 0);
  const long n1 = (long)nrows * I, n2 = (long)nrows * d;
  experts_f32_gateup_kernel<<<(unsigned)((n1 + 255) / 256), 256, 0, s>>>(
      T, d, I, E, k, P, nrows, h, offsets, row_pair, packed, expert_floats, abuf);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  experts_f32_down_kernel<<<(unsigned)((n2 + 255) / 256), 256, 0, s>>>(
      T, d, I, E, k, P, nrows, offsets, row_pair, packed, expert_floats, abuf, rows, shared_out,
      topk_w, weighted);
  return hipGetLastError();
}

}  // namespace k2
