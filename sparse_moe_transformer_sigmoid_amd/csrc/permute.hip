// Stable grouping of the (token, slot) pairs by expert, and the per-group
// m-tile prefix used to schedule the grouped GEMMs.
//
// The MoE treats batch and positions as one token axis ("Kimi-K2-Base",
// Mixture of experts, Load balancing: scores are viewed as
// [bsz * seq_len, n_experts]); every selected expert then processes its
// tokens.  Rows of expert e are its tokens in ascending order.  The rank of a
// token inside its expert is counted, not claimed with an atomic, so the
// permutation is the same on every run:
//   1. per chunk of tokens, count the pairs of every expert;
//   2. scan the counts over chunks (per expert) and over experts;
//   3. per chunk, set one bit per (expert, token) and take the rank of a
//      token as the number of set bits before it.
#include "k2_common.h"
#include "k2_launch.h"

namespace k2 {

namespace {

constexpr int MASK_WORDS = 2048;  // per-expert token bitmasks: 2 words x up to 1024 experts

// Exclusive scan of get(0..n-1) by a 1024-thread block; out[n] = total.
template <int IPT, class F>
__device__ void block_exclusive_scan(int n, F get, int32_t* out) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  int32_t local[IPT];
  int32_t sum = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int i = tid * IPT + j;
    local[j] = i < n ? get(i) : 0;
    sum += local[j];
  }
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - sum;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int i = tid * IPT + j;
    if (i < n) out[i] = run;
    run += local[j];
  }
  if (tid == 1023) out[n] = part[1023];
}

__global__ __launch_bounds__(256) void perm_count_kernel(int T, int E, int k, int chunk,
                                                        const int32_t* __restrict__ ids,
                                                        int32_t* __restrict__ chunk_counts) {
  __shared__ int32_t cnt[1024];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int t0 = c * chunk, t1 = min(T, t0 + chunk);
  for (int p = t0 * k + threadIdx.x; p < t1 * k; p += 256)
    atomicAdd(&cnt[min(max(ids[p], 0), E - 1)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(size_t)c * E + e] = cnt[e];
}

__global__ __launch_bounds__(1024) void perm_scan_kernel(int E, int nchunk,
                                                        const int32_t* __restrict__ chunk_counts,
                                                        int32_t* __restrict__ chunk_base,
                                                        int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[1024];
  for (int e = threadIdx.x; e < E; e += 1024) {
    int32_t run = 0;
#pragma unroll 8
    for (int c = 0; c < nchunk; ++c) {
      chunk_base[(size_t)c * E + e] = run;
      run += chunk_counts[(size_t)c * E + e];
    }
    tot[e] = run;
  }
  __syncthreads();
  block_exclusive_scan<1>(E, [&](int i) { return tot[i]; }, offsets);
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(int T, int E, int k, int chunk,
                                                          const int32_t* __restrict__ ids,
                                                          const int32_t* __restrict__ chunk_base,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ row_pair,
                                                          int32_t* __restrict__ pair_row) {
  __shared__ uint32_t mask[MASK_WORDS];
  const int c = blockIdx.x;
  const int words = chunk >> 5;
  for (int i = threadIdx.x; i < E * words; i += 256) mask[i] = 0u;
  __syncthreads();
  const int t0 = c * chunk, t1 = min(T, t0 + chunk);
  for (int p = t0 * k + threadIdx.x; p < t1 * k; p += 256) {
    const int tl = p / k - t0;
    const int e = min(max(ids[p], 0), E - 1);
    atomicOr(&mask[e * words + (tl >> 5)], 1u << (tl & 31));
  }
  __syncthreads();
  for (int p = t0 * k + threadIdx.x; p < t1 * k; p += 256) {
    const int e = min(max(ids[p], 0), E - 1);
    const int tl = p / k - t0;
    const uint32_t* me = mask + e * words;
    int rank = __popc(me[tl >> 5] & ((1u << (tl & 31)) - 1u));
    for (int w = 0; w < (tl >> 5); ++w) rank += __popc(me[w]);
    const int row = offsets[e] + chunk_base[(size_t)c * E + e] + rank;
    row_pair[row] = p;
    pair_row[p] = row;
  }
}

// All tokens in one chunk (decode-sized batches): the three passes above in
// one workgroup.  Counts are the popcounts of each expert's token mask, their
// exclusive scan gives the offsets, and a token's rank is again the number
// of set bits before it, so the rows equal those of the three-pass path.
// With mt_start non-null it also builds the GEMM m-tile table, as
// build_tiles_kernel does.
__global__ __launch_bounds__(1024) void perm_small_kernel(int T, int E, int k, int words,
                                                         const int32_t* __restrict__ ids,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ row_pair,
                                                         int32_t* __restrict__ pair_row,
                                                         int n_shared, int bm, int max_tiles,
                                                         int32_t* __restrict__ mt_start,
                                                         int32_t* __restrict__ tile_group) {
  __shared__ uint32_t mask[MASK_WORDS];
  __shared__ int32_t off[1025];
  const int tid = threadIdx.x;
  for (int i = tid; i < E * words; i += 1024) mask[i] = 0u;
  __syncthreads();
  for (int p = tid; p < T * k; p += 1024) {
    const int t = p / k;
    const int e = min(max(ids[p], 0), E - 1);
    atomicOr(&mask[e * words + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
  block_exclusive_scan<1>(
      E,
      [&](int e) {
        int c = 0;
        for (int w = 0; w < words; ++w) c += __popc(mask[e * words + w]);
        return c;
      },
      off);
  __syncthreads();
  for (int e = tid; e <= E; e += 1024) offsets[e] = off[e];
  for (int p = tid; p < T * k; p += 1024) {
    const int e = min(max(ids[p], 0), E - 1);
    const int t = p / k;
    const uint32_t* me = mask + e * words;
    int rank = __popc(me[t >> 5] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(me[w]);
    const int row = off[e] + rank;
    row_pair[row] = p;
    pair_row[p] = row;
  }
  if (mt_start == nullptr) return;
  const int P = T * k, G = E + n_shared;
  block_exclusive_scan<2>(
      G,
      [&](int g) {
        int m = T;
        if (g < E) {
          const int r0 = min(max(off[g], 0), P);
          m = min(max(off[g + 1] - r0, 0), P - r0);
        }
        return (m + bm - 1) / bm;
      },
      mt_start);
  __syncthreads();
  for (int g = tid; g < G; g += 1024) {
    const int q1 = min(mt_start[g + 1], max_tiles);
    for (int q = mt_start[g]; q < q1; ++q) tile_group[q] = g;
  }
}

// mt_start[g] = sum over groups before g of ceil(m_g / bm); groups are the
// routed experts 0..E-1 (m = expert count) and then the shared expert (m = T).
// Row ranges are clamped into [0, P) exactly as the GEMM kernels clamp them.
// tile_group[q] = the group of m-tile q, so a GEMM workgroup finds its group
// with one load (q < mt_start[G] <= max_tiles).
__global__ __launch_bounds__(1024) void build_tiles_kernel(int E, int n_shared, int T, int P,
                                                          int bm, int max_tiles,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ mt_start,
                                                          int32_t* __restrict__ tile_group) {
  const int G = E + n_shared;
  block_exclusive_scan<2>(
      G,
      [&](int g) {
        int m = T;
        if (g < E) {
          const int r0 = min(max(offsets[g], 0), P);
          m = min(max(offsets[g + 1] - r0, 0), P - r0);
        }
        return (m + bm - 1) / bm;
      },
      mt_start);
  __syncthreads();
  if (tile_group == nullptr) return;
  for (int g = threadIdx.x; g < G; g += 1024) {
    const int q1 = min(mt_start[g + 1], max_tiles);
    for (int q = mt_start[g]; q < q1; ++q) tile_group[q] = g;
  }
}

}  // namespace

// 64 tokens per chunk: a large batch spreads the count and scatter passes over
// many workgroups (8192 tokens -> 128), and a token's rank needs at most two
// mask words
int perm_chunk_tokens(int E) {
  int words = MASK_WORDS / E;
  if (words > 2) words = 2;
  return 32 * words;
}

hipError_t launch_permute(int T, int E, int k, const int32_t* ids, int32_t* chunk_counts,
                          int32_t* chunk_base, int32_t* offsets, int32_t* row_pair,
                          int32_t* pair_row, hipStream_t s, const TileReq* tiles,
                          bool* tiles_built) {
  const int chunk = perm_chunk_tokens(E);
  const int nchunk = (T + chunk - 1) / chunk;
  if (tiles_built) *tiles_built = false;
  if (nchunk == 1) {
    perm_small_kernel<<<1, 1024, 0, s>>>(T, E, k, chunk >> 5, ids, offsets, row_pair, pair_row,
                                         tiles ? tiles->n_shared : 0, tiles ? tiles->bm : 1,
                                         tiles ? tiles->max_tiles : 0,
                                         tiles ? tiles->mt_start : nullptr,
                                         tiles ? tiles->tile_group : nullptr);
    if (tiles && tiles_built) *tiles_built = true;
    return hipGetLastError();
  }
  perm_count_kernel<<<nchunk, 256, 0, s>>>(T, E, k, chunk, ids, chunk_counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  perm_scan_kernel<<<1, 1024, 0, s>>>(E, nchunk, chunk_counts, chunk_base, offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  perm_scatter_kernel<<<nchunk, 256, 0, s>>>(T, E, k, chunk, ids, chunk_base, offsets, row_pair,
                                             pair_row);
  return hipGetLastError();
}

hipError_t launch_build_tiles(int E, int n_shared, int T, int k, int bm, int max_tiles,
                              const int32_t* offsets, int32_t* mt_start, int32_t* tile_group,
                              hipStream_t s) {
  build_tiles_kernel<<<1, 1024, 0, s>>>(E, n_shared, T, T * k, bm, max_tiles, offsets, mt_start,
                                        tile_group);
  return hipGetLastError();
}

}  // namespace k2
