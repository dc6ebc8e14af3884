// Launchers of the grouped FP8 GEMM kernels (gemm_fp8_kernel.h) for
// decode-sized to medium groups, and the down projection of wide groups.
#include "gemm_fp8_kernel.h"

namespace k2 {

namespace {

// Gate/up launches up to 64-row tiles sum each block product exactly (EXACT):
// they wait on HBM, so the extra MFMA cycles are hidden, and the SwiGLU codes
// they requantise then match an exact evaluation except at true rounding
// ties.  Per m-tile width: TT = 1 (decode-sized groups) streams weights once, so
// non-temporal loads keep them from displacing the activations in L2; wider
// tiles share each weight chunk between m-tiles of one XCD through L2.
// NBUF = 3 at TT = 4 (two K blocks of weights in flight) fits in 2 waves/SIMD.
// TT = 8 halves the weight bytes per MFMA; with one activation register set
// and one token tile per scheduling group it also fits 2 waves/SIMD (two
// workgroups per CU), which hides each other's load and barrier waits.
template <bool GATEUP>
hipError_t launch_tt(int tt, const GemmArgs& a, int grid, hipStream_t s) {
  switch (tt) {
    case 1:   // uneven split over the XCDs: more workgroups than items
      gemm_fp8_kernel<GATEUP, 1, 2, true, 2, 1, 0, 0, 0, GATEUP><<<split_grid(grid), 256, 0, s>>>(a);
      break;
    case 2:
      gemm_fp8_kernel<GATEUP, 2, 2, false, 2, 1, 0, 0, 0, GATEUP><<<grid, 256, 0, s>>>(a);
      break;
    case 4:
      if constexpr (GATEUP)   // 2-deep ring, one token tile per group: no spill
        gemm_fp8_kernel<GATEUP, 4, 2, false, 2, 1, 1, 0, 0, true><<<grid, 256, 0, s>>>(a);
      else
        gemm_fp8_kernel<GATEUP, 4, 3, false, 2, 1><<<grid, 256, 0, s>>>(a);
      break;
    case 8:
      if constexpr (GATEUP) {
        return launch_gateup_tt8(a, grid, s);
      } else {
        gemm_fp8_kernel<GATEUP, 8, 2, false, 1, 2, 0, 1><<<grid, 256, 0, s>>>(a);
      }
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8(bool gateup, int tt, const GemmArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  return gateup ? launch_tt<true>(tt, a, grid, s) : launch_tt<false>(tt, a, grid, s);
}

// One weight matrix (a single group of T rows) in the down form, its K blocks
// cut into nsplit slices (grid.y); every block product summed exactly.
hipError_t launch_gemm_dense(int tt, int nsplit, const GemmArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  switch (tt) {
    case 1:
      gemm_fp8_kernel<false, 1, 2, false, 2, 1, 1, 0, 0, true, true>
          <<<dim3(split_grid(grid), nsplit), 256, 0, s>>>(a);
      break;
    case 2:
      gemm_fp8_kernel<false, 2, 2, false, 2, 1, 1, 0, 0, true, true>
          <<<dim3(grid, nsplit), 256, 0, s>>>(a);
      break;
    case 4:
      gemm_fp8_kernel<false, 4, 2, false, 2, 1, 1, 0, 0, true, true>
          <<<dim3(grid, nsplit), 256, 0, s>>>(a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace k2
