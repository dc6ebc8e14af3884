// Gate/up GEMM of wide groups (128-row m-tiles, two workgroups per CU).
// Built as its own translation unit with the register-minimising scheduler,
// which keeps the 128 accumulators, the weight ring and the activation
// staging within the 256-register budget of 2 waves/SIMD.  One token tile
// per scheduling group; inside it the MFMAs are interleaved with the fp32
// promotion FMAs of the MFMA two back (ILV 5).
#include "gemm_fp8_kernel.h"

namespace k2 {

hipError_t launch_gateup_tt8(const GemmArgs& a, int grid, hipStream_t s) {
  gemm_fp8_kernel<true, 8, 2, false, 1, 2, 1, 0, 5><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace k2
