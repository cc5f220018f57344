// Diagnostic: the bf16 MFMA rate the device sustains with no memory traffic,
// for the roofline context of the attention kernel (its clock under load
// depends on the operand data, so zero operands overstate what real data
// gets).
#include "fva_common.h"

namespace fva {

// Four independent v_mfma_f32_32x32x16_bf16 chains per wave, 4 waves per
// workgroup, operands zero or N(0,1)-like values from a hash of the lane id.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, int random_operands, float* __restrict__ sink) {
  const int t = threadIdx.x + blockIdx.x * 256;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t hsh = (uint32_t)(t * 8 + e) * 2654435761u;
    const float x = random_operands ? ((float)(hsh >> 8) * (1.0f / 16777216.0f) - 0.5f) * 3.4f : 0.0f;
    a[e] = (__bf16)x;
    b[e] = (__bf16)(random_operands ? x * 0.7f + 0.1f : 0.0f);
  }
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float f = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) f += acc[c][e];
  sink[t] = f;
}

}  // namespace fva

using namespace fva;

extern "C" int fva_mfma_probe(int32_t iters, int32_t random_operands, float* sink, int64_t sink_elems,
                              double* flops, void* stream) {
  if (iters < 1 || sink == nullptr || flops == nullptr) return FVA_ERR_ARG;
  const int grid = 2 * device_cu_count();
  if (grid < 2) return FVA_ERR_HIP;
  if (sink_elems < (int64_t)grid * 256) return FVA_ERR_WORKSPACE;
  mfma_probe_kernel<<<grid, 256, 0, (hipStream_t)stream>>>(iters, random_operands, sink);
  *flops = (double)grid * 4 /* waves */ * iters * 4 /* chains */ * 32768.0;
  return record_hip_error(hipGetLastError(), "mfma_probe launch");
}
