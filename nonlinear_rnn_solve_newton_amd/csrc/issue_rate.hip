// issue_rate.hip -- device ceilings for the roofline of the vector-ALU-bound
// fused Newton kernel, measured on the card: how many fp32 VALU lane
// operations per second the chip issues for plain (non-packed) FMAs, for the
// transcendental unit (v_exp_f32 / v_rcp_f32), and for a sigmoid-shaped mix of
// the two, at a chosen number of waves per SIMD. Not part of the solver:
// bench.py loads this library to report the ceilings beside the kernels.
#include <hip/hip_runtime.h>

namespace {

constexpr int kChains = 8;  // independent dependency chains per lane
constexpr int kUnroll = 16; // chain steps per loop trip

// KIND 0: x = fma(x, m, c)                      1 VALU op per step
// KIND 1: x = exp2(-|x|)                        1 transcendental per step
// KIND 2: x = rcp(1 + exp2(fma(x, m, c)))       2 VALU + 2 transcendental per step
template <int KIND>
__global__ void __launch_bounds__(256) issue_kernel(float* out, int iters, float m, float c) {
  float x[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) x[i] = static_cast<float>(threadIdx.x) * 1e-3f + 0.125f * i;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < kUnroll; ++r) {
#pragma unroll
      for (int i = 0; i < kChains; ++i) {
        if constexpr (KIND == 0) {
          x[i] = fmaf(x[i], m, c);
        } else if constexpr (KIND == 1) {
          x[i] = __builtin_amdgcn_exp2f(-fabsf(x[i]));
        } else {
          x[i] = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(fmaf(x[i], m, c)));
        }
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += x[i];
  out[static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// Launches `blocks` workgroups of 256 lanes (four waves), each lane running
// kChains chains of iters * kUnroll steps of the chosen kind, and writes one
// float per lane to out [blocks * 256]. Returns 0, or -1 for a bad argument,
// -4 when the launch fails. Instructions per lane: iters * kUnroll * kChains
// steps (KIND 2: four instructions per step).
extern "C" int issue_rate_launch(int kind, int blocks, int iters, float m, float c, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out || kind < 0 || kind > 2) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0) hipLaunchKernelGGL(issue_kernel<0>, dim3(blocks), dim3(256), 0, s, out, iters, m, c);
  else if (kind == 1) hipLaunchKernelGGL(issue_kernel<1>, dim3(blocks), dim3(256), 0, s, out, iters, m, c);
  else hipLaunchKernelGGL(issue_kernel<2>, dim3(blocks), dim3(256), 0, s, out, iters, m, c);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int issue_rate_steps_per_trip(void) { return kUnroll * kChains; }
