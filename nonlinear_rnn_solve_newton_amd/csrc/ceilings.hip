// ceilings.hip -- device ceilings for the rooflines of the solver's kernels,
// measured on the card. Not part of the solver: bench.py loads this library
// to report the ceilings beside the kernels of the same run.
//  - VALU issue rate (for the vector-ALU-bound fused Newton kernel): fp32 VALU
//    lane operations per second for plain (non-packed) FMAs, for the
//    transcendental unit (v_exp_f32 / v_rcp_f32), and for a sigmoid-shaped mix
//    of the two, at a chosen number of waves per SIMD.
//  - Streaming bandwidth (for the HBM-bound kernels): R arrays read and W
//    arrays written with 16-byte nontemporal accesses, grid-stride, as
//    read-only, write-only, copy and the adjoint's read/write mix.
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
extern "C" int ceil_issue_launch(int kind, int blocks, int iters, float m, float c, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out || kind < 0 || kind > 2) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0) hipLaunchKernelGGL(issue_kernel<0>, dim3(blocks), dim3(256), 0, s, out, iters, m, c);
  else if (kind == 1) hipLaunchKernelGGL(issue_kernel<1>, dim3(blocks), dim3(256), 0, s, out, iters, m, c);
  else hipLaunchKernelGGL(issue_kernel<2>, dim3(blocks), dim3(256), 0, s, out, iters, m, c);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int ceil_issue_steps_per_trip(void) { return kUnroll * kChains; }

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// the stream pointers, passed by value so that the accesses compile to global
// (not flat) instructions
struct Streams {
  const f32x4* in[5];
  f32x4* out[4];
};

// R input streams read, W output streams written, n16 16-byte elements each;
// NT: nontemporal loads and stores (else the default cache policy)
template <int R, int W, bool NT>
__global__ void __launch_bounds__(256) stream_kernel(const Streams p, long long n16, float* sink) {
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) {
    f32x4 v = {1.0f, 2.0f, 3.0f, 4.0f};
#pragma unroll
    for (int r = 0; r < R; ++r) v += NT ? __builtin_nontemporal_load(p.in[r] + i) : p.in[r][i];
#pragma unroll
    for (int w = 0; w < W; ++w) {
      if constexpr (NT) __builtin_nontemporal_store(v, p.out[w] + i);
      else p.out[w][i] = v;
    }
    acc += v;
  }
  if (W == 0 && acc.x == 1234.5f) sink[0] = acc.y;  // keeps the reads of a read-only stream
}

}  // namespace

// Streams: read `nread` and write `nwrite` device arrays of n16 16-byte
// elements (in: nread device pointers, out: nwrite device pointers, both host
// arrays), with nontemporal accesses when nt is 1. Supported (nread, nwrite):
// (1, 0), (0, 1), (1, 1), (5, 4). Returns 0, -1 for a bad argument, -4 when
// the launch fails.
template <bool NT>
int stream_launch(int nread, int nwrite, long long n16, const Streams& p, float* sink, int blocks, hipStream_t s) {
  if (nread == 1 && nwrite == 0) hipLaunchKernelGGL((stream_kernel<1, 0, NT>), dim3(blocks), dim3(256), 0, s, p, n16, sink);
  else if (nread == 0 && nwrite == 1) hipLaunchKernelGGL((stream_kernel<0, 1, NT>), dim3(blocks), dim3(256), 0, s, p, n16, sink);
  else if (nread == 1 && nwrite == 1) hipLaunchKernelGGL((stream_kernel<1, 1, NT>), dim3(blocks), dim3(256), 0, s, p, n16, sink);
  else if (nread == 5 && nwrite == 4) hipLaunchKernelGGL((stream_kernel<5, 4, NT>), dim3(blocks), dim3(256), 0, s, p, n16, sink);
  else return -1;
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int ceil_stream_launch(int nread, int nwrite, int nt, long long n16, void* const* in, void* const* out,
                                  float* sink, int blocks, void* stream) {
  if (n16 < 1 || blocks < 1 || !sink || nread < 0 || nread > 5 || nwrite < 0 || nwrite > 4) return -1;
  Streams p = {};
  for (int r = 0; r < nread; ++r) p.in[r] = static_cast<const f32x4*>(in[r]);
  for (int w = 0; w < nwrite; ++w) p.out[w] = static_cast<f32x4*>(out[w]);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return nt ? stream_launch<true>(nread, nwrite, n16, p, sink, blocks, s)
            : stream_launch<false>(nread, nwrite, n16, p, sink, blocks, s);
}
