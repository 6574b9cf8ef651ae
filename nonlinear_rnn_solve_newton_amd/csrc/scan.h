// scan.h -- the linear recurrence alone, s_l = A_l s_{l-1} + b_l per channel,
// with A_l a scalar (diagonal) or a 2x2 block over the channel's two state
// components. It is the solver step of every Newton iteration (ParaRNN
// article, cafecomtech.com, section "A sacada: metodo de Newton": each
// iteration is a linear SSM solved by a parallel scan), exported on its own
// for linear SSMs the caller assembles, e.g. from a cell whose Jacobian is
// formed outside this library (section "Como usar").
//
// Same hierarchy as the Newton iteration: T serial steps per lane, a shuffle
// scan over LL lane groups, an LDS scan over W waves, and the decoupled
// look-back across chunks of L. Loads of steps past L and of channels past D
// read zero through the buffer resources and come after every valid step of
// their channel in scan order, so no step is masked.
#pragma once

#include "newton_iter.h"

namespace pararnn {

struct ScanArgs {
  const float* A;   // [NS*NS][B][L][D] block entries, row-major within the block
  const float* b;   // [NS][B][L][D]
  const float* s0;  // [NS][B][D] or nullptr (zero)
  float* s;         // [NS][B][L][D]
  unsigned long long* incl;
  unsigned long long* agg;
  unsigned int* ctr;  // [0] ticket
  int B, L, D, nchunks, ntiles_d;
};

// INCL: the carry into a chunk is the predecessor's inclusive carry, waited
// for (no aggregates published or composed); chosen by the host where a chunk
// row has many tiles, so that predecessors run well ahead
template <int NS, int C, int T, int W, int LL, int OCC, bool INCL>
__global__ void __launch_bounds__(64 * W, OCC) scan_kernel(const ScanArgs p) {
  constexpr int LD = 64 / LL, CW = LD * C, CL = W * LL * T, NA = NS * NS + NS;
  constexpr uint32_t tag = 1u;

  __shared__ float s_agg[W][NA][CW];
  __shared__ float s_carry[NS][CW];
  __shared__ unsigned int s_ticket;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ld = lane % LD, ll = lane / LD;
  if (tid == 0) s_ticket = atomicAdd(p.ctr, 1u);
  __syncthreads();
  const unsigned int ticket = s_ticket;
  const unsigned int ntiles = static_cast<unsigned int>(p.B) * p.ntiles_d;
  const int chunk = static_cast<int>(ticket / ntiles);
  const int tile = static_cast<int>(ticket - static_cast<unsigned int>(chunk) * ntiles);
  const int b = tile / p.ntiles_d;
  const int d0 = (tile - b * p.ntiles_d) * CW + ld * C;
  const bool dv = d0 < p.D;
  const int lt0 = (wave * LL + ll) * T;
  const long long BD = static_cast<long long>(p.B) * p.ntiles_d * CW;
  const long long chan = static_cast<long long>(tile) * CW + ld;
  const long long plane = static_cast<long long>(p.B) * p.L * p.D;
  const long long wrow = static_cast<long long>(b) * p.L + static_cast<long long>(chunk) * CL;
  const uint32_t sstep = static_cast<uint32_t>(p.D * sizeof(float));
  const uint32_t rows = static_cast<uint32_t>(min(p.L - chunk * CL, CL));
  constexpr uint32_t kOOB = 0x80000000u;  // extents stay below 2^31 bytes
  const uint32_t vs0 = dv ? static_cast<uint32_t>(lt0) * sstep + static_cast<uint32_t>(d0 * sizeof(float)) : kOOB;
  __amdgpu_buffer_rsrc_t rA[NS * NS], rb[NS], rs[NS];
#pragma unroll
  for (int q = 0; q < NS * NS; ++q) rA[q] = make_rsrc(p.A + q * plane + wrow * p.D, rows * sstep);
#pragma unroll
  for (int r = 0; r < NS; ++r) {
    rb[r] = make_rsrc(p.b + r * plane + wrow * p.D, rows * sstep);
    rs[r] = make_rsrc(p.s + r * plane + wrow * p.D, rows * sstep);
  }

  float At[T][NS][NS][C], bt[T][NS][C];
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int r = 0; r < NS; ++r) {
#pragma unroll
      for (int q = 0; q < NS; ++q) buf_ld_f32<C>(rA[r * NS + q], vs0 + t * sstep, 0u, At[t][r][q]);
      buf_ld_f32<C>(rb[r], vs0 + t * sstep, 0u, bt[t][r]);
    }
  }

  // the lane's transform over its T steps, then the lane groups of the wave
  Aff<NS, C> acc;
  acc.set_identity();
#pragma unroll
  for (int t = 0; t < T; ++t) acc.pre(At[t], bt[t]);
  Aff<NS, C> excl;
  excl.set_identity();
  if constexpr (LL > 1) {
#pragma unroll
    for (int off = 1; off < LL; off *= 2) {
      const Aff<NS, C> prev = acc.shfl_up(off * LD);
      if (ll >= off) acc.after(prev);
    }
    const Aff<NS, C> prev = acc.shfl_up(LD);
    if (ll > 0) excl = prev;
  }
  if (ll == LL - 1) {
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) {
#pragma unroll
        for (int q = 0; q < NS; ++q) s_agg[wave][r * NS + q][ld * C + c] = acc.A[r][q][c];
        s_agg[wave][NS * NS + r][ld * C + c] = acc.b[r][c];
      }
  }
  __syncthreads();

  // workgroup total; the chunk's carry-in is s0 for the first chunk and the
  // look-back result for the others
  if (wave == 0 && ll == 0) {
    float carry[NS][C];
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) carry[r][c] = 0.0f;
    if (dv && chunk == 0 && p.s0) {
#pragma unroll
      for (int r = 0; r < NS; ++r) ld_f32<C>(p.s0 + (static_cast<long long>(r) * p.B + b) * p.D + d0, carry[r]);
    }
    if (dv && p.nchunks > 1) {
      Aff<NS, C> tot;
      tot.set_identity();
#pragma unroll
      for (int w = 0; w < W; ++w) {
        Aff<NS, C> e;
#pragma unroll
        for (int r = 0; r < NS; ++r)
#pragma unroll
          for (int c = 0; c < C; ++c) {
#pragma unroll
            for (int q = 0; q < NS; ++q) e.A[r][q][c] = s_agg[w][r * NS + q][ld * C + c];
            e.b[r][c] = s_agg[w][NS * NS + r][ld * C + c];
          }
        e.after(tot);
        tot = e;
      }
      if (chunk > 0) {
        if constexpr (INCL) {
          wait_incl<NS, C>(p.incl, BD, chan, LD, chunk - 1, tag, carry);
        } else {
          if (chunk < p.nchunks - 1) publish_agg<NS, C>(p.agg, BD, chan, LD, chunk, tag, tot);
          lookback<NS, C>(p.incl, p.agg, BD, chan, LD, chunk, -1, p.nchunks, tag, carry);
        }
      }
      if (chunk < p.nchunks - 1) {
        float x[NS][C];
#pragma unroll
        for (int r = 0; r < NS; ++r)
#pragma unroll
          for (int c = 0; c < C; ++c) x[r][c] = carry[r][c];
        tot.apply(x);
        publish_incl<NS, C>(p.incl, BD, chan, LD, chunk, tag, x);
      }
    }
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) s_carry[r][ld * C + c] = carry[r][c];
  }
  __syncthreads();

  // carry into the lane's first step: the chunk carry through the earlier
  // waves and lane groups
  float x[NS][C];
#pragma unroll
  for (int r = 0; r < NS; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) x[r][c] = s_carry[r][ld * C + c];
  for (int w = 0; w < wave; ++w) {
    Aff<NS, C> e;
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) {
#pragma unroll
        for (int q = 0; q < NS; ++q) e.A[r][q][c] = s_agg[w][r * NS + q][ld * C + c];
        e.b[r][c] = s_agg[w][NS * NS + r][ld * C + c];
      }
    e.apply(x);
  }
  if constexpr (LL > 1) excl.apply(x);

#pragma unroll
  for (int t = 0; t < T; ++t) {
    float y[NS][C];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        float a2 = bt[t][r][c];
#pragma unroll
        for (int q = 0; q < NS; ++q) a2 = fmaf(At[t][r][q][c], x[q][c], a2);
        y[r][c] = a2;
      }
#pragma unroll
    for (int r = 0; r < NS; ++r) {
#pragma unroll
      for (int c = 0; c < C; ++c) x[r][c] = y[r][c];
      buf_st_f32<C>(rs[r], vs0 + t * sstep, 0u, x[r]);  // dropped past L or D
    }
  }
}

}  // namespace pararnn
