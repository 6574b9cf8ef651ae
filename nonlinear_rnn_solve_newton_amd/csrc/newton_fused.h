// newton_fused.h -- all K Newton iterations of the ParaRNN solve in one launch
// (the fully fused form: Newton, Jacobian assembly and the parallel reduction
// in one kernel, ParaRNN article, cafecomtech.com, section "Engenharia pra
// escalar").
//
// Each workgroup owns one (chunk, channel tile) for the whole solve and keeps
// its iterate in registers from iteration to iteration; the intermediate
// iterates never reach HBM, and only the K-th is stored. Iteration k is the
// update form of the one-launch kernel (newton_iter.h): d_l = J_l d_{l-1} + r_l
// with r_l = f(S^(k-1)_{l-1}, u_l) - S^(k-1)_l. The one value a lane needs
// from outside its own steps is the iterate at the row before its first step,
// its linearisation point there. The carry entering the lane group in
// iteration k is exactly the update d^(k) at that row, so each lane keeps that
// iterate as a running sum, S^(k) = S^(k-1) + carry_k (S^(0) = 0; the first
// lane group of the first chunk sees the fixed initial state), and nothing
// crosses lanes, waves or workgroups for it.
// Every iteration has its own descriptor slots, so a predecessor that runs
// ahead never overwrites what a later chunk still has to read; workgroups
// take tickets in chunk-major order and only ever wait for earlier tickets,
// so no residency of the whole grid is needed.
//
// Latency hiding inside an iteration:
//   - every wave reads the predecessor chunk's inclusive carry halfway through
//     its cell evaluations, so in the common case (the predecessor has already
//     published it) the carry is in registers when the local scan ends, and
//     the look-back round trip to memory is off the critical path; only when
//     that early read finds nothing does the wave publish the chunk aggregate
//     and walk back through the descriptors;
//   - each wave forms its own carry-in from the chunk carry and the preceding
//     waves' aggregates, so one barrier per iteration is enough; the last wave
//     publishes the chunk's inclusive carry;
//   - per-wave maxima of |d| leave through a cross-lane (DPP) reduction, one
//     word per wave, reduced over the grid by the finalize launch;
//   - no descriptor read is left in flight past a branch (loads and stores
//     share one counter on this GPU: a read the compiler cannot count on
//     every path turns the next reuse of its registers into a wait for all
//     memory operations, the previous iteration's stores included).
//
// UMODE: where the gate inputs live between iterations. 0: streamed from
// memory again in every iteration; 1: kept in registers (one HBM read per
// solve); 2: read once and kept in workgroup memory, each wave in a region of
// its own (one HBM read per solve, and the registers go to occupancy); 3: as
// 2, but widened to fp32 and multiplied by the cell's exponential scales on
// the way in, so that no iteration widens or scales them again (twice the
// workgroup memory of 2 for bf16 inputs).
#pragma once

#include "newton_iter.h"

namespace pararnn {

struct FusedArgs {
  const void* u;             // [B][L][G][D] fp32 or bf16
  const float* a;            // [G][D]
  const float* s0[2];        // initial state per component [B][D]; nullptr = 0
  float* sout[2];            // iterate K per component [B][L][D]
  unsigned long long* incl;  // [K][nchunks][NS][slots]
  unsigned long long* agg;   // [K][nchunks][NS*NS+NS][slots] (look-back mode only)
  unsigned int* ctr;         // [0] ticket
  unsigned int* pmax;        // [K][B][nchunks][ntiles_d][W] per-wave max |update| bits
  int B, L, D, K, nchunks, ntiles_d;
};

// Maximum over the wave of a value whose bit pattern orders like an unsigned
// integer (non-negative floats, NaN above +inf), returned to every lane: row
// reductions by quad and row rotations, then row broadcasts into lane 63.
__device__ __forceinline__ uint32_t wave_max_bits(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xb1, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4e, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x124, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

template <class Cell, class UT, int C, int T, int W, int LL, int OCC, int UMODE, bool INCL>
__global__ void __launch_bounds__(64 * W, OCC) newton_fused_kernel(const FusedArgs p) {
  constexpr int NS = Cell::NS, G = Cell::G;
  constexpr int LD = 64 / LL, CW = LD * C, CL = W * LL * T, NA = NS * NS + NS;
  constexpr int TPOLL = T / 2;  // the predecessor's carry is read before this step

  __shared__ float s_agg[2][W][NA][CW];  // per-wave aggregates, double-buffered over iterations
  // UMODE 2: gate inputs [wave][lane group][step][gate][channel], one padding
  // segment per lane group so the lane groups of a wave read disjoint banks
  constexpr int USEG = LD * C;  // elements of one (step, gate) row of a lane group
  constexpr int UGRP = T * G * USEG + USEG;
  __shared__ __align__(16) UT s_u[UMODE == 2 ? W * LL * UGRP : 1];
  __shared__ __align__(16) float s_us[UMODE == 3 ? W * LL * UGRP : 1];  // UMODE 3: scaled fp32
  __shared__ unsigned int s_ticket;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ld = lane % LD, ll = lane / LD;
  const int q = wave * LL + ll;  // lane group in scan order
  if (tid == 0) s_ticket = atomicAdd(p.ctr, 1u);
  __syncthreads();
  const unsigned int ticket = s_ticket;
  const unsigned int ntiles = static_cast<unsigned int>(p.B) * p.ntiles_d;
  const int chunk = static_cast<int>(ticket / ntiles);
  const int tile = static_cast<int>(ticket - static_cast<unsigned int>(chunk) * ntiles);
  const int b = tile / p.ntiles_d;
  const int dt0 = (tile - b * p.ntiles_d) * CW;
  const int d0 = dt0 + ld * C;
  const bool dv = d0 < p.D;
  const int lt0 = q * T;
  const int l0 = chunk * CL + lt0;
  const long long BD = static_cast<long long>(p.B) * p.ntiles_d * CW;
  const long long chan = static_cast<long long>(tile) * CW + ld;
  const long long inc_k = static_cast<long long>(p.nchunks) * NS * BD;  // words per iteration
  const long long agg_k = static_cast<long long>(p.nchunks) * NA * BD;
  const long long wrow = static_cast<long long>(b) * p.L + static_cast<long long>(chunk) * CL;
  const uint32_t ustep = static_cast<uint32_t>(G * p.D * sizeof(UT));
  const uint32_t gstep = static_cast<uint32_t>(p.D * sizeof(UT));
  const uint32_t sstep = static_cast<uint32_t>(p.D * sizeof(float));
  const uint32_t rows = static_cast<uint32_t>(min(p.L - chunk * CL, CL));
  constexpr uint32_t kOOB = 0x80000000u;  // extents stay below 2^31 bytes
  const uint32_t vu0 = dv ? static_cast<uint32_t>(lt0) * ustep + static_cast<uint32_t>(d0 * sizeof(UT)) : kOOB;
  const uint32_t vs0 = dv ? static_cast<uint32_t>(lt0) * sstep + static_cast<uint32_t>(d0 * sizeof(float)) : kOOB;
  const __amdgpu_buffer_rsrc_t ru =
      make_rsrc(reinterpret_cast<const char*>(p.u) + wrow * G * p.D * static_cast<long long>(sizeof(UT)), rows * ustep);
  __amdgpu_buffer_rsrc_t rout[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) rout[s] = make_rsrc(p.sout[s] + wrow * p.D, rows * sstep);
  const int dc = dv ? d0 : p.D - C;  // channel group for the per-channel loads
  const bool pred = chunk > 0;       // the chunk carry comes from predecessor chunks
  // per-wave maxima: [K][B][nchunks][ntiles_d][W]
  unsigned int* pmax = p.pmax + ((static_cast<long long>(b) * p.nchunks + chunk) * p.ntiles_d + dt0 / CW) * W + wave;
  const long long pmax_k = static_cast<long long>(p.B) * p.nchunks * p.ntiles_d * W;

  auto tile_body = [&](auto full_tag) {
  constexpr bool FULL = decltype(full_tag)::value;
  float av[G][C];
#pragma unroll
  for (int g = 0; g < G; ++g) ld_f32<C>(p.a + static_cast<long long>(g) * p.D + dc, av[g]);
  URaw<UT, C> uu[UMODE == 1 ? T : 1][G];
  UT* su = s_u + (wave * LL + ll) * UGRP + ld * C;  // this lane's channels, step 0, gate 0
  float* sus = s_us + (wave * LL + ll) * UGRP + ld * C;
  float avs[UMODE == 3 ? G : 1][C];  // coefficients times the exponential scales
  if constexpr (UMODE == 3) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < C; ++c) avs[g][c] = av[g][c] * Cell::kScale[g];
  }
  if constexpr (UMODE == 1) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int g = 0; g < G; ++g) uu[t][g].load(ru, vu0 + t * ustep, static_cast<uint32_t>(g) * gstep);
  } else if constexpr (UMODE == 2) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      URaw<UT, C> x[G];
#pragma unroll
      for (int g = 0; g < G; ++g) x[g].load(ru, vu0 + t * ustep, static_cast<uint32_t>(g) * gstep);
#pragma unroll
      for (int g = 0; g < G; ++g) x[g].put_lds(su + (t * G + g) * USEG);
    }
  } else if constexpr (UMODE == 3) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      URaw<UT, C> x[G];
#pragma unroll
      for (int g = 0; g < G; ++g) x[g].load(ru, vu0 + t * ustep, static_cast<uint32_t>(g) * gstep);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < C; ++c) sus[(t * G + g) * USEG + c] = x[g].get(c) * Cell::kScale[g];
    }
  }
  // every iteration, the first included, reads the inputs back from workgroup
  // memory: the compiler may not keep the just-stored values in registers
  // instead, which would hold them live through the first iteration
  if constexpr (UMODE >= 2) __asm__ volatile("" ::: "memory");
  // iterate k-1 at the lane's steps (S^(0) = 0), and at the row before the
  // lane group's first step (the fixed initial state before the sequence)
  float so[T][NS][C];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int c = 0; c < C; ++c) so[t][s][c] = 0.0f;
  float sp[NS][C];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int c = 0; c < C; ++c) sp[s][c] = 0.0f;
    if (chunk == 0 && q == 0 && p.s0[s]) ld_f32<C>(p.s0[s] + static_cast<long long>(b) * p.D + dc, sp[s]);
  }

  // one Newton iteration; ZERO: the first, evaluated at the zero iterate
  // (reduced cell form from a lane's third step on, as in newton_iter.h)
  auto iterate = [&](int k, auto zero_tag) {
    constexpr bool ZERO = decltype(zero_tag)::value;
    const uint32_t tag = static_cast<uint32_t>(k);
    const int buf = k & 1;
    unsigned long long* incl = p.incl + (k - 1) * inc_k;
    [[maybe_unused]] unsigned long long* agg = p.agg + (k - 1) * agg_k;
    unsigned long long early[NS][C];  // the predecessor's inclusive carry, read early
    typename Cell::Jac Jt[T][C];
    float rt[T][NS][C];
    Aff<NS, C> acc;  // the lane's transform over its steps, from its first step
    // gate inputs held in workgroup memory (UMODE 2, 3) are read one step
    // ahead of their use, so that each read has a whole step of cell work to
    // complete behind
    URaw<UT, C> un[UMODE == 2 ? G : 1];
    float uns[UMODE == 3 ? G : 1][C];
    auto fetch = [&](int tt) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if constexpr (UMODE == 2) un[g].get_lds(su + (tt * G + g) * USEG);
        else if constexpr (UMODE == 3) {
#pragma unroll
          for (int c = 0; c < C; ++c) uns[g][c] = sus[(tt * G + g) * USEG + c];
        }
      }
    };
    if constexpr (UMODE >= 2) fetch(0);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (t == TPOLL) {
        __builtin_amdgcn_sched_barrier(0);
        // every workgroup issues the read, so that no branch hides it from
        // the compiler's count of loads in flight; the first chunk reads its
        // own slot and ignores the value
        const long long pc = pred ? chunk - 1 : 0;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int c = 0; c < C; ++c) early[s][c] = desc_get(incl + (pc * NS + s) * BD + chan + c * LD);
        __builtin_amdgcn_sched_barrier(0);
      }
      URaw<UT, C> ut[G];
      float uts[UMODE == 3 ? G : 1][C];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if constexpr (UMODE == 1) ut[g] = uu[t][g];
        else if constexpr (UMODE == 2) ut[g] = un[g];
        else if constexpr (UMODE == 3) {
#pragma unroll
          for (int c = 0; c < C; ++c) uts[g][c] = uns[g][c];
        } else {
          ut[g].load(ru, vu0 + t * ustep, static_cast<uint32_t>(g) * gstep);
        }
      }
      if constexpr (UMODE >= 2) {
        if (t + 1 < T) fetch(t + 1);
      }
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float ac[G], uc[G], pc[NS], f[NS], sc[NS], rr[NS];
        typename Cell::Jac J;
#pragma unroll
        for (int g = 0; g < G; ++g) { ac[g] = av[g][c]; uc[g] = UMODE == 3 ? uts[g][c] : ut[g].get(c); }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          pc[s] = (t == 0) ? sp[s][c] : so[t - 1][s][c];
          sc[s] = so[t][s][c];
        }
        if constexpr (UMODE == 3) {
          float acs[G];
#pragma unroll
          for (int g = 0; g < G; ++g) acs[g] = avs[g][c];
          if (ZERO && t > 1) Cell::step_zero_scaled(ac, uc, f, J);
          else Cell::step_scaled(ac, acs, uc, pc, f, J);
        } else {
          if (ZERO && t > 1) Cell::step_zero(ac, uc, f, J);
          else Cell::step(ac, uc, pc, f, J);
        }
        Cell::template residual<ZERO>(f, sc, J, rr);
        Jt[t][c] = J;
#pragma unroll
        for (int r = 0; r < NS; ++r) rt[t][r][c] = rr[r];
        if (t == 0) Cell::first(acc, c, J, rr);
        else Cell::pre(acc, c, J, rr);
      }
    }

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
          for (int s = 0; s < NS; ++s) s_agg[buf][wave][r * NS + s][ld * C + c] = acc.A[r][s][c];
          s_agg[buf][wave][NS * NS + r][ld * C + c] = acc.b[r][c];
        }
    }
    __syncthreads();
    // the early read completes here on every path: one still in flight
    // past the branches below would make the compiler wait for all memory
    // operations at the next iteration's start, the stores included
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int c = 0; c < C; ++c) __asm__ volatile("" ::"v"(early[s][c]));

    auto wave_agg = [&](int w) {
      Aff<NS, C> e;
#pragma unroll
      for (int r = 0; r < NS; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) {
#pragma unroll
          for (int s = 0; s < NS; ++s) e.A[r][s][c] = s_agg[buf][w][r * NS + s][ld * C + c];
          e.b[r][c] = s_agg[buf][w][NS * NS + r][ld * C + c];
        }
      return e;
    };

    // the chunk carry: the update d^(k) at the row before the chunk
    float x[NS][C];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int c = 0; c < C; ++c) x[s][c] = 0.0f;
    if (pred && dv) {
      bool ok = true;
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int c = 0; c < C; ++c) ok = ok && desc_ok(early[s][c], tag);
      if (ok) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int c = 0; c < C; ++c) x[s][c] = desc_val(early[s][c]);
      } else if constexpr (INCL) {
        wait_incl<NS, C>(incl, BD, chan, LD, chunk - 1, tag, x);
      } else {
        if (wave == W - 1 && ll == 0 && chunk < p.nchunks - 1) {
          Aff<NS, C> tot = wave_agg(0);
#pragma unroll
          for (int w = 1; w < W; ++w) {
            Aff<NS, C> e = wave_agg(w);
            e.after(tot);
            tot = e;
          }
          publish_agg<NS, C>(agg, BD, chan, LD, chunk, tag, tot);
        }
        lookback<NS, C>(incl, agg, BD, chan, LD, chunk, -1, p.nchunks, tag, x);
      }
    }
    // through the preceding waves of the chunk
#pragma unroll
    for (int w = 0; w < W - 1; ++w)
      if (w < wave) wave_agg(w).apply(x);
    if (wave == W - 1 && ll == 0 && dv && chunk < p.nchunks - 1) {
      float xi[NS][C];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int c = 0; c < C; ++c) xi[s][c] = x[s][c];
      wave_agg(W - 1).apply(xi);
      publish_incl<NS, C>(incl, BD, chan, LD, chunk, tag, xi);
    }
    if constexpr (LL > 1) excl.apply(x);
    // the next linearisation point at the row before the lane group
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int c = 0; c < C; ++c) sp[s][c] += x[s][c];

    float mx = 0.0f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float y[NS][C];  // the update d at the step: J d_prev + r
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float xs[NS], rr[NS];
#pragma unroll
        for (int r = 0; r < NS; ++r) {
          xs[r] = x[r][c];
          rr[r] = rt[t][r][c];
        }
        Cell::apply(Jt[t][c], rr, xs);
#pragma unroll
        for (int r = 0; r < NS; ++r) y[r][c] = xs[r];
      }
      const bool valid = FULL || (dv && l0 + t < p.L);
#pragma unroll
      for (int r = 0; r < NS; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) {
          x[r][c] = y[r][c];
          so[t][r][c] = ZERO ? y[r][c] : so[t][r][c] + y[r][c];
          if (valid) mx = __builtin_elementwise_maximum(mx, fabsf(y[r][c]));
        }
    }
    const uint32_t m = wave_max_bits(__float_as_uint(mx));
    if (lane == 0) pmax[(k - 1) * pmax_k] = m;
  };

  iterate(1, std::true_type{});
  for (int k = 2; k <= p.K; ++k) iterate(k, std::false_type{});

#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int s = 0; s < NS; ++s) buf_st_f32<C>(rout[s], vs0 + t * sstep, 0u, so[t][s]);  // dropped past L or D
  };

  const bool full = (chunk + 1) * CL <= p.L && dt0 + CW <= p.D;
  if (full) tile_body(std::true_type{});
  else tile_body(std::false_type{});
}

}  // namespace pararnn
