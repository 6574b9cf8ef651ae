// adjoint.h -- reverse linear scan for the gradient of a loss through the
// solved recurrence (one launch), plus the deterministic reduction of the
// coefficient gradient.
//
// Along a trajectory S (the solve's output) with upstream gradient dh:
//   lambda_{L-1} = G_{L-1},  lambda_l = J_{l+1}^T lambda_{l+1} + G_l,
//   J_{l+1} = df/ds(S_l, u_{l+1}),  G_l = dh_l on the h component,
//   du_l = (df/du(S_{l-1}, u_l))^T lambda_l,  ds0 = J_0^T lambda_0,
//   da_g = sum_{b,l} m_g(S_{l-1}) du_{l,g}   (m_g: multiplier of a_g in gate g).
// The recurrence for lambda is again a linear SSM (with the transposed
// Jacobians, run from the end of the sequence), so it uses the same scan
// hierarchy as the Newton iteration with the direction reversed: lanes,
// waves and chunks are ordered from the end of L, and the look-back walks to
// larger chunk indices. The ParaRNN pages state that training runs in
// parallel (cafecomtech.com article, opening; aifeed.sk article); the adjoint
// is the standard reverse-mode form of the recurrence.
#pragma once

#include "newton_iter.h"

namespace pararnn {

struct AdjArgs {
  const void* u;        // [B][L][G][D]
  const float* a;       // [G][D]
  const float* s0[2];   // [B][D] per component, nullptr = 0
  const float* S[2];    // trajectory per component [B][L][D]
  const float* dh;      // [B][L][D]
  float* du;            // [B][L][G][D]
  float* ds0;           // [NS][B][D] or nullptr
  float* da_part;       // [nchunks][B][G][D] partial sums, or nullptr
  unsigned long long* incl;
  unsigned long long* agg;
  unsigned int* ctr;    // [0] ticket
  int B, L, D, nchunks, ntiles_d;
};

template <class Cell, class UT, int C, int T, int W, int LL, int OCC>
__global__ void __launch_bounds__(64 * W, OCC) adjoint_kernel(const AdjArgs p) {
  constexpr int NS = Cell::NS, G = Cell::G;
  constexpr int LD = 64 / LL, CW = LD * C, CL = W * LL * T, NA = NS * NS + NS, NSEG = W * LL;
  constexpr uint32_t tag = 1u;

  __shared__ float s_agg[W][NA][CW];
  __shared__ float s_carry[NS][CW];
  __shared__ float s_da[G][CW];
  __shared__ unsigned int s_ticket;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ld = lane % LD, ll = lane / LD;
  if (tid == 0) s_ticket = atomicAdd(p.ctr, 1u);
  if (p.da_part)
    for (int i = tid; i < G * CW; i += blockDim.x) (&s_da[0][0])[i] = 0.0f;
  __syncthreads();
  const unsigned int ticket = s_ticket;
  const unsigned int ntiles = static_cast<unsigned int>(p.B) * p.ntiles_d;
  const int rchunk = static_cast<int>(ticket / ntiles);
  const int chunk = p.nchunks - 1 - rchunk;  // chunks are taken from the end of L
  const int tile = static_cast<int>(ticket - static_cast<unsigned int>(rchunk) * ntiles);
  const int b = tile / p.ntiles_d;
  const int d0 = (tile - b * p.ntiles_d) * CW + ld * C;
  const bool dv = d0 < p.D;
  const int q = wave * LL + ll;          // position in scan order (from the end)
  const int l0 = chunk * CL + (NSEG - 1 - q) * T;
  const long long BD = static_cast<long long>(p.B) * p.ntiles_d * CW;  // descriptor slots per component
  const long long chan = static_cast<long long>(tile) * CW + ld;
  const long long row0 = static_cast<long long>(b) * p.L;
  const UT* __restrict__ u = static_cast<const UT*>(p.u);

  float av[G][C];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (dv) ld_f32<C>(p.a + static_cast<long long>(g) * p.D + d0, av[g]);
    else
#pragma unroll
      for (int c = 0; c < C; ++c) av[g][c] = 0.0f;
  }
  // states S_{m-1} and inputs u_m for m = l0 .. l0 + T
  float sv[T + 1][NS][C];
  URaw<UT, C> uu[T + 1][G];
  float gv[T][C];
#pragma unroll
  for (int t = 0; t <= T; ++t) {
    const int m = l0 + t;
    const bool v = dv && m < p.L;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int c = 0; c < C; ++c) sv[t][s][c] = 0.0f;
      if (v) {
        if (m == 0) {
          if (p.s0[s]) ld_f32<C>(p.s0[s] + static_cast<long long>(b) * p.D + d0, sv[t][s]);
        } else {
          ld_f32<C>(p.S[s] + (row0 + m - 1) * p.D + d0, sv[t][s]);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (v) uu[t][g].load(u + ((row0 + m) * G + g) * p.D + d0);
      else uu[t][g].zero();
    }
    if (t < T) {
      if (v) ld_f32<C>(p.dh + (row0 + m) * p.D + d0, gv[t]);
      else
#pragma unroll
        for (int c = 0; c < C; ++c) gv[t][c] = 0.0f;
    }
  }

  // cell evaluations at m = l0 + t: J_m for t = 0..T, dfdu_m and m_g for t < T
  float Jm[T + 1][NS][NS][C];
  float dfdu[T][NS][G][C];
  float mult[T][G][C];
#pragma unroll
  for (int t = 0; t <= T; ++t) {
    const bool v = dv && (l0 + t) < p.L;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float ac[G], uc[G], sc[NS], J[NS][NS], du_[NS][G], mm[G];
#pragma unroll
      for (int g = 0; g < G; ++g) { ac[g] = av[g][c]; uc[g] = uu[t][g].get(c); }
#pragma unroll
      for (int s = 0; s < NS; ++s) sc[s] = sv[t][s][c];
      Cell::step_adj(ac, uc, sc, J, du_, mm);
#pragma unroll
      for (int r = 0; r < NS; ++r)
#pragma unroll
        for (int s = 0; s < NS; ++s) Jm[t][r][s][c] = v ? J[r][s] : (r == s ? 1.0f : 0.0f);
      if (t < T) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
          for (int r = 0; r < NS; ++r) dfdu[t][r][g][c] = du_[r][g];
          mult[t][g][c] = mm[g];
        }
      }
    }
  }

  // serial reverse scan over the lane's steps: lambda_l = J_{l+1}^T lambda_{l+1} + G_l
  Aff<NS, C> acc;
  acc.set_identity();
#pragma unroll
  for (int t = T - 1; t >= 0; --t) {
    Aff<NS, C> e;
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) {
#pragma unroll
        for (int s = 0; s < NS; ++s) e.A[r][s][c] = Jm[t + 1][s][r][c];  // transpose
        e.b[r][c] = (r == NS - 1) ? gv[t][c] : 0.0f;
      }
    e.after(acc);
    acc = e;
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
        for (int s = 0; s < NS; ++s) s_agg[wave][r * NS + s][ld * C + c] = acc.A[r][s][c];
        s_agg[wave][NS * NS + r][ld * C + c] = acc.b[r][c];
      }
  }
  __syncthreads();

  if (wave == 0 && ll == 0) {
    float carry[NS][C];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int c = 0; c < C; ++c) carry[s][c] = 0.0f;
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
            for (int s = 0; s < NS; ++s) e.A[r][s][c] = s_agg[w][r * NS + s][ld * C + c];
            e.b[r][c] = s_agg[w][NS * NS + r][ld * C + c];
          }
        e.after(tot);
        tot = e;
      }
      if (chunk < p.nchunks - 1) {
        if (chunk > 0) publish_agg<NS, C>(p.agg, BD, chan, LD, chunk, tag, tot);
        lookback<NS, C>(p.incl, p.agg, BD, chan, LD, chunk, +1, p.nchunks, tag, carry);
      }
      if (chunk > 0) {
        float x[NS][C];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int c = 0; c < C; ++c) x[s][c] = carry[s][c];
        tot.apply(x);
        publish_incl<NS, C>(p.incl, BD, chan, LD, chunk, tag, x);
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int c = 0; c < C; ++c) s_carry[s][ld * C + c] = carry[s][c];
  }
  __syncthreads();

  float lam[NS][C];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int c = 0; c < C; ++c) lam[s][c] = s_carry[s][ld * C + c];
  for (int w = 0; w < wave; ++w) {
    Aff<NS, C> e;
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) {
#pragma unroll
        for (int s = 0; s < NS; ++s) e.A[r][s][c] = s_agg[w][r * NS + s][ld * C + c];
        e.b[r][c] = s_agg[w][NS * NS + r][ld * C + c];
      }
    e.apply(lam);
  }
  if constexpr (LL > 1) excl.apply(lam);

  float dacc[G][C];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < C; ++c) dacc[g][c] = 0.0f;
#pragma unroll
  for (int t = T - 1; t >= 0; --t) {
    const int l = l0 + t;
    float y[NS][C];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        float a2 = (r == NS - 1) ? gv[t][c] : 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s) a2 = fmaf(Jm[t + 1][s][r][c], lam[s][c], a2);
        y[r][c] = a2;
      }
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) lam[r][c] = y[r][c];
    if (dv && l < p.L) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float o[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
          float a2 = 0.0f;
#pragma unroll
          for (int r = 0; r < NS; ++r) a2 = fmaf(dfdu[t][r][g][c], lam[r][c], a2);
          o[c] = a2;
          dacc[g][c] = fmaf(mult[t][g][c], a2, dacc[g][c]);
        }
        st_f32<C>(p.du + ((row0 + l) * G + g) * p.D + d0, o);
      }
      if (l == 0 && p.ds0) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          float o[C];
#pragma unroll
          for (int c = 0; c < C; ++c) {
            float a2 = 0.0f;
#pragma unroll
            for (int r = 0; r < NS; ++r) a2 = fmaf(Jm[0][r][s][c], lam[r][c], a2);
            o[c] = a2;
          }
          st_f32<C>(p.ds0 + (static_cast<long long>(s) * p.B + b) * p.D + d0, o);
        }
      }
    }
  }

  if (p.da_part) {
    // per-workgroup partial of da, summed in a fixed order: lane groups via
    // LDS atomics would reorder, so each (wave, lane group) adds in turn
    for (int k = 0; k < NSEG; ++k) {
      if (q == k) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int c = 0; c < C; ++c) s_da[g][ld * C + c] += dacc[g][c];
      }
      __syncthreads();
    }
    if (wave == 0 && ll == 0 && dv) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float o[C];
#pragma unroll
        for (int c = 0; c < C; ++c) o[c] = s_da[g][ld * C + c];
        st_f32<C>(p.da_part + ((static_cast<long long>(chunk) * p.B + b) * G + g) * p.D + d0, o);
      }
    }
  }
}

// da[g][d] = sum over chunks and rows of the partials, in a fixed order.
__global__ void __launch_bounds__(256) da_reduce_kernel(const float* part, float* da, int nchunks,
                                                        int B, int G, int D) {
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<long long>(G) * D) return;
  const int g = static_cast<int>(i / D), d = static_cast<int>(i - static_cast<long long>(g) * D);
  float acc = 0.0f;
  for (int k = 0; k < nchunks; ++k)
    for (int b = 0; b < B; ++b) acc += part[((static_cast<long long>(k) * B + b) * G + g) * D + d];
  da[i] = acc;
}

}  // namespace pararnn
