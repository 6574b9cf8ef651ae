// adjoint.h -- reverse linear scan for the gradient of a loss through the
// solved recurrence (one launch), plus the deterministic reduction of the
// coefficient gradient.
//
// Along a trajectory S (the solve's output) with upstream gradient dh:
//   lambda_{L-1} = G_{L-1},  lambda_l = J_{l+1}^T lambda_{l+1} + G_l,
//   J_{l+1} = df/ds(S_l, u_{l+1}),  G_l = dh_l on the h component,
//   du_l = (df/du(S_{l-1}, u_l))^T lambda_l,  ds0 = J_0^T lambda_0,
//   da_g = sum_{b,l} m_g(S_{l-1}) du_{l,g}   (m_g: multiplier of a_g in gate g).
// The scan runs on mu_l = J_l^T lambda_l, the gradient that step l passes
// back to S_{l-1}:
//   mu_L = 0,  lambda_l = mu_{l+1} + G_l,  mu_l = J_l^T lambda_l,  ds0 = mu_0,
// a linear SSM again (with the transposed Jacobians, run from the end of the
// sequence) in which step l needs only its own Jacobian, at (S_{l-1}, u_l).
// A lane that owns steps l0 .. l0+T-1 so reads exactly the rows it owns of u
// and dh, and the rows l0-1 .. l0+T-2 of S: the lanes tile every array
// without overlap. It uses the same scan hierarchy as the Newton iteration
// with the direction reversed: lanes, waves and chunks are ordered from the
// end of L, and the look-back walks to larger chunk indices. The ParaRNN pages state that training runs in
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

// INCL: the chunk carry is the successor chunk's inclusive carry, waited for
// (no aggregates published or composed); chosen by the host where a chunk row
// has many tiles, so that the chunks ahead in scan order run well ahead.
template <class Cell, class UT, int C, int T, int W, int LL, int OCC, bool INCL>
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
  const int dt0 = (tile - b * p.ntiles_d) * CW;
  const int d0 = dt0 + ld * C;
  const bool dv = d0 < p.D;
  const int q = wave * LL + ll;          // position in scan order (from the end)
  const int lt0 = (NSEG - 1 - q) * T;    // lane's first step within the chunk
  const int l0 = chunk * CL + lt0;
  const long long BD = static_cast<long long>(p.B) * p.ntiles_d * CW;  // descriptor slots per component
  const long long chan = static_cast<long long>(tile) * CW + ld;
  // Addressing as in the Newton iteration: per-chunk buffer resources over
  // batch row b, 32-bit lane offsets, rows at or past L read 0 and drop
  // stores, lanes past D get an offset beyond every extent.
  const long long wrow = static_cast<long long>(b) * p.L + static_cast<long long>(chunk) * CL;
  const uint32_t ustep = static_cast<uint32_t>(G * p.D * sizeof(UT));
  const uint32_t gstep = static_cast<uint32_t>(p.D * sizeof(UT));
  const uint32_t sstep = static_cast<uint32_t>(p.D * sizeof(float));
  const uint32_t dstep = static_cast<uint32_t>(G * p.D * sizeof(float));
  const int crow = p.L - chunk * CL;  // rows from the chunk start to the end of L
  const uint32_t rows = static_cast<uint32_t>(min(crow, CL));
  constexpr uint32_t kOOB = 0x80000000u;  // extents stay below 2^31 bytes
  const uint32_t vu0 = dv ? static_cast<uint32_t>(lt0) * ustep + static_cast<uint32_t>(d0 * sizeof(UT)) : kOOB;
  const uint32_t vs0 = dv ? static_cast<uint32_t>(lt0) * sstep + static_cast<uint32_t>(d0 * sizeof(float)) : kOOB;
  const uint32_t vd0 = dv ? static_cast<uint32_t>(lt0) * dstep + static_cast<uint32_t>(d0 * sizeof(float)) : kOOB;
  const __amdgpu_buffer_rsrc_t ru =
      make_rsrc(reinterpret_cast<const char*>(p.u) + wrow * G * p.D * static_cast<long long>(sizeof(UT)), rows * ustep);
  __amdgpu_buffer_rsrc_t rS[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) rS[s] = make_rsrc(p.S[s] + wrow * p.D, rows * sstep);
  const __amdgpu_buffer_rsrc_t rdh = make_rsrc(p.dh + wrow * p.D, rows * sstep);
  const __amdgpu_buffer_rsrc_t rdu = make_rsrc(p.du + wrow * G * p.D, rows * dstep);

  float dacc[G][C];  // this lane's part of da
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < C; ++c) dacc[g][c] = 0.0f;

  // The tile body, instantiated for tiles whose steps all lie below L and
  // whose channels all lie below D, and for the others, which mask the steps
  // past L to identity transforms.
  auto tile_body = [&](auto full_tag) {
  constexpr bool FULL = decltype(full_tag)::value;
  const int dc = dv ? d0 : p.D - C;  // channel group for the per-channel loads
  float av[G][C];
#pragma unroll
  for (int g = 0; g < G; ++g) ld_f32<C>(p.a + static_cast<long long>(g) * p.D + dc, av[g]);
  // states S_{m-1}, inputs u_m and dh_m for m = l0 .. l0 + T - 1; S_{l0-1} is
  // the initial state at l0 == 0 and otherwise the row before the lane
  // (clamped into the sequence for lanes past L, whose steps are masked)
  float sv[T][NS][C];
  URaw<UT, C> uu[T][G];
  float gv[T][C];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float v0[C], v1[C];
#pragma unroll
    for (int c = 0; c < C; ++c) v0[c] = 0.0f;
    if (p.s0[s]) ld_f32<C>(p.s0[s] + static_cast<long long>(b) * p.D + dc, v0);
    const long long prow = static_cast<long long>(b) * p.L + min(max(l0 - 1, 0), p.L - 1);
    ld_f32<C>(p.S[s] + prow * p.D + dc, v1);
#pragma unroll
    for (int c = 0; c < C; ++c) sv[0][s][c] = (l0 == 0) ? v0[c] : v1[c];
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (t > 0) {
#pragma unroll
      for (int s = 0; s < NS; ++s) buf_ld_f32<C>(rS[s], vs0 + (t - 1) * sstep, 0u, sv[t][s]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) uu[t][g].load(ru, vu0 + t * ustep, static_cast<uint32_t>(g) * gstep);
    buf_ld_f32<C>(rdh, vs0 + t * sstep, 0u, gv[t]);
  }

  // cell evaluations at m = l0 + t: J_m and the input-gradient coefficients
  constexpr int NK = Cell::NK;
  float Jm[T][NS][NS][C];
  float kc[T][NK][C];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const bool v = FULL || (dv && (l0 + t) < p.L);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float ac[G], uc[G], sc[NS], J[NS][NS], kk[NK];
#pragma unroll
      for (int g = 0; g < G; ++g) { ac[g] = av[g][c]; uc[g] = uu[t][g].get(c); }
#pragma unroll
      for (int s = 0; s < NS; ++s) sc[s] = sv[t][s][c];
      Cell::step_adj(ac, uc, sc, J, kk);
#pragma unroll
      for (int r = 0; r < NS; ++r)
#pragma unroll
        for (int s = 0; s < NS; ++s) Jm[t][r][s][c] = v ? J[r][s] : (r == s ? 1.0f : 0.0f);
#pragma unroll
      for (int i = 0; i < NK; ++i) kc[t][i][c] = kk[i];
    }
  }

  // serial reverse scan over the lane's steps: mu_l = J_l^T (mu_{l+1} + G_l)
  // (masked steps: identity, and dh reads 0 past L)
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
        for (int s = 0; s < NS; ++s) e.A[r][s][c] = Jm[t][s][r][c];  // transpose
        e.b[r][c] = Jm[t][NS - 1][r][c] * gv[t][c];  // J^T G, G on the h component
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
        if constexpr (INCL) {
          wait_incl<NS, C>(p.incl, BD, chan, LD, chunk + 1, tag, carry);
        } else {
          if (chunk > 0) publish_agg<NS, C>(p.agg, BD, chan, LD, chunk, tag, tot);
          lookback<NS, C>(p.incl, p.agg, BD, chan, LD, chunk, +1, p.nchunks, tag, carry);
        }
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

  float mu[NS][C];  // mu at the row after the lane's last step
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int c = 0; c < C; ++c) mu[s][c] = s_carry[s][ld * C + c];
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
    e.apply(mu);
  }
  if constexpr (LL > 1) excl.apply(mu);

#pragma unroll
  for (int t = T - 1; t >= 0; --t) {
    const int l = l0 + t;
    float lam[NS][C];  // lambda_l = mu_{l+1} + G_l
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) lam[r][c] = (r == NS - 1) ? mu[r][c] + gv[t][c] : mu[r][c];
    const bool valid = FULL || (dv && l < p.L);
    float o[G][C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float kk[NK], sc[NS], lc[NS], du_[G], mm[G];
#pragma unroll
      for (int i = 0; i < NK; ++i) kk[i] = kc[t][i][c];
#pragma unroll
      for (int s = 0; s < NS; ++s) { sc[s] = sv[t][s][c]; lc[s] = lam[s][c]; }
      Cell::grad_u(kk, sc, lc, du_, mm);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        o[g][c] = du_[g];
        if (valid) dacc[g][c] = fmaf(mm[g], du_[g], dacc[g][c]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
      buf_st_f32<C, kBufNT>(rdu, vd0 + t * dstep, static_cast<uint32_t>(g) * sstep, o[g]);  // dropped past L or D
    // mu_l = J_l^T lambda_l
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float a2 = 0.0f;
#pragma unroll
        for (int r = 0; r < NS; ++r) a2 = fmaf(Jm[t][r][s][c], lam[r][c], a2);
        mu[s][c] = a2;
      }
    if (l == 0 && dv && p.ds0) {
#pragma unroll
      for (int s = 0; s < NS; ++s) st_f32<C>(p.ds0 + (static_cast<long long>(s) * p.B + b) * p.D + d0, mu[s]);
    }
  }
  };
  const bool full = (chunk + 1) * CL <= p.L && dt0 + CW <= p.D;
  if (full) tile_body(std::true_type{});
  else tile_body(std::false_type{});

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

// da[g][d] = sum of the per-workgroup partials over all chunks and batch rows,
// in a fixed order: the partials form rows of G*D columns; row group q of a
// column adds rows q, q + RG, q + 2 RG, ... in turn (eight loads in flight),
// then the RG group sums of the column are added in order of q.
constexpr int kDaCols = 64, kDaGroups = 16;
__global__ void __launch_bounds__(kDaCols * kDaGroups) da_reduce_kernel(const float* part, float* da, int rows,
                                                                        long long GD) {
  __shared__ float s_sum[kDaGroups][kDaCols];
  const int j = threadIdx.x % kDaCols, q = threadIdx.x / kDaCols;
  const long long col = static_cast<long long>(blockIdx.x) * kDaCols + j;
  float acc = 0.0f;
  if (col < GD) {
    constexpr int U = 8;
    int r = q;
    for (; r + (U - 1) * kDaGroups < rows; r += U * kDaGroups) {
      float v[U];
#pragma unroll
      for (int i = 0; i < U; ++i) v[i] = part[static_cast<long long>(r + i * kDaGroups) * GD + col];
#pragma unroll
      for (int i = 0; i < U; ++i) acc += v[i];
    }
    for (; r < rows; r += kDaGroups) acc += part[static_cast<long long>(r) * GD + col];
  }
  s_sum[q][j] = acc;
  __syncthreads();
  if (q == 0 && col < GD) {
    float t = 0.0f;
    for (int k = 0; k < kDaGroups; ++k) t += s_sum[k][j];
    da[col] = t;
  }
}

}  // namespace pararnn
