// newton_iter.h -- one fused launch per Newton iteration of the ParaRNN solve.
//
// Iteration k (ParaRNN article, cafecomtech.com, section "A sacada: metodo de
// Newton"): linearise the whole-sequence system S_l = f(S_{l-1}, u_l) at the
// previous iterate S^(k-1) and solve the resulting linear SSM by a scan
// (section "O compromisso que SSMs fizeram": an associative combine turns the
// O(L) chain into a tree). The kernel works in the equivalent update form:
// with J_l = df/ds(S^(k-1)_{l-1}, u_l) and the residual
// r_l = f(S^(k-1)_{l-1}, u_l) - S^(k-1)_l, the update d_l = S^(k)_l - S^(k-1)_l
// obeys d_l = J_l d_{l-1} + r_l with d_{-1} = 0 (the initial state is fixed),
// and S^(k)_l = S^(k-1)_l + d_l. max |d| is the Newton update size.
//
// Work decomposition (all inside one launch):
//   lane      C consecutive channels x T consecutive timesteps (serial scan);
//   wave      64/LL lanes along D x LL lane groups along L (shuffle scan);
//   workgroup W waves along L (scan of wave totals through LDS);
//   grid      chunks of CL = W*LL*T timesteps per channel tile, chained by a
//             decoupled look-back over tagged descriptors. Workgroups take
//             their (chunk, tile) from an atomic ticket in chunk-major order,
//             so every predecessor a workgroup waits for has already started.
// The per-step (J, r) pairs never leave registers; HBM traffic per element is
// the gate inputs, the previous iterate and the new iterate.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace pararnn {

struct IterArgs {
  const void* u;          // [B][L][G][D] fp32 or bf16
  const float* a;         // [G][D]
  const float* s0[2];     // initial state per component, [B][D]; nullptr = 0
  const float* sin[2];    // iterate k-1 per component, [B][L][D]; nullptr when k == 1
  float* sout[2];         // iterate k per component
  unsigned long long* incl;  // [nchunks][NS][B*D] inclusive carries (value at chunk end)
  unsigned long long* agg;   // [nchunks][NS*NS+NS][B*D] chunk transforms
  unsigned int* ctr;      // [0,K) tickets
  unsigned int* maxupd;   // [K][B] fp32 bits of max |update| (reduced from pmax)
  unsigned int* pmax;     // [K][B][nchunks][ntiles_d] per-workgroup max |update| bits
  int B, L, D, k, K, nchunks, ntiles_d, early_exit;
  float tol;
};

// Descriptor layout: component q of chunk i for channel slot x lives at
// [(i * ncomp + q) * BD + x], where the slot of a lane's channel c is
// chan + c * cs (chan = tile * CW + lane index along D, cs = lanes along D), so
// one store or load instruction covers consecutive words across the wave.
//
// Looks back over predecessor chunks (chunk + dir, chunk + 2 dir, ...) until an
// inclusive carry is found, composing chunk transforms on the way. Returns the
// carry entering `chunk` (zero before the first chunk in scan order).
template <int NS, int C>
__device__ __forceinline__ void lookback(unsigned long long* incl, unsigned long long* agg,
                                         long long BD, long long chan, int cs, int chunk, int dir,
                                         int nchunks, uint32_t tag, float (&carry)[NS][C]) {
  constexpr int NA = NS * NS + NS;
  Aff<NS, C> M;
  M.set_identity();
  int i = chunk + dir;
  while (true) {
    if (i < 0 || i >= nchunks) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int c = 0; c < C; ++c) carry[s][c] = M.b[s][c];
      return;
    }
    unsigned long long wi[NS][C], wa[NA][C];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int c = 0; c < C; ++c) wi[s][c] = desc_get(incl + ((long long)i * NS + s) * BD + chan + c * cs);
#pragma unroll
    for (int q = 0; q < NA; ++q)
#pragma unroll
      for (int c = 0; c < C; ++c) wa[q][c] = desc_get(agg + ((long long)i * NA + q) * BD + chan + c * cs);
    // both reads complete here, also where only the first is used: a read
    // left in flight past the return makes the compiler wait for every
    // memory operation (stores included) at the caller's next use of its
    // registers
#pragma unroll
    for (int q = 0; q < NA; ++q)
#pragma unroll
      for (int c = 0; c < C; ++c) __asm__ volatile("" ::"v"(wa[q][c]));
    bool ok_i = true, ok_a = true;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int c = 0; c < C; ++c) ok_i = ok_i && desc_ok(wi[s][c], tag);
    if (ok_i) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int c = 0; c < C; ++c) carry[s][c] = desc_val(wi[s][c]);
      M.apply(carry);
      return;
    }
#pragma unroll
    for (int q = 0; q < NA; ++q)
#pragma unroll
      for (int c = 0; c < C; ++c) ok_a = ok_a && desc_ok(wa[q][c], tag);
    if (ok_a) {
      Aff<NS, C> e;
#pragma unroll
      for (int r = 0; r < NS; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) {
#pragma unroll
          for (int s = 0; s < NS; ++s) e.A[r][s][c] = desc_val(wa[r * NS + s][c]);
          e.b[r][c] = desc_val(wa[NS * NS + r][c]);
        }
      M.after(e);
      i += dir;
    } else {
      __builtin_amdgcn_s_sleep(1);
    }
  }
}

// Waits for chunk i's inclusive carry itself (no composition of aggregates)
// and returns it. Every word read is tested, so none is left in flight.
template <int NS, int C>
__device__ __forceinline__ void wait_incl(unsigned long long* incl, long long BD, long long chan, int cs, int i,
                                          uint32_t tag, float (&carry)[NS][C]) {
  while (true) {
    unsigned long long wi[NS][C];
    bool ok = true;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        wi[s][c] = desc_get(incl + ((long long)i * NS + s) * BD + chan + c * cs);
        ok = ok & desc_ok(wi[s][c], tag);
      }
    if (ok) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int c = 0; c < C; ++c) carry[s][c] = desc_val(wi[s][c]);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

template <int NS, int C>
__device__ __forceinline__ void publish_agg(unsigned long long* agg, long long BD, long long chan, int cs,
                                            int chunk, uint32_t tag, const Aff<NS, C>& e) {
  constexpr int NA = NS * NS + NS;
#pragma unroll
  for (int r = 0; r < NS; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
        desc_put(agg + ((long long)chunk * NA + r * NS + s) * BD + chan + c * cs, tag, e.A[r][s][c]);
      desc_put(agg + ((long long)chunk * NA + NS * NS + r) * BD + chan + c * cs, tag, e.b[r][c]);
    }
}

template <int NS, int C>
__device__ __forceinline__ void publish_incl(unsigned long long* incl, long long BD, long long chan, int cs,
                                             int chunk, uint32_t tag, const float (&x)[NS][C]) {
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int c = 0; c < C; ++c) desc_put(incl + ((long long)chunk * NS + s) * BD + chan + c * cs, tag, x[s][c]);
}

// FIRST: the launch of iteration 1, whose previous iterate is zero at every
// step (no state input); only the initial state s0 enters, at l = 0.
// INCL: the chunk carry is the predecessor's inclusive carry, waited for (no
// aggregates published or composed); chosen by the host where a chunk row
// has many tiles, so that predecessors run well ahead.
template <class Cell, class UT, int C, int T, int W, int LL, int OCC, bool FIRST, bool INCL>
__global__ void __launch_bounds__(64 * W, OCC) newton_iter_kernel(const IterArgs p) {
  constexpr int NS = Cell::NS, G = Cell::G;
  constexpr int LD = 64 / LL;   // lanes along D
  constexpr int CW = LD * C;    // channels per workgroup
  constexpr int CL = W * LL * T;
  constexpr int NA = NS * NS + NS;

  __shared__ float s_agg[W][NA][CW];
  __shared__ float s_carry[NS][CW];
  __shared__ unsigned int s_ticket;
  __shared__ uint32_t s_wmax[W];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ld = lane % LD, ll = lane / LD;
  const uint32_t tag = static_cast<uint32_t>(p.k);

  if (tid == 0) s_ticket = atomicAdd(p.ctr + (p.k - 1), 1u);
  __syncthreads();
  bool skip = false;
  if (!FIRST && p.early_exit && p.k > 1) {
    // early exit: once every row's update of the previous launch is within tol
    // (skipped launches leave their row maxima at 0), this launch only carries
    // the iterate forward. The previous launch finished before this one began.
    int ok = 1;
    for (int bb = tid; bb < p.B; bb += blockDim.x)
      ok &= (__uint_as_float(p.maxupd[static_cast<long long>(p.k - 2) * p.B + bb]) <= p.tol) ? 1 : 0;
    skip = __syncthreads_and(ok) != 0;
  }
  const unsigned int ticket = s_ticket;
  const unsigned int ntiles = static_cast<unsigned int>(p.B) * p.ntiles_d;
  const int chunk = static_cast<int>(ticket / ntiles);
  const int tile = static_cast<int>(ticket - static_cast<unsigned int>(chunk) * ntiles);
  const int b = tile / p.ntiles_d;
  const int d0 = (tile - b * p.ntiles_d) * CW + ld * C;
  const bool dv = d0 < p.D;  // C divides D: all C channels valid or none
  const int l0 = chunk * CL + (wave * LL + ll) * T;
  const long long BD = static_cast<long long>(p.B) * p.ntiles_d * CW;  // descriptor slots per component
  const long long chan = static_cast<long long>(tile) * CW + ld;
  // Addressing: one buffer resource per tensor covering this chunk's rows of
  // batch row b (scalar registers, extent = the chunk's rows below L), a
  // 32-bit lane offset that advances one row per step, and the gate offset as
  // the uniform offset. Rows at or past L read 0 and drop stores; lanes past D
  // get an offset beyond every extent. Steps past L follow every valid step of
  // their channel in scan order, so their (J, r) never reach a stored value.
  const int dt0 = (tile - b * p.ntiles_d) * CW;
  const int lt0 = (wave * LL + ll) * T;  // lane's first timestep within the chunk
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
  __amdgpu_buffer_rsrc_t rin[NS], rout[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    rin[s] = make_rsrc(p.sin[s] ? p.sin[s] + wrow * p.D : nullptr, p.sin[s] ? rows * sstep : 0u);
    rout[s] = make_rsrc(p.sout[s] + wrow * p.D, rows * sstep);
  }

  if (skip) {
    // early exit fired earlier: keep the converged iterate, moved to this launch's output
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float v[C];
        buf_ld_f32<C>(rin[s], vs0 + t * sstep, 0u, v);
        buf_st_f32<C>(rout[s], vs0 + t * sstep, 0u, v);
      }
    }
    return;
  }

  // The tile body, instantiated for full tiles (every step and channel valid,
  // so no step needs masking out of the update size) and partial ones.
  uint32_t mbits = 0u;
  auto tile_body = [&](auto full_tag) {
  constexpr bool FULL = decltype(full_tag)::value;
  // ---- a1: stream gate inputs and the previous iterate -------------------
  const int dc = dv ? d0 : p.D - C;  // channel group for the per-channel loads
  float av[G][C];
#pragma unroll
  for (int g = 0; g < G; ++g) ld_f32<C>(p.a + static_cast<long long>(g) * p.D + dc, av[g]);
  float sp[NS][C];  // iterate k-1 at l0 - 1 (the initial state at l0 == 0)
  const int lastrow = p.L - 1 - chunk * CL;  // >= 0: the chunk holds a valid row
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float v0[C], v1[C];
#pragma unroll
    for (int c = 0; c < C; ++c) v0[c] = v1[c] = 0.0f;
    if (p.s0[s]) ld_f32<C>(p.s0[s] + static_cast<long long>(b) * p.D + dc, v0);
    if (!FIRST && p.sin[s]) {
      const long long prow = wrow + min(max(lt0 - 1, -chunk * CL), lastrow);  // a row of batch b
      ld_f32<C>(p.sin[s] + prow * p.D + dc, v1);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) sp[s][c] = (l0 == 0) ? v0[c] : v1[c];
  }
  float so[T][NS][C];
  URaw<UT, C> uu[T][G];
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (!FIRST && p.sin[s]) buf_ld_f32<C>(rin[s], vs0 + t * sstep, 0u, so[t][s]);
      else
#pragma unroll
        for (int c = 0; c < C; ++c) so[t][s][c] = 0.0f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) uu[t][g].load(ru, vu0 + t * ustep, static_cast<uint32_t>(g) * gstep);
  }

  // ---- a2 + a3: residual and Jacobian per step; serial scan of the lane's T steps
  typename Cell::Jac Jt[T][C];
  float rt[T][NS][C];
  Aff<NS, C> acc;  // the lane's transform over its steps, from its first step
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float ac[G], uc[G], pc[NS], f[NS], sc[NS], rr[NS];
      typename Cell::Jac J;
#pragma unroll
      for (int g = 0; g < G; ++g) { ac[g] = av[g][c]; uc[g] = uu[t][g].get(c); }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        pc[s] = (t == 0) ? sp[s][c] : so[t - 1][s][c];
        sc[s] = so[t][s][c];
      }
      // Iteration 1 linearises at the zero iterate: from the third step of a
      // lane on the cell is evaluated in its reduced form at the zero state.
      // The general form on the first two steps (the second of the sequence's
      // first lane is the first at the zero state, its first reads s0) makes
      // a non-finite coefficient poison the lane as in the general form
      // (inf * 0 = NaN enters r_t, and the scan carries it to every later step).
      if (FIRST && t > 1) Cell::step_zero(ac, uc, f, J);
      else Cell::step(ac, uc, pc, f, J);
      Cell::template residual<FIRST>(f, sc, J, rr);
      Jt[t][c] = J;
#pragma unroll
      for (int r = 0; r < NS; ++r) rt[t][r][c] = rr[r];
      if (t == 0) Cell::first(acc, c, J, rr);
      else Cell::pre(acc, c, J, rr);
    }
  }

  // ---- a4: scan across the LL lane groups of the wave (shuffles) -----------
  Aff<NS, C> excl;  // transform of the wave's earlier lane groups
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

  // ---- a4 + a5: workgroup total, look-back for the chunk's carry -----------
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

  // ---- apply the carry, write the new iterate (a6) -----------------------
  float x[NS][C];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int c = 0; c < C; ++c) x[s][c] = s_carry[s][ld * C + c];
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
    e.apply(x);
  }
  if constexpr (LL > 1) excl.apply(x);

  // max |update| over the lane's valid steps; the NaN-propagating maximum keeps
  // a NaN anywhere in the row visible
  float mx = 0.0f;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int l = l0 + t;
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
      for (int r = 0; r < NS; ++r) x[r][c] = xs[r];
    }
    const bool valid = FULL || (dv && l < p.L);
#pragma unroll
    for (int r = 0; r < NS; ++r) {
      float o[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        o[c] = FIRST ? x[r][c] : so[t][r][c] + x[r][c];
        if (valid) mx = __builtin_elementwise_maximum(mx, fabsf(x[r][c]));
      }
      buf_st_f32<C>(rout[r], vs0 + t * sstep, 0u, o);  // dropped past L or D
    }
  }
  // row max of |update|: wave reduction (NaN-propagating)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, off, 64));
  mbits = __float_as_uint(mx);
  };
  const bool full = (chunk + 1) * CL <= p.L && dt0 + CW <= p.D;
  if (full) tile_body(std::true_type{});
  else tile_body(std::false_type{});

  // workgroup max, one plain store per workgroup (same-address atomics from
  // every wave would serialise at the device coherence point)
  if (lane == 0) s_wmax[wave] = mbits;
  __syncthreads();
  if (tid == 0) {
    uint32_t m = s_wmax[0];
#pragma unroll
    for (int w = 1; w < W; ++w) m = max(m, s_wmax[w]);
    // partials of one row are contiguous: [k][b][chunk][channel tile]
    p.pmax[((static_cast<long long>(p.k - 1) * p.B + b) * p.nchunks + chunk) * p.ntiles_d + (dt0 / CW)] = m;
  }
}

constexpr int kRowmaxThreads = 1024;  // block size of the row-max reductions

// Row max of the per-workgroup partials of iteration k for batch row b (whole
// block participates; result valid in every thread). A row's partials are
// contiguous: n = nchunks * ntiles_d values.
__device__ __forceinline__ uint32_t block_rowmax(const unsigned int* pmax, int B, int ntiles_d, int nchunks,
                                                 int k, int b, uint32_t* s_red) {
  const long long n = static_cast<long long>(nchunks) * ntiles_d;
  const unsigned int* row = pmax + (static_cast<long long>(k) * B + b) * n;
  // few blocks (one per row and iteration) read many partials: keep eight
  // independent loads in flight per thread
  constexpr int U = 8;
  uint32_t m = 0u;
  long long i = threadIdx.x;
  for (; i + (U - 1) * static_cast<long long>(blockDim.x) < n; i += U * static_cast<long long>(blockDim.x)) {
    uint32_t v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = row[i + j * static_cast<long long>(blockDim.x)];
#pragma unroll
    for (int j = 0; j < U; ++j) m = max(m, v[j]);
  }
  for (; i < n; i += blockDim.x) m = max(m, row[i]);
  s_red[threadIdx.x] = m;
  __syncthreads();
  for (int off = blockDim.x / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) s_red[threadIdx.x] = max(s_red[threadIdx.x], s_red[threadIdx.x + off]);
    __syncthreads();
  }
  const uint32_t r = s_red[0];
  __syncthreads();
  return r;
}

// Early-exit mode only: row maxima of iteration k, read by the next launch.
__global__ void __launch_bounds__(kRowmaxThreads) rowmax_kernel(const unsigned int* pmax, unsigned int* maxupd, int B,
                                                     int ntiles_d, int nchunks, int k) {
  __shared__ uint32_t s_red[kRowmaxThreads];
  const uint32_t m = block_rowmax(pmax, B, ntiles_d, nchunks, k, blockIdx.x, s_red);
  if (threadIdx.x == 0) maxupd[static_cast<long long>(k) * B + blockIdx.x] = m;
}

// After the last iteration, block (b, k) per batch row and iteration: the
// row maximum of iteration k (unless early exit already reduced it), copied
// out as a float; the last iteration's blocks also write the row's
// convergence flag, and block (0, K-1) the iteration count.
__global__ void __launch_bounds__(kRowmaxThreads) newton_finalize_kernel(const unsigned int* pmax, unsigned int* maxupd,
                                                              int B, int ntiles_d, int nchunks, int K, float tol,
                                                              int early_exit, int32_t* iters_out,
                                                              int32_t* conv_out, float* maxupd_out) {
  __shared__ uint32_t s_red[kRowmaxThreads];
  const int b = blockIdx.x, k = blockIdx.y, tid = threadIdx.x;
  uint32_t m;
  if (!early_exit) {
    m = block_rowmax(pmax, B, ntiles_d, nchunks, k, b, s_red);
    if (tid == 0) maxupd[static_cast<long long>(k) * B + b] = m;
  } else {
    m = maxupd[static_cast<long long>(k) * B + b];
  }
  if (tid == 0 && maxupd_out) maxupd_out[static_cast<long long>(k) * B + b] = __uint_as_float(m);
  if (k != K - 1) return;
  int iters = K;
  if (early_exit) {  // maxupd is complete: reduced after every launch
    for (int kk = 1; kk <= K; ++kk) {
      int ok = 1;
      for (int bb = tid; bb < B; bb += blockDim.x)
        ok &= (__uint_as_float(maxupd[static_cast<long long>(kk - 1) * B + bb]) <= tol) ? 1 : 0;
      if (__syncthreads_and(ok)) {
        iters = kk;
        break;
      }
    }
  }
  if (tid == 0) {
    const uint32_t mi = (iters == K) ? m : maxupd[static_cast<long long>(iters - 1) * B + b];
    if (conv_out) conv_out[b] = (__uint_as_float(mi) <= tol) ? 1 : 0;
    if (iters_out && b == 0) *iters_out = iters;
  }
}

// Clears the zero-initialised part of the workspace (counters, row maxima,
// descriptor tags) and the caller's max_update array, with vector stores.
__global__ void __launch_bounds__(256) ws_clear_kernel(f32x4* ws, long long n16, float* user,
                                                       long long nuser) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    ws[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (user)
    for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < nuser; i += stride)
      user[i] = 0.0f;
}

}  // namespace pararnn
