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
  unsigned int* ctr;      // [0,K) tickets, [K,2K) finished-workgroup counts, [2K] stop flag
  unsigned int* maxupd;   // [K][B] fp32 bits of max |update|
  int32_t* iters_out;     // [1] or nullptr
  int32_t* conv_out;      // [B] or nullptr
  float* maxupd_out;      // [K][B] or nullptr
  int B, L, D, k, K, nchunks, ntiles_d, early_exit;
  float tol;
};

// Looks back over predecessor chunks (chunk + dir, chunk + 2 dir, ...) until an
// inclusive carry is found, composing chunk transforms on the way. Returns the
// carry entering `chunk` (zero before the first chunk in scan order).
template <int NS, int C>
__device__ __forceinline__ void lookback(unsigned long long* incl, unsigned long long* agg,
                                         long long BD, long long chan, int chunk, int dir,
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
      for (int c = 0; c < C; ++c) wi[s][c] = desc_get(incl + ((long long)i * NS + s) * BD + chan + c);
#pragma unroll
    for (int q = 0; q < NA; ++q)
#pragma unroll
      for (int c = 0; c < C; ++c) wa[q][c] = desc_get(agg + ((long long)i * NA + q) * BD + chan + c);
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

template <int NS, int C>
__device__ __forceinline__ void publish_agg(unsigned long long* agg, long long BD, long long chan,
                                            int chunk, uint32_t tag, const Aff<NS, C>& e) {
  constexpr int NA = NS * NS + NS;
#pragma unroll
  for (int r = 0; r < NS; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
        desc_put(agg + ((long long)chunk * NA + r * NS + s) * BD + chan + c, tag, e.A[r][s][c]);
      desc_put(agg + ((long long)chunk * NA + NS * NS + r) * BD + chan + c, tag, e.b[r][c]);
    }
}

template <int NS, int C>
__device__ __forceinline__ void publish_incl(unsigned long long* incl, long long BD, long long chan,
                                             int chunk, uint32_t tag, const float (&x)[NS][C]) {
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int c = 0; c < C; ++c) desc_put(incl + ((long long)chunk * NS + s) * BD + chan + c, tag, x[s][c]);
}

template <class Cell, class UT, int C, int T, int W, int LL>
__global__ void __launch_bounds__(64 * W) newton_iter_kernel(const IterArgs p) {
  constexpr int NS = Cell::NS, G = Cell::G;
  constexpr int LD = 64 / LL;   // lanes along D
  constexpr int CW = LD * C;    // channels per workgroup
  constexpr int CL = W * LL * T;
  constexpr int NA = NS * NS + NS;

  __shared__ float s_agg[W][NA][CW];
  __shared__ float s_carry[NS][CW];
  __shared__ unsigned int s_ticket, s_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ld = lane % LD, ll = lane / LD;
  const uint32_t tag = static_cast<uint32_t>(p.k);

  if (tid == 0) {
    s_ticket = atomicAdd(p.ctr + (p.k - 1), 1u);
    // the stop flag was written by an earlier launch on the same stream
    s_flag = (p.early_exit && p.k > 1)
                 ? __hip_atomic_load(p.ctr + 2 * p.K, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                 : 0u;
  }
  __syncthreads();
  const unsigned int ticket = s_ticket;
  const unsigned int ntiles = static_cast<unsigned int>(p.B) * p.ntiles_d;
  const int chunk = static_cast<int>(ticket / ntiles);
  const int tile = static_cast<int>(ticket - static_cast<unsigned int>(chunk) * ntiles);
  const int b = tile / p.ntiles_d;
  const int d0 = (tile - b * p.ntiles_d) * CW + ld * C;
  const bool dv = d0 < p.D;  // C divides D: all C channels valid or none
  const int l0 = chunk * CL + (wave * LL + ll) * T;
  const long long BD = static_cast<long long>(p.B) * p.D;
  const long long chan = static_cast<long long>(b) * p.D + d0;
  const long long row0 = static_cast<long long>(b) * p.L;  // (b, l) -> (row0 + l) * D + d
  const UT* __restrict__ u = static_cast<const UT*>(p.u);

  if (s_flag) {
    // early exit fired earlier: keep the converged iterate, moved to this launch's output
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int l = l0 + t;
      if (dv && l < p.L) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          float v[C];
          ld_f32<C>(p.sin[s] + (row0 + l) * p.D + d0, v);
          st_f32<C>(p.sout[s] + (row0 + l) * p.D + d0, v);
        }
      }
    }
    return;
  }

  // ---- a1: stream gate inputs and the previous iterate -------------------
  float av[G][C];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (dv) ld_f32<C>(p.a + static_cast<long long>(g) * p.D + d0, av[g]);
    else
#pragma unroll
      for (int c = 0; c < C; ++c) av[g][c] = 0.0f;
  }
  float sp[NS][C];  // iterate k-1 at l0 - 1 (the initial state at l0 == 0)
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int c = 0; c < C; ++c) sp[s][c] = 0.0f;
    if (dv) {
      if (l0 == 0) {
        if (p.s0[s]) ld_f32<C>(p.s0[s] + static_cast<long long>(b) * p.D + d0, sp[s]);
      } else if (p.sin[s] && l0 <= p.L) {
        ld_f32<C>(p.sin[s] + (row0 + l0 - 1) * p.D + d0, sp[s]);
      }
    }
  }
  float so[T][NS][C];
  URaw<UT, C> uu[T][G];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int l = l0 + t;
    const bool v = dv && l < p.L;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (v && p.sin[s]) ld_f32<C>(p.sin[s] + (row0 + l) * p.D + d0, so[t][s]);
      else
#pragma unroll
        for (int c = 0; c < C; ++c) so[t][s][c] = 0.0f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (v) uu[t][g].load(u + ((row0 + l) * G + g) * p.D + d0);
      else uu[t][g].zero();
    }
  }

  // ---- a2 + a3: residual and Jacobian per step; serial scan of the lane's T steps
  float Jt[T][NS][NS][C], rt[T][NS][C];
  Aff<NS, C> acc;
  acc.set_identity();
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const bool v = dv && (l0 + t) < p.L;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float ac[G], uc[G], pc[NS], f[NS], J[NS][NS];
#pragma unroll
      for (int g = 0; g < G; ++g) { ac[g] = av[g][c]; uc[g] = uu[t][g].get(c); }
#pragma unroll
      for (int s = 0; s < NS; ++s) pc[s] = (t == 0) ? sp[s][c] : so[t - 1][s][c];
      Cell::step(ac, uc, pc, f, J);
#pragma unroll
      for (int r = 0; r < NS; ++r) {
#pragma unroll
        for (int s = 0; s < NS; ++s) Jt[t][r][s][c] = v ? J[r][s] : (r == s ? 1.0f : 0.0f);
        rt[t][r][c] = v ? (f[r] - so[t][r][c]) : 0.0f;
      }
    }
    Aff<NS, C> e;
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) {
#pragma unroll
        for (int s = 0; s < NS; ++s) e.A[r][s][c] = Jt[t][r][s][c];
        e.b[r][c] = rt[t][r][c];
      }
    e.after(acc);
    acc = e;
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
        if (chunk < p.nchunks - 1) publish_agg<NS, C>(p.agg, BD, chan, chunk, tag, tot);
        lookback<NS, C>(p.incl, p.agg, BD, chan, chunk, -1, p.nchunks, tag, carry);
      }
      if (chunk < p.nchunks - 1) {
        float x[NS][C];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int c = 0; c < C; ++c) x[s][c] = carry[s][c];
        tot.apply(x);
        publish_incl<NS, C>(p.incl, BD, chan, chunk, tag, x);
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

  uint32_t mbits = 0u;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int l = l0 + t;
    float y[NS][C];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        float acc2 = rt[t][r][c];
#pragma unroll
        for (int s = 0; s < NS; ++s) acc2 = fmaf(Jt[t][r][s][c], x[s][c], acc2);
        y[r][c] = acc2;
      }
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) x[r][c] = y[r][c];
    if (dv && l < p.L) {
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        float o[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
          o[c] = so[t][r][c] + x[r][c];
          mbits = max(mbits, __float_as_uint(fabsf(x[r][c])));
        }
        st_f32<C>(p.sout[r] + (row0 + l) * p.D + d0, o);
      }
    }
  }
  // row max of |update|: wave reduction on the bit patterns (NaN ranks above +inf)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mbits = max(mbits, static_cast<uint32_t>(__shfl_xor(mbits, off, 64)));
  if (lane == 0) atomicMax(p.maxupd + static_cast<long long>(p.k - 1) * p.B + b, mbits);

  // ---- flags: the last workgroup of the launch turns row maxima into flags
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const unsigned int n = atomicAdd(p.ctr + p.K + (p.k - 1), 1u);
    s_flag = (n == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (s_flag) {
    __threadfence();
    int allc = 1;
    for (int bb = tid; bb < p.B; bb += blockDim.x) {
      const uint32_t mb = __hip_atomic_load(p.maxupd + static_cast<long long>(p.k - 1) * p.B + bb,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float mf = __uint_as_float(mb);
      const int cv = (mf <= p.tol) ? 1 : 0;  // NaN compares false
      if (p.maxupd_out) p.maxupd_out[static_cast<long long>(p.k - 1) * p.B + bb] = mf;
      if (p.conv_out) p.conv_out[bb] = cv;
      allc &= cv;
    }
    allc = __syncthreads_and(allc);
    if (tid == 0) {
      const bool stop = p.early_exit && allc;
      if (p.iters_out && (stop || p.k == p.K)) *p.iters_out = p.k;
      if (stop) __hip_atomic_store(p.ctr + 2 * p.K, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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
