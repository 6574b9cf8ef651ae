// scan_dense.h -- the linear recurrence with a dense n x n matrix per step,
//   s_l = A_l s_{l-1} + b_l,   s_{-1} = s0,   n <= 32,
// the linearised system of a generic RNN whose Jacobians are dense (ParaRNN
// article, cafecomtech.com, section "Engenharia pra escalar": storage grows as
// n^2 and the products as n^3, which is why the diagonal cells exist; for
// small n it is still a few GEMM-shaped products per step).
//
// Three launches over chunks of kDenseChunk steps of one batch row:
//   1. dense_chunk_kernel: the transfer P = A_end ... A_start (a chain of
//      32 x 32 x 32 products on the matrix cores, fp32) and local solution v
//      from zero of every segment of kDenseSeg steps (one wave each), then an
//      inclusive scan of these over the chunk's segments through LDS: the
//      chunk's transfer, and for every segment the transfer and local
//      solution of the segments before it;
//   2. dense_carry_kernel: per batch row, the carries into the chunks,
//      x_{c+1} = P_c x_c + v_c from s0, one matrix-vector product per chunk;
//   3. dense_apply_kernel: per segment, its carry from the chunk's (one
//      matrix-vector product with the prefix), then the recurrence itself,
//      one matrix-vector product per step, writing s.
// Everything runs in a 32 x 32 frame: entries past n are zero, and so stay
// the padded state components.
//
// Matrix-core layout (v_mfma_f32_32x32x2f32, one 64-lane wave): lane
// (j, h) = (lane % 32, lane / 32) holds accumulator slots r = 0..15 with the
// entries D[R(r, h)][j], R(r, h) = 8 (r / 4) + 4 h + r % 4. Product step r
// contracts over the index pair (R(r, 0), R(r, 1)): lane (i, h) supplies
// A[i][R(r, h)] and lane (j, h) supplies the previous product's own slot r,
// so a chain Q <- A Q needs no data movement between products.
#pragma once

#include "device_common.h"

namespace pararnn {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kDenseMaxN = 32;          // largest state size
constexpr int kDenseSeg = 16;           // steps per wave in the transfer chain
constexpr int kDenseWaves = 8;          // waves (segments) per chunk
constexpr int kDenseChunk = kDenseSeg * kDenseWaves;
constexpr int kDenseRing = 4;           // steps of A in flight per wave in the transfer chain

__device__ __forceinline__ int dense_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

struct DenseArgs {
  const float* A;   // [B][L][n][n]
  const float* b;   // [B][L][n]
  const float* s0;  // [B][n] or nullptr
  float* s;         // [B][L][n]
  float* P;         // [B][nchunks][32][32] chunk transfers (workspace)
  float* v;         // [B][nchunks][32] chunk local solutions (workspace)
  float* carry;     // [B][nchunks][32] carries into the chunks (workspace)
  float* Pseg;      // [B][nchunks][kDenseWaves][32][32] transfers of the segments before each (workspace)
  float* vseg;      // [B][nchunks][kDenseWaves][32] their local solutions (workspace)
  int B, L, n, nchunks;
};

// Row i of A_l at the 16 columns R(r, h) (zero past n), and b_l[i]. N32: n is
// 32 and A is 16-byte aligned, so the four runs of four columns are vector
// loads; otherwise the address is clamped into the matrix and the value
// selected, so no load sits behind a branch.
template <bool N32>
__device__ __forceinline__ void dense_load_row(const DenseArgs& p, long long step, int i, int h, float (&a)[16],
                                               float& bi) {
  if constexpr (N32) {
    const float* row = p.A + (step * 32 + i) * 32;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(row + 8 * g + 4 * h);
      a[4 * g] = q.x;
      a[4 * g + 1] = q.y;
      a[4 * g + 2] = q.z;
      a[4 * g + 3] = q.w;
    }
    bi = p.b[step * 32 + i];
  } else {
    const int ic = min(i, p.n - 1);
    const float* row = p.A + (step * p.n + ic) * p.n;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = dense_row(r, h);
      const float t = row[min(c, p.n - 1)];
      a[r] = (i < p.n && c < p.n) ? t : 0.0f;
    }
    const float t = p.b[step * p.n + ic];
    bi = (i < p.n) ? t : 0.0f;
  }
}

// Lanes (i, 0) and (i, 1), which hold the same value, publish element i of
// the wave's vector in its LDS slot xl for the next dense_matvec (both write,
// so no lane mask splits the code around the store). The LDS operations of
// one wave complete in order, so the exchange needs no workgroup barrier; the
// fences and the wave barrier tell the compiler that other lanes wrote the
// slot. Without them a lane may keep what it read before, or read before the
// write.
__device__ __forceinline__ void dense_share(float* xl, int i, int h, float x) {
  (void)h;
  xl[i] = x;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// part[lane] + part[lane ^ 32]: one swap of the two half-waves' values
// between registers (gfx950), no LDS round trip
__device__ __forceinline__ float dense_halves_sum(float part) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// y[i] = sum_q a[i][q] x[q] + bi in lanes i and i + 32, with x[q] read from
// this wave's LDS vector xl (lane (i, h) reads its four runs of four)
__device__ __forceinline__ float dense_matvec(const float (&a)[16], const float* xl, int h, float bi) {
  float pg[4];  // four independent partial sums shorten the dependent chain
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 xv = *reinterpret_cast<const f32x4*>(xl + 8 * g + 4 * h);
    pg[g] = a[4 * g] * xv.x;
    pg[g] = fmaf(a[4 * g + 1], xv.y, pg[g]);
    pg[g] = fmaf(a[4 * g + 2], xv.z, pg[g]);
    pg[g] = fmaf(a[4 * g + 3], xv.w, pg[g]);
  }
  const float part = (pg[0] + pg[1]) + (pg[2] + pg[3]);
  return dense_halves_sum(part) + bi;
}

// Q <- A Q with A given as row values a (this lane's row, columns R(r, h))
__device__ __forceinline__ f32x16 dense_mfma_chain(const float (&a)[16], const f32x16& Q) {
  f32x16 out = {};
#pragma unroll
  for (int r = 0; r < 16; ++r) out = __builtin_amdgcn_mfma_f32_32x32x2f32(a[r], Q[r], out, 0, 0, 0);
  return out;
}

template <bool N32>
__global__ void __launch_bounds__(64 * kDenseWaves) dense_chunk_kernel(const DenseArgs p) {
  __shared__ float s_q[kDenseWaves][32][33];  // the waves' transfers at each scan level (padded rows)
  __shared__ __align__(16) float s_v[kDenseWaves][32];
  __shared__ __align__(16) float s_x[kDenseWaves][32];  // each wave's running vector
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 31, h = lane >> 5;
  const int b = blockIdx.x / p.nchunks, c = blockIdx.x - b * p.nchunks;
  const int l_begin = c * kDenseChunk + wave * kDenseSeg;
  const int l_end = min(l_begin + kDenseSeg, p.L);
  const long long row0 = static_cast<long long>(b) * p.L;
  float* xl = s_x[wave];

  // segment transfer Q (accumulator layout) and local solution v (lane i, both halves)
  f32x16 Q;
#pragma unroll
  for (int r = 0; r < 16; ++r) Q[r] = (dense_row(r, h) == j) ? 1.0f : 0.0f;
  float v = 0.0f;
  dense_share(xl, j, h, 0.0f);
  // rows stream through a ring of kDenseRing steps ahead of the chain. The
  // loads are unconditional, their step clamped into the row (steps past the
  // end are read and not used): a load behind a branch leaves the compiler
  // unable to count the loads in flight, and it then waits for all of them
  // before each step, which empties the ring.
  const int l_last = p.L - 1;
  float a[kDenseRing][16], bs[kDenseRing];
#pragma unroll
  for (int t = 0; t < kDenseRing; ++t)
    dense_load_row<N32>(p, row0 + min(l_begin + t, l_last), j, h, a[t], bs[t]);
  // Steps past the end of the sequence act as the identity (A = I, b = 0),
  // selected rather than branched around: each step is straight code, in
  // which the compiler can overlap the vector chain v with the independent
  // matrix-core chain Q. A scheduling barrier closes each step, so that its
  // prefetch load is not moved down to where the row is used.
#pragma unroll
  for (int t = 0; t < kDenseSeg; ++t) {
    const int k = t % kDenseRing;
    const bool live = l_begin + t < l_end;
    float ak[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ak[r] = live ? a[k][r] : (dense_row(r, h) == j ? 1.0f : 0.0f);
    v = dense_matvec(ak, xl, h, live ? bs[k] : 0.0f);
    dense_share(xl, j, h, v);
    Q = dense_mfma_chain(ak, Q);
    if (t + kDenseRing < kDenseSeg)
      dense_load_row<N32>(p, row0 + min(l_begin + t + kDenseRing, l_last), j, h, a[k], bs[k]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // inclusive scan over the chunk's segments (three levels): at distance d,
  // wave w >= d composes its range with the one that ends at wave w - d and
  // precedes it, Q_w <- Q_w Q_{w-d}, v_w <- Q_w v_{w-d} + v_w. Wave w's own
  // transfer is read back in row layout (the products' first operand), the
  // other's in accumulator layout.
  for (int d = 1; d < kDenseWaves; d *= 2) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s_q[wave][dense_row(r, h)][j] = Q[r];
    s_v[wave][j] = v;
    __syncthreads();
    if (wave >= d) {
      float aq[16];
      f32x16 Qo;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        aq[r] = s_q[wave][j][dense_row(r, h)];
        Qo[r] = s_q[wave - d][dense_row(r, h)][j];
      }
      v = dense_matvec(aq, s_v[wave - d], h, v);
      Q = dense_mfma_chain(aq, Qo);
    }
    __syncthreads();
  }
  // wave w now holds segments 0 .. w composed: the prefix of segment w + 1,
  // and for the last wave the chunk's transfer; segment 0's prefix is the
  // identity
  const long long cbi = static_cast<long long>(b) * p.nchunks + c;
  const bool last = wave == kDenseWaves - 1;
  float* Pd = last ? p.P + cbi * 1024 : p.Pseg + (cbi * kDenseWaves + wave + 1) * 1024;
  float* vd = last ? p.v + cbi * 32 : p.vseg + (cbi * kDenseWaves + wave + 1) * 32;
#pragma unroll
  for (int r = 0; r < 16; ++r) Pd[dense_row(r, h) * 32 + j] = Q[r];
  if (h == 0) vd[j] = v;
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) p.Pseg[cbi * kDenseWaves * 1024 + dense_row(r, h) * 32 + j] = (dense_row(r, h) == j) ? 1.0f : 0.0f;
    if (h == 0) p.vseg[cbi * kDenseWaves * 32 + j] = 0.0f;
  }
}

// One workgroup per batch row: the carries into every chunk, in order. The
// chain is one matrix-vector product per chunk; what bounds it is the latency
// of reading each chunk's transfer. So all waves stage the transfers into LDS
// a block of kDenseCarryBlock chunks at a time (every load of a block in
// flight at once), the next block loading while wave 0 runs the chain
// through the current one. Rows are padded to kDenseCarryRow floats, so the
// 16-byte row reads of the chain spread over the LDS banks.
constexpr int kDenseCarryBlock = 16;
constexpr int kDenseCarryWaves = 4;
constexpr int kDenseCarryRow = 36;
constexpr int kDenseCarryPieces = kDenseCarryBlock * 256 / (64 * kDenseCarryWaves);  // f32x4 per thread
constexpr int kDenseCarryVPieces = kDenseCarryBlock * 32 / (64 * kDenseCarryWaves);  // floats per thread
__global__ void __launch_bounds__(64 * kDenseCarryWaves) dense_carry_kernel(const DenseArgs p) {
  __shared__ __align__(16) float s_p[2][kDenseCarryBlock][32 * kDenseCarryRow];
  __shared__ float s_v[2][kDenseCarryBlock][32];
  __shared__ __align__(16) float xl[32];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
  const int b = blockIdx.x;
  const long long base = static_cast<long long>(b) * p.nchunks;
  const int nblk = (p.nchunks + kDenseCarryBlock - 1) / kDenseCarryBlock;
  f32x4 stage[kDenseCarryPieces];
  float vstage[kDenseCarryVPieces];
  // loads of block blk into registers; chunk indices past the end are
  // clamped onto the last chunk (read, never committed)
  auto issue = [&](int blk) {
    const int c0 = blk * kDenseCarryBlock, last = p.nchunks - 1 - c0;
#pragma unroll
    for (int i = 0; i < kDenseCarryPieces; ++i) {
      const int piece = tid + i * 64 * kDenseCarryWaves;
      const int k = min(piece >> 8, last);
      stage[i] = *reinterpret_cast<const f32x4*>(p.P + (base + c0 + k) * 1024 + (piece & 255) * 4);
    }
#pragma unroll
    for (int i = 0; i < kDenseCarryVPieces; ++i) {
      const int e = tid + i * 64 * kDenseCarryWaves;
      vstage[i] = p.v[(base + c0 + min(e >> 5, last)) * 32 + (e & 31)];
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kDenseCarryPieces; ++i) {
      const int piece = tid + i * 64 * kDenseCarryWaves;
      const int q = piece & 255;  // row q / 8, columns 4 (q % 8) ..
      *reinterpret_cast<f32x4*>(&s_p[buf][piece >> 8][(q >> 3) * kDenseCarryRow + (q & 7) * 4]) = stage[i];
    }
#pragma unroll
    for (int i = 0; i < kDenseCarryVPieces; ++i) {
      const int e = tid + i * 64 * kDenseCarryWaves;
      s_v[buf][e >> 5][e & 31] = vstage[i];
    }
  };
  float x = (p.s0 && j < p.n) ? p.s0[static_cast<long long>(b) * p.n + min(j, p.n - 1)] : 0.0f;
  if (wave == 0 && h == 0) xl[j] = x;
  issue(0);
  commit(0);
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int buf = blk & 1;
    if (blk + 1 < nblk) issue(blk + 1);
    if (wave == 0) {
      const int c0 = blk * kDenseCarryBlock, nc = min(kDenseCarryBlock, p.nchunks - c0);
      for (int k = 0; k < nc; ++k) {
        if (h == 0) p.carry[(base + c0 + k) * 32 + j] = x;
        float a[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 q = *reinterpret_cast<const f32x4*>(&s_p[buf][k][j * kDenseCarryRow + 8 * g + 4 * h]);
          a[4 * g] = q.x;
          a[4 * g + 1] = q.y;
          a[4 * g + 2] = q.z;
          a[4 * g + 3] = q.w;
        }
        x = dense_matvec(a, xl, h, s_v[buf][k][j]);
        dense_share(xl, j, h, x);
      }
    }
    // the other buffer was last read by the chain of block blk - 1, which
    // the barrier below (of that iteration) has ended
    if (blk + 1 < nblk) commit(buf ^ 1);
    __syncthreads();
  }
}

// one wave per segment: the carry into the segment, x = E x_c + e from the
// chunk's carry x_c with the transfer E and local solution e of the
// segments before it, then the recurrence from it. The rows of A stream
// through a ring of kDenseApplyRing steps ahead of the recurrence, loaded
// unconditionally with the step clamped into the row, so that the compiler
// counts the loads in flight and each step waits for its own rows only (a
// load behind a branch makes it wait for all of them). E, e and x_c are
// loaded first: the load counter is in order, so waiting for them leaves
// the ring in flight.
constexpr int kDenseApplyRing = 8;
template <bool N32>
__global__ void __launch_bounds__(64) dense_apply_kernel(const DenseArgs p) {
  __shared__ __align__(16) float xl[32];
  const int lane = threadIdx.x, j = lane & 31, h = lane >> 5;
  const long long sg = blockIdx.x;  // (b * nchunks + c) * kDenseWaves + w
  const int b = static_cast<int>(sg / (static_cast<long long>(p.nchunks) * kDenseWaves));
  const int cw = static_cast<int>(sg - static_cast<long long>(b) * p.nchunks * kDenseWaves);  // c * W + w
  const long long row0 = static_cast<long long>(b) * p.L;
  const int l_begin = cw * kDenseSeg, l_end = min(l_begin + kDenseSeg, p.L), l_last = p.L - 1;
  if (l_begin >= p.L) return;  // segment past the end of the sequence (uniform per wave)
  float e[16];
  {
    const float* E = p.Pseg + sg * 1024 + j * 32;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(E + 8 * g + 4 * h);
      e[4 * g] = q.x;
      e[4 * g + 1] = q.y;
      e[4 * g + 2] = q.z;
      e[4 * g + 3] = q.w;
    }
  }
  const float ev = p.vseg[sg * 32 + j];
  const float xc = p.carry[(sg / kDenseWaves) * 32 + j];
  __builtin_amdgcn_sched_barrier(0);
  float a[kDenseApplyRing][16], bs[kDenseApplyRing];
#pragma unroll
  for (int t = 0; t < kDenseApplyRing; ++t)
    dense_load_row<N32>(p, row0 + min(l_begin + t, l_last), j, h, a[t], bs[t]);
  __builtin_amdgcn_sched_barrier(0);
  dense_share(xl, j, h, xc);
  float x = dense_matvec(e, xl, h, ev);
  dense_share(xl, j, h, x);
#pragma unroll
  for (int t = 0; t < kDenseSeg; ++t) {
    const int k = t % kDenseApplyRing, l = l_begin + t;
    if (l < l_end) {
      x = dense_matvec(a[k], xl, h, bs[k]);
      dense_share(xl, j, h, x);
      if (h == 0 && j < p.n) p.s[(row0 + l) * p.n + j] = x;
    }
    if (t + kDenseApplyRing < kDenseSeg)
      dense_load_row<N32>(p, row0 + min(l + kDenseApplyRing, l_last), j, h, a[k], bs[k]);
  }
}

}  // namespace pararnn
