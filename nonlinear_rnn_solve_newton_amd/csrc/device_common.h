// device_common.h -- numerics, vector memory access, the two cells and the
// chunk-carry descriptors shared by the Newton-iteration and adjoint kernels.
// gfx950 (CDNA4) only: wave64, v_exp_f32 / v_rcp_f32, agent-scope atomics.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pararnn {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Storage tag for bfloat16 gate inputs (raw bits; widened to fp32 exactly).
struct bf16 {
  uint16_t bits;
};

// ---------------------------------------------------------------------------
// numerics: logistic sigmoid from the hardware base-2 exponential and
// reciprocal (about 1 ulp each); tanh(x) = 2 s(2x) - 1. Overflow of the
// exponential gives the correct limits (s -> 0 or 1); NaN propagates.
constexpr float kSigmScale = -1.4426950408889634f;  // -log2(e)
constexpr float kTanhScale = -2.8853900817779268f;  // -2 log2(e)
// the same functions of an argument already multiplied by their scale
__device__ __forceinline__ float sigm2(float y) { return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y)); }
__device__ __forceinline__ float tanh2(float y) {
  return fmaf(2.0f, __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y)), -1.0f);
}
__device__ __forceinline__ float sigm(float x) { return sigm2(x * kSigmScale); }
__device__ __forceinline__ float tanh_fast(float x) { return tanh2(x * kTanhScale); }

// ---------------------------------------------------------------------------
// vector loads / stores of C consecutive channels (C in {1, 2, 4}); the host
// only selects C when every pointer and row offset is aligned for it.
template <int C>
__device__ __forceinline__ void ld_f32(const float* p, float (&v)[C]) {
  if constexpr (C == 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else if constexpr (C == 2) {
    const f32x2 x = *reinterpret_cast<const f32x2*>(p);
    v[0] = x.x; v[1] = x.y;
  } else {
    v[0] = *p;
  }
}

// Streaming loads (read once per launch): nontemporal, so they do not displace
// reusable lines in the caches.
template <int C>
__device__ __forceinline__ void ld_f32_stream(const float* p, float (&v)[C]) {
  if constexpr (C == 4) {
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else if constexpr (C == 2) {
    const f32x2 x = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
    v[0] = x.x; v[1] = x.y;
  } else {
    v[0] = __builtin_nontemporal_load(p);
  }
}

template <int C>
__device__ __forceinline__ void st_f32(float* p, const float (&v)[C]) {
  if constexpr (C == 4) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  } else if constexpr (C == 2) {
    *reinterpret_cast<f32x2*>(p) = f32x2{v[0], v[1]};
  } else {
    *p = v[0];
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// Buffer-resource access: a 128-bit descriptor in scalar registers (base,
// byte extent) plus a 32-bit per-lane offset and a 32-bit uniform offset.
// Offsets at or past the extent read 0 and drop stores, which handles every
// tail without branches. Descriptors here cover one batch row of a tensor.
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufCfg = 0x00020000;  // 32-bit data format, raw (unformatted) access
constexpr int kBufNT = 2;            // nontemporal cache policy

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           kBufCfg);
}

template <int C>
__device__ __forceinline__ void buf_ld_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float (&v)[C]) {
  if constexpr (C == 4) {
    const i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kBufNT);
    v[0] = __int_as_float(x.x); v[1] = __int_as_float(x.y); v[2] = __int_as_float(x.z); v[3] = __int_as_float(x.w);
  } else if constexpr (C == 2) {
    const i32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kBufNT);
    v[0] = __int_as_float(x.x); v[1] = __int_as_float(x.y);
  } else {
    v[0] = __int_as_float(static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kBufNT)));
  }
}

// AUX: cache policy of the store (0 default, kBufNT for data not read again soon)
template <int C, int AUX = 0>
__device__ __forceinline__ void buf_st_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, const float (&v)[C]) {
  if constexpr (C == 4) {
    __builtin_amdgcn_raw_buffer_store_b128(i32x4{__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]),
                                                 __float_as_int(v[3])}, r, voff, soff, AUX);
  } else if constexpr (C == 2) {
    __builtin_amdgcn_raw_buffer_store_b64(i32x2{__float_as_int(v[0]), __float_as_int(v[1])}, r, voff, soff, AUX);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(__float_as_int(v[0])), r, voff, soff, AUX);
  }
}

// Raw gate-input registers: bf16 inputs stay packed (two per 32-bit
// register) until the cell evaluation widens them, which halves the registers
// held while the loads are in flight.
template <class UT, int C>
struct URaw;

template <int C>
struct URaw<float, C> {
  float v[C];
  __device__ __forceinline__ void load(const float* p) { ld_f32_stream<C>(p, v); }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int c = 0; c < C; ++c) v[c] = 0.0f;
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    buf_ld_f32<C>(r, voff, soff, v);
  }
  __device__ __forceinline__ float get(int c) const { return v[c]; }
  // raw bits to / from workgroup memory (C consecutive channels)
  __device__ __forceinline__ void put_lds(float* q) const {
#pragma unroll
    for (int c = 0; c < C; ++c) q[c] = v[c];
  }
  __device__ __forceinline__ void get_lds(const float* q) {
#pragma unroll
    for (int c = 0; c < C; ++c) v[c] = q[c];
  }
};

template <int C>
struct URaw<bf16, C> {
  static constexpr int NW = (C + 1) / 2;
  uint32_t w[NW];
  __device__ __forceinline__ void load(const bf16* p) {
    if constexpr (C == 4) {
      const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
      w[0] = x.x;
      w[1] = x.y;
    } else if constexpr (C == 2) {
      w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    } else {
      w[0] = static_cast<uint32_t>(__builtin_nontemporal_load(&p->bits));
    }
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (C == 4) {
      const i32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kBufNT);
      w[0] = static_cast<uint32_t>(x.x);
      w[1] = static_cast<uint32_t>(x.y);
    } else if constexpr (C == 2) {
      w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kBufNT);
    } else {
      w[0] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kBufNT));
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = 0u;
  }
  __device__ __forceinline__ float get(int c) const {
    return (c & 1) ? bf16_hi(w[c >> 1]) : bf16_lo(w[c >> 1]);
  }
  __device__ __forceinline__ void put_lds(bf16* q) const {
    if constexpr (C == 1) {
      q->bits = static_cast<uint16_t>(w[0]);
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) reinterpret_cast<uint32_t*>(q)[i] = w[i];
    }
  }
  __device__ __forceinline__ void get_lds(const bf16* q) {
    if constexpr (C == 1) {
      w[0] = q->bits;
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) w[i] = reinterpret_cast<const uint32_t*>(q)[i];
    }
  }
};

// ---------------------------------------------------------------------------
// Cells. step() evaluates the next state f and its Jacobian J = df/ds at the
// previous state s, J in the cell's compact form Jac. The scan of one Newton
// iteration, d_l = J_l d_{l-1} + r_l with the residual r_l = f_l - S_l, goes
// through the cell: residual() forms r in the cell's form, first() and pre()
// build a lane's composite transform over its steps, apply() takes one step
// of the recurrence. step_adj() returns J and NK coefficients k from which
// grad_u() forms, for an adjoint lambda, the input gradient
// du_g = sum_r lambda_r df_r/du_g and the multiplier m_g of a_g in gate g's
// pre-activation (dL/da_g = du_g * m_g); k is the compact form of df/du the
// reverse scan keeps per step.
// ParaGRU: diagonal Jacobian (1x1 per channel); ParaLSTM: 2x2 over (c, h),
// per the ParaRNN article's section "Engenharia pra escalar".
struct GruCell {
  static constexpr int NS = 1;  // state: h
  static constexpr int G = 3;   // gates: z, r, c

  struct Jac {
    float j;
  };

  // next state and Jacobian from the gate values at state h; Z: h = 0, with
  // the products of the zero state dropped
  template <bool Z>
  __device__ static __forceinline__ void assemble(const float (&a)[G], float z, float r, float c, float h,
                                                  float rh, float (&f)[NS], Jac& J) {
    // J = (1 - z) + z [a_z (1 - z)(c - h) + a_c (1 - c^2) d(rh)/dh], z taken
    // out of both gate terms (one multiply fewer than summing them), with
    // d(rh)/dh = r + a_r h r (1 - r) = r + a_r (rh - r rh).
    const float omz = 1.0f - z;
    const float dtc = fmaf(-c, c, 1.0f);  // d tanh / d pre_c
    if constexpr (Z) {
      f[0] = z * c;
      J.j = fmaf(z, fmaf(a[2], dtc * r, a[0] * (omz * c)), omz);
    } else {
      const float cmh = c - h;
      f[0] = fmaf(z, cmh, h);  // (1 - z) h + z c
      const float drh = fmaf(a[1], fmaf(-r, rh, rh), r);  // d (r h) / dh
      J.j = fmaf(z, fmaf(a[2], dtc * drh, a[0] * (omz * cmh)), omz);
    }
  }

  __device__ static __forceinline__ void step(const float (&a)[G], const float (&u)[G],
                                              const float (&s)[NS], float (&f)[NS], Jac& J) {
    const float h = s[0];
    const float z = sigm(fmaf(a[0], h, u[0]));
    const float r = sigm(fmaf(a[1], h, u[1]));
    const float rh = r * h;
    const float c = tanh_fast(fmaf(a[2], rh, u[2]));
    assemble<false>(a, z, r, c, h, rh, f, J);
  }

  // step() at the zero state h = 0, with the products of the zero state
  // dropped: the same values as step(a, u, {0}) when every a is finite (a * 0
  // is then a signed zero that the following add absorbs).
  __device__ static __forceinline__ void step_zero(const float (&a)[G], const float (&u)[G],
                                                   float (&f)[NS], Jac& J) {
    assemble<true>(a, sigm(u[0]), sigm(u[1]), tanh_fast(u[2]), 0.0f, 0.0f, f, J);
  }

  // r = f - S at the step (ZERO: the previous iterate is zero there)
  template <bool ZERO>
  __device__ static __forceinline__ void residual(const float (&f)[NS], const float (&so)[NS], const Jac&,
                                                  float (&r)[NS]) {
    r[0] = ZERO ? f[0] : f[0] - so[0];
  }
  // channel c of a lane's composite transform e: the first step alone, or
  // the next step composed after it
  template <class A>
  __device__ static __forceinline__ void first(A& e, int c, const Jac& J, const float (&r)[NS]) {
    e.A[0][0][c] = J.j;
    e.b[0][c] = r[0];
  }
  template <class A>
  __device__ static __forceinline__ void pre(A& e, int c, const Jac& J, const float (&r)[NS]) {
    e.A[0][0][c] *= J.j;
    e.b[0][c] = fmaf(J.j, e.b[0][c], r[0]);
  }
  // one step of the recurrence: x <- J x + r
  __device__ static __forceinline__ void apply(const Jac& J, const float (&r)[NS], float (&x)[NS]) {
    x[0] = fmaf(J.j, x[0], r[0]);
  }

  static constexpr int NK = 4;  // dh'/du_z, dh'/du_r, dh'/du_c, r h
  __device__ static __forceinline__ void step_adj(const float (&a)[G], const float (&u)[G],
                                                  const float (&s)[NS], float (&J)[NS][NS], float (&k)[NK]) {
    const float h = s[0];
    const float z = sigm(fmaf(a[0], h, u[0]));
    const float r = sigm(fmaf(a[1], h, u[1]));
    const float rh = r * h;
    const float c = tanh_fast(fmaf(a[2], rh, u[2]));
    const float cmh = c - h;
    const float omz = 1.0f - z;
    const float gz = cmh * z * omz;
    const float gc = z * fmaf(-c, c, 1.0f);
    const float rr = r - r * r;
    const float drh = fmaf(h * a[1], rr, r);
    J[0][0] = fmaf(gc * a[2], drh, fmaf(gz, a[0], omz));
    k[0] = gz;
    k[1] = gc * a[2] * h * rr;
    k[2] = gc;
    k[3] = rh;
  }

  __device__ static __forceinline__ void grad_u(const float (&k)[NK], const float (&s)[NS], const float (&lam)[NS],
                                                float (&du)[G], float (&m)[G]) {
    du[0] = k[0] * lam[0];
    du[1] = k[1] * lam[0];
    du[2] = k[2] * lam[0];
    m[0] = s[0];
    m[1] = s[0];
    m[2] = k[3];
  }

};

struct LstmCell {
  static constexpr int NS = 2;  // state: (c, h)
  static constexpr int G = 4;   // gates: i, f, o, g

  // multiplier of each gate's pre-activation inside its base-2 exponential
  static constexpr float kScale[G] = {kSigmScale, kSigmScale, kSigmScale, kTanhScale};

  // The 2x2 Jacobian over (c, h) factored as J = [[1, 0], [q, 1]] [[gf, X], [0, w]],
  // i.e. J = [[gf, X], [q gf, w + q X]]: gf = dc'/dc, X = dc'/dh, q = dh'/dc',
  // w = dh'/dh through the output gate. With the residual kept as
  // (r_c, r_h - q r_c), a step of the scan is y_c = gf x_c + X x_h + r_c,
  // y_h = q y_c + w x_h + (r_h - q r_c): J x + r with fewer operations than
  // the plain 2x2 form.
  struct Jac {
    float gf, X, q, w;
  };

  // next state and Jacobian from the gate values at previous cell state cp;
  // Z: the zero state, with its products dropped
  template <bool Z>
  __device__ static __forceinline__ void assemble(const float (&a)[G], float gi, float gf, float go, float gg,
                                                  float cp, float (&f)[NS], Jac& J) {
    const float cn = Z ? gi * gg : fmaf(gf, cp, gi * gg);
    const float t = tanh_fast(cn);
    const float h = go * t;
    f[0] = cn;
    f[1] = h;
    J.gf = gf;
    J.q = fmaf(-h, t, go);                  // go (1 - t^2)
    J.w = a[2] * fmaf(-go, h, h);           // a_o t go (1 - go)
    // X = a_i gg gi (1 - gi) + a_g gi (1 - gg^2) + a_f cp gf (1 - gf); its
    // first two terms are gi (a_g + gg (a_i - a_i gi - a_g gg))
    const float bi = fmaf(gg, fmaf(-a[3], gg, fmaf(-a[0], gi, a[0])), a[3]);
    J.X = Z ? gi * bi : fmaf(a[1] * cp, fmaf(-gf, gf, gf), gi * bi);
  }

  __device__ static __forceinline__ void step(const float (&a)[G], const float (&u)[G],
                                              const float (&s)[NS], float (&f)[NS], Jac& J) {
    const float hp = s[1];
    assemble<false>(a, sigm(fmaf(a[0], hp, u[0])), sigm(fmaf(a[1], hp, u[1])), sigm(fmaf(a[2], hp, u[2])),
                    tanh_fast(fmaf(a[3], hp, u[3])), s[0], f, J);
  }

  // step() at the zero state (c, h) = 0, with the products of the zero state
  // dropped: equal to step(a, u, {0, 0}) bit for bit when every a is finite.
  __device__ static __forceinline__ void step_zero(const float (&a)[G], const float (&u)[G],
                                                   float (&f)[NS], Jac& J) {
    assemble<true>(a, sigm(u[0]), sigm(u[1]), sigm(u[2]), tanh_fast(u[3]), 0.0f, f, J);
  }

  // step() and step_zero() with the coefficients and inputs already multiplied
  // by kScale (as, us), a keeping the plain coefficients for the Jacobian
  __device__ static __forceinline__ void step_scaled(const float (&a)[G], const float (&as)[G], const float (&us)[G],
                                                     const float (&s)[NS], float (&f)[NS], Jac& J) {
    const float hp = s[1];
    assemble<false>(a, sigm2(fmaf(as[0], hp, us[0])), sigm2(fmaf(as[1], hp, us[1])),
                    sigm2(fmaf(as[2], hp, us[2])), tanh2(fmaf(as[3], hp, us[3])), s[0], f, J);
  }
  __device__ static __forceinline__ void step_zero_scaled(const float (&a)[G], const float (&us)[G],
                                                          float (&f)[NS], Jac& J) {
    assemble<true>(a, sigm2(us[0]), sigm2(us[1]), sigm2(us[2]), tanh2(us[3]), 0.0f, f, J);
  }

  // r = (f_c - S_c, (f_h - S_h) - q (f_c - S_c)) at the step (ZERO: the
  // previous iterate is zero there)
  template <bool ZERO>
  __device__ static __forceinline__ void residual(const float (&f)[NS], const float (&so)[NS], const Jac& J,
                                                  float (&r)[NS]) {
    r[0] = ZERO ? f[0] : f[0] - so[0];
    r[1] = fmaf(-J.q, r[0], ZERO ? f[1] : f[1] - so[1]);
  }
  template <class A>
  __device__ static __forceinline__ void first(A& e, int c, const Jac& J, const float (&r)[NS]) {
    e.A[0][0][c] = J.gf;
    e.A[0][1][c] = J.X;
    e.A[1][0][c] = J.q * J.gf;
    e.A[1][1][c] = fmaf(J.q, J.X, J.w);
    e.b[0][c] = r[0];
    e.b[1][c] = fmaf(J.q, r[0], r[1]);
  }
  template <class A>
  __device__ static __forceinline__ void pre(A& e, int c, const Jac& J, const float (&r)[NS]) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const float n0 = fmaf(J.gf, e.A[0][j][c], J.X * e.A[1][j][c]);
      e.A[1][j][c] = fmaf(J.q, n0, J.w * e.A[1][j][c]);
      e.A[0][j][c] = n0;
    }
    const float b0 = fmaf(J.gf, e.b[0][c], fmaf(J.X, e.b[1][c], r[0]));
    e.b[1][c] = fmaf(J.q, b0, fmaf(J.w, e.b[1][c], r[1]));
    e.b[0][c] = b0;
  }
  __device__ static __forceinline__ void apply(const Jac& J, const float (&r)[NS], float (&x)[NS]) {
    const float y0 = fmaf(J.gf, x[0], fmaf(J.X, x[1], r[0]));
    x[1] = fmaf(J.q, y0, fmaf(J.w, x[1], r[1]));
    x[0] = y0;
  }

  // q = dh'/dc', then dc'/du_i, dc'/du_f, dc'/du_g and dh'/du_o; the input
  // gates reach h' only through c' (dh'/du_x = q dc'/du_x), and every gate
  // pre-activation multiplies its coefficient by h.
  static constexpr int NK = 5;
  __device__ static __forceinline__ void step_adj(const float (&a)[G], const float (&u)[G],
                                                  const float (&s)[NS], float (&J)[NS][NS], float (&k)[NK]) {
    const float cp = s[0], hp = s[1];
    const float gi = sigm(fmaf(a[0], hp, u[0]));
    const float gf = sigm(fmaf(a[1], hp, u[1]));
    const float go = sigm(fmaf(a[2], hp, u[2]));
    const float gg = tanh_fast(fmaf(a[3], hp, u[3]));
    const float cn = fmaf(gf, cp, gi * gg);
    const float t = tanh_fast(cn);
    const float dci = gg * (gi - gi * gi);
    const float dcf = cp * (gf - gf * gf);
    const float dcg = gi * fmaf(-gg, gg, 1.0f);
    const float q = go * fmaf(-t, t, 1.0f);
    const float dho = t * (go - go * go);
    const float X = fmaf(dci, a[0], fmaf(dcf, a[1], dcg * a[3]));
    J[0][0] = gf;
    J[0][1] = X;
    J[1][0] = q * gf;
    J[1][1] = fmaf(dho, a[2], q * X);
    k[0] = q;
    k[1] = dci;
    k[2] = dcf;
    k[3] = dcg;
    k[4] = dho;
  }

  __device__ static __forceinline__ void grad_u(const float (&k)[NK], const float (&s)[NS], const float (&lam)[NS],
                                                float (&du)[G], float (&m)[G]) {
    const float mu = fmaf(k[0], lam[1], lam[0]);  // total dL/dc' through c' and h'
    du[0] = mu * k[1];
    du[1] = mu * k[2];
    du[2] = lam[1] * k[4];
    du[3] = mu * k[3];
    m[0] = s[1];
    m[1] = s[1];
    m[2] = s[1];
    m[3] = s[1];
  }

};

// ---------------------------------------------------------------------------
// Chunk-carry descriptors for the decoupled look-back across workgroups.
// Every value travels in its own 64-bit word: high half = tag (the Newton
// iteration number, >= 1; 0 = not yet written in this call), low half = the
// fp32 bits. A word is written once per launch with a relaxed agent-scope
// atomic store and polled with relaxed agent-scope atomic loads, so a reader
// either sees the old tag or the complete new value; no fences are needed
// and no value can be mistaken for another launch's.
__device__ __forceinline__ void desc_put(unsigned long long* p, uint32_t tag, float v) {
  const unsigned long long w = (static_cast<unsigned long long>(tag) << 32) | __float_as_uint(v);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long desc_get(unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool desc_ok(unsigned long long w, uint32_t tag) {
  return static_cast<uint32_t>(w >> 32) == tag;
}
__device__ __forceinline__ float desc_val(unsigned long long w) {
  return __uint_as_float(static_cast<uint32_t>(w));
}

// ---------------------------------------------------------------------------
// Affine scan element over NS-vectors for C channels: x -> A x + b.
template <int NS, int C>
struct Aff {
  float A[NS][NS][C];
  float b[NS][C];

  __device__ __forceinline__ void set_identity() {
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int c = 0; c < C; ++c) A[i][j][c] = (i == j) ? 1.0f : 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int c = 0; c < C; ++c) b[i][c] = 0.0f;
  }

  // this <- this o e  (apply e first, then this)
  __device__ __forceinline__ void after(const Aff& e) {
    Aff r;
#pragma unroll
    for (int c = 0; c < C; ++c) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < NS; ++k) acc = fmaf(A[i][k][c], e.A[k][j][c], acc);
          r.A[i][j][c] = acc;
        }
        float acc = b[i][c];
#pragma unroll
        for (int k = 0; k < NS; ++k) acc = fmaf(A[i][k][c], e.b[k][c], acc);
        r.b[i][c] = acc;
      }
    }
    *this = r;
  }

  // this <- (J, r) o this, in place: A = J A, b = J b + r
  __device__ __forceinline__ void pre(const float (&J)[NS][NS][C], const float (&r)[NS][C]) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float nA[NS][NS], nb[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          float a2 = J[i][0][c] * A[0][j][c];
#pragma unroll
          for (int k = 1; k < NS; ++k) a2 = fmaf(J[i][k][c], A[k][j][c], a2);
          nA[i][j] = a2;
        }
        float b2 = r[i][c];
#pragma unroll
        for (int k = 0; k < NS; ++k) b2 = fmaf(J[i][k][c], b[k][c], b2);
        nb[i] = b2;
      }
#pragma unroll
      for (int i = 0; i < NS; ++i) {
#pragma unroll
        for (int j = 0; j < NS; ++j) A[i][j][c] = nA[i][j];
        b[i][c] = nb[i];
      }
    }
  }

  // y = A x + b on vectors x[NS][C]
  __device__ __forceinline__ void apply(float (&x)[NS][C]) const {
    float y[NS][C];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        float acc = b[i][c];
#pragma unroll
        for (int k = 0; k < NS; ++k) acc = fmaf(A[i][k][c], x[k][c], acc);
        y[i][c] = acc;
      }
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int i = 0; i < NS; ++i) x[i][c] = y[i][c];
  }

  // wave shuffle: value of the lane `delta` below (same value kept on lanes < delta)
  __device__ __forceinline__ Aff shfl_up(int delta) const {
    Aff r;
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int c = 0; c < C; ++c) {
#pragma unroll
        for (int j = 0; j < NS; ++j) r.A[i][j][c] = __shfl_up(A[i][j][c], delta, 64);
        r.b[i][c] = __shfl_up(b[i][c], delta, 64);
      }
    return r;
  }
};

}  // namespace pararnn
