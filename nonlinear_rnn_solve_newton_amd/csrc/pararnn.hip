// pararnn.hip -- host side of the C ABI declared in include/pararnn.h:
// argument validation, launch-configuration choice, workspace carving and the
// launch sequence (workspace reset, then one fused launch per Newton iteration,
// or one adjoint launch), all asynchronous on the caller's stream.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/pararnn.h"
#include "adjoint.h"
#include "newton_fused.h"
#include "newton_iter.h"
#include "scan.h"
#include "scan_dense.h"

namespace pararnn {
namespace {

// ---------------------------------------------------------------------------
// Launch configurations. Per (cell, C, operation): T timesteps per lane, W
// waves per workgroup, LL lane groups along L per wave, OCC the waves per SIMD
// the register allocation must allow; a workgroup covers (64/LL)*C channels x
// W*LL*T timesteps (one chunk of the look-back). The
// LSTM keeps one channel per lane (six scan values per channel).
template <class Cell, int C, bool ADJ>
struct Cfg;
template <> struct Cfg<GruCell, 2, false> { static constexpr int T = 16, W = 4, LL = 2, OCC = 3; };
template <> struct Cfg<GruCell, 1, false> { static constexpr int T = 32, W = 4, LL = 1, OCC = 3; };
template <> struct Cfg<LstmCell, 1, false> { static constexpr int T = 24, W = 4, LL = 1, OCC = 2; };
template <> struct Cfg<GruCell, 2, true> { static constexpr int T = 8, W = 4, LL = 2, OCC = 2; };
template <> struct Cfg<GruCell, 1, true> { static constexpr int T = 8, W = 8, LL = 2, OCC = 2; };
template <> struct Cfg<LstmCell, 1, true> { static constexpr int T = 9, W = 4, LL = 1, OCC = 3; };
// All K iterations in one launch (newton_fused.h): the iterate stays in
// registers between iterations; UMODE says where the gate inputs stay (1:
// registers, 2: workgroup memory as read, 3: workgroup memory widened and
// pre-scaled for the exponentials).
template <class Cell, int C>
struct FusedCfg;
template <> struct FusedCfg<GruCell, 2> { static constexpr int T = 16, W = 4, LL = 4, OCC = 3; static constexpr int UMODE = 2; };
template <> struct FusedCfg<GruCell, 1> { static constexpr int T = 16, W = 4, LL = 1, OCC = 2; static constexpr int UMODE = 1; };
template <> struct FusedCfg<LstmCell, 1> { static constexpr int T = 11, W = 4, LL = 2, OCC = 3; static constexpr int UMODE = 3; };
// Problems that would give the shapes above only a few workgroups (under
// half as many as the GPU has CUs) are latency-bound: short lanes over narrow
// channel tiles let more workgroups share the steps (the two-channel GRU and
// the LSTM; both measured faster up to 96 regular workgroups, and slower from
// 168 to 192 on).
template <class Cell, int C>
struct FusedSmallCfg;
template <> struct FusedSmallCfg<GruCell, 2> { static constexpr int T = 4, W = 4, LL = 8, OCC = 3; static constexpr int UMODE = 2; };
template <> struct FusedSmallCfg<LstmCell, 1> { static constexpr int T = 4, W = 4, LL = 8, OCC = 3; static constexpr int UMODE = 3; };
constexpr long long kSmallGrid = 128;  // workgroups of the regular shape below which the small one is used

// Iteration 1 (no state input, lighter cell form): same chunk length and
// channel tile, its own split into waves and steps.
template <class Cell, int C>
struct CfgFirst : Cfg<Cell, C, false> {};

// widest channel group per lane. Newton iteration: the GRU runs two channels
// per lane, the LSTM one (its per-step 2x2 Jacobian, residual and previous
// iterate leave no registers for more); adjoint: GRU two, LSTM one (wider
// groups either spill or need so few steps per lane that the per-lane scan
// overhead outweighs the wider loads).
template <class Cell, bool ADJ> constexpr int max_c() { return Cell::NS == 2 ? 1 : 2; }

// The linear scan alone: NS state components per channel (1: diagonal, 2:
// 2x2 blocks), C channels per lane. The scan streams 8 (NS = 1) or 24
// (NS = 2) bytes of coefficients per step and channel and does a few FMAs.
template <int NS, int C>
struct ScanCfg;
template <> struct ScanCfg<1, 4> { static constexpr int T = 16, W = 8, LL = 1, OCC = 2; };
template <> struct ScanCfg<1, 2> { static constexpr int T = 16, W = 4, LL = 2, OCC = 4; };
template <> struct ScanCfg<1, 1> { static constexpr int T = 16, W = 4, LL = 1, OCC = 4; };
template <> struct ScanCfg<2, 2> { static constexpr int T = 8, W = 8, LL = 1, OCC = 2; };
template <> struct ScanCfg<2, 1> { static constexpr int T = 16, W = 4, LL = 1, OCC = 3; };
template <int NS> constexpr int scan_max_c() { return NS == 1 ? 4 : 2; }

bool is_scan(int op) { return op == PARARNN_OP_SCAN_DIAG || op == PARARNN_OP_SCAN_BLOCK2; }
int scan_ns(int op) { return op == PARARNN_OP_SCAN_BLOCK2 ? 2 : 1; }

// workgroup footprint of one configuration: timesteps (one look-back chunk)
// and channels
struct Geo {
  int chunk, cw;
  int pm = 1;  // partial row maxima per workgroup
};

template <int NS, int C>
constexpr Geo scan_geo() {
  using K = ScanCfg<NS, C>;
  return Geo{K::T * K::W * K::LL, (64 / K::LL) * C};
}

template <int NS>
Geo scan_geo_for_c(int C) {
  if constexpr (scan_max_c<NS>() >= 4) {
    if (C == 4) return scan_geo<NS, 4>();
  }
  if (C == 2) return scan_geo<NS, 2>();
  return scan_geo<NS, 1>();
}

template <class Cell, int C, bool ADJ>
constexpr Geo geo() {
  using K = Cfg<Cell, C, ADJ>;
  return Geo{K::T * K::W * K::LL, (64 / K::LL) * C};
}

template <class Cell, bool ADJ>
Geo geo_for_c(int C) {
  if constexpr (max_c<Cell, ADJ>() >= 4) {
    if (C == 4) return geo<Cell, 4, ADJ>();
  }
  if constexpr (max_c<Cell, ADJ>() >= 2) {
    if (C == 2) return geo<Cell, 2, ADJ>();
  }
  return geo<Cell, 1, ADJ>();
}

template <class K, int C>
constexpr Geo fused_geo_of() {
  return Geo{K::T * K::W * K::LL, (64 / K::LL) * C, K::W};
}

template <class Cell>
Geo fused_geo_for_c(int C) {
  if constexpr (max_c<Cell, false>() >= 2) {
    if (C == 2) return fused_geo_of<FusedCfg<Cell, 2>, 2>();
  }
  return fused_geo_of<FusedCfg<Cell, 1>, 1>();
}

long long ceil_div(long long a, long long b);

// whether a fused solve runs the small-problem shape: the two-channel GRU and
// the LSTM, when the regular shape would launch only a few workgroups
bool fused_small(int cell, int C, const pararnn_opts* o) {
  const bool lstm = cell == PARARNN_LSTM;
  if (lstm ? C != 1 : C != 2) return false;
  const Geo g = lstm ? fused_geo_for_c<LstmCell>(1) : fused_geo_for_c<GruCell>(2);
  return static_cast<long long>(o->B) * ceil_div(o->D, g.cw) * ceil_div(o->L, g.chunk) < kSmallGrid;
}

Geo fused_geo_for(int cell, int C, const pararnn_opts* o) {
  if (fused_small(cell, C, o))
    return cell == PARARNN_LSTM ? fused_geo_of<FusedSmallCfg<LstmCell, 1>, 1>()
                                : fused_geo_of<FusedSmallCfg<GruCell, 2>, 2>();
  return cell == PARARNN_LSTM ? fused_geo_for_c<LstmCell>(C) : fused_geo_for_c<GruCell>(C);
}

Geo geo_for(int cell, int op, int C) {
  if (is_scan(op)) return scan_ns(op) == 2 ? scan_geo_for_c<2>(C) : scan_geo_for_c<1>(C);
  const bool adj = op == PARARNN_OP_ADJOINT;
  if (cell == PARARNN_LSTM) return adj ? geo_for_c<LstmCell, true>(C) : geo_for_c<LstmCell, false>(C);
  return adj ? geo_for_c<GruCell, true>(C) : geo_for_c<GruCell, false>(C);
}

int cmax_for(int cell, int op) {
  if (is_scan(op)) return scan_ns(op) == 2 ? scan_max_c<2>() : scan_max_c<1>();
  const bool adj = op == PARARNN_OP_ADJOINT;
  if (cell == PARARNN_LSTM) return adj ? max_c<LstmCell, true>() : max_c<LstmCell, false>();
  return adj ? max_c<GruCell, true>() : max_c<GruCell, false>();
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t ctr = 0, maxupd = 0, pmax = 0, incl = 0, agg = 0, dapart = 0, zero_end = 0, state = 0, total = 0;
  int nchunks = 0, ntiles_d = 0;
};

int nstate(int cell) { return cell == PARARNN_LSTM ? 2 : 1; }
int ngates(int cell) { return cell == PARARNN_LSTM ? 4 : 3; }

// ceil(a / b) for positive a, b without overflow
long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

bool opts_ok(int cell, int op, const pararnn_opts* o) {
  if (!o) return false;
  if (op == PARARNN_OP_SCAN_DENSE)  // the dense scan has no cell; D is the state size
    return o->B >= 1 && o->L >= 1 && o->D >= 1 && o->D <= kDenseMaxN &&
           static_cast<double>(o->B) * ceil_div(o->L, kDenseChunk) < 2.0e9;
  if (op != PARARNN_OP_SOLVE && op != PARARNN_OP_ADJOINT && !is_scan(op)) return false;
  if (!is_scan(op) && cell != PARARNN_GRU && cell != PARARNN_LSTM) return false;  // the scan has no cell
  if (o->B < 1 || o->L < 1 || o->D < 1) return false;
  if (op == PARARNN_OP_SOLVE && (o->max_iters < 1 || o->max_iters > 1000)) return false;
  if (op == PARARNN_OP_SOLVE &&
      (o->schedule < PARARNN_SCHEDULE_AUTO || o->schedule > PARARNN_SCHEDULE_PER_ITERATION ||
       (o->schedule == PARARNN_SCHEDULE_FUSED && o->early_exit)))
    return false;
  // element counts must stay addressable with 64-bit offsets and tickets in 32 bits
  const double n = static_cast<double>(o->B) * o->L * o->D * 4;
  if (n > 9.0e18) return false;
  for (int C = 1; C <= cmax_for(cell, op); C *= 2) {
    // both schedules of the solve: the per-iteration and the fused geometry
    for (int fused = 0; fused <= (op == PARARNN_OP_SOLVE ? 1 : 0); ++fused) {
      const Geo g = fused ? fused_geo_for(cell, C, o) : geo_for(cell, op, C);
      const double wgs = static_cast<double>(o->B) * ceil_div(o->D, g.cw) * ceil_div(o->L, g.chunk);
      if (wgs > 2.0e9) return false;
    }
  }
  return true;
}

// Workspace: [counters | row maxima | incl descriptors | agg descriptors | da partials]
// (cleared at the start of every call) followed by the ping-pong state buffer.
// fused: the one-launch schedule of the solve (descriptor slots for every
// iteration, no state buffer)
Layout layout(int cell, int op, const pararnn_opts* o, bool with_da, Geo g, bool fused = false) {
  Layout y;
  const int NS = is_scan(op) ? scan_ns(op) : nstate(cell), G = ngates(cell);
  const size_t B = o->B, L = o->L, D = o->D;
  const int K = (op == PARARNN_OP_SOLVE) ? o->max_iters : 1;
  y.nchunks = static_cast<int>((L + g.chunk - 1) / g.chunk);
  y.ntiles_d = static_cast<int>((D + g.cw - 1) / g.cw);
  const size_t nwg = B * static_cast<size_t>(y.ntiles_d) * y.nchunks;
  size_t off = 0;
  y.ctr = off;
  off = round_up(off + sizeof(uint32_t) * K);
  y.maxupd = off;
  off = round_up(off + sizeof(uint32_t) * static_cast<size_t>(K) * B);
  y.pmax = off;
  if (op == PARARNN_OP_SOLVE) off = round_up(off + sizeof(uint32_t) * static_cast<size_t>(K) * nwg * g.pm);
  y.incl = off;
  const size_t slots = B * static_cast<size_t>(y.ntiles_d) * g.cw;  // descriptor slots per component
  const size_t nk = fused ? static_cast<size_t>(K) : 1;  // descriptor sets
  // the fused kernel reads a descriptor slot in every workgroup, a single
  // chunk included
  if (y.nchunks > 1 || fused) off = round_up(off + sizeof(uint64_t) * nk * y.nchunks * NS * slots);
  y.agg = off;
  if (y.nchunks > 1) off = round_up(off + sizeof(uint64_t) * nk * y.nchunks * (NS * NS + NS) * slots);
  y.zero_end = off;
  y.dapart = off;
  if (op == PARARNN_OP_ADJOINT && with_da) off = round_up(off + sizeof(float) * y.nchunks * B * G * D);
  y.state = off;
  if (op == PARARNN_OP_SOLVE && K >= 2 && !fused) off = round_up(off + sizeof(float) * NS * B * L * D);
  y.total = off;
  return y;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// widest channel group C in {4, 2, 1} (at most cmax) that divides D and keeps
// every pointer aligned
int pick_c(int cmax, int D, size_t usize, const void* u, std::initializer_list<const void*> f32ptrs) {
  for (int C : {4, 2, 1}) {
    if (C > cmax || D % C) continue;
    bool ok = aligned(u, usize * C);
    for (const void* q : f32ptrs)
      if (q && !aligned(q, sizeof(float) * C)) ok = false;
    if (ok) return C;
  }
  return 0;
}

int check_hip(hipError_t e) { return e == hipSuccess ? PARARNN_OK : PARARNN_EHIP; }

int record(const pararnn_opts* o, int i, hipStream_t s) {
  if (!o->events || !o->events[i]) return PARARNN_OK;
  return check_hip(hipEventRecord(static_cast<hipEvent_t>(o->events[i]), s));
}

// Caller events that a kernel's own dispatch stamps at its start and end. A
// marker recorded between two kernels adds its own barrier to the interval
// it bounds (about 20 us on a 150 us launch); a stamp from the dispatch is
// the kernel's execution alone.
struct Stamps {
  hipEvent_t start = nullptr, stop = nullptr;
};
Stamps stamps(const pararnn_opts* o, int start, int stop) {
  Stamps t;
  if (o->events) {
    if (start >= 0) t.start = static_cast<hipEvent_t>(o->events[start]);
    if (stop >= 0) t.stop = static_cast<hipEvent_t>(o->events[stop]);
  }
  return t;
}

template <typename F, typename... Args>
int launch(F kernel, dim3 grid, dim3 block, hipStream_t s, Stamps t, Args... args) {
  if (t.start || t.stop) hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t.start, t.stop, 0, args...);
  else hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return check_hip(hipGetLastError());
}

int clear_ws(char* ws, const Layout& y, float* user, long long nuser, hipStream_t s) {
  const long long n16 = static_cast<long long>(y.zero_end / 16);
  const long long work = n16 > nuser ? n16 : nuser;
  long long blocks = (work + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(ws_clear_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     reinterpret_cast<f32x4*>(ws), n16, user, nuser);
  return check_hip(hipGetLastError());
}

template <class Cell, class UT, int C, bool INCL>
int launch_iter(const IterArgs& a, hipStream_t s, Stamps t) {
  using K = Cfg<Cell, C, false>;
  using K1 = CfgFirst<Cell, C>;
  static_assert(K1::W * K1::LL * K1::T == K::W * K::LL * K::T && K1::LL == K::LL,
                "iteration 1 shares the chunk length and channel tile of the later iterations");
  const unsigned grid = static_cast<unsigned>(a.B) * a.ntiles_d * static_cast<unsigned>(a.nchunks);
  const IterArgs& b = a;
  if (a.k == 1)  // iteration 1 starts from the zero iterate and reads no state
    return launch(newton_iter_kernel<Cell, UT, C, K1::T, K1::W, K1::LL, K1::OCC, true, INCL>, dim3(grid),
                  dim3(64 * K1::W), s, t, b);
  return launch(newton_iter_kernel<Cell, UT, C, K::T, K::W, K::LL, K::OCC, false, INCL>, dim3(grid),
                dim3(64 * K::W), s, t, b);
}

template <class Cell, class UT>
int launch_iter_c(int C, bool incl, const IterArgs& a, hipStream_t s, Stamps t) {
  if constexpr (max_c<Cell, false>() >= 4) {
    if (C == 4) return incl ? launch_iter<Cell, UT, 4, true>(a, s, t) : launch_iter<Cell, UT, 4, false>(a, s, t);
  }
  if constexpr (max_c<Cell, false>() >= 2) {
    if (C == 2) return incl ? launch_iter<Cell, UT, 2, true>(a, s, t) : launch_iter<Cell, UT, 2, false>(a, s, t);
  }
  return incl ? launch_iter<Cell, UT, 1, true>(a, s, t) : launch_iter<Cell, UT, 1, false>(a, s, t);
}

template <class Cell>
int launch_iter_any(int dtype, int C, bool incl, const IterArgs& a, hipStream_t s, Stamps t) {
  return dtype == PARARNN_BF16 ? launch_iter_c<Cell, bf16>(C, incl, a, s, t)
                               : launch_iter_c<Cell, float>(C, incl, a, s, t);
}

template <class Cell, class UT, int C, bool INCL>
int launch_adj(const AdjArgs& a, hipStream_t s, Stamps t) {
  using K = Cfg<Cell, C, true>;
  const unsigned grid = static_cast<unsigned>(a.B) * a.ntiles_d * static_cast<unsigned>(a.nchunks);
  const AdjArgs& b = a;
  return launch(adjoint_kernel<Cell, UT, C, K::T, K::W, K::LL, K::OCC, INCL>, dim3(grid), dim3(64 * K::W), s, t,
                b);
}

template <class Cell, class UT>
int launch_adj_c(int C, bool incl, const AdjArgs& a, hipStream_t s, Stamps t) {
  if constexpr (max_c<Cell, true>() >= 4) {
    if (C == 4) return incl ? launch_adj<Cell, UT, 4, true>(a, s, t) : launch_adj<Cell, UT, 4, false>(a, s, t);
  }
  if constexpr (max_c<Cell, true>() >= 2) {
    if (C == 2) return incl ? launch_adj<Cell, UT, 2, true>(a, s, t) : launch_adj<Cell, UT, 2, false>(a, s, t);
  }
  return incl ? launch_adj<Cell, UT, 1, true>(a, s, t) : launch_adj<Cell, UT, 1, false>(a, s, t);
}

template <class Cell>
int launch_adj_any(int dtype, int C, bool incl, const AdjArgs& a, hipStream_t s, Stamps t) {
  return dtype == PARARNN_BF16 ? launch_adj_c<Cell, bf16>(C, incl, a, s, t)
                               : launch_adj_c<Cell, float>(C, incl, a, s, t);
}

// The per-iteration Newton kernel's and the adjoint's chunk carry from the
// neighbouring chunk's inclusive carry alone where a chunk row has at least
// this many tiles (see kInclOnlyTiles for the fused kernel). Same-box
// measurements, inclusive only against look-back:
//   tiles per row              16      32      64      128 and more
//   per-iteration solve, GRU   +88%    +31%    +4%     -3%
//   per-iteration solve, LSTM                  -4.5%   -5%
//   adjoint, GRU               +80%    +25%    0%      -4%
//   adjoint, LSTM              +49%    +13%    -6%     -5.5%
long long iter_incl_tiles(int cell) { return cell == PARARNN_LSTM ? 64 : 128; }

template <int NS, int C>
int launch_scan(bool incl, const ScanArgs& a, hipStream_t s, Stamps t) {
  using K = ScanCfg<NS, C>;
  const unsigned grid = static_cast<unsigned>(a.B) * a.ntiles_d * static_cast<unsigned>(a.nchunks);
  const ScanArgs& b = a;
  if (incl)
    return launch(scan_kernel<NS, C, K::T, K::W, K::LL, K::OCC, true>, dim3(grid), dim3(64 * K::W), s, t, b);
  return launch(scan_kernel<NS, C, K::T, K::W, K::LL, K::OCC, false>, dim3(grid), dim3(64 * K::W), s, t, b);
}

// The scan's chunk carry from the predecessor's inclusive carry alone where a
// chunk row has at least this many tiles (see kInclOnlyTiles for the fused
// kernel). Same-box measurements, scan time, inclusive only against
// look-back, B = 1..8, D = 1024:
//   tiles per row   8        16       32       64
//   diagonal        +60%     +4.6%    -5.5%
//   2x2 blocks      +151%    +46%     -6.5%    -8%
constexpr long long kScanInclTiles = 32;

// The fused kernel's two ways to the chunk carry when the early read misses.
// Look-back: publish the chunk aggregate and compose predecessors' aggregates
// back to an inclusive carry. Inclusive only: wait for the predecessor's
// inclusive carry. Tickets are chunk-major, so a predecessor is one chunk row
// (B * ntiles_d tickets) ahead. With many tiles per row it runs well ahead and
// the plain wait is cheaper: it skips the aggregate code (about 16 VGPRs) and
// the reset of the aggregate descriptors. With few tiles, many chunk rows run
// at once and the look-back's shortcut through aggregates wins. Same-box
// measurements, fused solve time, inclusive only against look-back:
//   tiles per row   16          32          64            256
//   GRU             +33%        +2%         -4.5%         -5.6%
//   LSTM            +56%        +15%        -13%          -4.7%
constexpr long long kInclOnlyTiles = 64;

// The carry mode of a launch: inclusive only (the chunk waits for its
// neighbour's inclusive carry) where a chunk row has at least the family's
// threshold of tiles, else the decoupled look-back.
bool incl_only_for(int cell, int op, bool fused, long long tiles_per_row) {
  if (is_scan(op)) return tiles_per_row >= kScanInclTiles;
  if (op == PARARNN_OP_SOLVE && fused) return tiles_per_row >= kInclOnlyTiles;
  return tiles_per_row >= iter_incl_tiles(cell);
}

int scan(int ns, const float* A, const float* b, const float* s0, float* s, void* ws, size_t ws_bytes,
         const pararnn_opts* o, hipStream_t stream) {
  const int op = ns == 2 ? PARARNN_OP_SCAN_BLOCK2 : PARARNN_OP_SCAN_DIAG;
  if (!opts_ok(PARARNN_GRU, op, o)) return PARARNN_EINVAL;
  if (!A || !b || !s || !ws) return PARARNN_EINVAL;
  const int C = pick_c(cmax_for(PARARNN_GRU, op), o->D, sizeof(float), A, {b, s0, s});
  if (!C) return PARARNN_EUNSUPPORTED;
  const Geo g = geo_for(PARARNN_GRU, op, C);
  // one chunk of a plane is addressed with 32-bit offsets below 2^31
  if (static_cast<double>(g.chunk) * o->D * 4.0 >= 2147483648.0) return PARARNN_EUNSUPPORTED;
  const Layout y = layout(PARARNN_GRU, op, o, false, g);
  if (ws_bytes < y.total) return PARARNN_EWORKSPACE;
  if (!aligned(ws, kAlign)) return PARARNN_EUNSUPPORTED;
  char* w = static_cast<char*>(ws);

  const bool incl_only = incl_only_for(PARARNN_GRU, op, false, static_cast<long long>(o->B) * y.ntiles_d);
  Layout yc = y;  // inclusive only: the aggregate descriptors are never read
  if (incl_only) yc.zero_end = y.agg;
  int rc = record(o, 0, stream);
  if (rc) return rc;
  rc = clear_ws(w, yc, nullptr, 0, stream);
  if (rc) return rc;
  ScanArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.A = A;
  sa.b = b;
  sa.s0 = s0;
  sa.s = s;
  sa.incl = reinterpret_cast<unsigned long long*>(w + y.incl);
  sa.agg = reinterpret_cast<unsigned long long*>(w + y.agg);
  sa.ctr = reinterpret_cast<unsigned int*>(w + y.ctr);
  sa.B = o->B;
  sa.L = o->L;
  sa.D = o->D;
  sa.nchunks = y.nchunks;
  sa.ntiles_d = y.ntiles_d;
  const Stamps t = stamps(o, 1, 2);
  if (ns == 2)
    return C == 2 ? launch_scan<2, 2>(incl_only, sa, stream, t) : launch_scan<2, 1>(incl_only, sa, stream, t);
  return C == 4   ? launch_scan<1, 4>(incl_only, sa, stream, t)
         : C == 2 ? launch_scan<1, 2>(incl_only, sa, stream, t)
                  : launch_scan<1, 1>(incl_only, sa, stream, t);
}

bool use_fused(const pararnn_opts* o) {
  return o->schedule == PARARNN_SCHEDULE_FUSED || (o->schedule == PARARNN_SCHEDULE_AUTO && !o->early_exit);
}

template <class K, class Cell, class UT, int C, bool INCL>
int launch_fused(const FusedArgs& a, hipStream_t s, Stamps t) {
  // gate inputs in workgroup memory (UMODE 2) unless they would take more than
  // 64 KB of it there (fp32 inputs in the regular shapes): stream them instead
  constexpr int USEG = (64 / K::LL) * C;
  constexpr size_t ULDS = static_cast<size_t>(K::W) * K::LL * (K::T * Cell::G * USEG + USEG) * sizeof(UT);
  constexpr int UM = (K::UMODE == 2 && ULDS > 65536) ? 0 : K::UMODE;
  const unsigned grid = static_cast<unsigned>(a.B) * a.ntiles_d * static_cast<unsigned>(a.nchunks);
  const FusedArgs& b = a;
  return launch(newton_fused_kernel<Cell, UT, C, K::T, K::W, K::LL, K::OCC, UM, INCL>, dim3(grid),
                dim3(64 * K::W), s, t, b);
}

template <class K, class Cell, class UT, int C>
int launch_fused_mode(bool incl, const FusedArgs& a, hipStream_t s, Stamps t) {
  return incl ? launch_fused<K, Cell, UT, C, true>(a, s, t) : launch_fused<K, Cell, UT, C, false>(a, s, t);
}

template <class Cell, class UT>
int launch_fused_c(int C, bool small, bool incl, const FusedArgs& a, hipStream_t s, Stamps t) {
  if constexpr (max_c<Cell, false>() >= 2) {
    if (C == 2) {
      if constexpr (Cell::NS == 1) {
        if (small) return launch_fused_mode<FusedSmallCfg<Cell, 2>, Cell, UT, 2>(incl, a, s, t);
      }
      return launch_fused_mode<FusedCfg<Cell, 2>, Cell, UT, 2>(incl, a, s, t);
    }
  }
  if constexpr (Cell::NS == 2) {
    if (small) return launch_fused_mode<FusedSmallCfg<Cell, 1>, Cell, UT, 1>(incl, a, s, t);
  }
  return launch_fused_mode<FusedCfg<Cell, 1>, Cell, UT, 1>(incl, a, s, t);
}

template <class Cell>
int launch_fused_any(int dtype, int C, bool small, bool incl, const FusedArgs& a, hipStream_t s, Stamps t) {
  return dtype == PARARNN_BF16 ? launch_fused_c<Cell, bf16>(C, small, incl, a, s, t)
                               : launch_fused_c<Cell, float>(C, small, incl, a, s, t);
}


// The launch plan of a solve call: the channel group its pointers allow, the
// schedule, the launch shape and the workspace layout. Returns the status the
// call gives before any launch (every check that needs no workspace).
struct SolvePlan {
  int C = 0;
  bool fused = false;
  Geo g{};
  Layout y{};
};
int solve_plan(int cell, const void* u, const float* a, const float* c0, const float* h0, const float* c,
               const float* h, const pararnn_opts* o, SolvePlan* sp) {
  if (!opts_ok(cell, PARARNN_OP_SOLVE, o)) return PARARNN_EINVAL;
  if (!u || !a || !h || (cell == PARARNN_LSTM && !c)) return PARARNN_EINVAL;
  if (o->u_dtype != PARARNN_F32 && o->u_dtype != PARARNN_BF16) return PARARNN_EUNSUPPORTED;
  if (o->early_exit != 0 && o->early_exit != 1) return PARARNN_EINVAL;
  const size_t usize = o->u_dtype == PARARNN_BF16 ? 2 : 4;
  sp->C = pick_c(cmax_for(cell, PARARNN_OP_SOLVE), o->D, usize, u, {a, h0, h, c0, c});
  if (!sp->C || !aligned(u, usize)) return PARARNN_EUNSUPPORTED;
  sp->fused = use_fused(o);
  sp->g = sp->fused ? fused_geo_for(cell, sp->C, o) : geo_for(cell, PARARNN_OP_SOLVE, sp->C);
  // one chunk of gate inputs (and of states) is addressed with 32-bit offsets below 2^31
  if (static_cast<double>(sp->g.chunk) * ngates(cell) * o->D * 4.0 >= 2147483648.0) return PARARNN_EUNSUPPORTED;
  sp->y = layout(cell, PARARNN_OP_SOLVE, o, false, sp->g, sp->fused);
  return PARARNN_OK;
}

int solve(int cell, const void* u, const float* a, const float* c0, const float* h0, float* c, float* h,
          void* ws, size_t ws_bytes, const pararnn_opts* o, int32_t* iters, int32_t* converged,
          float* max_update, hipStream_t stream) {
  SolvePlan sp;
  const int prc = solve_plan(cell, u, a, c0, h0, c, h, o, &sp);
  if (prc) return prc;
  if (!ws) return PARARNN_EINVAL;
  const int C = sp.C;
  const bool fused = sp.fused;
  const Geo g = sp.g;
  const Layout y = sp.y;
  if (ws_bytes < y.total) return PARARNN_EWORKSPACE;
  if (!aligned(ws, kAlign)) return PARARNN_EUNSUPPORTED;

  const int K = o->max_iters, NS = nstate(cell);
  if (fused) {
    const bool incl_only = incl_only_for(cell, PARARNN_OP_SOLVE, true, static_cast<long long>(o->B) * y.ntiles_d);
    Layout yc = y;  // inclusive only: the aggregate descriptors are never read
    if (incl_only) yc.zero_end = y.agg;
    int rc = record(o, 0, stream);
    if (rc) return rc;
    rc = clear_ws(static_cast<char*>(ws), yc, nullptr, 0, stream);
    if (rc) return rc;
    char* w = static_cast<char*>(ws);
    FusedArgs fa;
    memset(&fa, 0, sizeof(fa));
    fa.u = u;
    fa.a = a;
    fa.s0[0] = cell == PARARNN_LSTM ? c0 : h0;
    fa.s0[1] = cell == PARARNN_LSTM ? h0 : nullptr;
    fa.sout[0] = cell == PARARNN_LSTM ? c : h;
    fa.sout[1] = cell == PARARNN_LSTM ? h : nullptr;
    fa.incl = reinterpret_cast<unsigned long long*>(w + y.incl);
    fa.agg = reinterpret_cast<unsigned long long*>(w + y.agg);
    fa.ctr = reinterpret_cast<unsigned int*>(w + y.ctr);
    fa.pmax = reinterpret_cast<unsigned int*>(w + y.pmax);
    fa.B = o->B;
    fa.L = o->L;
    fa.D = o->D;
    fa.K = K;
    fa.nchunks = y.nchunks;
    fa.ntiles_d = y.ntiles_d;
    // the one launch stamps events 1 and 2; iterations 2..K end with it
    const Stamps t = stamps(o, 1, 2);
    const bool small = fused_small(cell, C, o);
    rc = (cell == PARARNN_LSTM) ? launch_fused_any<LstmCell>(o->u_dtype, C, small, incl_only, fa, stream, t)
                                : launch_fused_any<GruCell>(o->u_dtype, C, small, incl_only, fa, stream, t);
    if (rc) return rc;
    for (int k = 2; k <= K; ++k) {
      rc = record(o, k + 1, stream);
      if (rc) return rc;
    }
    hipLaunchKernelGGL(newton_finalize_kernel, dim3(o->B, K), dim3(kRowmaxThreads), 0, stream,
                       static_cast<const unsigned int*>(fa.pmax), reinterpret_cast<unsigned int*>(w + y.maxupd),
                       o->B, y.ntiles_d * g.pm, y.nchunks, K, o->tol, 0, iters, converged, max_update);
    return check_hip(hipGetLastError());
  }
  const size_t BLD = static_cast<size_t>(o->B) * o->L * o->D;
  char* w = static_cast<char*>(ws);
  float* buf = reinterpret_cast<float*>(w + y.state);
  float* out[2] = {cell == PARARNN_LSTM ? c : h, cell == PARARNN_LSTM ? h : nullptr};
  float* alt[2] = {buf, NS == 2 ? buf + BLD : nullptr};

  int rc = record(o, 0, stream);
  if (rc) return rc;
  const bool incl_only = incl_only_for(cell, PARARNN_OP_SOLVE, false, static_cast<long long>(o->B) * y.ntiles_d);
  Layout yc = y;  // inclusive only: the aggregate descriptors are never read
  if (incl_only) yc.zero_end = y.agg;
  rc = clear_ws(w, yc, nullptr, 0, stream);
  if (rc) return rc;

  IterArgs ia;
  memset(&ia, 0, sizeof(ia));
  ia.u = u;
  ia.a = a;
  ia.s0[0] = cell == PARARNN_LSTM ? c0 : h0;
  ia.s0[1] = cell == PARARNN_LSTM ? h0 : nullptr;
  ia.incl = reinterpret_cast<unsigned long long*>(w + y.incl);
  ia.agg = reinterpret_cast<unsigned long long*>(w + y.agg);
  ia.ctr = reinterpret_cast<unsigned int*>(w + y.ctr);
  ia.maxupd = reinterpret_cast<unsigned int*>(w + y.maxupd);
  ia.pmax = reinterpret_cast<unsigned int*>(w + y.pmax);
  ia.ntiles_d = y.ntiles_d;
  ia.B = o->B;
  ia.L = o->L;
  ia.D = o->D;
  ia.K = K;
  ia.nchunks = y.nchunks;
  ia.early_exit = o->early_exit;
  ia.tol = o->tol;
  // ping-pong so that iterate K lands in the caller's output
  for (int k = 1; k <= K; ++k) {
    const bool k_in_out = ((K - k) % 2) == 0;
    for (int s = 0; s < NS; ++s) {
      ia.sout[s] = k_in_out ? out[s] : alt[s];
      ia.sin[s] = (k == 1) ? nullptr : (k_in_out ? alt[s] : out[s]);
    }
    ia.k = k;
    // launch k stamps event k + 1 at its end (and launch 1 event 1 at its start)
    const Stamps t = stamps(o, k == 1 ? 1 : -1, k + 1);
    rc = (cell == PARARNN_LSTM) ? launch_iter_any<LstmCell>(o->u_dtype, C, incl_only, ia, stream, t)
                                : launch_iter_any<GruCell>(o->u_dtype, C, incl_only, ia, stream, t);
    if (rc) return rc;
    if (o->early_exit) {  // the next launch decides from this launch's row maxima
      hipLaunchKernelGGL(rowmax_kernel, dim3(o->B), dim3(kRowmaxThreads), 0, stream, ia.pmax, ia.maxupd, o->B, y.ntiles_d,
                         y.nchunks, k - 1);
      rc = check_hip(hipGetLastError());
      if (rc) return rc;
    }
  }
  hipLaunchKernelGGL(newton_finalize_kernel, dim3(o->B, K), dim3(kRowmaxThreads), 0, stream,
                     static_cast<const unsigned int*>(ia.pmax), ia.maxupd, o->B, y.ntiles_d, y.nchunks, K, o->tol,
                     o->early_exit, iters, converged, max_update);
  return check_hip(hipGetLastError());
}

// Dense scan workspace: chunk transfers [B][nchunks][32][32], local solutions
// and carries [B][nchunks][32] each (nothing to clear: every entry is written
// before it is read)
struct DenseLayout {
  size_t P = 0, v = 0, carry = 0, Pseg = 0, vseg = 0, total = 0;
  int nchunks = 0;
};

DenseLayout dense_layout(const pararnn_opts* o) {
  DenseLayout y;
  y.nchunks = static_cast<int>(ceil_div(o->L, kDenseChunk));
  const size_t nc = static_cast<size_t>(o->B) * y.nchunks, ns = nc * kDenseWaves;
  y.P = 0;
  y.v = round_up(sizeof(float) * nc * 1024);
  y.carry = round_up(y.v + sizeof(float) * nc * 32);
  y.Pseg = round_up(y.carry + sizeof(float) * nc * 32);
  y.vseg = round_up(y.Pseg + sizeof(float) * ns * 1024);
  y.total = round_up(y.vseg + sizeof(float) * ns * 32);
  return y;
}

int scan_dense(const float* A, const float* b, const float* s0, float* s, void* ws, size_t ws_bytes,
               const pararnn_opts* o, hipStream_t stream) {
  if (!opts_ok(PARARNN_GRU, PARARNN_OP_SCAN_DENSE, o)) return PARARNN_EINVAL;
  if (!A || !b || !s || !ws) return PARARNN_EINVAL;
  for (const void* q : {static_cast<const void*>(A), static_cast<const void*>(b), static_cast<const void*>(s0),
                        static_cast<const void*>(s)})
    if (q && !aligned(q, sizeof(float))) return PARARNN_EUNSUPPORTED;
  const DenseLayout y = dense_layout(o);
  if (ws_bytes < y.total) return PARARNN_EWORKSPACE;
  if (!aligned(ws, kAlign)) return PARARNN_EUNSUPPORTED;
  char* w = static_cast<char*>(ws);
  DenseArgs da;
  da.A = A;
  da.b = b;
  da.s0 = s0;
  da.s = s;
  da.P = reinterpret_cast<float*>(w + y.P);
  da.v = reinterpret_cast<float*>(w + y.v);
  da.carry = reinterpret_cast<float*>(w + y.carry);
  da.Pseg = reinterpret_cast<float*>(w + y.Pseg);
  da.vseg = reinterpret_cast<float*>(w + y.vseg);
  da.B = o->B;
  da.L = o->L;
  da.n = o->D;
  da.nchunks = y.nchunks;
  const unsigned nwg = static_cast<unsigned>(o->B) * static_cast<unsigned>(y.nchunks);
  int rc = record(o, 0, stream);
  if (rc) return rc;
  // n = 32 with 16-byte aligned A reads whole runs of four columns; the first
  // launch stamps event 1 at its start, the last event 2 at its end
  const bool n32 = o->D == 32 && aligned(A, 16);
  rc = n32 ? launch(dense_chunk_kernel<true>, dim3(nwg), dim3(64 * kDenseWaves), stream, stamps(o, 1, -1), da)
           : launch(dense_chunk_kernel<false>, dim3(nwg), dim3(64 * kDenseWaves), stream, stamps(o, 1, -1), da);
  if (rc) return rc;
  hipLaunchKernelGGL(dense_carry_kernel, dim3(static_cast<unsigned>(o->B)), dim3(64 * kDenseCarryWaves), 0, stream, da);
  rc = check_hip(hipGetLastError());
  if (rc) return rc;
  const unsigned nseg = nwg * kDenseWaves;
  return n32 ? launch(dense_apply_kernel<true>, dim3(nseg), dim3(64), stream, stamps(o, -1, 2), da)
             : launch(dense_apply_kernel<false>, dim3(nseg), dim3(64), stream, stamps(o, -1, 2), da);
}

// ---------------------------------------------------------------------------
// Built-in device scratch for callers that cannot allocate (the scratch
// variant of the GRU solve). One array per GPU, reserved when the code object
// is loaded on that GPU and held until the process ends. In host code its name
// is only a host-side handle: the kernels get the device address found by
// hipGetSymbolAddress, kept per device.
constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device of `stream` (the current device
// for the null stream). Looked up once per device, with that device current.
int scratch_ptr(hipStream_t stream, void** out) {
  int dev = 0;
  if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess) return PARARNN_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return PARARNN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return PARARNN_EHIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return PARARNN_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return PARARNN_EHIP;
    if (e != hipSuccess || !p) return PARARNN_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PARARNN_OK;
}

}  // namespace
}  // namespace pararnn

using namespace pararnn;

extern "C" size_t pararnn_workspace_bytes(int32_t cell, int32_t op, const pararnn_opts* o) {
  if (!opts_ok(cell, op, o)) return 0;
  if (op == PARARNN_OP_SCAN_DENSE) return dense_layout(o).total;
  const bool fused = op == PARARNN_OP_SOLVE && use_fused(o);
  size_t n = 0;
  for (int C = 1; C <= cmax_for(cell, op); C *= 2) {
    const Geo g = fused ? fused_geo_for(cell, C, o) : geo_for(cell, op, C);
    const size_t t = layout(cell, op, o, true, g, fused).total;
    n = t > n ? t : n;
  }
  return n;
}

extern "C" int32_t pararnn_scan_diag(const float* A, const float* b, const float* s0, float* s, void* ws,
                                     size_t ws_bytes, const pararnn_opts* o, void* stream) {
  return scan(1, A, b, s0, s, ws, ws_bytes, o, static_cast<hipStream_t>(stream));
}

extern "C" int32_t pararnn_scan_dense(const float* A, const float* b, const float* s0, float* s, void* ws,
                                      size_t ws_bytes, const pararnn_opts* o, void* stream) {
  return scan_dense(A, b, s0, s, ws, ws_bytes, o, static_cast<hipStream_t>(stream));
}

extern "C" int32_t pararnn_scan_block2(const float* A, const float* b, const float* s0, float* s, void* ws,
                                       size_t ws_bytes, const pararnn_opts* o, void* stream) {
  return scan(2, A, b, s0, s, ws, ws_bytes, o, static_cast<hipStream_t>(stream));
}

extern "C" int32_t pararnn_solve_gru(const void* u, const float* a, const float* h0, float* h, void* ws,
                                     size_t ws_bytes, const pararnn_opts* o, int32_t* iters,
                                     int32_t* converged, float* max_update, void* stream) {
  return solve(PARARNN_GRU, u, a, nullptr, h0, nullptr, h, ws, ws_bytes, o, iters, converged, max_update,
               static_cast<hipStream_t>(stream));
}

extern "C" int32_t pararnn_plan_query(int32_t cell, int32_t op, const pararnn_opts* o, pararnn_plan* plan) {
  if (!plan || !opts_ok(cell, op, o)) return PARARNN_EINVAL;
  memset(plan, 0, sizeof(*plan));
  if (op == PARARNN_OP_SCAN_DENSE) {
    const DenseLayout y = dense_layout(o);
    plan->vec = 1;
    plan->chunk = kDenseChunk;
    plan->channels = o->D;
    plan->nchunks = y.nchunks;
    plan->tiles_per_row = o->B;
    plan->inclusive_only = 1;  // the chunk carries run in order, one workgroup per batch row
    return PARARNN_OK;
  }
  const bool fused = op == PARARNN_OP_SOLVE && use_fused(o);
  const bool scanop = is_scan(op);
  const int gcell = scanop ? PARARNN_GRU : cell;  // the scans have no cell
  const size_t usize = (!scanop && o->u_dtype == PARARNN_BF16) ? 2 : 4;
  // every pointer 16-byte aligned: the widest channel group that divides D
  alignas(16) static const char kAligned[16] = {0};
  const int C = pick_c(cmax_for(gcell, op), o->D, usize, kAligned, {});
  const Geo g = fused ? fused_geo_for(cell, C, o) : geo_for(gcell, op, C);
  const Layout y = layout(gcell, op, o, false, g, fused);
  plan->vec = C;
  plan->chunk = g.chunk;
  plan->channels = g.cw;
  plan->nchunks = y.nchunks;
  plan->tiles_per_row = o->B * y.ntiles_d;
  plan->inclusive_only = incl_only_for(gcell, op, fused, static_cast<long long>(o->B) * y.ntiles_d) ? 1 : 0;
  plan->fused = fused ? 1 : 0;
  return PARARNN_OK;
}

extern "C" size_t pararnn_scratch_bytes(void) { return kScratchBytes; }

extern "C" int32_t pararnn_solve_gru_scratch(const void* u, const float* a, const float* h0, float* h,
                                             const pararnn_opts* o, int32_t* iters, int32_t* converged,
                                             float* max_update, void* stream_) {
  // every check that needs no device comes first, so that a rejected call
  // makes no HIP call at all; the workspace needed is that of the launch
  // this call makes (its pointers fix the channel group)
  SolvePlan sp;
  const int prc = solve_plan(PARARNN_GRU, u, a, nullptr, h0, nullptr, h, o, &sp);
  if (prc) return prc;
  if (sp.y.total > kScratchBytes) return PARARNN_ESCRATCH;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  void* ws = nullptr;
  const int rc = scratch_ptr(stream, &ws);
  if (rc) return rc;
  return solve(PARARNN_GRU, u, a, nullptr, h0, nullptr, h, ws, kScratchBytes, o, iters, converged, max_update,
               stream);
}

extern "C" int32_t pararnn_solve_lstm(const void* u, const float* a, const float* c0, const float* h0,
                                      float* c, float* h, void* ws, size_t ws_bytes, const pararnn_opts* o,
                                      int32_t* iters, int32_t* converged, float* max_update, void* stream) {
  return solve(PARARNN_LSTM, u, a, c0, h0, c, h, ws, ws_bytes, o, iters, converged, max_update,
               static_cast<hipStream_t>(stream));
}

extern "C" int32_t pararnn_adjoint(int32_t cell, const void* u, const float* a, const float* c0,
                                   const float* h0, const float* c, const float* h, const float* dh,
                                   float* du, float* ds0, float* da, void* ws, size_t ws_bytes,
                                   const pararnn_opts* o, void* stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!opts_ok(cell, PARARNN_OP_ADJOINT, o)) return PARARNN_EINVAL;
  if (!u || !a || !h || !dh || !du || !ws || (cell == PARARNN_LSTM && !c)) return PARARNN_EINVAL;
  if (o->u_dtype != PARARNN_F32 && o->u_dtype != PARARNN_BF16) return PARARNN_EUNSUPPORTED;
  const size_t usize = o->u_dtype == PARARNN_BF16 ? 2 : 4;
  const bool lstm = cell == PARARNN_LSTM;
  const int C = pick_c(cmax_for(cell, PARARNN_OP_ADJOINT), o->D, usize, u,
                      {a, h0, h, dh, du, ds0, da, lstm ? c0 : nullptr, lstm ? c : nullptr});
  if (!C || !aligned(u, usize)) return PARARNN_EUNSUPPORTED;
  const Geo g = geo_for(cell, PARARNN_OP_ADJOINT, C);
  // one chunk of gate inputs and of du is addressed with 32-bit offsets below 2^31
  if (static_cast<double>(g.chunk) * ngates(cell) * o->D * 4.0 >= 2147483648.0) return PARARNN_EUNSUPPORTED;
  const Layout y = layout(cell, PARARNN_OP_ADJOINT, o, da != nullptr, g);
  if (ws_bytes < y.total) return PARARNN_EWORKSPACE;
  if (!aligned(ws, kAlign)) return PARARNN_EUNSUPPORTED;
  char* w = static_cast<char*>(ws);

  int rc = record(o, 0, stream);
  if (rc) return rc;
  const bool incl_only = incl_only_for(cell, PARARNN_OP_ADJOINT, false, static_cast<long long>(o->B) * y.ntiles_d);
  Layout yc = y;  // inclusive only: the aggregate descriptors are never read
  if (incl_only) yc.zero_end = y.agg;
  rc = clear_ws(w, yc, nullptr, 0, stream);
  if (rc) return rc;

  AdjArgs aa;
  memset(&aa, 0, sizeof(aa));
  aa.u = u;
  aa.a = a;
  aa.s0[0] = lstm ? c0 : h0;
  aa.s0[1] = lstm ? h0 : nullptr;
  aa.S[0] = lstm ? c : h;
  aa.S[1] = lstm ? h : nullptr;
  aa.dh = dh;
  aa.du = du;
  aa.ds0 = ds0;
  aa.da_part = da ? reinterpret_cast<float*>(w + y.dapart) : nullptr;
  aa.incl = reinterpret_cast<unsigned long long*>(w + y.incl);
  aa.agg = reinterpret_cast<unsigned long long*>(w + y.agg);
  aa.ctr = reinterpret_cast<unsigned int*>(w + y.ctr);
  aa.B = o->B;
  aa.L = o->L;
  aa.D = o->D;
  aa.nchunks = y.nchunks;
  aa.ntiles_d = y.ntiles_d;
  // the adjoint launch stamps event 1 at its start; event 2 at the end of
  // the last launch (the da reduction when requested)
  rc = lstm ? launch_adj_any<LstmCell>(o->u_dtype, C, incl_only, aa, stream, stamps(o, 1, da ? -1 : 2))
            : launch_adj_any<GruCell>(o->u_dtype, C, incl_only, aa, stream, stamps(o, 1, da ? -1 : 2));
  if (rc) return rc;
  if (da) {
    const int G = ngates(cell);
    const long long n = static_cast<long long>(G) * o->D;
    return launch(da_reduce_kernel, dim3(static_cast<unsigned>((n + kDaCols - 1) / kDaCols)),
                  dim3(kDaCols * kDaGroups), stream, stamps(o, -1, 2), reinterpret_cast<const float*>(w + y.dapart),
                  da, y.nchunks * o->B, n);
  }
  return PARARNN_OK;
}

extern "C" const char* pararnn_strerror(int32_t status) {
  switch (status) {
    case PARARNN_OK: return "ok";
    case PARARNN_EINVAL: return "invalid argument (null pointer, non-positive size, bad enum or iteration count, size overflow)";
    case PARARNN_EUNSUPPORTED: return "unsupported dtype or misaligned pointer";
    case PARARNN_EWORKSPACE: return "workspace smaller than pararnn_workspace_bytes()";
    case PARARNN_EHIP: return "HIP launch or runtime error";
    case PARARNN_ESCRATCH: return "problem needs more workspace than the built-in scratch holds (pararnn_scratch_bytes())";
    default: return "unknown status";
  }
}
