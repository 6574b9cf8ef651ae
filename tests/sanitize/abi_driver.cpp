// abi_driver.cpp -- runs the host-side code of the C ABI (include/pararnn.h)
// that needs no GPU, for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer: workspace sizing and launch plans over a sweep
// of shapes (tiny, ragged, at the size limits, invalid), and every argument
// check of every entry point, each called so that it returns before its first
// HIP call (a workspace of zero bytes is the last check before a launch).
// Exit status 0 when every status is the documented one.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "../../include/pararnn.h"

static int failures = 0;
#define CHECK(cond, ...)                     \
  do {                                       \
    if (!(cond)) {                           \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");                 \
      ++failures;                            \
    }                                        \
  } while (0)

static pararnn_opts opts(int B, int L, int D, int K, int dtype, int schedule, int early) {
  pararnn_opts o;
  memset(&o, 0, sizeof(o));
  o.B = B;
  o.L = L;
  o.D = D;
  o.max_iters = K;
  o.tol = 1e-4f;
  o.early_exit = early;
  o.u_dtype = dtype;
  o.events = nullptr;
  o.schedule = schedule;
  return o;
}

// never dereferenced: every call below returns before it touches memory
static void* fake(uintptr_t k) { return reinterpret_cast<void*>(k * 4096); }

int main() {
  const int dims[][3] = {{1, 1, 1},     {1, 2, 3},      {3, 5, 64},      {2, 1000, 200}, {1, 4097, 3},
                         {8, 4096, 1024}, {1, 65536, 2048}, {16, 2048, 4096}, {64, 65536, 4096},
                         {1, 2147483647, 1}, {2147483647, 2, 2}, {0, 4, 4}, {4, 0, 4}, {4, 4, -1}};
  for (auto& d : dims) {
    for (int op = 0; op <= 5; ++op)
      for (int cell = -1; cell <= 2; ++cell)
        for (int K : {0, 1, 3, 1001})
          for (int sch = 0; sch <= 3; ++sch)
            for (int early = 0; early <= 1; ++early) {
              const pararnn_opts o = opts(d[0], d[1], d[2], K, 1, sch, early);
              const size_t n = pararnn_workspace_bytes(cell, op, &o);
              pararnn_plan p;
              const int rc = pararnn_plan_query(cell, op, &o, &p);
              CHECK((n == 0) == (rc != 0) || op == 4, "sizes and plans agree on validity");
              if (rc == 0) {
                CHECK(p.chunk >= 1 && p.channels >= 1 && p.nchunks >= 1 && p.tiles_per_row >= 1,
                      "plan fields positive");
                CHECK(p.inclusive_only == 0 || p.inclusive_only == 1, "plan mode");
              }
            }
  }
  CHECK(pararnn_workspace_bytes(0, 0, nullptr) == 0, "NULL opts");
  CHECK(pararnn_plan_query(0, 0, nullptr, nullptr) == PARARNN_EINVAL, "NULL plan");

  // argument checks of the solves, the adjoint and the scans, all before any HIP call
  for (int dtype : {0, 1, 2}) {
    const pararnn_opts o = opts(2, 300, 64, 3, dtype, 0, 0);
    const int want = dtype == 2 ? PARARNN_EUNSUPPORTED : PARARNN_EWORKSPACE;
    CHECK(pararnn_solve_gru(fake(1), (float*)fake(2), nullptr, (float*)fake(3), fake(4), 0, &o, nullptr, nullptr,
                            nullptr, nullptr) == want, "gru status, dtype %d", dtype);
    CHECK(pararnn_solve_lstm(fake(1), (float*)fake(2), nullptr, nullptr, (float*)fake(5), (float*)fake(3), fake(4),
                             0, &o, nullptr, nullptr, nullptr, nullptr) == want, "lstm status, dtype %d", dtype);
    for (int cell = 0; cell <= 1; ++cell)
      CHECK(pararnn_adjoint(cell, fake(1), (float*)fake(2), nullptr, nullptr, (float*)fake(5), (float*)fake(3),
                            (float*)fake(6), (float*)fake(7), nullptr, nullptr, fake(4), 0, &o, nullptr) == want,
            "adjoint status, cell %d dtype %d", cell, dtype);
  }
  const pararnn_opts o = opts(2, 300, 64, 3, 1, 0, 0);
  CHECK(pararnn_solve_gru(nullptr, (float*)fake(2), nullptr, (float*)fake(3), fake(4), 1 << 30, &o, nullptr,
                          nullptr, nullptr, nullptr) == PARARNN_EINVAL, "NULL u");
  CHECK(pararnn_solve_lstm(fake(1), (float*)fake(2), nullptr, nullptr, nullptr, (float*)fake(3), fake(4), 1 << 30, &o,
                           nullptr, nullptr, nullptr, nullptr) == PARARNN_EINVAL, "NULL c");
  CHECK(pararnn_solve_gru(reinterpret_cast<char*>(fake(1)) + 1, (float*)fake(2), nullptr, (float*)fake(3), fake(4),
                          1 << 30, &o, nullptr, nullptr, nullptr, nullptr) == PARARNN_EUNSUPPORTED, "odd u");
  CHECK(pararnn_solve_gru(fake(1), (float*)fake(2), nullptr, (float*)fake(3), reinterpret_cast<char*>(fake(4)) + 16,
                          1 << 30, &o, nullptr, nullptr, nullptr, nullptr) == PARARNN_EUNSUPPORTED, "workspace align");
  const pararnn_opts fe = opts(2, 300, 64, 3, 1, 1, 1);  // fused with early exit
  CHECK(pararnn_solve_gru(fake(1), (float*)fake(2), nullptr, (float*)fake(3), fake(4), 1 << 30, &fe, nullptr,
                          nullptr, nullptr, nullptr) == PARARNN_EINVAL, "fused + early exit");
  for (int which = 0; which < 3; ++which) {
    const pararnn_opts so = opts(2, 300, which == 2 ? 16 : 64, 1, 0, 0, 0);
    int rc = which == 0   ? pararnn_scan_diag((float*)fake(1), (float*)fake(2), nullptr, (float*)fake(3), fake(4), 0,
                                              &so, nullptr)
             : which == 1 ? pararnn_scan_block2((float*)fake(1), (float*)fake(2), nullptr, (float*)fake(3), fake(4), 0,
                                                &so, nullptr)
                          : pararnn_scan_dense((float*)fake(1), (float*)fake(2), nullptr, (float*)fake(3), fake(4), 0,
                                               &so, nullptr);
    CHECK(rc == PARARNN_EWORKSPACE, "scan %d workspace", which);
    rc = which == 0 ? pararnn_scan_diag(nullptr, (float*)fake(2), nullptr, (float*)fake(3), fake(4), 0, &so, nullptr)
                    : pararnn_scan_dense(nullptr, (float*)fake(2), nullptr, (float*)fake(3), fake(4), 0, &so, nullptr);
    CHECK(rc == PARARNN_EINVAL, "scan %d NULL A", which);
  }
  // the largest channel count whose chunk of gate inputs (and of du) stays
  // below 2^31 bytes is accepted (the zero-byte workspace is then the first
  // refusal), the next one is not: LSTM solve under both schedules, adjoint
  for (int op = 0; op <= 1; ++op)
    for (int sch = 1; sch <= (op == 0 ? 2 : 1); ++sch) {
      // planned at a width near the limit, where the regular shapes apply
      pararnn_opts lo = opts(1, 64, 1 << 20, 3, 1, sch, 0);
      pararnn_plan p;
      CHECK(pararnn_plan_query(1, op, &lo, &p) == 0, "plan op %d schedule %d", op, sch);
      const long long per = static_cast<long long>(p.chunk) * 4 * 4;  // bytes of one channel's chunk: 4 gates, fp32
      const int dmax = static_cast<int>((2147483648LL + per - 1) / per - 1);
      for (int D : {dmax, dmax + 1}) {
        lo.D = D;
        const int rc = op == 0 ? pararnn_solve_lstm(fake(1), (float*)fake(2), nullptr, nullptr, (float*)fake(5),
                                                    (float*)fake(3), fake(4), 0, &lo, nullptr, nullptr, nullptr, nullptr)
                               : pararnn_adjoint(1, fake(1), (float*)fake(2), nullptr, nullptr, (float*)fake(5),
                                                 (float*)fake(3), (float*)fake(6), (float*)fake(7), nullptr, nullptr,
                                                 fake(4), 0, &lo, nullptr);
        CHECK(rc == (D == dmax ? PARARNN_EWORKSPACE : PARARNN_EUNSUPPORTED), "extent limit op %d schedule %d D %d: %d",
              op, sch, D, rc);
      }
    }
  const pararnn_opts big = opts(8, 4096, 1024, 3, 1, 2, 0);  // per-iteration state buffer beyond the scratch
  CHECK(pararnn_solve_gru_scratch(fake(1), (float*)fake(2), nullptr, (float*)fake(3), &big, nullptr, nullptr,
                                  nullptr, nullptr) == PARARNN_ESCRATCH, "scratch too small");
  CHECK(pararnn_solve_gru_scratch(nullptr, (float*)fake(2), nullptr, (float*)fake(3), &big, nullptr, nullptr,
                                  nullptr, nullptr) == PARARNN_EINVAL, "scratch NULL u");
  for (int st = -6; st <= 1; ++st) CHECK(pararnn_strerror(st) != nullptr, "strerror %d", st);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("C-ABI host driver: all checks passed\n");
  return 0;
}
