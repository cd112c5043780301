// plan_check.cpp — host-only check of the argument validation and workspace
// layout (kd_plan.cpp), built by the CPU tests with the host compiler under
// AddressSanitizer and UndefinedBehaviorSanitizer.
//
// For a grid of shapes (valid, edge and invalid, up to the 32-bit limits the
// kernels state) and every pass, make_plan must either return an error or a
// layout in which every region the kernels touch is 256-byte aligned, lies
// inside the workspace and overlaps no other region. Signed overflow in the
// size arithmetic is reported by UBSan and fails the run.
//
// Region sizes are the extents the kernels index, stated here from their
// launch shapes:
//   flag            256 B
//   counts          prep_chunks·nb int32        offsets  prep_chunks·nMt·(nVt + 1) int32
//   recs            prep_chunks·C·K × 8 B       rowS     prep_chunks·C floats (one-pass: C)
//   ht (bf16)       L·d·C_pad elements, L the chunks of one logit launch:
//                   fwd_group (forward), dw_window (backward), else 1
//   zhit            fwd_group·C·K floats (forward)
//   part            ((fwd_group − 1)·C + C_pad)·nVt × 8 B (forward; else fwd_group = 1)
//   loss            max(N, 1) floats
//   z               C·V_pad floats              lse, tau C_pad floats each
//   cnt             C_pad·⌈V_pad/8192⌉ int32    cand     C_pad·V_pad × 8 B
//   gscale          256 B
//   dl              ((window − 1)·C + C_pad)·V_pad elements
//   dhpart          splits·win_rows_pad·d floats (when splits > 1)
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <string>
#include <vector>

#include "kd_fused_kl.h"
#include "kd_plan.h"

namespace {

struct Region {
  const char* name;
  size_t off, bytes;
};

int g_fail = 0;

void fail(const char* what, int pass, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk,
          int dt, const std::string& detail) {
  if (g_fail < 20)
    fprintf(stderr, "FAIL %s: pass=%d N=%lld d=%lld V=%lld K=%lld chunk=%lld dtype=%d %s\n", what,
            pass, (long long)N, (long long)d, (long long)V, (long long)K, (long long)chunk, dt,
            detail.c_str());
  ++g_fail;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Checks one call, with the forward's logit launches capped at `cap` rows;
// returns its status.
int check(int pass, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk, int dt,
          int64_t cap = kd::kFwdGroupRows) {
  kd::Plan p;
  const int st = kd::make_plan(pass, N, d, V, K, chunk, dt, &p, cap);
  if (st != KD_OK) return st;
  const size_t es = dt == KD_BF16 ? 2 : 4;
  const int64_t C = std::min(chunk, std::max<int64_t>(N, 1));
  // the derived sizes
  if (p.C != C || p.C_pad % 256 != 0 || p.C_pad < C || p.C_pad - C >= 256 || p.V_pad % 256 != 0 ||
      p.V_pad < V || p.V_pad - V >= 256 || p.nVt * 256 != p.V_pad || p.nMt * 256 != p.C_pad ||
      p.nb != p.nMt * p.nVt || p.nbo != p.nMt * (p.nVt + 1) || p.nVt > 16383)
    fail("sizes", pass, N, d, V, K, chunk, dt, "");
  const int64_t n_chunks = N > 0 ? cdiv(N, C) : 1;
  if (p.dw_window < 1 || p.dw_window > kd::kDwMaxWindow || p.dw_window > n_chunks ||
      (p.dw_window > 1 && p.dw_window * C > kd::kDwRows))
    fail("dW window", pass, N, d, V, K, chunk, dt, std::to_string(p.dw_window));
  if (p.dh_splits < 1 || p.dh_splits > kd::kMaxDhSplits)
    fail("dH splits", pass, N, d, V, K, chunk, dt, std::to_string(p.dh_splits));
  if (p.win_rows_pad % 256 != 0 || p.win_rows_pad < p.dw_window * C)
    fail("window rows", pass, N, d, V, K, chunk, dt, "");
  if (p.prep_chunks < 1 || p.prep_chunks > n_chunks ||
      (p.prep_chunks > 1 && (p.prep_chunks * p.nb > kd::kPrepBuckets ||
                             p.prep_chunks * C > kd::kPrepRows)))
    fail("prep group", pass, N, d, V, K, chunk, dt, std::to_string(p.prep_chunks));
  // Launches never cross a prep group: the forward's logit launch covers
  // fwd_group chunks, the backward's dlogits launch one window.
  if (p.fwd_group < 1 || (pass != KD_PASS_FWD && p.fwd_group != 1) ||
      (p.fwd_group > 1 && p.fwd_group * C > cap) ||
      (pass == KD_PASS_FWD && p.prep_chunks % p.fwd_group != 0) ||
      (pass == KD_PASS_BWD && p.prep_chunks % p.dw_window != 0))
    fail("launch group", pass, N, d, V, K, chunk, dt,
         std::to_string(p.fwd_group) + "/" + std::to_string(p.dw_window) + "/" +
             std::to_string(p.prep_chunks));
  const int64_t logit_chunks =
      pass == KD_PASS_FWD ? p.fwd_group : pass == KD_PASS_BWD ? p.dw_window : 1;
  if (logit_chunks * p.nb > kd::kMaxBlocks)
    fail("logit grid", pass, N, d, V, K, chunk, dt, std::to_string(logit_chunks * p.nb));

  std::vector<Region> r;
  auto add = [&](const char* name, size_t off, size_t bytes) { r.push_back({name, off, bytes}); };
  const size_t G = size_t(p.prep_chunks), Cs = size_t(C), Cp = size_t(p.C_pad);
  const size_t Vp = size_t(p.V_pad), Ks = size_t(K), ds = size_t(d);
  add("flag", p.off_flag, 256);
  if (pass == KD_PASS_FWD || pass == KD_PASS_BWD) {
    add("counts", p.off_counts, 4 * G * size_t(p.nb));
    add("offsets", p.off_offsets, 4 * G * size_t(p.nMt) * size_t(p.nVt + 1));
    add("recs", p.off_recs, 8 * G * Cs * Ks);
    add("rowS", p.off_rowS, 4 * G * Cs);
  }
  if (pass == KD_PASS_FWD_BWD) add("rowS", p.off_rowS, 4 * Cs);
  if (dt == KD_BF16) add("ht", p.off_ht, es * size_t(logit_chunks) * ds * Cp);
  if (pass == KD_PASS_FWD) {
    const size_t Fg = size_t(p.fwd_group);
    add("zhit", p.off_zhit, 4 * Fg * Cs * Ks);
    add("part", p.off_part, 8 * ((Fg - 1) * Cs + Cp) * size_t(p.nVt));
    add("loss", p.off_loss, 4 * size_t(std::max<int64_t>(N, 1)));
  }
  if (pass == KD_PASS_TEACHER) {
    add("z", p.off_z, 4 * Cs * Vp);
    add("part", p.off_part, 8 * Cp * size_t(p.nVt));
    add("lse", p.off_lse, 4 * Cp);
    add("tau", p.off_tau, 4 * Cp);
    add("cnt", p.off_cnt, 4 * Cp * size_t(cdiv(p.V_pad, kd::kStreamCols)));
    add("cand", p.off_cand, 8 * Cp * Vp);
  }
  if (pass == KD_PASS_BWD || pass == KD_PASS_FWD_BWD) {
    if (pass == KD_PASS_FWD_BWD) {
      add("part", p.off_part, 8 * Cp * size_t(p.nVt));
      add("loss", p.off_loss, 4 * size_t(std::max<int64_t>(N, 1)));
      add("z", p.off_z, 4 * Cs * Vp);
    }
    add("gscale", p.off_gscale, 256);
    add("dl", p.off_dl, es * (size_t(p.dw_window - 1) * Cs + Cp) * Vp);
    if (p.dh_splits > 1)
      add("dhpart", p.off_dhpart, 4 * size_t(p.dh_splits) * size_t(p.win_rows_pad) * ds);
  }
  for (const Region& a : r) {
    if (a.off % 256 != 0) fail("alignment", pass, N, d, V, K, chunk, dt, a.name);
    if (a.off > p.total || a.bytes > p.total - a.off)
      fail("bounds", pass, N, d, V, K, chunk, dt, a.name);
  }
  for (size_t i = 0; i < r.size(); ++i)
    for (size_t j = i + 1; j < r.size(); ++j) {
      const Region &a = r[i], &b = r[j];
      if (a.off < b.off + b.bytes && b.off < a.off + a.bytes)
        fail("overlap", pass, N, d, V, K, chunk, dt, std::string(a.name) + "/" + b.name);
    }
  return st;
}

}  // namespace

int main() {
  const int64_t Ns[] = {-1, 0, 1, 7, 128, 255, 256, 1000, 1024, 4097, 8192, 65537, 262144,
                        (int64_t(1) << 31) - 1, int64_t(1) << 31, int64_t(1) << 40};
  const int64_t ds[] = {-8, 0, 8, 12, 16, 64, 200, 2880, 3072, 4096, int64_t(1) << 20,
                        (int64_t(1) << 20) + 8, int64_t(1) << 33};
  const int64_t Vs[] = {0, 1, 100, 129, 1000, 32000, 128256, 201088, 1 << 22, int64_t(1) << 28,
                        (int64_t(1) << 28) + 1, int64_t(1) << 45};
  const int64_t Ks[] = {-1, 0, 1, 8, 100, 2048, 2049, 16383, 16384, int64_t(1) << 35};
  const int64_t chunks[] = {-5, 0, 1, 7, 32, 256, 1000, 1024, 2048, 1 << 20, int64_t(1) << 40};
  int64_t ok = 0, rejected = 0;
  for (int pass = -1; pass <= 4; ++pass)
    for (int dt = -1; dt <= 2; ++dt)
      for (int64_t N : Ns)
        for (int64_t d : ds)
          for (int64_t V : Vs)
            for (int64_t K : Ks)
              for (int64_t c : chunks) {
                const int st = check(pass, N, d, V, K, c, dt);
                if (st == KD_OK) {
                  ++ok;
                  // One chunk per logit launch: the same call, valid too.
                  if (pass == KD_PASS_FWD) {
                    kd::Plan b;
                    if (check(pass, N, d, V, K, c, dt, 0) != KD_OK ||
                        kd::make_plan(pass, N, d, V, K, c, dt, &b, 0) != KD_OK ||
                        b.fwd_group != 1)
                      fail("one chunk per launch", pass, N, d, V, K, c, dt, "");
                  }
                } else {
                  ++rejected;
                  if (st != KD_ERR_INVALID_ARG && st != KD_ERR_UNSUPPORTED)
                    fail("status", pass, N, d, V, K, c, dt, std::to_string(st));
                }
              }
  // The argument checks that must reject.
  kd::Plan p;
  if (kd::make_plan(KD_PASS_FWD, 8, 16, 100, 8, 4, KD_F32, nullptr) != KD_ERR_INVALID_ARG)
    fail("null plan", 0, 8, 16, 100, 8, 4, 0, "");
  if (kd::make_plan(KD_PASS_FWD, 8, 16, 10, 11, 4, KD_F32, &p) != KD_ERR_INVALID_ARG)
    fail("K > V", 0, 8, 16, 10, 11, 4, 0, "");
  if (kd::make_plan(KD_PASS_FWD, 8, 6, 100, 8, 4, KD_BF16, &p) != KD_ERR_INVALID_ARG)
    fail("12-byte rows", 0, 8, 6, 100, 8, 4, 1, "");
  printf("plans: %lld valid, %lld rejected, %d failures\n", (long long)ok, (long long)rejected,
         g_fail);
  return g_fail == 0 && ok > 0 ? 0 : 1;
}
