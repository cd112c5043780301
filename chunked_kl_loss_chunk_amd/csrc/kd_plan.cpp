// kd_plan.cpp — validation and workspace layout (host only, no HIP calls).
#include "kd_plan.h"

#include "kd_fused_kl.h"

namespace kd {
namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

int make_plan(int pass, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk, int dtype,
              Plan* p, int64_t fwd_group_rows) {
  if (p == nullptr) return KD_ERR_INVALID_ARG;
  if (pass != KD_PASS_FWD && pass != KD_PASS_BWD && pass != KD_PASS_TEACHER &&
      pass != KD_PASS_FWD_BWD)
    return KD_ERR_INVALID_ARG;
  if (dtype != KD_F32 && dtype != KD_BF16) return KD_ERR_INVALID_ARG;
  if (N < 0 || d <= 0 || V <= 0 || K <= 0 || chunk <= 0) return KD_ERR_INVALID_ARG;
  if (K > V) return KD_ERR_INVALID_ARG;
  const int es = dtype == KD_BF16 ? 2 : 4;
  // 16-byte rows: every H, W and dH row starts on a 16-byte boundary.
  if ((d * es) % 16 != 0) return KD_ERR_INVALID_ARG;
  if (K > kMaxK) return KD_ERR_UNSUPPORTED;
  if (pass == KD_PASS_TEACHER && K > kMaxTeacherK) return KD_ERR_UNSUPPORTED;
  if (pass == KD_PASS_TEACHER && cdiv(cdiv(V, kTileN) * kTileN, kStreamCols) > kMaxTeacherSegs)
    return KD_ERR_UNSUPPORTED;
  // 32-bit limits inside the kernels (row counts, tile counts, per-chunk
  // entry counts); global byte offsets are computed in 64 bits.
  if (N > (int64_t(1) << 31) - 1 || V > (int64_t(1) << 28) || d > (int64_t(1) << 20))
    return KD_ERR_UNSUPPORTED;

  Plan q{};
  q.N = N;
  q.d = d;
  q.V = V;
  q.K = K;
  q.chunk = chunk;
  q.dtype = dtype;
  q.es = es;
  q.C = chunk < (N > 0 ? N : 1) ? chunk : (N > 0 ? N : 1);
  q.C_pad = cdiv(q.C, kTileM) * kTileM;
  q.V_pad = cdiv(V, kTileN) * kTileN;
  q.nVt = q.V_pad / kTileN;
  q.nMt = q.C_pad / kTileM;
  q.nb = q.nMt * q.nVt;
  q.nbo = q.nMt * (q.nVt + 1);
  q.kt_d = cdiv(d * es, kStageRowBytes);
  q.kt_v = cdiv(q.V_pad * es, kStageRowBytes);
  if (q.C * K > (int64_t(1) << 30) || q.nb > (int64_t(1) << 30)) return KD_ERR_UNSUPPORTED;
  // The GEMM loaders address one 256-row tile of an operand with 32-bit
  // offsets below 2^31: a dlogits row (V_pad elements) and an H/W row
  // (d elements) must each stay under 8 MiB.
  if (q.V_pad * es * kTileM >= (int64_t(1) << 31) || d * es * kTileM >= (int64_t(1) << 31))
    return KD_ERR_UNSUPPORTED;

  const int64_t n_chunks = N > 0 ? cdiv(N, q.C) : 1;
  // The prep group: chunks whose cached entries one prep pass buckets.
  int64_t group = kPrepBuckets / q.nb;
  if (group > kPrepRows / q.C) group = kPrepRows / q.C;
  if (group > n_chunks) group = n_chunks;
  if (group < 1) group = 1;
  // The backward's dlogits launch covers one dW window, so the window's
  // chunks must be bucketed at once: a window never exceeds the prep group.
  // Every pass takes the same window, so the one-pass call contracts dW over
  // the same rows in the same order as the backward.
  int64_t window = kDwRows / q.C;
  if (window > kDwMaxWindow) window = kDwMaxWindow;
  if (window > n_chunks) window = n_chunks;
  if (window > group) window = group;
  if (window < 1) window = 1;
  q.dw_window = static_cast<int>(window);
  // Launches do not cross prep groups: the forward's logit GEMM covers
  // fwd_group chunks (fwd_group_rows rows at most), the backward's one
  // window, and the prep group is a whole number of either.
  int64_t fwd_group = 1;
  if (pass == KD_PASS_FWD) {
    fwd_group = fwd_group_rows / q.C;
    if (fwd_group > group) fwd_group = group;
    if (fwd_group < 1) fwd_group = 1;
    group = group / fwd_group * fwd_group;
  } else if (pass == KD_PASS_BWD) {
    group = group / window * window;
  }
  q.fwd_group = fwd_group;
  q.prep_chunks = group;
  // dH = dlogits · W of a window has a short output (window rows × d) and a
  // long contraction (V): split the contraction so that enough workgroups
  // exist to fill the chip.
  q.win_rows_pad = cdiv(window * q.C, kTileM) * kTileM;
  const int64_t tiles_mn = (q.win_rows_pad / kTileM) * cdiv(d, 256);
  int64_t splits = cdiv(kDhTargetTiles, tiles_mn);
  if (splits > kMaxDhSplits) splits = kMaxDhSplits;
  if (splits > q.kt_v) splits = q.kt_v;
  if (splits < 1) splits = 1;
  q.dh_splits = static_cast<int>(splits);
  // Launch grids, in workgroups of 256 threads: the logit tiles of a chunk
  // (nb; a launch of several chunks stays inside a prep group, which holds
  // at most kPrepBuckets tiles), one workgroup per row (teacher finish), four
  // rows per workgroup (prep, combine), the dH and dW tiles of a window, and
  // the streaming passes over a chunk's stored logits (one-pass loss,
  // teacher cache).
  const int64_t dh_grid = (q.win_rows_pad / kTileM) * cdiv(d, kTileM) * q.dh_splits;
  const int64_t dw_grid = cdiv(d, kTileM) * q.nVt;
  const int64_t stream_grid = q.C * cdiv(q.V_pad, kStreamCols);
  if (q.nb > kMaxBlocks || q.C > kMaxBlocks || dh_grid > kMaxBlocks || dw_grid > kMaxBlocks ||
      ((pass == KD_PASS_FWD_BWD || pass == KD_PASS_TEACHER) && stream_grid > kMaxBlocks))
    return KD_ERR_UNSUPPORTED;

  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  q.off_flag = take(256);
  if (pass == KD_PASS_FWD_BWD || pass == KD_PASS_TEACHER) {
    // No buckets: the logits of a chunk are stored, so the cached entries are
    // read per row (one-pass loss: S_r of one chunk), or there are none
    // (teacher cache).
    q.prep_chunks = 1;
    q.off_counts = q.off_offsets = q.off_recs = 0;
    q.off_rowS = pass == KD_PASS_FWD_BWD ? take(sizeof(float) * size_t(q.C)) : 0;
  } else {
    // Prep buffers of one group of chunks: bucket counts (chunk slot major,
    // then token tile, nVt each) and offsets (nVt + 1 each), hit records, S_r.
    q.off_counts = take(sizeof(int32_t) * size_t(q.prep_chunks * q.nb));
    q.off_offsets = take(sizeof(int32_t) * size_t(q.prep_chunks * q.nbo));
    q.off_recs = take(8 * size_t(q.prep_chunks * q.C * K));
    q.off_rowS = take(sizeof(float) * size_t(q.prep_chunks * q.C));
  }
  // The transposed chunks of one logit launch: fwd_group chunks in the
  // forward, one window in the backward, one chunk otherwise.
  const int64_t ht_chunks = pass == KD_PASS_FWD ? q.fwd_group : pass == KD_PASS_BWD ? q.dw_window : 1;
  q.off_ht = dtype == KD_BF16 ? take(size_t(es) * size_t(ht_chunks) * size_t(d) * size_t(q.C_pad)) : 0;
  q.off_z = 0;
  if (pass == KD_PASS_TEACHER) {
    // The chunk's logits (float32, [C][V_pad]), tile partials, lse, τ, and
    // candidate lists of up to V_pad entries per row, so none overflows.
    q.off_z = take(sizeof(float) * size_t(q.C) * size_t(q.V_pad));
    q.off_part = take(8 * size_t(q.C_pad * q.nVt));
    q.off_lse = take(sizeof(float) * size_t(q.C_pad));
    q.off_tau = take(sizeof(float) * size_t(q.C_pad));
    // candidate counts per row and 8192-logit scan segment
    q.off_cnt = take(sizeof(int32_t) * size_t(q.C_pad) * size_t(cdiv(q.V_pad, kStreamCols)));
    q.off_cand = take(8 * size_t(q.C_pad) * size_t(q.V_pad));
  } else if (pass == KD_PASS_FWD) {
    // z at the cached ids and the tile partials of one launch, rows of its
    // chunks back to back.
    q.off_zhit = take(sizeof(float) * size_t(q.fwd_group * q.C * K));
    q.off_part = take(8 * size_t((q.fwd_group - 1) * q.C + q.C_pad) * size_t(q.nVt));
    q.off_loss = take(sizeof(float) * size_t(N > 0 ? N : 1));
    q.off_dl = q.off_dhpart = 0;
  } else {
    q.off_zhit = 0;
    q.off_part = q.off_loss = 0;
    if (pass == KD_PASS_FWD_BWD) {
      // Forward side: tile partials, per-row losses, and the chunk's logits
      // in float32 ([C][V_pad]), kept until its dlogits are formed.
      q.off_part = take(8 * size_t(q.C_pad * q.nVt));
      q.off_loss = take(sizeof(float) * size_t(N > 0 ? N : 1));
      q.off_z = take(sizeof(float) * size_t(q.C) * size_t(q.V_pad));
    }
    q.off_gscale = take(256);
    // The window's chunks are packed back to back ([window·C][V_pad]); the
    // last tile of the last chunk may read (never write) up to C_pad rows.
    q.off_dl = take(size_t(es) * size_t((q.dw_window - 1) * q.C + q.C_pad) * size_t(q.V_pad));
    q.off_dhpart = q.dh_splits > 1 ? take(sizeof(float) * size_t(q.dh_splits) * size_t(q.win_rows_pad) *
                                          size_t(d))
                                    : 0;
  }
  q.total = off;
  *p = q;
  return KD_OK;
}

}  // namespace kd
