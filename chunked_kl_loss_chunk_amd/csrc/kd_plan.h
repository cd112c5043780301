// kd_plan.h — argument validation and workspace layout of the fused, chunked
// top-K KL loss. Pure C++: no HIP calls, so it runs (and is tested) on a host
// without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace kd {

// Tile of the logit GEMM (tokens of a chunk × vocabulary entries). The top-K
// hit lists are bucketed by this tile, so the plan fixes it.
constexpr int kTileM = 256;  // tokens
constexpr int kTileN = 256;  // vocabulary
// Bytes of the contraction dimension staged per LDS row and pipeline stage.
constexpr int kStageRowBytes = 64;
// Packed hit record: token-in-tile (8 bits), vocab-in-tile (10 bits), k (14 bits).
constexpr int64_t kMaxK = (1 << 14) - 1;
// The teacher cache producer sorts each row's K winners in LDS.
constexpr int64_t kMaxTeacherK = 2048;
// Upper bound on the dH split-K factor.
constexpr int kMaxDhSplits = 32;
// Target number of dH workgroups per dW window (three waves of the 256 CUs).
constexpr int kDhTargetTiles = 768;
// The cached ids of a group of consecutive chunks are bucketed by one prep
// pass: at most kPrepBuckets buckets and kPrepRows rows per group.
constexpr int64_t kPrepBuckets = int64_t(1) << 20;
constexpr int64_t kPrepRows = 65536;
// The forward projects up to kFwdGroupRows rows (whole chunks, at least one)
// in one launch of the logit GEMM, and the backward one dW window per
// launch; neither launch crosses a prep group.
constexpr int64_t kFwdGroupRows = 16384;
// dW is contracted over a window of consecutive chunks at once: its fp32
// read-modify-write of V×d happens once per window instead of once per chunk,
// for a backward scratch of window × chunk × V dlogits. The window covers
// about kDwRows tokens (at most kDwMaxWindow chunks, at least one).
constexpr int64_t kDwRows = 4096;
constexpr int kDwMaxWindow = 4;
// A launch holds at most 2^32 − 1 work-items per grid dimension: with 256
// threads per workgroup, at most kMaxBlocks workgroups. The plan rejects
// sizes whose grids would not fit.
constexpr int64_t kMaxBlocks = (int64_t(1) << 24) - 1;
// Stored logits handled by one workgroup of the streaming kernels (one-pass
// dlogits, teacher candidate scan).
constexpr int64_t kStreamCols = 8192;
// Scan segments of one row the teacher cache's finish kernel indexes in LDS.
constexpr int64_t kMaxTeacherSegs = 512;

struct Plan {
  int64_t N, d, V, K, chunk;
  int dtype;      // 0 = f32, 1 = bf16
  int es;         // element size in bytes
  int64_t C;      // rows per chunk actually used: min(chunk, max(N, 1))
  int64_t C_pad;  // C rounded up to kTileM
  int64_t V_pad;  // V rounded up to kTileN
  int64_t nVt;    // vocabulary tiles
  int64_t nMt;    // row tiles per chunk
  int64_t nb;     // hit buckets per chunk = nMt * nVt
  int64_t nbo;    // bucket offsets per chunk = nMt * (nVt + 1): each token tile's
                  // nVt starts and its end
  int64_t prep_chunks;  // chunks bucketed by one prep pass (a multiple of fwd_group
                        // for the forward, of dw_window for the backward)
  int64_t fwd_group;    // forward: chunks per logit GEMM launch (1 for the other passes)
  int64_t kt_d;   // stages along d   (d * es / kStageRowBytes, rounded up)
  int64_t kt_v;   // stages along V_pad
  int dh_splits;  // split-K factor of the dH contraction (once per dW window)
  int64_t win_rows_pad;  // rows of a full dW window, rounded up to kTileM
  int dw_window;  // chunks whose dlogits are held before one dW contraction
  // byte offsets inside the workspace (all 256-byte aligned)
  size_t off_counts, off_offsets, off_recs, off_rowS, off_zhit, off_part, off_loss, off_flag;
  size_t off_dl, off_dhpart;
  size_t off_ht;      // bf16: the chunks of one launch transposed, each [d][C_pad]
  size_t off_gscale;  // backward: the device scalar g (sum) or g / Σw (mean)
  // teacher cache producer: per-row lse, threshold, candidate count, candidates
  size_t off_lse, off_tau, off_cnt, off_cand;
  // one-pass loss and gradients: the chunk's float32 logits, [C][V_pad]
  size_t off_z;
  size_t total;
};

// Fills *p for the given pass (0 forward, 1 backward, 2 teacher cache,
// 3 loss and gradients in one call). The forward's logit launches cover at
// most fwd_group_rows rows (whole chunks, at least one chunk); a smaller cap
// gives the same results in a smaller workspace.
// Returns a kd_status.
int make_plan(int pass, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk, int dtype,
              Plan* p, int64_t fwd_group_rows = kFwdGroupRows);

}  // namespace kd
