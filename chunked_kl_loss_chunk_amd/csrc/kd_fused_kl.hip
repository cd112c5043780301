// kd_fused_kl.hip — kernels, chunk scheduler and C entry points of the fused,
// chunked top-K KL distillation loss for MI355X (gfx950).
//
// Source pages (cited by title and section):
//  [P1] "Distilação de LLMs mais barata: top-K offline e KL fundida cortam
//       VRAM em até 15x" (imasters.com.br)
//  [P4] "Hugging Face：让知识蒸馏廉价到可大规模运行" (feinterview.poetries.top)
//  [P5] "Chunkovaná KL strata umožnila destilovať LLM s 32-tisícovým
//       kontextom na jednom H200" (aifeed.sk)
//
// Per chunk of C positions ([P1] "As duas mudanças"; [P4] 为什么蒸馏恢复代价高昂,
// "Fused chunked KL" paragraph: project one chunk, fold it into the running
// loss, discard it; recompute it in backward). One launch of a logit kernel
// covers a group of consecutive chunks (the forward's up to 16,384 rows, the
// backward's dW window) and walks them chunk by chunk:
//
//  forward   prep    bucket the top-K entries of a group of chunks by logit
//                    tile (a count and a scatter launch per group of up to
//                    65,536 rows, over token tile × vocabulary slice); S_r
//            logits  z tile = H_c Wᵀ on MFMA; per tile: row max and Σexp
//                    (online logsumexp partials) and z at the cached ids
//            combine lse_r from the partials; L_r = Σp·logp − Σp·z + S_r·lse_r;
//                    the total Σ_r w_r L_r (or its weighted mean) in fixed order
//  backward  prep    as above
//            dlogits recompute the z tile; dl = g w_r (S_r e^{z−lse_r} − p_sparse)
//                    formed on its way into LDS, corrected at the cached ids
//                    there, written once per chunk (bf16 or fp32)
//            dH      dH_c = dl · W      (split over the vocabulary, fixed-order sum)
//            dW      dW  += dlᵀ · H     (once per window of chunks; fp32
//                    read-modify-write, chunk order fixed)
//
// The offline teacher cache that feeds the loss (top-K ids by logit and their
// full-softmax log-probabilities; [P1] "As duas mudanças", [P4] 离线蒸馏) is
// produced by one pass of the logit GEMM that keeps the chunk's logits, and a
// streaming selection over them (kd_teacher_topk).
//
// The teacher distribution stays sparse and is not renormalised ([P5] "Čo
// dopĺňajú podrobnejšie experimenty"). The gradient is the closed form of the
// dense KL: ∂L_r/∂z_rj = S_r q_rj − p_rj (the pages name a closed-form
// gradient without printing it; [P4] 得到的 student).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "kd_fused_kl.h"
#include "kd_gemm.h"
#include "kd_plan.h"

namespace kd {
namespace {

constexpr float kNegInf = -__builtin_inff();
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <bool BF16>
struct Elt;
template <>
struct Elt<true> {
  typedef __bf16 T;
};
template <>
struct Elt<false> {
  typedef float T;
};

// Two floats to two bf16 (round to nearest even) in one word, lo in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Hit record of one cached teacher entry inside a logit tile.
__device__ __forceinline__ uint32_t pack_hit(int row_in_tile, int col_in_tile, int k) {
  return uint32_t(row_in_tile) | (uint32_t(col_in_tile) << 8) | (uint32_t(k) << 18);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Merge two (max, Σexp(x − max)) pairs of an online logsumexp.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == kNegInf) {
    m = mn;
    s = 0.f;
    return;
  }
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}

// --------------------------------------------------------------------------
// small utility kernels
// --------------------------------------------------------------------------
__global__ void k_fill_i32(int* __restrict__ p, int64_t n, int v) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void k_fill_f32(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

// x *= s in place (s a device scalar). Every workgroup reads s first and
// leaves at once when s == 1, so scaling by one costs only the launch.
template <bool BF16>
__global__ void k_scale(void* __restrict__ x, int64_t n, const float* __restrict__ s) {
  const float g = *s;
  if (g == 1.f) return;
  typedef typename Elt<BF16>::T T;
  T* const p = static_cast<T*>(x);
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = T(float(p[i]) * g);
}

__global__ void k_cast_f32_bf16(const float* __restrict__ src, __bf16* __restrict__ dst, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    dst[i] = __bf16(src[i]);
}

// dst[c][r] = src[r][c] for a [rows][cols] matrix of 16-bit elements (bf16
// chunks of H into the [d][tokens] layout the logit GEMM streams as a column
// operand), one chunk of C source rows per blockIdx.z: chunk z is rows
// z·C .. min(rows, (z+1)·C) − 1 of src, and becomes its own [cols][rows_pad]
// block at dst + z·dst_chunk. Block rows are written for r < rows_pad, zero
// past the chunk's rows. Needs cols % 8 == 0, rows_pad % 8 == 0 and 16-byte
// aligned rows.
__global__ __launch_bounds__(256) void k_transpose16(const uint16_t* __restrict__ src,
                                                     int64_t ld_src, int rows, int cols,
                                                     uint16_t* __restrict__ dst, int64_t ld_dst,
                                                     int rows_pad, int C, int64_t dst_chunk) {
  __shared__ uint16_t t[64][66];
  const int z = blockIdx.z;
  src += int64_t(z) * C * ld_src;
  dst += int64_t(z) * dst_chunk;
  rows = rows - z * C < C ? rows - z * C : C;
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64, tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = tid + i * 256, rr = u >> 3, cc = (u & 7) * 8;
    const int r = r0 + rr, c = c0 + cc;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows && c < cols) v = *reinterpret_cast<const uint4*>(src + int64_t(r) * ld_src + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t[rr][cc + 2 * j] = uint16_t(w[j] & 0xFFFFu);
      t[rr][cc + 2 * j + 1] = uint16_t(w[j] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = tid + i * 256, cc = u >> 3, rr = (u & 7) * 8;
    const int c = c0 + cc, r = r0 + rr;
    if (c < cols && r < rows_pad) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = uint32_t(t[rr + 2 * j][cc]) | (uint32_t(t[rr + 2 * j + 1][cc]) << 16);
      *reinterpret_cast<uint4*>(dst + int64_t(c) * ld_dst + r) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Σ w_i x_i and Σ w_i over i < n in a fixed order (contiguous per-thread
// ranges, then a tree); w == nullptr means every w_i = 1. One block of 1024.
__device__ __forceinline__ float2 fixed_wsum(const float* __restrict__ x, const float* __restrict__ w,
                                             int64_t n, float2* sh) {
  const int t = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t b = t * per, e = b + per < n ? b + per : n;
  float sx = 0.f, sw = 0.f;
  for (int64_t i = b; i < e; ++i) {
    const float wi = w ? w[i] : 1.f;
    if (x) sx += wi * x[i];
    sw += wi;
  }
  sh[t] = make_float2(sx, sw);
  __syncthreads();
  for (int h = 512; h >= 1; h >>= 1) {
    if (t < h) sh[t] = make_float2(sh[t].x + sh[t + h].x, sh[t].y + sh[t + h].y);
    __syncthreads();
  }
  return sh[0];
}

// The accumulated loss: Σ_r w_r L_r, divided by Σ_r w_r for the mean (a zero
// total weight gives 0).
__global__ __launch_bounds__(1024) void k_loss_reduce(const float* __restrict__ loss,
                                                      const float* __restrict__ w, int64_t n,
                                                      int mean, float* __restrict__ out) {
  __shared__ float2 sh[1024];
  const float2 s = fixed_wsum(loss, w, n, sh);
  if (threadIdx.x == 0) out[0] = mean ? (s.y != 0.f ? s.x / s.y : 0.f) : s.x;
}

// The upstream gradient each row's dlogits is scaled by, before its weight:
// g for the sum, g / Σ_r w_r for the mean (0 for a zero total weight).
__global__ __launch_bounds__(1024) void k_grad_scale(const float* __restrict__ grad,
                                                     const float* __restrict__ w, int64_t n,
                                                     int mean, float* __restrict__ out) {
  __shared__ float2 sh[1024];
  const float2 s = fixed_wsum(nullptr, w, mean ? n : 0, sh);
  if (threadIdx.x == 0) out[0] = mean ? (s.y != 0.f ? grad[0] / s.y : 0.f) : grad[0];
}

// --------------------------------------------------------------------------
// prep: bucket the cached entries of a group of chunks by (chunk, row tile,
// vocabulary tile)
// --------------------------------------------------------------------------
// Token tile T = chunk·nMt + the tile's index in its chunk; its rows start at
// group row row0 = chunk·C + 256·tile, and its records fill their own range
// of recs, [row0·K, (row0 + rows)·K). offsets[T·(nVt+1) + v] is the first
// record of vocabulary tile v, offsets[T·(nVt+1) + nVt] the end of the
// tile's records. The order inside a bucket does not matter: every record
// touches a distinct output element.
//
// Two launches over (token tile, vocabulary slice) workgroups, so that a
// group of few token tiles still fills the chip: slice s of a tile covers
// its vocabulary tiles [s·span, (s+1)·span). Each workgroup reads all of its
// tile's entries and keeps those of its slice.
//   k_prep_count   counts the slice's valid entries per vocabulary tile in
//                  LDS into counts[T·nVt + v]; it also writes S_r for the
//                  tile rows r ≡ s (mod slices), one wave per row, each lane
//                  summing k = lane, lane + 64, ... and then a butterfly over
//                  the wave (the order the one-pass combine repeats).
//   k_prep_scatter sums the counts of the tile's earlier slices, scans its
//                  own in LDS, writes the offsets, and scatters the slice's
//                  8-byte hit records.
// Ids outside [0, V) raise `flag` (slice 0 reports them) and are skipped;
// p = 0 entries are skipped.
constexpr int kPrepThreads = 1024;
constexpr int kPrepWaves = kPrepThreads / 64;
constexpr int kPrepMaxVt = 16384;  // the plan keeps nVt below this (8 MiB rows)
constexpr int kPrepUnroll = 4;     // entries (or rows) per thread (or wave) in flight
constexpr int kPrepTargetBlocks = 256;  // workgroups a prep launch aims at

struct PrepTile {
  int T, s;        // token tile, vocabulary slice
  int row0, rows;  // first group row, rows
  int v0, v1;      // the slice's vocabulary tiles
};

__device__ __forceinline__ PrepTile prep_tile(int rows, int C, int nMt, int nVt, int span,
                                              int slices) {
  PrepTile t;
  t.T = blockIdx.x / slices;
  t.s = blockIdx.x % slices;
  const int c = t.T / nMt;
  t.row0 = c * C + (t.T % nMt) * kTileM;
  const int chunk_end = rows < (c + 1) * C ? rows : (c + 1) * C;
  const int left = chunk_end - t.row0;
  t.rows = left <= 0 ? 0 : left < kTileM ? left : kTileM;
  t.v0 = t.s * span;
  t.v1 = t.v0 + span < nVt ? t.v0 + span : nVt;
  return t;
}

// Visits the valid entries of the tile whose vocabulary tile is in the
// slice: f(entry index within the tile, id, p). The tile's entries are
// contiguous, kPrepUnroll per thread in flight.
template <class F>
__device__ __forceinline__ void prep_visit(const int* ir, const float* lr, int n, int V, int v0,
                                           int v1, int* flag, F&& f) {
  for (int e0 = threadIdx.x; e0 < n; e0 += kPrepUnroll * kPrepThreads) {
    int j[kPrepUnroll];
    float lp[kPrepUnroll];
#pragma unroll
    for (int u = 0; u < kPrepUnroll; ++u) {
      const int e = e0 + u * kPrepThreads;
      j[u] = e < n ? ir[e] : 0;
      lp[u] = e < n ? lr[e] : kNegInf;
    }
#pragma unroll
    for (int u = 0; u < kPrepUnroll; ++u) {
      const int e = e0 + u * kPrepThreads;
      if (e >= n) continue;
      const bool ok = j[u] >= 0 && j[u] < V;
      if (!ok) {
        if (flag) atomicOr(flag, 1);
        continue;
      }
      const int vt = j[u] / kTileN;
      if (vt < v0 || vt >= v1) continue;
      const float p = __expf(lp[u]);
      if (p > 0.f) f(e, j[u], p);
    }
  }
}

__global__ __launch_bounds__(kPrepThreads) void k_prep_count(const int* __restrict__ idx,
                                                             const float* __restrict__ logp,
                                                             int64_t r0, int rows, int C, int nMt,
                                                             int K, int V, int nVt, int span,
                                                             int slices, int* __restrict__ counts,
                                                             float* __restrict__ rowS,
                                                             int* __restrict__ flag) {
  __shared__ int cnt[kPrepMaxVt];
  const PrepTile t = prep_tile(rows, C, nMt, nVt, span, slices);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int* ir = idx + (r0 + t.row0) * K;
  const float* lr = logp + (r0 + t.row0) * K;
  for (int v = tid; v < t.v1 - t.v0; v += kPrepThreads) cnt[v] = 0;

  // S_r of the tile rows s, s + slices, ...: kPrepUnroll rows per wave at a
  // time, rows in the order of the tile.
  const int nmine = t.rows > t.s ? (t.rows - t.s + slices - 1) / slices : 0;
  for (int ib = w * kPrepUnroll; ib < nmine; ib += kPrepWaves * kPrepUnroll) {
    float sr[kPrepUnroll];
#pragma unroll
    for (int u = 0; u < kPrepUnroll; ++u) sr[u] = 0.f;
    for (int k = lane; k < K; k += 64) {
#pragma unroll
      for (int u = 0; u < kPrepUnroll; ++u) {
        if (ib + u < nmine) {
          const int64_t rr = t.s + int64_t(ib + u) * slices;
          const int j = ir[rr * K + k];
          const float p = __expf(lr[rr * K + k]);
          if (j >= 0 && j < V && p > 0.f) sr[u] += p;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kPrepUnroll; ++u) {
      const float x = wave_sum(sr[u]);
      if (lane == 0 && ib + u < nmine) rowS[t.row0 + t.s + (ib + u) * slices] = x;
    }
  }
  __syncthreads();

  prep_visit(ir, lr, t.rows * K, V, t.v0, t.v1, t.s == 0 ? flag : nullptr,
             [&](int, int j, float) { atomicAdd(&cnt[j / kTileN - t.v0], 1); });
  __syncthreads();
  int* const out = counts + int64_t(t.T) * nVt + t.v0;
  for (int v = tid; v < t.v1 - t.v0; v += kPrepThreads) out[v] = cnt[v];
}

__global__ __launch_bounds__(kPrepThreads) void k_prep_scatter(const int* __restrict__ idx,
                                                               const float* __restrict__ logp,
                                                               int64_t r0, int rows, int C,
                                                               int nMt, int K, int V, int nVt,
                                                               int span, int slices,
                                                               const int* __restrict__ counts,
                                                               int* __restrict__ offsets,
                                                               uint2* __restrict__ recs) {
  __shared__ int cnt[kPrepMaxVt + 1];
  __shared__ int wsum[kPrepWaves];
  const PrepTile t = prep_tile(rows, C, nMt, nVt, span, slices);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int* tc = counts + int64_t(t.T) * nVt;
  const int nv = t.v1 - t.v0;

  // The records of the tile's earlier slices come first.
  int before = 0;
  for (int v = tid; v < t.v0; v += kPrepThreads) before += tc[v];
  // exclusive scan of the slice's counts: each thread a run of `per` counts,
  // the runs' sums scanned by wave shuffles and the wave totals
  const int per = (nv + kPrepThreads - 1) / kPrepThreads;
  const int b = tid * per, e = b + per < nv ? b + per : nv;
  int sum = 0;
  for (int v = b; v < e; ++v) {
    cnt[v] = tc[t.v0 + v];
    sum += cnt[v];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  // one pass of wave totals for the earlier slices' sum, one for the scan
  const int wb = __shfl_xor(before, 32) + before;
  int btot = wb;
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) btot += __shfl_xor(btot, off);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int run = incl - sum, total = 0;
#pragma unroll
  for (int q = 0; q < kPrepWaves; ++q) {
    run += q < w ? wsum[q] : 0;
    total += wsum[q];
  }
  __syncthreads();  // wsum is reused for the earlier slices' sum
  if (lane == 0) wsum[w] = btot;
  __syncthreads();
  int base = t.row0 * K;
#pragma unroll
  for (int q = 0; q < kPrepWaves; ++q) base += wsum[q];
  for (int v = b; v < e; ++v) {
    const int x = cnt[v];
    cnt[v] = run;
    run += x;
  }
  __syncthreads();
  int* const off = offsets + int64_t(t.T) * (nVt + 1);
  for (int v = tid; v < nv; v += kPrepThreads) off[t.v0 + v] = base + cnt[v];
  if (t.v1 == nVt && tid == 0) off[nVt] = base + total;

  // scatter, the scanned counts serving as cursors
  const int* ir = idx + (r0 + t.row0) * K;
  const float* lr = logp + (r0 + t.row0) * K;
  prep_visit(ir, lr, t.rows * K, V, t.v0, t.v1, nullptr, [&](int en, int j, float p) {
    const int pos = base + atomicAdd(&cnt[j / kTileN - t.v0], 1);
    recs[pos] = make_uint2(pack_hit(en / K, j % kTileN, en % K), __float_as_uint(p));
  });
}

// --------------------------------------------------------------------------
// forward: fused logit tile with online-logsumexp partials and top-K gather
// --------------------------------------------------------------------------
// The tile is zᵀ: 256 vocabulary entries (MFMA M, from W) × 256 tokens (MFMA
// N, from the chunk of H). Each lane holds, for one token column per block,
// 64 vocabulary values; a token's (max, Σexp) over the tile needs one
// cross-half shuffle and one exchange between the two waves sharing it.
//
// A launch covers nch consecutive chunks of C rows (`rows` in all; only the
// last chunk may be shorter). Its tiles run chunk by chunk, and inside a
// chunk vocabulary-tile major, token tile fastest. Each chunk's operands and
// buffers follow the previous chunk's at fixed strides, so the kernel forms
// the chunk's own view (ChunkView) and works on that.
struct FwdArgs {
  RowOp W;   // [V][d]
  RowOp H;   // rows of H from the first chunk's first, [.][d] (float32 path)
  ColOp Ht;  // the first chunk transposed, [d][C_pad] (bf16 path)
  int kt;   // stages along d
  int tiles_t, tiles_v;  // token tiles of all the launch's chunks; vocabulary tiles
  int nch, C, nMt, nb;   // chunks, rows per chunk, token tiles and bucket offsets per full chunk
  int64_t ht_chunk;      // bytes from one chunk's transposed block to the next
  int rows, V, K, nVt;
  const int* offsets;  // bucket offsets of the first chunk: nVt + 1 per token tile, nb per chunk
  const uint2* recs;
  float* zhit;     // [rows, K]: z at the cached ids
  float2* part;    // [rows, nVt]: (max, Σexp) of each token over each vocabulary tile
  float* z;        // STORE_Z (one chunk only): the chunk's logits, [rows][ld_z] float32
  int64_t ld_z;
};

// Chunk and tile of a logical workgroup index, in the order above.
struct ChunkView {
  int c;       // chunk within the launch
  int rows;    // its rows
  int tt, vt;  // token and vocabulary tile within the chunk
};

__device__ __forceinline__ ChunkView chunk_view(int logical, int nch, int C, int nMt, int rows,
                                                int tiles_v) {
  ChunkView v;
  const int per = nMt * tiles_v;  // tiles of a full chunk
  v.c = logical / per;
  const int rem = logical - v.c * per;
  const int left = rows - v.c * C;
  v.rows = left < C ? left : C;
  const int tc = v.c + 1 < nch ? nMt : (v.rows + kBN - 1) / kBN;
  v.tt = rem % tc;
  v.vt = rem / tc;
  return v;
}

// The launch's arguments narrowed to the chunk of `v`.
__device__ __forceinline__ FwdArgs narrow(const FwdArgs& a, const ChunkView& v) {
  FwdArgs n = a;
  n.H.base += int64_t(v.c) * a.C * a.H.ld;
  n.H.rows = v.rows;
  n.Ht.base += int64_t(v.c) * a.ht_chunk;
  n.Ht.cbytes = v.rows * 2;
  n.rows = v.rows;
  if (a.offsets) n.offsets += int64_t(v.c) * a.nb;
  if (a.zhit) n.zhit += int64_t(v.c) * a.C * a.K;
  n.part += int64_t(v.c) * a.C * a.nVt;
  return n;
}

// Hit records of one tile. The epilogue starts by loading the first 64
// records (one coalesced 8-byte load per lane) so their latency overlaps the
// epilogue's other work; each wave then keeps the records that fall in its
// 128×128 quadrant (a ballot), and every lane handles its own record.
struct TileHits {
  const uint2* recs;
  int h0, n;
  uint2 first;  // record h0 + lane, if lane < n
};

__device__ __forceinline__ TileHits hits_begin(const int* offsets, const uint2* recs, int bkt,
                                               int lane) {
  TileHits t;
  t.recs = recs;
  t.h0 = offsets[bkt];
  t.n = offsets[bkt + 1] - t.h0;
  t.first = lane < t.n ? recs[t.h0 + lane] : make_uint2(0xffffffffu, 0u);
  return t;
}

// Records base..base+63 (one per lane) and the ballot of those in this
// wave's quadrant.
__device__ __forceinline__ uint2 hits_load(const TileHits& t, int base, int lane) {
  const int i = base + lane;
  return base == 0 ? t.first : (i < t.n ? t.recs[t.h0 + i] : make_uint2(0xffffffffu, 0u));
}
__device__ __forceinline__ uint64_t hits_mine(const TileHits& t, const uint2& r, int base, int wm,
                                              int wn, int lane) {
  const int wr = int((r.x >> 8) & 1023u) - wm * kWTM;  // vocabulary row in the wave's quadrant
  const int wc = int(r.x & 255u) - wn * kWTN;          // token column in the wave's quadrant
  return __ballot(base + lane < t.n && unsigned(wr) < unsigned(kWTM) && unsigned(wc) < unsigned(kWTN));
}

// Any lane can read any accumulator element of its wave once one 128×32
// column block (b) is staged in a wave-private LDS region as [col][row] fp32
// with a padded column stride (consecutive lanes write different columns;
// the pad spreads them over the banks). LDS operations of one wave execute
// in order, so the wave reads its own writes without a barrier.
constexpr int kColStride = kWTM + 4;                       // floats per staged column
constexpr int kStageBlockBytes = 32 * kColStride * 4;       // one wave's region
typedef __attribute__((address_space(3))) float lds_f32;

__device__ __forceinline__ void stage_block_column(const Acc& acc, int b, lds_f32* region, int lane) {
#pragma unroll
  for (int t = 0; t < kTM; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = t * 32 + 8 * q + 4 * (lane >> 5);
      *reinterpret_cast<__attribute__((address_space(3))) f32x4_t*>(region + (lane & 31) * kColStride + row) =
          f32x4_t{acc[t][b][4 * q], acc[t][b][4 * q + 1], acc[t][b][4 * q + 2], acc[t][b][4 * q + 3]};
    }
}

__device__ __forceinline__ float staged_at(const lds_f32* region, int wr, int wc) {
  return region[(wc & 31) * kColStride + wr];
}

// As stage_block_column, but each element leaves as gs · exp(z − l).
__device__ __forceinline__ void stage_block_dl(const Acc& acc, int b, lds_f32* region, int lane,
                                               float l, float gs) {
#pragma unroll
  for (int t = 0; t < kTM; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = t * 32 + 8 * q + 4 * (lane >> 5);
      f32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = gs * __expf(acc[t][b][4 * q + e] - l);
      *reinterpret_cast<__attribute__((address_space(3))) f32x4_t*>(region + (lane & 31) * kColStride + row) = v;
    }
}

// The forward tile's epilogue, one-pass variant: the tile leaves one 32-token
// column block at a time, staged in LDS as [token][vocabulary] and written as
// 16-byte pieces, each token's 128 entries of this wave in one contiguous
// 512-byte run. Vocabulary rows past V hold 0 (zero-filled operand rows) and
// land in the row padding.
__device__ __forceinline__ void store_tile_logits(const Acc& acc, lds_f32* region,
                                                  const FwdArgs& a, int t_base, int v_base, int wm,
                                                  int wn, int lane) {
  const int sub = lane >> 4, c8 = (lane & 15) * 8;  // 4 tokens × 16 lanes
#pragma unroll
  for (int b = 0; b < kTN; ++b) {
    stage_block_column(acc, b, region, lane);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tl = sub + 4 * j;
      const int64_t tok = t_base + wn * kWTN + b * 32 + tl;
      const lds_f32* src = region + tl * kColStride + c8;
      const f32x4_t v0 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>(src);
      const f32x4_t v1 =
          *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>(src + 4);
      if (tok >= a.rows) continue;
      float* dst = a.z + tok * a.ld_z + v_base + wm * kWTM + c8;
      *reinterpret_cast<float4*>(dst) = make_float4(v0[0], v0[1], v0[2], v0[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(v1[0], v1[1], v1[2], v1[3]);
    }
  }
}

// The forward tile's epilogue, two-pass variant: z at the cached teacher ids
// that fall in this tile (bucket `bkt`), one column block at a time.
__device__ __forceinline__ void gather_hit_logits(const Acc& acc, lds_f32* region,
                                                  const FwdArgs& a, int bkt, int t_base, int wm,
                                                  int wn, int lane) {
  const TileHits hits = hits_begin(a.offsets, a.recs, bkt, lane);
  for (int base = 0; base < hits.n; base += 64) {
    const uint2 r = hits_load(hits, base, lane);
    const uint64_t mine = hits_mine(hits, r, base, wm, wn, lane);
    if (mine == 0) continue;
    const int tok = int(r.x & 255u), voc = int((r.x >> 8) & 1023u), k = int(r.x >> 18);
    const int wc = tok - wn * kWTN;
#pragma unroll
    for (int b = 0; b < kTN; ++b) {
      // Every lane holding a record of this block reads its own entry.
      const bool in_b = ((mine >> lane) & 1) && (wc >> 5) == b;
      if (__ballot(in_b) == 0) continue;
      stage_block_column(acc, b, region, lane);
      if (in_b) a.zhit[int64_t(t_base + tok) * a.K + k] = staged_at(region, voc - wm * kWTM, wc);
    }
  }
}

// STORE_Z: the one-pass variant. Instead of gathering z at the cached ids it
// writes the whole tile of logits (float32, token-major), and the cached ids
// are read back from there per row.
template <bool BF16, bool STORE_Z>
__global__ __launch_bounds__(kThreads) void k_fwd_logits(FwdArgs args) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kSmemBytes];
  lds_t* smem = (lds_t*)(smem_raw);
  const int nblk = args.tiles_t * args.tiles_v;
  const int logical = xcd_logical(blockIdx.x, nblk);
  const ChunkView cv = chunk_view(logical, args.nch, args.C, args.nMt, args.rows, args.tiles_v);
  const FwdArgs a = narrow(args, cv);
  const int tt = cv.tt, vt = cv.vt;
  const int t_base = tt * kBN, v_base = vt * kBM;

  Acc acc;
  if constexpr (BF16)
    gemm_tile<BF16, RowDirect, RowOp, ColDirect, ColOp>(acc, a.W, v_base, a.Ht, t_base, 0, a.kt, smem);
  else
    gemm_tile<BF16, RowDirect, RowOp, RowDirect, RowOp>(acc, a.W, v_base, a.H, t_base, 0, a.kt, smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWM, wn = wave / kWM;

  // Per token: max and Σexp over this tile's valid vocabulary rows.
  const int vlim = a.V - (v_base + wm * kWTM);  // rows of this wave below vlim are valid
  const bool full = vlim >= kWTM;
  float2* red = reinterpret_cast<float2*>(smem_raw);  // [kWM][kBN]
#pragma unroll
  for (int b = 0; b < kTN; ++b) {
    float m = kNegInf;
    if (full) {
#pragma unroll
      for (int t = 0; t < kTM; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, acc[t][b][i]);
    } else {
#pragma unroll
      for (int t = 0; t < kTM; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = t * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          m = r < vlim ? fmaxf(m, acc[t][b][i]) : m;
        }
    }
    m = fmaxf(m, __shfl_xor(m, 32));
    const float ms = m == kNegInf ? 0.f : m;
    float s = 0.f;
    if (full) {
#pragma unroll
      for (int t = 0; t < kTM; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += __expf(acc[t][b][i] - ms);
    } else {
#pragma unroll
      for (int t = 0; t < kTM; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = t * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          s += r < vlim ? __expf(acc[t][b][i] - ms) : 0.f;
        }
    }
    s += __shfl_xor(s, 32);
    if (lane < 32) red[wm * kBN + acc_col(wn, b, lane)] = make_float2(m, s);
  }

  lds_f32* region = reinterpret_cast<lds_f32*>(smem + kWM * kBN * sizeof(float2)) +
                    wave * (kStageBlockBytes / 4);
  if constexpr (STORE_Z)
    store_tile_logits(acc, region, a, t_base, v_base, wm, wn, lane);
  else
    gather_hit_logits(acc, region, a, tt * (a.nVt + 1) + vt, t_base, wm, wn, lane);

  __syncthreads();
  if (t_base + tid < a.rows) {
    float m = red[tid].x, s = red[tid].y;
#pragma unroll
    for (int w = 1; w < kWM; ++w) lse_merge(m, s, red[w * kBN + tid].x, red[w * kBN + tid].y);
    a.part[int64_t(t_base + tid) * a.nVt + vt] = make_float2(m, s);
  }
}

// One wave per token: lse_r from the tile partials (fixed order), then
// L_r = Σ_k p_k (logp_k − z_k + lse_r). z_k comes from the gathered zhit
// [C][K], or, when zhit is null, from the stored logits z [rows][ld_z]; a
// non-null rowS also receives S_r = Σ_k p_k over the valid entries, summed
// exactly as the prep pass sums it.
__global__ __launch_bounds__(256) void k_fwd_combine(const float2* __restrict__ part, int nVt,
                                                     const float* __restrict__ zhit,
                                                     const float* __restrict__ z, int64_t ld_z,
                                                     const int* __restrict__ idx,
                                                     const float* __restrict__ logp, int64_t r0,
                                                     int rows, int K, int V,
                                                     float* __restrict__ lse_out,
                                                     float* __restrict__ loss_out,
                                                     float* __restrict__ rowS) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  float m = kNegInf, s = 0.f;
  const float2* pr = part + int64_t(row) * nVt;
  for (int t = lane; t < nVt; t += 64) {
    const float2 v = pr[t];
    lse_merge(m, s, v.x, v.y);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    lse_merge(m, s, m2, s2);
  }
  const float lse = m + __logf(s);
  const int* ir = idx + (r0 + row) * K;
  const float* lr = logp + (r0 + row) * K;
  const float* zr = zhit ? zhit + int64_t(row) * K : nullptr;
  const float* zrow = zhit ? nullptr : z + int64_t(row) * ld_z;
  // L_r = Σ_k p_k (logp_k − (z_k − lse)): the log-probability z − lse is
  // formed per entry, so a large common offset of the logits cancels before
  // the sum instead of between two large sums.
  float L = 0.f, S = 0.f;
  for (int k = lane; k < K; k += 64) {
    const int j = ir[k];
    const float lp = lr[k];
    const float p = __expf(lp);
    if (j >= 0 && j < V && p > 0.f) {
      L += p * (lp - ((zr ? zr[k] : zrow[j]) - lse));
      S += p;
    }
  }
  L = wave_sum(L);
  if (rowS) S = wave_sum(S);
  if (lane == 0) {
    lse_out[r0 + row] = lse;
    loss_out[r0 + row] = L;
    if (rowS) rowS[row] = S;
  }
}

// --------------------------------------------------------------------------
// one-pass loss and gradients: stored logits -> dlogits
// --------------------------------------------------------------------------
// dl = g w_r S_r exp(z − lse_r) for every vocabulary entry below V and 0 in
// the row padding up to V_pad, with the same float32 expressions as the
// recomputing dlogits kernel. A workgroup covers 8192 entries of one row:
// each lane reads 16 bytes of logits per step (a wave: 1 KiB contiguous) and
// writes 8 (bf16) or 16 (float32) bytes. The logits are read exactly once, so
// the loads are nontemporal (13% faster than cached loads on the 8K head; the
// same hint on the logit stores slowed the GEMM down more than it saved).
constexpr int kDlGroups = 8;                             // 4-entry groups per lane
constexpr int kDlCols = 256 * 4 * kDlGroups;             // entries per workgroup
static_assert(kDlCols == kStreamCols, "the plan sizes the streaming grid by kStreamCols");
template <bool BF16>
__global__ __launch_bounds__(256) void k_dl_dense(const float* __restrict__ z, int64_t ld_z,
                                                  const float* __restrict__ lse,
                                                  const float* __restrict__ rowS,
                                                  const float* __restrict__ grad,
                                                  const float* __restrict__ w, int nseg, int V,
                                                  int V_pad, void* __restrict__ dl_out,
                                                  int64_t ld_dl) {
  typedef typename Elt<BF16>::T T;
  const int row = blockIdx.x / nseg, seg = blockIdx.x % nseg;
  const float g = *grad;
  const float l = lse[row];
  const float gs = g * (w ? w[row] : 1.f) * rowS[row];
  const float* zr = z + int64_t(row) * ld_z;
  T* dr = reinterpret_cast<T*>(dl_out) + int64_t(row) * ld_dl;
  const int c0 = seg * kDlCols + threadIdx.x * 4;
  float4 v[kDlGroups];
#pragma unroll
  for (int u = 0; u < kDlGroups; ++u) {
    const int c = c0 + u * 1024;
    f32x4_t t = {0.f, 0.f, 0.f, 0.f};
    if (c < V_pad) t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(zr + c));
    v[u] = make_float4(t[0], t[1], t[2], t[3]);
  }
#pragma unroll
  for (int u = 0; u < kDlGroups; ++u) {
    const int c = c0 + u * 1024;
    if (c >= V_pad) continue;
    float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = c + i < V ? gs * __expf(e[i] - l) : 0.f;
    if constexpr (BF16) {
      *reinterpret_cast<uint2*>(dr + c) = make_uint2(pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]));
    } else {
      *reinterpret_cast<float4*>(dr + c) = make_float4(e[0], e[1], e[2], e[3]);
    }
  }
}

// The cached entries of the chunk, one lane each, launched after k_dl_dense:
// dl at a cached id becomes g w_r (S_r q − p), formed in float32 from the
// stored logit and rounded once, as in the recomputing dlogits kernel.
template <bool BF16>
__global__ __launch_bounds__(256) void k_dl_hits(const float* __restrict__ z, int64_t ld_z,
                                                 const float* __restrict__ lse,
                                                 const float* __restrict__ rowS,
                                                 const float* __restrict__ grad,
                                                 const float* __restrict__ w,
                                                 const int* __restrict__ idx,
                                                 const float* __restrict__ logp, int64_t r0,
                                                 int rows, int K, int V, void* __restrict__ dl_out,
                                                 int64_t ld_dl) {
  typedef typename Elt<BF16>::T T;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(rows) * K) return;
  const int row = int(i / K);
  const int j = idx[r0 * K + i];
  const float p = __expf(logp[r0 * K + i]);
  if (!(j >= 0 && j < V && p > 0.f)) return;
  const float g = *grad;
  const float gs = g * (w ? w[row] : 1.f) * rowS[row];
  const float gw = w ? g * w[row] : g;
  // The product is rounded on its own before the fused correction, as it is
  // when the recomputing kernel stages it in LDS.
  const float v = __fmul_rn(gs, __expf(z[int64_t(row) * ld_z + j] - lse[row]));
  reinterpret_cast<T*>(dl_out)[int64_t(row) * ld_dl + j] = T(__fmaf_rn(-gw, p, v));
}

// --------------------------------------------------------------------------
// backward: recompute the logit tile and turn it into dlogits in registers
// --------------------------------------------------------------------------
// A launch covers the chunks of one dW window, laid out and walked as in the
// forward (FwdArgs).
struct DlArgs {
  RowOp W;
  RowOp H;   // float32 path: rows of H from the first chunk's first
  ColOp Ht;  // bf16 path: the first chunk transposed, [d][C_pad]
  int kt;
  int tiles_t, tiles_v;  // token tiles of all the launch's chunks; vocabulary tiles
  int nch, C, nMt, nb;   // chunks, rows per chunk, token tiles and bucket offsets per full chunk
  int64_t ht_chunk;      // bytes from one chunk's transposed block to the next
  int rows, V, nVt;
  const int* offsets;  // bucket offsets of the first chunk: nVt + 1 per token tile, nb per chunk
  const uint2* recs;
  const float* lse;   // the rows' lse (forward output)
  const float* rowS;  // the rows' S_r
  const float* grad;  // device scalar: g, or g / Σw for the mean
  const float* w;     // the rows' per-token weights, or nullptr (all 1)
  void* dl;           // [rows, V_pad] of the compute dtype, token-major
  int64_t ld_dl;      // elements
};

template <bool BF16>
__device__ __forceinline__ DlArgs narrow(const DlArgs& a, const ChunkView& v) {
  typedef typename Elt<BF16>::T T;
  DlArgs n = a;
  const int64_t r0 = int64_t(v.c) * a.C;
  n.H.base += r0 * a.H.ld;
  n.H.rows = v.rows;
  n.Ht.base += int64_t(v.c) * a.ht_chunk;
  n.Ht.cbytes = v.rows * 2;
  n.rows = v.rows;
  n.offsets += int64_t(v.c) * a.nb;
  n.lse += r0;
  n.rowS += r0;
  if (a.w) n.w += r0;
  n.dl = static_cast<T*>(a.dl) + r0 * a.ld_dl;
  return n;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_bwd_dlogits(DlArgs args) {
  typedef typename Elt<BF16>::T T;
  __shared__ __attribute__((aligned(16))) char smem_raw[kSmemBytes];
  lds_t* smem = (lds_t*)(smem_raw);
  const int nblk = args.tiles_t * args.tiles_v;
  const int logical = xcd_logical(blockIdx.x, nblk);
  const ChunkView cv = chunk_view(logical, args.nch, args.C, args.nMt, args.rows, args.tiles_v);
  const DlArgs a = narrow<BF16>(args, cv);
  const int tt = cv.tt, vt = cv.vt;
  const int t_base = tt * kBN, v_base = vt * kBM;

  Acc acc;
  if constexpr (BF16)
    gemm_tile<BF16, RowDirect, RowOp, ColDirect, ColOp>(acc, a.W, v_base, a.Ht, t_base, 0, a.kt, smem);
  else
    gemm_tile<BF16, RowDirect, RowOp, RowDirect, RowOp>(acc, a.W, v_base, a.H, t_base, 0, a.kt, smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWM, wn = wave / kWM;
  const float g = *a.grad;
  const int vlim = a.V - (v_base + wm * kWTM);
  const TileHits hits = hits_begin(a.offsets, a.recs, tt * (a.nVt + 1) + vt, lane);

  // The per-token factors of the four 32-token column blocks.
  float lv[kTN], gsv[kTN];
#pragma unroll
  for (int b = 0; b < kTN; ++b) {
    const int tok = t_base + acc_col(wn, b, lane);
    const bool tok_ok = tok < a.rows;
    lv[b] = tok_ok ? a.lse[tok] : 0.f;
    gsv[b] = tok_ok ? g * (a.w ? a.w[tok] : 1.f) * a.rowS[tok] : 0.f;
  }
  const bool full = vlim >= kWTM;

  // Store, one 32-token column block at a time: the block is staged in LDS in
  // fp32 (token-major, the wave's 128 vocabulary entries contiguous), the
  // entries at cached ids become S_r q − p there, and the block leaves as
  // 16-byte pieces that cover each token's 128 entries in one contiguous run.
  // Only the chunk's own rows are written (the next chunk's rows follow
  // them); vocabulary entries past V are 0 and land in the row padding.
  T* dl = reinterpret_cast<T*>(a.dl);
  lds_f32* region = reinterpret_cast<lds_f32*>(smem) + wave * (kStageBlockBytes / 4);
  const int sub = lane >> 4, c8 = (lane & 15) * 8;  // store mapping: 4 tokens × 16 lanes
#pragma unroll
  for (int b = 0; b < kTN; ++b) {
    // dl = g S_r exp(z − lse_r), formed on the way into LDS; tokens past the
    // chunk give 0 (gs = 0). Vocabulary rows past V (only in the last
    // vocabulary tile) are set to 0 on the way out.
    stage_block_dl(acc, b, region, lane, lv[b], gsv[b]);
    for (int base = 0; base < hits.n; base += 64) {
      // Every lane holding a record of this block corrects its own entry
      // (the ids of a row are distinct, so no two lanes share a cell).
      const uint2 r = hits_load(hits, base, lane);
      const uint64_t mine = hits_mine(hits, r, base, wm, wn, lane);
      const int tok = int(r.x & 255u), voc = int((r.x >> 8) & 1023u);
      const int wc = tok - wn * kWTN;
      if (((mine >> lane) & 1) && (wc >> 5) == b) {
        const float gw = a.w ? g * a.w[t_base + tok] : g;
        lds_f32* cell = region + (wc & 31) * kColStride + voc - wm * kWTM;
        *cell = __fmaf_rn(-gw, __uint_as_float(r.y), *cell);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tl = sub + 4 * j;
      const int64_t tok = t_base + wn * kWTN + b * 32 + tl;
      const lds_f32* src = region + tl * kColStride + c8;
      f32x4_t v0 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>(src);
      f32x4_t v1 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>(src + 4);
      if (tok >= a.rows) continue;
      if (!full) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v0[e] = c8 + e < vlim ? v0[e] : 0.f;
          v1[e] = c8 + 4 + e < vlim ? v1[e] : 0.f;
        }
      }
      T* dst = dl + tok * a.ld_dl + v_base + wm * kWTM + c8;
      if constexpr (BF16) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]),
                                                    pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3]));
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(v0[0], v0[1], v0[2], v0[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(v1[0], v1[1], v1[2], v1[3]);
      }
    }
  }
}

// --------------------------------------------------------------------------
// dHᵀ = Wᵀ · dlᵀ   (A = W as [K=V][cols=d]; B = dl as [tokens][K=V_pad])
// --------------------------------------------------------------------------
struct DhArgs {
  ColOp W;
  RowOp dl;
  int tiles_t, tiles_d, splits, kt_total;
  int rows, d;
  void* dH;          // chunk rows of dH, used when splits == 1
  float* part;       // [splits, C_pad, d] fp32 partials, used when splits > 1
  int64_t part_stride;
};

template <bool BF16, class LA>
__global__ __launch_bounds__(kThreads) void k_bwd_dh(DhArgs a) {
  typedef typename Elt<BF16>::T T;
  __shared__ __attribute__((aligned(16))) char smem_raw[kSmemBytes];
  lds_t* smem = (lds_t*)(smem_raw);
  const int nblk = a.tiles_t * a.tiles_d * a.splits;
  const int logical = xcd_logical(blockIdx.x, nblk);
  const int tt = logical % a.tiles_t;
  const int rest = logical / a.tiles_t;
  const int dt = rest % a.tiles_d, split = rest / a.tiles_d;
  const int kt0 = int(int64_t(split) * a.kt_total / a.splits);
  const int kt1 = int(int64_t(split + 1) * a.kt_total / a.splits);
  const int d_base = dt * kBM, t_base = tt * kBN;

  Acc acc;
  gemm_tile<BF16, LA, ColOp, RowDirect, RowOp>(acc, a.W, d_base, a.dl, t_base, kt0, kt1, smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWM, wn = wave / kWM;
  // Full tiles of a split write their fp32 partial through LDS-staged
  // 32-token blocks: every store instruction covers two whole 512-byte runs.
  if (a.splits > 1 && t_base + kBN <= a.rows && d_base + kBM <= a.d) {
    lds_f32* region = reinterpret_cast<lds_f32*>(smem) + wave * (kStageBlockBytes / 4);
    const int vr = lane >> 5, c4 = (lane & 31) * 4;
    float* const part = a.part + split * a.part_stride;
#pragma unroll
    for (int b = 0; b < kTN; ++b) {
      stage_block_column(acc, b, region, lane);
      float* rows = part + int64_t(t_base + wn * kWTN + b * 32) * a.d + d_base + wm * kWTM + c4;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const f32x4_t x = *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>(
            region + (vr + 2 * j) * kColStride + c4);
        *reinterpret_cast<float4*>(rows + int64_t(vr + 2 * j) * a.d) = make_float4(x[0], x[1], x[2], x[3]);
      }
    }
    return;
  }
#pragma unroll
  for (int b = 0; b < kTN; ++b) {
    const int tok = t_base + acc_col(wn, b, lane);
    if (tok >= a.rows) continue;
#pragma unroll
    for (int t = 0; t < kTM; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dd = d_base + acc_row(wm, t, 4 * q, lane);
        if (dd >= a.d) continue;
        const int64_t o = int64_t(tok) * a.d + dd;
        const float4 v = make_float4(acc[t][b][4 * q], acc[t][b][4 * q + 1], acc[t][b][4 * q + 2],
                                     acc[t][b][4 * q + 3]);
        if (a.splits > 1) {
          *reinterpret_cast<float4*>(a.part + split * a.part_stride + o) = v;
        } else if constexpr (BF16) {
          *reinterpret_cast<uint2*>(reinterpret_cast<T*>(a.dH) + o) =
              make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<T*>(a.dH) + o) = v;
        }
      }
  }
}

// Sum the dH split partials in split order and write dH (4 elements per thread).
template <bool BF16>
__global__ __launch_bounds__(256) void k_bwd_dh_reduce(const float* __restrict__ part, int splits,
                                                       int64_t stride, int64_t n4, void* dH) {
  typedef typename Elt<BF16>::T T;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += int64_t(gridDim.x) * blockDim.x) {
    float4 s = reinterpret_cast<const float4*>(part)[i];
    for (int sp = 1; sp < splits; ++sp) {
      const float4 v = reinterpret_cast<const float4*>(part + sp * stride)[i];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    T* o = reinterpret_cast<T*>(dH) + 4 * i;
    o[0] = T(s.x);
    o[1] = T(s.y);
    o[2] = T(s.z);
    o[3] = T(s.w);
  }
}

// --------------------------------------------------------------------------
// dWᵀ (+)= H_cᵀ · dl   (A = H_c as [K=tokens][cols=d]; B = dl as [K=tokens][cols=V_pad])
// --------------------------------------------------------------------------
struct DwArgs {
  ColOp H;
  ColOp dl;
  int tiles_d, tiles_v, kt;
  int V, d;
  float* dW;
  int beta;  // 0: overwrite, 1: accumulate
};

// dW tiles are walked in groups of up to kDwGroup d tiles: inside a group d
// is fastest, then the vocabulary. The 32 tiles an XCD runs at once then
// share 6 slices of the H window (2 MB each at 4096 tokens) instead of all
// of them, which cuts dW's L2 misses by a quarter at the 8K head (same
// results: only the order of independent tiles changes).
constexpr int kDwGroup = 6;

template <bool BF16, class LC>
__global__ __launch_bounds__(kThreads) void k_bwd_dw(DwArgs a) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kSmemBytes];
  lds_t* smem = (lds_t*)(smem_raw);
  const int nblk = a.tiles_d * a.tiles_v;
  const int logical = xcd_logical(blockIdx.x, nblk);
  int dt, vt;
  {
    const int G = kDwGroup < a.tiles_d ? kDwGroup : a.tiles_d;
    const int full_groups = a.tiles_d / G;
    const int per_group = G * a.tiles_v;
    if (logical < full_groups * per_group) {
      const int grp = logical / per_group, r = logical % per_group;
      dt = grp * G + r % G;
      vt = r / G;
    } else {  // the last, narrower group of d tiles
      const int r = logical - full_groups * per_group;
      const int g2 = a.tiles_d - full_groups * G;
      dt = full_groups * G + r % g2;
      vt = r / g2;
    }
  }
  const int d_base = dt * kBM, v_base = vt * kBN;

  Acc acc;
  gemm_tile<BF16, LC, ColOp, LC, ColOp>(acc, a.H, d_base, a.dl, v_base, 0, a.kt, smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWM, wn = wave / kWM;
  // Full tiles: each 32-row vocabulary block of the wave is staged in LDS
  // (fp32, vocabulary-major), then read back so that every instruction
  // covers two whole 512-byte runs of dW rows; a block's 16 loads of the
  // old values are issued before the first add, so the read-modify-write
  // costs one memory round trip per block.
  const bool full = v_base + kBN <= a.V && d_base + kBM <= a.d;
  if (full) {
    lds_f32* region = reinterpret_cast<lds_f32*>(smem) + wave * (kStageBlockBytes / 4);
    const int vr = lane >> 5, c4 = (lane & 31) * 4;
#pragma unroll
    for (int b = 0; b < kTN; ++b) {
      stage_block_column(acc, b, region, lane);
      float* rows = a.dW + int64_t(v_base + wn * kWTN + b * 32) * a.d + d_base + wm * kWTM + c4;
      float4 old[16];
      if (a.beta) {
#pragma unroll
        for (int j = 0; j < 16; ++j) old[j] = *reinterpret_cast<const float4*>(rows + int64_t(vr + 2 * j) * a.d);
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) old[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const f32x4_t x = *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>(
            region + (vr + 2 * j) * kColStride + c4);
        *reinterpret_cast<float4*>(rows + int64_t(vr + 2 * j) * a.d) =
            make_float4(x[0] + old[j].x, x[1] + old[j].y, x[2] + old[j].z, x[3] + old[j].w);
      }
    }
    return;
  }
#pragma unroll
  for (int b = 0; b < kTN; ++b) {
    const int v = v_base + acc_col(wn, b, lane);
    if (v >= a.V) continue;
#pragma unroll
    for (int t = 0; t < kTM; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dd = d_base + acc_row(wm, t, 4 * q, lane);
        if (dd >= a.d) continue;
        float4* p = reinterpret_cast<float4*>(a.dW + int64_t(v) * a.d + dd);
        float4 x = make_float4(acc[t][b][4 * q], acc[t][b][4 * q + 1], acc[t][b][4 * q + 2],
                               acc[t][b][4 * q + 3]);
        if (a.beta) {
          const float4 y = *p;
          x.x += y.x;
          x.y += y.y;
          x.z += y.z;
          x.w += y.w;
        }
        *p = x;
      }
  }
}

// --------------------------------------------------------------------------
// offline teacher cache: top-K ids by logit and their full-softmax log-probs
// --------------------------------------------------------------------------
// The teacher runs once and keeps the most probable tokens of every position
// with their log-probabilities, not renormalised. One pass of the logit GEMM
// per chunk, whose float32 logits are kept for the chunk only (no [N, V] grid):
//   logits  k_fwd_logits<…, true>: per-tile (max, Σexp) of each row, and the
//           chunk's logits stored;
//   select  lse, and τ = the K-th largest tile maximum: at least K logits of
//           the row are ≥ τ, so every top-K logit is ≥ τ;
//   scan    every stored logit ≥ τ is appended to its row's candidate list;
//   finish  an exact radix select of the K-th largest (logit, −id) key among
//           the row's candidates, then a sort of the K winners.

// Order-preserving map of a float to an unsigned key, and back.
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// One wave per row: lse_r from the tile partials (fixed order) and τ_r, the
// K-th largest tile maximum (bit-by-bit search of its key), or −inf when the
// vocabulary has fewer than K tiles. Up to 64·kSelectRegs tiles per row
// (V ≤ 262,144) the keys are searched from registers.
constexpr int kSelectRegs = 16;
__global__ __launch_bounds__(256) void k_tk_select(const float2* __restrict__ part, int nVt,
                                                   int rows, int K, float* __restrict__ lse_out,
                                                   float* __restrict__ tau_out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float2* pr = part + int64_t(row) * nVt;
  float m = kNegInf, s = 0.f;
  for (int t = lane; t < nVt; t += 64) lse_merge(m, s, pr[t].x, pr[t].y);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    lse_merge(m, s, m2, s2);
  }
  float tau = kNegInf;
  if (nVt >= K) {
    uint32_t T = 0u;
    if (nVt <= 64 * kSelectRegs) {
      // The row's tile-maximum keys stay in registers (0 below every real
      // key) for the 32 steps of the search.
      uint32_t key[kSelectRegs];
#pragma unroll
      for (int q = 0; q < kSelectRegs; ++q) {
        const int t = lane + 64 * q;
        key[q] = t < nVt ? fkey(pr[t].x) : 0u;
      }
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = T | (1u << bit);
        int n = 0;
#pragma unroll
        for (int q = 0; q < kSelectRegs; ++q) n += key[q] >= c ? 1 : 0;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) n += __shfl_xor(n, off);
        if (n >= K) T = c;
      }
    } else {
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = T | (1u << bit);
        int n = 0;
        for (int t = lane; t < nVt; t += 64) n += fkey(pr[t].x) >= c ? 1 : 0;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) n += __shfl_xor(n, off);
        if (n >= K) T = c;
      }
    }
    tau = fkey_inv(T);
  }
  if (lane == 0) {
    lse_out[row] = m + __logf(s);
    tau_out[row] = tau;
  }
}

// Candidates from the chunk's stored logits ([rows][ld_z] float32): every
// z_rj ≥ τ_r with j < V joins row r's list as (float bits of z, id). A
// workgroup scans 8192 logits of one row (segment seg), as the one-pass
// dlogits pass does, and owns the list slots [seg·8192, seg·8192 + its
// count): a segment never holds more candidates than logits, so no slot is
// shared and no atomic is needed. The waves' hit counts are combined by a
// prefix sum over lanes and then over the four waves; the count goes to
// cnt[row·nseg + seg]. The set is exactly {j : z_rj ≥ τ_r}.
__global__ __launch_bounds__(256) void k_tk_scan(const float* __restrict__ z, int64_t ld_z,
                                                 int nseg, int V, int V_pad,
                                                 const float* __restrict__ tau,
                                                 int* __restrict__ cnt, uint2* __restrict__ cand,
                                                 int64_t cap) {
  __shared__ int wave_total[4];
  const int row = blockIdx.x / nseg, seg = blockIdx.x % nseg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float t = tau[row];
  const float* zr = z + int64_t(row) * ld_z;
  const int c0 = seg * kDlCols + threadIdx.x * 4;
  f32x4_t v[kDlGroups];
#pragma unroll
  for (int u = 0; u < kDlGroups; ++u) {
    const int c = c0 + u * 1024;
    v[u] = f32x4_t{kNegInf, kNegInf, kNegInf, kNegInf};
    if (c < V_pad) v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(zr + c));
  }
  const auto hit = [&](int u, int i) { return c0 + u * 1024 + i < V && v[u][i] >= t; };
  int n = 0;
#pragma unroll
  for (int u = 0; u < kDlGroups; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) n += hit(u, i) ? 1 : 0;
  int incl = n;  // inclusive prefix over the wave's lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_total[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    base += w < wave ? wave_total[w] : 0;
    total += wave_total[w];
  }
  if (threadIdx.x == 0) cnt[int64_t(row) * nseg + seg] = total;
  uint2* const cr = cand + int64_t(row) * cap + int64_t(seg) * kDlCols;
  int pos = base + incl - n;
#pragma unroll
  for (int u = 0; u < kDlGroups; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (hit(u, i)) cr[pos++] = make_uint2(__float_as_uint(v[u][i]), uint32_t(c0 + u * 1024 + i));
}

constexpr int kTkMaxK = int(kMaxTeacherK);  // the K winners are sorted in LDS

// 64-bit rank key of a candidate: larger logit first, then lower id.
__device__ __forceinline__ uint64_t tk_key(uint2 c) {
  return (uint64_t(fkey(__uint_as_float(c.x))) << 32) | uint64_t(0xFFFFFFFFu - c.y);
}

// One workgroup per row. With at most kTkMaxK candidates (the usual case)
// they are all sorted in LDS by a bitonic network; otherwise an 8-bit radix
// select finds the K-th largest key and the K keys at or above it (keys are
// unique, so exactly K) are gathered and sorted. The first K are written out
// with logp = z − lse. The candidates sit in nseg segments of 8192 slots
// (k_tk_scan); candidate i of the row is found through the segments' prefix
// sums, kept in LDS.
constexpr int kTkMaxSegs = int(kMaxTeacherSegs);  // the plan rejects larger vocabularies
__global__ __launch_bounds__(256) void k_tk_finish(const uint2* __restrict__ cand, int64_t cap,
                                                   const int* __restrict__ cnt, int nseg,
                                                   const float* __restrict__ lse, int K,
                                                   int32_t* __restrict__ idx_out,
                                                   float* __restrict__ logp_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t keys[kTkMaxK];
  __shared__ int seg_start[kTkMaxSegs + 1];
  __shared__ uint64_t s_prefix;
  __shared__ int s_krem, s_sel;
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint2* list = cand + int64_t(row) * cap;
  for (int sg = tid; sg < nseg; sg += 256) seg_start[sg + 1] = cnt[int64_t(row) * nseg + sg];
  if (tid == 0) {
    s_prefix = 0;
    s_krem = K;
    s_sel = 0;
  }
  __syncthreads();
  if (tid == 0) {
    seg_start[0] = 0;
    for (int sg = 0; sg < nseg; ++sg) seg_start[sg + 1] += seg_start[sg];
  }
  __syncthreads();
  const int n = seg_start[nseg];
  // Candidate i: the last segment starting at or before i holds it.
  const auto at = [&](int i) {
    int lo = 0, hi = nseg;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (seg_start[mid] <= i) lo = mid; else hi = mid;
    }
    return list[int64_t(lo) * kDlCols + (i - seg_start[lo])];
  };
  int m;  // keys gathered into LDS for the sort
  if (n <= kTkMaxK) {
    // Few candidates (the usual case: about K + 10): all of them are sorted
    // and the first K win; no selection pass is needed.
    for (int i = tid; i < n; i += 256) keys[i] = tk_key(at(i));
    m = n;
  } else {
    uint64_t mask = 0;
    for (int pass = 7; pass >= 0; --pass) {
      hist[tid] = 0u;
      __syncthreads();
      const uint64_t prefix = s_prefix;
      const int shift = 8 * pass;
      for (int i = tid; i < n; i += 256) {
        const uint64_t key = tk_key(at(i));
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int krem = s_krem, above = 0, bin = 255;
        for (; bin > 0; --bin) {
          if (above + int(hist[bin]) >= krem) break;
          above += int(hist[bin]);
        }
        s_krem = krem - above;
        s_prefix = prefix | (uint64_t(bin) << shift);
      }
      mask |= uint64_t(255) << shift;
      __syncthreads();
    }
    const uint64_t kth = s_prefix;
    for (int i = tid; i < n; i += 256) {
      const uint64_t key = tk_key(at(i));
      if (key >= kth) {
        const int slot = atomicAdd(&s_sel, 1);
        if (slot < kTkMaxK) keys[slot] = key;
      }
    }
    m = K;
  }
  __syncthreads();
  int P = 1;
  while (P < m) P <<= 1;
  for (int i = m + tid; i < P; i += 256) keys[i] = 0;  // below every real key
  __syncthreads();
  // Bitonic sort of keys[0, P), descending.
  for (int size = 2; size <= P; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P; i += 256) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;
          const uint64_t x = keys[i], y = keys[j];
          if (desc ? x < y : x > y) {
            keys[i] = y;
            keys[j] = x;
          }
        }
      }
      __syncthreads();
    }
  const float l = lse[row];
  for (int k = tid; k < K; k += 256) {
    const uint64_t key = keys[k];
    idx_out[int64_t(row) * K + k] = int32_t(0xFFFFFFFFu - uint32_t(key & 0xFFFFFFFFu));
    logp_out[int64_t(row) * K + k] = fkey_inv(uint32_t(key >> 32)) - l;
  }
}

// --------------------------------------------------------------------------
// debug check of the cache's preconditions (not on the hot path)
// --------------------------------------------------------------------------
constexpr int kCheckMaxK = 16384;  // power of two ≥ the largest K of the loss

// One workgroup per row: ids in range and log-probs ≤ 0 (or −inf, never NaN),
// then the row's ids sorted in LDS (bitonic, padded with INT_MAX) and
// neighbours compared for duplicates. Violations are OR-ed into *flags.
__global__ __launch_bounds__(256) void k_check_inputs(const int* __restrict__ idx,
                                                      const float* __restrict__ logp, int64_t N,
                                                      int K, int V, int* __restrict__ flags) {
  __shared__ int ids[kCheckMaxK];
  const int tid = threadIdx.x;
  int P = 1;
  while (P < K) P <<= 1;
  int bad = 0;
  // Rows are taken grid-stride (the grid is capped), one row at a time per
  // workgroup; the row index is uniform, so every barrier is reached by all.
  for (int64_t row = blockIdx.x; row < N; row += gridDim.x) {
    for (int k = tid; k < P; k += 256) {
      int j = 0x7FFFFFFF;
      if (k < K) {
        j = idx[row * K + k];
        const float lp = logp[row * K + k];
        if (j < 0 || j >= V) bad |= KD_CHECK_ID_RANGE;
        if (!(lp <= 0.f)) bad |= KD_CHECK_LOGP;  // positive, +inf or NaN
      }
      ids[k] = j;
    }
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < P; i += 256) {
          const int j = i ^ stride;
          if (j > i) {
            const bool up = (i & size) == 0;
            const int x = ids[i], y = ids[j];
            if (up ? x > y : x < y) {
              ids[i] = y;
              ids[j] = x;
            }
          }
        }
        __syncthreads();
      }
    for (int k = tid + 1; k < K; k += 256)
      if (ids[k] == ids[k - 1]) bad |= KD_CHECK_DUPLICATE;
    __syncthreads();  // the next row overwrites ids
  }
  if (bad) atomicOr(flags, bad);
}

// --------------------------------------------------------------------------
// host side: chunk scheduler
// --------------------------------------------------------------------------
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Ws {
  char* base;
  const Plan& p;
  template <class T>
  T* at(size_t off) const {
    return reinterpret_cast<T*>(base + off);
  }
};

int launch_status() { return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_HIP; }

// Optional kernel timing: when enabled, launches are bracketed by HIP events
// on the caller's stream and read back by kd_timing_read.
struct TimingRec {
  int cls;
  hipEvent_t a, b;
};
bool g_timing = false;
std::vector<hipEvent_t> g_event_pool;
size_t g_events_used = 0;
std::vector<TimingRec> g_timing_recs;

hipEvent_t timing_event() {
  if (g_events_used == g_event_pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_event_pool.push_back(e);
  }
  return g_event_pool[g_events_used++];
}

// Set while the no-allocation entry point runs on this thread: its launches
// are not bracketed by events (creating one may allocate).
thread_local bool t_no_events = false;

template <class F>
void timed(int cls, hipStream_t st, F&& launch) {
  if (!g_timing || t_no_events) {
    launch();
    return;
  }
  hipEvent_t a = timing_event(), b = timing_event();
  if (a) (void)hipEventRecord(a, st);
  launch();
  if (b) (void)hipEventRecord(b, st);
  if (a && b) g_timing_recs.push_back(TimingRec{cls, a, b});
}

// Buckets the cached entries of the group of chunks starting at row r0: two
// launches over (token tile, vocabulary slice) workgroups, with enough slices
// per tile that a group of few token tiles still spreads over the chip.
void launch_prep(const Plan& p, const Ws& ws, const int32_t* idx, const float* logp, int64_t r0,
                 hipStream_t st) {
  const int64_t left = p.N - r0, span_rows = p.prep_chunks * p.C;
  const int rows = int(left < span_rows ? left : span_rows);
  const int64_t ntiles = cdiv(rows, p.C) * p.nMt;
  int64_t slices = cdiv(kPrepTargetBlocks, ntiles);
  if (slices > p.nVt) slices = p.nVt;
  const int span = int(cdiv(p.nVt, slices));
  slices = cdiv(p.nVt, span);  // no empty slice
  const unsigned grid = unsigned(ntiles * slices);
  timed(KD_KERNEL_PREP, st, [&] {
    hipLaunchKernelGGL(k_prep_count, dim3(grid), dim3(kPrepThreads), 0, st, idx, logp, r0, rows,
                       int(p.C), int(p.nMt), int(p.K), int(p.V), int(p.nVt), span, int(slices),
                       ws.at<int>(p.off_counts), ws.at<float>(p.off_rowS), ws.at<int>(p.off_flag));
    hipLaunchKernelGGL(k_prep_scatter, dim3(grid), dim3(kPrepThreads), 0, st, idx, logp, r0, rows,
                       int(p.C), int(p.nMt), int(p.K), int(p.V), int(p.nVt), span, int(slices),
                       ws.at<int>(p.off_counts), ws.at<int>(p.off_offsets),
                       ws.at<uint2>(p.off_recs));
  });
}

// Bucket offsets and S_r of the chunk in slot `slot` of the current group.
inline int64_t prep_slot(const Plan& p, int64_t r0) { return (r0 / p.C) % p.prep_chunks; }

// The bf16 logit GEMMs stream each chunk of H as a column operand: the
// launch's chunks (`rows` rows from Hc on) are transposed, each into its own
// [d][C_pad] block, in one launch before the GEMM. Returns the first block.
ColOp chunks_transposed(const Plan& p, const Ws& ws, const char* Hc, int rows, hipStream_t st) {
  uint16_t* ht = ws.at<uint16_t>(p.off_ht);
  const int nch = int(cdiv(rows, p.C));
  timed(KD_KERNEL_PREP, st, [&] {
    hipLaunchKernelGGL(k_transpose16, dim3(cdiv(p.C_pad, 64), cdiv(p.d, 64), nch), dim3(256), 0,
                       st, reinterpret_cast<const uint16_t*>(Hc), p.d, rows, int(p.d), ht,
                       p.C_pad, int(p.C_pad), int(p.C), p.d * p.C_pad);
  });
  const int first = rows < p.C ? rows : int(p.C);
  return ColOp{reinterpret_cast<const char*>(ht), p.C_pad * 2, int(p.d), first * 2};
}

// The chunk-group fields shared by FwdArgs and DlArgs, for a launch over the
// chunks holding rows r0 .. r0 + rows − 1 (whole chunks but the last).
template <class Args>
void set_chunk_group(Args& a, const Plan& p, const void* H, const void* W, int64_t r0, int rows,
                     const ColOp& Ht) {
  const int64_t row_bytes = p.d * p.es;
  const int nch = int(cdiv(rows, p.C));
  a.W = RowOp{static_cast<const char*>(W), row_bytes, int(p.V), int(row_bytes)};
  a.H = RowOp{static_cast<const char*>(H) + r0 * row_bytes, row_bytes,
              rows < p.C ? rows : int(p.C), int(row_bytes)};
  a.Ht = Ht;
  a.kt = int(p.kt_d);
  a.nch = nch;
  a.C = int(p.C);
  a.nMt = int(p.nMt);
  a.nb = int(p.nbo);
  a.ht_chunk = p.d * p.C_pad * 2;
  a.tiles_t = int((nch - 1) * p.nMt + cdiv(rows - int64_t(nch - 1) * p.C, kBN));
  a.tiles_v = int(p.nVt);
  a.rows = rows;
  a.V = int(p.V);
  a.nVt = int(p.nVt);
}

void launch_reset(const Plan& p, const Ws& ws, hipStream_t st) {
  hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(64), 0, st, ws.at<int>(p.off_flag), int64_t(64), 0);
}

template <bool BF16>
using ColLoad = typename std::conditional<BF16, ColDirect, ColReg>::type;

template <bool BF16>
int run_fwd(const Plan& p, const void* H, const void* W, const int32_t* idx, const float* logp,
            const float* weight, int mean, float* loss_tok, float* lse, float* loss_sum,
            void* workspace, hipStream_t st) {
  Ws ws{static_cast<char*>(workspace), p};
  float* loss = loss_tok ? loss_tok : ws.at<float>(p.off_loss);
  if (p.N > 0) {
    launch_reset(p, ws, st);
    const int64_t row_bytes = p.d * p.es;
    const int64_t span = p.fwd_group * p.C;  // rows of one logit launch
    for (int64_t r0 = 0; r0 < p.N; r0 += span) {
      const int rows = int(p.N - r0 < span ? p.N - r0 : span);
      const int64_t slot = prep_slot(p, r0);
      if (slot == 0) launch_prep(p, ws, idx, logp, r0, st);
      FwdArgs a;
      set_chunk_group(a, p, H, W, r0, rows,
                      BF16 ? chunks_transposed(p, ws, static_cast<const char*>(H) + r0 * row_bytes,
                                               rows, st)
                           : ColOp{});
      a.K = int(p.K);
      a.offsets = ws.at<int>(p.off_offsets) + slot * p.nbo;
      a.recs = ws.at<uint2>(p.off_recs);
      a.zhit = ws.at<float>(p.off_zhit);
      a.part = ws.at<float2>(p.off_part);
      a.z = nullptr;
      a.ld_z = 0;
      timed(KD_KERNEL_FWD_LOGITS, st, [&] {
        hipLaunchKernelGGL((k_fwd_logits<BF16, false>), dim3(a.tiles_t * a.tiles_v),
                           dim3(kThreads), 0, st, a);
      });
      timed(KD_KERNEL_OTHER, st, [&] {
        hipLaunchKernelGGL(k_fwd_combine, dim3(cdiv(rows, 4)), dim3(256), 0, st, a.part, a.nVt,
                           a.zhit, nullptr, int64_t(0), idx, logp, r0, rows, a.K, a.V, lse, loss,
                           nullptr);
      });
    }
  }
  hipLaunchKernelGGL(k_loss_reduce, dim3(1), dim3(1024), 0, st, loss, weight, p.N, mean, loss_sum);
  return launch_status();
}

// dW and dH of one window of chunks whose dlogits rows ([krows][V_pad], the
// chunks back to back) are complete in the scratch. dW goes first: of two
// back-to-back heavy launches the second runs at a lower clock, and dH is the
// shorter one.
template <bool BF16>
void launch_window(const Plan& p, const Ws& ws, const void* H, const void* W, int64_t win_r0,
                   int krows, void* dH, float* dW, bool& dw_written, hipStream_t st) {
  const int64_t row_bytes = p.d * p.es;
  const int64_t dl_ld_bytes = p.V_pad * p.es;
  const int k_per_stage = kLdsRow / p.es;
  if (dW) {
    // dW (+)= dlᵀ H over the window's rows, in chunk order.
    DwArgs w;
    w.H = ColOp{static_cast<const char*>(H) + win_r0 * row_bytes, row_bytes, krows,
                int(row_bytes)};
    w.dl = ColOp{ws.at<char>(p.off_dl), dl_ld_bytes, krows, int(dl_ld_bytes)};
    w.tiles_d = int(cdiv(p.d, kBM));
    w.tiles_v = int(cdiv(p.V, kBN));
    w.kt = int(cdiv(krows, k_per_stage));
    w.V = int(p.V);
    w.d = int(p.d);
    w.dW = dW;
    w.beta = dw_written ? 1 : 0;
    timed(KD_KERNEL_BWD_DW, st, [&] {
      hipLaunchKernelGGL((k_bwd_dw<BF16, ColLoad<BF16>>), dim3(w.tiles_d * w.tiles_v),
                         dim3(kThreads), 0, st, w);
    });
    dw_written = true;
  }
  if (dH) {
    // dH of the window's rows = dl · W, split over the vocabulary.
    DhArgs h;
    h.W = ColOp{static_cast<const char*>(W), row_bytes, int(p.V), int(row_bytes)};
    h.dl = RowOp{ws.at<char>(p.off_dl), dl_ld_bytes, krows, int(dl_ld_bytes)};
    h.tiles_t = int(cdiv(krows, kBN));
    h.tiles_d = int(cdiv(p.d, kBM));
    h.splits = p.dh_splits;
    h.kt_total = int(p.kt_v);
    h.rows = krows;
    h.d = int(p.d);
    h.dH = static_cast<char*>(dH) + win_r0 * row_bytes;
    h.part = p.dh_splits > 1 ? ws.at<float>(p.off_dhpart) : nullptr;
    h.part_stride = p.win_rows_pad * p.d;
    timed(KD_KERNEL_BWD_DH, st, [&] {
      hipLaunchKernelGGL((k_bwd_dh<BF16, ColLoad<BF16>>), dim3(h.tiles_t * h.tiles_d * h.splits),
                         dim3(kThreads), 0, st, h);
    });
    if (p.dh_splits > 1) {
      const int64_t n4 = int64_t(krows) * p.d / 4;
      const int nb = int(cdiv(n4, 256) < 4096 ? cdiv(n4, 256) : 4096);
      timed(KD_KERNEL_OTHER, st, [&] {
        hipLaunchKernelGGL(k_bwd_dh_reduce<BF16>, dim3(nb), dim3(256), 0, st, h.part, h.splits,
                           h.part_stride, n4, h.dH);
      });
    }
  }
}

template <bool BF16>
int run_bwd(const Plan& p, const void* H, const void* W, const int32_t* idx, const float* logp,
            const float* weight, int mean, const float* lse, const float* grad, void* dH, float* dW,
            int accumulate, void* workspace, hipStream_t st) {
  Ws ws{static_cast<char*>(workspace), p};
  if (p.N == 0) {
    if (dW && !accumulate)
      hipLaunchKernelGGL(k_fill_f32, dim3(1024), dim3(256), 0, st, dW, p.V * p.d, 0.f);
    return launch_status();
  }
  launch_reset(p, ws, st);
  float* const gscale = ws.at<float>(p.off_gscale);
  hipLaunchKernelGGL(k_grad_scale, dim3(1), dim3(1024), 0, st, grad, weight, p.N, mean, gscale);
  const int64_t row_bytes = p.d * p.es;
  const int64_t span = int64_t(p.dw_window) * p.C;  // rows of one dW window
  bool dw_written = accumulate != 0;
  for (int64_t r0 = 0; r0 < p.N; r0 += span) {
    const int rows = int(p.N - r0 < span ? p.N - r0 : span);
    const int64_t slot = prep_slot(p, r0);
    if (slot == 0) launch_prep(p, ws, idx, logp, r0, st);
    // The window's dlogits, all its chunks in one launch, into the scratch
    // ([rows][V_pad], the chunks back to back).
    DlArgs a;
    set_chunk_group(a, p, H, W, r0, rows,
                    BF16 ? chunks_transposed(p, ws, static_cast<const char*>(H) + r0 * row_bytes,
                                             rows, st)
                         : ColOp{});
    a.offsets = ws.at<int>(p.off_offsets) + slot * p.nbo;
    a.recs = ws.at<uint2>(p.off_recs);
    a.lse = lse + r0;
    a.rowS = ws.at<float>(p.off_rowS) + slot * p.C;
    a.grad = gscale;
    a.w = weight ? weight + r0 : nullptr;
    a.dl = ws.at<char>(p.off_dl);
    a.ld_dl = p.V_pad;
    timed(KD_KERNEL_BWD_DLOGITS, st, [&] {
      hipLaunchKernelGGL(k_bwd_dlogits<BF16>, dim3(a.tiles_t * a.tiles_v), dim3(kThreads), 0, st,
                         a);
    });
    launch_window<BF16>(p, ws, H, W, r0, rows, dH, dW, dw_written, st);
  }
  return launch_status();
}

// Loss and gradients in one call. Per chunk: the logit GEMM stores the
// chunk's logits (float32) besides its partials; the combine gives lse_r, L_r
// and S_r; two streaming kernels turn the stored logits into the chunk's
// dlogits rows; dW and dH follow per window of chunks as in the backward.
template <bool BF16>
int run_fwd_bwd(const Plan& p, const void* H, const void* W, const int32_t* idx, const float* logp,
                const float* weight, int mean, const float* grad, float* loss_tok, float* lse,
                float* loss_sum, void* dH, float* dW, int accumulate, void* workspace,
                hipStream_t st) {
  Ws ws{static_cast<char*>(workspace), p};
  float* loss = loss_tok ? loss_tok : ws.at<float>(p.off_loss);
  if (p.N == 0) {
    if (dW && !accumulate)
      hipLaunchKernelGGL(k_fill_f32, dim3(1024), dim3(256), 0, st, dW, p.V * p.d, 0.f);
    hipLaunchKernelGGL(k_loss_reduce, dim3(1), dim3(1024), 0, st, loss, weight, p.N, mean,
                       loss_sum);
    return launch_status();
  }
  float* const gscale = ws.at<float>(p.off_gscale);
  hipLaunchKernelGGL(k_grad_scale, dim3(1), dim3(1024), 0, st, grad, weight, p.N, mean, gscale);
  const int64_t row_bytes = p.d * p.es;
  const int64_t dl_ld_bytes = p.V_pad * p.es;
  float* const z = ws.at<float>(p.off_z);
  float* const rowS = ws.at<float>(p.off_rowS);
  const int nseg = int(cdiv(p.V_pad, kDlCols));
  int64_t win_r0 = 0;
  int win_chunks = 0;
  bool dw_written = accumulate != 0;
  for (int64_t r0 = 0; r0 < p.N; r0 += p.C) {
    const int rows = int(p.N - r0 < p.C ? p.N - r0 : p.C);
    const char* Hc = static_cast<const char*>(H) + r0 * row_bytes;
    if (win_chunks == 0) win_r0 = r0;
    char* const dl_c = ws.at<char>(p.off_dl) + int64_t(win_chunks) * p.C * dl_ld_bytes;

    FwdArgs a;
    set_chunk_group(a, p, H, W, r0, rows, BF16 ? chunks_transposed(p, ws, Hc, rows, st) : ColOp{});
    a.K = int(p.K);
    a.offsets = nullptr;
    a.recs = nullptr;
    a.zhit = nullptr;
    a.part = ws.at<float2>(p.off_part);
    a.z = z;
    a.ld_z = p.V_pad;
    timed(KD_KERNEL_FWD_LOGITS, st, [&] {
      hipLaunchKernelGGL((k_fwd_logits<BF16, true>), dim3(a.tiles_t * a.tiles_v), dim3(kThreads),
                         0, st, a);
    });
    timed(KD_KERNEL_OTHER, st, [&] {
      hipLaunchKernelGGL(k_fwd_combine, dim3(cdiv(rows, 4)), dim3(256), 0, st, a.part, a.nVt,
                         nullptr, z, p.V_pad, idx, logp, r0, rows, a.K, a.V, lse, loss, rowS);
    });
    const float* const wc = weight ? weight + r0 : nullptr;
    timed(KD_KERNEL_DL_STREAM, st, [&] {
      hipLaunchKernelGGL(k_dl_dense<BF16>, dim3(unsigned(int64_t(rows) * nseg)), dim3(256), 0, st,
                         z, p.V_pad, lse + r0, rowS, gscale, wc, nseg, int(p.V), int(p.V_pad),
                         dl_c, p.V_pad);
      hipLaunchKernelGGL(k_dl_hits<BF16>, dim3(unsigned(cdiv(int64_t(rows) * p.K, 256))),
                         dim3(256), 0, st, z, p.V_pad, lse + r0, rowS, gscale, wc, idx, logp, r0,
                         rows, int(p.K), int(p.V), dl_c, p.V_pad);
    });

    ++win_chunks;
    const bool last = r0 + rows >= p.N;
    if (win_chunks == p.dw_window || last) {
      launch_window<BF16>(p, ws, H, W, win_r0, int(r0 + rows - win_r0), dH, dW, dw_written, st);
      win_chunks = 0;
    }
  }
  hipLaunchKernelGGL(k_loss_reduce, dim3(1), dim3(1024), 0, st, loss, weight, p.N, mean, loss_sum);
  return launch_status();
}

template <bool BF16>
int run_teacher(const Plan& p, const void* Ht, const void* Wt, int32_t* idx, float* logp,
                float* lse, void* workspace, hipStream_t st) {
  Ws ws{static_cast<char*>(workspace), p};
  if (p.N == 0) return KD_OK;
  const int64_t row_bytes = p.d * p.es;
  float* const z = ws.at<float>(p.off_z);
  float* const tau = ws.at<float>(p.off_tau);
  int* const cnt = ws.at<int>(p.off_cnt);
  uint2* const cand = ws.at<uint2>(p.off_cand);
  const int nseg = int(cdiv(p.V_pad, kDlCols));
  for (int64_t r0 = 0; r0 < p.N; r0 += p.C) {
    const int rows = int(p.N - r0 < p.C ? p.N - r0 : p.C);
    const char* Hc = static_cast<const char*>(Ht) + r0 * row_bytes;
    FwdArgs a;
    set_chunk_group(a, p, Ht, Wt, r0, rows, BF16 ? chunks_transposed(p, ws, Hc, rows, st) : ColOp{});
    a.K = int(p.K);
    a.offsets = nullptr;  // there are no cached ids
    a.recs = nullptr;
    a.zhit = nullptr;
    a.part = ws.at<float2>(p.off_part);
    a.z = z;
    a.ld_z = p.V_pad;
    timed(KD_KERNEL_FWD_LOGITS, st, [&] {
      hipLaunchKernelGGL((k_fwd_logits<BF16, true>), dim3(a.tiles_t * a.tiles_v), dim3(kThreads),
                         0, st, a);
    });
    float* const lse_c = lse ? lse + r0 : ws.at<float>(p.off_lse);
    timed(KD_KERNEL_OTHER, st, [&] {
      hipLaunchKernelGGL(k_tk_select, dim3(cdiv(rows, 4)), dim3(256), 0, st, a.part, a.nVt, rows,
                         int(p.K), lse_c, tau);
    });
    timed(KD_KERNEL_DL_STREAM, st, [&] {
      hipLaunchKernelGGL(k_tk_scan, dim3(unsigned(int64_t(rows) * nseg)), dim3(256), 0, st, z,
                         p.V_pad, nseg, int(p.V), int(p.V_pad), tau, cnt, cand, p.V_pad);
    });
    timed(KD_KERNEL_OTHER, st, [&] {
      hipLaunchKernelGGL(k_tk_finish, dim3(rows), dim3(256), 0, st, cand, p.V_pad, cnt, nseg,
                         lse_c, int(p.K), idx + r0 * p.K, logp + r0 * p.K);
    });
  }
  return launch_status();
}

inline bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// --------------------------------------------------------------------------
// library-held scratch of the no-allocation forward entry point
// --------------------------------------------------------------------------
// Every GPU the library runs on holds its own copy of this array from the
// moment the code object is loaded until the process ends. In host code the
// name is only a handle: its device address on the current device comes from
// hipGetSymbolAddress, looked up once per device and kept in g_scratch_ptr.
static __device__ __align__(256) char scratch[KD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's copy of `scratch`.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KD_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return KD_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KD_OK;
}

struct NoEventsScope {
  NoEventsScope() { t_no_events = true; }
  ~NoEventsScope() { t_no_events = false; }
};

// The forward call's argument checks and launches, for a plan of its shape.
int fwd_with_plan(const Plan& p, const void* H, const void* W, int dtype, const int32_t* topk_idx,
                  const float* topk_logp, const float* weight, int reduction, float* loss_tok,
                  float* lse, float* loss, void* workspace, size_t workspace_bytes, void* stream) {
  if (reduction != KD_REDUCE_SUM && reduction != KD_REDUCE_MEAN) return KD_ERR_INVALID_ARG;
  if (loss == nullptr || !aligned(loss, 4)) return KD_ERR_INVALID_ARG;
  if (p.N > 0) {
    if (!H || !W || !topk_idx || !topk_logp || !lse) return KD_ERR_INVALID_ARG;
    if (!aligned(H, 16) || !aligned(W, 16) || !aligned(topk_idx, 4) || !aligned(topk_logp, 4) ||
        !aligned(lse, 4) || (loss_tok && !aligned(loss_tok, 4)) || (weight && !aligned(weight, 4)))
      return KD_ERR_INVALID_ARG;
  }
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < p.total) return KD_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float* w = p.N > 0 ? weight : nullptr;
  const int mean = reduction == KD_REDUCE_MEAN;
  return dtype == KD_BF16 ? run_fwd<true>(p, H, W, topk_idx, topk_logp, w, mean, loss_tok, lse,
                                          loss, workspace, s)
                          : run_fwd<false>(p, H, W, topk_idx, topk_logp, w, mean, loss_tok, lse,
                                           loss, workspace, s);
}

}  // namespace
}  // namespace kd

// --------------------------------------------------------------------------
// C entry points
// --------------------------------------------------------------------------
extern "C" {

const char* kd_status_str(int status) {
  switch (status) {
    case KD_OK: return "KD_OK";
    case KD_ERR_INVALID_ARG: return "KD_ERR_INVALID_ARG";
    case KD_ERR_UNSUPPORTED: return "KD_ERR_UNSUPPORTED";
    case KD_ERR_WORKSPACE: return "KD_ERR_WORKSPACE";
    case KD_ERR_HIP: return "KD_ERR_HIP";
    default: return "KD_UNKNOWN_STATUS";
  }
}

size_t kd_fused_kl_workspace_bytes(int pass, int64_t N, int64_t d, int64_t V, int64_t K,
                                   int64_t chunk, int dtype) {
  kd::Plan p;
  if (kd::make_plan(pass, N, d, V, K, chunk, dtype, &p) != KD_OK) return 0;
  return p.total;
}

int kd_fused_kl_fwd_ex(const void* H, const void* W, int dtype, const int32_t* topk_idx,
                       const float* topk_logp, const float* weight, int reduction, int64_t N,
                       int64_t d, int64_t V, int64_t K, int64_t chunk, float* loss_tok, float* lse,
                       float* loss, void* workspace, size_t workspace_bytes, void* stream) {
  kd::Plan p;
  const int st = kd::make_plan(KD_PASS_FWD, N, d, V, K, chunk, dtype, &p);
  if (st != KD_OK) return st;
  return kd::fwd_with_plan(p, H, W, dtype, topk_idx, topk_logp, weight, reduction, loss_tok, lse,
                           loss, workspace, workspace_bytes, stream);
}

int kd_fused_kl_fwd_noalloc(const void* H, const void* W, int dtype, const int32_t* topk_idx,
                            const float* topk_logp, const float* weight, int reduction,
                            int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk,
                            float* loss_tok, float* lse, float* loss, void* stream) {
  kd::Plan p;
  int st = kd::make_plan(KD_PASS_FWD, N, d, V, K, chunk, dtype, &p);
  if (st != KD_OK) return st;
  // Past the scratch, one chunk per logit launch: the same results from a
  // smaller workspace.
  if (p.total > KD_NOALLOC_SCRATCH_BYTES) {
    st = kd::make_plan(KD_PASS_FWD, N, d, V, K, chunk, dtype, &p, 0);
    if (st != KD_OK) return st;
    if (p.total > KD_NOALLOC_SCRATCH_BYTES) return KD_ERR_WORKSPACE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return KD_ERR_HIP;
  if (s != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return KD_ERR_INVALID_ARG;
    if (int(sdev) != cur) return KD_ERR_INVALID_ARG;
  }
  void* ws = nullptr;
  const int got = kd::scratch_on_current_device(&ws);
  if (got != KD_OK) return got;
  kd::NoEventsScope no_events;
  return kd::fwd_with_plan(p, H, W, dtype, topk_idx, topk_logp, weight, reduction, loss_tok, lse,
                           loss, ws, KD_NOALLOC_SCRATCH_BYTES, stream);
}

int kd_fused_kl_fwd(const void* H, const void* W, int dtype, const int32_t* topk_idx,
                    const float* topk_logp, int64_t N, int64_t d, int64_t V, int64_t K,
                    int64_t chunk, float* loss_tok, float* lse, float* loss_sum, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return kd_fused_kl_fwd_ex(H, W, dtype, topk_idx, topk_logp, nullptr, KD_REDUCE_SUM, N, d, V, K,
                            chunk, loss_tok, lse, loss_sum, workspace, workspace_bytes, stream);
}

int kd_fused_kl_bwd_ex(const void* H, const void* W, int dtype, const int32_t* topk_idx,
                       const float* topk_logp, const float* weight, int reduction, const float* lse,
                       int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk,
                       const float* grad_loss, void* dH, float* dW, int dW_accumulate,
                       void* workspace, size_t workspace_bytes, void* stream) {
  kd::Plan p;
  const int st = kd::make_plan(KD_PASS_BWD, N, d, V, K, chunk, dtype, &p);
  if (st != KD_OK) return st;
  if (reduction != KD_REDUCE_SUM && reduction != KD_REDUCE_MEAN) return KD_ERR_INVALID_ARG;
  if (dW_accumulate != 0 && dW_accumulate != 1) return KD_ERR_INVALID_ARG;
  if (dW && !kd::aligned(dW, 16)) return KD_ERR_INVALID_ARG;
  if (N > 0) {
    if (!H || !W || !topk_idx || !topk_logp || !lse || !grad_loss) return KD_ERR_INVALID_ARG;
    if (!kd::aligned(H, 16) || !kd::aligned(W, 16) || !kd::aligned(topk_idx, 4) ||
        !kd::aligned(topk_logp, 4) || !kd::aligned(lse, 4) || !kd::aligned(grad_loss, 4) ||
        (dH && !kd::aligned(dH, 16)) || (weight && !kd::aligned(weight, 4)))
      return KD_ERR_INVALID_ARG;
  }
  if (!workspace || !kd::aligned(workspace, 256) || workspace_bytes < p.total)
    return KD_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int mean = reduction == KD_REDUCE_MEAN;
  return dtype == KD_BF16 ? kd::run_bwd<true>(p, H, W, topk_idx, topk_logp, weight, mean, lse,
                                              grad_loss, dH, dW, dW_accumulate, workspace, s)
                          : kd::run_bwd<false>(p, H, W, topk_idx, topk_logp, weight, mean, lse,
                                               grad_loss, dH, dW, dW_accumulate, workspace, s);
}

int kd_fused_kl_fwd_bwd(const void* H, const void* W, int dtype, const int32_t* topk_idx,
                        const float* topk_logp, const float* weight, int reduction, int64_t N,
                        int64_t d, int64_t V, int64_t K, int64_t chunk, const float* grad_loss,
                        float* loss_tok, float* lse, float* loss, void* dH, float* dW,
                        int dW_accumulate, void* workspace, size_t workspace_bytes, void* stream) {
  kd::Plan p;
  const int st = kd::make_plan(KD_PASS_FWD_BWD, N, d, V, K, chunk, dtype, &p);
  if (st != KD_OK) return st;
  if (reduction != KD_REDUCE_SUM && reduction != KD_REDUCE_MEAN) return KD_ERR_INVALID_ARG;
  if (dW_accumulate != 0 && dW_accumulate != 1) return KD_ERR_INVALID_ARG;
  if (loss == nullptr || !kd::aligned(loss, 4)) return KD_ERR_INVALID_ARG;
  if (dW && !kd::aligned(dW, 16)) return KD_ERR_INVALID_ARG;
  if (N > 0) {
    if (!H || !W || !topk_idx || !topk_logp || !lse || !grad_loss) return KD_ERR_INVALID_ARG;
    if (!kd::aligned(H, 16) || !kd::aligned(W, 16) || !kd::aligned(topk_idx, 4) ||
        !kd::aligned(topk_logp, 4) || !kd::aligned(lse, 4) || !kd::aligned(grad_loss, 4) ||
        (loss_tok && !kd::aligned(loss_tok, 4)) || (dH && !kd::aligned(dH, 16)) ||
        (weight && !kd::aligned(weight, 4)))
      return KD_ERR_INVALID_ARG;
  }
  if (!workspace || !kd::aligned(workspace, 256) || workspace_bytes < p.total)
    return KD_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float* w = N > 0 ? weight : nullptr;
  const int mean = reduction == KD_REDUCE_MEAN;
  return dtype == KD_BF16
             ? kd::run_fwd_bwd<true>(p, H, W, topk_idx, topk_logp, w, mean, grad_loss, loss_tok,
                                     lse, loss, dH, dW, dW_accumulate, workspace, s)
             : kd::run_fwd_bwd<false>(p, H, W, topk_idx, topk_logp, w, mean, grad_loss, loss_tok,
                                      lse, loss, dH, dW, dW_accumulate, workspace, s);
}

int kd_fused_kl_bwd(const void* H, const void* W, int dtype, const int32_t* topk_idx,
                    const float* topk_logp, const float* lse, int64_t N, int64_t d, int64_t V,
                    int64_t K, int64_t chunk, const float* grad_loss, void* dH, float* dW,
                    int dW_accumulate, void* workspace, size_t workspace_bytes, void* stream) {
  return kd_fused_kl_bwd_ex(H, W, dtype, topk_idx, topk_logp, nullptr, KD_REDUCE_SUM, lse, N, d, V,
                            K, chunk, grad_loss, dH, dW, dW_accumulate, workspace, workspace_bytes,
                            stream);
}

int kd_teacher_topk(const void* Ht, const void* Wt, int dtype, int64_t N, int64_t d, int64_t V,
                    int64_t K, int64_t chunk, int32_t* topk_idx, float* topk_logp, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream) {
  kd::Plan p;
  const int st = kd::make_plan(KD_PASS_TEACHER, N, d, V, K, chunk, dtype, &p);
  if (st != KD_OK) return st;
  if (N > 0) {
    if (!Ht || !Wt || !topk_idx || !topk_logp) return KD_ERR_INVALID_ARG;
    if (!kd::aligned(Ht, 16) || !kd::aligned(Wt, 16) || !kd::aligned(topk_idx, 4) ||
        !kd::aligned(topk_logp, 4) || (lse && !kd::aligned(lse, 4)))
      return KD_ERR_INVALID_ARG;
  }
  if (!workspace || !kd::aligned(workspace, 256) || workspace_bytes < p.total)
    return KD_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == KD_BF16
             ? kd::run_teacher<true>(p, Ht, Wt, topk_idx, topk_logp, lse, workspace, s)
             : kd::run_teacher<false>(p, Ht, Wt, topk_idx, topk_logp, lse, workspace, s);
}

int kd_fused_kl_check_inputs(const int32_t* topk_idx, const float* topk_logp, int64_t N,
                             int64_t K, int64_t V, int32_t* flags, void* stream) {
  if (N < 0 || K <= 0 || V <= 0 || K > V || K > kd::kMaxK || V > (int64_t(1) << 31) - 1)
    return KD_ERR_INVALID_ARG;
  if (N > (int64_t(1) << 31) - 1) return KD_ERR_UNSUPPORTED;
  if (!flags || !kd::aligned(flags, 4)) return KD_ERR_INVALID_ARG;
  if (N > 0 && (!topk_idx || !topk_logp || !kd::aligned(topk_idx, 4) || !kd::aligned(topk_logp, 4)))
    return KD_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(kd::k_fill_i32, dim3(1), dim3(64), 0, s, reinterpret_cast<int*>(flags),
                     int64_t(1), 0);
  if (N > 0)
    hipLaunchKernelGGL(kd::k_check_inputs, dim3(unsigned(N < 65536 ? N : 65536)), dim3(256), 0, s,
                       topk_idx, topk_logp, N, int(K), int(V), reinterpret_cast<int*>(flags));
  return kd::launch_status();
}

int kd_timing_enable(int enable) {
  if (enable != 0 && enable != 1) return KD_ERR_INVALID_ARG;
  kd::g_timing = enable == 1;
  return KD_OK;
}

int kd_timing_read(double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return KD_ERR_INVALID_ARG;
  for (int c = 0; c < KD_KERNEL_CLASSES; ++c) {
    total_ms[c] = 0.0;
    launches[c] = 0;
  }
  int st = KD_OK;
  for (const kd::TimingRec& r : kd::g_timing_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = KD_ERR_HIP;
      continue;
    }
    total_ms[r.cls] += ms;
    launches[r.cls] += 1;
  }
  kd::g_timing_recs.clear();
  kd::g_events_used = 0;
  return st;
}

int kd_scale(void* x, int dtype, int64_t n, const float* s, void* stream) {
  if (n < 0 || (dtype != KD_F32 && dtype != KD_BF16)) return KD_ERR_INVALID_ARG;
  if (n == 0) return KD_OK;
  if (!x || !s || !kd::aligned(x, dtype == KD_BF16 ? 2 : 4) || !kd::aligned(s, 4))
    return KD_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == KD_BF16)
    hipLaunchKernelGGL(kd::k_scale<true>, dim3(4096), dim3(256), 0, st, x, n, s);
  else
    hipLaunchKernelGGL(kd::k_scale<false>, dim3(4096), dim3(256), 0, st, x, n, s);
  return kd::launch_status();
}

int kd_cast_f32_to_bf16(const float* src, void* dst, int64_t n, void* stream) {
  if (n < 0) return KD_ERR_INVALID_ARG;
  if (n == 0) return KD_OK;
  if (!src || !dst || !kd::aligned(src, 4) || !kd::aligned(dst, 2)) return KD_ERR_INVALID_ARG;
  const char* s0 = reinterpret_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  if (d0 < s0 + 4 * n && s0 < d0 + 2 * n) return KD_ERR_INVALID_ARG;
  hipLaunchKernelGGL(kd::k_cast_f32_bf16, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream),
                     src, static_cast<__bf16*>(dst), n);
  return kd::launch_status();
}

}  // extern "C"
