// kd_gemm.h — the MFMA tile engine shared by the four contractions of the
// fused top-K KL loss on gfx950 (CDNA4):
//
//   logits      z  = H_c · Wᵀ      (forward, and recomputed in backward)
//   dH          dH = dl · W        (contraction over the vocabulary)
//   dW          dW = dlᵀ · H_c     (contraction over the chunk's rows)
//
// A workgroup of 256 threads (4 wave64s, 2×2) owns a 128×128 output tile;
// each wave owns 64×64 as 2×2 blocks of the 32×32 MFMA. The contraction is
// staged through LDS 128 bytes at a time (64 bf16 or 32 fp32 elements), two
// stages in flight. Every operand is staged in the same LDS layout — one
// 128-byte row per output row/column, contraction index contiguous, 16-byte
// chunks XOR-swizzled by the row — so the MFMA fragment reads never depend on
// how the operand sits in HBM:
//   RowLoader: operand stored [rows][K] (K contiguous): straight 16-byte copies.
//   ColLoader: operand stored [K][cols] (cols contiguous): four K-rows are
//              loaded per thread and transposed in registers on the way into
//              LDS, so the transposed operands of dH and dW need no copy in HBM.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kLdsRow = 128;  // bytes of contraction per LDS row and stage

// Physical 16-byte chunk of logical chunk c in LDS row `row`. XOR with the
// low three bits keeps eight consecutive rows (one MFMA fragment read) on
// distinct banks; XOR with the next three bits does the same for the strided
// rows written by the transposing loader.
__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7) ^ ((row >> 3) & 7); }

// Operand stored [rows][K], K contiguous. `ld` and `kbytes` are in bytes.
struct RowOp {
  const char* base;
  int64_t ld;
  int rows;    // valid rows; rows beyond read as zero
  int kbytes;  // valid bytes of K; beyond reads as zero (16-byte granularity)
};

// Operand stored [K][cols], cols contiguous. `ld` and `cbytes` are in bytes.
struct ColOp {
  const char* base;
  int64_t ld;
  int krows;   // valid K rows; beyond reads as zero
  int cbytes;  // valid bytes of a row; beyond reads as zero (16-byte granularity)
};

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int ROWS>
struct RowLoader {
  static constexpr int kPer = ROWS * (kLdsRow / 16) / kThreads;
  static_assert(kPer * kThreads == ROWS * (kLdsRow / 16), "tile rows must fill the workgroup");
  uint4 v[kPer];

  __device__ __forceinline__ void load(const RowOp& op, int r0, int kt, int tid) {
    const int kb0 = kt * kLdsRow;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = tid + i * kThreads;
      const int row = id >> 3, c = id & 7;
      const int gr = r0 + row, kb = kb0 + c * 16;
      if (gr < op.rows && kb < op.kbytes)
        v[i] = *reinterpret_cast<const uint4*>(op.base + int64_t(gr) * op.ld + kb);
      else
        v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = tid + i * kThreads;
      const int row = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(lds + row * kLdsRow + swz(row, c) * 16) = v[i];
    }
  }
};

template <bool BF16, int ROWS>
struct ColLoader {
  static constexpr int kEs = BF16 ? 2 : 4;
  static constexpr int kE = 16 / kEs;        // elements per 16-byte chunk
  static constexpr int kBK = kLdsRow / kEs;  // contraction elements per stage
  static constexpr int kNC = ROWS / kE;      // 16-byte chunks across the tile
  static constexpr int kUnits = (kBK / 4) * kNC;
  static constexpr int kPer = kUnits / kThreads;
  static_assert(kPer * kThreads == kUnits, "tile must fill the workgroup");
  uint4 v[kPer][4];

  __device__ __forceinline__ void load(const ColOp& op, int c0, int kt, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * kThreads;
      const int kq = u / kNC, nc = u % kNC;
      const int cb = (c0 + nc * kE) * kEs;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = kt * kBK + 4 * kq + j;
        if (k < op.krows && cb < op.cbytes)
          v[i][j] = *reinterpret_cast<const uint4*>(op.base + int64_t(k) * op.ld + cb);
        else
          v[i][j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * kThreads;
      const int kq = u / kNC, nc = u % kNC;
      const int kb = 4 * kq * kEs;  // byte offset of this thread's first K inside the row
      const int c = kb >> 4, sub = kb & 15;
      if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int n = nc * 8 + e;
          const uint32_t a0 = word(v[i][0], e >> 1), a1 = word(v[i][1], e >> 1);
          const uint32_t a2 = word(v[i][2], e >> 1), a3 = word(v[i][3], e >> 1);
          uint32_t x0, x1;
          if (e & 1) {
            x0 = (a0 >> 16) | (a1 & 0xffff0000u);
            x1 = (a2 >> 16) | (a3 & 0xffff0000u);
          } else {
            x0 = (a0 & 0xffffu) | (a1 << 16);
            x1 = (a2 & 0xffffu) | (a3 << 16);
          }
          *reinterpret_cast<uint2*>(lds + n * kLdsRow + swz(n, c) * 16 + sub) = make_uint2(x0, x1);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = nc * 4 + e;
          *reinterpret_cast<uint4*>(lds + n * kLdsRow + swz(n, c) * 16) =
              make_uint4(word(v[i][0], e), word(v[i][1], e), word(v[i][2], e), word(v[i][3], e));
        }
      }
    }
  }
};

// One 32×32 MFMA block step over 16 bytes of contraction per lane-half.
// bf16: one v_mfma_f32_32x32x16_bf16 (8 K-elements per lane).
// fp32: four v_mfma_f32_32x32x2_f32; the i-th uses element i of the chunk, so
// lane-half h covers K = 4h + i. A and B use the same assignment, so each of
// the 8 K-elements of the chunk pair is summed exactly once.
template <bool BF16>
__device__ __forceinline__ void mma(f32x16_t& acc, const uint4& a, const uint4& b) {
  if constexpr (BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
}

// Tile geometry: 128×128 per workgroup, 2×2 waves of 64×64, 2×2 MFMA blocks each.
constexpr int kBM = 128, kBN = 128, kWM = 2, kWN = 2;
constexpr int kWTM = kBM / kWM, kWTN = kBN / kWN;  // 64×64 per wave
constexpr int kTM = kWTM / 32, kTN = kWTN / 32;    // 2×2 MFMA blocks per wave
constexpr int kSmemBytes = 2 * (kBM + kBN) * kLdsRow;  // two stages: 64 KiB

typedef f32x16_t Acc[kTM][kTN];

// Position of accumulator element (tm, tn, i) of `lane` inside the 128×128
// tile, for the 32×32 MFMA output layout: lane owns column lane%32 and, per
// block, rows 8*(i/4) + 4*(lane/32) + i%4.
__device__ __forceinline__ int acc_row(int wm, int tm, int i, int lane) {
  return wm * kWTM + tm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}
__device__ __forceinline__ int acc_col(int wn, int tn, int lane) {
  return wn * kWTN + tn * 32 + (lane & 31);
}

// Inverse: which lane holds tile element (r, c) of the wave's 64×64 sub-tile,
// and at which flattened accumulator index.
__device__ __forceinline__ void acc_owner(int wr, int wc, int* lane, int* sel) {
  const int rr = wr & 31;
  *lane = (wc & 31) + 32 * ((rr >> 2) & 1);
  *sel = ((wr >> 5) * kTN + (wc >> 5)) * 16 + (rr & 3) + 4 * (rr >> 3);
}

__device__ __forceinline__ float acc_get(const Acc& acc, int sel) {
  float v = 0.f;
#pragma unroll
  for (int a = 0; a < kTM; ++a)
#pragma unroll
    for (int b = 0; b < kTN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) v = ((a * kTN + b) * 16 + i == sel) ? acc[a][b][i] : v;
  return v;
}

__device__ __forceinline__ void acc_sub(Acc& acc, int sel, float x) {
#pragma unroll
  for (int a = 0; a < kTM; ++a)
#pragma unroll
    for (int b = 0; b < kTN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((a * kTN + b) * 16 + i == sel) acc[a][b][i] -= x;
}

// acc = Σ over stages [kt0, kt1) of A-tile(a0) · B-tile(b0)ᵀ. Ends with a
// barrier, so the caller may reuse `smem` at once.
template <bool BF16, class LA, class OA, class LB, class OB>
__device__ __forceinline__ void gemm_tile(Acc& acc, const OA& oa, int a0, const OB& ob, int b0,
                                          int kt0, int kt1, char* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % kWM, wn = wave / kWM;
#pragma unroll
  for (int a = 0; a < kTM; ++a)
#pragma unroll
    for (int b = 0; b < kTN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
  if (kt0 >= kt1) return;

  LA la;
  LB lb;
  char* const stage0 = smem;
  char* const stage1 = smem + (kBM + kBN) * kLdsRow;
  la.load(oa, a0, kt0, tid);
  lb.load(ob, b0, kt0, tid);
  la.store(stage0, tid);
  lb.store(stage0 + kBM * kLdsRow, tid);
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    char* const cur = ((kt - kt0) & 1) ? stage1 : stage0;
    char* const nxt = ((kt - kt0) & 1) ? stage0 : stage1;
    const bool more = kt + 1 < kt1;
    if (more) {
      la.load(oa, a0, kt + 1, tid);
      lb.load(ob, b0, kt + 1, tid);
    }
    const char* As = cur;
    const char* Bs = cur + kBM * kLdsRow;
#pragma unroll
    for (int s = 0; s < kLdsRow / 32; ++s) {
      const int c = 2 * s + (lane >> 5);
      uint4 af[kTM], bfr[kTN];
#pragma unroll
      for (int a = 0; a < kTM; ++a) {
        const int row = wm * kWTM + a * 32 + (lane & 31);
        af[a] = *reinterpret_cast<const uint4*>(As + row * kLdsRow + swz(row, c) * 16);
      }
#pragma unroll
      for (int b = 0; b < kTN; ++b) {
        const int row = wn * kWTN + b * 32 + (lane & 31);
        bfr[b] = *reinterpret_cast<const uint4*>(Bs + row * kLdsRow + swz(row, c) * 16);
      }
#pragma unroll
      for (int a = 0; a < kTM; ++a)
#pragma unroll
        for (int b = 0; b < kTN; ++b) mma<BF16>(acc[a][b], af[a], bfr[b]);
    }
    if (more) {
      la.store(nxt, tid);
      lb.store(nxt + kBM * kLdsRow, tid);
    }
    __syncthreads();
  }
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i goes to
// XCD i % 8). Give each XCD a contiguous range of logical tiles, so tiles that
// share an operand slice run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_logical(int bid, int nblocks) {
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nblocks >> 3, rem = nblocks & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

}  // namespace kd
