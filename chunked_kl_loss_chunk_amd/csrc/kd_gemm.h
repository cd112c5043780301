// kd_gemm.h — the MFMA tile engine shared by the four contractions of the
// fused top-K KL loss on gfx950 (CDNA4):
//
//   logits  zᵀ  = W · H_cᵀ      vocabulary × tokens   (forward; recomputed in backward)
//   dHᵀ         = Wᵀ · dlᵀ      d × tokens            (contraction over the vocabulary)
//   dWᵀ         = H_cᵀ · dl     d × vocabulary        (contraction over the chunk's tokens)
//
// The MFMA M dimension is the vocabulary (or d) and N is tokens (or the
// vocabulary), so each lane's four consecutive accumulator rows are four
// consecutive elements of the row-major output: the epilogues store 8 or 16
// bytes per lane, and per-token reductions stay inside one lane plus one
// cross-half shuffle.
//
// A workgroup of 256 threads (4 wave64s, 2×2) owns a 256×256 output tile;
// each wave owns 128×128 as 4×4 blocks of the 32×32 MFMA (256 fp32
// accumulators per lane). The contraction is staged through LDS 128 bytes per
// row at a time (64 bf16 or 32 fp32), two stages in flight (128 KiB of LDS).
// Operands are copied global→LDS by the LDS-DMA path (global_load_lds, 16
// bytes per lane, no VGPRs), in one of two layouts:
//
//   RowDirect  operand stored [rows][K] (K contiguous). LDS [256 rows][128 B],
//              16-byte chunks XOR-swizzled by the row; fragments are
//              ds_read_b128.
//   ColDirect  operand stored [K][cols] (cols contiguous), bf16. LDS [64 K][512 B]
//              as in HBM, 32-byte segments XOR-swizzled by K; fragments are
//              read transposed with ds_read_b64_tr_b16, so the transposed
//              operands of dH and dW need no copy in HBM and no VALU work.
//   ColReg     the fp32 form of ColDirect (no 32-bit transpose read exists):
//              four K-rows per thread are transposed in registers on their way
//              into the row layout.
//
// Out-of-range rows, columns and K-tails are fetched from a 64-byte block of
// zeros, so partial tiles need no special cases.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;

constexpr int kThreads = 256;
constexpr int kBM = 256, kBN = 256;                 // workgroup tile
constexpr int kWM = 2, kWN = 2;                     // waves along M and N
constexpr int kWTM = kBM / kWM, kWTN = kBN / kWN;   // 128×128 per wave
constexpr int kTM = kWTM / 32, kTN = kWTN / 32;     // 4×4 MFMA blocks per wave
constexpr int kLdsRow = 128;                    // contraction bytes per row and stage
constexpr int kOpBytes = kBM * kLdsRow;         // one operand tile per stage: 32 KiB
constexpr int kSmemBytes = 4 * kOpBytes;            // A and B, two stages: 128 KiB

// Source of out-of-range fetches.
__device__ __attribute__((aligned(64))) uint4 g_zero16[4];

typedef f32x16_t Acc[kTM][kTN];

// Operand stored [rows][K], K contiguous; `ld`, `kbytes` in bytes.
struct RowOp {
  const char* base;
  int64_t ld;
  int rows;    // valid rows; beyond read as zero
  int kbytes;  // valid bytes of K (multiple of 16); beyond read as zero
};

// Operand stored [K][cols], cols contiguous; `ld`, `cbytes` in bytes.
struct ColOp {
  const char* base;
  int64_t ld;
  int krows;   // valid K rows; beyond read as zero
  int cbytes;  // valid bytes of a row (multiple of 16); beyond read as zero
};

// Row layout: physical 16-byte chunk of logical chunk c in row `row` is
// c ^ rswz(row). Eight consecutive rows (one fragment read) hit eight
// different chunks; so do rows eight apart (the fp32 transposing writes).
__device__ __forceinline__ int rswz(int row) { return (row & 7) ^ ((row >> 3) & 7); }

// Column layout: physical 32-byte segment of logical segment s in K-row k is
// s ^ cswz(k), cswz = {0, 2, 5, 7} over k mod 4. A transpose read touches
// four consecutive K-rows and two adjacent segments; these land on eight
// distinct segments of a 256-byte bank row and four distinct ones of each
// 128-byte half.
__device__ __forceinline__ int cswz(int k) { return ((k & 3) << 1) | ((k >> 1) & 1); }

__device__ __forceinline__ void lds_dma16(const void* src, lds_t* dst_wave_base) {
  __builtin_amdgcn_global_load_lds(src, reinterpret_cast<__attribute__((address_space(3))) void*>(dst_wave_base), 16, 0, 0);
}

__device__ __forceinline__ uint4 lds_read16(const lds_t* p) {
  const u32x4_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void lds_write16(lds_t* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(p) = u32x4_t{a, b, c, d};
}

__device__ __forceinline__ uint2 lds_read_tr8(const lds_t* p) {
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(const_cast<lds_t*>(p)));
  return __builtin_bit_cast(uint2, v);
}

// --------------------------------------------------------------------------
// operand loaders
// --------------------------------------------------------------------------
struct RowDirect {
  // 256 rows × 128 B = 32 blocks of 8 rows (1 KiB); each wave copies 8 blocks.
  __device__ __forceinline__ void fetch(const RowOp& op, int r0, int kt, lds_t* tile, int wave,
                                        int lane, int) {
    const char* zero = reinterpret_cast<const char*>(g_zero16);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = wave * 8 + j;
      const int row = blk * 8 + (lane >> 3);
      const int c = (lane & 7) ^ rswz(row);  // logical chunk held at physical chunk lane&7
      const int gr = r0 + row, kb = kt * kLdsRow + c * 16;
      const char* src = (gr < op.rows && kb < op.kbytes) ? op.base + int64_t(gr) * op.ld + kb : zero;
      lds_dma16(src, tile + blk * 1024);
    }
  }
  __device__ __forceinline__ void commit(lds_t*, int) {}
  // Fragment of a 32-row block: lane l holds row rb + l%32, chunk 2s + l/32.
  __device__ static __forceinline__ uint4 frag(const lds_t* tile, int rb, int s, int lane) {
    const int row = rb + (lane & 31), c = 2 * s + (lane >> 5);
    return lds_read16(tile + row * kLdsRow + ((c ^ rswz(row)) << 4));
  }
};

struct ColDirect {  // bf16 only
  // 64 K-rows × 512 B = 32 blocks of 2 K-rows (1 KiB); each wave copies 8 blocks.
  __device__ __forceinline__ void fetch(const ColOp& op, int c0, int kt, lds_t* tile, int wave,
                                        int lane, int) {
    const char* zero = reinterpret_cast<const char*>(g_zero16);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = wave * 8 + j;
      const int k = blk * 2 + (lane >> 5);
      const int lbyte = ((lane & 31) << 4) ^ (cswz(k) << 5);  // logical byte at physical (lane&31)*16
      const int gk = kt * 64 + k, cb = c0 * 2 + lbyte;
      const char* src = (gk < op.krows && cb < op.cbytes) ? op.base + int64_t(gk) * op.ld + cb : zero;
      lds_dma16(src, tile + blk * 1024);
    }
  }
  __device__ __forceinline__ void commit(lds_t*, int) {}
  // Fragment of a 32-column block cb..cb+31 at contraction step s (16 K):
  // lane l gets column cb + l%32 and K = 16s + 8(l/32) + 0..7, the same
  // assignment as RowDirect::frag. Each 16-lane group reads a 4×16 block per
  // ds_read_b64_tr_b16: lane L addresses K-row L/4, columns 4(L%4)..+3, and
  // receives column L of the four rows.
  __device__ static __forceinline__ uint4 frag(const lds_t* tile, int cb, int s, int lane) {
    const int g = lane >> 4, L = lane & 15;
    const int colb = (cb + 16 * (g & 1) + 4 * (L & 3)) * 2;
    const int seg = colb >> 5, within = colb & 31;
    const int k0 = s * 16 + 8 * (g >> 1) + (L >> 2);
    const int k1 = k0 + 4;
    const uint2 lo = lds_read_tr8(tile + k0 * 512 + ((seg ^ cswz(k0)) << 5) + within);
    const uint2 hi = lds_read_tr8(tile + k1 * 512 + ((seg ^ cswz(k1)) << 5) + within);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
};

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

struct ColReg {  // fp32 only: 32 K-rows per stage, 256 columns, row layout in LDS
  static constexpr int kPer = 2;  // (32/4) K-groups × (256/4) chunks / 256 threads
  uint4 v[kPer][4];
  __device__ __forceinline__ void fetch(const ColOp& op, int c0, int kt, lds_t*, int, int, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * kThreads;
      const int kq = u >> 6, nc = u & 63;
      const int cb = (c0 + nc * 4) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = kt * 32 + 4 * kq + j;
        if (k < op.krows && cb < op.cbytes)
          v[i][j] = *reinterpret_cast<const uint4*>(op.base + int64_t(k) * op.ld + cb);
        else
          v[i][j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  __device__ __forceinline__ void commit(lds_t* tile, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * kThreads;
      const int kq = u >> 6, nc = u & 63;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = nc * 4 + e;
        lds_write16(tile + n * kLdsRow + ((kq ^ rswz(n)) << 4), word(v[i][0], e), word(v[i][1], e),
                    word(v[i][2], e), word(v[i][3], e));
      }
    }
  }
  __device__ static __forceinline__ uint4 frag(const lds_t* tile, int rb, int s, int lane) {
    return RowDirect::frag(tile, rb, s, lane);
  }
};

// One 32×32 MFMA block step over 16 bytes of contraction per lane.
// bf16: one v_mfma_f32_32x32x16_bf16 (8 K-elements per lane).
// fp32: four v_mfma_f32_32x32x2_f32; the i-th takes element i of the chunk,
// so lane-half h covers K = 4h + i. A and B use the same assignment, so each
// of the 8 K-elements of a chunk pair is summed exactly once.
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

// Wait until every LDS-DMA and global load of this wave has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
// Wait until every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)

// LDS reads one fragment of an operand costs: 1 (ds_read_b128) or 2 (transpose reads).
template <class L>
struct FragReads {
  static constexpr int n = 1;
};
template <>
struct FragReads<ColDirect> {
  static constexpr int n = 2;
};

struct Frags {
  uint4 a[kTM], b[kTN];
};

template <class LA, class LB>
__device__ __forceinline__ void read_frags(Frags& f, const lds_t* A, const lds_t* B, int wm, int wn,
                                           int s, int lane) {
#pragma unroll
  for (int a = 0; a < kTM; ++a) f.a[a] = LA::frag(A, wm * kWTM + a * 32, s, lane);
#pragma unroll
  for (int b = 0; b < kTN; ++b) f.b[b] = LB::frag(B, wn * kWTN + b * 32, s, lane);
}

template <bool BF16>
__device__ __forceinline__ void mma_step(Acc& acc, const Frags& f) {
#pragma unroll
  for (int a = 0; a < kTM; ++a)
#pragma unroll
    for (int b = 0; b < kTN; ++b) mma<BF16>(acc[a][b], f.a[a], f.b[b]);
}

// Ask the scheduler to interleave the next step's LDS reads with this step's
// MFMAs: one MFMA, one read, ..., then the remaining MFMAs.
template <bool BF16, int NREADS>
__device__ __forceinline__ void interleave_step() {
  constexpr int kMfma = kTM * kTN * (BF16 ? 1 : 4);
  constexpr int kPairs = NREADS < kMfma ? NREADS : kMfma;
#pragma unroll
  for (int j = 0; j < kPairs; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kPairs, 0);
}

// acc = Σ over stages [kt0, kt1) of A-tile(a0) · B-tile(b0)ᵀ, where A rows are
// the M index and B rows the N index of the 256×256 tile; kt1 > kt0. Ends
// with a barrier, so the caller may reuse `smem` at once.
//
// Per stage (4 contraction steps of 16 bytes per lane): the DMA of the next
// stage is issued first; each step's MFMAs run while the next step's
// fragments are read; before the last step every wave waits for its DMA and
// its LDS reads and meets the others at the one barrier of the stage, then
// reads the next stage's first fragments under the last step's MFMAs. The
// last stage is peeled so the steady-state loop has no branches.
template <bool BF16, class LA, class OA, class LB, class OB>
__device__ __forceinline__ void gemm_tile(Acc& acc, const OA& oa, int a0, const OB& ob, int b0,
                                          int kt0, int kt1, lds_t* smem) {
  constexpr int kReads = kTM * FragReads<LA>::n + kTN * FragReads<LB>::n;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWM, wn = wave / kWM;
#pragma unroll
  for (int a = 0; a < kTM; ++a)
#pragma unroll
    for (int b = 0; b < kTN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  LA la;
  LB lb;
  lds_t* const A0 = smem;
  lds_t* const B0 = smem + kOpBytes;
  lds_t* const A1 = smem + 2 * kOpBytes;
  lds_t* const B1 = smem + 3 * kOpBytes;
  la.fetch(oa, a0, kt0, A0, wave, lane, tid);
  lb.fetch(ob, b0, kt0, B0, wave, lane, tid);
  la.commit(A0, tid);
  lb.commit(B0, tid);
  wait_vmem();
  __syncthreads();

  Frags f0, f1;
  read_frags<LA, LB>(f0, A0, B0, wm, wn, 0, lane);
  int kt = kt0;
  for (; kt + 1 < kt1; ++kt) {
    const bool odd = (kt - kt0) & 1;
    const lds_t* const Ac = odd ? A1 : A0;
    const lds_t* const Bc = odd ? B1 : B0;
    lds_t* const An = odd ? A0 : A1;
    lds_t* const Bn = odd ? B0 : B1;
    la.fetch(oa, a0, kt + 1, An, wave, lane, tid);
    lb.fetch(ob, b0, kt + 1, Bn, wave, lane, tid);
    read_frags<LA, LB>(f1, Ac, Bc, wm, wn, 1, lane);
    mma_step<BF16>(acc, f0);
    interleave_step<BF16, kReads>();
    read_frags<LA, LB>(f0, Ac, Bc, wm, wn, 2, lane);
    mma_step<BF16>(acc, f1);
    interleave_step<BF16, kReads>();
    read_frags<LA, LB>(f1, Ac, Bc, wm, wn, 3, lane);
    mma_step<BF16>(acc, f0);
    interleave_step<BF16, kReads>();
    la.commit(An, tid);
    lb.commit(Bn, tid);
    wait_vmem();
    wait_lds();
    __syncthreads();  // next stage landed everywhere; nobody reads this stage any more
    read_frags<LA, LB>(f0, An, Bn, wm, wn, 0, lane);
    mma_step<BF16>(acc, f1);
    interleave_step<BF16, kReads>();
  }
  {
    const bool odd = (kt - kt0) & 1;
    const lds_t* const Ac = odd ? A1 : A0;
    const lds_t* const Bc = odd ? B1 : B0;
    read_frags<LA, LB>(f1, Ac, Bc, wm, wn, 1, lane);
    mma_step<BF16>(acc, f0);
    interleave_step<BF16, kReads>();
    read_frags<LA, LB>(f0, Ac, Bc, wm, wn, 2, lane);
    mma_step<BF16>(acc, f1);
    interleave_step<BF16, kReads>();
    read_frags<LA, LB>(f1, Ac, Bc, wm, wn, 3, lane);
    mma_step<BF16>(acc, f0);
    interleave_step<BF16, kReads>();
    mma_step<BF16>(acc, f1);
  }
  __syncthreads();
}

// Position of accumulator element (a, b, i) of `lane` inside the 256×256
// tile, for the 32×32 MFMA output layout: per block, lane owns column lane%32
// and rows 8(i/4) + 4(lane/32) + i%4.
__device__ __forceinline__ int acc_row(int wm, int a, int i, int lane) {
  return wm * kWTM + a * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}
__device__ __forceinline__ int acc_col(int wn, int b, int lane) {
  return wn * kWTN + b * 32 + (lane & 31);
}

// Inverse for element (wr, wc) of a wave's 128×128 sub-tile: the owning lane,
// the (uniform) block index a*kTN + b, and the register inside the block.
struct Owner {
  int lane, blk, reg;
};
__device__ __forceinline__ Owner acc_owner(int wr, int wc) {
  const int rr = wr & 31;
  Owner o;
  o.lane = (wc & 31) + 32 * ((rr >> 2) & 1);
  o.blk = (wr >> 5) * kTN + (wc >> 5);
  o.reg = (rr & 3) + 4 * (rr >> 3);
  return o;
}

// Apply f(block, register-select) to the one accumulator block `blk`
// (wave-uniform): a uniform branch per block, a 16-way select inside it.
template <class F>
__device__ __forceinline__ void acc_visit(Acc& acc, int blk, F&& f) {
#pragma unroll
  for (int a = 0; a < kTM; ++a)
#pragma unroll
    for (int b = 0; b < kTN; ++b)
      if (blk == a * kTN + b) f(acc[a][b]);
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
