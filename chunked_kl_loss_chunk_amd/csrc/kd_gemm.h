// kd_gemm.h — the MFMA tile engine shared by the four contractions of the
// fused top-K KL loss on gfx950 (CDNA4):
//
//   logits  zᵀ  = W · H_cᵀ      vocabulary × tokens   (forward; recomputed in backward)
//   dHᵀ         = Wᵀ · dlᵀ      d × tokens            (contraction over the vocabulary)
//   dWᵀ         = H_cᵀ · dl     d × vocabulary        (contraction over the chunk's tokens)
//
// The MFMA M dimension is the vocabulary (or d) and N is tokens (or the
// vocabulary), so each lane's four consecutive accumulator rows are four
// consecutive elements of a row-major output row: per-token reductions stay
// inside one lane plus one cross-half shuffle, and an epilogue that writes a
// whole output row stages 32-column blocks in LDS first.
//
// A workgroup of 256 threads (4 wave64s, 2×2) owns a 256×256 output tile;
// each wave owns 128×128 as 4×4 blocks of the 32×32 MFMA (256 fp32
// accumulators per lane). The contraction is staged through LDS 64 bytes per
// row at a time (32 bf16 or 16 fp32) in a ring of four stages (128 KiB of
// LDS), three of them in flight while the fourth is consumed. Operands are
// copied global→LDS by the LDS-DMA path (buffer_load ... lds, 16 bytes per lane,
// no VGPRs), in one of two layouts:
//
//   RowDirect  operand stored [rows][K] (K contiguous). LDS [256 rows][64 B],
//              16-byte chunks XOR-swizzled by the row; fragments are
//              ds_read_b128.
//   ColDirect  operand stored [K][cols] (cols contiguous), bf16. LDS [32 K][512 B]
//              as in HBM, 32-byte segments XOR-swizzled by K; fragments are
//              read transposed with ds_read_b64_tr_b16, so the transposed
//              operands of dH and dW need no copy in HBM and no VALU work.
//   ColReg     the fp32 form of ColDirect (no 32-bit transpose read exists):
//              four K-rows per thread are transposed in registers on their way
//              into the row layout.
//
// Operands are read through buffer resources whose record counts end at the
// operand's last valid row (or K-row): out-of-range rows, columns and K-tails
// read as zero, so partial tiles need no special cases.
//
// A DMA loader computes its lanes' offsets once per tile (init), gives the
// uniform resource of a stage (stage) and issues one of its kDma loads
// (issue); the pipeline spreads a stage's loads over the MFMA slots of a
// step. The register loader (ColReg) has no DMA and loads and writes a stage
// in fetch instead.
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
#ifndef KD_GEMM_ROW
#define KD_GEMM_ROW 64
#endif
constexpr int kLdsRow = KD_GEMM_ROW;                // contraction bytes per row and stage (64 or 128)
constexpr int kSteps = kLdsRow / 32;                // MFMA steps (16 bytes per lane-half) per stage
#ifndef KD_GEMM_STAGES
#define KD_GEMM_STAGES 4
#endif
constexpr int kStages = KD_GEMM_STAGES;             // ring of stages in LDS
constexpr int kOpBytes = kBM * kLdsRow;             // one operand tile per stage: 16 KiB
constexpr int kStageBytes = 2 * kOpBytes;           // A and B of one stage
constexpr int kSmemBytes = kStages * kStageBytes;   // 128 KiB with four stages

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
// c ^ rswz(row). A fragment read puts 8 (or 16) consecutive rows on the same
// logical chunk; rswz gives rows that share a 128-byte (256-byte) bank row
// distinct chunks. 64-byte rows: two (four) rows per bank row. 128-byte rows:
// one (two) per bank row.
__device__ __forceinline__ int rswz(int row) {
  if constexpr (kLdsRow == 64) return ((row >> 1) ^ (row >> 2)) & 3;
  return (row & 7) ^ ((row >> 3) & 1);
}

// Column layout: physical 32-byte segment of logical segment s in K-row k is
// s ^ cswz(k), cswz = {0, 2, 5, 7} over k mod 4. A transpose read touches
// four consecutive K-rows and two adjacent segments; these land on eight
// distinct segments of a 256-byte bank row and four distinct ones of each
// 128-byte half.
__device__ __forceinline__ int cswz(int k) { return ((k & 3) << 1) | ((k >> 1) & 1); }

// LDS-DMA through a buffer resource (buffer_load_dwordx4 ... lds): the
// resource holds a wave-uniform base and a byte count, each lane adds a 32-bit
// offset, and an offset at or beyond the count reads as zero without touching
// memory. So the per-lane offsets of a tile are computed once, each stage
// only moves the uniform base, and rows or K-tails outside the operand need
// no per-lane pointer arithmetic or selects.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kOOB = int(0x80000000u);  // an offset beyond every record count used here
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, 32-bit dwords, no swizzle

__device__ __forceinline__ rsrc_t make_rsrc(const char* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, nbytes, kRsrcWord3);
}
__device__ __forceinline__ void lds_dma16(rsrc_t rs, int voff, lds_t* dst_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, reinterpret_cast<lds_void_t*>(dst_wave_base), 16,
                                           voff, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t lds_read16(const lds_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(p);
}

__device__ __forceinline__ void lds_write16(lds_t* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(p) = u32x4_t{a, b, c, d};
}

// Transposed LDS read (ds_read_b64_tr_b16), issued as inline asm. As an
// intrinsic the compiler makes it wait for every in-flight LDS-DMA
// (vmcnt(0)), which would drain the stage pipeline; as asm it is ordered only
// by the pipeline's own explicit waits and barriers. The compiler does not
// track its completion either: callers wait with lds_wait_frags() before
// using the result.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_t lds_read_tr8(const lds_t* p) {
  u32x2_t v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(p));
  return v;
}

// --------------------------------------------------------------------------
// operand loaders
// --------------------------------------------------------------------------
struct RowDirect {
  static constexpr int kDma = kOpBytes / 1024 / 4;  // LDS-DMA instructions per wave and stage
  static constexpr int kChunks = kLdsRow / 16;       // 16-byte chunks per row
  static constexpr int kRowsPerBlk = 1024 / kLdsRow;
  // 256 rows × kLdsRow = blocks of 1 KiB (kRowsPerBlk rows); each wave copies
  // kDma blocks. Stage kt of the tile starting at row r0 is read from
  // base + r0·ld + kt·kLdsRow; lane offsets are row·ld + 16·chunk. The record
  // count stops at the tile's last valid row, so the offsets need
  // 256·ld < 2^31 (checked by the host).
  int voff[kDma];
  int rows_in;
  __device__ __forceinline__ void init(const RowOp& op, int r0, int wave, int lane) {
    const int left = op.rows - r0;
    rows_in = left < 0 ? 0 : left > kBM ? kBM : left;
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
      const int row = (wave * kDma + j) * kRowsPerBlk + lane / kChunks;
      const int c = (lane % kChunks) ^ rswz(row);  // logical chunk held at physical chunk lane%kChunks
      voff[j] = row * int(op.ld) + c * 16;
    }
  }
  __device__ __forceinline__ rsrc_t stage(const RowOp& op, int r0, int kt) const {
    const int kb0 = kt * kLdsRow;
    const int n = (kb0 < op.kbytes && rows_in > 0) ? rows_in * int(op.ld) - kb0 : 0;
    return make_rsrc(op.base + int64_t(r0) * op.ld + kb0, n);
  }
  // The K-tail of the last stage: chunks at or past kbytes read as zero.
  __device__ __forceinline__ void issue(rsrc_t rs, const RowOp& op, int kt, int j, lds_t* tile,
                                        int wave, int lane) const {
    int vo = voff[j];
    const int rem = op.kbytes - kt * kLdsRow;
    if (rem < kLdsRow) {
      const int row = (wave * kDma + j) * kRowsPerBlk + lane / kChunks;
      const int c = (lane % kChunks) ^ rswz(row);
      vo = c * 16 < rem ? vo : kOOB;
    }
    lds_dma16(rs, vo, tile + (wave * kDma + j) * 1024);
  }
  __device__ __forceinline__ void fetch(const RowOp&, int, int, lds_t*, int) {}
  __device__ __forceinline__ void commit(lds_t*, int) {}
  // Fragment of a 32-row block: lane l holds row rb + l%32, chunk 2s + l/32.
  __device__ static __forceinline__ u32x4_t frag(const lds_t* tile, int rb, int s, int lane) {
    const int row = rb + (lane & 31), c = 2 * s + (lane >> 5);
    return lds_read16(tile + row * kLdsRow + ((c ^ rswz(row)) << 4));
  }
  // Reads are whole fragments.
  static constexpr int kReads = 1;
  __device__ static __forceinline__ void frag_part(u32x4_t& f, const lds_t* tile, int rb, int s,
                                                   int, int lane) {
    f = frag(tile, rb, s, lane);
  }
};

struct ColDirect {  // bf16 only
  static constexpr int kK = kLdsRow / 2;            // contraction rows per stage (32 or 64)
  static constexpr int kDma = kOpBytes / 1024 / 4;  // LDS-DMA instructions per wave and stage
  // kK K-rows × 512 B = blocks of 2 K-rows (1 KiB); each wave copies kDma
  // blocks. Stage kt of the tile starting at column c0 is read from
  // base + kt·kK·ld + 2·c0; lane offsets are k·ld + byte, or kOOB for a
  // column past the operand. The record count stops at the last valid K-row,
  // so the offsets need kK·ld < 2^31 (checked by the host).
  int voff[kDma];
  __device__ __forceinline__ void init(const ColOp& op, int c0, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
      const int k = (wave * kDma + j) * 2 + (lane >> 5);
      const int lbyte = ((lane & 31) << 4) ^ (cswz(k) << 5);  // logical byte at physical (lane&31)*16
      voff[j] = c0 * 2 + lbyte < op.cbytes ? k * int(op.ld) + lbyte : kOOB;
    }
  }
  __device__ __forceinline__ rsrc_t stage(const ColOp& op, int c0, int kt) const {
    const int kv = op.krows - kt * kK;
    const int n = kv > 0 ? (kv < kK ? kv : kK) * int(op.ld) - c0 * 2 : 0;
    return make_rsrc(op.base + int64_t(kt) * kK * op.ld + c0 * 2, n);
  }
  __device__ __forceinline__ void issue(rsrc_t rs, const ColOp&, int, int j, lds_t* tile,
                                        int wave, int) const {
    lds_dma16(rs, voff[j], tile + (wave * kDma + j) * 1024);
  }
  __device__ __forceinline__ void fetch(const ColOp&, int, int, lds_t*, int) {}
  __device__ __forceinline__ void commit(lds_t*, int) {}
  // Fragment of a 32-column block cb..cb+31 at contraction step s (16 K):
  // lane l gets column cb + l%32 and K = 16s + 8(l/32) + 0..7, the same
  // assignment as RowDirect::frag, in two halves of four K. Each 16-lane
  // group reads a 4×16 block per ds_read_b64_tr_b16: lane L addresses K-row
  // L/4, columns 4(L%4)..+3, and receives column L of the four rows.
  static constexpr int kReads = 2;
  __device__ static __forceinline__ void frag_part(u32x4_t& f, const lds_t* tile, int cb, int s,
                                                   int half, int lane) {
    const int g = lane >> 4, L = lane & 15;
    const int colb = (cb + 16 * (g & 1) + 4 * (L & 3)) * 2;
    const int seg = colb >> 5, within = colb & 31;
    const int k = s * 16 + 8 * (g >> 1) + 4 * half + (L >> 2);
    const u32x2_t v = lds_read_tr8(tile + k * 512 + ((seg ^ cswz(k)) << 5) + within);
    if (half == 0) {
      f[0] = v[0];
      f[1] = v[1];
    } else {
      f[2] = v[0];
      f[3] = v[1];
    }
  }
};

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

struct ColReg {  // fp32 only: kLdsRow/4 K-rows per stage, 256 columns, row layout in LDS
  static constexpr int kDma = 0;
  static constexpr int kK = kLdsRow / 4;  // contraction rows per stage
  static constexpr int kPer = (kK / 4) * 64 / kThreads;
  // (kK/4) K-groups × (256/4) column chunks, kPer per thread. The load is
  // consumed at once (fp32 is the small, exact path, not the fast one).
  __device__ __forceinline__ void init(const ColOp&, int, int, int) {}
  __device__ __forceinline__ rsrc_t stage(const ColOp&, int, int) const { return make_rsrc(nullptr, 0); }
  __device__ __forceinline__ void issue(rsrc_t, const ColOp&, int, int, lds_t*, int, int) const {}
  __device__ __forceinline__ void fetch(const ColOp& op, int c0, int kt, lds_t* tile, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * kThreads;
      const int kq = u >> 6, nc = u & 63;
      const int cb = (c0 + nc * 4) * 4;
      uint4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = kt * kK + 4 * kq + j;
        if (k < op.krows && cb < op.cbytes)
          v[j] = *reinterpret_cast<const uint4*>(op.base + int64_t(k) * op.ld + cb);
        else
          v[j] = make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = nc * 4 + e;
        lds_write16(tile + n * kLdsRow + ((kq ^ rswz(n)) << 4), word(v[0], e), word(v[1], e),
                    word(v[2], e), word(v[3], e));
      }
    }
  }
  __device__ __forceinline__ void commit(lds_t*, int) {}
  static constexpr int kReads = 1;
  __device__ static __forceinline__ void frag_part(u32x4_t& f, const lds_t* tile, int rb, int s,
                                                   int, int lane) {
    f = RowDirect::frag(tile, rb, s, lane);
  }
};

// One 32×32 MFMA block step over 16 bytes of contraction per lane.
// bf16: one v_mfma_f32_32x32x16_bf16 (8 K-elements per lane).
// fp32: four v_mfma_f32_32x32x2_f32; the i-th takes element i of the chunk,
// so lane-half h covers K = 4h + i. A and B use the same assignment, so each
// of the 8 K-elements of a chunk pair is summed exactly once.
template <bool BF16>
__device__ __forceinline__ void mma(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
  if constexpr (BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc,
                                                 0, 0, 0);
  }
}

// Wait until every LDS-DMA and global load of this wave has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
// Wait until every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)

struct Frags {
  u32x4_t a[kTM], b[kTN];
};

// Wait for this wave's outstanding LDS reads; tying the fragment registers
// keeps every use of them after the wait.
__device__ __forceinline__ void lds_wait_frags(Frags& f) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0]),
                 "+v"(f.b[1]), "+v"(f.b[2]), "+v"(f.b[3]));
}

// The j-th LDS read of a step's fragments: A blocks first, then B blocks.
template <class LA, class LB>
__device__ __forceinline__ void issue_read(int j, Frags& f, const lds_t* A, const lds_t* B, int wm,
                                           int wn, int s, int lane) {
  constexpr int RA = LA::kReads, RB = LB::kReads;
  if (j < kTM * RA) {
    const int a = j / RA, h = j % RA;
    LA::frag_part(f.a[a], A, wm * kWTM + a * 32, s, h, lane);
  } else {
    const int jb = j - kTM * RA;
    const int b = jb / RB, h = jb % RB;
    LB::frag_part(f.b[b], B, wn * kWTN + b * 32, s, h, lane);
  }
}

// The LDS-DMA of one stage, spread over the MFMA slots of a step: with T
// loads per wave, slot j issues load j / (16/T) when j is the last slot of its
// group, so the address-free issue sits in the shadow of the MFMAs instead of
// stalling them in one block.
template <class LA, class OA, class LB, class OB>
struct StageLoads {
  static constexpr int kT = LA::kDma + LB::kDma;
  const LA& la;
  const LB& lb;
  const OA& oa;
  const OB& ob;
  rsrc_t ra, rb;
  int kt;
  lds_t* fill;
  int wave, lane;
  __device__ __forceinline__ void operator()(int j) const {
    if constexpr (kT > 0) {
      static_assert((kTM * kTN) % kT == 0, "loads spread evenly over the MFMA slots");
      constexpr int gap = kTM * kTN / kT;
      if (j % gap == gap - 1) {
        const int q = j / gap;
        if (q < LA::kDma) la.issue(ra, oa, kt, q, fill, wave, lane);
        else lb.issue(rb, ob, kt, q - LA::kDma, fill + kOpBytes, wave, lane);
      }
    }
  }
};
struct NoLoads {
  __device__ __forceinline__ void operator()(int) const {}
};

// One contraction step: the 16 MFMA block products on `cur`, with the reads
// of the fragments `nxt` for step s interleaved one per MFMA, and the hook's
// DMA issues after them. The order is pinned with scheduling barriers.
template <bool BF16, class LA, class LB, class Hook>
__device__ __forceinline__ void step(Acc& acc, const Frags& cur, Frags& nxt, const lds_t* A,
                                     const lds_t* B, int wm, int wn, int s, int lane,
                                     const Hook& hook) {
  constexpr int kReads = kTM * LA::kReads + kTN * LB::kReads;
  static_assert(kReads <= kTM * kTN, "one read per MFMA slot");
#pragma unroll
  for (int j = 0; j < kTM * kTN; ++j) {
    mma<BF16>(acc[j / kTN][j % kTN], cur.a[j / kTN], cur.b[j % kTN]);
    if (j < kReads) issue_read<LA, LB>(j, nxt, A, B, wm, wn, s, lane);
    hook(j);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// All reads of one step's fragments, for the pipeline prologue.
template <class LA, class LB>
__device__ __forceinline__ void read_all(Frags& f, const lds_t* A, const lds_t* B, int wm, int wn,
                                         int s, int lane) {
  constexpr int kReads = kTM * LA::kReads + kTN * LB::kReads;
#pragma unroll
  for (int j = 0; j < kReads; ++j) issue_read<LA, LB>(j, f, A, B, wm, wn, s, lane);
}

// Workgroup barrier without a memory fence. __syncthreads() also fences,
// which waits for every outstanding LDS-DMA of the wave (vmcnt(0)) and so
// would drain the whole pipeline; here the waits are explicit (wait_vmem_le,
// wait_lds) and the signal fences only stop the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void block_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until at most N LDS-DMA / global loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// acc = Σ over stages [kt0, kt1) of A-tile(a0) · B-tile(b0)ᵀ, where A rows are
// the M index and B rows the N index of the 256×256 tile; kt1 > kt0. Ends
// with a barrier, so the caller may reuse `smem` at once.
//
// LDS holds a ring of kStages stages. Every iteration issues the DMA of stage
// kt + kStages - 1 (past the end it fetches zeros into a slot nobody reads),
// so exactly (kStages - 2) stages' worth of DMA may stay in flight when the
// wave waits for stage kt + 1: the vmcnt threshold is a constant. Each step's
// MFMAs run while the next step's fragments are read; before the last step
// every wave waits for its DMA and its LDS reads and meets the others at the
// one barrier of the iteration, then reads the next stage's first fragments
// under the last step's MFMAs.
template <bool BF16, class LA, class OA, class LB, class OB>
__device__ __forceinline__ void gemm_tile(Acc& acc, const OA& oa, int a0, const OB& ob, int b0,
                                          int kt0, int kt1, lds_t* smem) {
  constexpr int kDma = LA::kDma + LB::kDma;
  static_assert(kSteps % 2 == 0, "steps alternate between two fragment sets");
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
  la.init(oa, a0, wave, lane);
  lb.init(ob, b0, wave, lane);
#pragma unroll
  for (int j = 0; j < kStages - 1; ++j) {
    lds_t* const st = smem + j * kStageBytes;
    const int k = kt0 + j;
    const rsrc_t ra = la.stage(oa, a0, k), rb = lb.stage(ob, b0, k);
#pragma unroll
    for (int q = 0; q < LA::kDma; ++q) la.issue(ra, oa, k, q, st, wave, lane);
#pragma unroll
    for (int q = 0; q < LB::kDma; ++q) lb.issue(rb, ob, k, q, st + kOpBytes, wave, lane);
    la.fetch(oa, a0, k, st, tid);
    lb.fetch(ob, b0, k, st + kOpBytes, tid);
    la.commit(st, tid);
    lb.commit(st + kOpBytes, tid);
  }
  wait_vmem_le<(kStages - 2) * kDma>();
  wait_lds();
  block_barrier();

  Frags f0, f1;
  read_all<LA, LB>(f0, smem, smem + kOpBytes, wm, wn, 0, lane);
  int slot = 0;  // ring slot of stage kt
  for (int kt = kt0; kt < kt1; ++kt) {
    const lds_t* const cur = smem + slot * kStageBytes;
    const int next_slot = slot + 1 == kStages ? 0 : slot + 1;
    const int fill_slot = slot == 0 ? kStages - 1 : slot - 1;  // held stage kt - 1
    lds_t* const fill = smem + fill_slot * kStageBytes;
    const int kf = kt + kStages - 1;
    const StageLoads<LA, OA, LB, OB> loads{la, lb, oa, ob, la.stage(oa, a0, kf), lb.stage(ob, b0, kf),
                                          kf, fill, wave, lane};
    la.fetch(oa, a0, kf, fill, tid);
    lb.fetch(ob, b0, kf, fill + kOpBytes, tid);
    lds_wait_frags(f0);
#pragma unroll
    for (int st = 0; st + 1 < kSteps; ++st) {
      if (st % 2 == 0) {
        if (st == 0)
          step<BF16, LA, LB>(acc, f0, f1, cur, cur + kOpBytes, wm, wn, st + 1, lane, loads);
        else
          step<BF16, LA, LB>(acc, f0, f1, cur, cur + kOpBytes, wm, wn, st + 1, lane, NoLoads{});
        if (st + 2 < kSteps) lds_wait_frags(f1);
      } else {
        step<BF16, LA, LB>(acc, f1, f0, cur, cur + kOpBytes, wm, wn, st + 1, lane, NoLoads{});
        lds_wait_frags(f0);
      }
    }
    la.commit(fill, tid);
    lb.commit(fill + kOpBytes, tid);
    wait_vmem_le<(kStages - 2) * kDma>();
    lds_wait_frags(f1);
    block_barrier();  // stage kt+1 landed everywhere; nobody reads stage kt any more
    const lds_t* const nxt = smem + next_slot * kStageBytes;
    step<BF16, LA, LB>(acc, f1, f0, nxt, nxt + kOpBytes, wm, wn, 0, lane, NoLoads{});
    slot = next_slot;
  }
  wait_vmem_le<0>();
  wait_lds();
  block_barrier();
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

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i goes to
// XCD i % 8). Give each XCD a contiguous range of logical tiles, so tiles that
// share an operand slice run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_logical(int bid, int nblocks) {
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nblocks >> 3, rem = nblocks & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

}  // namespace kd
