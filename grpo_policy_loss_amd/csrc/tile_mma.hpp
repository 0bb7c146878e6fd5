// tile_mma.hpp -- the MFMA tile main loop shared by every GEMM-shaped kernel.
//
// Computes one 256 x 256 float32 tile of C[m][n] = sum_k A[m][k] * B[n][k]
// (both operands "K-contiguous": row m of A and row n of B are contiguous
// along k), on gfx950 (CDNA4) matrix cores.
//
// Layout and schedule:
//  * 256 threads = 4 wave64s, one per SIMD, in a 2 (M) x 2 (N) grid; each wave
//    owns 128 x 128 of the tile as 8 x 8 blocks of the 16 x 16 MFMA output
//    (256 accumulator registers per lane, which the compiler keeps in AGPRs).
//    The 128 x 128 wave tile needs a third less LDS fragment traffic than
//    eight 128 x 64 wave tiles, and that data movement costs clock: the chip
//    is power-limited under this load.
//  * K advances in 128-byte slices (64 bf16 or 32 f32), two k-steps of 64 bytes
//    each.  Each slice of A and B (256 rows x 128 B = 32 KB each) is copied
//    global -> LDS by the buffer unit directly (buffer_load_dwordx4 ... lds):
//    no VGPR staging.  A has three slice slots and B two (160 KB in all).
//  * Slice kt: k-step 0 runs its 64 MFMAs, reads the fragments of k-step 1
//    and copies A's slice kt + 2 into the third A slot (free since slice
//    kt - 1 was consumed); then the slice barrier; k-step 1 runs its MFMAs,
//    reads the fragments of slice kt + 1's k-step 0, and copies B's slice
//    kt + 2 into the B slot that slice kt just left.  Each k-step thus carries
//    8 copies and 16 fragment reads per wave, and every copy moves whole
//    128-byte lines.  (With two slots for each operand all 16 copies of a
//    slice fall into k-step 1, which then has twice the LDS and buffer-unit
//    traffic of k-step 0; the even spread measured 2 to 6 % less kernel time.
//    Four stages of one 64-byte k-step each spread the copies as well, but
//    fetch half lines of K-contiguous rows and were 5 to 6.5 % slower there.)
//  * Every instruction of a k-step is placed by hand (scheduling fences): a
//    fragment read after each even MFMA of its first half and a copy after
//    MFMA q for q mod 8 = kCopyAt.  Left to itself the compiler clusters the
//    copies (each needs its own M0 write) and the matrix core idles.
//  * With one wave per SIMD, whatever sits between two MFMAs must issue within
//    the 16 cycles of the first one.  A copy of a slice that lies wholly inside
//    k therefore costs no vector instruction: each lane's row-and-chunk offset
//    is computed once, the slice offset rides in the scalar offset, and only
//    M0 changes per copy.  The per-lane k-bound check (three VALU operations
//    per copy, measured 3 to 5 points of peak) is left to the slices at and
//    past the k tail.
//  * Slice barrier after the first k-step: every wave then holds the slice's
//    last fragments, so its B slot is free for the copy of slice kt + 2, and
//    (after each wave's own vmcnt wait) slice kt + 1 is visible.  A copy of
//    A has two to three k-steps to land before it is waited for, one of B
//    one to two.
//  * Out-of-range rows and k-columns read as zero: each operand is addressed
//    through a buffer resource whose range ends at its last valid row, and an
//    invalid row or column gets an offset past that range.  Tails in M, N
//    and K therefore need no separate code path.
//  * gfx950's LDS serves 256 bytes per clock, i.e. one ds_read_b128 cycle
//    covers 16 lanes = 16 rows of a fragment.  The eight 16-byte chunks of a
//    128-byte LDS row are XOR-swizzled by f(r) = (r & 7) ^ ((r >> 3) & 1), so
//    any 16 consecutive rows at one logical chunk hit 16 distinct bank groups.
//  * bf16: v_mfma_f32_16x16x32_bf16; lane l supplies row l % 16 of A (of B)
//          and the 16-byte chunk l / 16 of the 64-byte k-step.
//    f32:  v_mfma_f32_16x16x4_f32, four per k-step; lane l supplies element e
//          of its 4-float chunk l / 16 to MFMA e, so the four MFMAs together
//          cover the 16 k of the step (in a permuted k order that A and B share).
//
//  * Either operand may instead be "K-major": stored k-row by k-row, the tile's
//    256 rows (m or n) contiguous within each k-row (so an operand that is read
//    transposed needs no transposed copy in memory).  A slice is then 64 k-rows
//    (bf16; 32 for f32) of 512 B, copied by the same buffer-to-LDS instructions
//    (two k-rows per instruction), its 32-byte blocks XOR-swizzled by the k-row.
//    bf16 fragments come out of LDS through gfx950's transposing read
//    ds_read_b64_tr_b16: within each 16-lane group, lane s addresses the four
//    rows 4 (s % 4) .. + 3 of k-row s / 4 and receives element i of its own row
//    at k-row i, so two such reads (k-rows +0..3 and +4..7) give a lane the
//    eight consecutive k of its row that the MFMA takes.  The swizzle puts the
//    eight k-rows a half-wave reads at one column into eight distinct 32-byte
//    bank groups.  f32 fragments take four 4-byte reads.
//
// Output register layout (both MFMAs): lane l of wave w, block (i, j),
// element e holds C[128 (w / 2) + 16 i + 4 (l / 16) + e][128 (w % 2) + 16 j + l % 16].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grpo {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

#define GRPO_LDS __attribute__((address_space(3)))

constexpr int kBM = 256;          // tile rows (A rows)
constexpr int kBN = 256;          // tile cols (B rows)
constexpr int kBKB = 128;         // K slice in bytes
constexpr int kThreads = 256;
constexpr int kWM = 8;            // 16-row MFMA blocks per wave
constexpr int kWN = 8;            // 16-col MFMA blocks per wave
constexpr int kAcc = 4;           // accumulator values per block and lane
constexpr int kTileBytes = kBM * kBKB;   // one operand slice in LDS: 32 KB
constexpr int kASlots = 3, kBSlots = 2;
constexpr int kBRegion = kASlots * kTileBytes;                // B's slots follow A's
constexpr int kLdsBytes = (kASlots + kBSlots) * kTileBytes;   // 160 KB
constexpr uint32_t kOOB = 0x80000000u;   // an offset past every resource range
// Cache policy of the slice copies: sc1 (device scope) takes them past the per-CU L1.
// Each workgroup streams its panels once per slice, so L1 allocation buys nothing;
// measured +1 to +3 points of bf16 peak on the tile GEMM.  (nt, the streaming hint,
// costs 6 points: the L2 then stops keeping panels that neighbouring CUs reuse.)
constexpr int kCopyPolicy = 16;

typedef f32x4_t Acc[kWM][kWN];

// Number of 128-byte K slices that cover `bytes` of k.
__host__ __device__ constexpr int k_slices_of(int64_t bytes) {
  return (int)((bytes + kBKB - 1) / kBKB);
}

// Raw buffer resource: base, no stride, `bytes` valid bytes from base.  The
// inputs are workgroup-uniform; readfirstlane makes that visible to the
// compiler so the descriptor lives in SGPRs (otherwise every buffer
// instruction is wrapped in a waterfall loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// One operand's view for the loader.
// K-contiguous (the default): rows [row0, row0 + rows_valid) of a row-major
// matrix with row pitch `ld_bytes`, k-bytes [0, k_bytes) valid.
// K-major: `base` is the tile's first row (m or n) at k = 0, `ld_bytes` the
// pitch between consecutive k, k-rows [0, k_rows) are valid and `range` is the
// number of readable bytes from base (at most 2^31 - 1); everything past it
// reads as zero.  (k_rows + 192) * ld_bytes must stay below 2^32 and 256
// ld_bytes below 2^31.  Tile rows past the operand's end are read unmasked.
struct Operand {
  const char* base;
  uint32_t ld_bytes;
  int rows_valid;        // rows of this tile that exist (may be <= 0)
  uint32_t k_bytes;      // K-contiguous: valid k extent in bytes (multiple of 16)
  uint32_t k_rows = 0;   // K-major: valid k
  uint32_t range = 0;    // K-major, and K-contiguous with blk_stride: readable bytes from base
  // K-contiguous, blocked along k: k is stored in blocks of 256 elements, block
  // b of a row at base + b * blk_stride + row * ld_bytes (0: one block).  Rows
  // are then read unmasked within `range` (they feed only output rows the
  // caller does not store).
  uint32_t blk_stride = 0;
};

// Each wave copies 64 rows of an operand slice: 8 DMA instructions, each
// moving 8 rows x 128 B (lane i fills slot i & 7 of row i >> 3 of the group).
// BLK: the operand is blocked along k (Operand::blk_stride).
template <bool BLK = false>
struct Loader {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t chunk_bytes;     // logical 16-byte chunk this lane copies, even 8-row groups
  uint32_t chunk_bytes_odd; // the same for odd 8-row groups (f(r) flips bit 0)
  uint32_t k_bytes;
  uint32_t blk_stride;      // blocked k (see Operand); 0 for one block
  int blk_shift;            // log2 of the slices per block
  uint32_t voff[8];         // byte offset of this lane's row j plus its chunk (kOOB if absent)

  // byte offset of slice kt from the row start
  __device__ __forceinline__ uint32_t slice_off(int kt) const {
    if (!BLK) return (uint32_t)kt * kBKB;
    return (uint32_t)(kt >> blk_shift) * blk_stride +
           (uint32_t)(kt & ((1 << blk_shift) - 1)) * kBKB;
  }
  __device__ __forceinline__ void init(const Operand& op, int wave, int lane, int elem_bytes) {
    int rv = op.rows_valid < 0 ? 0 : (op.rows_valid > kBM ? kBM : op.rows_valid);
    if (BLK) {
      blk_stride = (uint32_t)__builtin_amdgcn_readfirstlane(op.blk_stride);
      blk_shift = elem_bytes == 4 ? 3 : 2;   // a 256-element block is 8 (f32) or 4 (bf16) slices
      rv = kBM;                              // unmasked rows, bounded by the range
    }
    rsrc = make_rsrc(op.base, BLK ? op.range : (uint32_t)rv * op.ld_bytes);
    const int r_in = lane >> 3;                          // row within an 8-row group
    chunk_bytes = (uint32_t)(((lane & 7) ^ r_in) << 4);  // slot lane & 7 holds chunk slot ^ f(r)
    chunk_bytes_odd = chunk_bytes ^ 16u;
    k_bytes = op.k_bytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = wave * 64 + j * 8 + r_in;
      voff[j] = r < rv ? (uint32_t)r * op.ld_bytes + ((j & 1) ? chunk_bytes_odd : chunk_bytes)
                       : kOOB;
    }
  }

  // Copy instruction j (rows 8 j .. 8 j + 7 of this wave's 64) of slice `kt`.
  // A slice past the end reads as zeros.
  __device__ __forceinline__ void issue1(int kt, int j, char GRPO_LDS* tile, int wave) const {
    const uint32_t kb = (uint32_t)kt * kBKB + ((j & 1) ? chunk_bytes_odd : chunk_bytes);
    const uint32_t off = kb < k_bytes ? voff[j] + slice_off(kt) : kOOB;
    char GRPO_LDS* dst = tile + (wave * 64 + j * 8) * kBKB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (GRPO_LDS void*)dst, 16, off, 0, 0, kCopyPolicy);
  }
  // The same copy for a slice with kt * 128 + 128 <= k_bytes: the slice offset
  // travels in the scalar offset.  A present row stays inside its own bytes and
  // an absent one (voff = kOOB) stays past the range, whether or not the range
  // check counts the scalar offset.
  __device__ __forceinline__ void issue1_full(int kt, int j, char GRPO_LDS* tile, int wave) const {
    char GRPO_LDS* dst = tile + (wave * 64 + j * 8) * kBKB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (GRPO_LDS void*)dst, 16, voff[j],
                                             (int)slice_off(kt), 0, kCopyPolicy);
  }
  __device__ __forceinline__ void issue(int kt, char GRPO_LDS* tile, int wave) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) issue1(kt, j, tile, wave);
  }
};

// Swizzle of a K-major slice: 32-byte block b of k-row r sits at block b ^ ksw(r).
// A half-wave's transposing read touches k-rows {0..3} and {8..11} (+4, +32
// multiples): ksw gives them the eight distinct values 0..7.
__device__ __forceinline__ uint32_t ksw(uint32_t r) { return (r & 3u) | (((r >> 3) & 1u) << 2); }

// Loader of a K-major operand slice (kBKB / sizeof(T) k-rows of 256 elements):
// 8 DMA instructions per wave, each moving 1 KB into LDS at (8 wave + j) KB.
// Lane i's 16 bytes land at physical chunk i of that KB; it loads the logical
// chunk the swizzle puts there.  k-rows at or past k_rows read as zero (their
// offset is at least the range).  Tile rows at or past rows_valid are not
// masked: they read whatever lies there within the range, and feed only
// output rows or columns the caller never stores.  (A masked offset of kOOB
// would not do here: with a slice offset of up to ~2^31 added it could wrap
// past 2^32 back into the range.)  Generic form (f32: one k-row per instruction).
template <typename T>
struct LoaderK {
  static constexpr int kES = (int)sizeof(T);
  static constexpr int kKS = kBKB / kES;        // k-rows per slice
  static constexpr int kRB = kBM * kES;         // LDS bytes per k-row
  static constexpr int kLPR = kRB / 16;         // lanes per k-row in one instruction
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t slice_bytes;     // global bytes between consecutive slices
  uint32_t voff[8];         // byte offset of this lane's chunk in slice 0

  __device__ __forceinline__ void init(const Operand& op, int wave, int lane, int) {
    rsrc = make_rsrc(op.base, op.range);
    slice_bytes = (uint32_t)__builtin_amdgcn_readfirstlane(kKS * op.ld_bytes);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t r = (uint32_t)((1024 / kRB) * (8 * wave + j) + lane / kLPR);
      const uint32_t c = (uint32_t)(lane % kLPR);
      const uint32_t mb = (((c >> 1) ^ ksw(r)) << 5) | ((c & 1u) << 4);
      voff[j] = r * op.ld_bytes + mb;
    }
  }
  // Copy instruction j of slice kt; k-rows past k_rows fall outside the range.
  __device__ __forceinline__ void issue1(int kt, int j, char GRPO_LDS* tile, int wave) const {
    char GRPO_LDS* dst = tile + (8 * wave + j) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (GRPO_LDS void*)dst, 16,
                                             voff[j] + (uint32_t)kt * slice_bytes, 0, 0,
                                             kCopyPolicy);
  }
  // A slice wholly inside k: the slice offset rides in the scalar offset.
  __device__ __forceinline__ void issue1_full(int kt, int j, char GRPO_LDS* tile, int wave) const {
    char GRPO_LDS* dst = tile + (8 * wave + j) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (GRPO_LDS void*)dst, 16, voff[j],
                                             (int)((uint32_t)kt * slice_bytes), 0, kCopyPolicy);
  }
  __device__ __forceinline__ void issue(int kt, char GRPO_LDS* tile, int wave) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) issue1(kt, j, tile, wave);
  }
  __device__ __forceinline__ static int full_slices(const Operand& op) {
    return (int)(op.k_rows / (uint32_t)kKS);
  }
  // LDS byte offset of k-row r of a slice
  __device__ __forceinline__ static uint32_t row_slot(uint32_t r) { return r * kRB; }
};

// bf16: a slice is 64 k-rows of 512 B, two per copy instruction.  The k-rows
// sit in LDS in a permuted order so that the eight copies of one lane share a
// swizzle and differ only by whole k-rows: k-row r lives in 512-byte slot
//   slot(r) = r0 | r2 << 1 | r4 << 2 | r5 << 3 | r1 << 4 | r3 << 5   (r_i bit i of r)
// so copy j of wave w, lane half h (lanes 32 h .. 32 h + 31) moves k-row
//   h | w0 << 1 | w1 << 3 | j0 << 2 | j1 << 4 | j2 << 5,
// whose swizzle bits (k-row bits 0, 1, 3) are the lane's own.  One offset
// register per lane; the k-row and slice offsets travel in the scalar offset.
template <>
struct LoaderK<__bf16> {
  static constexpr int kKS = 64;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t ld;              // global bytes between consecutive k-rows
  uint32_t voff;            // this lane's chunk in its first k-row

  __device__ __forceinline__ static uint32_t row_of(int j) {   // k-row offset of copy j
    return (uint32_t)(4 * (j & 1) + 16 * ((j >> 1) & 1) + 32 * (j >> 2));
  }
  __device__ __forceinline__ void init(const Operand& op, int wave, int lane, int) {
    rsrc = make_rsrc(op.base, op.range);
    ld = (uint32_t)__builtin_amdgcn_readfirstlane(op.ld_bytes);
    const uint32_t h = (uint32_t)(lane >> 5), c = (uint32_t)(lane & 31);
    const uint32_t r0 = h | (((uint32_t)wave & 1u) << 1) | (((uint32_t)wave >> 1) << 3);
    const uint32_t mb = (((c >> 1) ^ ksw(r0)) << 5) | ((c & 1u) << 4);
    voff = r0 * op.ld_bytes + mb;
  }
  __device__ __forceinline__ void issue1(int kt, int j, char GRPO_LDS* tile, int wave) const {
    char GRPO_LDS* dst = tile + (8 * wave + j) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (GRPO_LDS void*)dst, 16,
                                             voff + ((uint32_t)kt * 64u + row_of(j)) * ld, 0, 0,
                                             kCopyPolicy);
  }
  __device__ __forceinline__ void issue1_full(int kt, int j, char GRPO_LDS* tile, int wave) const {
    char GRPO_LDS* dst = tile + (8 * wave + j) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (GRPO_LDS void*)dst, 16, voff,
                                             (int)(((uint32_t)kt * 64u + row_of(j)) * ld), 0,
                                             kCopyPolicy);
  }
  __device__ __forceinline__ void issue(int kt, char GRPO_LDS* tile, int wave) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) issue1(kt, j, tile, wave);
  }
  __device__ __forceinline__ static int full_slices(const Operand& op) {
    return (int)(op.k_rows / 64u);
  }
  __device__ __forceinline__ static uint32_t row_slot(uint32_t r) {
    return ((r & 1u) | ((r >> 2) & 1u) << 1 | ((r >> 4) & 1u) << 2 | ((r >> 5) & 1u) << 3 |
            ((r >> 1) & 1u) << 4 | ((r >> 3) & 1u) << 5) * 512u;
  }
};

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]); the counters not named are left unconstrained.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// vmcnt(16): all but the 16 copies (one slice of A and B) issued last have landed
__device__ __forceinline__ void wait_vmem_but_one_slice() { __builtin_amdgcn_s_waitcnt(0x0F70 | 0x4000); }
__device__ __forceinline__ void wait_lds_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

#define GRPO_FENCE() __builtin_amdgcn_sched_barrier(0)

// 32 wait states: more than any MFMA needs before a VALU or memory
// instruction may read its result registers.  Then every accumulator passes
// through an empty statement that takes it in place in its AGPRs: whatever
// reads the accumulators afterwards reads values defined after the wait
// states, so the compiler cannot place a copy of one (to VGPRs, or to
// scratch) right behind the MFMA that writes it.
__device__ __forceinline__ void mfma_drain(Acc& acc) {
  GRPO_FENCE();
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
  for (int i = 0; i < kWM; ++i)
    asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]),
                      "+a"(acc[i][4]), "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
  GRPO_FENCE();
}

template <typename T> struct Frag;
template <> struct Frag<__bf16> { typedef bf16x8_t type; };
template <> struct Frag<float> { typedef f32x4_t type; };

// The bf16 MFMA accumulates in place: its result takes the accumulator's own
// registers.  (With all 256 AGPRs holding accumulators, the compiler's free
// choice of a result register other than the accumulator's leaves it
// permuting accumulators through VGPRs inside the loop.)  The compiler does
// not see this instruction as an MFMA, so it inserts no wait states for
// reads of its result: the main loop ends with them (mfma_drain).
__device__ __forceinline__ f32x4_t mfma_block(f32x4_t c, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  return c;
}
__device__ __forceinline__ f32x4_t mfma_block(f32x4_t c, const f32x4_t& a, const f32x4_t& b) {
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

// Fragment readers.  A wave's operand rows are row0 .. row0 + 127 of the tile
// (row0 = 128 (wave / 2) for A, 128 (wave % 2) for B); fragment f covers rows
// row0 + 16 f .. + 15; k-step s (0 or 1) is k-bytes 64 s .. 64 s + 63 of a slice.
// Lane l gets row l % 16 of the fragment and k-chunk l / 16 of the k-step
// (bf16: 8 consecutive k; f32: 4 consecutive k, element e feeding MFMA e).
template <typename T, bool KMAJOR> struct Reader;

// K-contiguous operand: one 16-byte read from the row-swizzled slice.
template <typename T> struct Reader<T, false> {
  typedef typename Frag<T>::type F;
  uint32_t base, sw0, sw1;
  __device__ __forceinline__ void init(int lane, int row0) {
    base = (uint32_t)(row0 + (lane & 15)) * kBKB;
    // fragment rows are 16-aligned blocks + lane % 16, so f(row) depends on the lane only
    const uint32_t fr = (uint32_t)((lane & 7) ^ ((lane >> 3) & 1));
    sw0 = ((0u + (uint32_t)(lane >> 4)) ^ fr) << 4;
    sw1 = ((4u + (uint32_t)(lane >> 4)) ^ fr) << 4;
  }
  __device__ __forceinline__ void read(F& out, int f, const char GRPO_LDS* region, int s) const {
    out = *(const F GRPO_LDS*)(region + base + f * 16 * kBKB + (s ? sw1 : sw0));
  }
};

// K-major bf16 operand: two transposing 8-byte reads per fragment.  Lane s of a
// 16-lane group g addresses rows 4 (s % 4) .. + 3 of k-row 8 g + s / 4 (and of
// the k-row four further), and receives k 8 g .. 8 g + 7 of its own row.
template <> struct Reader<__bf16, true> {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
  uint32_t kb0;       // this lane's address of fragment 0, k-step 0, k-rows + 0..3
  __device__ __forceinline__ void init(int lane, int row0) {
    const uint32_t g = (uint32_t)(lane >> 4), sl = (uint32_t)(lane & 15);
    // k-row 8 g + sl / 4 (+ 4 for the second read, + 32 in k-step 1): its swizzle
    // (ksw) depends on the lane only, and the + 4 and + 32 move it by whole slots
    const uint32_t r = 8u * g + (sl >> 2);
    const uint32_t sw = ksw(r);
    // bits 5..7 of the address are the swizzled block: fragment f is one XOR away
    kb0 = LoaderK<__bf16>::row_slot(r) + (uint32_t)row0 * 2u + 8u * (sl & 3u) + (sw << 5);
  }
  // The two transposing reads of one fragment.  The builtin carries no alias
  // information of its own, and an LDS read without any is taken to alias
  // every buffer-to-LDS copy still in flight, so the compiler would wait for
  // all of them (vmcnt(0)) before each read, exposing the copies' latency and
  // more than doubling the loop time.  The restrict parameter gives both reads
  // an alias scope once inlined, as the type-based metadata of the plain
  // 16-byte reads does for them.  The loop's own waits and barriers order
  // every read after the copies of the slice it reads.
  __device__ __forceinline__ static bf16x8_t tr_pair(const char GRPO_LDS* __restrict__ p) {
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GRPO_LDS bf16x4_t*)p);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GRPO_LDS bf16x4_t*)(p + 1024));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  __device__ __forceinline__ void read(bf16x8_t& out, int f, const char GRPO_LDS* region,
                                       int s) const {
    // k-row + 32 s is slot bit 3 (4 KB), k-row + 4 slot bit 1 (1 KB)
    out = tr_pair(region + (kb0 ^ ((uint32_t)f << 5)) + s * 4096);
  }
};

// K-major f32 operand (small shapes only): four 4-byte reads, k-rows
// 16 s + 4 g + e of the lane's row.
template <> struct Reader<float, true> {
  uint32_t g, col;
  __device__ __forceinline__ void init(int lane, int row0) {
    g = (uint32_t)(lane >> 4);
    col = (uint32_t)(row0 + (lane & 15));
  }
  __device__ __forceinline__ void read(f32x4_t& out, int f, const char GRPO_LDS* region,
                                       int s) const {
    const uint32_t m = col + 16u * (uint32_t)f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t r = 16u * (uint32_t)s + 4u * g + (uint32_t)e;
      out[e] = *(const float GRPO_LDS*)(region + r * (kBM * 4) + (((m >> 3) ^ ksw(r)) << 5) +
                                        (m & 7u) * 4u);
    }
  }
};

template <typename T, bool KM, bool BLK = false> struct LoaderOf { typedef Loader<BLK> type; };
template <typename T, bool BLK> struct LoaderOf<T, true, BLK> { typedef LoaderK<T> type; };

template <typename T, bool KM>
__device__ __forceinline__ int full_slices(const Operand& op) {
  if constexpr (KM) return LoaderK<T>::full_slices(op);
  else return (int)(op.k_bytes / kBKB);
}

// Position of the copies within a k-step: after MFMA q with q % 8 == kCopyAt.
constexpr int kCopyAt = 5;

// One 64-byte k-step of the wave's 8 x 8 blocks, in a fixed order.  After
// block q: for READ and even q < 32, fragment q / 2 of k-step `rs` (a0..a7,
// then b0..b7) from A's slot `ra_at` and B's slot `rb_at`; for q % 8 ==
// kCopyAt, copy instruction q / 8 of slice `ckt` of A (COPY = 1) or of B
// (COPY = 2) into slot `cst`, unchecked when FULL.  SWAP: each block is the
// MFMA of (b[j], a[i]) instead of (a[i], b[j]), i.e. the block's transpose.
template <typename T, bool READ, int COPY, bool FULL, bool SWAP, typename LA, typename LB,
          typename RA, typename RB>
__device__ __forceinline__ void kstep(Acc& acc, const typename Frag<T>::type (&a)[kWM],
                                      const typename Frag<T>::type (&b)[kWN],
                                      typename Frag<T>::type (&na)[kWM], typename Frag<T>::type (&nb)[kWN],
                                      const char GRPO_LDS* ra_at, const char GRPO_LDS* rb_at, int rs,
                                      const RA& ra, const RB& rb, const LA& la, const LB& lb, int ckt,
                                      char GRPO_LDS* cst, int wave) {
#pragma unroll
  for (int q = 0; q < kWM * kWN; ++q) {
    const int i = q / kWN, j = q % kWN;
    acc[i][j] = SWAP ? mfma_block(acc[i][j], b[j], a[i]) : mfma_block(acc[i][j], a[i], b[j]);
    GRPO_FENCE();
    if (READ && (q & 1) == 0 && q < 32) {
      const int f = q >> 1;
      if (f < kWM) ra.read(na[f], f, ra_at, rs);
      else rb.read(nb[f - kWM], f - kWM, rb_at, rs);
      GRPO_FENCE();
    }
    if (COPY && (q & 7) == kCopyAt) {
      const int c = q >> 3;
      if (COPY == 1) {
        if (FULL) la.issue1_full(ckt, c, cst, wave);
        else la.issue1(ckt, c, cst, wave);
      } else {
        if (FULL) lb.issue1_full(ckt, c, cst, wave);
        else lb.issue1(ckt, c, cst, wave);
      }
      GRPO_FENCE();
    }
  }
}

// The slice barrier: this wave's copies of slice kt + 1 have landed (the 8 of
// A's slice kt + 2 may still fly) and its fragment reads are done.
__device__ __forceinline__ void slice_sync() {
  __builtin_amdgcn_s_waitcnt(0x0F78);   // vmcnt(8)
  wait_lds_all();
  __builtin_amdgcn_s_barrier();
  GRPO_FENCE();
}

// One slice of the main loop (see the top of this file), copying slice `ck`
// (normally the slice after next).  as/bs: the slots of this slice (A and B),
// an/bn: of the next, af: A's free slot.
template <typename T, bool FULL, bool SWAP, typename LA, typename LB, typename RA, typename RB,
          typename F>
__device__ __forceinline__ void slice_step(Acc& acc, F (&fa0)[kWM], F (&fb0)[kWN], F (&fa1)[kWM],
                                           F (&fb1)[kWN], char GRPO_LDS* as, char GRPO_LDS* bs,
                                           char GRPO_LDS* an, char GRPO_LDS* bn,
                                           char GRPO_LDS* af, const RA& ra, const RB& rb,
                                           const LA& la, const LB& lb, int ck, int wave) {
  kstep<T, true, 1, FULL, SWAP>(acc, fa0, fb0, fa1, fb1, as, bs, 1, ra, rb, la, lb, ck, af, wave);
  slice_sync();
  kstep<T, true, 2, FULL, SWAP>(acc, fa1, fb1, fa0, fb0, an, bn, 0, ra, rb, la, lb, ck, bs, wave);
}

// The main loop.  `lds` must be kLdsBytes of workgroup memory.  AK / BK: the
// A / B operand is K-major (see Operand); BBLK: B is K-contiguous and blocked
// along k (Operand::blk_stride).  k_slices is the number of 128-byte
// K slices (both operands must agree).  SWAP: every 16 x 16 block is computed
// transposed, so lane l of wave w holds, in block (i, j), element e,
//   C[128 (w / 2) + 16 i + l % 16][128 (w % 2) + 16 j + 4 (l / 16) + e]
// (four consecutive B rows at one A row; the default layout is stated at the
// top of this file).  On return no copy is in flight and the accumulators may
// be read; the caller must barrier before reusing LDS.
template <typename T, bool AK = false, bool BK = false, bool SWAP = false, bool BBLK = false>
__device__ __forceinline__ void tile_mainloop(Acc& acc, const Operand& A, const Operand& B,
                                              int k_slices, char GRPO_LDS* lds) {
  typedef typename Frag<T>::type F;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
#pragma unroll
  for (int i = 0; i < kWM; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j)
#pragma unroll
      for (int e = 0; e < kAcc; ++e) acc[i][j][e] = 0.f;
  if (k_slices <= 0) return;
  typename LoaderOf<T, AK>::type la;
  typename LoaderOf<T, BK, BBLK>::type lb;
  la.init(A, wave, lane, (int)sizeof(T));
  lb.init(B, wave, lane, (int)sizeof(T));
  Reader<T, AK> ra;
  Reader<T, BK> rb;
  ra.init(lane, (wave >> 1) * 128);
  rb.init(lane, (wave & 1) * 128);
  char GRPO_LDS* const lb0 = lds + kBRegion;

  // slices 0 and 1 (slice 1 reads as zeros when there is none)
  la.issue(0, lds, wave);
  lb.issue(0, lb0, wave);
  la.issue(1, lds + kTileBytes, wave);
  lb.issue(1, lb0 + kTileBytes, wave);
  wait_vmem_but_one_slice();
  __builtin_amdgcn_s_barrier();
  F fa0[kWM], fb0[kWN], fa1[kWM], fb1[kWN];
#pragma unroll
  for (int f = 0; f < kWM; ++f) ra.read(fa0[f], f, lds, 0);
#pragma unroll
  for (int f = 0; f < kWN; ++f) rb.read(fb0[f], f, lb0, 0);

  // Slot offsets (workgroup-uniform), rotated per slice: A's slices kt,
  // kt + 1 and the free slot; B's slices kt and kt + 1.
  uint32_t ac = 0, an = kTileBytes, af = 2 * kTileBytes, bc = 0, bn = kTileBytes;
  int kt = 0;
  // Slices whose copies (slice kt + 2) lie wholly inside k in both operands
  // take unchecked copies; the k tail and the zero slices past it take the
  // checked ones.
  const int full_a = full_slices<T, AK>(A), full_b = full_slices<T, BK>(B);
  const int full = full_a < full_b ? full_a : full_b;
  for (; kt + 2 < full; ++kt) {
    slice_step<T, true, SWAP>(acc, fa0, fb0, fa1, fb1, lds + ac, lb0 + bc, lds + an, lb0 + bn,
                              lds + af, ra, rb, la, lb, kt + 2, wave);
    const uint32_t t = ac; ac = an; an = af; af = t;
    const uint32_t u = bc; bc = bn; bn = u;
  }
  for (; kt + 1 < k_slices; ++kt) {
    slice_step<T, false, SWAP>(acc, fa0, fb0, fa1, fb1, lds + ac, lb0 + bc, lds + an, lb0 + bn,
                               lds + af, ra, rb, la, lb, kt + 2, wave);
    const uint32_t t = ac; ac = an; an = af; af = t;
    const uint32_t u = bc; bc = bn; bn = u;
  }
  // the last slice: copies nothing, and its k-step 1 reads nothing
  kstep<T, true, 0, false, SWAP>(acc, fa0, fb0, fa1, fb1, lds + ac, lb0 + bc, 1, ra, rb, la, lb, 0,
                                 lds, wave);
  kstep<T, false, 0, false, SWAP>(acc, fa1, fb1, fa0, fb0, lds + ac, lb0 + bc, 0, ra, rb, la, lb, 0,
                                  lds, wave);
  mfma_drain(acc);
  wait_vmem_all();
}

// ---------------------------------------------------------------- fp8 main loop
// The same tile with float8 e4m3 operands (one byte per element):
// v_mfma_f32_16x16x128_f8f6f4 takes a whole 128-byte slice row per k-step, so
// a slice is one k-step of 64 MFMAs (32 cycles each, twice the bf16 rate).
// A lane's 32-byte fragment is the two 16-byte chunks that the bf16 loop reads
// for its two k-steps (chunks l/16 and 4 + l/16 of the row, same swizzle):
// the instruction sums over k, so any k order that A and B share is exact.
// Fragments are 8 VGPRs, so only B's are double buffered; A's rows 0..6 are
// reloaded in place once their 8 MFMAs have issued (row 6 nine MFMAs before
// the slice barrier), and row 7 has two buffers (fa[7] and fa[8]) that
// alternate between iterations, so no LDS read is left in flight at the
// barrier.  Its LDS layout is [A stage 0 | A stage 1 | B stage 0 | B stage 1]
// (32 KB each), so both stages of an operand sit within the 16-bit offset of
// one ds_read base: two base registers per operand instead of four.
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;

__device__ __forceinline__ f32x4_t mfma_fp8(f32x4_t c, const i32x8_t& a, const i32x8_t& b) {
  // zero scale operands: no block scaling
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ void read_frag_half(i32x8_t& f, int half, const char GRPO_LDS* p) {
  const i32x4_t v = *(const i32x4_t GRPO_LDS*)p;
  if (half == 0) f.lo = v;
  else f.hi = v;
}

// One slice (k-step) of 64 MFMAs.  PAR selects the buffer of A row 7 this
// iteration uses (fa[7] or fa[8]); the next slice's fragments are read from
// stage `rst`: fbn after even q < 32, A row 7 into the other buffer after
// q = 33 and 35, A row i < 7 after its last MFMA.  COPY: copy instruction c of
// slice `ckt` into stage `cst` after MFMA 2c + 1.
// Fragment reads address lds + (lane base) + (compile-time offset): the lane
// bases a0/a1 (A rows, chunks sw0/sw1) and b0/b1 (B rows) are loop invariant,
// and RS (the stage read) and CS (the stage refilled) are template constants.
template <bool PAR, bool READ, bool COPY, bool FULL, int RS, int CS>
__device__ __forceinline__ void kstep_fp8(Acc& acc, i32x8_t (&fa)[9], const i32x8_t (&fbc)[8],
                                          i32x8_t (&fbn)[8], const char GRPO_LDS* lds,
                                          uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                          const Loader<>& la, const Loader<>& lb, int ckt, int wave) {
  constexpr int kAoff = RS * kTileBytes, kBoff = (2 + RS) * kTileBytes;
  char GRPO_LDS* cstA = (char GRPO_LDS*)lds + CS * kTileBytes;
  char GRPO_LDS* cstB = (char GRPO_LDS*)lds + (2 + CS) * kTileBytes;
#pragma unroll
  for (int q = 0; q < 64; ++q) {
    const int i = q >> 3, j = q & 7;
    const int ai = (i == 7 && PAR) ? 8 : i;
    acc[i][j] = mfma_fp8(acc[i][j], fa[ai], fbc[j]);
    GRPO_FENCE();
    if (READ && (q & 1) == 0 && q < 32) {
      const int f = q >> 2, h = (q >> 1) & 1;
      read_frag_half(fbn[f], h, lds + (h ? b1 : b0) + (kBoff + f * 16 * kBKB));
      GRPO_FENCE();
    }
    if (READ && (q == 33 || q == 35)) {
      const int h = (q - 33) >> 1;
      read_frag_half(fa[PAR ? 7 : 8], h, lds + (h ? a1 : a0) + (kAoff + 7 * 16 * kBKB));
      GRPO_FENCE();
    }
    if (READ && j == 7 && i < 7) {
      read_frag_half(fa[i], 0, lds + a0 + (kAoff + i * 16 * kBKB));
      read_frag_half(fa[i], 1, lds + a1 + (kAoff + i * 16 * kBKB));
      GRPO_FENCE();
    }
    if (COPY && (q & 1) == 1 && q < 32) {
      const int c = q >> 1;
      if (FULL) {
        if (c < 8) la.issue1_full(ckt, c, cstA, wave);
        else lb.issue1_full(ckt, c - 8, cstB, wave);
      } else {
        if (c < 8) la.issue1(ckt, c, cstA, wave);
        else lb.issue1(ckt, c - 8, cstB, wave);
      }
      GRPO_FENCE();
    }
  }
}

// Slice barrier: this wave's copies of the next slice have landed and its reads
// of the current stage are done; after it every wave may read the next slice
// and overwrite the current one.
__device__ __forceinline__ void slice_barrier() {
  wait_vmem_all();
  wait_lds_all();
  __builtin_amdgcn_s_barrier();
  GRPO_FENCE();
}

template <bool PAR, bool FULL>
__device__ __forceinline__ void fp8_iter(Acc& acc, i32x8_t (&fa)[9], i32x8_t (&fbA)[8],
                                         i32x8_t (&fbB)[8], char GRPO_LDS* lds, int kt,
                                         uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                         const Loader<>& la, const Loader<>& lb, int wave) {
  // this iteration's stage is PAR (= kt & 1): it reads the other and refills its own
  slice_barrier();
  if (PAR)
    kstep_fp8<true, true, true, FULL, 0, 1>(acc, fa, fbB, fbA, lds, a0, a1, b0, b1, la, lb,
                                            kt + 2, wave);
  else
    kstep_fp8<false, true, true, FULL, 1, 0>(acc, fa, fbA, fbB, lds, a0, a1, b0, b1, la, lb,
                                             kt + 2, wave);
}

// fp8 main loop: A and B rows of k_bytes e4m3 codes.  Same contract as
// tile_mainloop.
__device__ __forceinline__ void tile_mainloop_fp8(Acc& acc, const Operand& A, const Operand& B,
                                                  int k_slices, char GRPO_LDS* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
#pragma unroll
  for (int i = 0; i < kWM; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j)
#pragma unroll
      for (int e = 0; e < kAcc; ++e) acc[i][j][e] = 0.f;
  if (k_slices <= 0) return;
  Loader<> la, lb;
  la.init(A, wave, lane, 1);
  lb.init(B, wave, lane, 1);
  const uint32_t abase = (uint32_t)((wave >> 1) * 128 + (lane & 15)) * kBKB;
  const uint32_t bbase = (uint32_t)((wave & 1) * 128 + (lane & 15)) * kBKB;
  const uint32_t fr = (uint32_t)((lane & 7) ^ ((lane >> 3) & 1));
  const uint32_t sw0 = ((0u + (uint32_t)(lane >> 4)) ^ fr) << 4;
  const uint32_t sw1 = ((4u + (uint32_t)(lane >> 4)) ^ fr) << 4;
  const uint32_t a0 = abase + sw0, a1 = abase + sw1, b0 = bbase + sw0, b1 = bbase + sw1;

  la.issue(0, lds, wave);
  lb.issue(0, lds + 2 * kTileBytes, wave);
  la.issue(1, lds + kTileBytes, wave);
  lb.issue(1, lds + 3 * kTileBytes, wave);
  wait_vmem_but_one_slice();
  __builtin_amdgcn_s_barrier();
  i32x8_t fa[9], fbA[8], fbB[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    read_frag_half(fa[f], 0, lds + abase + f * 16 * kBKB + sw0);
    read_frag_half(fa[f], 1, lds + abase + f * 16 * kBKB + sw1);
    read_frag_half(fbA[f], 0, lds + 2 * kTileBytes + bbase + f * 16 * kBKB + sw0);
    read_frag_half(fbA[f], 1, lds + 2 * kTileBytes + bbase + f * 16 * kBKB + sw1);
  }
  // Copies take the checked form throughout: with 32-cycle MFMAs the three
  // VALU operations per copy fit in the issue shadow.  The slice count is
  // rounded up to even (a zero slice past the end adds nothing), so every
  // iteration's buffer parity is known at compile time.
  const int k_even = (k_slices + 1) & ~1;
  int kt = 0;
  for (; kt + 2 < k_even; kt += 2) {
    fp8_iter<false, false>(acc, fa, fbA, fbB, lds, kt, a0, a1, b0, b1, la, lb, wave);
    fp8_iter<true, false>(acc, fa, fbA, fbB, lds, kt + 1, a0, a1, b0, b1, la, lb, wave);
  }
  // the last two slices: read the last one's fragments, copy nothing
  slice_barrier();
  kstep_fp8<false, true, false, false, 1, 0>(acc, fa, fbA, fbB, lds, a0, a1, b0, b1, la, lb, 0,
                                             wave);
  kstep_fp8<true, false, false, false, 0, 0>(acc, fa, fbB, fbA, lds, a0, a1, b0, b1, la, lb, 0,
                                             wave);
  wait_vmem_all();
}

// Coordinates of accumulator element (i, j, e) of this lane, tile-relative.
__device__ __forceinline__ int acc_row(int wave, int lane, int i, int e) {
  return (wave >> 1) * 128 + 16 * i + 4 * (lane >> 4) + e;
}
__device__ __forceinline__ int acc_col(int wave, int lane, int j) {
  return (wave & 1) * 128 + 16 * j + (lane & 15);
}

}  // namespace grpo
