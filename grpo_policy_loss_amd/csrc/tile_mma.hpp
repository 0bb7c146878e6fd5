// tile_mma.hpp -- the MFMA tile main loop shared by every GEMM-shaped kernel.
//
// Computes one 256 x 256 float32 tile of C[m][n] = sum_k A[m][k] * B[n][k]
// (both operands "K-contiguous": row m of A and row n of B are contiguous
// along k), on gfx950 (CDNA4) matrix cores.
//
// Layout and schedule:
//  * 512 threads = 8 wave64s, two per SIMD (waves w and w + 4 share a SIMD),
//    in a 2 (M) x 4 (N) grid; each wave owns 128 x 64 of the tile as 4 x 2
//    blocks of the 32 x 32 MFMA output (128 accumulator registers per lane).
//    Two waves per SIMD let one wave's LDS or barrier stalls be covered by
//    the other's MFMAs, while all eight share one 256 x 256 tile (the tile
//    size sets the L2 -> LDS traffic per flop).
//  * K advances in 128-byte slices (64 bf16 or 32 f32).  Each slice of A and
//    B (256 rows x 128 B = 32 KB each) is copied global -> LDS by the buffer
//    unit directly (buffer_load_dwordx4 ... lds): no VGPR staging.  LDS is
//    double buffered (2 x 64 KB), so the copy of slice k+1 runs while the
//    matrix cores consume slice k.
//  * Only waves 0..3 (one per SIMD) issue those copies.  Issuing a copy can
//    hold a wave for many cycles while the address unit drains; when both
//    waves of a SIMD did it at once (right after the slice barrier) the
//    matrix core sat idle.  With one copying wave per SIMD, its partner's
//    MFMAs keep the matrix core busy meanwhile (measured: +2.5 to +5 points
//    of bf16 peak on 8k-16k GEMMs).
//  * MFMA operand fragments are double buffered in registers: the LDS reads
//    of k-step s+1 are issued between the MFMAs of k-step s.
//  * Out-of-range rows and k-columns read as zero: each operand is addressed
//    through a buffer resource whose range ends at its last valid row, and an
//    invalid row or column gets an offset past that range.  Tails in M, N
//    and K therefore need no separate code path.
//  * gfx950's LDS serves 256 bytes per clock, i.e. one ds_read_b128 cycle
//    covers 16 lanes = 16 rows of a fragment.  The eight 16-byte chunks of a
//    128-byte LDS row are XOR-swizzled by f(r) = (r & 7) ^ ((r >> 3) & 1), so
//    any 16 consecutive rows at one logical chunk hit 16 distinct bank groups.
//  * bf16: v_mfma_f32_32x32x16_bf16, one per 16-byte chunk pair.
//    f32:  v_mfma_f32_32x32x2_f32, four per chunk pair; lane l supplies
//          element e of its 4-float chunk as its k = l/32 operand, so the
//          four MFMAs together cover the 8 k of the pair.
//
// Output register layout (for both MFMAs): lane l of wave w, block (i, j),
// element e holds C[128 (w / 4) + 32 i + 8 (e / 4) + 4 (l / 32) + e % 4]
//                  [64 (w % 4) + 32 j + l % 32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grpo {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

#define GRPO_LDS __attribute__((address_space(3)))

constexpr int kBM = 256;          // tile rows (A rows)
constexpr int kBN = 256;          // tile cols (B rows)
constexpr int kBKB = 128;         // K slice in bytes
constexpr int kThreads = 512;
constexpr int kWM = 4;           // 32-row MFMA blocks per wave
constexpr int kWN = 2;           // 32-col MFMA blocks per wave
constexpr int kTileBytes = kBM * kBKB;   // one operand slice in LDS: 32 KB
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kLdsBytes = 2 * kStageBytes;  // double buffered A + B: 128 KB
constexpr uint32_t kOOB = 0x80000000u;   // an offset past every resource range
// Cache policy of the slice copies: sc1 (device scope) takes them past the per-CU L1.
// Each workgroup streams its panels once per slice, so L1 allocation buys nothing;
// measured +1 to +3 points of bf16 peak on the tile GEMM.  (nt, the streaming hint,
// costs 6 points: the L2 then stops keeping panels that neighbouring CUs reuse.)
constexpr int kCopyPolicy = 16;

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

// One operand's view for the loader: rows [row0, row0 + rows_valid) of a
// row-major matrix with row pitch `ld_bytes`, k-bytes [0, k_bytes) valid.
struct Operand {
  const char* base;      // address of row row0, column 0
  uint32_t ld_bytes;     // row pitch in bytes
  int rows_valid;        // rows of this tile that exist (may be <= 0)
  uint32_t k_bytes;      // valid k extent in bytes (multiple of 16)
};

// Waves 0..3 each copy 64 rows of an operand slice: 8 DMA instructions, each
// moving 8 rows x 128 B (lane i fills slot i & 7 of row i >> 3).  Waves 4..7
// copy nothing (their issue() is empty).
struct Loader {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t rowoff[8];       // byte offset of each of this lane's 8 rows (kOOB if absent)
  uint32_t chunk_bytes;     // logical 16-byte chunk this lane copies, even 8-row groups
  uint32_t chunk_bytes_odd; // the same for odd 8-row groups (f(r) flips bit 0)
  uint32_t k_bytes;

  __device__ __forceinline__ void init(const Operand& op, int wave, int lane) {
    int rv = op.rows_valid < 0 ? 0 : (op.rows_valid > kBM ? kBM : op.rows_valid);
    rsrc = make_rsrc(op.base, (uint32_t)rv * op.ld_bytes);
    const int r_in = lane >> 3;                          // row within an 8-row group
    chunk_bytes = (uint32_t)(((lane & 7) ^ r_in) << 4);  // slot lane & 7 holds chunk slot ^ f(r)
    chunk_bytes_odd = chunk_bytes ^ 16u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int r = (wave & 3) * 64 + j * 8 + r_in;
      rowoff[j] = r < rv ? (uint32_t)r * op.ld_bytes : kOOB;
    }
    k_bytes = op.k_bytes;
  }

  // Issue the 8 direct-to-LDS copies of this wave's 64 rows of slice `kt`
  // (waves 0..3 only).
  __device__ __forceinline__ void issue(int kt, char GRPO_LDS* tile, int wave) const {
    if (wave >= 4) return;
    const uint32_t kb0 = (uint32_t)kt * kBKB + chunk_bytes;
    const uint32_t kb1 = (uint32_t)kt * kBKB + chunk_bytes_odd;
    const bool kok0 = kb0 < k_bytes, kok1 = kb1 < k_bytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t kb = (j & 1) ? kb1 : kb0;
      const bool kok = (j & 1) ? kok1 : kok0;
      uint32_t off = kok ? rowoff[j] + kb : kOOB;
      char GRPO_LDS* dst = tile + (wave * 64 + j * 8) * kBKB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (GRPO_LDS void*)dst, 16, off, 0, 0, kCopyPolicy);
    }
  }
};

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]); the counters not named are left unconstrained.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// vmcnt(16): all but the 16 copies (one slice of A and B) issued last have landed
__device__ __forceinline__ void wait_vmem_but_one_slice() { __builtin_amdgcn_s_waitcnt(0x0F70 | 0x4000); }
__device__ __forceinline__ void wait_lds_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <typename T> struct Frag;
template <> struct Frag<__bf16> { typedef bf16x8_t type; };
template <> struct Frag<float> { typedef f32x4_t type; };

template <typename T>
__device__ __forceinline__ void load_frags(typename Frag<T>::type (&a)[4], typename Frag<T>::type (&b)[kWN],
                                           const char GRPO_LDS* buf, const uint32_t (&aoff)[4],
                                           const uint32_t (&boff)[kWN], uint32_t swz) {
  typedef typename Frag<T>::type F;
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = *(const F GRPO_LDS*)(buf + aoff[i] + swz);
#pragma unroll
  for (int j = 0; j < kWN; ++j) b[j] = *(const F GRPO_LDS*)(buf + kTileBytes + boff[j] + swz);
}

__device__ __forceinline__ void mfma_all(f32x16_t (&acc)[4][kWN], const bf16x8_t (&a)[4], const bf16x8_t (&b)[kWN]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}
__device__ __forceinline__ void mfma_all(f32x16_t (&acc)[4][kWN], const f32x4_t (&a)[4], const f32x4_t (&b)[kWN]) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kWN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
}

// Scheduling hint: alternate one MFMA and one LDS read, n times.
#define GRPO_SCHED_MFMA_DS(n)                                  \
  _Pragma("unroll") for (int q_ = 0; q_ < (n); ++q_) {          \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          \
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);          \
  }

// The main loop.  `lds` must be kLdsBytes of workgroup memory.  On return
// the caller must barrier before reusing LDS.
template <typename T>
__device__ __forceinline__ void tile_mainloop(f32x16_t (&acc)[4][kWN], const Operand& A,
                                              const Operand& B, int k_slices,
                                              char GRPO_LDS* lds) {
  typedef typename Frag<T>::type F;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm0 = (wave >> 2) * 128;
  const int wn0 = (wave & 3) * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  Loader la, lb;
  la.init(A, wave, lane);
  lb.init(B, wave, lane);
  uint32_t aoff[4], boff[kWN];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = (uint32_t)(wm0 + 32 * i + (lane & 31)) * kBKB;
#pragma unroll
  for (int j = 0; j < kWN; ++j) boff[j] = (uint32_t)(wn0 + 32 * j + (lane & 31)) * kBKB;
  const uint32_t half = (uint32_t)(lane >> 5);
  const uint32_t r7 = (uint32_t)((lane & 7) ^ ((lane >> 3) & 1));
  uint32_t swz[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) swz[s] = (((2u * s + half) ^ r7) << 4);
  if (k_slices <= 0) return;

  la.issue(0, lds, wave);
  lb.issue(0, lds + kTileBytes, wave);
  if (k_slices > 1) {
    la.issue(1, lds + kStageBytes, wave);
    lb.issue(1, lds + kStageBytes + kTileBytes, wave);
    wait_vmem_but_one_slice();
  } else {
    wait_vmem_all();
  }
  __builtin_amdgcn_s_barrier();
  F fa[2][4], fb[2][kWN];
  load_frags<T>(fa[0], fb[0], lds, aoff, boff, swz[0]);

  // Steady state: every slice but the last.  The slice barrier sits after the
  // third k-step, once every wave holds the slice's last fragments in
  // registers: the stage is then free for the copy of slice kt + 2, and after
  // the copying waves' vmcnt wait slice kt + 1 is visible, so its first
  // fragments load under the fourth k-step's MFMAs instead of after the barrier.
  for (int kt = 0; kt + 1 < k_slices; ++kt) {
    char GRPO_LDS* cur = lds + (kt & 1) * kStageBytes;
    char GRPO_LDS* nxt = lds + ((kt + 1) & 1) * kStageBytes;
    load_frags<T>(fa[1], fb[1], cur, aoff, boff, swz[1]);
    mfma_all(acc, fa[0], fb[0]);
    GRPO_SCHED_MFMA_DS(6);
    load_frags<T>(fa[0], fb[0], cur, aoff, boff, swz[2]);
    mfma_all(acc, fa[1], fb[1]);
    GRPO_SCHED_MFMA_DS(6);
    load_frags<T>(fa[1], fb[1], cur, aoff, boff, swz[3]);
    mfma_all(acc, fa[0], fb[0]);
    GRPO_SCHED_MFMA_DS(6);
    wait_vmem_all();
    wait_lds_all();
    __builtin_amdgcn_s_barrier();
    if (kt + 2 < k_slices) {
      la.issue(kt + 2, cur, wave);
      lb.issue(kt + 2, cur + kTileBytes, wave);
    }
    load_frags<T>(fa[0], fb[0], nxt, aoff, boff, swz[0]);
    mfma_all(acc, fa[1], fb[1]);
    GRPO_SCHED_MFMA_DS(6);
  }
  // last slice: no copy left to wait for
  {
    char GRPO_LDS* cur = lds + ((k_slices - 1) & 1) * kStageBytes;
    load_frags<T>(fa[1], fb[1], cur, aoff, boff, swz[1]);
    mfma_all(acc, fa[0], fb[0]);
    GRPO_SCHED_MFMA_DS(6);
    load_frags<T>(fa[0], fb[0], cur, aoff, boff, swz[2]);
    mfma_all(acc, fa[1], fb[1]);
    GRPO_SCHED_MFMA_DS(6);
    load_frags<T>(fa[1], fb[1], cur, aoff, boff, swz[3]);
    mfma_all(acc, fa[0], fb[0]);
    GRPO_SCHED_MFMA_DS(6);
    mfma_all(acc, fa[1], fb[1]);
  }
}

// Coordinates of accumulator element (i, j, e) of this lane, tile-relative.
__device__ __forceinline__ int acc_row(int wave, int lane, int i, int e) {
  return (wave >> 2) * 128 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
__device__ __forceinline__ int acc_col(int wave, int lane, int j) {
  return (wave & 3) * 64 + 32 * j + (lane & 31);
}

}  // namespace grpo
