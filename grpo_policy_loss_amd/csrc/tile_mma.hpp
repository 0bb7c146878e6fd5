// tile_mma.hpp -- the MFMA tile main loop shared by every GEMM-shaped kernel.
//
// Computes one 256 x 256 float32 tile of C[m][n] = sum_k A[m][k] * B[n][k]
// (both operands "K-contiguous": row m of A and row n of B are contiguous
// along k), on gfx950 (CDNA4) matrix cores.
//
// Layout and schedule:
//  * 256 threads = 4 wave64s in a 2 x 2 grid; each wave owns 128 x 128 of the
//    tile as 4 x 4 blocks of the 32 x 32 MFMA output (256 accumulator
//    registers per lane).
//  * K advances in 128-byte slices (64 bf16 or 32 f32).  Each slice of A and
//    B (256 rows x 128 B = 32 KB each) is copied global -> LDS by the buffer
//    unit directly (buffer_load_dwordx4 ... lds): no VGPR staging.  LDS is
//    double buffered (2 x 64 KB), so the copy of slice k+1 runs while the
//    matrix cores consume slice k.
//  * Out-of-range rows and k-columns read as zero: each operand is addressed
//    through a buffer resource whose range ends at its last valid row, and an
//    invalid row or column gets an offset past that range.  Tails in M, N
//    and K therefore need no separate code path.
//  * Within a 128-byte LDS row the eight 16-byte chunks are XOR-swizzled by
//    (row & 7), so the ds_read_b128 of 8 consecutive rows at the same logical
//    chunk hits 8 distinct bank groups.
//  * bf16: v_mfma_f32_32x32x16_bf16, one per 16-byte chunk pair.
//    f32:  v_mfma_f32_32x32x2_f32, four per chunk pair; lane l supplies
//          element e of its 4-float chunk as its k = l/32 operand, so the
//          four MFMAs together cover the 8 k of the pair.
//
// Output register layout (for both MFMAs): lane l, block (i, j), element e
// holds C[wm0 + 32 i + 8 (e / 4) + 4 (l / 32) + e % 4][wn0 + 32 j + l % 32].
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
constexpr int kThreads = 256;
constexpr int kTileBytes = kBM * kBKB;   // one operand slice in LDS: 32 KB
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kLdsBytes = 2 * kStageBytes;  // double buffered A + B: 128 KB
constexpr uint32_t kOOB = 0x80000000u;   // an offset past every resource range

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

// Element-type policy.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kSize = 4;
};
template <> struct Elem<__bf16> {
  static constexpr int kSize = 2;
};

// One operand's view for the loader: rows [row0, row0 + rows_valid) of a
// row-major matrix with row pitch `ld_bytes`, k-bytes [0, k_bytes) valid.
struct Operand {
  const char* base;      // address of row row0, column 0
  uint32_t ld_bytes;     // row pitch in bytes
  int rows_valid;        // rows of this tile that exist (may be <= 0)
  uint32_t k_bytes;      // valid k extent in bytes (multiple of 16)
};

struct Loader {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t rowoff[8];    // byte offset of each of this lane's 8 rows (kOOB if absent)
  uint32_t chunk_bytes;  // this lane's logical 16-byte chunk within a 128-byte slice
  uint32_t k_bytes;

  __device__ __forceinline__ void init(const Operand& op, int wave, int lane) {
    int rv = op.rows_valid < 0 ? 0 : (op.rows_valid > kBM ? kBM : op.rows_valid);
    rsrc = make_rsrc(op.base, (uint32_t)rv * op.ld_bytes);
    const int r_in = lane >> 3;                       // row within an 8-row group
    chunk_bytes = (uint32_t)(((lane & 7) ^ r_in) << 4);  // logical chunk stored at slot lane&7
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int r = wave * 64 + j * 8 + r_in;
      rowoff[j] = r < rv ? (uint32_t)r * op.ld_bytes : kOOB;
    }
    k_bytes = op.k_bytes;
  }

  // Issue the 8 direct-to-LDS copies of this wave's 64 rows of slice `kt`.
  __device__ __forceinline__ void issue(int kt, char GRPO_LDS* tile, int wave) const {
    const uint32_t kb = (uint32_t)kt * kBKB + chunk_bytes;
    const bool kok = kb < k_bytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t off = kok ? rowoff[j] + kb : kOOB;
      char GRPO_LDS* dst = tile + (wave * 64 + j * 8) * kBKB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (GRPO_LDS void*)dst, 16, off, 0, 0, 0);
    }
  }
};

__device__ __forceinline__ void wait_vmem_all() {
  // s_waitcnt vmcnt(0), leaving expcnt / lgkmcnt unconstrained
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <typename T> struct Mma;

template <> struct Mma<__bf16> {
  // one k16 step for the whole 4 x 4 block set of a wave
  __device__ __forceinline__ static void step(f32x16_t (&acc)[4][4], const char GRPO_LDS* As,
                                              const char GRPO_LDS* Bs, const uint32_t (&aoff)[4],
                                              const uint32_t (&boff)[4], uint32_t swz) {
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8_t GRPO_LDS*)(As + aoff[i] + swz);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *(const bf16x8_t GRPO_LDS*)(Bs + boff[j] + swz);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
};

template <> struct Mma<float> {
  __device__ __forceinline__ static void step(f32x16_t (&acc)[4][4], const char GRPO_LDS* As,
                                              const char GRPO_LDS* Bs, const uint32_t (&aoff)[4],
                                              const uint32_t (&boff)[4], uint32_t swz) {
    f32x4_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const f32x4_t GRPO_LDS*)(As + aoff[i] + swz);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *(const f32x4_t GRPO_LDS*)(Bs + boff[j] + swz);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
  }
};

// The main loop.  `lds` must be kLdsBytes of workgroup memory.  On return all
// waves have finished reading LDS only if the caller issues a barrier.
template <typename T>
__device__ __forceinline__ void tile_mainloop(f32x16_t (&acc)[4][4], const Operand& A,
                                              const Operand& B, int k_slices,
                                              char GRPO_LDS* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm0 = (wave >> 1) * 128;
  const int wn0 = (wave & 1) * 128;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  Loader la, lb;
  la.init(A, wave, lane);
  lb.init(B, wave, lane);

  // fragment row offsets inside a slice (bytes) and the per-step swizzle
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    aoff[i] = (uint32_t)(wm0 + 32 * i + (lane & 31)) * kBKB;
    boff[i] = (uint32_t)(wn0 + 32 * i + (lane & 31)) * kBKB;
  }
  const uint32_t half = (uint32_t)(lane >> 5);
  const uint32_t r7 = (uint32_t)(lane & 7);

  if (k_slices > 0) {
    la.issue(0, lds, wave);
    lb.issue(0, lds + kTileBytes, wave);
  }
  for (int kt = 0; kt < k_slices; ++kt) {
    char GRPO_LDS* cur = lds + (kt & 1) * kStageBytes;
    wait_vmem_all();
    __builtin_amdgcn_s_barrier();
    if (kt + 1 < k_slices) {
      char GRPO_LDS* nxt = lds + ((kt + 1) & 1) * kStageBytes;
      la.issue(kt + 1, nxt, wave);
      lb.issue(kt + 1, nxt + kTileBytes, wave);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t swz = (((2u * s + half) ^ r7) << 4);
      Mma<T>::step(acc, cur, cur + kTileBytes, aoff, boff, swz);
    }
  }
}

// Coordinates of accumulator element (i, j, e) of this lane, tile-relative.
__device__ __forceinline__ int acc_row(int wave, int lane, int i, int e) {
  return (wave >> 1) * 128 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
__device__ __forceinline__ int acc_col(int wave, int lane, int j) {
  return (wave & 1) * 128 + 32 * j + (lane & 31);
}

}  // namespace grpo
