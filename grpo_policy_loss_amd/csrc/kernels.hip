// kernels.hip -- HIP kernels of the fused chunked GRPO loss for gfx950.
//
// Forward (per chunk of flattened tokens):
//   k_lse_partials: MFMA tile z^T = W_tile . H_tile^T (vocab rows x token
//     columns), transformed (scale, softcap, temperature) and folded in
//     registers into a (max, sum-exp) pair per token for that 256-row
//     vocabulary tile, plus the transformed target logit when the target falls
//     in the tile.  Logits never leave registers.
//   k_lse_merge: fixed-order merge of the per-tile pairs into lse and lp; in
//     loss mode also kl and the masked per-block loss sums.
//   k_loss_final: fixed-order sum of the block sums -> loss.
//   (k_seq_counts: unmasked tokens per sequence, for the per-sequence mean.)
// Backward (per chunk of ACTIVE tokens, per vocabulary slab):
//   k_dz: the same tile recomputed; the epilogue forms
//     dZ = c_t (onehot(y_t) - exp(z - lse_t)) in registers and stores it once,
//     in H's dtype, into a bounded [chunk x slab] buffer laid out in strips of
//     256 vocabulary columns: strip s holds [cpad tokens][256] contiguously, so
//     a tile's 256 x 256 block is one contiguous 128 KB store.
//   k_dh_gemm: dH_acc[t][:] (+)= sum_v dZ[t][v] W[v][:]   (MFMA, fp32 acc;
//     W read K-major straight from the caller's [V, d] array)
//   k_dw_gemm: dW[v][:]     +=  sum_t dZ[t][v] h_t[:]     (MFMA, fp32 RMW;
//     the dZ slab read K-major)
// Every reduction runs in a fixed order, so results are bitwise reproducible.
#include <math.h>

#include <type_traits>

#include "kernels.hpp"
#include "tile_mma.hpp"
#include "timing.hpp"

namespace grpo {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh(x) = 1 - 2 / (exp(2x) + 1): saturates to +-1 for large |x|, absolute
// error ~1e-7 near 0 (relative to the softcap that multiplies it).
__device__ __forceinline__ float tanh_fast(float x) {
  return 1.f - 2.f * __builtin_amdgcn_rcpf(ex2(x * (2.f * kLog2e)) + 1.f);
}

// The logit transform of one raw logit (see LogitXform).
template <bool SC>
__device__ __forceinline__ float xform(float z, const LogitXform& xf) {
  return SC ? xf.b * tanh_fast(xf.a * z) : xf.k * z;
}

// Online log-sum-exp pair combination in base e, carried as (max, sum of
// exp(z - max)).  An empty side has max = -inf and sum = 0.
__device__ __forceinline__ void lse_combine(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == kNegInf) {
    s = 0.f;
    m = M;
    return;
  }
  s = s * ex2((m - M) * kLog2e) + s2 * ex2((m2 - M) * kLog2e);
  m = M;
}

// Logical tile id p -> (M-tile, N-tile), in groups of GM M-tiles (M
// fastest), so the ~32 workgroups resident on one XCD share GM A-panels and
// ~32/GM B-panels in that XCD's L2.
template <int GM>
__device__ __forceinline__ void group_coords(int p, int tm, int tn, int& mt, int& nt) {
  const int per_group = GM * tn;
  const int g = p / per_group;
  const int first = g * GM;
  const int gm = (tm - first) < GM ? (tm - first) : GM;
  const int rem = p - g * per_group;
  mt = first + rem % gm;
  nt = rem / gm;
}

// Hardware dispatches workgroup b to XCD b % 8.  Deal the logical tile ids
// [0, tiles) to the XCDs in whole blocks of 32, one wave of an XCD's 32 CUs:
// XCD x takes a contiguous range of blocks, so the tiles resident on it at
// one time are always one aligned block of the raster.  (A range starting
// part-way into a block would straddle two groups of the raster for some of
// its waves.)  The grid is xcd_grid(tiles) workgroups; false for those past
// this XCD's range.
__device__ __forceinline__ bool xcd_tile(int bid, int tiles, int& p) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int nb = (tiles + 31) >> 5;
  const int q = nb >> 3, r = nb & 7;
  const int nmine = (q + (xcd < r ? 1 : 0)) << 5;
  p = ((xcd * q + (xcd < r ? xcd : r)) << 5) + slot;
  return slot < nmine && p < tiles;
}

// Tile (mt, nt) of workgroup bid in a tm x tn grid: ids in groups of 4
// M-tiles, so one 32-tile block (with tn a multiple of 8) lies inside one
// group and its workgroups share 4 A-panels and 8 B-panels in the XCD's L2.
__device__ __forceinline__ bool tile_coords_blk(int bid, int tm, int tn, int& mt, int& nt) {
  int p;
  if (!xcd_tile(bid, tm * tn, p)) return false;
  group_coords<4>(p, tm, tn, mt, nt);
  return true;
}

template <typename T>
__device__ __forceinline__ T to_elem(float x);
template <>
__device__ __forceinline__ float to_elem<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ __bf16 to_elem<__bf16>(float x) {
  return (__bf16)x;
}

// Store 4 consecutive values (16 B for f32, 8 B for bf16).
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *(f32x4_t*)p = f32x4_t{a, b, c, d};
}
__device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
  *(bf16x4_t*)p = bf16x4_t{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------- advantages
// One wave64 per group; sums in double, fixed order.
__global__ void __launch_bounds__(64) k_advantages(const float* __restrict__ r, int64_t G,
                                                   float eps, float* __restrict__ adv) {
  const int64_t base = (int64_t)blockIdx.x * G;
  const int lane = threadIdx.x;
  double s = 0.0;
  for (int64_t i = lane; i < G; i += 64) s += (double)r[base + i];
  const double mean = wave_sum(s) / (double)G;
  double q = 0.0;
  for (int64_t i = lane; i < G; i += 64) {
    const double dv = (double)r[base + i] - mean;
    q += dv * dv;
  }
  q = wave_sum(q);
  const double sd = G > 1 ? sqrt(q / (double)(G - 1)) : 0.0;
  for (int64_t i = lane; i < G; i += 64)
    adv[base + i] = (float)(((double)r[base + i] - mean) / (sd + (double)eps));
}

// Reductions over the four 16-lane groups of a wave (lane l with l ^ 16,
// l ^ 32, l ^ 48) through the VALU lane swaps, with no LDS round trip.  The
// swaps hand every lane the same pair in the same order, so all lanes end with
// the same bits.
__device__ __forceinline__ float bits_f(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned f_bits(float f) { return __builtin_bit_cast(unsigned, f); }
__device__ __forceinline__ float group4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  x = __builtin_elementwise_maximum(bits_f(a[0]), bits_f(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  return __builtin_elementwise_maximum(bits_f(b[0]), bits_f(b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  x = bits_f(a[0]) + bits_f(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  return bits_f(b[0]) + bits_f(b[1]);
}

// (max, sum exp) of the transformed logits of every token column of this
// wave, over the wave's 128 vocabulary rows.  ROWS: rows at or past `mvalid`
// (tile-relative) are left out; otherwise every row counts and the loops have
// no per-element test.  cs[j] turns the accumulator into the logit (fp8
// scales; exactly 1 otherwise).  mx[j] is the transformed max (-inf when no
// row counts), sm[j] the sum of exp(logit - mx[j]).
template <bool SC, bool ROWS>
__device__ __forceinline__ void lse_columns(const Acc& acc, int wave, int lane, int mvalid,
                                            const float (&cs)[kWN], const LogitXform& xf,
                                            float (&mx)[kWN], float (&sm)[kWN]) {
  auto valid = [&](int i, int e) { return !ROWS || acc_row(wave, lane, i, e) < mvalid; };
  // one token column at a time, so only its 32 values are live in VGPRs
#pragma unroll
  for (int j = 0; j < kWN; ++j) {
    // the max: two independent chains of three-input maxima (v_maximum3_f32,
    // which needs no canonicalisation of its inputs)
    float ma = kNegInf, mb = kNegInf;
#pragma unroll
    for (int i = 0; i < kWM; ++i) {
      const float a0 = valid(i, 0) ? acc[i][j][0] : kNegInf;
      const float a1 = valid(i, 1) ? acc[i][j][1] : kNegInf;
      const float a2 = valid(i, 2) ? acc[i][j][2] : kNegInf;
      const float a3 = valid(i, 3) ? acc[i][j][3] : kNegInf;
      if (i == 0) {
        ma = __builtin_elementwise_maximum(a0, a1);
        mb = __builtin_elementwise_maximum(a2, a3);
      } else {
        ma = __builtin_elementwise_maximum(__builtin_elementwise_maximum(ma, a0), a1);
        mb = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mb, a2), a3);
      }
    }
    const float m = group4_max(__builtin_elementwise_maximum(ma, mb));
    const float mt = m == kNegInf ? kNegInf : xform<SC>(m * cs[j], xf);
    const float mbase = mt * kLog2e;
    // the sum: four partial sums keep four exps in flight
    float s[kAcc] = {0.f, 0.f, 0.f, 0.f};
    if (!ROWS || mt != kNegInf) {
      const float kl = xf.k * kLog2e * cs[j];
#pragma unroll
      for (int i = 0; i < kWM; ++i)
#pragma unroll
        for (int e = 0; e < kAcc; ++e) {
          const float z = acc[i][j][e];
          const float p = SC ? ex2(fmaf(xform<true>(z * cs[j], xf), kLog2e, -mbase))
                             : ex2(fmaf(z, kl, -mbase));
          if (valid(i, e)) s[e] = i == 0 ? p : s[e] + p;
        }
    }
    mx[j] = mt;
    sm[j] = group4_sum((s[0] + s[1]) + (s[2] + s[3]));
  }
}


// threadIdx.x & 63 through an opaque move, so lane-derived epilogue addresses
// are formed after the main loop instead of being hoisted across it (where
// every register is in use) and spilled.  Used by the fp8 instances, whose
// main loop holds the most fragment registers; the bf16 ones do not spill.
__device__ __forceinline__ int lane_fresh() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t & 63;
}

// ---------------------------------------------------------------- forward tile
// Epilogue of one forward tile (vocabulary rows [m0, m0 + mvalid), tokens
// [n0, n0 + 256) of the chunk): fold the accumulators into one (max, sum exp)
// pair per token for this vocabulary tile and pick the target logits.  yv[j]
// is the target of this lane's token column j (any value when the token is
// past n_tok); `red` is 512 floats of workgroup memory the main loop does not
// use.  Contains two workgroup barriers.
template <typename T, bool SC>
__device__ __forceinline__ void lse_epilogue(const Acc& acc, int mt, int64_t m0, int mvalid,
                                             int n0, int n_tok, int cpad, const LogitXform& xf,
                                             const float* __restrict__ w_scale,
                                             const float* __restrict__ h_scale,
                                             const int (&yv)[kWN], float* red,
                                             float* __restrict__ part_m,
                                             float* __restrict__ part_s, float* __restrict__ zy) {
  constexpr bool kFp8 = std::is_same<T, uint8_t>::value;
  const int lane = kFp8 ? lane_fresh() : (int)(threadIdx.x & 63), wave = wave_id();
  const int wm0 = (wave >> 1) * 128;
  const bool full = mvalid >= wm0 + 128;
  // per token column: the factor that turns the accumulator into the logit
  // (the fp8 scales, powers of two; exactly 1 otherwise)
  float cs[kWN];
#pragma unroll
  for (int j = 0; j < kWN; ++j) {
    cs[j] = 1.f;
    if constexpr (kFp8) {
      const int t = n0 + acc_col(wave, lane, j);
      cs[j] = t < n_tok ? w_scale[0] * h_scale[t] : 1.f;
    }
  }

  // per token column j: (max, sum exp) of the transformed logits over the
  // wave's 128 vocabulary rows (32 per lane, the four 16-lane groups hold the
  // rest).  The transform is increasing, so the max of the transformed logits
  // is the transform of the raw max.  The max is reduced over the wave first,
  // so every exp already uses the wave's shift and nothing is rescaled.
  float mx[kWN], sm[kWN];
  if (full)
    lse_columns<SC, false>(acc, wave, lane, mvalid, cs, xf, mx, sm);
  else
    lse_columns<SC, true>(acc, wave, lane, mvalid, cs, xf, mx, sm);

  // target logit: exactly one lane of the grid holds z[t][y_t]
#pragma unroll
  for (int j = 0; j < kWN; ++j) {
    const int t = n0 + acc_col(wave, lane, j);
    if (t < n_tok) {
      const int r = yv[j] - (int)(m0 + wm0);
      if (r >= 0 && r < 128 && r < mvalid - wm0 && ((r >> 2) & 3) == (lane >> 4)) {
        const int ti = r >> 4, te = r & 3;
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < kWM; ++i)
#pragma unroll
          for (int e = 0; e < kAcc; ++e)
            if (i == ti && e == te) v = acc[i][j][e];
        zy[t] = xform<SC>(v * cs[j], xf);
      }
    }
  }

  // combine the two waves that share token columns (w and w + 2), through LDS
  __syncthreads();
  if ((wave >> 1) == 1 && lane < 16) {
#pragma unroll
    for (int j = 0; j < kWN; ++j) {
      red[acc_col(wave, lane, j)] = mx[j];
      red[256 + acc_col(wave, lane, j)] = sm[j];
    }
  }
  __syncthreads();
  if ((wave >> 1) == 0 && lane < 16) {
#pragma unroll
    for (int j = 0; j < kWN; ++j) {
      const int c = acc_col(wave, lane, j);
      float m = mx[j], s = sm[j];
      lse_combine(m, s, red[c], red[256 + c]);
      const int t = n0 + c;
      if (t < n_tok) {
        part_m[(int64_t)mt * cpad + t] = m;
        part_s[(int64_t)mt * cpad + t] = s;
      }
    }
  }
}

// Targets of this lane's token columns.
template <bool kFresh>
__device__ __forceinline__ void load_targets(const int32_t* __restrict__ y, int n0, int n_tok,
                                             int (&yv)[kWN]) {
  const int lane = kFresh ? lane_fresh() : (int)(threadIdx.x & 63), wave = wave_id();
#pragma unroll
  for (int j = 0; j < kWN; ++j) {
    const int t = n0 + acc_col(wave, lane, j);
    yv[j] = t < n_tok ? y[t] : -1;
  }
}

// T = uint8_t: float8 e4m3 codes, with w_scale[0] the head's scale and h_scale[t]
// each token's (the logit is acc * w_scale * h_scale[t]); other T ignore both.
template <typename T, bool SC>
__global__ void __launch_bounds__(kThreads, 1)
    k_lse_partials(const T* __restrict__ W, const T* __restrict__ H, const int32_t* __restrict__ y,
                   int64_t V, int64_t d, int n_tok, int cpad, int tm, int tn, LogitXform xf,
                   const float* __restrict__ w_scale, const float* __restrict__ h_scale,
                   float* __restrict__ part_m, float* __restrict__ part_s,
                   float* __restrict__ zy) {
  constexpr bool kFp8 = std::is_same<T, uint8_t>::value;
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  char GRPO_LDS* lds = (char GRPO_LDS*)smem;
  int mt, nt;
  if (!tile_coords_blk(blockIdx.x, tm, tn, mt, nt)) return;
  const int64_t m0 = (int64_t)mt * kBM;  // first vocab row
  const int n0 = nt * kBN;               // first token (chunk-local)
  const uint32_t rowb = (uint32_t)(d * (int64_t)sizeof(T));
  const int mvalid = (int)((V - m0) < kBM ? (V - m0) : kBM);
  const Operand A{(const char*)(W + m0 * d), rowb, mvalid, rowb};
  const Operand B{(const char*)(H + (int64_t)n0 * d), rowb, n_tok - n0, rowb};

  Acc acc;
  if constexpr (kFp8)
    tile_mainloop_fp8(acc, A, B, k_slices_of(rowb), lds);
  else
    tile_mainloop<T>(acc, A, B, k_slices_of(rowb), lds);
  int yv[kWN];
  load_targets<kFp8>(y, n0, n_tok, yv);
  lse_epilogue<T, SC>(acc, mt, m0, mvalid, n0, n_tok, cpad, xf, w_scale, h_scale, yv,
                      (float*)smem, part_m, part_s, zy);
}

// ---------------------------------------------------------------- per-token KL
// The KL estimators of the blog's ablation (GRPO maths), x = ref_lp - lp:
//   reverse k3:      e^x - x - 1                      (the default)
//   forward:         r ln r - (r - 1), r = e^x, written x (e^x - 1) - (e^x - 1 - x):
//                    both terms are O(x^2), so nothing cancels near x = 0
//   reverse with q:  e^lp (e^x - x - 1), q the policy's probability of the token
__device__ __forceinline__ float kl_value(int kl, float x, float lp) {
  const float em = expm1f(x);
  const float k3 = em - x;
  if (kl == 1) return fmaf(x, em, -k3);
  if (kl == 2) return expf(lp) * k3;
  return k3;
}
// d kl / d lp (dx / dlp = -1): -(e^x - 1), -x e^x and -x e^lp.
__device__ __forceinline__ float kl_slope(int kl, float x, float lp) {
  if (kl == 1) return -x * expf(x);
  if (kl == 2) return -x * expf(lp);
  return -expm1f(x);
}

// ---------------------------------------------------------------- forward merge
// 256 threads = 16 tokens x 16 splits of the vocabulary-tile partials (256
// workgroups per 4096 tokens, so every CU gets one).  Split q folds partials
// q, q + 16, ... of its token in order, loading four at a time; the 16 split
// results are then folded in order 0..15, so the result is independent of
// timing.
constexpr int kMergeTok = kMergeTokens;
constexpr int kMergeSplit = 256 / kMergeTok;

__device__ __forceinline__ void lse_fold(float& M, float& Ssum, float m, float v) {
  if (m > M) {
    Ssum = Ssum * exp2f((M - m) * kLog2e) + v;
    M = m;
  } else {
    Ssum += v * exp2f((m - M) * kLog2e);
  }
}

__global__ void __launch_bounds__(256)
    k_lse_merge(int mode, const float* __restrict__ part_m, const float* __restrict__ part_s,
                const float* __restrict__ zy, int S, int cpad, int n_tok, int64_t c0,
                const int32_t* __restrict__ y, int64_t V, float* __restrict__ out_lp,
                float* __restrict__ out_lse, float* __restrict__ out_kl,
                const float* __restrict__ ref_lp, const uint8_t* __restrict__ mask,
                const float* __restrict__ adv, int64_t L, float beta, LossVariant lv,
                const int32_t* __restrict__ seq_n, double* loss_part, int* cnt_part, int part0) {
  __shared__ float sm_m[kMergeSplit][kMergeTok], sm_s[kMergeSplit][kMergeTok];
  const int tt = threadIdx.x % kMergeTok, q = threadIdx.x / kMergeTok;
  const int t = blockIdx.x * kMergeTok + tt;
  float M = kNegInf, Ssum = 0.f;
  if (t < n_tok) {
    const float* pm = part_m + t;
    const float* ps = part_s + t;
    int sp = q;
    for (; sp + 3 * kMergeSplit < S; sp += 4 * kMergeSplit) {
      float m4[4], v4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        m4[u] = pm[(int64_t)(sp + u * kMergeSplit) * cpad];
        v4[u] = ps[(int64_t)(sp + u * kMergeSplit) * cpad];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) lse_fold(M, Ssum, m4[u], v4[u]);
    }
    for (; sp < S; sp += kMergeSplit) lse_fold(M, Ssum, pm[(int64_t)sp * cpad], ps[(int64_t)sp * cpad]);
  }
  sm_m[q][tt] = M;
  sm_s[q][tt] = Ssum;
  __syncthreads();
  // split 0 (lanes 0..15 of wave 0) finishes its token; waves 1..3 are done
  if (threadIdx.x >= 64) return;
  double ml = 0.0;
  int cnt = 0;
  if (q == 0 && t < n_tok) {
    M = sm_m[0][tt];
    Ssum = sm_s[0][tt];
    for (int k = 1; k < kMergeSplit; ++k) lse_combine(M, Ssum, sm_m[k][tt], sm_s[k][tt]);
    const float lse = M + logf(Ssum);
    const int64_t tg = c0 + t;
    const int32_t yt = y[tg];
    const float lp = (yt >= 0 && yt < V) ? zy[t] - lse : __builtin_nanf("");
    out_lp[tg] = lp;
    if (mode == 1) {
      out_lse[tg] = lse;
      const float x = ref_lp[tg] - lp;
      const float kl = kl_value(lv.kl, x, lp);
      out_kl[tg] = kl;
      if (mask[tg] != 0) {
        // the ratio exp(lp - sg(lp)) (or exp(lp - lp)) is exactly 1 in value
        ml = (double)(-(adv[tg / L] - beta * kl));
        if (seq_n != nullptr) ml /= (double)(seq_n[tg / L] > 0 ? seq_n[tg / L] : 1);
        cnt = 1;
      }
    }
  }
  if (mode == 1) {
    // fixed-order butterfly over wave 0 (lanes 16..63 contribute 0)
    ml = wave_sum(ml);
    cnt = wave_sum(cnt);
    if (threadIdx.x == 0) {
      loss_part[part0 + blockIdx.x] = ml;
      cnt_part[part0 + blockIdx.x] = cnt;
    }
  }
}

__global__ void __launch_bounds__(256)
    k_loss_final(const double* __restrict__ loss_part, const int* __restrict__ cnt_part,
                 int nparts, int64_t seq_B, float* __restrict__ loss) {
  double s = 0.0;
  long long c = 0;
  for (int i = threadIdx.x; i < nparts; i += 256) {
    s += loss_part[i];
    c += cnt_part[i];
  }
  __shared__ double ss[256];
  __shared__ long long sc[256];
  ss[threadIdx.x] = s;
  sc[threadIdx.x] = c;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) {
      ss[threadIdx.x] += ss[threadIdx.x + w];
      sc[threadIdx.x] += sc[threadIdx.x + w];
    }
    __syncthreads();
  }
  // token mean: over the unmasked tokens; per-sequence mean: the block sums
  // already hold each sequence's mean share, so divide by the sequence count
  const double den = seq_B > 0 ? (double)seq_B : (double)(sc[0] > 0 ? sc[0] : 1);
  if (threadIdx.x == 0) loss[0] = (float)(ss[0] / den);
}

__global__ void __launch_bounds__(256)
    k_seq_counts(const uint8_t* __restrict__ mask, int64_t L, int32_t* __restrict__ n) {
  const int64_t b = blockIdx.x;
  int c = 0;
  for (int64_t j = threadIdx.x; j < L; j += 256) c += mask[b * L + j] != 0;
  c = wave_sum(c);
  __shared__ int sc[4];
  if ((threadIdx.x & 63) == 0) sc[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) n[b] = sc[0] + sc[1] + sc[2] + sc[3];
}

// ---------------------------------------------------------------- backward helpers
// Indices of the unmasked tokens in increasing order, and their count.
__global__ void __launch_bounds__(1024)
    k_active_scan(const uint8_t* __restrict__ mask, int64_t N, int32_t* __restrict__ idx,
                  int32_t* __restrict__ count) {
  __shared__ int sc[1024];
  const int tid = threadIdx.x;
  const int64_t seg = (N + 1023) / 1024;
  const int64_t b = tid * seg;
  const int64_t e = (b + seg) < N ? (b + seg) : N;
  int c = 0;
  for (int64_t i = b; i < e; ++i) c += mask[i] != 0;
  sc[tid] = c;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
    const int v = tid >= o ? sc[tid - o] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  int off = sc[tid] - c;
  for (int64_t i = b; i < e; ++i)
    if (mask[i] != 0) idx[off++] = (int32_t)i;
  if (tid == 1023) count[0] = sc[1023];
}

// out[c][r] = in[r][c] for r < R; out[c][r] = 0 for R <= r < Rpad.  One
// workgroup moves a 64 x 64 block with 16-byte accesses on both sides: rows
// of `in` are read 16 B per lane into LDS, and each lane then gathers 16 B
// worth of one column (E consecutive r) and writes it as one store.  Needs
// Cc and Rpad to be multiples of E = 16 / sizeof(T) (the host checks d).
template <typename T>
__global__ void __launch_bounds__(256)
    k_transpose(const T* __restrict__ in, int64_t R, int64_t Cc, T* __restrict__ out,
                int64_t Rpad) {
  constexpr int E = 16 / (int)sizeof(T);   // elements per 16 B
  constexpr int LPR = 64 / E;              // lanes per 64-element row
  constexpr int RPP = 256 / LPR;           // rows per pass
  constexpr int P = 64 + 2;                // LDS row pitch (elements)
  __shared__ T tile[64 * P];
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int lx = threadIdx.x % LPR, ly = threadIdx.x / LPR;
#pragma unroll
  for (int r = ly; r < 64; r += RPP) {
    const int64_t rr = r0 + r, cc = c0 + lx * E;
    int4 v = {0, 0, 0, 0};
    if (rr < R && cc < Cc) v = *(const int4*)(in + rr * Cc + cc);
    const T* e = (const T*)&v;
#pragma unroll
    for (int k = 0; k < E; ++k) tile[r * P + lx * E + k] = e[k];
  }
  __syncthreads();
#pragma unroll
  for (int c = ly; c < 64; c += RPP) {
    const int64_t cc = c0 + c, rr = r0 + lx * E;
    int4 v;
    T* e = (T*)&v;
#pragma unroll
    for (int k = 0; k < E; ++k) e[k] = tile[(lx * E + k) * P + c];
    if (cc < Cc && rr < Rpad) *(int4*)(out + cc * Rpad + rr) = v;
  }
}

// Gather the hidden states of chunk c's active tokens into H_act and form
// the per-token backward coefficient c_t, lse and target; padding rows are 0.
template <typename T>
__global__ void __launch_bounds__(256)
    k_bwd_prep(const T* __restrict__ H, int64_t d, const int32_t* __restrict__ idx,
               const int32_t* __restrict__ count, int64_t c0, int C,
               const int32_t* __restrict__ y, const float* __restrict__ adv,
               const float* __restrict__ ref_lp, const float* __restrict__ lp,
               const float* __restrict__ lse, int64_t L, float beta, float grad_loss,
               LogitXform xf, LossVariant lv, const int32_t* __restrict__ seq_n, int64_t B,
               T* __restrict__ H_act, float* __restrict__ coef,
               float* __restrict__ lse_c, int32_t* __restrict__ y_c, float* __restrict__ tgt_c) {
  const int cnt = count[0];
  if (c0 >= cnt) return;
  const int j = blockIdx.x;
  const bool valid = j < C && c0 + j < cnt;
  const int64_t t = valid ? idx[c0 + j] : 0;
  const int nvec = (int)(d * (int64_t)sizeof(T) / 16);
  const int4* src = (const int4*)(H + t * d);
  int4* dst = (int4*)(H_act + (int64_t)j * d);
  for (int v = threadIdx.x; v < nvec; v += 256) dst[v] = valid ? src[v] : int4{0, 0, 0, 0};
  if (threadIdx.x == 0) {
    if (valid) {
      // c_t = d loss / d lp_t = w_t (-[detached] A + beta d kl / d lp), w_t the
      // aggregation weight of an unmasked token
      const float x = ref_lp[t] - lp[t];
      const int64_t b = t / L;
      const float scale =
          seq_n != nullptr
              ? grad_loss / ((float)B * (float)(seq_n[b] > 0 ? seq_n[b] : 1))
              : grad_loss / (float)(cnt > 0 ? cnt : 1);
      const float a_term = lv.no_detach ? 0.f : -adv[b];
      const float c = scale * (a_term + beta * kl_slope(lv.kl, x, lp[t]));
      coef[j] = c;
      lse_c[j] = lse[t];
      y_c[j] = y[t];
      // the target's own dZ entry c (1 - p_y) f'(z_y), with p_y = exp(lp): the
      // logit the backward recomputes is bitwise the forward's, so lp holds the
      // same p_y; with a cap, f'(z_y) = a b (1 - t^2), t = z'_y / b = (lp + lse) / b
      float slope = xf.k;
      if (xf.softcap) {
        const float tt = fminf(1.f, fmaxf(-1.f, (lp[t] + lse[t]) / xf.b));
        slope = xf.a * xf.b * (1.f - tt * tt);
      }
      tgt_c[j] = c * -expm1f(lp[t]) * slope;
    } else {
      coef[j] = 0.f;
      lse_c[j] = 0.f;
      y_c[j] = -1;
      tgt_c[j] = 0.f;
    }
  }
}

// ---------------------------------------------------------------- backward tiles
// LDS staging tile for the dZ stores: 256 rows of 256 bf16 with a 528-byte
// pitch (16-byte aligned rows, shifted by one 16-byte bank group per row).
constexpr int kStagePitch = 528;
constexpr int kDzLdsBytes = (kLdsBytes > 256 * kStagePitch) ? kLdsBytes : 256 * kStagePitch;

// c_t (onehot - p) f'(z) for one raw logit z (float32 path).
template <bool SC>
__device__ __forceinline__ float dz_value(float z, float ct, float lb, int64_t v, int64_t yl,
                                          int vs_valid, const LogitXform& xf) {
  float slope = xf.k, zt = xf.k * z;
  if (SC) {
    const float t = tanh_fast(xf.a * z);
    zt = xf.b * t;
    slope = xf.a * xf.b * (1.f - t * t);
  }
  const float p = ex2(fmaf(zt, kLog2e, -lb));
  const float onehot = v == yl ? 1.f : 0.f;
  return v < vs_valid ? ct * (onehot - p) * slope : 0.f;
}

// Stage -c_t p f'(z) of every accumulator entry of this lane as bf16 into the
// [token][vocabulary] LDS tile (pitch kStagePitch).  ROWS: vocabulary rows at
// or past `rows` (tile-relative) are written as 0; otherwise no per-element
// test.  Values go from the accumulators straight to packed bf16 in VGPRs.
template <bool SC, bool ROWS>
__device__ __forceinline__ void dz_stage(const Acc& acc, int wave, int lane, int rows,
                                         const float (&ct)[kWN], const float (&lb)[kWN],
                                         const float (&cs)[kWN], const LogitXform& xf,
                                         char GRPO_LDS* lds) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
#pragma unroll
  for (int j = 0; j < kWN; ++j) {
    const int tl = acc_col(wave, lane, j);
    const float nc = SC ? -ct[j] * xf.a * xf.b : -ct[j] * xf.k;
    const float kl = xf.k * kLog2e * cs[j];
#pragma unroll
    for (int i = 0; i < kWM; ++i) {
      const int vl = acc_row(wave, lane, i, 0);
      float q[kAcc];
#pragma unroll
      for (int e = 0; e < kAcc; ++e) {
        if (SC) {
          const float t = tanh_fast(xf.a * (acc[i][j][e] * cs[j]));
          q[e] = nc * (1.f - t * t) * ex2(fmaf(xf.b * t, kLog2e, -lb[j]));
        } else {
          q[e] = nc * ex2(fmaf(acc[i][j][e], kl, -lb[j]));
        }
        if (ROWS && vl + e >= rows) q[e] = 0.f;
      }
      *(bf16x4_t GRPO_LDS*)(lds + tl * kStagePitch + vl * 2) =
          bf16x4_t{(__bf16)q[0], (__bf16)q[1], (__bf16)q[2], (__bf16)q[3]};
    }
  }
}

// T = uint8_t: the logits are recomputed from float8 e4m3 codes (w_scale[0] the
// head's scale, hs_act[j] active token j's), exactly as the fp8 forward formed
// them, and dZ is bfloat16; other T ignore both scale pointers.
template <typename T, bool SC>
__global__ void __launch_bounds__(kThreads, 1)
    k_dz(const T* __restrict__ W, const T* __restrict__ H_act, int64_t d, int64_t v0,
         int vs_valid, int vs, const int32_t* __restrict__ count, int64_t c0, int C, int cpad,
         int tm, int tn, LogitXform xf, const float* __restrict__ w_scale,
         const float* __restrict__ hs_act, const float* __restrict__ coef,
         const float* __restrict__ lse_c,
         const int32_t* __restrict__ y_c, const float* __restrict__ tgt_c,
         typename DzOut<T>::type* __restrict__ dZ) {
  constexpr bool kFp8 = std::is_same<T, uint8_t>::value;
  __shared__ __attribute__((aligned(1024))) char smem[kDzLdsBytes];
  char GRPO_LDS* lds = (char GRPO_LDS*)smem;
  int n_act = count[0] - (int)c0;
  n_act = n_act < 0 ? 0 : (n_act > C ? C : n_act);
  int mt, nt;
  if (!tile_coords_blk(blockIdx.x, tm, tn, mt, nt)) return;
  const int n0 = nt * kBN;
  if (n0 >= n_act) return;
  const int m0 = mt * kBM;
  const uint32_t rowb = (uint32_t)(d * (int64_t)sizeof(T));
  const Operand A{(const char*)(W + (v0 + m0) * d), rowb, vs_valid - m0, rowb};
  const Operand B{(const char*)(H_act + (int64_t)n0 * d), rowb, n_act - n0, rowb};
  Acc acc;
  if constexpr (kFp8)
    tile_mainloop_fp8(acc, A, B, k_slices_of(rowb), lds);
  else
    tile_mainloop<T>(acc, A, B, k_slices_of(rowb), lds);

  const int lane = kFp8 ? lane_fresh() : (int)(threadIdx.x & 63), wave = wave_id();
  float ct[kWN], lb[kWN], cs[kWN];
  int64_t yl[kWN];
#pragma unroll
  for (int j = 0; j < kWN; ++j) {
    const int t = n0 + acc_col(wave, lane, j);
    ct[j] = coef[t];
    lb[j] = lse_c[t] * kLog2e;
    yl[j] = (int64_t)y_c[t] - v0;  // target relative to the slab
    cs[j] = 1.f;                    // accumulator -> logit (fp8 scales; exactly 1 otherwise)
    if constexpr (kFp8) cs[j] = w_scale[0] * hs_act[t];
  }
  if constexpr (std::is_same<T, float>::value) {
    // float32 (small shapes only): direct stores
#pragma unroll
    for (int j = 0; j < kWN; ++j) {
      const int t = n0 + acc_col(wave, lane, j);
#pragma unroll
      for (int i = 0; i < kWM; ++i) {
        const int v = m0 + acc_row(wave, lane, i, 0);
        float q[kAcc];
#pragma unroll
        for (int u = 0; u < kAcc; ++u)
          q[u] = dz_value<SC>(acc[i][j][u], ct[j], lb[j], v + u, yl[j], vs_valid, xf);
        store4(dZ + ((int64_t)(v >> 8) * cpad + t) * 256 + (v & 255), q[0], q[1], q[2], q[3]);
      }
    }
    return;
  }
  typedef __attribute__((ext_vector_type(4))) int i32x4_t;
  // 1. every entry as if it were not the target, -c_t p f'(z), rounded to bf16
  // and staged as [token][vocab]: each lane holds 4 consecutive vocabulary rows
  // of one token per block.  Rows past the slab (ragged last vocabulary tile)
  // hold zeros.  The barrier first: other waves may still read the main loop's
  // operands from LDS.
  __syncthreads();
  if (m0 + kBM > vs_valid)
    dz_stage<SC, true>(acc, wave, lane, vs_valid - m0, ct, lb, cs, xf, lds);
  else
    dz_stage<SC, false>(acc, wave, lane, vs_valid - m0, ct, lb, cs, xf, lds);
  __syncthreads();
  // 2. the target entry of each token, c_t (1 - p_y) f'(z_y), if it falls in this tile
  for (int tl = (int)threadIdx.x; tl < kBN; tl += kThreads) {
    const int64_t yr = (int64_t)y_c[n0 + tl] - v0 - m0;  // y_c = -1 for padding tokens
    if (yr >= 0 && yr < kBM && m0 + yr < vs_valid)
      *(__bf16 GRPO_LDS*)(lds + tl * kStagePitch + yr * 2) = (__bf16)tgt_c[n0 + tl];
  }
  __syncthreads();
  // 3. The tile: tokens n0 .. n0 + 255 of strip m0 / 256, one contiguous
  // 128 KB block (512 bytes per token), 16 bytes per thread.  The slab is read
  // back only after the whole launch, so its stores are non-temporal: they do
  // not evict the W panels the other tiles re-read.
  typename DzOut<T>::type* const blk = dZ + ((int64_t)(m0 >> 8) * cpad + n0) * 256;
#pragma unroll 8
  for (int it = 0; it < kBN * 32 / kThreads; ++it) {
    const int idx = it * kThreads + (int)threadIdx.x;
    const int r = idx >> 5, c = idx & 31;
    __builtin_nontemporal_store(*(const i32x4_t GRPO_LDS*)(lds + r * kStagePitch + c * 16),
                                (i32x4_t*)(blk + r * 256 + c * 8));
  }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Write (accumulate = false) or add (accumulate = true) the tile's fp32
// accumulators into a row-major [rows x d] block whose tile row r (the GEMM's
// N index) starts at base + r * d and whose columns are m0 + (the GEMM's M
// index).  Addressing goes through a buffer resource spanning exactly the
// valid rows: a row past `rows` or a column past d (offset kOOB) loads 0 and
// drops its store, so there is no branch.  When accumulating, the 8 loads of
// column block j+1 are in flight while block j is added and stored: one
// memory round trip per block instead of one per load.
// SW: the accumulators are in the transposed layout of tile_mainloop<..., SWAP>
// (tile row r = its A index, columns m0 + its B index); acc[i][j] then plays
// the part of acc[j][i] below.
template <bool SW = false>
__device__ __forceinline__ void store_tile_f32(float* base, int rows, int64_t m0, int64_t d,
                                               const Acc& acc, bool accumulate) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(base, (uint32_t)((int64_t)rows * d * (int64_t)sizeof(float)));
  // tile row of block j's lane, and its first column in block i
  const int wr = SW ? (wave >> 1) * 128 : (wave & 1) * 128;
  const int wc = SW ? (wave & 1) * 128 : (wave >> 1) * 128;
  uint32_t coff[kWM];
#pragma unroll
  for (int i = 0; i < kWM; ++i) {
    const int64_t nd = m0 + wc + 16 * i + 4 * (lane >> 4);   // 4 consecutive d
    coff[i] = nd < d ? (uint32_t)nd * 4u : kOOB;
  }
  auto row_off = [&](int j) { return (uint32_t)(wr + 16 * j + (lane & 15)) * (uint32_t)d * 4u; };
  auto blk = [&](int i, int j) -> const f32x4_t& { return SW ? acc[j][i] : acc[i][j]; };
  auto at = [](uint32_t r, uint32_t c) { return c == kOOB ? c : r + c; };
  if (!accumulate) {
#pragma unroll
    for (int j = 0; j < kWN; ++j) {
      const uint32_t r = row_off(j);
#pragma unroll
      for (int i = 0; i < kWM; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, blk(i, j)), rs,
                                               at(r, coff[i]), 0, 0);
    }
    return;
  }
  f32x4_t cur[kWM], nxt[kWM];
#pragma unroll
  for (int i = 0; i < kWM; ++i)
    cur[i] = __builtin_bit_cast(
        f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, at(row_off(0), coff[i]), 0, 0));
#pragma unroll
  for (int j = 0; j < kWN; ++j) {
    if (j + 1 < kWN) {
      const uint32_t rn = row_off(j + 1);
#pragma unroll
      for (int i = 0; i < kWM; ++i)
        nxt[i] = __builtin_bit_cast(
            f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, at(rn, coff[i]), 0, 0));
    }
    const uint32_t r = row_off(j);
#pragma unroll
    for (int i = 0; i < kWM; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, cur[i] + blk(i, j)), rs,
                                             at(r, coff[i]), 0, 0);
    if (j + 1 < kWN) {
#pragma unroll
      for (int i = 0; i < kWM; ++i) cur[i] = nxt[i];
    }
  }
}

// dH partial of split `sp`: vocabulary columns [k0, k1) of the slab.  Split
// sp accumulates into its own buffer dH_acc[sp], so no two workgroups ever
// write the same element and the final sum over splits has a fixed order.
// The GEMM's A operand (rows = hidden dimension, K = vocabulary) is W itself,
// read K-major: no transposed copy of the head is made.
template <typename T>
__global__ void __launch_bounds__(kThreads, 1)
    k_dh_gemm(const T* __restrict__ W, int64_t v0, int vs_valid, const T* __restrict__ dZ, int vs,
              int64_t d, const int32_t* __restrict__ count, int64_t c0, int C, int cpad, int tm,
              int tn, int nsplit, int kchunk, int first, float* __restrict__ dH_acc) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  char GRPO_LDS* lds = (char GRPO_LDS*)smem;
  int n_act = count[0] - (int)c0;
  n_act = n_act < 0 ? 0 : (n_act > C ? C : n_act);
  // split index outermost, then the raster inside one split; the XCDs take
  // whole blocks of the flattened order, so each holds few splits at a time
  const int per_split = tm * tn;
  int p;
  if (!xcd_tile(blockIdx.x, per_split * nsplit, p)) return;
  const int sp = p / per_split;
  int mt, nt;
  group_coords<4>(p - sp * per_split, tm, tn, mt, nt);
  const int n0 = nt * kBN;
  if (n0 >= n_act) return;
  const int64_t m0 = (int64_t)mt * kBM;
  const int k0 = sp * kchunk;
  const int k1 = (k0 + kchunk) < vs_valid ? (k0 + kchunk) : vs_valid;
  const int klen = k1 > k0 ? k1 - k0 : 0;
  const uint32_t kb = (uint32_t)(((int64_t)klen * (int64_t)sizeof(T) + 15) & ~(int64_t)15);
  const int64_t ldw = d * (int64_t)sizeof(T);
  Operand A{(const char*)(W + (v0 + k0) * d + m0), (uint32_t)ldw,
            (int)((d - m0) < kBM ? (d - m0) : kBM), 0};
  A.k_rows = (uint32_t)klen;
  A.range = klen > 0 ? (uint32_t)((int64_t)klen * ldw - m0 * (int64_t)sizeof(T)) : 0u;
  // B: the slab's tokens n0 .. (rows), vocabulary columns from k0 (a multiple of
  // 256: strip k0 / 256), read strip by strip
  const int64_t strip = (int64_t)cpad * 256;   // elements of one 256-column strip
  Operand B{(const char*)(dZ + (k0 >> 8) * strip + (int64_t)n0 * 256),
            (uint32_t)(256 * sizeof(T)), n_act - n0, kb};
  B.blk_stride = (uint32_t)(strip * (int64_t)sizeof(T));
  const int64_t rest = ((int64_t)(vs >> 8) - (k0 >> 8)) * strip - (int64_t)n0 * 256;
  B.range = rest > 0 ? (uint32_t)(rest * (int64_t)sizeof(T)) : 0u;   // 0: empty split
  Acc acc;
  tile_mainloop<T, true, false, false, true>(acc, A, B, k_slices_of(kb), lds);
  if (klen == 0 && !first) return;

  const int rows = (n_act - n0) < kBN ? (n_act - n0) : kBN;
  store_tile_f32(dH_acc + ((int64_t)sp * cpad + n0) * d, rows, m0, d, acc, !first);
}

// dW rows v0 + [m0, m0 + 256) (the GEMM's M = vocabulary) by hidden columns
// [n0, n0 + 256) (N = hidden dimension), K = the chunk's active tokens: A is
// one 256-column strip of the dZ slab read K-major, B the transposed
// hidden-state chunk.
// The blocks are computed transposed (SWAP), so each lane holds four
// consecutive hidden columns of one vocabulary row, as dW's rows are laid out.
template <typename T>
__global__ void __launch_bounds__(kThreads, 1)
    k_dw_gemm(const T* __restrict__ HT, int cpad, const T* __restrict__ dZ, int vs, int64_t d,
              int64_t v0, int vs_valid, const int32_t* __restrict__ count, int64_t c0, int C,
              int tm, int tn, float* __restrict__ dW) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  char GRPO_LDS* lds = (char GRPO_LDS*)smem;
  int n_act = count[0] - (int)c0;
  n_act = n_act < 0 ? 0 : (n_act > C ? C : n_act);
  if (n_act <= 0) return;
  int mt, nt;
  if (!tile_coords_blk(blockIdx.x, tm, tn, mt, nt)) return;
  const int m0 = mt * kBM;                  // first vocabulary row of the slab
  const int64_t n0 = (int64_t)nt * kBN;     // first hidden column
  const uint32_t kb = (uint32_t)(((int64_t)n_act * (int64_t)sizeof(T) + 15) & ~(int64_t)15);
  // A: strip m0 / 256 of the slab, [tokens][256 vocabulary columns], K-major
  const int64_t ldz = 256 * (int64_t)sizeof(T);
  Operand A{(const char*)(dZ + (int64_t)(m0 >> 8) * cpad * 256), (uint32_t)ldz, vs_valid - m0, 0};
  A.k_rows = (uint32_t)n_act;
  A.range = (uint32_t)((int64_t)n_act * ldz);
  const uint32_t ldb = (uint32_t)(cpad * (int64_t)sizeof(T));
  const Operand B{(const char*)(HT + n0 * cpad), ldb, (int)((d - n0) < kBN ? (d - n0) : kBN), kb};
  Acc acc;
  tile_mainloop<T, true, false, true>(acc, A, B, k_slices_of(kb), lds);

  const int rows = (vs_valid - m0) < kBM ? (vs_valid - m0) : kBM;
  store_tile_f32<true>(dW + (v0 + m0) * d, rows, n0, d, acc, true);
}

template <typename T>
__global__ void __launch_bounds__(256)
    k_dh_scatter(const float* __restrict__ dH_acc, int nsplit, int cpad, int64_t d,
                 const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int64_t c0,
                 int C, T* __restrict__ dH) {
  int n_act = count[0] - (int)c0;
  n_act = n_act < 0 ? 0 : (n_act > C ? C : n_act);
  const int j = blockIdx.x;
  if (j >= n_act) return;
  const int64_t t = idx[c0 + j];
  for (int64_t k = threadIdx.x * 4; k < d; k += 1024) {
    f32x4_t v = *(const f32x4_t*)(dH_acc + (int64_t)j * d + k);
    for (int sp = 1; sp < nsplit; ++sp)
      v += *(const f32x4_t*)(dH_acc + ((int64_t)sp * cpad + j) * d + k);
    store4(dH + t * d + k, v[0], v[1], v[2], v[3]);
  }
}

__global__ void __launch_bounds__(256) k_zero(int4* __restrict__ p, int64_t n16, char* tail,
                                              int ntail) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    p[i] = int4{0, 0, 0, 0};
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

template <typename T>
__global__ void __launch_bounds__(kThreads, 1)
    k_gemm_nt(const T* __restrict__ A, const T* __restrict__ B, int64_t M, int64_t N, int64_t K,
              int tm, int tn, float* __restrict__ C) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  char GRPO_LDS* lds = (char GRPO_LDS*)smem;
  int mt, nt;
  if (!tile_coords_blk(blockIdx.x, tm, tn, mt, nt)) return;
  const int64_t m0 = (int64_t)mt * kBM, n0 = (int64_t)nt * kBN;
  const uint32_t rowb = (uint32_t)(K * (int64_t)sizeof(T));
  const Operand Ao{(const char*)(A + m0 * K), rowb, (int)((M - m0) < kBM ? (M - m0) : kBM), rowb};
  const Operand Bo{(const char*)(B + n0 * K), rowb, (int)((N - n0) < kBN ? (N - n0) : kBN), rowb};
  Acc acc;
  tile_mainloop<T>(acc, Ao, Bo, k_slices_of(rowb), lds);
  const int lane = threadIdx.x & 63, wave = wave_id();
#pragma unroll
  for (int i = 0; i < kWM; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j)
#pragma unroll
      for (int e = 0; e < kAcc; ++e) {
        const int64_t m = m0 + acc_row(wave, lane, i, e), n = n0 + acc_col(wave, lane, j);
        if (m < M && n < N) C[m * N + n] = acc[i][j][e];
      }
}

// ---------------------------------------------------------------- fp8 quantisation
// Scale exponent of a block of values: the smallest e with absmax <= 448 * 2^e
// (0 for absmax = 0), decided by exact comparisons: absmax = f 2^k with
// f in [0.5, 1) and 448 = 0.875 2^9.
__device__ __forceinline__ int fp8_exponent(float absmax) {
  if (!(absmax > 0.f)) return 0;
  int k;
  const float f = frexpf(absmax, &k);
  return f <= 0.875f ? k - 9 : k - 8;
}

__device__ __forceinline__ float block_max256(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <typename T>
__device__ __forceinline__ float to_float(T x) { return (float)x; }

// Largest |x| of each block's share of X[0 .. n): part[blockIdx.x].  A pure
// read of the tensor (HBM-bound): 16-byte loads, four in flight per thread,
// when X is 16-byte aligned; element loads for the rest.
template <typename T>
__global__ void __launch_bounds__(256)
    k_fp8_absmax_partial(const T* __restrict__ X, int64_t n, float* __restrict__ part) {
  typedef __attribute__((ext_vector_type(4))) int i32x4_t;
  constexpr int E = 16 / (int)sizeof(T);   // elements per 16-byte vector
  __shared__ float red[4];
  float m = 0.f;
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t first = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t done = 0;   // elements covered by the vector loop
  if (((uintptr_t)X & 15) == 0) {
    const int64_t nv = n / E;
    const i32x4_t* V = (const i32x4_t*)X;
    auto fold = [&](const i32x4_t& v) {
      const T* e = (const T*)&v;
#pragma unroll
      for (int k = 0; k < E; ++k) m = fmaxf(m, fabsf(to_float(e[k])));
    };
    int64_t i = first;
    for (; i + 3 * stride < nv; i += 4 * stride) {
      const i32x4_t v0 = V[i], v1 = V[i + stride], v2 = V[i + 2 * stride], v3 = V[i + 3 * stride];
      fold(v0);
      fold(v1);
      fold(v2);
      fold(v3);
    }
    for (; i < nv; i += stride) fold(V[i]);
    done = nv * E;
  }
  for (int64_t i = done + first; i < n; i += stride) m = fmaxf(m, fabsf(to_float(X[i])));
  m = block_max256(m, red);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// The tensor's exponent and scale from the partial maxima.
__global__ void __launch_bounds__(256)
    k_fp8_tensor_exponent(const float* __restrict__ part, int nparts, int* __restrict__ e_out,
                          float* __restrict__ scale_out) {
  __shared__ float red[4];
  float m = 0.f;
  for (int i = threadIdx.x; i < nparts; i += 256) m = fmaxf(m, part[i]);
  m = block_max256(m, red);
  if (threadIdx.x == 0) {
    const int e = fp8_exponent(m);
    e_out[0] = e;
    scale_out[0] = ldexpf(1.f, e);
  }
}

// One block per row: the row's exponent (its own, or the tensor's from e_tensor),
// its scale, and the e4m3 codes of x * 2^-e (an exact scaling; the conversion
// rounds to nearest, ties to even).  cols is a multiple of 4.
template <typename T>
__global__ void __launch_bounds__(256)
    k_fp8_quant_rows(const T* __restrict__ X, int64_t cols, const int* __restrict__ e_tensor,
                     uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const T* x = X + r * cols;
  int e;
  if (e_tensor != nullptr) {
    e = e_tensor[0];
  } else {
    float m = 0.f;
    for (int64_t c = threadIdx.x; c < cols; c += 256) m = fmaxf(m, fabsf(to_float(x[c])));
    e = fp8_exponent(block_max256(m, red));
    if (threadIdx.x == 0) scales[r] = ldexpf(1.f, e);
  }
  uint32_t* out = (uint32_t*)(codes + r * cols);
  for (int64_t w = threadIdx.x; w < cols / 4; w += 256) {
    const float a = ldexpf(to_float(x[4 * w + 0]), -e), b = ldexpf(to_float(x[4 * w + 1]), -e);
    const float c = ldexpf(to_float(x[4 * w + 2]), -e), dd = ldexpf(to_float(x[4 * w + 3]), -e);
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, dd, v, true);
    out[w] = (uint32_t)v;
  }
}

// bf16 copy of codes * scale (exact: 4 significant bits times a power of two).
__global__ void __launch_bounds__(256)
    k_fp8_dequant_rows(const uint8_t* __restrict__ codes, int64_t cols,
                       const float* __restrict__ scales, int per_row, __bf16* __restrict__ out) {
  const int64_t r = blockIdx.x;
  const float sc = scales[per_row ? r : 0];
  const uint32_t* in = (const uint32_t*)(codes + r * cols);
  __bf16* o = out + r * cols;
  for (int64_t w = threadIdx.x; w < cols / 4; w += 256) {
    const int v = (int)in[w];
    store4(o + 4 * w, __builtin_amdgcn_cvt_f32_fp8(v, 0) * sc, __builtin_amdgcn_cvt_f32_fp8(v, 1) * sc,
           __builtin_amdgcn_cvt_f32_fp8(v, 2) * sc, __builtin_amdgcn_cvt_f32_fp8(v, 3) * sc);
  }
}

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
// Workgroups for tile_coords_blk: whole 32-tile blocks, the same number on each
// of the 8 XCDs (ceil(tiles / 256) waves, as for tiles workgroups).
inline int xcd_grid(int tiles) { return 256 * cdiv(cdiv(tiles, 32), 8); }

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_advantages(const float* rewards, int64_t groups, int64_t G, float eps,
                             float* adv, hipStream_t s) {
  ScopedKernelTimer timer_(KK_ADVANTAGES, s);
  hipLaunchKernelGGL(k_advantages, dim3((unsigned)groups), dim3(64), 0, s, rewards, G, eps, adv);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_lse_partials(const T* W, const T* H, const int32_t* y, int64_t V, int64_t d,
                               int n_tok, int cpad, const LogitXform& xf, const float* w_scale,
                               const float* h_scale, float* part_m, float* part_s, float* zy,
                               hipStream_t s) {
  ScopedKernelTimer timer_(KK_LSE_PARTIALS, s);
  const int tm = cdiv(V, kBM), tn = cdiv(n_tok, kBN);
  if (xf.softcap)
    hipLaunchKernelGGL((k_lse_partials<T, true>), dim3(xcd_grid(tm * tn)), dim3(kThreads), 0, s, W, H, y, V,
                       d, n_tok, cpad, tm, tn, xf, w_scale, h_scale, part_m, part_s, zy);
  else
    hipLaunchKernelGGL((k_lse_partials<T, false>), dim3(xcd_grid(tm * tn)), dim3(kThreads), 0, s, W, H, y,
                       V, d, n_tok, cpad, tm, tn, xf, w_scale, h_scale, part_m, part_s, zy);
  return hipGetLastError();
}

hipError_t launch_lse_merge(int mode, const float* part_m, const float* part_s, const float* zy,
                            int S, int cpad, int n_tok, int64_t c0, const int32_t* y, int64_t V,
                            float* out_lp, float* out_lse, float* out_kl, const float* ref_lp,
                            const uint8_t* mask, const float* adv, int64_t L, float beta,
                            const LossVariant& lv, const int32_t* seq_n, double* loss_part,
                            int* cnt_part, int part0, hipStream_t s) {
  ScopedKernelTimer timer_(KK_LSE_MERGE, s);
  hipLaunchKernelGGL(k_lse_merge, dim3(cdiv(n_tok, kMergeTok)), dim3(256), 0, s, mode, part_m, part_s,
                     zy, S, cpad, n_tok, c0, y, V, out_lp, out_lse, out_kl, ref_lp, mask, adv, L,
                     beta, lv, seq_n, loss_part, cnt_part, part0);
  return hipGetLastError();
}

hipError_t launch_loss_final(const double* loss_part, const int* cnt_part, int nparts,
                             int64_t seq_B, float* loss, hipStream_t s) {
  ScopedKernelTimer timer_(KK_LOSS_FINAL, s);
  hipLaunchKernelGGL(k_loss_final, dim3(1), dim3(256), 0, s, loss_part, cnt_part, nparts, seq_B,
                     loss);
  return hipGetLastError();
}

hipError_t launch_seq_counts(const uint8_t* mask, int64_t B, int64_t L, int32_t* n, hipStream_t s) {
  ScopedKernelTimer timer_(KK_SEQ_COUNTS, s);
  hipLaunchKernelGGL(k_seq_counts, dim3((unsigned)B), dim3(256), 0, s, mask, L, n);
  return hipGetLastError();
}

hipError_t launch_active_scan(const uint8_t* mask, int64_t N, int32_t* idx, int32_t* count,
                              hipStream_t s) {
  ScopedKernelTimer timer_(KK_ACTIVE_SCAN, s);
  hipLaunchKernelGGL(k_active_scan, dim3(1), dim3(1024), 0, s, mask, N, idx, count);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_transpose(const T* in, int64_t R, int64_t Cc, T* out, int64_t Rpad,
                            hipStream_t s) {
  ScopedKernelTimer timer_(KK_TRANSPOSE, s);
  hipLaunchKernelGGL(k_transpose<T>, dim3(cdiv(Rpad, 64), cdiv(Cc, 64)), dim3(256), 0, s, in, R,
                     Cc, out, Rpad);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_prep(const T* H, int64_t d, const int32_t* idx, const int32_t* count,
                           int64_t c0, int C, int cpad, const int32_t* y, const uint8_t* mask,
                           const float* adv, const float* ref_lp, const float* lp,
                           const float* lse, int64_t L, float beta, float grad_loss,
                           const LogitXform& xf, const LossVariant& lv, const int32_t* seq_n,
                           int64_t B, T* H_act, float* coef, float* lse_c, int32_t* y_c,
                           float* tgt_c, hipStream_t s) {
  ScopedKernelTimer timer_(KK_BWD_PREP, s);
  (void)mask;
  hipLaunchKernelGGL(k_bwd_prep<T>, dim3(cpad), dim3(256), 0, s, H, d, idx, count, c0, C, y, adv,
                     ref_lp, lp, lse, L, beta, grad_loss, xf, lv, seq_n, B, H_act, coef, lse_c,
                     y_c, tgt_c);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dz(const T* W, const T* H_act, int64_t d, int64_t V, int64_t v0, int vs_valid,
                     int vs, const int32_t* count, int64_t c0, int C, int cpad,
                     const LogitXform& xf, const float* w_scale, const float* hs_act,
                     const float* coef, const float* lse_c, const int32_t* y_c,
                     const float* tgt_c, typename DzOut<T>::type* dZ, hipStream_t s) {
  ScopedKernelTimer timer_(KK_DZ, s);
  (void)V;
  const int tm = cdiv(vs_valid, kBM), tn = cdiv(C, kBN);
  if (xf.softcap)
    hipLaunchKernelGGL((k_dz<T, true>), dim3(xcd_grid(tm * tn)), dim3(kThreads), 0, s, W, H_act, d, v0,
                       vs_valid, vs, count, c0, C, cpad, tm, tn, xf, w_scale, hs_act, coef, lse_c,
                       y_c, tgt_c, dZ);
  else
    hipLaunchKernelGGL((k_dz<T, false>), dim3(xcd_grid(tm * tn)), dim3(kThreads), 0, s, W, H_act, d, v0,
                       vs_valid, vs, count, c0, C, cpad, tm, tn, xf, w_scale, hs_act, coef, lse_c,
                       y_c, tgt_c, dZ);
  return hipGetLastError();
}

// fp8 codes and scales of chunk c's active tokens (zeros past the count).
__global__ void __launch_bounds__(256)
    k_fp8_gather_rows(const uint8_t* __restrict__ H8, const float* __restrict__ h_scale,
                      int64_t d, const int32_t* __restrict__ idx,
                      const int32_t* __restrict__ count, int64_t c0, int C,
                      uint8_t* __restrict__ H8_act, float* __restrict__ hs_act) {
  const int cnt = count[0];
  const int j = blockIdx.x;
  const bool valid = j < C && c0 + j < cnt;
  const int64_t t = valid ? idx[c0 + j] : 0;
  const int4* src = (const int4*)(H8 + t * d);
  int4* dst = (int4*)(H8_act + (int64_t)j * d);
  for (int v = threadIdx.x; v < (int)(d / 16); v += 256) dst[v] = valid ? src[v] : int4{0, 0, 0, 0};
  if (threadIdx.x == 0) hs_act[j] = valid ? h_scale[t] : 0.f;
}

hipError_t launch_fp8_gather_rows(const uint8_t* H8, const float* h_scale, int64_t d,
                                  const int32_t* idx, const int32_t* count, int64_t c0, int C,
                                  int cpad, uint8_t* H8_act, float* hs_act, hipStream_t s) {
  ScopedKernelTimer timer_(KK_BWD_PREP, s);
  hipLaunchKernelGGL(k_fp8_gather_rows, dim3(cpad), dim3(256), 0, s, H8, h_scale, d, idx, count,
                     c0, C, H8_act, hs_act);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dh_gemm(const T* W, int64_t v0, int vs_valid, const T* dZ, int vs, int64_t d,
                          const int32_t* count, int64_t c0, int C, int cpad, int nsplit, int first,
                          float* dH_acc, hipStream_t s) {
  ScopedKernelTimer timer_(KK_DH_GEMM, s);
  const int tm = cdiv(d, kBM), tn = cdiv(C, kBN);
  // K range per split: a whole number of the slab's 256-column strips
  const int kchunk = (int)(((int64_t)cdiv(vs_valid, nsplit) + 255) / 256 * 256);
  hipLaunchKernelGGL(k_dh_gemm<T>, dim3(xcd_grid(tm * tn * nsplit)), dim3(kThreads), 0, s, W, v0, vs_valid,
                     dZ, vs, d, count, c0, C, cpad, tm, tn, nsplit, kchunk, first, dH_acc);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dw_gemm(const T* HT, int cpad, const T* dZ, int vs, int64_t d, int64_t v0,
                          int vs_valid, const int32_t* count, int64_t c0, int C, float* dW,
                          hipStream_t s) {
  ScopedKernelTimer timer_(KK_DW_GEMM, s);
  const int tm = cdiv(vs_valid, kBM), tn = cdiv(d, kBN);
  hipLaunchKernelGGL(k_dw_gemm<T>, dim3(xcd_grid(tm * tn)), dim3(kThreads), 0, s, HT, cpad, dZ, vs, d, v0,
                     vs_valid, count, c0, C, tm, tn, dW);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dh_scatter(const float* dH_acc, int nsplit, int cpad, int64_t d,
                             const int32_t* idx, const int32_t* count, int64_t c0, int C, T* dH,
                             hipStream_t s) {
  ScopedKernelTimer timer_(KK_DH_SCATTER, s);
  hipLaunchKernelGGL(k_dh_scatter<T>, dim3(C), dim3(256), 0, s, dH_acc, nsplit, cpad, d, idx,
                     count, c0, C, dH);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  ScopedKernelTimer timer_(KK_ZERO, s);
  if (bytes == 0) return hipSuccess;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int ntail = (int)(bytes % 16);
  int blocks = (int)((n16 + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_zero, dim3(blocks), dim3(256), 0, s, (int4*)p, n16,
                     (char*)p + n16 * 16, ntail);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gemm_nt(const T* A, const T* B, int64_t M, int64_t N, int64_t K, float* C,
                          hipStream_t s) {
  ScopedKernelTimer timer_(KK_GEMM_NT, s);
  const int tm = cdiv(M, kBM), tn = cdiv(N, kBN);
  hipLaunchKernelGGL(k_gemm_nt<T>, dim3(xcd_grid(tm * tn)), dim3(kThreads), 0, s, A, B, M, N, K, tm, tn, C);
  return hipGetLastError();
}

#define GRPO_INSTANTIATE(T)                                                                       \
  template hipError_t launch_lse_partials<T>(const T*, const T*, const int32_t*, int64_t,         \
                                             int64_t, int, int, const LogitXform&, const float*,  \
                                             const float*, float*, float*, float*, hipStream_t);  \
  template hipError_t launch_transpose<T>(const T*, int64_t, int64_t, T*, int64_t, hipStream_t);  \
  template hipError_t launch_bwd_prep<T>(const T*, int64_t, const int32_t*, const int32_t*,       \
                                         int64_t, int, int, const int32_t*, const uint8_t*,        \
                                         const float*, const float*, const float*, const float*,  \
                                         int64_t, float, float, const LogitXform&,                \
                                         const LossVariant&, const int32_t*, int64_t, T*, float*,  \
                                         float*, int32_t*, float*, hipStream_t);                  \
  template hipError_t launch_dz<T>(const T*, const T*, int64_t, int64_t, int64_t, int, int,       \
                                   const int32_t*, int64_t, int, int, const LogitXform&,         \
                                   const float*, const float*, const float*, const float*,        \
                                   const int32_t*, const float*, T*, hipStream_t);                \
  template hipError_t launch_dh_gemm<T>(const T*, int64_t, int, const T*, int, int64_t,           \
                                        const int32_t*, int64_t, int, int, int, int, float*,      \
                                        hipStream_t);                                             \
  template hipError_t launch_dw_gemm<T>(const T*, int, const T*, int, int64_t, int64_t, int,      \
                                        const int32_t*, int64_t, int, float*, hipStream_t);       \
  template hipError_t launch_dh_scatter<T>(const float*, int, int, int64_t, const int32_t*,      \
                                           const int32_t*, int64_t, int, T*, hipStream_t);        \
  template hipError_t launch_gemm_nt<T>(const T*, const T*, int64_t, int64_t, int64_t, float*,    \
                                        hipStream_t);

GRPO_INSTANTIATE(float)
GRPO_INSTANTIATE(__bf16)
template hipError_t launch_dz<uint8_t>(const uint8_t*, const uint8_t*, int64_t, int64_t, int64_t,
                                         int, int, const int32_t*, int64_t, int, int,
                                         const LogitXform&, const float*, const float*,
                                         const float*, const float*, const int32_t*, const float*,
                                         __bf16*, hipStream_t);
template hipError_t launch_lse_partials<uint8_t>(const uint8_t*, const uint8_t*, const int32_t*,
                                                 int64_t, int64_t, int, int, const LogitXform&,
                                                 const float*, const float*, float*, float*,
                                                 float*, hipStream_t);


// ---------------------------------------------------------------- fp8 launchers
template <typename T>
hipError_t launch_fp8_quantize(const T* X, int64_t rows, int64_t cols, int per_row, float* part,
                               int nparts, int* e_tensor, uint8_t* codes, float* scales,
                               hipStream_t s) {
  ScopedKernelTimer timer_(KK_FP8_QUANT, s);
  if (!per_row) {
    hipLaunchKernelGGL(k_fp8_absmax_partial<T>, dim3(nparts), dim3(256), 0, s, X, rows * cols, part);
    hipLaunchKernelGGL(k_fp8_tensor_exponent, dim3(1), dim3(256), 0, s, part, nparts, e_tensor,
                       scales);
  }
  hipLaunchKernelGGL(k_fp8_quant_rows<T>, dim3((unsigned)rows), dim3(256), 0, s, X, cols,
                     per_row ? nullptr : e_tensor, codes, scales);
  return hipGetLastError();
}
template hipError_t launch_fp8_quantize<float>(const float*, int64_t, int64_t, int, float*, int,
                                               int*, uint8_t*, float*, hipStream_t);
template hipError_t launch_fp8_quantize<__bf16>(const __bf16*, int64_t, int64_t, int, float*, int,
                                                int*, uint8_t*, float*, hipStream_t);

hipError_t launch_fp8_dequantize(const uint8_t* codes, int64_t rows, int64_t cols,
                                 const float* scales, int per_row, __bf16* out, hipStream_t s) {
  ScopedKernelTimer timer_(KK_FP8_DEQUANT, s);
  hipLaunchKernelGGL(k_fp8_dequant_rows, dim3((unsigned)rows), dim3(256), 0, s, codes, cols,
                     scales, per_row, out);
  return hipGetLastError();
}

}  // namespace grpo
