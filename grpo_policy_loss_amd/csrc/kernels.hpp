// kernels.hpp -- host-side launchers of the HIP kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grpo {

// Tokens per block of the forward merge kernel (one loss partial per block).
constexpr int kMergeTokens = 16;

// Logit transform applied to every z = h . w before the log-softmax:
//   without a cap:  z' = k z                      (k = scale / temperature)
//   with a cap:     z' = b tanh(a z)              (a = scale / cap, b = cap / temperature)
// with scale = multiply / divide.  k, a, b > 0.  The identity is k = 1, no cap.
struct LogitXform {
  float k;
  float a;
  float b;
  int softcap;
};

// The loss variant: KL estimator, detach and aggregation.
struct LossVariant {
  int kl;         // 0 reverse k3, 1 forward r log r - (r - 1), 2 reverse k3 times q = exp(lp)
  int no_detach;  // 1: exp(lp - lp) in place of exp(lp - stopgrad(lp)): no advantage gradient
  int seq_mean;   // 1: per-sequence masked mean, then the mean over sequences
};

// Logical tile grid of one GEMM-shaped launch.
struct Grid2 {
  int tm;  // tiles along M (A rows)
  int tn;  // tiles along N (B rows)
};

hipError_t launch_advantages(const float* rewards, int64_t groups, int64_t G, float eps,
                             float* adv, hipStream_t s);

// Forward: per-(vocab tile, token) online-LSE partials and the target logit
// for the tokens [0, n_tok) of one chunk whose hidden states start at H.
template <typename T>
hipError_t launch_lse_partials(const T* W, const T* H, const int32_t* y, int64_t V, int64_t d,
                               int n_tok, int cpad, const LogitXform& xf, const float* w_scale,
                               const float* h_scale, float* part_m, float* part_s, float* zy,
                               hipStream_t s);

// fp8 e4m3 codes of X (rows x cols, cols a multiple of 4) with power-of-two
// scales, per row (scales[rows]) or for the tensor (scales[0]; part holds
// nparts partial maxima and e_tensor the exponent).
template <typename T>
hipError_t launch_fp8_quantize(const T* X, int64_t rows, int64_t cols, int per_row, float* part,
                               int nparts, int* e_tensor, uint8_t* codes, float* scales,
                               hipStream_t s);
// out (bf16, rows x cols) = codes * scale, exact.
hipError_t launch_fp8_dequantize(const uint8_t* codes, int64_t rows, int64_t cols,
                                 const float* scales, int per_row, __bf16* out, hipStream_t s);

// Merge the partials of one chunk (tokens c0 .. c0 + n_tok - 1).
// mode 0: reference log-probs -> out_lp.  mode 1: loss forward.
// seq_n (per-sequence unmasked counts) is null for the token mean.
hipError_t launch_lse_merge(int mode, const float* part_m, const float* part_s, const float* zy,
                            int S, int cpad, int n_tok, int64_t c0, const int32_t* y, int64_t V,
                            float* out_lp, float* out_lse, float* out_kl, const float* ref_lp,
                            const uint8_t* mask, const float* adv, int64_t L, float beta,
                            const LossVariant& lv, const int32_t* seq_n, double* loss_part,
                            int* cnt_part, int part0, hipStream_t s);

// seq_B: the number of sequences for the per-sequence mean, 0 for the token mean.
hipError_t launch_loss_final(const double* loss_part, const int* cnt_part, int nparts,
                             int64_t seq_B, float* loss, hipStream_t s);

// n[b] = unmasked tokens of sequence b (B sequences of L tokens).
hipError_t launch_seq_counts(const uint8_t* mask, int64_t B, int64_t L, int32_t* n, hipStream_t s);

// Backward helpers.
hipError_t launch_active_scan(const uint8_t* mask, int64_t N, int32_t* idx, int32_t* count,
                              hipStream_t s);

template <typename T>
hipError_t launch_transpose(const T* in, int64_t R, int64_t Cc, T* out, int64_t Rpad,
                            hipStream_t s);

template <typename T>
hipError_t launch_bwd_prep(const T* H, int64_t d, const int32_t* idx, const int32_t* count,
                           int64_t c0, int C, int cpad, const int32_t* y, const uint8_t* mask,
                           const float* adv, const float* ref_lp, const float* lp,
                           const float* lse, int64_t L, float beta, float grad_loss,
                           const LogitXform& xf, const LossVariant& lv, const int32_t* seq_n,
                           int64_t B, T* H_act, float* coef, float* lse_c, int32_t* y_c,
                           float* tgt_c, hipStream_t s);

// Element type of the dZ slabs: bfloat16 for fp8 operands, the operand type otherwise.
template <typename T> struct DzOut { typedef T type; };
template <> struct DzOut<uint8_t> { typedef __bf16 type; };

// dZ: the slab, vs / 256 strips of [cpad][256].  T = uint8_t: fp8 operands (w_scale,
// hs_act as in k_lse_partials), bf16 dZ; other T: both scale pointers unused (null).
template <typename T>
hipError_t launch_dz(const T* W, const T* H_act, int64_t d, int64_t V, int64_t v0, int vs_valid,
                     int vs, const int32_t* count, int64_t c0, int C, int cpad,
                     const LogitXform& xf, const float* w_scale, const float* hs_act,
                     const float* coef, const float* lse_c, const int32_t* y_c,
                     const float* tgt_c, typename DzOut<T>::type* dZ, hipStream_t s);

// The fp8 codes and scales of chunk c's active tokens, for the fp8 recompute.
hipError_t launch_fp8_gather_rows(const uint8_t* H8, const float* h_scale, int64_t d,
                                  const int32_t* idx, const int32_t* count, int64_t c0, int C,
                                  int cpad, uint8_t* H8_act, float* hs_act, hipStream_t s);

// dH_acc holds nsplit partial buffers of [cpad, d] floats; split sp covers
// one contiguous share of the slab's vocabulary columns.  W is the caller's
// [V, d] head (read K-major); vs_valid * d * sizeof(T) must be < 2^31.
template <typename T>
hipError_t launch_dh_gemm(const T* W, int64_t v0, int vs_valid, const T* dZ, int vs, int64_t d,
                          const int32_t* count, int64_t c0, int C, int cpad, int nsplit, int first,
                          float* dH_acc, hipStream_t s);

// dZ is the slab of strips [vs / 256][cpad][256] (each strip read K-major);
// C * vs * sizeof(T) must be < 2^31.
template <typename T>
hipError_t launch_dw_gemm(const T* HT, int cpad, const T* dZ, int vs, int64_t d, int64_t v0,
                          int vs_valid, const int32_t* count, int64_t c0, int C, float* dW,
                          hipStream_t s);

template <typename T>
hipError_t launch_dh_scatter(const float* dH_acc, int nsplit, int cpad, int64_t d,
                             const int32_t* idx, const int32_t* count, int64_t c0, int C, T* dH,
                             hipStream_t s);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// Plain tile GEMM C[m][n] = sum_k A[m][k] B[n][k] into float32 C (diagnostic).
template <typename T>
hipError_t launch_gemm_nt(const T* A, const T* B, int64_t M, int64_t N, int64_t K, float* C,
                          hipStream_t s);

}  // namespace grpo
