// grpo_api.hip -- the C ABI (include/grpo.h): argument checks, workspace
// planning and the launch sequence of each call.  No allocation, no host
// synchronisation: every call enqueues on the caller's stream and returns.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/grpo.h"
#include "kernels.hpp"
#include "tile_mma.hpp"
#include "timing.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(GRPO_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

inline size_t esize(int dtype) { return dtype == GRPO_F32 ? 4 : dtype == GRPO_FP8_E4M3 ? 1 : 2; }

// Bump allocator over the caller's workspace.
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

// Forward / reference workspace: per-(vocab tile, token) partial pairs of
// one chunk, the chunk's target logits, and the per-block loss sums.
struct FwdPlan {
  int64_t C, cpad, S, nchunks, parts_per_chunk;
  size_t o_pm, o_ps, o_zy, o_lpart, o_cpart, o_seq, total;
};

FwdPlan plan_fwd(int64_t N, int64_t V, int64_t chunk) {
  FwdPlan p{};
  p.C = std::min<int64_t>(chunk, N);
  p.cpad = round_up(p.C, grpo::kBN);
  p.S = (V + grpo::kBM - 1) / grpo::kBM;
  p.nchunks = (N + p.C - 1) / p.C;
  p.parts_per_chunk = (p.C + grpo::kMergeTokens - 1) / grpo::kMergeTokens;  // merge blocks per chunk
  Carve c;
  p.o_pm = c.take((size_t)(p.S * p.cpad) * 4);
  p.o_ps = c.take((size_t)(p.S * p.cpad) * 4);
  p.o_zy = c.take((size_t)p.cpad * 4);
  p.o_lpart = c.take((size_t)(p.nchunks * p.parts_per_chunk) * 8);
  p.o_cpart = c.take((size_t)(p.nchunks * p.parts_per_chunk) * 4);
  p.o_seq = c.take((size_t)N * 4);   // per-sequence counts: B <= N sequences
  p.total = c.off;
  return p;
}

// Backward workspace: the fixed part (active-token index list, one chunk of
// gathered hidden states and its transpose, the chunk's per-token coefficient /
// lse / target id / target dZ entry, nsplit float32 dH partials of the chunk,
// per-sequence counts), then one dZ slab: the bf16 (or f32) gradient of `vs`
// vocabulary columns of the chunk's logits, stored once as vs / 256 strips of
// [cpad tokens][256 columns].
//
// The slab width comes from the workspace the caller passes: the widest
// multiple of 256 vocabulary columns (at most the padded vocabulary) that fits
// after the fixed part, then, among widths down to half of that, the one with
// the fewest modelled GEMM waves.  grpo_workspace_bytes(GRPO_OP_BWD) sizes the
// workspace for a slab of at most kSlabBytesDefault; GRPO_OP_BWD_MIN for one
// 256-column slab.  Narrow slabs mean more read-modify-write passes over the dH
// partials: at the Qwen2.5-1.5B LM-head shape one whole-vocabulary slab
// (1.16 GiB) ran the backward 2 % faster than two, and 512 MiB slabs 6 %
// slower.  Past that the width stops mattering: at Llama-3.1-8B and gpt-oss-20b
// with 8192-token chunks, 1.25 GiB slabs ran within 0.5 % of 2 GiB ones (one
// and two slabs per chunk) and keep 0.8 GB less workspace.  Two hardware
// bounds cap the width: the dW GEMM reads the slab K-major through one buffer
// resource (cpad x vs elements) and the dH GEMM reads W the same way
// (vs x d elements), and a resource spans less than 2^31 bytes.
constexpr int64_t kSlabBytesDefault = 1280ll << 20;
constexpr int64_t kCUs = 256;  // MI355X compute units (one GEMM workgroup each: 160 KB LDS, 4 full-register waves)

struct BwdPlan {
  bool ok;
  int64_t C, cpad, vpad, vs, nslabs, nchunks, nsplit;
  size_t o_idx, o_cnt, o_hact, o_ht, o_coef, o_lse, o_y, o_tgt, o_dhacc, o_seq, o_dz, fixed, total;
};

// ws_bytes: the caller's workspace size; 0 plans the default slab budget and
// -1 the narrowest slab (the minimum workspace).
BwdPlan plan_bwd(int64_t N, int64_t d, int64_t V, int dtype, int64_t chunk, int64_t ws_bytes) {
  BwdPlan p{};
  const int64_t es = (int64_t)esize(dtype);
  p.C = std::min<int64_t>(chunk, N);
  p.cpad = round_up(p.C, grpo::kBN);
  p.vpad = round_up(V, grpo::kBM);
  p.nchunks = (N + p.C - 1) / p.C;
  // Split the dH GEMM's vocabulary range when its tile grid alone cannot fill the
  // chip: pick the split count (1..8) whose launch wastes the least of its last
  // wave of workgroups (one GEMM workgroup per CU), preferring fewer splits.
  const int64_t ct = p.cpad / 256, dt = (d + 255) / 256;
  const int64_t dh_tiles = dt * ct;
  int64_t nsplit_grid = 1;
  if (dh_tiles < 2 * kCUs) {
    double best = -1.0;
    for (int64_t n = 1; n <= 8; ++n) {
      const int64_t wg = dh_tiles * n;
      const double fill = (double)wg / (double)(((wg + kCUs - 1) / kCUs) * kCUs);
      const double score = fill * std::min(1.0, (double)wg / (2.0 * kCUs));
      if (score > best + 1e-9) {
        best = score;
        nsplit_grid = n;
      }
    }
  }
  Carve c;
  p.o_idx = c.take((size_t)N * 4);
  p.o_cnt = c.take(4);
  p.o_hact = c.take((size_t)(p.cpad * d) * es);
  p.o_ht = c.take((size_t)(d * p.cpad) * es);
  p.o_coef = c.take((size_t)p.cpad * 4);
  p.o_lse = c.take((size_t)p.cpad * 4);
  p.o_y = c.take((size_t)p.cpad * 4);
  p.o_tgt = c.take((size_t)p.cpad * 4);
  p.o_dhacc = c.take((size_t)(nsplit_grid * p.cpad * d) * 4);
  p.o_seq = c.take((size_t)N * 4);   // per-sequence counts: B <= N sequences
  p.o_dz = c.off;
  p.fixed = c.off;

  const int64_t col_bytes = p.cpad * es;            // one vocabulary column of the slab
  const int64_t lim = ((1ll << 31) - 1) / (std::max(p.cpad, d) * es) / 256 * 256;
  int64_t vs_max;
  if (ws_bytes == 0)
    vs_max = kSlabBytesDefault / col_bytes / 256 * 256;
  else if (ws_bytes < 0)
    vs_max = 256;
  else
    vs_max = ws_bytes > (int64_t)p.fixed ? (ws_bytes - (int64_t)p.fixed) / col_bytes / 256 * 256 : 0;
  vs_max = std::min(std::min(vs_max, p.vpad), lim);
  p.ok = vs_max >= 256;
  if (!p.ok) vs_max = 256;
  p.nsplit = std::min<int64_t>(nsplit_grid, vs_max / 256);
  // Slab width: every launch runs in whole waves of kCUs workgroups, so model a
  // chunk's backward as sum over slabs of waves(launch) x K-length(launch) for the
  // dz (K = d), dW (K = chunk) and dH (K = slab / nsplit) GEMMs, and take the
  // cheapest multiple of 256 down to half the widest.
  auto waves = [](int64_t wg) { return (wg + kCUs - 1) / kCUs; };
  double best_cost = 0.0;
  p.vs = vs_max;
  for (int64_t vs = vs_max; vs >= std::max<int64_t>(256, vs_max / 2); vs -= 256) {
    const int64_t ns = (V + vs - 1) / vs;
    double cost = 0.0;
    for (int64_t sl = 0; sl < ns; ++sl) {
      const int64_t w = std::min<int64_t>(vs, V - sl * vs);
      const int64_t vt = (w + 255) / 256;
      cost += (double)waves(vt * ct) * (double)d;
      cost += (double)waves(dt * vt) * (double)p.cpad;
      cost += (double)waves(dh_tiles * p.nsplit) * (double)w / (double)p.nsplit;
    }
    if (vs == vs_max || cost < best_cost * (1.0 - 1e-6)) {
      best_cost = cost;
      p.vs = vs;
    }
  }
  p.nslabs = (V + p.vs - 1) / p.vs;
  p.total = align_up(p.fixed + (size_t)(p.cpad * p.vs * es));
  return p;
}

// Shape checks shared by all calls.  Operands are addressed per 256-row tile
// with 32-bit offsets, so one tile's rows must span < 2 GiB.
// fp8_ok: GRPO_FP8_E4M3 is accepted (the fp8 calls and the size queries)
int check_shape(int64_t N, int64_t d, int64_t V, int dtype, int64_t chunk, bool fp8_ok = false) {
  if (N <= 0 || d <= 0 || V <= 0 || chunk <= 0)
    return fail(GRPO_ERR_INVALID_ARG, "sizes must be positive (N=%lld d=%lld V=%lld chunk=%lld)",
                (long long)N, (long long)d, (long long)V, (long long)chunk);
  if (dtype != GRPO_F32 && dtype != GRPO_BF16 && !(fp8_ok && dtype == GRPO_FP8_E4M3))
    return fail(GRPO_ERR_INVALID_ARG, "dtype %d is not accepted here", dtype);
  const int64_t vec = 16 / (int64_t)esize(dtype);
  if (d % vec != 0)
    return fail(GRPO_ERR_UNSUPPORTED, "d=%lld must be a multiple of %lld for this dtype",
                (long long)d, (long long)vec);
  if (N > INT32_MAX || V > INT32_MAX || d > INT32_MAX || chunk > (1 << 24))
    return fail(GRPO_ERR_UNSUPPORTED, "N, V, d must fit int32 and chunk <= 2^24");
  // every factor is below 2^31 here, so the product cannot overflow
  const int64_t cpad = round_up(std::min(chunk, N), grpo::kBN);
  const int64_t row_span = 256 * std::max<int64_t>(std::max(d, round_up(V, 256)), cpad) * 4;
  if (row_span >= (1ll << 31))
    return fail(GRPO_ERR_UNSUPPORTED, "a 256-row tile would span >= 2 GiB (d=%lld V=%lld)",
                (long long)d, (long long)V);
  return GRPO_OK;
}

#define GRPO_CHECK_PTR(p)                                                          \
  do {                                                                             \
    if ((p) == nullptr) return fail(GRPO_ERR_INVALID_ARG, "null pointer: %s", #p); \
  } while (0)

#define GRPO_HIP(call)                                    \
  do {                                                    \
    hipError_t e_ = (call);                               \
    if (e_ != hipSuccess) return hip_fail(e_, #call);     \
  } while (0)

// The kernels' form of the logit transform of a grpo_opts (NULL: identity).
int make_xform(const grpo_opts* o, grpo::LogitXform* xf) {
  *xf = grpo::LogitXform{1.f, 1.f, 1.f, 0};
  if (o == nullptr) return GRPO_OK;
  const float v[4] = {o->logit_scale_multiply, o->logit_scale_divide, o->logit_softcapping,
                      o->temperature};
  for (float x : v)
    if (!isfinite(x) || x < 0.f)
      return fail(GRPO_ERR_INVALID_ARG,
                  "logit opts must be finite and >= 0 (multiply %g divide %g cap %g T %g)",
                  (double)v[0], (double)v[1], (double)v[2], (double)v[3]);
  const double scale = (v[0] != 0.f ? (double)v[0] : 1.0) / (v[1] != 0.f ? (double)v[1] : 1.0);
  const double T = v[3] != 0.f ? (double)v[3] : 1.0;
  xf->k = (float)(scale / T);
  if (v[2] != 0.f) {
    xf->softcap = 1;
    xf->a = (float)(scale / (double)v[2]);
    xf->b = (float)((double)v[2] / T);
  }
  if (!isfinite(xf->k) || xf->k <= 0.f || !isfinite(xf->a) || xf->a <= 0.f ||
      !isfinite(xf->b) || xf->b <= 0.f)
    return fail(GRPO_ERR_INVALID_ARG, "logit opts give a degenerate scale");
  return GRPO_OK;
}

// The kernels' form of the loss variant of a grpo_opts (NULL: the default loss).
int make_variant(const grpo_opts* o, grpo::LossVariant* lv) {
  *lv = grpo::LossVariant{0, 0, 0};
  if (o == nullptr) return GRPO_OK;
  if (o->kl_estimator < GRPO_KL_REVERSE || o->kl_estimator > GRPO_KL_REVERSE_Q)
    return fail(GRPO_ERR_INVALID_ARG, "kl_estimator %d is not 0, 1 or 2", (int)o->kl_estimator);
  if (o->no_detach != 0 && o->no_detach != 1)
    return fail(GRPO_ERR_INVALID_ARG, "no_detach %d is not 0 or 1", (int)o->no_detach);
  if (o->aggregation != GRPO_AGG_TOKEN_MEAN && o->aggregation != GRPO_AGG_SEQUENCE_MEAN)
    return fail(GRPO_ERR_INVALID_ARG, "aggregation %d is not 0 or 1", (int)o->aggregation);
  *lv = grpo::LossVariant{(int)o->kl_estimator, (int)o->no_detach,
                          o->aggregation == GRPO_AGG_SEQUENCE_MEAN ? 1 : 0};
  return GRPO_OK;
}

template <typename T>
int lse_pass(int mode, const T* H, const T* W, const int32_t* y, const uint8_t* mask,
             const float* adv, const float* ref_lp, int64_t N, int64_t L, int64_t d, int64_t V,
             float beta, int64_t chunk, const grpo::LogitXform& xf, const grpo::LossVariant& lv,
             float* loss, float* out_lp, float* out_kl, float* out_lse, char* ws, hipStream_t s,
             const float* w_scale = nullptr, const float* h_scale = nullptr) {
  const FwdPlan p = plan_fwd(N, V, chunk);
  float* pm = (float*)(ws + p.o_pm);
  float* ps = (float*)(ws + p.o_ps);
  float* zy = (float*)(ws + p.o_zy);
  double* lpart = (double*)(ws + p.o_lpart);
  int* cpart = (int*)(ws + p.o_cpart);
  const bool seq_mean = mode == 1 && lv.seq_mean;
  int32_t* seq_n = seq_mean ? (int32_t*)(ws + p.o_seq) : nullptr;
  if (seq_mean) GRPO_HIP(grpo::launch_seq_counts(mask, N / L, L, seq_n, s));
  for (int64_t c = 0; c < p.nchunks; ++c) {
    const int64_t c0 = c * p.C;
    const int n_tok = (int)std::min<int64_t>(p.C, N - c0);
    GRPO_HIP(grpo::launch_lse_partials<T>(W, H + c0 * d, y + c0, V, d, n_tok, (int)p.cpad, xf,
                                          w_scale, h_scale ? h_scale + c0 : nullptr, pm, ps, zy,
                                          s));
    GRPO_HIP(grpo::launch_lse_merge(mode, pm, ps, zy, (int)p.S, (int)p.cpad, n_tok, c0, y, V,
                                    out_lp, out_lse, out_kl, ref_lp, mask, adv, L, beta, lv, seq_n,
                                    lpart, cpart, (int)(c * p.parts_per_chunk), s));
  }
  if (mode == 1) {
    // every full chunk writes all of its slots; a short last chunk
    // writes only its first blocks, and the final sum reads exactly those
    const int64_t last_c0 = (p.nchunks - 1) * p.C;
    const int64_t last_blocks =
        (std::min<int64_t>(p.C, N - last_c0) + grpo::kMergeTokens - 1) / grpo::kMergeTokens;
    const int64_t nparts = (p.nchunks - 1) * p.parts_per_chunk + last_blocks;
    GRPO_HIP(grpo::launch_loss_final(lpart, cpart, (int)nparts, seq_mean ? N / L : 0, loss, s));
  }
  return GRPO_OK;
}

// fp8 operands of the backward's logit recompute (all null on the bf16 / f32 path):
// the codes and scales of H and W, and room for one chunk of gathered active rows.
struct Fp8Recompute {
  const uint8_t* H8 = nullptr;
  const float* h_scale = nullptr;
  const uint8_t* W8 = nullptr;
  const float* w_scale = nullptr;
  uint8_t* H8_act = nullptr;
  float* hs_act = nullptr;
};

template <typename T>
int bwd_pass(const T* H, const T* W, const int32_t* y, const uint8_t* mask, const float* adv,
             const float* ref_lp, const float* lp, const float* lse, int64_t N, int64_t L,
             int64_t d, int64_t V, float beta, float grad_loss, int64_t chunk,
             const grpo::LogitXform& xf, const grpo::LossVariant& lv, T* dH, float* dW,
             const BwdPlan& p, char* ws, hipStream_t s, const Fp8Recompute& f8 = Fp8Recompute()) {
  int32_t* idx = (int32_t*)(ws + p.o_idx);
  int32_t* cnt = (int32_t*)(ws + p.o_cnt);
  T* H_act = (T*)(ws + p.o_hact);
  T* HT = (T*)(ws + p.o_ht);
  float* coef = (float*)(ws + p.o_coef);
  float* lse_c = (float*)(ws + p.o_lse);
  int32_t* y_c = (int32_t*)(ws + p.o_y);
  float* tgt_c = (float*)(ws + p.o_tgt);
  T* dZ = (T*)(ws + p.o_dz);
  float* dH_acc = (float*)(ws + p.o_dhacc);
  int32_t* seq_n = lv.seq_mean ? (int32_t*)(ws + p.o_seq) : nullptr;
  const int64_t B = N / L;

  GRPO_HIP(grpo::launch_zero(dH, (size_t)(N * d) * sizeof(T), s));
  GRPO_HIP(grpo::launch_active_scan(mask, N, idx, cnt, s));
  if (seq_n != nullptr) GRPO_HIP(grpo::launch_seq_counts(mask, B, L, seq_n, s));
  // Chunks are planned for the worst case (every token active); chunks past
  // the device-side active count exit at once, so no host sync is needed.
  for (int64_t c = 0; c < p.nchunks; ++c) {
    const int64_t c0 = c * p.C;
    const int C = (int)p.C;
    GRPO_HIP(grpo::launch_bwd_prep<T>(H, d, idx, cnt, c0, C, (int)p.cpad, y, mask, adv, ref_lp, lp,
                                      lse, L, beta, grad_loss, xf, lv, seq_n, B, H_act, coef,
                                      lse_c, y_c, tgt_c, s));
    GRPO_HIP(grpo::launch_transpose<T>(H_act, p.cpad, d, HT, p.cpad, s));
    if (f8.H8 != nullptr)
      GRPO_HIP(grpo::launch_fp8_gather_rows(f8.H8, f8.h_scale, d, idx, cnt, c0, C, (int)p.cpad,
                                            f8.H8_act, f8.hs_act, s));
    for (int64_t sl = 0; sl < p.nslabs; ++sl) {
      const int64_t v0 = sl * p.vs;
      const int vs_valid = (int)std::min<int64_t>(p.vs, V - v0);
      if (f8.W8 != nullptr)
        GRPO_HIP(grpo::launch_dz<uint8_t>(f8.W8, f8.H8_act, d, V, v0, vs_valid, (int)p.vs, cnt,
                                          c0, C, (int)p.cpad, xf, f8.w_scale, f8.hs_act, coef,
                                          lse_c, y_c, tgt_c, (__bf16*)dZ, s));
      else
        GRPO_HIP(grpo::launch_dz<T>(W, H_act, d, V, v0, vs_valid, (int)p.vs, cnt, c0, C,
                                    (int)p.cpad, xf, nullptr, nullptr, coef, lse_c, y_c, tgt_c,
                                    dZ, s));
      GRPO_HIP(grpo::launch_dh_gemm<T>(W, v0, vs_valid, dZ, (int)p.vs, d, cnt, c0, C, (int)p.cpad,
                                       (int)p.nsplit, sl == 0 ? 1 : 0, dH_acc, s));
      GRPO_HIP(grpo::launch_dw_gemm<T>(HT, (int)p.cpad, dZ, (int)p.vs, d, v0, vs_valid, cnt, c0,
                                       C, dW, s));
    }
    GRPO_HIP(grpo::launch_dh_scatter<T>(dH_acc, (int)p.nsplit, (int)p.cpad, d, idx, cnt, c0, C, dH,
                                        s));
  }
  return GRPO_OK;
}

}  // namespace

extern "C" {

const char* grpo_strerror(int code) {
  switch (code) {
    case GRPO_OK: return "success";
    case GRPO_ERR_INVALID_ARG: return "invalid argument";
    case GRPO_ERR_WORKSPACE: return "workspace missing or too small";
    case GRPO_ERR_UNSUPPORTED: return "unsupported shape";
    case GRPO_ERR_HIP: return "HIP runtime error";
    default: return "unknown grpo status";
  }
}

const char* grpo_last_error(void) { return g_last_error; }

// The fp8 backward runs the bf16 backward on exact bf16 copies of H and W,
// which come first in its workspace; the bf16 plan (with its slab) follows.
struct Fp8BwdPlan {
  size_t o_h, o_w, o_h8act, o_hsact, o_bf16;
  BwdPlan b;
  size_t total;
};
// ws_bytes as for plan_bwd.
Fp8BwdPlan plan_bwd_fp8(int64_t N, int64_t d, int64_t V, int64_t chunk, int64_t ws_bytes) {
  Fp8BwdPlan p{};
  const int64_t cpad = round_up(std::min<int64_t>(chunk, N), grpo::kBN);
  Carve c;
  p.o_h = c.take((size_t)(N * d) * 2);
  p.o_w = c.take((size_t)(V * d) * 2);
  p.o_h8act = c.take((size_t)(cpad * d));      // one chunk of active fp8 rows
  p.o_hsact = c.take((size_t)cpad * 4);
  p.o_bf16 = c.off;
  int64_t rest = ws_bytes;
  if (ws_bytes > 0) rest = ws_bytes > (int64_t)p.o_bf16 ? ws_bytes - (int64_t)p.o_bf16 : 1;
  p.b = plan_bwd(N, d, V, GRPO_BF16, chunk, rest);
  p.total = p.o_bf16 + p.b.total;
  return p;
}

size_t grpo_workspace_bytes(int op, int64_t N, int64_t d, int64_t V, int dtype, int64_t chunk) {
  if (check_shape(N, d, V, dtype, chunk, true) != GRPO_OK) return 0;
  switch (op) {
    case GRPO_OP_REF:
    case GRPO_OP_FWD: return plan_fwd(N, V, chunk).total;
    case GRPO_OP_BWD:
    case GRPO_OP_BWD_MIN: {
      const int64_t how = op == GRPO_OP_BWD ? 0 : -1;
      return dtype == GRPO_FP8_E4M3 ? plan_bwd_fp8(N, d, V, chunk, how).total
                                    : plan_bwd(N, d, V, dtype, chunk, how).total;
    }
    default: fail(GRPO_ERR_INVALID_ARG, "unknown op %d", op); return 0;
  }
}

int64_t grpo_auto_chunk(int64_t B, int64_t L, int64_t d, int64_t V, int dtype,
                        size_t budget_bytes) {
  g_last_error[0] = 0;
  if (B <= 0 || L <= 0) {
    fail(GRPO_ERR_INVALID_ARG, "B and L must be positive");
    return 0;
  }
  if (B > INT32_MAX / L) {
    fail(GRPO_ERR_UNSUPPORTED, "B*L exceeds int32");
    return 0;
  }
  const int64_t N = B * L;
  if (check_shape(N, d, V, dtype, 1, true) != GRPO_OK) return 0;
  constexpr int64_t kStep = 256, kCap = 8192;  // best measured chunk at d = 1536 and 4096
  const int64_t top = std::min<int64_t>(kCap, round_up(N, kStep));
  for (int64_t c = top; c > kStep; c -= kStep)
    if (grpo_workspace_bytes(GRPO_OP_FWD, N, d, V, dtype, c) +
            grpo_workspace_bytes(GRPO_OP_BWD, N, d, V, dtype, c) <= budget_bytes)
      return c;
  return kStep;
}

int grpo_advantages(const float* rewards, int64_t num_groups, int64_t group_size, float eps,
                    float* adv, void* stream) {
  g_last_error[0] = 0;
  GRPO_CHECK_PTR(rewards);
  GRPO_CHECK_PTR(adv);
  if (num_groups <= 0 || group_size <= 0)
    return fail(GRPO_ERR_INVALID_ARG, "num_groups and group_size must be positive");
  if (num_groups > INT32_MAX) return fail(GRPO_ERR_UNSUPPORTED, "num_groups exceeds int32");
  if (!isfinite(eps) || eps < 0.f) return fail(GRPO_ERR_INVALID_ARG, "eps must be finite, >= 0");
  GRPO_HIP(grpo::launch_advantages(rewards, num_groups, group_size, eps, adv,
                                   (hipStream_t)stream));
  return GRPO_OK;
}

int grpo_ref_logprobs_ex(const void* H_ref, const void* W, const int32_t* y, int64_t N, int64_t d,
                         int64_t V, int dtype, int64_t chunk, const grpo_opts* opts,
                         float* ref_lp, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  grpo::LogitXform xf;
  grpo::LossVariant lv;
  if (make_xform(opts, &xf) != GRPO_OK || make_variant(opts, &lv) != GRPO_OK)
    return GRPO_ERR_INVALID_ARG;
  GRPO_CHECK_PTR(H_ref);
  GRPO_CHECK_PTR(W);
  GRPO_CHECK_PTR(y);
  GRPO_CHECK_PTR(ref_lp);
  int st = check_shape(N, d, V, dtype, chunk);
  if (st != GRPO_OK) return st;
  const size_t need = plan_fwd(N, V, chunk).total;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GRPO_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == GRPO_BF16)
    return lse_pass<__bf16>(0, (const __bf16*)H_ref, (const __bf16*)W, y, nullptr, nullptr,
                            nullptr, N, 1, d, V, 0.f, chunk, xf, lv, nullptr, ref_lp, nullptr,
                            nullptr, (char*)workspace, s);
  return lse_pass<float>(0, (const float*)H_ref, (const float*)W, y, nullptr, nullptr, nullptr, N,
                         1, d, V, 0.f, chunk, xf, lv, nullptr, ref_lp, nullptr, nullptr,
                         (char*)workspace, s);
}

int grpo_ref_logprobs(const void* H_ref, const void* W, const int32_t* y, int64_t N, int64_t d,
                      int64_t V, int dtype, int64_t chunk, float* ref_lp, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return grpo_ref_logprobs_ex(H_ref, W, y, N, d, V, dtype, chunk, nullptr, ref_lp, workspace,
                              workspace_bytes, stream);
}

int grpo_loss_fwd_ex(const void* H, const void* W, const int32_t* y, const uint8_t* mask,
                     const float* adv, const float* ref_lp, int64_t B, int64_t L, int64_t d,
                     int64_t V, int dtype, float beta, int64_t chunk, const grpo_opts* opts,
                     float* loss, float* lp, float* kl, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  grpo::LogitXform xf;
  grpo::LossVariant lv;
  if (make_xform(opts, &xf) != GRPO_OK || make_variant(opts, &lv) != GRPO_OK)
    return GRPO_ERR_INVALID_ARG;
  GRPO_CHECK_PTR(H);
  GRPO_CHECK_PTR(W);
  GRPO_CHECK_PTR(y);
  GRPO_CHECK_PTR(mask);
  GRPO_CHECK_PTR(adv);
  GRPO_CHECK_PTR(ref_lp);
  GRPO_CHECK_PTR(loss);
  GRPO_CHECK_PTR(lp);
  GRPO_CHECK_PTR(kl);
  GRPO_CHECK_PTR(lse);
  if (B <= 0 || L <= 0) return fail(GRPO_ERR_INVALID_ARG, "B and L must be positive");
  if (B > INT32_MAX / L) return fail(GRPO_ERR_UNSUPPORTED, "B*L exceeds int32");
  const int64_t N = B * L;
  int st = check_shape(N, d, V, dtype, chunk);
  if (st != GRPO_OK) return st;
  if (!isfinite(beta)) return fail(GRPO_ERR_INVALID_ARG, "beta must be finite");
  const size_t need = plan_fwd(N, V, chunk).total;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GRPO_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == GRPO_BF16)
    return lse_pass<__bf16>(1, (const __bf16*)H, (const __bf16*)W, y, mask, adv, ref_lp, N, L, d,
                            V, beta, chunk, xf, lv, loss, lp, kl, lse, (char*)workspace, s);
  return lse_pass<float>(1, (const float*)H, (const float*)W, y, mask, adv, ref_lp, N, L, d, V,
                         beta, chunk, xf, lv, loss, lp, kl, lse, (char*)workspace, s);
}

int grpo_loss_fwd(const void* H, const void* W, const int32_t* y, const uint8_t* mask,
                  const float* adv, const float* ref_lp, int64_t B, int64_t L, int64_t d,
                  int64_t V, int dtype, float beta, int64_t chunk, float* loss, float* lp,
                  float* kl, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return grpo_loss_fwd_ex(H, W, y, mask, adv, ref_lp, B, L, d, V, dtype, beta, chunk, nullptr,
                          loss, lp, kl, lse, workspace, workspace_bytes, stream);
}

int grpo_loss_bwd_ex(const void* H, const void* W, const int32_t* y, const uint8_t* mask,
                     const float* adv, const float* ref_lp, const float* lp, const float* lse,
                     int64_t B, int64_t L, int64_t d, int64_t V, int dtype, float beta,
                     float grad_loss, int64_t chunk, const grpo_opts* opts, void* dH,
                     float* dW, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  grpo::LogitXform xf;
  grpo::LossVariant lv;
  if (make_xform(opts, &xf) != GRPO_OK || make_variant(opts, &lv) != GRPO_OK)
    return GRPO_ERR_INVALID_ARG;
  GRPO_CHECK_PTR(H);
  GRPO_CHECK_PTR(W);
  GRPO_CHECK_PTR(y);
  GRPO_CHECK_PTR(mask);
  GRPO_CHECK_PTR(adv);
  GRPO_CHECK_PTR(ref_lp);
  GRPO_CHECK_PTR(lp);
  GRPO_CHECK_PTR(lse);
  GRPO_CHECK_PTR(dH);
  GRPO_CHECK_PTR(dW);
  if (B <= 0 || L <= 0) return fail(GRPO_ERR_INVALID_ARG, "B and L must be positive");
  if (B > INT32_MAX / L) return fail(GRPO_ERR_UNSUPPORTED, "B*L exceeds int32");
  const int64_t N = B * L;
  int st = check_shape(N, d, V, dtype, chunk);
  if (st != GRPO_OK) return st;
  if (!isfinite(beta)) return fail(GRPO_ERR_INVALID_ARG, "beta must be finite");
  if (!isfinite(grad_loss)) return fail(GRPO_ERR_INVALID_ARG, "grad_loss must be finite");
  // a caller's size is always a size (>= 1 here): 0 and -1 select the default and
  // minimum plans only in the workspace queries
  const int64_t wsb = std::max<int64_t>(1, (int64_t)std::min<size_t>(workspace_bytes, (size_t)INT64_MAX));
  const BwdPlan p = plan_bwd(N, d, V, dtype, chunk, workspace == nullptr ? 1 : wsb);
  if (workspace == nullptr || !p.ok)
    return fail(GRPO_ERR_WORKSPACE, "workspace needs at least %zu bytes, got %zu",
                plan_bwd(N, d, V, dtype, chunk, -1).total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == GRPO_BF16)
    return bwd_pass<__bf16>((const __bf16*)H, (const __bf16*)W, y, mask, adv, ref_lp, lp, lse, N,
                            L, d, V, beta, grad_loss, chunk, xf, lv, (__bf16*)dH, dW, p,
                            (char*)workspace, s);
  return bwd_pass<float>((const float*)H, (const float*)W, y, mask, adv, ref_lp, lp, lse, N, L, d,
                         V, beta, grad_loss, chunk, xf, lv, (float*)dH, dW, p, (char*)workspace,
                         s);
}

int grpo_loss_bwd(const void* H, const void* W, const int32_t* y, const uint8_t* mask,
                  const float* adv, const float* ref_lp, const float* lp, const float* lse,
                  int64_t B, int64_t L, int64_t d, int64_t V, int dtype, float beta,
                  float grad_loss, int64_t chunk, void* dH, float* dW, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return grpo_loss_bwd_ex(H, W, y, mask, adv, ref_lp, lp, lse, B, L, d, V, dtype, beta,
                          grad_loss, chunk, nullptr, dH, dW, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- fp8 e4m3 path
namespace {
constexpr int kQuantParts = 1024;   // partial maxima of a per-tensor scale
}

size_t grpo_quantize_fp8_workspace_bytes(void) { return kQuantParts * 4 + 256; }

int grpo_quantize_fp8(const void* X, int dtype, int64_t rows, int64_t cols, int per_row,
                      uint8_t* codes, float* scales, void* workspace, size_t workspace_bytes,
                      void* stream) {
  g_last_error[0] = 0;
  GRPO_CHECK_PTR(X);
  GRPO_CHECK_PTR(codes);
  GRPO_CHECK_PTR(scales);
  if (dtype != GRPO_F32 && dtype != GRPO_BF16)
    return fail(GRPO_ERR_INVALID_ARG, "quantize takes GRPO_F32 or GRPO_BF16 input, not %d", dtype);
  if (rows <= 0 || cols <= 0) return fail(GRPO_ERR_INVALID_ARG, "rows and cols must be positive");
  if (per_row != 0 && per_row != 1) return fail(GRPO_ERR_INVALID_ARG, "per_row must be 0 or 1");
  if (cols % 16 != 0) return fail(GRPO_ERR_UNSUPPORTED, "cols=%lld must be a multiple of 16",
                                  (long long)cols);
  if (rows > INT32_MAX) return fail(GRPO_ERR_UNSUPPORTED, "rows must fit int32");
  if (!per_row && (workspace == nullptr || workspace_bytes < grpo_quantize_fp8_workspace_bytes()))
    return fail(GRPO_ERR_WORKSPACE, "a per-tensor scale needs %zu bytes of workspace",
                grpo_quantize_fp8_workspace_bytes());
  const int64_t n = rows * cols;
  const int nparts = (int)std::min<int64_t>(kQuantParts, (n + 4095) / 4096);
  float* part = per_row ? nullptr : (float*)workspace;
  int* e = per_row ? nullptr : (int*)((char*)workspace + kQuantParts * 4);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == GRPO_BF16)
    GRPO_HIP(grpo::launch_fp8_quantize<__bf16>((const __bf16*)X, rows, cols, per_row, part, nparts,
                                               e, codes, scales, s));
  else
    GRPO_HIP(grpo::launch_fp8_quantize<float>((const float*)X, rows, cols, per_row, part, nparts, e,
                                              codes, scales, s));
  return GRPO_OK;
}

int grpo_dequantize_fp8(const uint8_t* codes, const float* scales, int64_t rows, int64_t cols,
                        int per_row, void* out, void* stream) {
  g_last_error[0] = 0;
  GRPO_CHECK_PTR(codes);
  GRPO_CHECK_PTR(scales);
  GRPO_CHECK_PTR(out);
  if (rows <= 0 || cols <= 0) return fail(GRPO_ERR_INVALID_ARG, "rows and cols must be positive");
  if (per_row != 0 && per_row != 1) return fail(GRPO_ERR_INVALID_ARG, "per_row must be 0 or 1");
  if (cols % 16 != 0) return fail(GRPO_ERR_UNSUPPORTED, "cols=%lld must be a multiple of 16",
                                  (long long)cols);
  if (rows > INT32_MAX) return fail(GRPO_ERR_UNSUPPORTED, "rows must fit int32");
  GRPO_HIP(grpo::launch_fp8_dequantize(codes, rows, cols, scales, per_row, (__bf16*)out,
                                       (hipStream_t)stream));
  return GRPO_OK;
}

int grpo_ref_logprobs_fp8(const uint8_t* H8, const float* h_scale, const uint8_t* W8,
                          const float* w_scale, const int32_t* y, int64_t N, int64_t d, int64_t V,
                          int64_t chunk, const grpo_opts* opts, float* ref_lp, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  grpo::LogitXform xf;
  grpo::LossVariant lv;
  if (make_xform(opts, &xf) != GRPO_OK || make_variant(opts, &lv) != GRPO_OK)
    return GRPO_ERR_INVALID_ARG;
  GRPO_CHECK_PTR(H8);
  GRPO_CHECK_PTR(h_scale);
  GRPO_CHECK_PTR(W8);
  GRPO_CHECK_PTR(w_scale);
  GRPO_CHECK_PTR(y);
  GRPO_CHECK_PTR(ref_lp);
  int st = check_shape(N, d, V, GRPO_FP8_E4M3, chunk, true);
  if (st != GRPO_OK) return st;
  const size_t need = plan_fwd(N, V, chunk).total;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GRPO_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  return lse_pass<uint8_t>(0, H8, W8, y, nullptr, nullptr, nullptr, N, 1, d, V, 0.f, chunk, xf, lv,
                           nullptr, ref_lp, nullptr, nullptr, (char*)workspace,
                           (hipStream_t)stream, w_scale, h_scale);
}

int grpo_loss_fwd_fp8(const uint8_t* H8, const float* h_scale, const uint8_t* W8,
                      const float* w_scale, const int32_t* y, const uint8_t* mask,
                      const float* adv, const float* ref_lp, int64_t B, int64_t L, int64_t d,
                      int64_t V, float beta, int64_t chunk, const grpo_opts* opts, float* loss,
                      float* lp, float* kl, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream) {
  g_last_error[0] = 0;
  grpo::LogitXform xf;
  grpo::LossVariant lv;
  if (make_xform(opts, &xf) != GRPO_OK || make_variant(opts, &lv) != GRPO_OK)
    return GRPO_ERR_INVALID_ARG;
  GRPO_CHECK_PTR(H8);
  GRPO_CHECK_PTR(h_scale);
  GRPO_CHECK_PTR(W8);
  GRPO_CHECK_PTR(w_scale);
  GRPO_CHECK_PTR(y);
  GRPO_CHECK_PTR(mask);
  GRPO_CHECK_PTR(adv);
  GRPO_CHECK_PTR(ref_lp);
  GRPO_CHECK_PTR(loss);
  GRPO_CHECK_PTR(lp);
  GRPO_CHECK_PTR(kl);
  GRPO_CHECK_PTR(lse);
  if (B <= 0 || L <= 0) return fail(GRPO_ERR_INVALID_ARG, "B and L must be positive");
  if (B > INT32_MAX / L) return fail(GRPO_ERR_UNSUPPORTED, "B*L exceeds int32");
  const int64_t N = B * L;
  int st = check_shape(N, d, V, GRPO_FP8_E4M3, chunk, true);
  if (st != GRPO_OK) return st;
  if (!isfinite(beta)) return fail(GRPO_ERR_INVALID_ARG, "beta must be finite");
  const size_t need = plan_fwd(N, V, chunk).total;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GRPO_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  return lse_pass<uint8_t>(1, H8, W8, y, mask, adv, ref_lp, N, L, d, V, beta, chunk, xf, lv, loss,
                           lp, kl, lse, (char*)workspace, (hipStream_t)stream, w_scale, h_scale);
}

int grpo_loss_bwd_fp8(const uint8_t* H8, const float* h_scale, const uint8_t* W8,
                      const float* w_scale, const int32_t* y, const uint8_t* mask,
                      const float* adv, const float* ref_lp, const float* lp, const float* lse,
                      int64_t B, int64_t L, int64_t d, int64_t V, float beta, float grad_loss,
                      int64_t chunk, const grpo_opts* opts, void* dH, float* dW, void* workspace,
                      size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  grpo::LogitXform xf;
  grpo::LossVariant lv;
  if (make_xform(opts, &xf) != GRPO_OK || make_variant(opts, &lv) != GRPO_OK)
    return GRPO_ERR_INVALID_ARG;
  GRPO_CHECK_PTR(H8);
  GRPO_CHECK_PTR(h_scale);
  GRPO_CHECK_PTR(W8);
  GRPO_CHECK_PTR(w_scale);
  GRPO_CHECK_PTR(y);
  GRPO_CHECK_PTR(mask);
  GRPO_CHECK_PTR(adv);
  GRPO_CHECK_PTR(ref_lp);
  GRPO_CHECK_PTR(lp);
  GRPO_CHECK_PTR(lse);
  GRPO_CHECK_PTR(dH);
  GRPO_CHECK_PTR(dW);
  if (B <= 0 || L <= 0) return fail(GRPO_ERR_INVALID_ARG, "B and L must be positive");
  if (B > INT32_MAX / L) return fail(GRPO_ERR_UNSUPPORTED, "B*L exceeds int32");
  const int64_t N = B * L;
  int st = check_shape(N, d, V, GRPO_FP8_E4M3, chunk, true);
  if (st != GRPO_OK) return st;
  if (!isfinite(beta)) return fail(GRPO_ERR_INVALID_ARG, "beta must be finite");
  if (!isfinite(grad_loss)) return fail(GRPO_ERR_INVALID_ARG, "grad_loss must be finite");
  // a caller's size is always a size (>= 1 here): 0 and -1 select the default and
  // minimum plans only in the workspace queries
  const int64_t wsb = std::max<int64_t>(1, (int64_t)std::min<size_t>(workspace_bytes, (size_t)INT64_MAX));
  const Fp8BwdPlan p = plan_bwd_fp8(N, d, V, chunk, workspace == nullptr ? 1 : wsb);
  if (workspace == nullptr || !p.b.ok)
    return fail(GRPO_ERR_WORKSPACE, "workspace needs at least %zu bytes, got %zu",
                plan_bwd_fp8(N, d, V, chunk, -1).total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  __bf16* Hb = (__bf16*)(ws + p.o_h);
  __bf16* Wb = (__bf16*)(ws + p.o_w);
  GRPO_HIP(grpo::launch_fp8_dequantize(H8, N, d, h_scale, 1, Hb, s));
  GRPO_HIP(grpo::launch_fp8_dequantize(W8, V, d, w_scale, 0, Wb, s));
  // the logits are recomputed from the fp8 codes (as the forward formed them);
  // dH and dW come from the bf16 GEMMs on the exact copies
  Fp8Recompute f8;
  f8.H8 = H8;
  f8.h_scale = h_scale;
  f8.W8 = W8;
  f8.w_scale = w_scale;
  f8.H8_act = (uint8_t*)(ws + p.o_h8act);
  f8.hs_act = (float*)(ws + p.o_hsact);
  return bwd_pass<__bf16>(Hb, Wb, y, mask, adv, ref_lp, lp, lse, N, L, d, V, beta, grad_loss, chunk,
                          xf, lv, (__bf16*)dH, dW, p.b, ws + p.o_bf16, s, f8);
}

}  // extern "C"

// ---------------------------------------------------------------- forward without allocation
// grpo_loss_fwd_noalloc keeps the forward's per-chunk scratch (split partials,
// target logits, loss block sums, per-sequence counts) in this file-scope
// device array instead of a caller's workspace.  Each device that runs the
// library holds its own copy, at its own address, until the process ends.
// In host code `scratch` names a host-side stand-in: only the address from
// hipGetSymbolAddress, taken once per device with that device current, is
// ever handed to a kernel.
namespace {
constexpr size_t kScratchBytes = 64ull << 20;
__device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];

int device_scratch(char** out) {
  int dev = -1;
  GRPO_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GRPO_ERR_UNSUPPORTED, "device %d is past the %d devices this library serves", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    GRPO_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr) return fail(GRPO_ERR_HIP, "hipGetSymbolAddress gave a null scratch address");
    g_scratch_ptr[dev] = (char*)p;
  }
  *out = g_scratch_ptr[dev];
  return GRPO_OK;
}
}  // namespace

extern "C" {

size_t grpo_noalloc_scratch_bytes(void) { return kScratchBytes; }

int grpo_loss_fwd_noalloc(const void* H, const void* W, const int32_t* y, const uint8_t* mask,
                          const float* adv, const float* ref_lp, int64_t B, int64_t L, int64_t d,
                          int64_t V, int dtype, float beta, int64_t chunk, const grpo_opts* opts,
                          float* loss, float* lp, float* kl, float* lse, void* stream) {
  g_last_error[0] = 0;
  if (B <= 0 || L <= 0) return fail(GRPO_ERR_INVALID_ARG, "B and L must be positive");
  if (B > INT32_MAX / L) return fail(GRPO_ERR_UNSUPPORTED, "B*L exceeds int32");
  const int st = check_shape(B * L, d, V, dtype, chunk);
  if (st != GRPO_OK) return st;
  const size_t need = plan_fwd(B * L, V, chunk).total;
  if (need > kScratchBytes)
    return fail(GRPO_ERR_WORKSPACE,
                "the forward needs %zu bytes of scratch at this V and chunk; the static scratch "
                "holds %zu (use a smaller chunk, or grpo_loss_fwd with a workspace)",
                need, kScratchBytes);
  char* ws = nullptr;
  const int sc = device_scratch(&ws);
  if (sc != GRPO_OK) return sc;
  // every scratch slot the kernels read is written earlier in the same call, so
  // nothing needs clearing between calls
  return grpo_loss_fwd_ex(H, W, y, mask, adv, ref_lp, B, L, d, V, dtype, beta, chunk, opts, loss,
                          lp, kl, lse, ws, kScratchBytes, stream);
}

int grpo_gemm_nt(const void* A, const void* B, int64_t M, int64_t N, int64_t K, int dtype,
                 float* C, void* stream) {
  g_last_error[0] = 0;
  GRPO_CHECK_PTR(A);
  GRPO_CHECK_PTR(B);
  GRPO_CHECK_PTR(C);
  if (M <= 0 || N <= 0 || K <= 0) return fail(GRPO_ERR_INVALID_ARG, "M, N, K must be positive");
  if (dtype != GRPO_F32 && dtype != GRPO_BF16)
    return fail(GRPO_ERR_INVALID_ARG, "dtype %d is neither GRPO_F32 nor GRPO_BF16", dtype);
  if ((K * (int64_t)esize(dtype)) % 16 != 0)
    return fail(GRPO_ERR_UNSUPPORTED, "K * element size must be a multiple of 16 bytes");
  if (256 * K * (int64_t)esize(dtype) >= (1ll << 31) || M > INT32_MAX || N > INT32_MAX)
    return fail(GRPO_ERR_UNSUPPORTED, "shape too large");
  hipStream_t s = (hipStream_t)stream;
  if (dtype == GRPO_BF16)
    GRPO_HIP(grpo::launch_gemm_nt<__bf16>((const __bf16*)A, (const __bf16*)B, M, N, K, C, s));
  else
    GRPO_HIP(grpo::launch_gemm_nt<float>((const float*)A, (const float*)B, M, N, K, C, s));
  return GRPO_OK;
}

int grpo_timing_begin(void) {
  grpo::timing_begin();
  return GRPO_OK;
}

int grpo_timing_end(const char** names, int* launches, double* total_ms, int max_entries) {
  return grpo::timing_end(names, launches, total_ms, max_entries);
}

}  // extern "C"
