// dust_host.cpp -- host-only entry points of libdust.so: argument validation,
// workspace sizing and the thread-local error text.  No HIP calls here, so
// these work (and are tested) on machines without a GPU.
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "dust.h"
#include "dust_internal.hpp"
#include "dust_plan.hpp"

namespace {
thread_local char g_last_error[512] = "";
}

namespace dust {

dust_status_t fail(dust_status_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

dust_status_t ok() {
  g_last_error[0] = '\0';
  return DUST_OK;
}

}  // namespace dust

extern "C" {

size_t dust_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int32_t K,
                            int32_t antithetic, int32_t dtype) {
  if (dtype != DUST_F32 && dtype != DUST_BF16) return 0;
  dust::Plan p;
  if (!dust::make_plan(T, d_in, d_out, K, antithetic, dtype, &p)) return 0;
  return p.total;
}

size_t dust_workspace_bytes_seq(int64_t T, int64_t d_in, int64_t d_out, int64_t seq_len,
                                int32_t K, float gamma, int32_t antithetic, int32_t dtype) {
  if (dtype != DUST_F32 && dtype != DUST_BF16) return 0;
  dust::Plan p;
  if (!dust::make_plan(T, d_in, d_out, K, antithetic, dtype, &p)) return 0;
  const dust::ChainPlan c = dust::make_chain_plan(p, seq_len, gamma);
  return c.ok ? c.total : p.total;
}

}  // extern "C"

namespace {

// The checks both estimators share (everything but their own pointers).
dust_status_t validate_common(int64_t T, int64_t d_in, int64_t d_out, int64_t seq_len,
                              int32_t dtype, int32_t K, float sigma, float gamma,
                              int32_t antithetic, const void* workspace,
                              size_t workspace_bytes) {
  using dust::fail;
  if (T <= 0 || d_in <= 0 || d_out <= 0)
    return fail(DUST_ERR_INVALID_ARG, "T=%lld, d_in=%lld, d_out=%lld must be positive",
                (long long)T, (long long)d_in, (long long)d_out);
  if (T >= (int64_t(1) << 31) || d_out >= (int64_t(1) << 31) || d_in >= (int64_t(1) << 31))
    return fail(DUST_ERR_INVALID_ARG, "T, d_in and d_out must be below 2^31");
  if (T >= (int64_t(1) << 24))
    return fail(DUST_ERR_UNSUPPORTED, "T=%lld: at most 2^24 - 1 tokens per call", (long long)T);
  if (seq_len <= 0 || T % seq_len != 0)
    return fail(DUST_ERR_INVALID_ARG, "seq_len=%lld must be positive and divide T=%lld",
                (long long)seq_len, (long long)T);
  if (K < 2)
    return fail(DUST_ERR_INVALID_ARG, "K=%d: at least 2 draws are needed for centring", K);
  if (antithetic && (K % 2) != 0)
    return fail(DUST_ERR_INVALID_ARG, "K=%d must be even with antithetic pairs", K);
  if (!(std::isfinite(sigma) && sigma > 0.0f))
    return fail(DUST_ERR_INVALID_ARG, "sigma=%g must be finite and positive", (double)sigma);
  if (!(std::isfinite(gamma) && gamma >= 0.0f && gamma <= 1.0f))
    return fail(DUST_ERR_INVALID_ARG, "gamma=%g must lie in [0, 1]", (double)gamma);
  if (dtype != DUST_F32 && dtype != DUST_BF16)
    return fail(DUST_ERR_UNSUPPORTED, "dtype=%d: only DUST_F32 (0) and DUST_BF16 (1)", dtype);
  dust::Plan p;
  if (!dust::make_plan(T, d_in, d_out, K, antithetic, dtype, &p))
    return fail(DUST_ERR_UNSUPPORTED, "sizes exceed the kernels' index range");
  if (!workspace || workspace_bytes < p.total)
    return fail(DUST_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                workspace ? workspace_bytes : (size_t)0, p.total);
  return dust::ok();
}

}  // namespace

extern "C" {

dust_status_t dust_validate(const void* X, const void* W, const void* target,
                            int64_t T, int64_t d_in, int64_t d_out,
                            int64_t seq_len, int32_t dtype, int32_t K,
                            float sigma, float gamma, int32_t antithetic,
                            const float* G_W, const void* workspace,
                            size_t workspace_bytes) {
  if (!X || !W || !target || !G_W)
    return dust::fail(DUST_ERR_INVALID_ARG, "X, W, target and G_W must not be NULL");
  return validate_common(T, d_in, d_out, seq_len, dtype, K, sigma, gamma, antithetic,
                         workspace, workspace_bytes);
}

dust_status_t dust_validate_local(const void* X, const float* E, int64_t T, int64_t d_in,
                                  int64_t d_out, int64_t seq_len, int32_t dtype, int32_t K,
                                  float sigma, float gamma, int32_t antithetic,
                                  const float* G_W, const void* workspace,
                                  size_t workspace_bytes) {
  if (!E) return dust::fail(DUST_ERR_INVALID_ARG, "E must not be NULL");
  // without X there is no outer product: X and G_W are given or omitted together
  if ((X == nullptr) != (G_W == nullptr))
    return dust::fail(DUST_ERR_INVALID_ARG, "X and G_W must both be given or both be NULL");
  if ((uintptr_t)E % 4 != 0)
    return dust::fail(DUST_ERR_INVALID_ARG, "E must be 4-byte aligned (fp32)");
  return validate_common(T, d_in, d_out, seq_len, dtype, K, sigma, gamma, antithetic,
                         workspace, workspace_bytes);
}

dust_status_t dust_validate_head(const void* X, const void* W, const int32_t* labels,
                                 int64_t T, int64_t d_in, int64_t V, int32_t dtype, int32_t K,
                                 float sigma, int32_t antithetic, const float* G_W,
                                 const void* workspace, size_t workspace_bytes) {
  if (!X || !W || !labels || !G_W)
    return dust::fail(DUST_ERR_INVALID_ARG, "X, W, labels and G_W must not be NULL");
  if ((uintptr_t)labels % 4 != 0)
    return dust::fail(DUST_ERR_INVALID_ARG, "labels must be 4-byte aligned (int32)");
  if (V <= 0 || V % 256 != 0)
    return dust::fail(DUST_ERR_INVALID_ARG, "V=%lld must be a positive multiple of 256",
                      (long long)V);
  // the loss is per token: every token is its own sequence, gamma = 0
  return validate_common(T, d_in, V, 1, dtype, K, sigma, 0.0f, antithetic, workspace,
                         workspace_bytes);
}

size_t dust_embedding_workspace_bytes(int64_t T, int64_t V, int64_t d, int32_t K,
                                      int32_t antithetic, int32_t dtype) {
  if (dtype != DUST_F32 && dtype != DUST_BF16) return 0;
  dust::Plan p;
  dust::ReassemblyPlan r;
  size_t base = 0, total = 0;
  if (!dust::make_embedding_plan(T, V, d, K, antithetic, dtype, &p, &r, &base, &total)) return 0;
  return total;
}

size_t dust_reassemble_workspace_bytes(int64_t T, int64_t V, int64_t d) {
  dust::ReassemblyPlan r;
  if (!dust::make_reassembly_plan(T, V, d, &r)) return 0;
  return r.total;
}

dust_status_t dust_validate_embedding(const void* table, const int32_t* ids,
                                      const void* target, int64_t T, int64_t V, int64_t d,
                                      int64_t seq_len, int32_t dtype, int32_t K, float sigma,
                                      float gamma, int32_t antithetic, float scale,
                                      const float* G_E, const void* workspace,
                                      size_t workspace_bytes) {
  if (!table || !ids || !target || !G_E)
    return dust::fail(DUST_ERR_INVALID_ARG, "table, ids, target and G_E must not be NULL");
  if ((uintptr_t)ids % 4 != 0)
    return dust::fail(DUST_ERR_INVALID_ARG, "ids must be 4-byte aligned (int32)");
  if (V <= 0 || V >= (int64_t(1) << 31))
    return dust::fail(DUST_ERR_INVALID_ARG, "V=%lld must lie in [1, 2^31)", (long long)V);
  if (!std::isfinite(scale))
    return dust::fail(DUST_ERR_INVALID_ARG, "scale must be finite");
  // the estimator's own checks, on a workspace of the estimator's size
  const dust_status_t st = validate_common(T, 1, d, seq_len, dtype, K, sigma, gamma, antithetic,
                                           workspace, (size_t)-1);
  if (st != DUST_OK) return st;
  dust::Plan p;
  dust::ReassemblyPlan r;
  size_t base = 0, total = 0;
  if (!dust::make_embedding_plan(T, V, d, K, antithetic, dtype, &p, &r, &base, &total))
    return dust::fail(DUST_ERR_UNSUPPORTED, "sizes exceed the kernels' index range");
  if (!workspace || workspace_bytes < total)
    return dust::fail(DUST_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                      workspace ? workspace_bytes : (size_t)0, total);
  return dust::ok();
}

dust_status_t dust_validate_reassemble(const int32_t* ids, const float* g, int64_t T,
                                       int64_t V, int64_t d, float scale, const float* G_E,
                                       const void* workspace, size_t workspace_bytes) {
  using dust::fail;
  if (!ids || !g || !G_E) return fail(DUST_ERR_INVALID_ARG, "ids, g and G_E must not be NULL");
  if ((uintptr_t)ids % 4 != 0 || (uintptr_t)g % 4 != 0 || (uintptr_t)G_E % 4 != 0)
    return fail(DUST_ERR_INVALID_ARG, "ids, g and G_E must be 4-byte aligned");
  if (T <= 0 || V <= 0 || d <= 0)
    return fail(DUST_ERR_INVALID_ARG, "T=%lld, V=%lld, d=%lld must be positive", (long long)T,
                (long long)V, (long long)d);
  if (!std::isfinite(scale)) return fail(DUST_ERR_INVALID_ARG, "scale must be finite");
  dust::ReassemblyPlan r;
  if (!dust::make_reassembly_plan(T, V, d, &r))
    return fail(DUST_ERR_UNSUPPORTED, "T=%lld, V=%lld, d=%lld exceed the kernels' index range",
                (long long)T, (long long)V, (long long)d);
  if (!workspace || workspace_bytes < r.total)
    return fail(DUST_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                workspace ? workspace_bytes : (size_t)0, r.total);
  return dust::ok();
}

size_t dust_attention_workspace_bytes(int64_t T, int64_t d_in, int64_t heads, int64_t d_head,
                                      int64_t seq_len, int32_t site, int32_t K,
                                      int32_t antithetic, int32_t dtype) {
  if (dtype != DUST_BF16 || heads <= 0 || d_head <= 0) return 0;
  dust::Plan p;
  if (!dust::make_plan(T, d_in, heads * d_head, K, antithetic, dtype, &p)) return 0;
  dust::AttnPlan a;
  if (!dust::make_attn_plan(p, seq_len, heads, d_head, site, &a)) return 0;
  return a.total;
}

dust_status_t dust_validate_attention(const void* X, const void* Qa, const void* Ka,
                                      const void* Va, const float* E, int64_t T, int64_t d_in,
                                      int64_t heads, int64_t d_head, int64_t seq_len,
                                      int32_t site, int32_t dtype, int32_t K, float sigma,
                                      float gamma, int32_t antithetic, const float* G_W,
                                      const void* workspace, size_t workspace_bytes) {
  using dust::fail;
  if (!Qa || !Ka || !Va || !E)
    return fail(DUST_ERR_INVALID_ARG, "Qa, Ka, Va and E must not be NULL");
  if ((X == nullptr) != (G_W == nullptr))
    return fail(DUST_ERR_INVALID_ARG, "X and G_W must both be given or both be NULL");
  if ((uintptr_t)Qa % 16 || (uintptr_t)Ka % 16 || (uintptr_t)Va % 16 || (uintptr_t)E % 16)
    return fail(DUST_ERR_INVALID_ARG, "Qa, Ka, Va and E must be 16-byte aligned");
  if (site != DUST_ATTN_QUERY && site != DUST_ATTN_KEY && site != DUST_ATTN_VALUE)
    return fail(DUST_ERR_INVALID_ARG, "site=%d: DUST_ATTN_QUERY, _KEY or _VALUE", site);
  if (heads <= 0 || d_head <= 0 || heads * d_head >= (int64_t(1) << 31))
    return fail(DUST_ERR_INVALID_ARG, "heads=%lld, d_head=%lld must be positive",
                (long long)heads, (long long)d_head);
  // the estimator's own checks, on a workspace of unbounded size
  const dust_status_t st = validate_common(T, X ? d_in : 1, heads * d_head, seq_len, dtype, K,
                                           sigma, gamma, antithetic, workspace, (size_t)-1);
  if (st != DUST_OK) return st;
  if (dtype != DUST_BF16)
    return fail(DUST_ERR_UNSUPPORTED, "dtype=%d: the attention site takes bf16 activations",
                dtype);
  if (d_head != 64 && d_head != 128)
    return fail(DUST_ERR_UNSUPPORTED, "d_head=%lld: 64 or 128", (long long)d_head);
  if (seq_len > dust::kAttnMaxSeqLen)
    return fail(DUST_ERR_UNSUPPORTED, "seq_len=%lld: at most %lld", (long long)seq_len,
                (long long)dust::kAttnMaxSeqLen);
  const size_t need = dust_attention_workspace_bytes(T, X ? d_in : 1, heads, d_head, seq_len,
                                                     site, K, antithetic, dtype);
  if (need == 0) return fail(DUST_ERR_UNSUPPORTED, "sizes exceed the kernels' index range");
  if (!workspace || workspace_bytes < need)
    return fail(DUST_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                workspace ? workspace_bytes : (size_t)0, need);
  return dust::ok();
}

const char* dust_last_error(void) { return g_last_error; }

}  // extern "C"
