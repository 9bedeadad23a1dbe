/*
 * dust.h -- C ABI of the MI355X (gfx950) Dust estimator library, libdust.so.
 *
 * Dust estimates the weight gradient of one linear layer y_t = W x_t from
 * loss values alone: it jitters every token's output by sigma a_t over K
 * draws, scores each token by its own centred loss reduction c_t, discounts
 * the credit along the sequence r_t = sum_{s>=t} gamma^(s-t) c_s, averages the
 * reward-weighted noise into g_t = -1/(K sigma) sum_i r_t^(i) a_t^(i), and
 * contracts G_W = sum_t g_t x_t^T ("Dust: every token is a member of the
 * population", section "Perturb the activations, not the weights", the three
 * estimator equations; reward = clean minus perturbed loss and the centring
 * across draws of one forward: section "What the released code actually
 * does", step 2).  Here the layer-local loss L_t = 1/2 ||y_t - target_t||^2
 * stands in for the network downstream of the layer.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller; tensors are
 *    row-major and contiguous.  The library never allocates, frees or
 *    synchronizes; all work is enqueued on `stream` (a hipStream_t passed as
 *    void*; NULL is the default stream) and returns before it runs.
 *  - Status codes are returned; on a non-OK status dust_last_error() gives a
 *    message (thread-local, valid until the next call on the thread).
 *    Argument errors are found on the host before anything is enqueued.
 *    Faults while kernels run surface at the caller's next synchronization.
 *  - Non-finite input values are not checked; they propagate.
 *  - Results are deterministic: the same arguments give bitwise-equal
 *    outputs (every reduction has a fixed order; no float atomics).
 */
#ifndef DUST_H
#define DUST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DUST_F32 = 0, DUST_BF16 = 1 } dust_dtype_t;

typedef enum {
  DUST_OK = 0,
  DUST_ERR_INVALID_ARG = 1, /* a size, scalar or required pointer is invalid */
  DUST_ERR_UNSUPPORTED = 2, /* dtype or size outside what the kernels take  */
  DUST_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required      */
  DUST_ERR_HIP = 4          /* a HIP launch or runtime call failed          */
} dust_status_t;

/*
 * Bytes of device workspace dust_estimate needs for these sizes (0 when the
 * sizes are invalid).  Pure host function.  The workspace holds what the
 * stages of the estimate hand to each other ("Dust: every token is a member
 * of the population", section "Perturb the activations, not the weights",
 * the three estimator equations): delta_t = W x_t - target_t, the per-draw
 * loss reductions and their centred, discounted credit, g_t (for bf16 as
 * its hi/lo split), and the token-split partial sums of G_W.  The noise is
 * never part of it: a counter-based generator regenerates it where needed
 * ("Scaling To Unfathomable Depth", section "MeZO": store the seed, not the
 * perturbation).
 */
size_t dust_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int32_t K,
                            int32_t antithetic, int32_t dtype);

/*
 * Bytes of device workspace that let dust_estimate and dust_estimate_local
 * generate each noise value once for gamma > 0 ("Dust: every token is a
 * member of the population", section "Perturb the activations, not the
 * weights": the credit r_t = c_t + gamma r_(t+1)).  One walk over each
 * sequence in reverse token order per chain forms the chain's R_t from the
 * same noise values it reweights:
 *  - antithetic pairs: centring and curvature cancel within a pair, so
 *    r+ - r- = -2 sigma R_t with R_t = P_t + gamma R_(t+1), P_t = <delta_t,
 *    a_t>, and g_t = (2/K) sum_p R_t^p a_t^p;
 *  - plain draws: r_t^(i) = R_t^(i) - M_t with R_t^(i) = rho_t^(i) +
 *    gamma R_(t+1)^(i) and M_t = m_t + gamma M_(t+1) (m_t the mean of rho_t
 *    over the draws, the same for every draw), so
 *    g_t = -1/(K sigma) (sum_i R_t^(i) a_t^(i) - M_t sum_i a_t^(i)).
 * Larger than dust_workspace_bytes exactly when that path applies to these
 * sizes: gamma > 0, seq_len >= 2 dividing T, d_out <= 1024, (T / seq_len)
 * chains >= 2048 (a chain is a pair, K / 2 per sequence, or a plain draw,
 * K), and seq_len <= 8192 for plain draws; it adds, per group of 16 chains,
 * the partial sum of R a (T x d_out fp32) and for plain draws those of a
 * (T x d_out) and of rho (T), plus M (T).  A call takes that path when its
 * workspace is at least this size and it asks for neither rho nor reward
 * (which need every draw's centred credit); otherwise it regenerates the
 * noise in a second pass.  The two paths agree within fp32 rounding
 * (different summation orders); each is bitwise reproducible.  0 when the
 * sizes are invalid.  Pure host function.
 */
size_t dust_workspace_bytes_seq(int64_t T, int64_t d_in, int64_t d_out,
                                int64_t seq_len, int32_t K, float gamma,
                                int32_t antithetic, int32_t dtype);

/*
 * Host-side check of dust_estimate's arguments, the same check dust_estimate
 * runs first.  Touches no device memory and makes no HIP call.  The rules
 * follow from the estimator ("Dust: every token is a member of the
 * population", section "Perturb the activations, not the weights": K draws
 * per token centred across the draws of one forward, the credit summed
 * within a sequence with decay gamma; section "What a zeroth-order gradient
 * is" on antithetic pairs, two evaluations of one noise vector).  Rejects: a
 * NULL X, W, target or G_W; T, d_in, d_out <= 0; seq_len <= 0 or T not a
 * multiple of seq_len; T >= 2^31 or d_out >= 2^31 (the noise counter words
 * are 32-bit); K < 2 (centring over one draw leaves nothing); odd K with
 * antithetic pairs; sigma <= 0 or non-finite; gamma outside [0,1] or
 * non-finite; an unknown dtype or T >= 2^24 tokens in one call
 * (DUST_ERR_UNSUPPORTED); a NULL or too small workspace (DUST_ERR_WORKSPACE).
 */
dust_status_t dust_validate(const void* X, const void* W, const void* target,
                            int64_t T, int64_t d_in, int64_t d_out,
                            int64_t seq_len, int32_t dtype, int32_t K,
                            float sigma, float gamma, int32_t antithetic,
                            const float* G_W, const void* workspace,
                            size_t workspace_bytes);

/*
 * The estimator, all stages, enqueued on `stream`.
 *
 * Inputs (dtype `dtype`, all three the same):
 *   X      [T, d_in]      layer inputs, token t = b*seq_len + pos
 *   W      [d_out, d_in]  weights (nn.Linear layout)
 *   target [T, d_out]     target of the layer-local squared-error loss
 * Scalars:
 *   seq_len  tokens per sequence; the credit scan restarts at each end
 *   K        draws; with antithetic != 0 draws 2p and 2p+1 share noise
 *            vector p with signs +1 and -1 (K must be even)
 *   sigma    jitter scale (fp32); gamma credit decay in [0,1] (fp32)
 *   seed     64-bit noise key.  Noise value a_t^(n)[c] is Box-Muller of
 *            Philox4x32-10 words, counter (c/4, t, n, 0), key (seed low,
 *            seed high): words (w0, w1) give channels 4q, 4q+1 and (w2, w3)
 *            4q+2, 4q+3 as sqrt(-2 ln u) (cos 2 pi v, sin 2 pi v) with
 *            u = 1 - (w_even >> 9) 2^-23, v = (w_odd >> 9) 2^-23; it is
 *            regenerated where needed, never stored.
 * Outputs (fp32, overwritten, not accumulated):
 *   G_W        [d_out, d_in]  sum_t g_t x_t^T (NOT divided by T); required
 *   loss_clean [T]            L_t = 1/2 ||W x_t - target_t||^2; optional
 *   rho        [T, K]         loss reductions L_t - L_t^(i); optional
 *   reward     [T, K]         discounted centred credit r_t^(i); optional
 *   g          [T, d_out]     per-token error estimate g_t; optional
 *   (optional outputs may be NULL)
 * Workspace: device memory of at least dust_workspace_bytes(...) bytes,
 * owned by the caller, contents undefined on return; with
 * dust_workspace_bytes_seq(...) bytes a gamma > 0 call with antithetic pairs
 * generates each noise value once (see there).
 */
dust_status_t dust_estimate(const void* X, const void* W, const void* target,
                            int64_t T, int64_t d_in, int64_t d_out,
                            int64_t seq_len, int32_t dtype, int32_t K,
                            float sigma, float gamma, uint64_t seed,
                            int32_t antithetic, float* G_W, float* loss_clean,
                            float* rho, float* reward, float* g,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * dust_estimate for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace argument: its workspace is a file-scope device array
 * of DUST_NOALLOC_WORKSPACE_BYTES (64 MiB) inside the library, one copy per
 * GPU, placed when the library's code is first loaded on that GPU and held
 * until the process ends.  The call makes no hipMalloc, hipFree or other
 * allocating call (its first call on a GPU looks up that copy's address).
 * Sizes whose dust_workspace_bytes(...) exceeds the array are rejected with
 * DUST_ERR_UNSUPPORTED before anything is enqueued; the other argument
 * checks, the outputs and the errors are dust_estimate's.  The estimate is
 * the one dust_estimate computes with a workspace of that many bytes
 * (single generation for gamma > 0 where dust_workspace_bytes_seq(...) fits
 * in it).  Nothing in the array needs to start at zero: every stage writes
 * what the next one reads.  Every call on one GPU shares that GPU's array and
 * it keeps the last call's contents: calls that overlap on one GPU (on
 * different streams, or from threads without ordering between them) race
 * and give undefined results; calls ordered on one stream are safe.
 */
#define DUST_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
size_t dust_noalloc_workspace_capacity(void);
dust_status_t dust_estimate_noalloc(const void* X, const void* W, const void* target,
                                    int64_t T, int64_t d_in, int64_t d_out,
                                    int64_t seq_len, int32_t dtype, int32_t K,
                                    float sigma, float gamma, uint64_t seed,
                                    int32_t antithetic, float* G_W, float* loss_clean,
                                    float* rho, float* reward, float* g, void* stream);

/*
 * Host-side check of dust_estimate_local's arguments: the same rules as
 * dust_validate, with E required (4-byte aligned) and X and G_W either both
 * given or both NULL.  No HIP call.
 */
dust_status_t dust_validate_local(const void* X, const float* E, int64_t T,
                                  int64_t d_in, int64_t d_out, int64_t seq_len,
                                  int32_t dtype, int32_t K, float sigma,
                                  float gamma, int32_t antithetic,
                                  const float* G_W, const void* workspace,
                                  size_t workspace_bytes);

/*
 * The estimator with local scoring, for sites whose jitter never reaches the
 * loss ("Dust: every token is a member of the population", section "What the
 * released code actually does", step 4: a perturbed attention internal
 * earns c_s = -<g_s, Delta o_s>, the inner product of its output's change
 * with an error estimate of that output; keys, values and gates add later
 * tokens' scores with decay gamma = 0.98, queries use their own, gamma = 0).  Draw i jitters the
 * layer's own output by Delta o_t^(i) = s_i sigma a_t^(n(i)) and is scored
 * rho_t^(i) = -<E_t, Delta o_t^(i)>; centring, credit, g and
 * G_W = sum_t g_t x_t^T follow as in dust_estimate.  E[g_t] = E_t with
 * antithetic pairs ((K-1)/K E_t with plain draws); g does not depend on
 * sigma.  Per-site gamma is this call's gamma.
 *
 * Inputs:
 *   X  [T, d_in]   layer inputs, dtype `dtype`; or NULL together with G_W
 *                  for a site with no input matrix (a value embedding, whose
 *                  gradient is then dust_reassemble_embedding of g): the
 *                  outer product is skipped, d_in only sizes the workspace
 *                  (pass 1) and dtype must still be a valid code
 *   E  [T, d_out]  fp32 error estimate of the layer's output
 * Scalars, noise and workspace (dust_workspace_bytes) as for dust_estimate.
 * Outputs (fp32, overwritten): G_W [d_out, d_in] (with X); rho [T, K] (the
 * scores), reward [T, K] and g [T, d_out] optional (NULL to skip).
 */
dust_status_t dust_estimate_local(const void* X, const float* E, int64_t T,
                                  int64_t d_in, int64_t d_out, int64_t seq_len,
                                  int32_t dtype, int32_t K, float sigma,
                                  float gamma, uint64_t seed,
                                  int32_t antithetic, float* G_W, float* rho,
                                  float* reward, float* g, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Local scoring through a recomputed attention ("Dust: every token is a
 * member of the population", section "What the released code actually
 * does", step 4, in the form that perturbs a query, key or value of an
 * attention block and evaluates that block's attention again from the
 * activations kept from the clean forward; the score is c_s =
 * -<e_s, Delta o_s>, e an error estimate of the attention output).  The attention is causal
 * softmax attention inside each sequence, heads of width d_head:
 * o_s,h = sum_{t<=s} softmax_t(<q_s,h, k_t,h> / sqrt(d_head)) v_t,h.  Draw i
 * jitters the site's token t by s_i sigma a_t^(n(i)) over its heads * d_head
 * channels (the noise of dust_estimate with d_out = heads * d_head), and the
 * score of token s is rho_s^(i) = -sum_h <E_s,h, o'_s,h - o_s,h>, o' the
 * attention with the jittered site.  Centring, credit (per-site gamma is this
 * call's gamma), g [T, heads * d_head] and G_W = sum_t g_t x_t^T (the site's
 * projection weight, with x the block's input) follow as in dust_estimate.
 */
typedef enum { DUST_ATTN_QUERY = 0, DUST_ATTN_KEY = 1, DUST_ATTN_VALUE = 2 } dust_attn_site_t;

/*
 * Bytes of device workspace dust_estimate_attention needs (0 when the sizes
 * are invalid).  Pure host function.  Besides the estimator's own regions
 * (dust_workspace_bytes with d_out = heads * d_head) it holds, per sequence
 * and head, the clean probabilities and for keys and queries the clean
 * weights p_st <e_s, v_t - o_s> as fp32 [Lp][Lp] (Lp = seq_len rounded up to
 * 64), and the score kernels' partial row sums, fp32 [slots][sums][K][Lp]
 * (keys and values: one slot per 64 tokens; queries: one; two sums, values
 * one).
 */
size_t dust_attention_workspace_bytes(int64_t T, int64_t d_in, int64_t heads, int64_t d_head,
                                      int64_t seq_len, int32_t site, int32_t K,
                                      int32_t antithetic, int32_t dtype);

/*
 * Host-side check of dust_estimate_attention's arguments: the rules of
 * dust_validate for T, seq_len, K, sigma, gamma and the workspace, with
 * d_out = heads * d_head; Qa, Ka, Va and E required and 16-byte aligned; X
 * and G_W both given or both NULL (without X, d_in only sizes the workspace:
 * pass 1); site one of dust_attn_site_t; dtype DUST_BF16 only
 * (DUST_ERR_UNSUPPORTED otherwise: the cached activations and X are bf16);
 * d_head 64 or 128 and seq_len at most 4096 (DUST_ERR_UNSUPPORTED).  No HIP
 * call.
 */
dust_status_t dust_validate_attention(const void* X, const void* Qa, const void* Ka,
                                      const void* Va, const float* E, int64_t T, int64_t d_in,
                                      int64_t heads, int64_t d_head, int64_t seq_len,
                                      int32_t site, int32_t dtype, int32_t K, float sigma,
                                      float gamma, int32_t antithetic, const float* G_W,
                                      const void* workspace, size_t workspace_bytes);

/*
 * The estimator with scores through a recomputed attention, enqueued on
 * `stream`.
 *
 * Inputs (device, row-major, contiguous):
 *   X      [T, d_in]             the block's input (bf16), or NULL with G_W
 *   Qa, Ka, Va [T, heads*d_head] the cached queries, keys and values (bf16);
 *                                head h on channels h*d_head .. +d_head-1,
 *                                token t = b*seq_len + pos
 *   E      [T, heads*d_head]     fp32 error estimate of the attention output
 * Scalars: site (which of Qa, Ka, Va is jittered); seq_len, K, sigma, gamma,
 * seed and antithetic as for dust_estimate.
 * Outputs (fp32, overwritten): G_W [heads*d_head, d_in] (with X); rho [T, K]
 * (the scores), reward [T, K] and g [T, heads*d_head] optional (NULL to
 * skip).  Workspace: at least dust_attention_workspace_bytes(...) bytes.
 * The scores use the closed forms of the recomputed output change (values:
 * sigma P A; keys and queries: the softmax re-weighted by e^x, with
 * x = s_i sigma <q_s, a_t> / sqrt(d_head) or s_i sigma <a_s, k_t> /
 * sqrt(d_head)), the noise entering a bf16 contraction as its hi + lo split.
 */
dust_status_t dust_estimate_attention(const void* X, const void* Qa, const void* Ka,
                                      const void* Va, const float* E, int64_t T, int64_t d_in,
                                      int64_t heads, int64_t d_head, int64_t seq_len,
                                      int32_t site, int32_t dtype, int32_t K, float sigma,
                                      float gamma, uint64_t seed, int32_t antithetic, float* G_W,
                                      float* rho, float* reward, float* g, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * Host-side check of dust_estimate_head's arguments: the rules of
 * dust_validate for T, d_in, K, sigma, dtype and the workspace (sized by
 * dust_workspace_bytes(T, d_in, V, K, antithetic, dtype)); X, W, labels and
 * G_W must not be NULL, labels 4-byte aligned, V a positive multiple of 256.
 * Label values live in device memory and are not checked here.  No HIP call.
 */
dust_status_t dust_validate_head(const void* X, const void* W, const int32_t* labels,
                                 int64_t T, int64_t d_in, int64_t V, int32_t dtype,
                                 int32_t K, float sigma, int32_t antithetic,
                                 const float* G_W, const void* workspace,
                                 size_t workspace_bytes);

/*
 * The estimator for a cross-entropy head ("Dust: every token is a member of
 * the population", section "What the released code actually does", step 5:
 * the head's logits are perturbed in 256-column slabs of the vocabulary,
 * and for each only the cross-entropy is formed again from cached sums).
 * Logits z_t = W x_t; loss CE_t = logsumexp(z_t) - z_t[labels[t]].  Each
 * slab j (columns 256 j .. 256 j + 255) is its own site with K draws: draw i
 * adds s_i sigma a_t^(n(i))[c] to the slab's columns only (the noise of
 * dust_estimate with the vocabulary column as channel), its loss reduction
 * rho = CE(z) - CE(z + jitter) is centred over the slab's K draws (no credit
 * scan: the loss is per token), and g_t on the slab's columns is
 * -1/(K sigma) sum_i c_i s_i a_i over that slab's draws;
 * G_W = sum_t g_t x_t^T.
 *
 * Inputs (device):
 *   X      [T, d_in]   layer inputs, dtype `dtype`, row-major
 *   W      [V, d_in]   head weights (nn.Linear layout), dtype `dtype`
 *   labels [T]         int32 targets in [0, V) (a value outside is clamped to
 *                      the range: memory-safe, result unspecified)
 * V must be a multiple of 256.  K, sigma, seed, antithetic as for
 * dust_estimate (gamma and seq_len do not apply).
 * Outputs (device fp32, overwritten; the caller owns them):
 *   G_W        [V, d_in]       required
 *   loss_clean [T]             optional (NULL skips)
 *   rho        [T, V/256, K]   optional: loss reductions per slab and draw
 *   g          [T, V]          optional: the estimated logit gradient
 * Workspace: dust_workspace_bytes(T, d_in, V, K, antithetic, dtype) bytes.
 * Errors as for dust_estimate (validation first, nothing enqueued on error).
 */
dust_status_t dust_estimate_head(const void* X, const void* W, const int32_t* labels,
                                 int64_t T, int64_t d_in, int64_t V, int32_t dtype,
                                 int32_t K, float sigma, uint64_t seed,
                                 int32_t antithetic, float* G_W, float* loss_clean,
                                 float* rho, float* g, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Workspace bytes dust_estimate_embedding needs (0 for sizes it cannot
 * plan, an unknown dtype included), and the bytes dust_reassemble_embedding
 * needs (0 for sizes it cannot plan).  Host-only, no HIP call.
 */
size_t dust_embedding_workspace_bytes(int64_t T, int64_t V, int64_t d, int32_t K,
                                      int32_t antithetic, int32_t dtype);
size_t dust_reassemble_workspace_bytes(int64_t T, int64_t V, int64_t d);

/*
 * Host-side check of dust_estimate_embedding's arguments: the rules of
 * dust_validate for T, K, sigma, gamma, seq_len and dtype with d_out = d;
 * table, ids, target and G_E must not be NULL, ids 4-byte aligned,
 * 1 <= V < 2^31, scale finite, the workspace at least
 * dust_embedding_workspace_bytes(T, V, d, K, antithetic, dtype) bytes.  Id
 * values live in device memory and are not checked here.  No HIP call.
 */
dust_status_t dust_validate_embedding(const void* table, const int32_t* ids,
                                      const void* target, int64_t T, int64_t V, int64_t d,
                                      int64_t seq_len, int32_t dtype, int32_t K,
                                      float sigma, float gamma, int32_t antithetic,
                                      float scale, const float* G_E,
                                      const void* workspace, size_t workspace_bytes);

/*
 * The estimator for a token embedding o_t = E[ids[t]] ("Dust: every token
 * is a member of the population", section "What the released code actually
 * does", step 7: an embedding's per-token error becomes its weight gradient
 * by a scatter-add, and every estimate is divided by the token count before
 * it is written to .grad).  Step 1 of dust_estimate becomes the gather
 * delta_t = E[ids[t]] - target_t (layer-local loss); the jitter, loss
 * reductions, centring, credit scan and g are dust_estimate's with
 * d_out = d; the outer product becomes
 *   G_E[v] = scale * sum_{t: ids[t] = v} g_t,
 * every row written (zero for ids absent from the batch), summed in a fixed
 * order (bitwise reproducible).  scale = 1/T writes what the page writes to
 * .grad; scale = 1 gives the plain sum of the other entry points.
 *
 * Inputs (device): table [V, d] and target [T, d] in dtype `dtype`;
 * ids [T] int32 in [0, V) (a value outside is clamped into the range:
 * memory-safe, result unspecified).  K, sigma, gamma, seed, antithetic,
 * seq_len as for dust_estimate.
 * Outputs (device fp32, overwritten; the caller owns them): G_E [V, d]
 * required; loss_clean [T], rho [T, K], reward [T, K], g [T, d] optional.
 * Workspace: dust_embedding_workspace_bytes(T, V, d, K, antithetic, dtype).
 */
dust_status_t dust_estimate_embedding(const void* table, const int32_t* ids,
                                      const void* target, int64_t T, int64_t V, int64_t d,
                                      int64_t seq_len, int32_t dtype, int32_t K,
                                      float sigma, float gamma, uint64_t seed,
                                      int32_t antithetic, float scale, float* G_E,
                                      float* loss_clean, float* rho, float* reward,
                                      float* g, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * Host-side check of dust_reassemble_embedding's arguments: ids, g and G_E
 * not NULL and 4-byte aligned, T, V, d positive (T < 2^24, V < 2^31), scale
 * finite, the workspace at least dust_reassemble_workspace_bytes(T, V, d)
 * bytes.  No HIP call.
 */
dust_status_t dust_validate_reassemble(const int32_t* ids, const float* g, int64_t T,
                                       int64_t V, int64_t d, float scale, const float* G_E,
                                       const void* workspace, size_t workspace_bytes);

/*
 * The embedding's weight gradient from per-token errors alone (the
 * scatter-add of the same passage, step 7), for an error g that comes from
 * elsewhere (dust_estimate_local's g for value embeddings, for instance):
 *   G_E[v] = scale * sum_{t: ids[t] = v} g_t   for every v in [0, V),
 * zero rows for absent ids, a fixed summation order (a stable counting sort
 * of the tokens by id, then a tiled reduce-by-key).
 * Inputs (device): ids [T] int32 (clamped into [0, V) as above), g [T, d]
 * fp32.  Output: G_E [V, d] fp32, overwritten.  Workspace:
 * dust_reassemble_workspace_bytes(T, V, d).
 */
dust_status_t dust_reassemble_embedding(const int32_t* ids, const float* g, int64_t T,
                                        int64_t V, int64_t d, float scale, float* G_E,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * Test hook: the noise the estimator uses, written out.  The estimator's
 * noise is a pure function of (seed, noise index, token, channel) from a
 * counter-based generator, so any value can be produced on its own and none
 * is stored ("Scaling To Unfathomable Depth", section "MeZO": counter-based
 * generators such as Philox give the n-th value from the seed and n alone;
 * the layout and transform are those of dust_estimate's `seed` argument).
 * For noise indices n0..n0+n_cnt-1 and tokens t0..t0+t_cnt-1:
 *   words [n_cnt, t_cnt, 4*ceil(d_out/4)] uint32  Philox words (optional)
 *   gauss [n_cnt, t_cnt, d_out]           fp32    Gaussians    (optional)
 * Sizes must be positive and n0+n_cnt, t0+t_cnt, d_out below 2^31.
 */
dust_status_t dust_noise_fill(uint64_t seed, int64_t n0, int64_t n_cnt,
                              int64_t t0, int64_t t_cnt, int64_t d_out,
                              uint32_t* words, float* gauss, void* stream);

/*
 * Measurement hook (used by the benchmark to time the dominant kernel with
 * HIP events inside its timed region).  After this call, estimate call
 * number i (dust_estimate, dust_estimate_local, dust_estimate_head or
 * dust_estimate_embedding) has
 * start[i % n_pairs] and stop[i % n_pairs] (hipEvent_t values passed as
 * void*, created with timing enabled and owned by the caller) stamped by the
 * dispatch of its noise kernel (the single-generation kernel when gamma = 0,
 * else the jitter-loss kernel; the slab kernel of dust_estimate_head), at the
 * kernel's start and end (hipExtLaunchKernelGGL's events).
 * n_pairs = 0 turns the hook off.  The pointer arrays are copied; the events
 * must outlive their use.  The hook belongs to the calling thread: it times
 * the estimate calls that thread makes.
 */
dust_status_t dust_set_timing_events(void* const* start, void* const* stop,
                                     int32_t n_pairs);

/*
 * Measurement hook: per-kernel durations and algorithmic work of this
 * thread's library calls (used by the benchmark to report every stage
 * against its roofline).  dust_profile_begin creates 2 * max_launches HIP
 * events owned by the library (1 <= max_launches <= 2^20) and turns the
 * profile on for the calling thread; from then on each kernel launch of the
 * thread's library calls, up to max_launches of them, is stamped by its own
 * event pair at the dispatch's start and end (hipExtLaunchKernelGGL's
 * events; while the profile is on it takes the place of the
 * dust_set_timing_events pair).  dust_profile_end turns it off, waits for
 * the recorded launches, and writes for the first `cap` of them, in launch
 * order: the stage name (a static string: "base_gemm", "fused_g0_kernel",
 * "outer_gemm", "split_sum_kernel", ...), the duration in milliseconds, the
 * method's MFMA flops of the launch (2 x the contraction's multiply-adds;
 * 0 for kernels without a contraction), and the least HBM bytes the launch
 * must move (its inputs read once, its outputs written once); *count gets
 * the number of launches recorded.  It then destroys the events.  A HIP
 * error returns DUST_ERR_HIP (the profile is released either way).
 */
dust_status_t dust_profile_begin(int32_t max_launches);
dust_status_t dust_profile_end(const char** kernel, float* ms, double* flops, double* bytes,
                               int32_t cap, int32_t* count);

/* Message for the last non-OK status on this thread ("" if none). */
const char* dust_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DUST_H */
