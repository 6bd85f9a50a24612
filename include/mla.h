/*
 * mla.h - C ABI of libmla: gated, no-position Multi-head Latent Attention (MLA)
 * with a fused per-head maximum logit, and the QK-Clip weight rescale, for
 * AMD Instinct MI355X (gfx950).
 *
 * What the calls compute follows these pages:
 *  - "Kimi K3 · Gated MLA · OpenModelAtlas", the 20-step equation list:
 *      [k^C v] = c^KV W_UKV, K^C_h = cols 1:128, V_h = cols 129:256 of head h,
 *      K_h = [K^C_h, k^S], S = Q K^T, S <- S/sqrt(192), causal softmax
 *      (A_{t,s} = 0 for s > t), O~ = A V, o~ = reshape(O~), o = sigma(g) . o~;
 *      and the KimiMLAAttention excerpts (no rotary embedding, scaling =
 *      q_head_dim^-1/2, kv_b_proj / q_b_proj weights).
 *  - "Gated MLA et NoPE" (mkdocs.reaper.mx): the cache keeps one latent row of
 *      512 + 64 values per token; the output gate is a full-rank sigmoid; no
 *      position encoding; the attention output is kept in FP32 in training.
 *  - "Kimi Qkclip" (Fireworks blog): at inference the K up-projection is
 *      skipped (here: W_UK folded into the queries, W_UV applied afterwards).
 *  - "SOTA-131" (anthology-of-the-sota, QK-Clip practice): after each step,
 *      every head whose maximum attention logit exceeds a threshold has its
 *      query and key projection weights rescaled so that it does not.
 *
 * Conventions for every call
 *  - Row-major, contiguous tensors. Weights use the nn.Linear layout of the
 *    pages' code (out_features x in_features):
 *      w_kv_b = kv_b_proj.weight [H*(N+V), R]: head h owns rows h*(N+V) ...;
 *               its first N rows produce K^C_h (W_UK_h), the next V rows V_h (W_UV_h);
 *      w_q_b  = q_b_proj.weight  [H*D, q_in]:  head h owns rows h*D ...; its
 *               first N rows produce q^C_h, the last S rows q^R_h.
 *    Here H = heads, R = kv_rank, S = shared_dim, N = nope_dim, V = v_dim,
 *    D = N + S.
 *  - Activations: q [tokens, H, D] (per head q^C then q^R); c^KV [tokens, R]
 *    is the latent after its RMSNorm; k^S [tokens, S] is the shared key part
 *    (never normalised, one row per token used by every head); gate logits
 *    [tokens, H*V]; outputs [tokens, H*V] head-major.
 *  - Every pointer argument is a DEVICE pointer, 16-byte aligned (cu_seqlens
 *    and lens: 4-byte), owned by the caller.
 *    The library never allocates device memory. Apart from two opt-in
 *    exceptions (the per-kernel timing of mla_timing_*, host state, and the
 *    static scratch array of mla_absorbed_noalloc, device state), it keeps no
 *    state between calls. All work is enqueued asynchronously on `stream`.
 *  - Arguments are validated before anything is launched. On error nothing is
 *    launched, the status is returned and mla_last_error() (thread-local)
 *    describes it. No C++ exception crosses this interface.
 *  - There are no position inputs (no rotary embedding) and no dropout.
 *
 * Supported shapes: in bf16, the Kimi K3 head shape R=512, S=64, N=128, V=128
 * with any number of heads; in fp32, any R <= 1024, S+N <= 256, V <= 256.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID = 1,      /* bad pointer, size, alignment or value        */
  MLA_ERR_UNSUPPORTED = 2,  /* valid request outside the compiled shapes    */
  MLA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required   */
  MLA_ERR_HIP = 4           /* a HIP launch or runtime call failed          */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

typedef struct {
  int32_t heads;       /* H: number of attention heads (96 in Kimi K3)          */
  int32_t kv_rank;     /* R: width of the latent c^KV (kv_lora_rank, 512)       */
  int32_t shared_dim;  /* S: width of the shared key part k^S and of q^R (64)   */
  int32_t nope_dim;    /* N: width of q^C and K^C (qk_nope_head_dim, 128)       */
  int32_t v_dim;       /* V: width of V_h (v_head_dim, 128)                     */
  float scale;         /* score scale; 0 selects (N + S)^-1/2 = 1/sqrt(192)     */
} mla_dims;

/*
 * Optional QK-norm variant of the attention calls ("SOTA-131", Variations:
 * the other route to bounded logits, an RMSNorm on the attention queries and
 * on the KV entries instead of clipping the weights; Mechanism: normalising
 * the input of the logit). Passed as `q_norm` to mla_prefill, mla_absorbed and
 * mla_absorbed_noalloc; NULL leaves the query as given. When set, each head's
 * query is first replaced by
 *   q_h <- q_h / sqrt(mean over its N+S features of q_h^2 + eps) * weight
 * (q^C and q^R together), rounded to the input dtype, and the call proceeds
 * unchanged. The KV entries are the caller's: c^KV already leaves its own
 * RMSNorm (kv_a_layernorm), and a normalised k^S is produced where k^S is
 * (mla_rms_norm), as the cache rows are.
 * The norm bounds every scaled logit of head h by
 *   max|weight| * sqrt(sigma_h^2 max|c^KV|^2 + max|k^S|^2),
 * sigma_h the largest singular value of W_UK_h: through the key
 * up-projection the bound grows with the weights, which QK-Clip rescales.
 */
typedef struct {
  const void* weight;  /* [N+S] per-feature weight, in_dtype, shared by the heads;
                          NULL = ones                                            */
  float eps;           /* added to the mean square; finite, >= 0                 */
} mla_qk_norm;

/* ------------------------------------------------------------------------ */
/* Training form (materialised K and V)                                      */
/* ------------------------------------------------------------------------ */

/* Bytes of scratch memory mla_prefill needs for these sizes. */
size_t mla_prefill_workspace_size(const mla_dims* dims, mla_dtype in_dtype,
                                  int64_t total_tokens, int32_t nseq);

/*
 * Gated causal MLA over packed variable-length sequences ("Kimi K3 · Gated MLA",
 * equation list from "[k^C v] = c^KV W_UKV" to "o = sigma(g) . o~").
 *
 * For each head h and each sequence s = [cu_seqlens[s], cu_seqlens[s+1]):
 *   K^C_h = c^KV W_UK_h, V_h = c^KV W_UV_h   (expanded once into `workspace`)
 *   K_h = [K^C_h, k^S];  S = scale * Q_h K_h^T;  softmax over keys s' <= t of
 *   the same sequence;  O~_h = A V_h;  out[t, h*V + d] = sigma(gate[t, h*V+d]) * O~_h[t, d]
 *   (no gate factor when gate == NULL).
 *
 * q         [total_tokens, H, N+S]  in_dtype
 * ckv       [total_tokens, R]       in_dtype  (post-RMSNorm latent)
 * ks        [total_tokens, S]       in_dtype
 * w_kv_b    [H*(N+V), R]            in_dtype
 * gate      [total_tokens, H*V]     in_dtype, or NULL
 * q_norm    the QK-norm variant (see mla_qk_norm), or NULL
 * cu_seqlens[nseq+1] int32, device, non-decreasing, cu_seqlens[0] = 0 and
 *           cu_seqlens[nseq] = total_tokens (not checked on the device; a
 *           violation gives undefined results). Empty sequences are allowed.
 * out       [total_tokens, H*V]     out_dtype (MLA_F32: the FP32 training
 *           output; MLA_BF16 allowed when in_dtype is MLA_BF16)
 * lse       [H, total_tokens] fp32 natural-log sum-exp of each row's scaled
 *           logits, or NULL
 * max_logit [H] fp32: per-head maximum of the scaled logit S over every
 *           unmasked (t, s' <= t) pair of every sequence. accumulate = 0 resets
 *           it first; accumulate = 1 folds this call into the values already
 *           there (max), e.g. across the micro-batches of a training step.
 * workspace at least mla_prefill_workspace_size(...) bytes.
 *
 * bf16: products in bf16 MFMA with fp32 accumulation, K^C and V rounded to
 * bf16 in the workspace, softmax in fp32, probabilities rounded to bf16 for
 * the value product. max_logit is refined: the rows whose streamed row
 * maximum lies within twice the bound of the bf16 rounding of K^C below the
 * head's streamed maximum have every logit re-scored in fp32 against q_abs =
 * W_UK q^C carried to about 16 significant bits, so the result is the exact
 * maximum up to fp32 rounding. A head with more than 64 such rows (near-ties:
 * q = 0, repeated queries) takes the streamed maximum instead, within
 * (1.01 * 2^-8 + 3e-5) * max|q| * max|K| * scale of the exact one.
 * fp32: fp32 throughout.
 */
mla_status mla_prefill(const mla_dims* dims, mla_dtype in_dtype, mla_dtype out_dtype,
                       const void* q, const void* ckv, const void* ks,
                       const void* w_kv_b, const void* gate, const mla_qk_norm* q_norm,
                       const int32_t* cu_seqlens, int32_t nseq, int64_t total_tokens,
                       void* out, float* lse, float* max_logit, int32_t accumulate,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of scratch memory mla_prefill_backward needs (0 for invalid sizes):
 * O(total_tokens * heads), independent of the sequence lengths. */
size_t mla_prefill_backward_workspace_size(const mla_dims* dims, int64_t total_tokens, int32_t nseq);

/*
 * Backward of mla_prefill (bf16, Kimi K3 head shape): the gradients of the
 * "Kimi K3 · Gated MLA" equation list ([k^C v] = c^KV W_UKV, K_h = [K^C_h,
 * k^S], S = Q K^T / sqrt(192), causal softmax, O~ = A V, o = sigma(g) . o~)
 * for an upstream gradient dout of o:
 *   dO~ = dout . sigma(g), dgate = dout . o . (1 - sigma(g)),
 *   per head and sequence: dV = P^T dO~, dS = P . (dO~ V^T - rowsum(dout . o)),
 *   dq = scale dS K, dK = scale dS^T Q;
 *   dckv = sum_h [dK^C_h | dV_h] [W_UK_h; W_UV_h], dw_kv_b = [dK^C | dV]^T c^KV,
 *   dks = sum_h of the k^S part of dK.
 * P is recomputed tile by tile from the forward's lse (no L x L buffer); the
 * call only enqueues work on the stream (nothing is read back to the host).
 *
 * q, ckv, ks, w_kv_b, gate: the forward's bf16 inputs (gate may be NULL);
 * cu_seqlens [nseq+1] int32 in DEVICE memory: non-decreasing from 0 to
 * total_tokens (as for mla_prefill; every token belongs to one sequence);
 * out [T, H*V] and lse [H, T] fp32 from mla_prefill; dout [T, H*V] fp32.
 * Outputs (fp32, device, fully overwritten): dq [T, H, N+S], dckv [T, R],
 * dks [T, S], dw_kv_b [H*(N+V), R], dgate [T, H*V] (required when gate is
 * given). total_tokens at most 2^20.
 */
mla_status mla_prefill_backward(const mla_dims* dims, const void* q, const void* ckv, const void* ks,
                                const void* w_kv_b, const void* gate, const int32_t* cu_seqlens,
                                int32_t nseq, int64_t total_tokens, const float* out, const float* lse,
                                const float* dout, float* dq, float* dckv, float* dks, float* dw_kv_b,
                                float* dgate, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Inference form (absorbed W_UK / W_UV over the latent cache)              */
/* ------------------------------------------------------------------------ */

/* Bytes of scratch memory mla_absorbed needs for these sizes (0 for invalid
 * sizes). */
size_t mla_absorbed_workspace_size(const mla_dims* dims, mla_dtype in_dtype,
                                   int32_t batch, int32_t tq);

/*
 * Absorbed-form gated MLA: the same result as mla_prefill for the last `tq`
 * positions of each sequence, computed from the latent cache without
 * materialising K or V ("Kimi Qkclip": the inference form skips the K
 * up-projection; "Gated MLA et NoPE": the cache holds 512 + 64 values per token).
 * By associativity of the equations:
 *   q~_h = W_UK_h q^C_h (length R), q_abs = [q~_h, q^R_h] (length R+S),
 *   s_j = scale * q_abs . cache[b, j],  j over the visible rows,
 *   o_lat = sum_j softmax(s)_j c^KV_j,  O~_h = o_lat W_UV_h,  out = sigma(g) . O~.
 * The tq queries of sequence b are its last tq positions: query i sees rows
 * j <= lens[b] - tq + i. The scale is the training form's.
 *
 * q         [batch, tq, H, N+S]     in_dtype
 * cache     [batch, cap, R+S]       in_dtype, rows [c^KV | k^S]; rows at or
 *           beyond lens[b] are never read (they may hold anything, NaN included)
 * lens      [batch] int32, device; tq <= lens[b] <= cap (not checked on the
 *           device; a violation gives undefined results)
 * w_kv_b    [H*(N+V), R]            in_dtype
 * gate      [batch, tq, H*V]        in_dtype, or NULL
 * q_norm    the QK-norm variant (see mla_qk_norm), or NULL
 * out       [batch, tq, H*V]        out_dtype
 * max_logit [H] fp32, as for mla_prefill (over every visible (query, row) pair).
 *
 * bf16: q_abs is rounded to bf16 for the MFMA products; the softmax, the
 * split-K partials and their log-sum-exp merge stay in fp32. max_logit is
 * refined: with the rounding of q_abs bounded per 32-row tile (by the
 * tile's largest row norm), every tile that could hold the head's exact
 * maximum is re-scored in fp32 against q_abs carried to about 16 significant
 * bits, so the result is the exact maximum up to fp32 rounding. Where more
 * tiles tie within that bound than the refinement lists (q = 0, repeated
 * rows), it re-scores the rows of the split ranges concerned directly: the
 * same result, reached more slowly.
 * cap is at most 2^31 - 1.
 */
mla_status mla_absorbed(const mla_dims* dims, mla_dtype in_dtype, mla_dtype out_dtype,
                        const void* q, const void* cache, int64_t cap,
                        const int32_t* lens, int32_t batch, int32_t tq,
                        const void* w_kv_b, const void* gate, const mla_qk_norm* q_norm,
                        void* out, float* max_logit, int32_t accumulate,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mla_absorbed for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * arguments and the result are those of mla_absorbed without the workspace;
 * its kernels (the same ones) take their scratch memory from a static device
 * array of 128 MiB built into the library instead. Each GPU the library runs
 * on holds its own copy of that array until the process ends. The call makes
 * no device allocation and no allocating library call.
 *
 * Limit: the call succeeds only when mla_absorbed_workspace_size(dims,
 * in_dtype, batch, tq) <= 128 MiB (for Kimi K3's 96 heads, batch * tq up to
 * about 170; 64 single-token sequences need about 90 MB); larger sizes return
 * MLA_ERR_UNSUPPORTED before anything is launched.
 *
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (the kernels set up everything they read in each call, so no state
 * carries over). Calls that overlap on one GPU (on different streams, or from
 * several host threads without ordering) race on the array and give
 * undefined results; calls ordered on one stream are safe.
 */
mla_status mla_absorbed_noalloc(const mla_dims* dims, mla_dtype in_dtype, mla_dtype out_dtype,
                                const void* q, const void* cache, int64_t cap,
                                const int32_t* lens, int32_t batch, int32_t tq,
                                const void* w_kv_b, const void* gate, const mla_qk_norm* q_norm,
                                void* out, float* max_logit, int32_t accumulate, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Expanded-cache decode (per-head K and V rows; bandwidth comparator)       */
/* ------------------------------------------------------------------------ */

/* Bytes of scratch memory mla_expanded needs for these sizes (0 for invalid
 * sizes). */
size_t mla_expanded_workspace_size(const mla_dims* dims, mla_dtype in_dtype,
                                   int32_t batch, int32_t tq, int64_t cap);

/*
 * The result of mla_absorbed, read from a cache that keeps every token's
 * materialised per-head key K_h = [K^C_h, k^S] and value V_h (the training
 * form's "[k^C v] = c^KV W_UKV", "K_h = [K^C_h k^S]" of "Kimi K3 · Gated MLA"),
 * instead of the single latent row of "Gated MLA et NoPE". Per token it reads
 * H*(N+S+V)*2 bytes (61,440 for Kimi K3) against the latent row's (R+S)*2
 * (1,152): it exists to measure that difference.
 *   s_j = scale * q[b, i, h] . k_cache[b, h, j],  j <= lens[b] - tq + i,
 *   O~_h = sum_j softmax(s)_j v_cache[b, h, j],  out = sigma(g) . O~.
 *
 * q         [batch, tq, H, N+S]     bf16
 * k_cache   [batch, H, cap, N+S]    bf16, per head K^C_h then k^S
 * v_cache   [batch, H, cap, V]      bf16
 *           rows at or beyond lens[b] are never read (they may hold anything)
 * lens      [batch] int32, device; tq <= lens[b] <= cap (not checked on the
 *           device; a violation gives undefined results)
 * gate      [batch, tq, H*V]        bf16, or NULL
 * out       [batch, tq, H*V]        out_dtype
 * max_logit [H] fp32, as for mla_prefill (over every visible (query, row)
 *           pair; scores in fp32 from the bf16 inputs).
 * bf16 only, Kimi K3 head shape; cap at most 2^27.
 */
mla_status mla_expanded(const mla_dims* dims, mla_dtype in_dtype, mla_dtype out_dtype,
                        const void* q, const void* k_cache, const void* v_cache, int64_t cap,
                        const int32_t* lens, int32_t batch, int32_t tq,
                        const void* gate, void* out, float* max_logit, int32_t accumulate,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* The whole attention layer ("Kimi K3 · Gated MLA", all 20 steps) and its    */
/* building blocks                                                           */
/* ------------------------------------------------------------------------ */

/*
 * nn.Linear without bias, as every projection of the layer: y = x W^T.
 * x [m, k], w [n, k] (weight [out, in]), y [m, n]; bf16, fp32 accumulation,
 * one rounding to bf16. k a multiple of 128 (at most 65536), n a multiple of 8.
 */
mla_status mla_linear(mla_dtype dtype, const void* x, int64_t m, int32_t k, const void* w, int32_t n,
                      void* y, hipStream_t stream);

/*
 * RMSNorm over rows of n features: y = x / sqrt(mean(x^2) + eps) * weight.
 * The pages name KimiRMSNorm (q_a_layernorm, kv_a_layernorm) without printing
 * it; this is the standard definition, with eps a parameter. x, y [rows, n],
 * weight [n]; bf16 with fp32 arithmetic and one rounding. n a multiple of 8,
 * at most 2048.
 */
mla_status mla_rms_norm(mla_dtype dtype, const void* x, int64_t rows, int32_t n, const void* weight, float eps,
                        void* y, hipStream_t stream);

/* Bytes of scratch memory mla_layer_forward needs (0 for invalid sizes). */
size_t mla_layer_workspace_size(const mla_dims* dims, int32_t hidden, int32_t q_rank,
                                int64_t total_tokens, int32_t nseq);

/*
 * Delta_attn of the gated MLA layer for packed sequences, the equation list of
 * "Kimi K3 · Gated MLA" end to end with the KimiMLAAttention projections:
 *   c^Q = x W_DQ (q_a_proj), c^Q^ = RMSNorm(c^Q) (q_a_layernorm),
 *   q = c^Q^ W_UQ (q_b_proj), [c^KV | k^S] = x W_DKV (kv_a_proj_with_mqa),
 *   c^KV^ = RMSNorm(c^KV) (kv_a_layernorm), g = x W_g (g_proj),
 *   o = sigma(g) . causal attention (as mla_prefill), Delta = o W_O (o_proj).
 * Every activation between the steps is kept in bf16 (the model's dtype);
 * products accumulate in fp32.
 *
 * x       [total_tokens, hidden]        w_dq   [q_rank, hidden]   g_q  [q_rank]
 * w_uq    [H*(N+S), q_rank]             w_kv_a [R+S, hidden]      g_kv [R]
 * w_kv_b  [H*(N+V), R]                  w_g    [H*V, hidden]      w_o  [hidden, H*V]
 * out     [total_tokens, hidden]        all bf16; cu_seqlens and max_logit as mla_prefill.
 * Kimi K3 head shape; hidden a multiple of 128 (at most 65536), q_rank a
 * multiple of 128 (at most 2048).
 */
mla_status mla_layer_forward(const mla_dims* dims, int32_t hidden, int32_t q_rank, float eps,
                             const void* x, const void* w_dq, const void* g_q, const void* w_uq,
                             const void* w_kv_a, const void* g_kv, const void* w_kv_b,
                             const void* w_g, const void* w_o,
                             const int32_t* cu_seqlens, int32_t nseq, int64_t total_tokens,
                             void* out, float* max_logit, int32_t accumulate,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* QK-Clip ("SOTA-131": rescale the query and key projection weights of every
 * head whose maximum logit exceeds tau)                                     */
/* ------------------------------------------------------------------------ */

/*
 * gamma_h = tau / max_logit[h] if max_logit[h] > tau, else 1 (and the head is
 * left bit-for-bit unchanged). For a clipped head, in place:
 *   w_q_b  rows h*D .. h*D+N-1      (q^C_h)  *= sqrt(gamma_h)
 *   w_q_b  rows h*D+N .. h*D+D-1    (q^R_h)  *= gamma_h
 *   w_kv_b rows h*(N+V) .. +N-1     (W_UK_h) *= sqrt(gamma_h)
 * so every logit of head h becomes gamma_h times its old value. The shared
 * k^S projection is not an argument (it is shared by all heads and stays
 * untouched) and the W_UV_h rows are not written.
 * Products are formed in fp32 and rounded to nearest-even into wdtype.
 *
 * w_q_b     [H*D, q_in]   wdtype, in place
 * w_kv_b    [H*(N+V), R]  wdtype, in place
 * max_logit [H] fp32 (device), tau > 0 (finite)
 * clipped   [H] uint8 (1 = rescaled) or NULL;  gamma [H] fp32 or NULL
 */
mla_status mla_qk_clip(const mla_dims* dims, mla_dtype wdtype,
                       void* w_q_b, int32_t q_in, void* w_kv_b,
                       const float* max_logit, float tau,
                       uint8_t* clipped, float* gamma, hipStream_t stream);

/* ------------------------------------------------------------------------ */

const char* mla_status_string(mla_status status);
/* Detail of the last error returned on the calling thread ("" if none). */
const char* mla_last_error(void);
/* Library version string. */
const char* mla_version(void);

/*
 * Optional per-kernel timing (tracing aid; not part of the computation).
 * mla_timing_enable(1) clears the totals and from then on brackets every
 * kernel launch with a pair of HIP events recorded on the caller's stream;
 * mla_timing_enable(0) stops it. mla_timing_read waits for the recorded
 * events and returns the summed milliseconds and launch count of one kernel
 * ("prefill_expand", "prefill_attn", "absorb_q", "absorbed_split",
 * "absorbed_finish", "expanded_split", "qk_clip", ...); it returns 0 if that kernel has not
 * run. This is the library's one piece of process-global host state (the
 * pending events and the per-kernel totals, behind a mutex): it is off by
 * default, changes no result, and while on, the events it creates are the
 * only HIP objects the library creates. Intended for one thread at a time.
 */
void mla_timing_enable(int32_t on);
int32_t mla_timing_read(const char* kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
