/*
 * mla.h -- C ABI of the MI355X (gfx950) weight-absorbed Multi-head Latent
 * Attention library (libmla.so).
 *
 * What it computes (notation of the pages this library follows):
 *   The cache holds one row per position, [c_t | k_pe_t]: the RMS-normed
 *   latent c_t (d_c wide) followed by the roped rope key k_pe_t (d_r wide)
 *   (docs.rs ferrox-core 0.23.0, src/mla_absorbed.rs: documentation of
 *   `causal_mla_absorbed_attention`, llama.cpp's concat(kv_cmpr, k_pe) order).
 *   A query row is [q_abs | q_pe] with q_abs = W_UK[h]^T q_nope[h] (same page,
 *   module documentation; MLA_tutorial formula.md Part 3, inference form).
 *   Every head scores against the SAME key row and sums the SAME value c_t:
 *     score[h][t] = (q_abs[h].c_t + q_pe[h].k_pe_t) * kq_scale
 *     out_lat[h]  = sum_t softmax_t(score[h]) c_t         (d_c wide)
 *     v[h]        = W_UV[h] out_lat[h]                     (d_v wide)
 *   kq_scale is the caller's 1/sqrt(d_nope + d_r): the width of the
 *   unabsorbed head, never the latent width (ferrox-core module doc).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers to caller-owned memory, row-major
 *     and contiguous in the innermost dimension. The library never
 *     allocates, frees or synchronises the host in these calls; scratch for
 *     split-sequence partial results comes from the caller's workspace.
 *   - Inputs are never written (the gated-MLA problem statement requires
 *     the inputs to stay unchanged); every element of every output is written.
 *   - All tensors of one call share `dtype` (MLA_F32 or MLA_BF16);
 *     accumulation is fp32; outputs are in `dtype`; lse outputs are fp32.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously. Calls keep no state between them apart from
 *     a cached per-device compute-unit count.
 *   - Errors are returned as negative status codes BEFORE any launch for
 *     argument problems; MLA_ERR_HIP reports a failed launch. A call that
 *     returns an error has enqueued nothing, except MLA_ERR_HIP, after which
 *     the state of the outputs is unspecified.
 *   - Size arguments of value 0 in a batch-like dimension (tokens, batch,
 *     query rows) are valid and do nothing; the call's pointers are then
 *     not checked (empty tensors may have NULL data).
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL                         */
  MLA_ERR_SHAPE = -2,       /* a size is negative, zero where it must be positive,
                               or sizes are inconsistent with each other          */
  MLA_ERR_DTYPE = -3,       /* dtype is neither MLA_F32 nor MLA_BF16              */
  MLA_ERR_UNSUPPORTED = -4, /* sizes beyond the library's limits (see each call)  */
  MLA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than the query returns   */
  MLA_ERR_ALIGN = -6,       /* a pointer not aligned to its element size          */
  MLA_ERR_SCALE = -7,       /* kq_scale is not a finite number                    */
  MLA_ERR_HIP = -8          /* a HIP runtime call or kernel launch failed          */
};

/* Text for a status code (static storage; never NULL). */
const char* mla_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int mla_version(void);

/* Default worker count used when num_workers == 0: the compute-unit count of
 * the current HIP device (one attention workgroup per compute unit).
 * Returns a negative status if no device is available. */
int mla_default_workers(void);

/* ---------------------------------------------------------------------------
 * Query absorption (ferrox-core test, absorbed branch: the query pushed
 * through k_b; lab "MLA math exercise" Bloque B identity
 * q^T W_UK c = (W_UK^T q)^T c; MLA_tutorial inference form q W_qc W_kc^T):
 *   q[n,h,j]       = sum_i W_UK[h,i,j] * q_nope[n,h,i]   for j < d_c
 *   q[n,h,d_c + k] = q_pe[n,h,k]                         for k < d_r
 * q_nope [n_tokens, n_heads, d_nope]; q_pe [n_tokens, n_heads, d_r] (may be
 * NULL only when d_r == 0); w_uk [n_heads, d_nope, d_c] (the k_b rows of
 * kv_b); q [n_tokens, n_heads, d_c + d_r] (output).
 * Limits: n_heads <= 65535, d_nope, d_c <= 4096, d_r <= 1024.
 * ------------------------------------------------------------------------- */
int mla_absorb_q(const void* q_nope, const void* q_pe, const void* w_uk, void* q,
                 int64_t n_tokens, int n_heads, int d_nope, int d_c, int d_r,
                 int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Value up-projection after the latent attention (ferrox-core module doc
 * v[h] = wv_b[h] . out_lat[h]; MLA_tutorial inference form o^(s) W_v^(s)):
 *   out[n,h,i] = sum_j W_UV[h,i,j] * out_lat[n,h,j]
 * out_lat [n_tokens, n_heads, d_c]; w_uv [n_heads, d_v, d_c] (the v_b rows
 * of kv_b); out [n_tokens, n_heads, d_v].
 * Limits: n_heads <= 65535, d_c, d_v <= 4096.
 * ------------------------------------------------------------------------- */
int mla_up_v(const void* out_lat, const void* w_uv, void* out,
             int64_t n_tokens, int n_heads, int d_c, int d_v, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Absorbed decode: one query token per sequence attends to its sequence's
 * latent cache (ferrox-core `causal_mla_absorbed_attention`, generalised to
 * a batch, a dense or paged cache and split-sequence execution).
 *   q            [batch, n_heads, d_c + d_r]  rows [q_abs | q_pe]
 *   latent_cache dense (block_table == NULL): [batch, cache_stride, d_c + d_r];
 *                paged: a pool [num_pages, page_size, d_c + d_r]
 *   seq_lens     [batch] int32, DEVICE memory: positions 0..len-1 attend.
 *                Values are clamped to [0, cache_stride] (dense) or
 *                [0, max_pages * page_size] (paged) before use.
 *   block_table  [batch, max_pages] int32, DEVICE memory, or NULL for dense.
 *                Entry (b, j) is the pool page of positions j*page_size ..;
 *                entries are clamped to [0, num_pages - 1] before use.
 *   out_lat      [batch, n_heads, d_c] output (the weighted sum of c_t, before W_UV)
 *   lse          [batch, n_heads] fp32 output (natural-log softmax
 *                normaliser, max included), or NULL.
 * A sequence of length 0 yields out_lat = 0 and lse = -inf (the empty-sum
 * guard of `causal_mla_absorbed_attention`).
 * workspace / workspace_bytes: device scratch of at least
 *   mla_latent_decode_workspace(batch, n_heads, d_c, num_workers) bytes;
 *   contents on entry are ignored. Concurrent calls need separate workspaces.
 * num_workers: attention workgroups to launch (0 = mla_default_workers(),
 *   at most 65535). Results do not depend on it beyond floating-point rounding.
 * timing_events: NULL, or a pointer to two hipEvent_t passed with the
 *   attention kernel's launch on `stream`: they take the start and end times
 *   of its dispatch (for profiling; the planning and combine kernels fall
 *   outside them).
 * Limits: d_c <= 1024, d_c + d_r <= 1152, n_heads <= 65535,
 *   page_size >= 1 when paged, batch * (ceil(cap / 16) + 12) <= 2^30 - 1
 *   with cap = cache_stride (dense) or max_pages * page_size (paged): the
 *   split plan counts 16-position tiles plus a fixed cost per row in int32.
 * ------------------------------------------------------------------------- */
size_t mla_latent_decode_workspace(int batch, int n_heads, int d_c, int num_workers);

int mla_latent_decode(const void* q, const void* latent_cache,
                      const int32_t* seq_lens, const int32_t* block_table,
                      int batch, int n_heads, int d_c, int d_r,
                      int cache_stride, int page_size, int max_pages, int num_pages,
                      float kq_scale, int dtype,
                      void* out_lat, float* lse,
                      void* workspace, size_t workspace_bytes,
                      int num_workers, void* const* timing_events, void* stream);

/* ---------------------------------------------------------------------------
 * Allocation-free absorbed decode, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Computes exactly what mla_latent_decode computes, with
 * the same kernels and results, but takes no workspace: the split plan and
 * the partial results live in a fixed scratch array inside the library, one
 * per device (MLA_NOALLOC_SCRATCH_BYTES = 66 MiB, taken when the library's
 * code is loaded on the device and held until the process ends). The call
 * allocates nothing and calls no allocating routine.
 *   Arguments as mla_latent_decode, without workspace / workspace_bytes /
 *   timing_events.
 *   Every call on a device shares that device's scratch: calls that may
 *   overlap on one device (other streams, other threads) race and must be
 *   serialised by the caller. Nothing in the scratch needs clearing between
 *   calls: every value a kernel of the call reads is written earlier in the
 *   same call.
 *   Returns MLA_ERR_UNSUPPORTED, before any launch, when the call needs more
 *   than the scratch holds: mla_latent_decode_noalloc_scratch_bytes(batch,
 *   n_heads, d_c, dtype, num_workers) gives the need (bf16 at 256 workers,
 *   128 heads, d_c = 512 takes about 64.3 MiB, which fits up to some two
 *   hundred thousand sequences; fp32 needs twice the partial region).
 * ------------------------------------------------------------------------- */
#define MLA_NOALLOC_SCRATCH_BYTES (66u << 20)

size_t mla_latent_decode_noalloc_scratch_bytes(int batch, int n_heads, int d_c, int dtype, int num_workers);

int mla_latent_decode_noalloc(const void* q, const void* latent_cache,
                              const int32_t* seq_lens, const int32_t* block_table,
                              int batch, int n_heads, int d_c, int d_r,
                              int cache_stride, int page_size, int max_pages, int num_pages,
                              float kq_scale, int dtype,
                              void* out_lat, float* lse,
                              int num_workers, void* stream);

/* ---------------------------------------------------------------------------
 * Absorbed decode followed by the value up-projection, in one call (ferrox-
 * core module documentation: v[h] = wv_b[h] . out_lat[h]; the chain
 * mla_latent_decode -> mla_up_v without storing out_lat):
 *   out [batch, n_heads, d_v] = W_UV[h] out_lat[b, h] for every (b, h), with
 *   out_lat the result mla_latent_decode computes (rounded to dtype first);
 *   w_uv [n_heads, d_v, d_c] as in mla_up_v; lse as in mla_latent_decode.
 * All other arguments as mla_latent_decode. workspace: at least
 *   mla_latent_decode_up_v_workspace(batch, n_heads, d_c, num_workers)
 *   bytes (the decode workspace plus room for out_lat). When the attention
 *   runs on its bf16 MFMA kernel (d_c = 512, d_r = 64, n_heads a multiple of
 *   32 up to 128, page_size a multiple of 16, 16-byte aligned q, cache, w_uv
 *   and out) and d_v = 128, the merge of split rows and the up-projection
 *   run as one kernel; otherwise the call runs decode, combine and
 *   up-projection. Results agree either way up to rounding order.
 * Limits: as mla_latent_decode and mla_up_v (d_v <= 4096).
 * ------------------------------------------------------------------------- */
size_t mla_latent_decode_up_v_workspace(int batch, int n_heads, int d_c, int num_workers);

int mla_latent_decode_up_v(const void* q, const void* latent_cache,
                           const int32_t* seq_lens, const int32_t* block_table,
                           int batch, int n_heads, int d_c, int d_r,
                           int cache_stride, int page_size, int max_pages, int num_pages,
                           float kq_scale, const void* w_uv, int d_v, int dtype,
                           void* out, float* lse,
                           void* workspace, size_t workspace_bytes,
                           int num_workers, void* const* timing_events, void* stream);

/* ---------------------------------------------------------------------------
 * Causal prefill over the latent cache: every query of a chunk attends to
 * the cache positions the causal mask leaves visible (gated-MLA statement:
 * later positions are masked before the softmax, diagonal included;
 * MLA_tutorial: sums over i <= t). Alignment is bottom-right: query i
 * (0-based, of s_q) sees positions t <= i + s_kv - s_q.
 *   q            [batch, s_q, n_heads, d_c + d_r]
 *   latent_cache [batch, s_kv, d_c + d_r]
 *   out_lat      [batch, s_q, n_heads, d_c]; lse [batch, s_q, n_heads] or NULL.
 * Queries that see no position (s_q > s_kv) get zeros and lse = -inf.
 * workspace: at least mla_latent_prefill_causal_workspace(batch, s_q,
 *   n_heads, d_c, num_workers) bytes. num_workers, timing_events: as decode.
 * Limits: as decode, with batch * s_q rows of cap = s_kv positions;
 *   batch * s_q <= 2^31 - 1.
 * ------------------------------------------------------------------------- */
size_t mla_latent_prefill_causal_workspace(int batch, int s_q, int n_heads, int d_c, int num_workers);

int mla_latent_prefill_causal(const void* q, const void* latent_cache,
                              int batch, int s_q, int s_kv, int n_heads, int d_c, int d_r,
                              float kq_scale, int dtype,
                              void* out_lat, float* lse,
                              void* workspace, size_t workspace_bytes,
                              int num_workers, void* const* timing_events, void* stream);

/* ---------------------------------------------------------------------------
 * Log-sum-exp merge of softmax results computed over disjoint position
 * ranges of the same queries (the split-sequence combine step; it is the
 * identity softmax over a union of ranges satisfies, not a formula of the
 * pages):
 *   lse[r,h]   = log sum_p exp(lse_parts[p,r,h])
 *   out[r,h,:] = sum_p exp(lse_parts[p,r,h] - lse[r,h]) * o_parts[p,r,h,:]
 * o_parts [n_parts, rows, n_heads, d_c] fp32, each normalised over its own
 * range; lse_parts [n_parts, rows, n_heads] fp32. Parts with lse = -inf
 * (empty ranges) are skipped and their o_parts values never read; if all
 * are -inf the output is 0 and lse -inf. out [rows, n_heads, d_c] in
 * `dtype`; lse [rows, n_heads] fp32 or NULL.
 * Limits: 1 <= n_parts <= 4096, d_c <= 4096, n_heads <= 65535.
 * ------------------------------------------------------------------------- */
int mla_lse_combine(const float* o_parts, const float* lse_parts, int n_parts,
                    int64_t rows, int n_heads, int d_c, int dtype,
                    void* out, float* lse, void* stream);

/* ===========================================================================
 * The steps around the core path
 * ========================================================================= */

/* ---------------------------------------------------------------------------
 * Fused cache append: the new tokens' latent rows written straight into the
 * cache. Per token n (MLA_tutorial formula.md Part 3, training form: the
 * latent c = x W_c and the rope key x W_kr R_i, taken from x and not from c;
 * ferrox-core module documentation: the cached latent is RMS-normed and the
 * rope key roped; notebook MLA_RoPE-less.ipynb, cache update: the new row is
 * appended before the query attends, so the token sees itself):
 *   z   = W_c x_n                      (w_c  [d_c, d_model], a row per latent dim)
 *   c   = z / sqrt(mean(z^2) + eps) * gain      (gain [d_c] or NULL = 1)
 *   kr  = W_kr x_n                     (w_kr [d_r, d_model])
 *   k_pe = kr with pair (2i, 2i+1) turned by positions[n] * rope_base^(-2i/d_r)
 *   row [c | k_pe] written at sequence seq_ids[n], position positions[n]:
 *     dense  (block_table NULL): latent_cache[seq][pos], [n_seqs, cache_stride, d_c + d_r];
 *     paged: pool page block_table[seq][pos / page_size], slot pos % page_size.
 * x [n_tokens, d_model]; seq_ids, positions [n_tokens] int32 DEVICE memory.
 * latent_cache is the one buffer written (only the addressed rows); a token
 * whose sequence, position or page falls outside the cache is skipped.
 * Rotation angles are formed in double precision on the device.
 * workspace: mla_cache_append_workspace(n_tokens, d_model, d_c, d_r, dtype)
 *   bytes (fp32 partial projections).
 * Status: MLA_ERR_SCALE for eps < 0, a non-finite eps or rope_base <= 0.
 * Limits: d_model <= 65536, d_c <= 4096, d_r <= 1024 and even, d_c + d_r <= 5120.
 * ------------------------------------------------------------------------- */
size_t mla_cache_append_workspace(int n_tokens, int d_model, int d_c, int d_r, int dtype);

int mla_cache_append(const void* x, const void* w_c, const void* w_kr, const void* gain,
                     float eps, float rope_base,
                     const int32_t* seq_ids, const int32_t* positions,
                     void* latent_cache, const int32_t* block_table,
                     int n_seqs, int cache_stride, int page_size, int max_pages, int num_pages,
                     int n_tokens, int d_model, int d_c, int d_r, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Query absorption with the query's rope part rotated on the way (the query
 * side of the fused append; MLA_tutorial inference form: q = [c' W_qc W_kc^T,
 * c' W_qr R_i]):
 *   q[n,h,:d_c] as mla_absorb_q;  q[n,h,d_c:] = q_pe[n,h,:] turned by
 *   positions[n] as in mla_cache_append (same angles).
 * positions [n_tokens] int32 DEVICE memory. d_r > 0 and even.
 * ------------------------------------------------------------------------- */
int mla_absorb_q_rope(const void* q_nope, const void* q_pe, const void* w_uk,
                      const int32_t* positions, float rope_base, void* q,
                      int64_t n_tokens, int n_heads, int d_nope, int d_c, int d_r,
                      int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Unabsorbed causal prefill: keys and values expanded per head, then
 * standard softmax attention (MLA_tutorial formula.md Part 3, training form:
 * k[t,h] = [W_UK[h] c_t | k_pe_t], v[t,h] = W_UV[h] c_t, the rope key shared
 * by all heads; its closing remarks: absorption widens the head to d_c + d_r,
 * so the expanded form is the cheaper one where the work is compute-bound).
 *   out[b,i,h,:] = sum_t softmax_t(([q_nope | q_pe][b,i,h] . k[b,t,h]) kq_scale) v[b,t,h]
 * over t <= i + s_kv - s_q (bottom-right causal alignment), i.e. the same
 * result as mla_absorb_q -> mla_latent_prefill_causal -> mla_up_v.
 * q_nope [batch, s_q, n_heads, d_nope], q_pe [batch, s_q, n_heads, d_r];
 * latent_cache [batch, s_kv, d_c + d_r]; w_uk [n_heads, d_nope, d_c];
 * w_uv [n_heads, d_v, d_c]; out [batch, s_q, n_heads, d_v]; lse
 * [batch, s_q, n_heads] fp32 or NULL (queries that see nothing: 0, -inf).
 * workspace: mla_prefill_unabsorbed_workspace(batch, s_kv, n_heads, d_nope,
 *   d_v) bytes (the expanded keys and values).
 * Supported: bf16, d_nope = d_v = 128, d_r 0 or 64, d_c a multiple of 64 up
 * to 4096, 16-byte aligned tensors; anything else is MLA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
size_t mla_prefill_unabsorbed_workspace(int batch, int s_kv, int n_heads, int d_nope, int d_v);

int mla_prefill_unabsorbed(const void* q_nope, const void* q_pe, const void* latent_cache,
                           const void* w_uk, const void* w_uv,
                           int batch, int s_q, int s_kv, int n_heads, int d_nope, int d_c, int d_r,
                           int d_v, float kq_scale, int dtype, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Full absorption (notebook MLA_RoPE-less.ipynb: matrix absorption and the
 * sum over heads; MLA_tutorial inference form: c' W_qc W_kc^T).
 * Weights: w_uq [n_heads, d_nope, d_cq] (q_nope[h] = W_UQ[h] c', c' the
 * query latent), w_uk [n_heads, d_nope, d_c], w_uv [n_heads, d_v, d_c],
 * w_o [d_model, n_heads * d_v] (layer output = sum_h W_O[:, h block] v[h]).
 * mla_absorb_weights writes (once per weight set):
 *   a_qk [n_heads, d_c, d_cq],   a_qk[h] = W_UK[h]^T W_UQ[h]
 *   a_vo [d_model, n_heads * d_c], columns h*d_c.. = W_O[:, h block] W_UV[h]
 * workspace: mla_absorb_weights_workspace(...) bytes (transposed copies).
 * ------------------------------------------------------------------------- */
size_t mla_absorb_weights_workspace(int n_heads, int d_nope, int d_cq, int d_c, int d_v, int dtype);

int mla_absorb_weights(const void* w_uq, const void* w_uk, const void* w_uv, const void* w_o,
                       int n_heads, int d_nope, int d_cq, int d_c, int d_v, int d_model, int dtype,
                       void* a_qk, void* a_vo, void* workspace, size_t workspace_bytes, void* stream);

/* Absorbed query straight from the query latent:
 *   q[n,h,:d_c] = a_qk[h] c_q[n];  q[n,h,d_c:] = q_pe[n,h,:], turned by
 *   positions[n] as in mla_absorb_q_rope when positions is not NULL.
 * c_q [n_tokens, d_cq]; q [n_tokens, n_heads, d_c + d_r]. */
int mla_absorb_q_full(const void* c_q, const void* q_pe, const void* a_qk,
                      const int32_t* positions, float rope_base, void* q,
                      int64_t n_tokens, int n_heads, int d_cq, int d_c, int d_r, int dtype, void* stream);

/* Layer output straight from the latent attention output, summed over heads:
 *   out[n,:] = a_vo . concat_h(out_lat[n,h,:])   (the notebook's adding trick)
 * out_lat [n_tokens, n_heads, d_c]; out [n_tokens, d_model].
 * workspace: mla_out_absorbed_workspace(...) bytes (fp32 split partials). */
size_t mla_out_absorbed_workspace(int64_t n_tokens, int n_heads, int d_c, int d_model, int dtype);

int mla_out_absorbed(const void* out_lat, const void* a_vo, void* out,
                     int64_t n_tokens, int n_heads, int d_c, int d_model, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Gated MLA (tensortonic "Kimi K3 step 2: Gated MLA", problem statement):
 *   Q = X W_q^T, C = X W_c^T, K = C W_k^T, V = C W_v^T; per head of width
 *   D_h = d_model / n_heads: A = softmax(Q K^T / sqrt(D_h) + M), M masking
 *   later positions when causal != 0; O~ = heads side by side;
 *   Y = [sigmoid(X W_g^T) * O~] W_o^T.
 * x [batch, seq, d_model]; w_q, w_g, w_o [d_model, d_model]; w_c [latent,
 * d_model]; w_k, w_v [d_model, latent]. Outputs: out [batch, seq, d_model]
 * and latent_cache [batch, seq, latent] (= C). No positional encoding.
 * bf16 with D_h = 128 runs per-head attention over the expanded keys and
 * values; every other case runs the absorbed form (q_abs[h] = W_k[h]^T q[h],
 * latent attention over C with C as the value, then W_v[h]) through the
 * latent-attention kernels. num_workers as mla_latent_decode (absorbed form).
 * workspace: mla_gated_mla_workspace(batch, seq, d_model, latent, n_heads,
 *   dtype, num_workers) bytes.
 * Limits: d_model divisible by n_heads, d_model <= 65536, latent <= 1024.
 * ------------------------------------------------------------------------- */
size_t mla_gated_mla_workspace(int batch, int seq, int d_model, int latent, int n_heads, int dtype,
                               int num_workers);

int mla_gated_mla(const void* x, const void* w_q, const void* w_c, const void* w_k, const void* w_v,
                  const void* w_g, const void* w_o, int batch, int seq, int d_model, int latent,
                  int n_heads, int causal, int dtype, void* out, void* latent_cache,
                  void* workspace, size_t workspace_bytes, int num_workers, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
