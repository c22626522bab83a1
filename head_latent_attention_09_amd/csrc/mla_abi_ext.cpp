// C ABI of libmla, the steps around the core path: the new token's cache row
// (fused append), the unabsorbed prefill, full absorption of the query and
// output projections, and the gated MLA variant. Argument validation runs
// before any launch, as in mla_abi.cpp.
#include <cmath>
#include <cstdint>

#include "mla_internal.h"

#include <initializer_list>

using namespace mla;

namespace {

constexpr int kCuRef = 256;  // compute units assumed when sizing split-K workspaces (MI355X)

#define MLA_TRY(x)                    \
  do {                                \
    const int st_ = (x);              \
    if (st_ != MLA_OK) return st_;    \
  } while (0)

GemmDesc gemm(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int M, int N, int K,
              int dtype) {
  GemmDesc g{};
  g.A = A;
  g.B = B;
  g.C = C;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.K = K;
  g.batch = 1;
  g.splits = 1;
  g.dtype = dtype;
  return g;
}

// split-K partial count of the cache-append projection (depends on sizes only)
int append_splits(int n_tokens, int d_model, int d_c, int dtype) {
  GemmDesc g = gemm((const void*)16, d_model, (const void*)16, d_model, (void*)16, d_c, n_tokens, d_c, d_model,
                    dtype);
  g.out_f32 = true;
  return gemm_nt_splits(g, kCuRef, 16);  // the row epilogue reads every split
}

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// out_absorbed: split count of out[N, d_model] = lat[N, H d_c] a_vo^T on the
// tiled product
int out_splits(int64_t n_tokens, int n_heads, int d_c, int d_model, int dtype) {
  GemmDesc g = gemm((const void*)16, (int64_t)n_heads * d_c, (const void*)16, (int64_t)n_heads * d_c, (void*)16,
                    d_model, (int)n_tokens, d_model, n_heads * d_c, dtype);
  g.out_f32 = true;
  return gemm_nt_splits(g, kCuRef);
}

// out_absorbed on the weight stream (at most 64 tokens): the same product with
// split-K partials; its split count never exceeds the tiled product's, so one
// workspace size serves both
StreamDesc out_stream(const void* out_lat, const void* a_vo, float* P, int64_t n_tokens, int n_heads, int d_c,
                      int d_model, int dtype) {
  StreamDesc d{};
  const int K = n_heads * d_c;
  d.X = out_lat;
  d.ldx = K;
  d.W = a_vo;
  d.ldw = K;
  d.P = P;
  d.p_split = n_tokens * d_model;
  d.M = (int)n_tokens;
  d.N = d_model;
  d.K = K;
  d.splits = 0;
  if (dtype != MLA_BF16 || n_tokens > 64) return d;
  const int cap = out_splits(n_tokens, n_heads, d_c, d_model, dtype);
  d.splits = stream_gemm_splits(d_model, K, kCuRef, cap);
  return d;
}

// The gated layer's products on 256 x 256 tiles: they pay off once they fill
// the chip (at least one tile per CU for an output of n rows and 2 d_model
// columns); contractions over d_model and the latent width in whole 64-wide
// slices, every operand 16-byte aligned (bf16 only, checked by the caller).
bool pair_fits(int64_t n, int d_model, int latent, std::initializer_list<const void*> ptrs) {
  if (n < 256 || (n / 256) * ((2 * (int64_t)d_model) / 256) < kCuRef) return false;
  if (d_model % 64 || latent % 64) return false;
  for (const void* p : ptrs)
    if ((uintptr_t)p & 15) return false;
  return true;
}

bool gated_flash_route(int d_model, int n_heads, int dtype) {
  return dtype == MLA_BF16 && d_model % n_heads == 0 && flash_fits(d_model / n_heads, 0, d_model / n_heads);
}

}  // namespace

extern "C" {

// ===========================================================================
// fused cache append
// ===========================================================================
size_t mla_cache_append_workspace(int n_tokens, int d_model, int d_c, int d_r, int dtype) {
  if (n_tokens < 0 || d_model <= 0 || d_c <= 0 || d_r < 0 || !abi_dtype_ok(dtype)) return 0;
  const int s = append_splits(n_tokens, d_model, d_c, dtype);
  return a256((size_t)s * n_tokens * (d_c + d_r) * sizeof(float)) + 256;
}

int mla_cache_append(const void* x, const void* w_c, const void* w_kr, const void* gain, float eps, float rope_base,
                     const int32_t* seq_ids, const int32_t* positions, void* latent_cache,
                     const int32_t* block_table, int n_seqs, int cache_stride, int page_size, int max_pages,
                     int num_pages, int n_tokens, int d_model, int d_c, int d_r, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!abi_dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (n_tokens < 0 || n_seqs < 0 || d_model <= 0 || d_c <= 0 || d_r < 0 || (d_r & 1)) return MLA_ERR_SHAPE;
  if (d_model > 65536 || d_c > 4096 || d_r > 1024 || d_c + d_r > 5120) return MLA_ERR_UNSUPPORTED;
  if (!std::isfinite(eps) || eps < 0.f || !std::isfinite(rope_base) || rope_base <= 0.f) return MLA_ERR_SCALE;
  if (n_tokens == 0) return MLA_OK;
  if (!x || !w_c || (d_r > 0 && !w_kr) || !seq_ids || !positions || !latent_cache) return MLA_ERR_NULL;
  const int es = abi_esize(dtype);
  if (!abi_aligned(x, es) || !abi_aligned(w_c, es) || (w_kr && !abi_aligned(w_kr, es)) ||
      (gain && !abi_aligned(gain, es)) || !abi_aligned(latent_cache, es) || !abi_aligned(seq_ids, 4) ||
      !abi_aligned(positions, 4) || (block_table && !abi_aligned(block_table, 4)))
    return MLA_ERR_ALIGN;
  RowMap map{};
  if (block_table) {
    if (page_size <= 0 || max_pages <= 0 || num_pages <= 0) return MLA_ERR_SHAPE;
    map.mode = 1;
    map.page_size = page_size;
    map.max_pages = max_pages;
    map.num_pages = num_pages;
    map.block_table = block_table;
  } else {
    if (cache_stride <= 0) return MLA_ERR_SHAPE;
    map.mode = 0;
    map.cache_stride = cache_stride;
  }
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (!abi_aligned(workspace, 256)) return MLA_ERR_ALIGN;
  if (workspace_bytes < mla_cache_append_workspace(n_tokens, d_model, d_c, d_r, dtype)) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int W = d_c + d_r;
  const int splits = append_splits(n_tokens, d_model, d_c, dtype);
  float* P = (float*)workspace;
  const int64_t sstride = (int64_t)n_tokens * W;
  // [z_c | z_r] = x [W_c ; W_kr]^T as fp32 partial sums (split over the model width): one
  // product reading W_c and W_kr as one weight where the MFMA path takes it, else two
  GemmDesc g = gemm(x, d_model, w_c, d_model, P, W, n_tokens, d_c, d_model, dtype);
  g.out_f32 = true;
  g.splits = splits;
  g.c_split = sstride;
  GemmDesc gf = g;
  gf.N = W;
  gf.B2 = w_kr;
  gf.n1 = d_c;
  const bool one = d_r > 0 && gemm_nt_mfma_ok(gf);
  MLA_TRY(launch_gemm_nt(one ? gf : g, s));
  if (d_r > 0 && !one) {
    GemmDesc gr = gemm(x, d_model, w_kr, d_model, P + d_c, W, n_tokens, d_r, d_model, dtype);
    gr.out_f32 = true;
    gr.splits = splits;
    gr.c_split = sstride;
    MLA_TRY(launch_gemm_nt(gr, s));
  }
  return launch_cache_rows(P, splits, sstride, gain, eps, rope_base, seq_ids, positions, latent_cache, map, n_seqs,
                           n_tokens, d_c, d_r, dtype, s);
}

int mla_absorb_q_rope(const void* q_nope, const void* q_pe, const void* w_uk, const int32_t* positions,
                      float rope_base, void* q, int64_t n_tokens, int n_heads, int d_nope, int d_c, int d_r,
                      int dtype, void* stream) {
  if (!abi_dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (n_tokens < 0 || n_heads <= 0 || d_nope <= 0 || d_c <= 0 || d_r <= 0 || (d_r & 1)) return MLA_ERR_SHAPE;
  if (n_heads > 65535 || d_nope > 4096 || d_c > 4096 || d_r > 1024) return MLA_ERR_UNSUPPORTED;
  if (!std::isfinite(rope_base) || rope_base <= 0.f) return MLA_ERR_SCALE;
  if (n_tokens == 0) return MLA_OK;
  if (!q_nope || !q_pe || !w_uk || !positions || !q) return MLA_ERR_NULL;
  const int es = abi_esize(dtype);
  if (!abi_aligned(q_nope, es) || !abi_aligned(q_pe, es) || !abi_aligned(w_uk, es) || !abi_aligned(q, es) ||
      !abi_aligned(positions, 4))
    return MLA_ERR_ALIGN;
  if (n_tokens * (int64_t)n_heads * (d_c + d_r) > ((int64_t)1 << 40)) return MLA_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  // absorbed part without the tail copy, then the rotated tail
  MLA_TRY(launch_absorb(q_nope, nullptr, w_uk, q, n_tokens, n_heads, d_nope, d_c, d_r, dtype, s));
  return launch_rope_rows(q_pe, q, positions, n_tokens, n_heads, d_r, d_c + d_r, d_c, rope_base, dtype, s);
}

// ===========================================================================
// unabsorbed prefill
// ===========================================================================
size_t mla_prefill_unabsorbed_workspace(int batch, int s_kv, int n_heads, int d_nope, int d_v) {
  if (batch < 0 || s_kv < 0 || n_heads <= 0 || d_nope <= 0 || d_v <= 0) return 0;
  return a256((size_t)batch * s_kv * n_heads * (d_nope + d_v) * 2) + 256;
}

int mla_prefill_unabsorbed(const void* q_nope, const void* q_pe, const void* latent_cache, const void* w_uk,
                           const void* w_uv, int batch, int s_q, int s_kv, int n_heads, int d_nope, int d_c, int d_r,
                           int d_v, float kq_scale, int dtype, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!abi_dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (batch < 0 || s_q < 0 || s_kv < 0 || n_heads <= 0 || d_nope <= 0 || d_c <= 0 || d_r < 0 || d_v <= 0)
    return MLA_ERR_SHAPE;
  if (!std::isfinite(kq_scale)) return MLA_ERR_SCALE;
  if (dtype != MLA_BF16 || !flash_fits(d_nope, d_r, d_v) || d_c % 64 != 0 || d_c > 4096 || n_heads > 65535)
    return MLA_ERR_UNSUPPORTED;
  if ((int64_t)batch * s_q == 0) return MLA_OK;
  if ((int64_t)batch * s_kv > INT32_MAX || (int64_t)batch * s_q > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if (!q_nope || (d_r > 0 && !q_pe) || !latent_cache || !w_uk || !w_uv || !out) return MLA_ERR_NULL;
  if (!abi_aligned(q_nope, 16) || (q_pe && !abi_aligned(q_pe, 16)) || !abi_aligned(latent_cache, 16) ||
      !abi_aligned(w_uk, 16) || !abi_aligned(w_uv, 16) || !abi_aligned(out, 16) || (lse && !abi_aligned(lse, 4)))
    return MLA_ERR_ALIGN;
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (!abi_aligned(workspace, 256)) return MLA_ERR_ALIGN;
  if (workspace_bytes < mla_prefill_unabsorbed_workspace(batch, s_kv, n_heads, d_nope, d_v)) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int W = d_c + d_r, KV = d_nope + d_v;
  bf16* kv = (bf16*)workspace;  // [batch * s_kv, n_heads, d_nope + d_v]: k_nope | v per head
  if (s_kv > 0) {
    // k_nope[t, h] = W_UK[h] c_t and v[t, h] = W_UV[h] c_t (c_t: the first d_c values of cache row t),
    // as one product: output row t = [k_nope | v] of every head, B rows alternating d_nope rows of
    // W_UK[h] and d_v rows of W_UV[h]
    MLA_TRY(launch_gemm_pair(latent_cache, W, w_uk, w_uv, d_c, d_nope, d_v, kv, (int64_t)n_heads * KV,
                             batch * s_kv, n_heads * KV, d_c, s));
  }
  FlashDesc f{};
  f.q = q_nope;
  f.q_row = (int64_t)n_heads * d_nope;
  f.q_head = d_nope;
  f.qr = q_pe;
  f.qr_row = (int64_t)n_heads * d_r;
  f.qr_head = d_r;
  f.k = kv;
  f.k_row = (int64_t)n_heads * KV;
  f.k_head = KV;
  f.kr = (const bf16*)latent_cache + d_c;
  f.kr_row = W;
  f.v = kv + d_nope;
  f.v_row = (int64_t)n_heads * KV;
  f.v_head = KV;
  f.o = out;
  f.o_row = (int64_t)n_heads * d_v;
  f.o_head = d_v;
  f.lse = lse;
  f.B = batch;
  f.S_q = s_q;
  f.S_kv = s_kv;
  f.H = n_heads;
  f.d_r = d_r;
  f.scale = kq_scale;
  f.causal = true;
  return launch_flash(f, s);
}

// ===========================================================================
// full absorption
// ===========================================================================
size_t mla_absorb_weights_workspace(int n_heads, int d_nope, int d_cq, int d_c, int d_v, int dtype) {
  if (n_heads <= 0 || d_nope <= 0 || d_cq <= 0 || d_c <= 0 || d_v <= 0 || !abi_dtype_ok(dtype)) return 0;
  const size_t es = abi_esize(dtype);
  return a256((size_t)n_heads * d_c * d_nope * es) + a256((size_t)n_heads * d_cq * d_nope * es) +
         a256((size_t)n_heads * d_c * d_v * es) + 256;
}

int mla_absorb_weights(const void* w_uq, const void* w_uk, const void* w_uv, const void* w_o, int n_heads, int d_nope,
                       int d_cq, int d_c, int d_v, int d_model, int dtype, void* a_qk, void* a_vo, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!abi_dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (n_heads <= 0 || d_nope <= 0 || d_cq <= 0 || d_c <= 0 || d_v <= 0 || d_model <= 0) return MLA_ERR_SHAPE;
  if (n_heads > 65535 || d_nope > 4096 || d_cq > 16384 || d_c > 4096 || d_v > 4096 || d_model > 65536 ||
      (int64_t)n_heads * d_c > INT32_MAX / 2 || (int64_t)n_heads * d_v > INT32_MAX / 2)
    return MLA_ERR_UNSUPPORTED;
  if (!w_uq || !w_uk || !w_uv || !w_o || !a_qk || !a_vo) return MLA_ERR_NULL;
  const int es = abi_esize(dtype);
  if (!abi_aligned(w_uq, es) || !abi_aligned(w_uk, es) || !abi_aligned(w_uv, es) || !abi_aligned(w_o, es) ||
      !abi_aligned(a_qk, es) || !abi_aligned(a_vo, es))
    return MLA_ERR_ALIGN;
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (!abi_aligned(workspace, 256)) return MLA_ERR_ALIGN;
  if (workspace_bytes < mla_absorb_weights_workspace(n_heads, d_nope, d_cq, d_c, d_v, dtype))
    return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  void* ukT = ws;                                                           // [H, d_c, d_nope]
  void* uqT = ws + a256((size_t)n_heads * d_c * d_nope * es);               // [H, d_cq, d_nope]
  void* uvT = (char*)uqT + a256((size_t)n_heads * d_cq * d_nope * es);      // [H, d_c, d_v]
  MLA_TRY(launch_transpose(w_uk, ukT, d_nope, d_c, n_heads, (int64_t)d_nope * d_c, (int64_t)d_nope * d_c, dtype, s));
  MLA_TRY(launch_transpose(w_uq, uqT, d_nope, d_cq, n_heads, (int64_t)d_nope * d_cq, (int64_t)d_nope * d_cq, dtype, s));
  MLA_TRY(launch_transpose(w_uv, uvT, d_v, d_c, n_heads, (int64_t)d_v * d_c, (int64_t)d_v * d_c, dtype, s));
  // a_qk[h] = W_UK[h]^T W_UQ[h]: [d_c, d_cq], contraction over d_nope
  GemmDesc gq = gemm(ukT, d_nope, uqT, d_nope, a_qk, d_cq, d_c, d_cq, d_nope, dtype);
  gq.batch = n_heads;
  gq.a_batch = (int64_t)d_c * d_nope;
  gq.b_batch = (int64_t)d_cq * d_nope;
  gq.c_batch = (int64_t)d_c * d_cq;
  MLA_TRY(launch_gemm_nt(gq, s));
  // a_vo[:, h d_c ..] = W_O[:, h d_v ..] W_UV[h]: [d_model, d_c], contraction over d_v
  GemmDesc go = gemm(w_o, (int64_t)n_heads * d_v, uvT, d_v, a_vo, (int64_t)n_heads * d_c, d_model, d_c, d_v, dtype);
  go.batch = n_heads;
  go.a_batch = d_v;
  go.b_batch = (int64_t)d_c * d_v;
  go.c_batch = d_c;
  return launch_gemm_nt(go, s);
}

int mla_absorb_q_full(const void* c_q, const void* q_pe, const void* a_qk, const int32_t* positions,
                      float rope_base, void* q, int64_t n_tokens, int n_heads, int d_cq, int d_c, int d_r, int dtype,
                      void* stream) {
  if (!abi_dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (n_tokens < 0 || n_heads <= 0 || d_cq <= 0 || d_c <= 0 || d_r < 0 || (d_r & 1)) return MLA_ERR_SHAPE;
  if (n_heads > 65535 || d_cq > 16384 || d_c > 4096 || d_r > 1024 || n_tokens > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if (positions && !(std::isfinite(rope_base) && rope_base > 0.f)) return MLA_ERR_SCALE;
  if (n_tokens == 0) return MLA_OK;
  if (!c_q || !a_qk || !q || (d_r > 0 && !q_pe)) return MLA_ERR_NULL;
  const int es = abi_esize(dtype);
  if (!abi_aligned(c_q, es) || !abi_aligned(a_qk, es) || !abi_aligned(q, es) || (q_pe && !abi_aligned(q_pe, es)) ||
      (positions && !abi_aligned(positions, 4)))
    return MLA_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int W = d_c + d_r;
  // q[n, h, :d_c] = a_qk[h] c'_n
  GemmDesc g = gemm(c_q, d_cq, a_qk, d_cq, q, (int64_t)n_heads * W, (int)n_tokens, d_c, d_cq, dtype);
  g.batch = n_heads;
  g.b_batch = (int64_t)d_c * d_cq;
  g.c_batch = W;
  MLA_TRY(launch_gemm_nt(g, s));
  if (d_r == 0) return MLA_OK;
  return launch_rope_rows(q_pe, q, positions, n_tokens, n_heads, d_r, W, d_c, rope_base, dtype, s);
}

size_t mla_out_absorbed_workspace(int64_t n_tokens, int n_heads, int d_c, int d_model, int dtype) {
  if (n_tokens < 0 || n_heads <= 0 || d_c <= 0 || d_model <= 0 || !abi_dtype_ok(dtype)) return 0;
  const int sp = out_splits(n_tokens, n_heads, d_c, d_model, dtype);
  return a256((size_t)sp * n_tokens * d_model * sizeof(float)) + 256;
}

int mla_out_absorbed(const void* out_lat, const void* a_vo, void* out, int64_t n_tokens, int n_heads, int d_c,
                     int d_model, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!abi_dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (n_tokens < 0 || n_heads <= 0 || d_c <= 0 || d_model <= 0) return MLA_ERR_SHAPE;
  if ((int64_t)n_heads * d_c > INT32_MAX / 2 || d_model > 65536 || n_tokens > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if (n_tokens == 0) return MLA_OK;
  if (!out_lat || !a_vo || !out) return MLA_ERR_NULL;
  const int es = abi_esize(dtype);
  if (!abi_aligned(out_lat, es) || !abi_aligned(a_vo, es) || !abi_aligned(out, es)) return MLA_ERR_ALIGN;
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (!abi_aligned(workspace, 256)) return MLA_ERR_ALIGN;
  if (workspace_bytes < mla_out_absorbed_workspace(n_tokens, n_heads, d_c, d_model, dtype)) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int K = n_heads * d_c;
  float* P = (float*)workspace;
  const StreamDesc sd = out_stream(out_lat, a_vo, P, n_tokens, n_heads, d_c, d_model, dtype);
  if (sd.splits > 0 && stream_gemm_ok(sd)) {
    MLA_TRY(launch_stream_gemm(sd, s));
    return launch_splitk_reduce(P, sd.splits, sd.p_split, d_model, out, d_model, (int)n_tokens, d_model, dtype, s);
  }
  const int sp = out_splits(n_tokens, n_heads, d_c, d_model, dtype);
  // out[n, i] = sum over heads and latent dims of a_vo[i, (h, j)] out_lat[n, h, j]: the head sum is the contraction
  GemmDesc g = gemm(out_lat, K, a_vo, K, P, d_model, (int)n_tokens, d_model, K, dtype);
  g.out_f32 = true;
  g.splits = sp;
  g.c_split = (int64_t)n_tokens * d_model;
  MLA_TRY(launch_gemm_nt(g, s));
  return launch_splitk_reduce(P, sp, (int64_t)n_tokens * d_model, d_model, out, d_model, (int)n_tokens, d_model, dtype,
                              s);
}

// ===========================================================================
// gated MLA
// ===========================================================================
size_t mla_gated_mla_workspace(int batch, int seq, int d_model, int latent, int n_heads, int dtype, int num_workers) {
  if (batch < 0 || seq < 0 || d_model <= 0 || latent <= 0 || n_heads <= 0 || d_model % n_heads != 0 ||
      !abi_dtype_ok(dtype))
    return 0;
  const size_t es = abi_esize(dtype);
  const size_t n = (size_t)batch * seq;
  size_t b = 4 * a256(n * d_model * es);  // Q, G, and the two value-side buffers
  if (gated_flash_route(d_model, n_heads, dtype)) {
    b += a256(n * d_model * es);  // K
  } else {
    // absorbed latent route: absorbed queries and latent outputs, plus the attention plan
    const int G = num_workers > 0 ? num_workers : kCuRef;
    b += 2 * a256(n * n_heads * latent * es);
    b += a256(mla_latent_prefill_causal_workspace(batch, seq, n_heads, latent, G));
  }
  return b + 256;
}

int mla_gated_mla(const void* x, const void* w_q, const void* w_c, const void* w_k, const void* w_v, const void* w_g,
                  const void* w_o, int batch, int seq, int d_model, int latent, int n_heads, int causal, int dtype,
                  void* out, void* latent_cache, void* workspace, size_t workspace_bytes, int num_workers,
                  void* stream) {
  if (!abi_dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (batch < 0 || seq < 0 || d_model <= 0 || latent <= 0 || n_heads <= 0 || num_workers < 0) return MLA_ERR_SHAPE;
  if (d_model % n_heads != 0) return MLA_ERR_SHAPE;
  const int64_t n = (int64_t)batch * seq;
  if (d_model > 65536 || latent > 1024 || n > INT32_MAX / 2) return MLA_ERR_UNSUPPORTED;
  if (n == 0) return MLA_OK;
  if (!x || !w_q || !w_c || !w_k || !w_v || !w_g || !w_o || !out || !latent_cache) return MLA_ERR_NULL;
  const int es = abi_esize(dtype);
  for (const void* p : {x, w_q, w_c, w_k, w_v, w_g, w_o, (const void*)out, (const void*)latent_cache})
    if (!abi_aligned(p, es)) return MLA_ERR_ALIGN;
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (!abi_aligned(workspace, 256)) return MLA_ERR_ALIGN;
  const int G = num_workers > 0 ? num_workers : kCuRef;
  if (workspace_bytes < mla_gated_mla_workspace(batch, seq, d_model, latent, n_heads, dtype, G))
    return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int D = d_model, L = latent, Dh = d_model / n_heads;
  const size_t nd = a256((size_t)n * D * es);
  char* ws = (char*)workspace;
  void* Q = ws;
  void* Gt = ws + nd;
  void* Ot = ws + 2 * nd;   // the head contexts (then gated)
  void* V = ws + 3 * nd;    // values (flash route) / scratch
  char* rest = ws + 4 * nd;
  const float scale = 1.0f / std::sqrt((float)Dh);
  // C = X W_c^T (the returned latent cache)
  MLA_TRY(launch_gemm_nt(gemm(x, D, w_c, D, latent_cache, L, (int)n, L, D, dtype), s));
  if (gated_flash_route(D, n_heads, dtype) && pair_fits(n, D, L, {x, w_q, w_g, w_k, w_v, w_o, out, latent_cache})) {
    // Large products on 256 x 256 tiles: [Q | G] = X [W_q ; W_g]^T in one product (row t =
    // [q_t | g_t], over the Q and G regions, which are adjacent), [K | V] = C [W_k ; W_v]^T
    // likewise (over the V and K regions), then attention per head with the gate fused,
    // reading Q, G, K and V through their row strides
    void* QG = Q;
    void* KV = V;
    MLA_TRY(launch_gemm_pair(x, D, w_q, w_g, D, D, D, QG, 2 * D, (int)n, 2 * D, D, s));
    MLA_TRY(launch_gemm_pair(latent_cache, L, w_k, w_v, L, D, D, KV, 2 * D, (int)n, 2 * D, L, s));
    FlashDesc f{};
    f.q = QG;
    f.q_row = 2 * D;
    f.q_head = Dh;
    f.k = KV;
    f.k_row = 2 * D;
    f.k_head = Dh;
    f.v = (char*)KV + (size_t)D * es;
    f.v_row = 2 * D;
    f.v_head = Dh;
    f.o = Ot;
    f.o_row = D;
    f.o_head = Dh;
    f.gate = (char*)QG + (size_t)D * es;
    f.g_row = 2 * D;
    f.g_head = Dh;
    f.B = batch;
    f.S_q = seq;
    f.S_kv = seq;
    f.H = n_heads;
    f.d_r = 0;
    f.scale = scale;
    f.causal = causal != 0;
    MLA_TRY(launch_flash(f, s));
    // Y = (sigmoid(G) * O~) W_o^T
    return launch_gemm_pair(Ot, D, w_o, nullptr, D, D, 0, out, D, (int)n, D, D, s);
  }
  // Q = X W_q^T, gate pre-activations X W_g^T
  MLA_TRY(launch_gemm_nt(gemm(x, D, w_q, D, Q, D, (int)n, D, D, dtype), s));
  MLA_TRY(launch_gemm_nt(gemm(x, D, w_g, D, Gt, D, (int)n, D, D, dtype), s));
  if (gated_flash_route(D, n_heads, dtype)) {
    // K = C W_k^T, V = C W_v^T per position, then attention per head with the gate fused
    void* K = rest;
    MLA_TRY(launch_gemm_nt(gemm(latent_cache, L, w_k, L, K, D, (int)n, D, L, dtype), s));
    MLA_TRY(launch_gemm_nt(gemm(latent_cache, L, w_v, L, V, D, (int)n, D, L, dtype), s));
    FlashDesc f{};
    f.q = Q;
    f.q_row = D;
    f.q_head = Dh;
    f.k = K;
    f.k_row = D;
    f.k_head = Dh;
    f.v = V;
    f.v_row = D;
    f.v_head = Dh;
    f.o = Ot;
    f.o_row = D;
    f.o_head = Dh;
    f.gate = Gt;
    f.g_row = D;
    f.g_head = Dh;
    f.B = batch;
    f.S_q = seq;
    f.S_kv = seq;
    f.H = n_heads;
    f.d_r = 0;
    f.scale = scale;
    f.causal = causal != 0;
    MLA_TRY(launch_flash(f, s));
  } else {
    // absorbed latent route: q_abs[h] = W_k[h]^T Q[h] (W_k[h] = rows h D_h .. of W_k, [D_h, L]),
    // latent attention over C with value C, then O[h] = W_v[h] out_lat[h]
    const size_t nl = a256((size_t)n * n_heads * L * es);
    void* qa = rest;
    void* lat = rest + nl;
    void* plan = rest + 2 * nl;
    MLA_TRY(launch_absorb(Q, nullptr, w_k, qa, n, n_heads, Dh, L, 0, dtype, s));
    AttnCall c{};
    c.q = qa;
    c.cache = latent_cache;
    c.map.mode = 2;
    c.map.s_q = seq;
    c.map.s_kv = seq;
    c.map.non_causal = causal ? 0 : 1;
    c.R = (int)n;
    c.H = n_heads;
    c.d_c = L;
    c.d_r = 0;
    c.kq_scale = scale;
    c.dtype = dtype;
    c.out = lat;
    c.lse = nullptr;
    c.ws = plan;
    c.G = G;
    c.stream = s;
    MLA_TRY(launch_attention(c));
    MLA_TRY(launch_up_v(lat, w_v, Ot, n, n_heads, L, Dh, dtype, s));
    MLA_TRY(launch_gate(Ot, Gt, n * D, dtype, s));
  }
  // Y = (sigmoid(G) * O~) W_o^T
  return launch_gemm_nt(gemm(Ot, D, w_o, D, out, D, (int)n, D, D, dtype), s);
}

}  // extern "C"
