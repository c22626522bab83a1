// C ABI of libmla: argument validation (before any HIP call that launches
// work), worker-count and workspace sizing, and dispatch to the kernels.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "mla_internal.h"

using namespace mla;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // cached compute-unit count per device (0 = unknown)

int elem_size(int dtype) { return dtype == MLA_BF16 ? 2 : 4; }
bool valid_dtype(int dtype) { return dtype == MLA_F32 || dtype == MLA_BF16; }
bool aligned(const void* p, int a) { return ((uintptr_t)p % (uintptr_t)a) == 0; }

// Largest worker count: the combine kernels put the split rows (at most one
// per worker) on the grid's y axis, whose limit is 65535.
constexpr int kMaxWorkers = 65535;

int resolve_workers(int num_workers) {
  if (num_workers < 0) return MLA_ERR_SHAPE;
  if (num_workers > kMaxWorkers) return MLA_ERR_UNSUPPORTED;
  if (num_workers > 0) return num_workers;
  return mla_default_workers();
}

// The plan counts work in int32 units: one per 16-position tile plus a fixed
// cost of SEG_COST units per non-empty row; the unit total (and prefix sums)
// must stay far from overflow.
bool units_fit(int64_t rows, int64_t max_len) {
  return rows * ((max_len + 15) / 16 + SEG_COST) <= INT32_MAX / 2;
}

}  // namespace

// ---------------------------------------------------------------------------
// Fixed scratch of the allocation-free decode entry (mla_latent_decode_noalloc):
// one array per device, held until the process ends. Host code never uses the
// array's name as an address: the device address of each device's copy is
// taken once, with that device current, by hipGetSymbolAddress and kept in
// g_scratch_ptr.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null = not yet taken)

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}
}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case MLA_ERR_DTYPE: return "dtype must be MLA_F32 or MLA_BF16";
    case MLA_ERR_UNSUPPORTED: return "sizes beyond the library's limits";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_ALIGN: return "pointer not aligned to its element size";
    case MLA_ERR_SCALE: return "kq_scale is not finite";
    case MLA_ERR_HIP: return "HIP runtime call or kernel launch failed";
    default: return "unknown status";
  }
}

int mla_version(void) { return 100; }

int mla_default_workers(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) {
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
    return MLA_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(cu, std::memory_order_relaxed);
  return cu;
}

// ---------------------------------------------------------------------------
int mla_absorb_q(const void* q_nope, const void* q_pe, const void* w_uk, void* q, int64_t n_tokens, int n_heads,
                 int d_nope, int d_c, int d_r, int dtype, void* stream) {
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (n_tokens < 0 || n_heads <= 0 || d_nope <= 0 || d_c <= 0 || d_r < 0) return MLA_ERR_SHAPE;
  if (n_heads > 65535 || d_nope > 4096 || d_c > 4096 || d_r > 1024) return MLA_ERR_UNSUPPORTED;
  if (n_tokens == 0) return MLA_OK;  // nothing to do; empty tensors may have NULL data
  if (!q_nope || !w_uk || !q || (d_r > 0 && !q_pe)) return MLA_ERR_NULL;
  const int es = elem_size(dtype);
  if (!aligned(q_nope, es) || !aligned(w_uk, es) || !aligned(q, es) || (q_pe && !aligned(q_pe, es)))
    return MLA_ERR_ALIGN;
  if (n_tokens * (int64_t)n_heads * (d_c + d_r) > ((int64_t)1 << 40)) return MLA_ERR_UNSUPPORTED;
  return launch_absorb(q_nope, q_pe, w_uk, q, n_tokens, n_heads, d_nope, d_c, d_r, dtype, (hipStream_t)stream);
}

int mla_up_v(const void* out_lat, const void* w_uv, void* out, int64_t n_tokens, int n_heads, int d_c, int d_v,
             int dtype, void* stream) {
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (n_tokens < 0 || n_heads <= 0 || d_c <= 0 || d_v <= 0) return MLA_ERR_SHAPE;
  if (n_heads > 65535 || d_c > 4096 || d_v > 4096) return MLA_ERR_UNSUPPORTED;
  if (n_tokens == 0) return MLA_OK;  // nothing to do; empty tensors may have NULL data
  if (!out_lat || !w_uv || !out) return MLA_ERR_NULL;
  const int es = elem_size(dtype);
  if (!aligned(out_lat, es) || !aligned(w_uv, es) || !aligned(out, es)) return MLA_ERR_ALIGN;
  if (n_tokens * (int64_t)n_heads * d_c > ((int64_t)1 << 40)) return MLA_ERR_UNSUPPORTED;
  return launch_up_v(out_lat, w_uv, out, n_tokens, n_heads, d_c, d_v, dtype, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
static int attn_dims_check(int rows, int n_heads, int d_c, int d_r) {
  if (rows < 0 || n_heads <= 0 || d_c <= 0 || d_r < 0) return MLA_ERR_SHAPE;
  if (n_heads > 65535 || d_c > 1024 || d_c + d_r > 1152) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

size_t mla_latent_decode_workspace(int batch, int n_heads, int d_c, int num_workers) {
  if (batch < 0 || n_heads <= 0 || d_c <= 0) return 0;
  int G = resolve_workers(num_workers);
  if (G <= 0) return 0;
  return plan_bytes(batch, G, n_heads, d_c);
}

size_t mla_latent_prefill_causal_workspace(int batch, int s_q, int n_heads, int d_c, int num_workers) {
  if (batch < 0 || s_q < 0 || n_heads <= 0 || d_c <= 0) return 0;
  if ((int64_t)batch * s_q > INT32_MAX - 1) return 0;
  int G = resolve_workers(num_workers);
  if (G <= 0) return 0;
  return plan_bytes((int64_t)batch * s_q, G, n_heads, d_c);
}

static int common_attn_checks(const void* q, const void* cache, void* out, float* lse, void* ws, int dtype,
                              float kq_scale) {
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (!std::isfinite(kq_scale)) return MLA_ERR_SCALE;
  if (!q || !cache || !out) return MLA_ERR_NULL;
  const int es = elem_size(dtype);
  if (!aligned(q, es) || !aligned(cache, es) || !aligned(out, es) || (lse && !aligned(lse, 4))) return MLA_ERR_ALIGN;
  if (ws && !aligned(ws, 256)) return MLA_ERR_ALIGN;
  return MLA_OK;
}

// decode, with the up-projection when w_uv is given (v then receives it and
// out_lat is scratch inside the workspace)
static int decode_call(const void* q, const void* latent_cache, const int32_t* seq_lens, const int32_t* block_table,
                       int batch, int n_heads, int d_c, int d_r, int cache_stride, int page_size, int max_pages,
                       int num_pages, float kq_scale, int dtype, void* out_lat, float* lse, void* workspace,
                       size_t workspace_bytes, int num_workers, void* const* timing_events, void* stream,
                       const void* w_uv, int d_v, void* v, bool use_scratch = false) {
  int st = attn_dims_check(batch, n_heads, d_c, d_r);
  if (st != MLA_OK) return st;
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (!std::isfinite(kq_scale)) return MLA_ERR_SCALE;
  if (num_workers < 0 || (!block_table && cache_stride < 0)) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;  // nothing to do; empty tensors may have NULL data
  st = common_attn_checks(q, latent_cache, out_lat, lse, workspace, dtype, kq_scale);
  if (st != MLA_OK) return st;
  if (!seq_lens) return MLA_ERR_NULL;
  if (!aligned(seq_lens, 4) || (block_table && !aligned(block_table, 4))) return MLA_ERR_ALIGN;
  int64_t cap;
  if (block_table) {
    if (page_size <= 0 || max_pages <= 0 || num_pages <= 0) return MLA_ERR_SHAPE;
    cap = (int64_t)page_size * max_pages;
  } else {
    if (cache_stride < 0) return MLA_ERR_SHAPE;
    cap = cache_stride;
  }
  if (!units_fit(batch, cap)) return MLA_ERR_UNSUPPORTED;
  const int G = resolve_workers(num_workers);
  if (G <= 0) return G == 0 ? MLA_ERR_SHAPE : G;
  int part_esize = 4;
  if (use_scratch) {  // the library's fixed scratch: partials sized for the call's dtype
    part_esize = elem_size(dtype);
    if (plan_bytes(batch, G, n_heads, d_c, part_esize) > (size_t)MLA_NOALLOC_SCRATCH_BYTES)
      return MLA_ERR_UNSUPPORTED;
    st = scratch_address(&workspace);
    if (st != MLA_OK) return st;
    workspace_bytes = MLA_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace) return MLA_ERR_WORKSPACE;
  size_t need = plan_bytes(batch, G, n_heads, d_c, part_esize);
  if (w_uv) {  // out_lat in the workspace, after the plan
    out_lat = (char*)workspace + need;
    need += align256((size_t)batch * n_heads * d_c * sizeof(float));
  }
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE;

  AttnCall c{};
  c.q = q;
  c.cache = latent_cache;
  c.map.mode = block_table ? 1 : 0;
  c.map.cache_stride = cache_stride;
  c.map.page_size = page_size;
  c.map.max_pages = max_pages;
  c.map.num_pages = num_pages;
  c.map.block_table = block_table;
  c.map.seq_lens = seq_lens;
  c.R = batch;
  c.H = n_heads;
  c.d_c = d_c;
  c.d_r = d_r;
  c.kq_scale = kq_scale;
  c.dtype = dtype;
  c.out = out_lat;
  c.lse = lse;
  c.ws = workspace;
  c.part_esize = part_esize;
  c.G = G;
  c.timing_events = timing_events;
  c.stream = (hipStream_t)stream;
  c.w_uv = w_uv;
  c.v = v;
  c.d_v = d_v;
  return launch_attention(c);
}

int mla_latent_decode(const void* q, const void* latent_cache, const int32_t* seq_lens, const int32_t* block_table,
                      int batch, int n_heads, int d_c, int d_r, int cache_stride, int page_size, int max_pages,
                      int num_pages, float kq_scale, int dtype, void* out_lat, float* lse, void* workspace,
                      size_t workspace_bytes, int num_workers, void* const* timing_events, void* stream) {
  return decode_call(q, latent_cache, seq_lens, block_table, batch, n_heads, d_c, d_r, cache_stride, page_size,
                     max_pages, num_pages, kq_scale, dtype, out_lat, lse, workspace, workspace_bytes, num_workers,
                     timing_events, stream, nullptr, 0, nullptr);
}

int mla_latent_decode_noalloc(const void* q, const void* latent_cache, const int32_t* seq_lens,
                              const int32_t* block_table, int batch, int n_heads, int d_c, int d_r, int cache_stride,
                              int page_size, int max_pages, int num_pages, float kq_scale, int dtype, void* out_lat,
                              float* lse, int num_workers, void* stream) {
  return decode_call(q, latent_cache, seq_lens, block_table, batch, n_heads, d_c, d_r, cache_stride, page_size,
                     max_pages, num_pages, kq_scale, dtype, out_lat, lse, nullptr, 0, num_workers, nullptr, stream,
                     nullptr, 0, nullptr, true);
}

size_t mla_latent_decode_noalloc_scratch_bytes(int batch, int n_heads, int d_c, int dtype, int num_workers) {
  if (batch < 0 || n_heads <= 0 || d_c <= 0 || !valid_dtype(dtype)) return 0;
  int G = resolve_workers(num_workers);
  if (G <= 0) return 0;
  return plan_bytes(batch, G, n_heads, d_c, elem_size(dtype));
}

size_t mla_latent_decode_up_v_workspace(int batch, int n_heads, int d_c, int num_workers) {
  const size_t b = mla_latent_decode_workspace(batch, n_heads, d_c, num_workers);
  return b == 0 ? 0 : b + align256((size_t)batch * n_heads * d_c * sizeof(float));
}

int mla_latent_decode_up_v(const void* q, const void* latent_cache, const int32_t* seq_lens,
                           const int32_t* block_table, int batch, int n_heads, int d_c, int d_r, int cache_stride,
                           int page_size, int max_pages, int num_pages, float kq_scale, const void* w_uv, int d_v,
                           int dtype, void* out, float* lse, void* workspace, size_t workspace_bytes, int num_workers,
                           void* const* timing_events, void* stream) {
  if (d_v <= 0) return MLA_ERR_SHAPE;
  if (d_v > 4096) return MLA_ERR_UNSUPPORTED;
  if (batch > 0) {
    if (!w_uv || !out) return MLA_ERR_NULL;
    const int es = (dtype == MLA_BF16) ? 2 : 4;
    if (((uintptr_t)w_uv % es) || ((uintptr_t)out % es)) return MLA_ERR_ALIGN;
  }
  // out_lat is scratch in the workspace (out stands in for it in the argument checks)
  return decode_call(q, latent_cache, seq_lens, block_table, batch, n_heads, d_c, d_r, cache_stride, page_size,
                     max_pages, num_pages, kq_scale, dtype, out, lse, workspace, workspace_bytes, num_workers,
                     timing_events, stream, w_uv, d_v, out);
}

int mla_latent_prefill_causal(const void* q, const void* latent_cache, int batch, int s_q, int s_kv, int n_heads,
                              int d_c, int d_r, float kq_scale, int dtype, void* out_lat, float* lse, void* workspace,
                              size_t workspace_bytes, int num_workers, void* const* timing_events, void* stream) {
  if (s_q < 0 || s_kv < 0) return MLA_ERR_SHAPE;
  if ((int64_t)batch * s_q > INT32_MAX - 1) return MLA_ERR_UNSUPPORTED;
  int st = attn_dims_check(batch, n_heads, d_c, d_r);
  if (st != MLA_OK) return st;
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (!std::isfinite(kq_scale)) return MLA_ERR_SCALE;
  if (num_workers < 0) return MLA_ERR_SHAPE;
  const int64_t rows = (int64_t)batch * s_q;
  if (rows == 0) return MLA_OK;  // nothing to do; empty tensors may have NULL data
  st = common_attn_checks(q, latent_cache, out_lat, lse, workspace, dtype, kq_scale);
  if (st != MLA_OK) return st;
  if (!units_fit(rows, s_kv)) return MLA_ERR_UNSUPPORTED;
  const int G = resolve_workers(num_workers);
  if (G <= 0) return G == 0 ? MLA_ERR_SHAPE : G;
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < plan_bytes(rows, G, n_heads, d_c)) return MLA_ERR_WORKSPACE;

  AttnCall c{};
  c.q = q;
  c.cache = latent_cache;
  c.map.mode = 2;
  c.map.s_q = s_q;
  c.map.s_kv = s_kv;
  c.R = (int)rows;
  c.H = n_heads;
  c.d_c = d_c;
  c.d_r = d_r;
  c.kq_scale = kq_scale;
  c.dtype = dtype;
  c.out = out_lat;
  c.lse = lse;
  c.ws = workspace;
  c.G = G;
  c.timing_events = timing_events;
  c.stream = (hipStream_t)stream;
  return launch_attention(c);
}

int mla_lse_combine(const float* o_parts, const float* lse_parts, int n_parts, int64_t rows, int n_heads, int d_c,
                    int dtype, void* out, float* lse, void* stream) {
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (n_parts <= 0 || rows < 0 || n_heads <= 0 || d_c <= 0) return MLA_ERR_SHAPE;
  if (n_parts > 4096 || d_c > 4096 || n_heads > 65535 || rows > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if (rows == 0) return MLA_OK;  // nothing to do; empty tensors may have NULL data
  if (!o_parts || !lse_parts || !out) return MLA_ERR_NULL;
  if (!aligned(o_parts, 4) || !aligned(lse_parts, 4) || !aligned(out, elem_size(dtype)) || (lse && !aligned(lse, 4)))
    return MLA_ERR_ALIGN;
  return launch_lse_combine(o_parts, lse_parts, n_parts, rows, n_heads, d_c, dtype, out, lse, (hipStream_t)stream);
}

}  // extern "C"
