// Internal declarations of libmla: device helpers and kernel launchers.
// Target: gfx950 (CDNA4) only; 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "mla.h"

namespace mla {

// ---------------------------------------------------------------------------
// vector types used as MFMA operands
// ---------------------------------------------------------------------------
typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f32_to_bf16(float x) { return (bf16)x; }  // nearest-even (v_cvt_pk_bf16_f32)

template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<bf16>(const bf16* p) { return (float)*p; }
// four consecutive elements (16-byte aligned for fp32, 8-byte for bf16) as fp32
template <typename T> __device__ __forceinline__ f32x4 load4_f32(const T* p);
template <> __device__ __forceinline__ f32x4 load4_f32<float>(const float* p) { return *(const f32x4*)p; }
template <> __device__ __forceinline__ f32x4 load4_f32<bf16>(const bf16* p) {
  const bf16x4 v = *(const bf16x4*)p;
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <typename T> __device__ __forceinline__ void store_f32(T* p, float v);
template <> __device__ __forceinline__ void store_f32<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_f32<bf16>(bf16* p, float v) { *p = (bf16)v; }

// ---------------------------------------------------------------------------
// split-sequence plan shared by the attention kernels and the combine.
//
// The work of a call is a list of R "rows" (decode: one per sequence;
// prefill: one per query), each with len[r] visible positions cut into
// tiles of TILE positions. Work is measured in units: one per tile, plus a
// fixed cost c for every row that has tiles (a segment's fixed work: query
// load, pipeline fill, normalisation and output write). Rows are laid out in
// row order on the unit axis, a non-empty row as c units of fixed cost
// followed by one unit per tile, and the axis is dealt out in equal
// contiguous ranges of `per_worker` units to G workers (one workgroup
// each). c is SEG_COST when rows are on average shorter than a worker's
// share of tiles: without it, workers given many short rows (the first
// queries of a causal prefill) would take several times longer than the
// rest. Otherwise c is 0: long rows are cut into pieces that each pay the
// fixed cost, which equal tile ranges already balance. The plan stores c in
// split[1]. A worker's range is a run of segments, one per row with tiles in
// it. A row whose tiles all fall in one worker is finished there; a row
// whose tiles are cut by worker boundaries leaves one partial result
// (normalised output in the call's dtype + fp32 lse) per worker holding
// some of its tiles, merged by the combine.
// Partial slot of (worker w, row r): 2w if r's tiles started before w's
// range (r is w's first segment), else 2w + 1 (r runs past w's end). So 2G
// slots.
// ---------------------------------------------------------------------------
struct Plan {
  int32_t* cum;     // [R + 1]: exclusive prefix sum of units per row (cum[R] = total)
  int32_t* len;     // [R]: visible positions per row (clamped)
  int32_t* split;   // [4 + 4G]: count, the fixed cost per row c, then per row cut by a worker boundary
                    //   {row, slot of its first part, its first worker, number of parts} (16-byte entries
                    //   from index 4)
  int32_t* wrow;    // [G]: first row of every worker that has tiles
  float* part_o;    // [2G, H, d_c] partial outputs, stored in the call's dtype (bf16 calls use half the region)
  float* part_lse;  // [2G, H]
  int R;
  int G;
  int tile;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// workspace layout: cum | len | split | wrow | part_o | part_lse. The partial
// outputs are stored in the call's dtype; `part_esize` is the element size
// the region is sized for (4 for caller workspaces, whose size query takes no
// dtype; the call's own size for the library's fixed scratch).
inline size_t plan_bytes(int64_t R, int G, int H, int d_c, int part_esize = 4) {
  size_t b = align256(sizeof(int32_t) * (size_t)(R + 1));
  b += align256(sizeof(int32_t) * (size_t)R);
  b += align256(sizeof(int32_t) * (size_t)(4 + 4 * G));
  b += align256(sizeof(int32_t) * (size_t)G);
  b += align256((size_t)part_esize * 2 * G * H * d_c);
  b += align256(sizeof(float) * (size_t)2 * G * H);
  return b;
}

inline Plan plan_layout(void* ws, int R, int G, int H, int d_c, int tile, int part_esize = 4) {
  char* p = (char*)ws;
  Plan pl;
  pl.cum = (int32_t*)p;
  p += align256(sizeof(int32_t) * (size_t)(R + 1));
  pl.len = (int32_t*)p;
  p += align256(sizeof(int32_t) * (size_t)R);
  pl.split = (int32_t*)p;
  p += align256(sizeof(int32_t) * (size_t)(4 + 4 * G));
  pl.wrow = (int32_t*)p;
  p += align256(sizeof(int32_t) * (size_t)G);
  pl.part_o = (float*)p;
  p += align256((size_t)part_esize * 2 * G * H * d_c);
  pl.part_lse = (float*)p;
  pl.R = R;
  pl.G = G;
  pl.tile = tile;
  return pl;
}

constexpr int SEG_COST = 12;  // fixed work of a segment, in tile units (measured: about 12 tiles' time)

// units of a row with n tiles under a fixed cost c per row
__host__ __device__ inline int row_units(int n, int c) { return n > 0 ? n + c : 0; }

__device__ __forceinline__ int plan_per_worker(int total, int G) {
  int q = (total + G - 1) / G;
  return q < 1 ? 1 : q;
}

// Worker index of this workgroup. Workgroups are dispatched round-robin over
// the 8 XCDs (blockIdx.x % 8); consecutive workers share rows (and the
// query rows they re-read), so place consecutive workers on the same XCD.
__device__ __forceinline__ int xcd_worker(int bx, int G) {
  if (G % 8 != 0) return bx;
  return (bx % 8) * (G / 8) + bx / 8;
}

__device__ __forceinline__ int plan_slot(int w, int row_tile_start, int per_worker) {
  return (row_tile_start < w * per_worker) ? 2 * w : 2 * w + 1;
}

// The segment of row r (units [c0, c1), fixed cost `cost`) in a worker's unit range [t_begin,
// t_end): tiles [lt0, lt1) of the row, whether they are all of its tiles,
// and the partial slot. False when the worker holds none of its tiles.
struct Segment {
  int lt0, lt1, slot;
  bool full;
};
__device__ __forceinline__ bool plan_segment(int c0, int c1, int cost, int t_begin, int t_end, int w, int per,
                                             Segment& sg) {
  if (c1 == c0) return false;
  const int s0 = c0 + cost;
  if (c1 <= t_begin || s0 >= t_end) return false;
  sg.lt0 = max(t_begin, s0) - s0;
  sg.lt1 = min(t_end, c1) - s0;
  sg.full = s0 >= t_begin && c1 <= t_end;
  sg.slot = plan_slot(w, s0, per);
  return true;
}

// description of where row r's query, cache and output live
struct RowMap {
  int mode;            // 0 = decode dense, 1 = decode paged, 2 = prefill
  int s_q, s_kv;       // prefill
  int non_causal;      // prefill: every query sees all s_kv positions (no mask)
  int cache_stride;    // dense rows per sequence
  int page_size, max_pages, num_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
};

// ---------------------------------------------------------------------------
// launchers (mla_attn.hip / mla_gemm.hip)
// ---------------------------------------------------------------------------
struct AttnCall {
  const void* q;
  const void* cache;
  RowMap map;
  int R, H, d_c, d_r;
  float kq_scale;
  int dtype;
  void* out;
  float* lse;
  void* ws;
  int part_esize = 4;  // element size the workspace's partial-output region is sized for
  int G;
  void* const* timing_events;
  hipStream_t stream;
  // optional up-projection of the result (decode): v[r, h] = W_UV[h] out[r, h];
  // out is then scratch for rows finished by one worker
  const void* w_uv = nullptr;  // [H, d_v, d_c]
  void* v = nullptr;           // [R, H, d_v]
  int d_v = 0;
};

int attn_tile_size(const AttnCall& c);          // tile used by the kernel path chosen for c
int launch_attention(const AttnCall& c);        // plan + attention + combine
int launch_lse_combine(const float* o_parts, const float* lse_parts, int n_parts, int64_t rows,
                       int H, int d_c, int dtype, void* out, float* lse, hipStream_t stream);
int launch_absorb(const void* q_nope, const void* q_pe, const void* w_uk, void* q, int64_t N,
                  int H, int d_nope, int d_c, int d_r, int dtype, hipStream_t stream);
int launch_up_v(const void* lat, const void* w_uv, void* out, int64_t N, int H, int d_c,
                int d_v, int dtype, hipStream_t stream);
// decode rows' merge fused with the up-projection: lat = the attention kernel's
// outputs of rows finished by one worker, pl = its plan (bf16, d_c = 512, d_v = 128)
bool upv_merge_fits(int d_c, int d_v, const void* w_uv, const void* v);
int launch_upv_merge(const Plan& pl, int R, int H, const void* lat, const void* w_uv, void* v, float* lse,
                     hipStream_t stream);

// ---------------------------------------------------------------------------
// argument helpers shared by the C ABI sources
// ---------------------------------------------------------------------------
inline int abi_esize(int dtype) { return dtype == MLA_BF16 ? 2 : 4; }
inline bool abi_dtype_ok(int dtype) { return dtype == MLA_F32 || dtype == MLA_BF16; }
inline bool abi_aligned(const void* p, int a) { return ((uintptr_t)p % (uintptr_t)a) == 0; }

// ---------------------------------------------------------------------------
// dense products and row kernels (mla_dense.hip)
// ---------------------------------------------------------------------------
// C[batch][split][m][n] = sum_k A[batch][m][k] B[batch][n][k] (row strides lda,
// ldb, ldc in elements; batch strides may be 0). bf16 inputs on the MFMA path
// need K a multiple of 64 and 16-byte aligned rows; anything else runs the
// generic kernel (one split). out_f32: fp32 output (split-K partials at
// c_split apart), else the output has the inputs' dtype (one split).
struct GemmDesc {
  const void* A;
  const void* B;
  const void* B2;  // optional: rows n >= n1 of the weight come from B2 (MFMA path only)
  int n1;
  void* C;
  int64_t lda, ldb, ldc;
  int64_t a_batch, b_batch, c_batch, c_split;
  int M, N, K, batch;
  int splits;
  int dtype;
  bool out_f32;
};
bool gemm_nt_mfma_ok(const GemmDesc& g);
int gemm_nt_splits(const GemmDesc& g, int cus, int max_splits = 64);
int launch_gemm_nt(const GemmDesc& g, hipStream_t s);
// bf16 C[m, n] = sum_k A[m, k] B(n)[k] for large M and N, row n of B taken
// from B1 or B2 in groups of n1 + n2 rows (see mla_dense.hip); K a multiple
// of 64, N a multiple of 8, 16-byte aligned rows
int launch_gemm_pair(const void* A, int64_t lda, const void* B1, const void* B2, int64_t ldb, int n1, int n2,
                     void* C, int64_t ldc, int M, int N, int K, hipStream_t s);
// C[m, n] = sum_k X[m, k] W[n, k] for at most 64 rows of X against a weight
// stream (see mla_stream.hip); bf16 inputs, fp32 partials P[split][M][N]
// out (K a multiple of 256).
struct StreamDesc {
  const void* X;
  int64_t ldx;
  const void* W;
  int64_t ldw;
  float* P;
  int64_t p_split;
  int M, N, K, splits;
};
bool stream_gemm_ok(const StreamDesc& d);
// split count that fills `cus` compute units with one workgroup each, at most max_splits
int stream_gemm_splits(int N, int K, int cus, int max_splits);
int launch_stream_gemm(const StreamDesc& d, hipStream_t s);
int launch_splitk_reduce(const float* P, int splits, int64_t split_stride, int64_t ldp, void* C, int64_t ldc, int M,
                         int N, int dtype, hipStream_t s);
int launch_transpose(const void* in, void* out, int rows, int cols, int batch, int64_t in_batch, int64_t out_batch,
                     int dtype, hipStream_t s);
int launch_cache_rows(const float* P, int splits, int64_t split_stride, const void* gain, float eps, float rope_base,
                      const int32_t* seq_ids, const int32_t* positions, void* cache, const RowMap& map, int n_seqs,
                      int n_tokens, int d_c, int d_r, int dtype, hipStream_t s);
// dst[n, h, col0 + j] = rotation of src[n, h, j] at positions[n] (positions
// NULL: a plain copy)
int launch_rope_rows(const void* src, void* dst, const int32_t* positions, int64_t rows, int H, int d_r, int ldd,
                     int col0, float rope_base, int dtype, hipStream_t s);
// x[i] *= sigmoid(g[i]) for i < n
int launch_gate(void* x, const void* g, int64_t n, int dtype, hipStream_t s);

// ---------------------------------------------------------------------------
// standard per-head attention (mla_flash.hip): bf16, d_nope = d_v = 128,
// d_r 0 or 64 (rope key shared by all heads). Element (row, head, dim) of a
// tensor sits at base + row * X_row + head * X_head + dim; rows are
// batch * S + position.
// ---------------------------------------------------------------------------
struct FlashDesc {
  const void* q;  int64_t q_row, q_head;    // [.., 128] nope (or whole) query
  const void* qr; int64_t qr_row, qr_head;  // [.., d_r] rope query (d_r > 0)
  const void* k;  int64_t k_row, k_head;    // [.., 128] keys (nope part)
  const void* kr; int64_t kr_row;           // [.., d_r] shared rope key (d_r > 0)
  const void* v;  int64_t v_row, v_head;    // [.., 128]
  void* o;        int64_t o_row, o_head;    // [.., 128] output
  float* lse;                               // [B * S_q, H] or null
  const void* gate; int64_t g_row, g_head;  // output times sigmoid(gate), or null
  int B, S_q, S_kv, H, d_r;
  float scale;
  bool causal;
};
bool flash_fits(int d_nope, int d_r, int d_v);
int launch_flash(const FlashDesc& f, hipStream_t s);

}  // namespace mla
