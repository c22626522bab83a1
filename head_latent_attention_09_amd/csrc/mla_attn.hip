// Latent attention kernels for gfx950: planning, the bf16 MFMA attention
// kernel (d_c = 512, d_r = 64, 32..128 heads), a generic fp32/bf16 kernel for
// other shapes, and the log-sum-exp combine.
//
// Method (ferrox-core 0.23.0 mla_absorbed.rs module documentation; MLA_tutorial
// formula.md Part 3, inference form): every head's query row [q_abs | q_pe]
// scores against ONE key row per position, [c_t | k_pe_t], shared by all
// heads, and sums the shared value c_t (the d_c prefix of that row):
//   s[h,t] = (q_abs[h].c_t + q_pe[h].k_pe_t) * kq_scale,  out[h] = sum_t softmax(s[h])_t c_t.
// The page's scalar function loops head by head over the whole cache; here a
// tile of positions is streamed from HBM once into LDS and every head of the
// query reads it from there, so the cache is read once per query, not once
// per head.
#include "mla_internal.h"

#include <hip/hip_ext.h>
#include <math.h>

namespace mla {

// ===========================================================================
// planning: visible length and tile prefix sum of every row, the list of
// rows cut by worker boundaries, and the (final) output of empty rows
// ===========================================================================
__device__ __forceinline__ int row_len(const RowMap& m, int r) {
  if (m.mode == 2) {  // prefill, bottom-right causal alignment: t <= i + s_kv - s_q
    if (m.non_causal) return m.s_kv;
    int i = r % m.s_q;
    long long n = (long long)i + 1 + m.s_kv - m.s_q;
    return n < 0 ? 0 : (n > m.s_kv ? m.s_kv : (int)n);
  }
  long long cap = (m.mode == 0) ? (long long)m.cache_stride : (long long)m.max_pages * m.page_size;
  long long n = m.seq_lens[r];
  return n < 0 ? 0 : (int)(n > cap ? cap : n);
}

template <typename OutT>
__global__ __launch_bounds__(1024) void plan_kernel(RowMap m, Plan pl, int H, int d_c, OutT* out, float* lse) {
  __shared__ int wsum_t[16], wsum_r[16], wsum_z[16];
  __shared__ int nsplit;
  __shared__ int zrows[256];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int R = pl.R, tile = pl.tile;
  const int chunk = (R + 1023) / 1024;
  const int r0 = min(tid * chunk, R), r1 = min(r0 + chunk, R);
  if (tid == 0) nsplit = 0;
  int nt = 0, nr = 0, nz0 = 0;  // this thread's tiles, non-empty rows and empty rows
  int n_first = 0;              // the first row's length stays in a register (one row per thread up to 1024 rows)
  for (int r = r0; r < r1; ++r) {
    int n = row_len(m, r);
    if (r == r0) n_first = n;
    pl.len[r] = n;
    nt += (n + tile - 1) / tile;
    nr += n > 0;
    nz0 += n == 0;
  }
  // inclusive scans of the three counts over the block: within each wave by shuffles,
  // then across the 16 wave totals (one barrier)
  int st = nt, sr = nr, sz = nz0;
  for (int o = 1; o < 64; o <<= 1) {
    const int yt = __shfl_up(st, o), yr = __shfl_up(sr, o), yz = __shfl_up(sz, o);
    if (lane >= o) {
      st += yt;
      sr += yr;
      sz += yz;
    }
  }
  if (lane == 63) {
    wsum_t[wid] = st;
    wsum_r[wid] = sr;
    wsum_z[wid] = sz;
  }
  __syncthreads();
  int all_tiles = 0, all_rows = 0, nz = 0;
  for (int i = 0; i < 16; ++i) {
    const int t = wsum_t[i], c = wsum_r[i], z = wsum_z[i];
    if (i < wid) {
      st += t;
      sr += c;
      sz += z;
    }
    all_tiles += t;
    all_rows += c;
    nz += z;
  }
  // list the empty rows (written at the end)
  auto len_of = [&](int r) { return r == r0 ? n_first : pl.len[r]; };
  for (int r = r0, i = sz - nz0; r < r1; ++r)
    if (len_of(r) == 0 && i < 256) zrows[i++] = r;
  // fixed cost per row only when rows are shorter on average than a worker's
  // share of the tiles (many rows per worker); longer rows are cut into about
  // equal pieces anyway, and every piece pays the fixed cost
  const int seg_cost = all_rows > 0 && all_tiles / all_rows < plan_per_worker(all_tiles, pl.G) ? SEG_COST : 0;
  const int total = all_tiles + seg_cost * all_rows;
  const int per = plan_per_worker(total, pl.G);
  if (tid == 0) {
    pl.split[1] = seg_cost;
    pl.cum[R] = total;
  }
  int base = (st - nt) + seg_cost * (sr - nr);  // first unit of this thread's rows
  for (int r = r0; r < r1; ++r) {
    const int n = row_units((len_of(r) + tile - 1) / tile, seg_cost);
    pl.cum[r] = base;
    const int s0 = base + seg_cost;  // first unit of the row's tiles
    if (n > 0 && s0 / per != (base + n - 1) / per) {
      const int w0 = s0 / per;
      *(int4*)(pl.split + 4 + 4 * atomicAdd(&nsplit, 1)) =
          int4{r, plan_slot(w0, s0, per), w0, (base + n - 1) / per - w0 + 1};
    }
    // workers whose range starts inside this row's units begin with this row
    for (int w = (base + per - 1) / per; n > 0 && w * per < base + n && w < pl.G; ++w) pl.wrow[w] = r;
    base += n;
  }
  __syncthreads();
  if (tid == 0) pl.split[0] = nsplit;
  // rows with nothing visible: zeros and lse = -inf (no later kernel touches
  // them). The rare empty rows, listed above, are written by the whole
  // workgroup.
  for (int j = 0; j < (nz < 256 ? nz : 256); ++j) {
    const int r = zrows[j];
    for (int i = tid; i < H * d_c; i += 1024) store_f32(out + (size_t)r * H * d_c + i, 0.f);
    if (lse)
      for (int h = tid; h < H; h += 1024) lse[(size_t)r * H + h] = -INFINITY;
  }
  if (nz > 256) {  // more empty rows than the list holds: each thread writes its own
    for (int r = r0; r < r1; ++r)
      if (len_of(r) == 0) {
        for (int i = 0; i < H * d_c; ++i) store_f32(out + (size_t)r * H * d_c + i, 0.f);
        if (lse)
          for (int h = 0; h < H; ++h) lse[(size_t)r * H + h] = -INFINITY;
      }
  }
}

__device__ __forceinline__ int row_batch(const RowMap& m, int r) { return m.mode == 2 ? r / m.s_q : r; }

// element offset of cache position t of batch entry b (dense and prefill layouts)
__device__ __forceinline__ size_t dense_row(const RowMap& m, int b, int t, int width) {
  size_t stride = m.mode == 2 ? (size_t)m.s_kv : (size_t)m.cache_stride;
  return ((size_t)b * stride + t) * width;
}

// Page of position t of batch entry b. The table is read through the constant
// address space so that wave-uniform lookups become scalar loads (counted
// apart from the vector loads of the tile pipeline).
__device__ __forceinline__ int page_of(const RowMap& m, int b, int t) {
  const __attribute__((address_space(4))) int32_t* bt =
      (const __attribute__((address_space(4))) int32_t*)m.block_table;
  int p = bt[(size_t)b * m.max_pages + t / m.page_size];
  return p < 0 ? 0 : (p >= m.num_pages ? m.num_pages - 1 : p);
}

// Planning inside a kernel, for batches of at most SELF_MAX_R rows: every
// workgroup of 256 threads derives the same unit prefix sums as plan_kernel
// from the row lengths, into LDS (cum_s [R + 1], len_s [R]); returns the
// fixed cost per row and the total. This spares a decode call the planning
// kernel and its launch; the first attention workgroup stores the prefix
// sums, lengths and fixed cost for the combine kernel.
constexpr int SELF_MAX_R = 256;
__device__ void self_plan(const RowMap& m, int R, int G, int tile, int* cum_s, int* len_s, int& seg_cost,
                          int& total) {
  __shared__ int wt[4], wr[4];  // per-wave totals of tiles and non-empty rows
  constexpr int CH = SELF_MAX_R / 256;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r0 = tid * CH;
  int tl[CH];
  int nt = 0, nr = 0;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int r = r0 + j;
    int n = 0;
    if (r < R) {
      n = row_len(m, r);
      len_s[r] = n;
    }
    tl[j] = (n + tile - 1) / tile;
    nt += tl[j];
    nr += n > 0;
  }
  int st = nt, sr = nr;  // inclusive scans: within the wave, then over the 4 wave totals
  for (int o = 1; o < 64; o <<= 1) {
    const int yt = __shfl_up(st, o), yr = __shfl_up(sr, o);
    if (lane >= o) {
      st += yt;
      sr += yr;
    }
  }
  if (lane == 63) {
    wt[wid] = st;
    wr[wid] = sr;
  }
  __syncthreads();
  int all_t = 0, all_r = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < wid) {
      st += wt[i];
      sr += wr[i];
    }
    all_t += wt[i];
    all_r += wr[i];
  }
  const int c = all_r > 0 && all_t / all_r < plan_per_worker(all_t, G) ? SEG_COST : 0;
  int base = (st - nt) + c * (sr - nr);
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int r = r0 + j;
    if (r < R) {
      cum_s[r] = base;
      base += row_units(tl[j], c);
    }
  }
  if (tid == 0) cum_s[R] = all_t + c * all_r;
  __syncthreads();
  seg_cost = __builtin_amdgcn_readfirstlane(c);  // the same in every lane
  total = __builtin_amdgcn_readfirstlane(all_t + c * all_r);
}

// ===========================================================================
// generic attention (fp32 or bf16 storage, any d_c <= 1024, d_c + d_r <= 1152)
// fp32 arithmetic on the vector ALUs; 16 heads per workgroup, 16-position tiles.
// ===========================================================================
namespace gn {
constexpr int TT = 16, HG = 8, WMAX = 1152, DCMAX = 1024, NT = 256;
// heads per workgroup of the standalone kernel: every tile staged in LDS serves
// 16 heads (the query block and the tile fill 148 KiB of LDS); the redo inside
// the MFMA kernel takes 8 at a time in that kernel's smaller scratch
constexpr int HGK = 16;

template <typename T>
struct Args {
  const T* q;
  const T* cache;
  RowMap map;
  Plan pl;
  int H, d_c, d_r;
  float scale_log2;
  T* out;
  float* lse;
};

template <typename T, int HG>
__device__ void attend_segment(const Args<T>& a, int r, int len, int lt0, int lt1, bool full, int slot, int h0,
                               float* tile, float* qs, float* ps, float* alpha_s, float* stat_s,
                               float& m_run, float& l_run) {
  const int tid = threadIdx.x;
  const int W = a.d_c + a.d_r, WP = W + 1, H = a.H, d_c = a.d_c;
  const int nh = min(HG, H - h0);
  const int b = row_batch(a.map, r);
  __syncthreads();
  for (int i = tid; i < HG * W; i += NT) {
    int hh = i / W, d = i - hh * W;
    qs[i] = hh < nh ? load_f32(a.q + ((size_t)r * H + h0 + hh) * W + d) : 0.f;
  }
  float acc[HG][4];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[hh][k] = 0.f;
  if (tid < HG) { m_run = -INFINITY; l_run = 0.f; }

  for (int lt = lt0; lt < lt1; ++lt) {
    const int t0 = lt * TT;
    __syncthreads();
    for (int i = tid; i < TT * W; i += NT) {
      int row = i / W, d = i - row * W;
      int t = min(t0 + row, len - 1);
      size_t off;
      if (a.map.mode == 1) {
        int pg = page_of(a.map, b, t);
        off = ((size_t)pg * a.map.page_size + (t % a.map.page_size)) * W;
      } else {
        off = dense_row(a.map, b, t, W);
      }
      tile[row * WP + d] = load_f32(a.cache + off + d);
    }
    __syncthreads();
    if (tid < HG * TT) {
      const int hh = tid / TT, row = tid % TT;
      float s = 0.f;
      for (int d = 0; d < W; ++d) s += qs[hh * W + d] * tile[row * WP + d];
      ps[hh * TT + row] = (t0 + row < len) ? s * a.scale_log2 : -INFINITY;
    }
    __syncthreads();
    if (tid < HG) {
      float mx = -INFINITY;
      for (int row = 0; row < TT; ++row) mx = fmaxf(mx, ps[tid * TT + row]);
      const float mn = fmaxf(m_run, mx);
      const float al = exp2f(m_run - mn);
      float sum = 0.f;
      for (int row = 0; row < TT; ++row) {
        float p = exp2f(ps[tid * TT + row] - mn);
        ps[tid * TT + row] = p;
        sum += p;
      }
      l_run = l_run * al + sum;
      m_run = mn;
      alpha_s[tid] = al;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = tid + k * NT;
      if (d < d_c) {
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) acc[hh][k] *= alpha_s[hh];
        for (int row = 0; row < TT; ++row) {
          const float c = tile[row * WP + d];
#pragma unroll
          for (int hh = 0; hh < HG; ++hh) acc[hh][k] += ps[hh * TT + row] * c;
        }
      }
    }
  }
  __syncthreads();
  if (tid < HG) {
    stat_s[tid] = 1.0f / l_run;
    stat_s[HG + tid] = (m_run + log2f(l_run)) * kLn2;
  }
  __syncthreads();
  // (a guard, not a break: the loop unrolls fully, so acc stays in registers)
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    if (hh < nh) {
      const int h = h0 + hh;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d = tid + k * NT;
        if (d < d_c) {
          float v = acc[hh][k] * stat_s[hh];
          if (full) store_f32(a.out + ((size_t)r * H + h) * d_c + d, v);
          else store_f32((T*)a.pl.part_o + ((size_t)slot * H + h) * d_c + d, v);
        }
      }
      if (tid == 0) {
        if (full) { if (a.lse) a.lse[(size_t)r * H + h] = stat_s[HG + hh]; }
        else a.pl.part_lse[(size_t)slot * H + h] = stat_s[HG + hh];
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void attn_generic_kernel(Args<T> a) {
  __shared__ float tile[TT * (WMAX + 1)];
  __shared__ float qs[HGK * WMAX];
  __shared__ float ps[HGK * TT];
  __shared__ float alpha_s[HGK];
  __shared__ float stat_s[2 * HGK];
  float m_run = -INFINITY, l_run = 0.f;
  const int G = a.pl.G;
  const int w = xcd_worker(blockIdx.x, G);
  const int h0 = blockIdx.y * HGK;
  const int total = a.pl.cum[a.pl.R];
  const int seg_cost = a.pl.split[1];
  const int per = plan_per_worker(total, G);
  const int t_begin = w * per;
  if (t_begin >= total) return;
  const int t_end = min(t_begin + per, total);
  for (int r = a.pl.wrow[w]; r < a.pl.R; ++r) {
    const int c0 = a.pl.cum[r], c1 = a.pl.cum[r + 1];
    if (c0 >= t_end) break;
    Segment sg;
    if (!plan_segment(c0, c1, seg_cost, t_begin, t_end, w, per, sg)) continue;
    attend_segment<T, HGK>(a, r, a.pl.len[r], sg.lt0, sg.lt1, sg.full, sg.slot, h0, tile, qs, ps, alpha_s, stat_s,
                           m_run, l_run);
  }
}
}  // namespace gn

// ===========================================================================
// bf16 MFMA attention: d_c = 512, d_r = 64, 32..128 heads
// ===========================================================================
namespace mf {
constexpr int DC = 512, DR = 64, WD = 576;
constexpr int TILE = 16;                     // positions per tile
constexpr int C_BYTES = TILE * DC * 2;       // latent rows: 16 x 1024 B
constexpr int TILE_BYTES = TILE * WD * 2;    // + rope rows: 16 x 128 B = 18 KiB
constexpr int NBUF = 4;                      // tile buffers in LDS
static_assert((NBUF & (NBUF - 1)) == 0, "buffer indices are taken with & (NBUF - 1)");
constexpr int AHEAD = NBUF - 1;              // tiles issued ahead of the tile whose values are read
constexpr int KS = WD / 32;                  // k-steps of 32 dims in the score contraction (18)
constexpr int KL = DC / 32;                  // k-steps over the latent dims (16); the rest are rope dims
constexpr int KQ = 14;                       // k-steps whose query operand stays in registers
constexpr int NW = 4;                        // waves per workgroup
constexpr int QR_ROW = (WD - 32 * KQ) * 2 + 32;     // query rest: bytes per head row (32 B of padding)
constexpr int QR_BYTES = 9 * 1024;                  // per wave: 32 rows of QR_ROW bytes, in whole 1 KiB loads
static_assert(32 * QR_ROW <= QR_BYTES, "query block in LDS");
constexpr int P_BYTES = 32 * NW * TILE * 2;  // bf16 softmax weights of one tile, 128 heads (4 KiB)
constexpr int RING = 5;                      // score operand (tile) reads in flight per wave
constexpr int QA = 2;                        // k-steps the query operand reads from LDS run ahead
constexpr int DW = DC / NW;                  // output dims per wave in the value product
constexpr float SLACK = 0x1p64f;             // bound on a segment's sum of weights 2^(s - m_ref)
constexpr int LDS_QR = NBUF * TILE_BYTES;
constexpr int LDS_P = LDS_QR + NW * QR_BYTES;
constexpr int LDS_INV = LDS_P + 2 * P_BYTES;
constexpr int LDS_MFIX = LDS_INV + 32 * NW * 4;   // a redo's softmax reference per head
constexpr int SMEM_BYTES = LDS_MFIX + 32 * NW * 4;

// Work split inside a workgroup (4 waves, one per SIMD). Scores and softmax
// weights are split by head: wave w owns heads 32w .. 32w+31 and computes
// S^T = K_tile Q^T for them (18 k-steps x 2 head blocks of 16x16x32). The
// bf16 weights go through LDS and the value product is split by output dims:
// wave w accumulates O^T[128w .. 128w+127][all heads] (4 x 4 MFMAs of
// 32x32x16), so each wave reads a quarter of the tile's values.
//
// Software pipeline, one workgroup barrier per tile. Iteration i:
//   scores of tile i+1, with the loads of tile i+AHEAD between the MFMAs,
//   and the softmax of tile i (scores from the previous iteration; written
//   between the MFMAs too, the compiler places most of it after the chain;
//   forcing it to stay there measured 1-2 % slower); value fragments of tile
//   i; weights of tile i to LDS; barrier; weight fragments of tile i and the
//   first score operands of tile i+2; value product of tile i.
// Tile j is loaded into buffer j % NBUF during iteration j - AHEAD, after the
// barrier that ends every read of the buffer's previous tile j - NBUF (its
// value fragments are read, and waited for, before the barrier of iteration
// j - NBUF), and published by the barrier of iteration j - 2. Every
// iteration does the same work: the last ones load and score stand-in tiles
// past the segment's end (results unused), so the loop has no branches on
// the tile index and each wave has the same loads in flight at every wait.
//
// LDS layouts (XOR swizzles; chosen with the LDS bank-conflict counter on
// this chip, since its banking is not a plain 4-byte interleave: the score
// operand reads, the transposing value reads and the query reads below
// count no conflict):
//   tile latent row t at t*1024, 16-byte chunk c at c ^ sC(t) inside its
//     aligned group of 16 chunks; rope row t at C_BYTES + t*128, chunk c at
//     c ^ sR(t);
//   query dims 32KQ .. 575: wave block of 32 rows of QR_ROW bytes (32 bytes
//     of padding per row);
//   weights: head hh at hh*32 (16 positions), 8-byte quarter q at
//     q ^ (2 * ((hh >> 3) & 1)).
// sC is linear in the bits of t (sC(a | b) = sC(a) ^ sC(b) for disjoint a, b)
// and a permutation of 0..15 over the 16 rows of a tile.
__device__ __forceinline__ int sC(int r) {
  return ((r & 1) ? 4 : 0) ^ ((r & 2) ? 8 : 0) ^ ((r & 4) ? 3 : 0) ^ ((r & 8) ? 6 : 0);
}
__device__ __forceinline__ int sR(int r) { return (r ^ (r >> 3)) & 7; }

struct Args {
  const bf16* q;
  const bf16* cache;
  RowMap map;
  Plan pl;
  int H;
  float scale_log2;  // kq_scale * log2(e): scores in log2 units
  bf16* out;
  float* lse;
};

typedef short s16x8 __attribute__((ext_vector_type(8)));

// Score MFMAs with the accumulator pinned to VGPRs (the AGPRs hold the output
// accumulator). Invisible to the compiler's hazard checker, so the code covers
// both sides itself. Before the MFMA: an operand written by a VALU
// instruction needs two wait states; GUARD adds them, for kernels whose free
// AGPRs the compiler uses to park query registers (fewer than 128 heads: it
// copies them back right before the MFMA). With 128 heads every AGPR holds the
// output and no such copy is made; a CPU test scans the generated code of
// every instantiation for a VALU write of an operand within two wait states
// of an unguarded MFMA. After the chain: the last k-step's two MFMAs and the
// wait states a read of their results needs are one asm block (mfma16_last),
// so no instruction the compiler places after it, a register copy included,
// can read a result too early.
template <bool GUARD>
__device__ __forceinline__ void mfma16(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  if (GUARD)
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
template <bool GUARD>
__device__ __forceinline__ void mfma16_last(f32x4& c0, f32x4& c1, const bf16x8& a, const bf16x8& b0,
                                            const bf16x8& b1) {
  if (GUARD)
    asm volatile(
        "s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %2, %3, %0\n\tv_mfma_f32_16x16x32_bf16 %1, %2, %4, %1\n\t"
        "s_nop 7\n\ts_nop 7\n\ts_nop 3"
        : "+v"(c0), "+v"(c1)
        : "v"(a), "v"(b0), "v"(b1));
  else
    asm volatile(
        "v_mfma_f32_16x16x32_bf16 %0, %2, %3, %0\n\tv_mfma_f32_16x16x32_bf16 %1, %2, %4, %1\n\t"
        "s_nop 7\n\ts_nop 7\n\ts_nop 3"
        : "+v"(c0), "+v"(c1)
        : "v"(a), "v"(b0), "v"(b1));
}
template <bool GUARD>
__device__ __forceinline__ void mfma16_first(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  if (GUARD)
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}

// Direct global->LDS load of 64 lanes x 16 bytes: lane l reads 16 bytes at
// gbase + voff and writes them to LDS address lds + 16 l. Issued from inline
// asm so that the compiler does not know about the LDS write: it would
// otherwise wait for every such load in flight before any LDS read it cannot
// prove disjoint, which serialises the tile pipeline. Completion is waited
// for explicitly (vmcnt) before the workgroup barrier that publishes a tile.
// M0 holds the LDS base; one wait state is required between writing M0 and
// the load that reads it. The kernel makes no other use of M0.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(gbase), "s"(lds) : "memory");
}
// Cache tile loads. Decode reads each cache row once: non-temporal, so the
// stream does not displace reused lines (measured 1.27x the streaming rate
// of the default policy for this load pattern). A causal prefill reads the
// same rows for every query of the sequence: default policy, so they stay
// in L2 (measured 7 % faster there).
template <bool STREAM>
__device__ __forceinline__ void dma16_tile(const void* gbase, uint32_t voff, uint32_t lds) {
  if (STREAM)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(voff), "s"(gbase), "s"(lds) : "memory");
  else
    dma16(gbase, voff, lds);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const MLA_LDS char*)p;
}

// Keep a value's uses inside the loop that contains this call: the compiler
// would otherwise hoist per-lane values derived from it out of the loop and
// hold (or spill) one register per use.
template <typename T>
__device__ __forceinline__ void opaque(T& x) {
  asm volatile("" : "+v"(x));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "");
  // vmcnt in bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15) left unconstrained
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// vmcnt wait for the tile loads issued after the one being waited for:
// AHEAD - 2 tiles of this wave's loads (5 for waves 0 and 1, 4 for the others)
// plus EXTRA later loads
template <int EXTRA>
__device__ __forceinline__ void wait_tiles(int wv) {
  if (wv < 2)
    wait_vmcnt<(AHEAD - 2) * 5 + EXTRA>();
  else
    wait_vmcnt<(AHEAD - 2) * 4 + EXTRA>();
}

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14)); }

// v from lane (ln ^ mask); ln is the caller's (opaque) lane id
__device__ __forceinline__ float shfl_xor(float v, int ln, int mask) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((ln ^ mask) << 2, __builtin_bit_cast(int, v)));
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Source of one tile: row 0 of positions t0 .. t0+15 of batch entry b in
// global memory, and the last row of it that is visible.
struct TileSrc {
  const char* p;
  int last;
  int lastb;  // byte offset of the last visible row from row 0
};

__device__ __forceinline__ TileSrc tile_src(const Args& a, int b, int t0, int len) {
  const RowMap& m = a.map;
  TileSrc s;
  if (m.mode == 1) {
    const int pg = page_of(m, b, t0);
    s.p = (const char*)(a.cache + ((size_t)pg * m.page_size + (t0 % m.page_size)) * WD);
  } else {
    s.p = (const char*)(a.cache + dense_row(m, b, t0, WD));
  }
  s.last = len - 1 - t0;
  s.lastb = s.last * (WD * 2);
  return s;
}

// Loads of one tile: 18 loads of 64 lanes x 16 B. Load k < 4 of wave wv fills
// latent row wv + 4k (1 KiB); load 4 of waves 0 and 1 the rope chunks of
// rows 8wv .. 8wv+7 (one load issue costs the issuing wave about as much as
// another, so the two rope loads are not split four ways). Rows past the last
// visible one re-read it (finite data; their weights are zeroed). lx is
// lane ^ sC(wv): sC(wv + 4k) = sC(wv) ^ sC(4k).
template <bool STREAM>
__device__ __forceinline__ void issue_load(const TileSrc& s, char* buf, int k, int lx, int lane, int wv) {
  if (k < 4) {
    const int ld = wv + NW * k;
    const int row = ld < s.last ? ld : s.last;
    dma16_tile<STREAM>(s.p + (size_t)row * (WD * 2), (uint32_t)((lx ^ sC(4 * k)) << 4), lds_addr(buf + ld * 1024));
  } else if (wv < 2) {
    const int rl = 8 * wv + (lane >> 3);
    const int row = rl < s.last ? rl : s.last;
    dma16_tile<STREAM>(s.p, (uint32_t)(row * (WD * 2) + DC * 2 + (((lane & 7) ^ sR(rl)) << 4)),
                 lds_addr(buf + C_BYTES + wv * 1024));
  }
}

template <bool STREAM>
__device__ __forceinline__ void issue_tile(const TileSrc& s, char* buf, int lx, int lane, int wv) {
#pragma unroll
  for (int k = 0; k < 5; ++k) issue_load<STREAM>(s, buf, k, lx, lane, wv);
}


// A segment redone by the generic kernel's code (running maximum with
// rescaling, 8 heads at a time), writing the same outputs as attend_segment:
// for a segment whose weights overflowed fp32 (a score 128 or more log2
// units above its first tile's maximum). The tile ring serves as its scratch.
__device__ void generic_segment(const Args& a, int r, int len, int lt0, int lt1, bool full, int slot, char* smem) {
  gn::Args<bf16> ga;
  ga.q = a.q;
  ga.cache = a.cache;
  ga.map = a.map;
  ga.pl = a.pl;
  ga.H = a.H;
  ga.d_c = DC;
  ga.d_r = DR;
  ga.scale_log2 = a.scale_log2;
  ga.out = a.out;
  ga.lse = a.lse;
  float* tile = (float*)smem;
  float* qs = tile + gn::TT * (gn::WMAX + 1);
  float* ps = qs + gn::HG * gn::WMAX;
  float* alpha_s = ps + gn::HG * gn::TT;
  float* stat_s = alpha_s + gn::HG;
  static_assert((gn::TT * (gn::WMAX + 1) + gn::HG * (gn::WMAX + gn::TT + 3)) * 4 <= SMEM_BYTES, "generic scratch");
  float m_run = -INFINITY, l_run = 0.f;
  for (int h0 = 0; h0 < a.H; h0 += gn::HG)
    gn::attend_segment<bf16, gn::HG>(ga, r, len, lt0, lt1, full, slot, h0, tile, qs, ps, alpha_s, stat_s, m_run,
                                     l_run);
  __syncthreads();
}

// One segment (tiles lt0 .. lt1-1 of row r). On a first pass the softmax
// reference of each owned head is the largest score of the first tile; on a
// redo (seg_flag[1] set) it is the reference stored at LDS_MFIX. Returns 0
// once the segment's outputs are written. When the first-tile reference
// overflowed (see the reference note at the end) it writes nothing and
// returns 1, having stored a safe reference for a redo and set seg_flag[1],
// or 2 when the weights themselves overflowed. The redo state lives in LDS,
// not registers: values held in registers across the segment pushed the
// kernel into spills whose reloads drain the tile loads in flight.
template <int NHB, bool STREAM>
__device__ __forceinline__ int attend_segment(const Args& a, int r, int len, int lt0, int lt1, bool full, int slot,
                                               char* smem, int* seg_flag, int lane, int wv) {
  constexpr int H = 32 * NHB;
  const int b = row_batch(a.map, r);
  const bool owner = NHB >= NW || wv < NHB;  // the wave scores heads 32wv .. 32wv+31 (known at 128 heads)
  // Waves without heads (fewer than 128) also load a query block and score
  // the first tile (results unused): every path into the tile loop then passes
  // the compiler's waits for the query registers.
  const int wq = owner ? wv : 0;
  const int ntiles = lt1 - lt0;
  char* const qr_lds = smem + LDS_QR + wv * QR_BYTES;
  float* const inv_s = (float*)(smem + LDS_INV);
  float* const m_fix_s = (float*)(smem + LDS_MFIX);
  auto tbuf = [&](int j) { return smem + (j % NBUF) * TILE_BYTES; };
  // Source of tile j of the segment. Past the segment's end the pipeline
  // still loads a tile, so that every step has the same loads in flight and
  // runs without branches: row 0 of the segment's last tile (a visible row)
  // into every row, into a buffer whose scores are never used.
  auto src_of = [&](int j) {
    TileSrc s = tile_src(a, b, (lt0 + (j < ntiles ? j : ntiles - 1)) * TILE, len);
    if (j >= ntiles) s.last = s.lastb = 0;
    return s;
  };

  // every wave must be done with the previous segment's LDS (and flag)
  block_barrier();
  if (threadIdx.x == 0) *seg_flag = 0;

  // ---- prologue: tiles 0 and 1, the query's rope dims to LDS, tiles 2 ..
  // AHEAD-1, the query's latent dims to registers (B operand of 16x16x32:
  // lane l holds head 16hb + l%16 of the wave's 32, dims 32ks + 8(l/16) .. +7)
  bf16x8 qf[2][KQ];
  {
    int ln = lane;  // per-lane offsets stay in this segment's code (see the tile loop)
    opaque(ln);
    const int lx = ln ^ sC(wv);
    for (int j = 0; j < 2; ++j) issue_tile<STREAM>(src_of(j), tbuf(j), lx, ln, wv);
    {
      const char* qbase = (const char*)(a.q + ((size_t)r * H + wq * 32) * WD + 32 * KQ);
      constexpr int QC = QR_ROW / 16;  // 16-byte slots per row, the last two padding
#pragma unroll
      for (int k = 0; k < QR_BYTES / 1024; ++k) {
        const int p = k * 64 + ln;  // 16-byte slot of this wave's block
        int hr = p / QC, pc = p - hr * QC;
        if (hr > 31 || pc >= QC - 2) hr = pc = 0;  // padding and slack: any valid chunk
        dma16(qbase, (uint32_t)(hr * (WD * 2) + (pc << 4)), lds_addr(qr_lds + k * 1024));
      }
    }
    for (int j = 2; j < AHEAD; ++j) issue_tile<STREAM>(src_of(j), tbuf(j), lx, ln, wv);
    {
      const bf16* qrow = a.q + ((size_t)r * H + wq * 32 + (ln & 15)) * WD + (ln >> 4) * 8;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int ks = 0; ks < KQ; ++ks) qf[hb][ks] = *(const bf16x8*)(qrow + hb * 16 * WD + ks * 32);
    }
    // tiles 0, 1 and the query rope dims complete; the later tiles and the
    // query registers (waited for by the compiler) may be in flight
    wait_tiles<2 * KQ>(wv);
  }
  block_barrier();

  // ---- per-lane LDS offsets, computed once per segment from an opaque lane
  // id (values derived from the plain lane id get hoisted out of the segment
  // loop and spilled); per tile only the buffer base is added
  int ln = lane;
  opaque(ln);
  const int t16 = ln & 15, q4 = ln >> 4;
  // score A operand (tile rows, lane: row l%16, dims 8(l/16) .. +7 of the
  // k-step): latent k-step ks: chunk 4ks + l/16 at (4(ks&3) + l/16) ^ sC(row)
  // in group ks/4, i.e. kofs[ks&3] + 256(ks/4); rope k-steps at rofs[]
  int kofs[4], rofs[2];
  {
    const int y = q4 ^ sC(t16);
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) kofs[a4] = t16 * 1024 + 16 * (y & 3) + 64 * (a4 ^ (y >> 2));
    const int pr = q4 ^ sR(t16);
    rofs[0] = C_BYTES + t16 * 128 + 16 * pr;
    rofs[1] = C_BYTES + t16 * 128 + 16 * (pr ^ 4);
  }
  // score B operand of k-steps KQ + k (query dims in LDS): chunk 4k + l/16 of
  // row 16hb + l%16
  const int qofs = LDS_QR + wv * QR_BYTES + t16 * QR_ROW + 16 * q4;
  // value A operand (transposing loads, lane l: dim 128wv + 32d + l%32,
  // positions 8(l/32) .. +3 from vofs[d], +4 .. +7 from vofs[4 + d])
  // (rows tA and tA + 4 have the same sC bits 2-3: vx = 64 (sC >> 2) serves both)
  int vA, vB, vx;
  {
    const int tA = 8 * (q4 >> 1) + (t16 >> 2), tB = tA + 4;
    const int cb = 2 * (q4 & 1) + ((t16 & 3) >> 1);
    const int sA = sC(tA), sB = sC(tB);
    vA = tA * 1024 + ((cb ^ (sA & 3)) << 4) + (t16 & 1) * 8 + 256 * wv;
    vB = tB * 1024 + ((cb ^ (sB & 3)) << 4) + (t16 & 1) * 8 + 256 * wv;
    vx = (sA >> 2) << 6;
  }
  // weights: this lane's 4 positions of head 32wv + 16hb + l%16 (write), and
  // positions 8(l/32) .. +7 of head 32hb + l%32 (read)
  const int pwo = LDS_P + (wv * 32 + t16) * 32 + ((q4 ^ (2 * ((ln >> 3) & 1))) << 3);
  const int pro = LDS_P + (ln & 31) * 32 + (((ln >> 5) ^ ((ln >> 3) & 1)) << 4);
  // tile loads: latent load k reads chunk (lane ^ sC(wv) ^ sC(4k)); the rope load
  // (waves 0, 1) reads row 8wv + l/8, chunk (l&7) ^ sR(row)
  const int dofs = (ln ^ sC(wv)) << 4;
  const int rrow = 8 * wv + (ln >> 3);
  const int rdofs = DC * 2 + (((ln & 7) ^ sR(rrow)) << 4);

  auto load_tile = [&](const TileSrc& s, int boff, int k) {
    char* buf = smem + boff;
    if (k < 4) {
      // the row offset (clamped to the last visible row) rides in the lane offset; the base is the tile's
      // (wvb is made opaque here so that the four rows' offsets are not each kept in a register)
      const int ld = wv + NW * k;
      int wvb = wv * (WD * 2);
      asm volatile("" : "+s"(wvb));
      const int rb = wvb + k * NW * (WD * 2);
      const int rowb = rb < s.lastb ? rb : s.lastb;
      dma16_tile<STREAM>(s.p, (uint32_t)((dofs ^ (sC(4 * k) << 4)) + rowb), lds_addr(buf + ld * 1024));
    } else if (wv < 2) {
      const int row = rrow < s.last ? rrow : s.last;
      dma16_tile<STREAM>(s.p, (uint32_t)(row * (WD * 2) + rdofs), lds_addr(buf + C_BYTES + wv * 1024));
    }
  };

  float m_ref[2] = {0.f, 0.f};  // per owned head: reference max (log2 units)
  float lsum[2] = {0.f, 0.f};   // per owned head: this lane's part of the denominator
  f32x4 s0[2], s1[2];           // scores of two consecutive tiles (S^T blocks per 16 heads)
  bf16x8 kr[RING];              // score operand ring
  f32x16 o[NHB][4];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int d = 0; d < 4; ++d) o[hb][d] = f32x16{};

  auto kread = [&](int boff, int ks) -> bf16x8 {
    const int off = ks < KL ? kofs[ks & 3] + 256 * (ks >> 2) : rofs[ks - KL];
    return *(const MLA_LDS bf16x8*)(smem + boff + off);
  };
  auto kprefetch = [&](int boff) {
#pragma unroll
    for (int i = 0; i < RING; ++i) kr[i] = kread(boff, i);
  };

  // scores of the tile in buffer boff into acc; `between(ks)` runs after the
  // MFMAs of k-step ks
  auto scores = [&](int boff, f32x4* acc, auto between) {
    bf16x8 qx[KS - KQ][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 b0 = ks < KQ ? qf[0][ks] : qx[ks - KQ][0];
      const bf16x8 b1 = ks < KQ ? qf[1][ks] : qx[ks - KQ][1];
      const bf16x8 a_op = kr[ks % RING];
      __builtin_amdgcn_sched_barrier(0);
      if (ks == 0) {
        mfma16_first<(NHB < 4)>(acc[0], a_op, b0);
        mfma16_first<(NHB < 4)>(acc[1], a_op, b1);
      } else if (ks == KS - 1) {
        mfma16_last<(NHB < 4)>(acc[0], acc[1], a_op, b0, b1);
      } else {
        mfma16<(NHB < 4)>(acc[0], a_op, b0);
        mfma16<(NHB < 4)>(acc[1], a_op, b1);
      }
      if (ks + RING < KS) kr[ks % RING] = kread(boff, ks + RING);
      if (ks + QA >= KQ && ks + QA < KS) {
        qx[ks + QA - KQ][0] = *(const MLA_LDS bf16x8*)(smem + qofs + 64 * (ks + QA - KQ));
        qx[ks + QA - KQ][1] = *(const MLA_LDS bf16x8*)(smem + qofs + 64 * (ks + QA - KQ) + 16 * QR_ROW);
      }
      between(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // first tile's scores and the segment's reference max
  kprefetch(0);
  scores(0, s0, [](int) {});
  {
    const int nvalid = len - lt0 * TILE;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float mx = -INFINITY;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, 4 * q4 + rr < nvalid ? s0[hb][rr] * a.scale_log2 : -INFINITY);
      mx = fmaxf(mx, shfl_xor(mx, ln, 16));
      mx = fmaxf(mx, shfl_xor(mx, ln, 32));
      m_ref[hb] = mx;
    }
    if (seg_flag[1]) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) m_ref[hb] = m_fix_s[wv * 32 + hb * 16 + t16] * kLog2e + 1.f;
    }
  }
  if (owner) kprefetch(TILE_BYTES);

  // One pipeline step (tile it, scores in sc; scores of tile it+1 into sn).
  auto step = [&](int it, f32x4* sc, f32x4* sn) {
    const int boff = (it % NBUF) * TILE_BYTES;
    const int nvalid = len - (lt0 + it) * TILE;  // positions < nvalid of this tile are visible
    TileSrc ns = src_of(it + AHEAD);             // loaded during this step
    // materialise the (possibly table-derived) source now: a scalar-load wait
    // later would also drain the operand reads in flight
    asm volatile("" : "+s"(ns.p), "+s"(ns.last), "+s"(ns.lastb));
    const int nboff = ((it + AHEAD) % NBUF) * TILE_BYTES;

    // ---- softmax of tile it: weights 2^(s - m_ref) (see the reference note
    // below), two at a time, written between the score MFMAs of tile it+1
    // (the last step scores the stand-in past the segment's end). The
    // denominator sums exactly the bf16 weights the value MFMAs use (a dot
    // product of each rounded pair with (1, 1)).
    bf16x2 pp[4];  // pair p: positions 4(l/16) + 2(p&1) + {0, 1} of head block p/2
    // Positions past the visible length (last tile only) get weight 0: their
    // rows repeat the last visible row (finite values for the value product)
    // and their scores are set to -inf, whose weight 2^-inf is exactly 0.
    if (nvalid < TILE) {
      const int lim = nvalid - 4 * q4;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          sc[hb][rr] = rr < lim ? sc[hb][rr] : -INFINITY;
    }
    auto soft2 = [&](int p) {
      const int hb = p >> 1, r0 = 2 * (p & 1);
      const float x0 = sc[hb][r0] * a.scale_log2 - m_ref[hb];
      const float x1 = sc[hb][r0 + 1] * a.scale_log2 - m_ref[hb];
      const float w0 = __builtin_amdgcn_exp2f(x0), w1 = __builtin_amdgcn_exp2f(x1);
      bf16x2 q;
      q[0] = f32_to_bf16(w0);
      q[1] = f32_to_bf16(w1);
      pp[p] = q;
      const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
      lsum[hb] = __builtin_amdgcn_fdot2_f32_bf16(q, ones, lsum[hb], false);
    };
    if (owner) {
      // pairs 0..3 after k-steps 1, 5, 9, 13; loads 0..4 after k-steps 0, 4, .., 16
      scores(((it + 1) % NBUF) * TILE_BYTES, sn, [&](int ks) {
        if ((ks & 3) == 1 && ks < 16) soft2(ks >> 2);
        if ((ks & 3) == 0) load_tile(ns, nboff, ks >> 2);
      });
      const int pw = pwo + (it & 1) * P_BYTES;
      *(MLA_LDS bf16x4*)(smem + pw) = __builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3);
      *(MLA_LDS bf16x4*)(smem + pw + 16 * 32) = __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3);
    } else {
#pragma unroll
      for (int k = 0; k < 5; ++k) load_tile(ns, nboff, k);
    }

    // ---- V^T fragments of this wave's dims
    s16x4 va[4], vb[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int xo = vx ^ (d << 6);
      va[d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(smem + boff + vA + xo));
      vb[d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(smem + boff + vB + xo));
    }

    // tile it+2 complete (published by this barrier); tile it+3 in flight
    wait_tiles<0>(wv);
    wait_lgkm0();
    block_barrier();  // weights of tile it and tile it+2 visible

    // ---- weight fragments (B operand of 32x32x16: lane l holds head
    // 32hb + l%32, positions 8(l/32) .. +7) and the first score operands of tile it+2
    bf16x8 pf[NHB];
    {
      const int pr = pro + (it & 1) * P_BYTES;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) pf[hb] = *(const MLA_LDS bf16x8*)(smem + pr + hb * 32 * 32);
    }
    if (owner) kprefetch(((it + 2) % NBUF) * TILE_BYTES);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const s16x8 v8 = __builtin_shufflevector(va[d], vb[d], 0, 1, 2, 3, 4, 5, 6, 7);
        o[hb][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8), pf[hb], o[hb][d], 0, 0,
                                                           0);
      }
  };
  for (int it = 0; it < ntiles; ++it) {
    step(it, s0, s1);
    s0[0] = s1[0];
    s0[1] = s1[1];
  }
  wait_vmcnt<0>();  // the stand-in tiles' loads end before the ring is reused

  // Softmax reference. Each head's reference max m_ref is the largest score
  // of the segment's first tile and the weights are 2^(x - m_ref). Keeping
  // the reference fixed keeps the output accumulator free of data-dependent
  // rescaling (a conditional rescale moves it out of the accumulation
  // registers). A later score far above m_ref shows in the sum of weights l:
  // a segment whose sum reaches SLACK = 2^64 is abandoned before anything is
  // written and redone alone. While l is finite it bounds every weight, so
  // the largest score x_max (log2 units) of each head satisfies
  // x_max <= m_ref + log2 l + 2^-8 (bf16 rounding of a weight) and
  // x_max >= m_ref + log2 l - log2 n (n positions): the redo takes
  // m_ref + log2 l + 1 as the reference, its weights are at most 1/2 and the
  // largest at least 1/(4n), so it neither overflows nor underflows. A sum
  // that is inf or NaN (a weight past the fp32 range: a score 128 or more
  // above m_ref) sends the segment to the generic running-max code. Either
  // way only this segment is redone; the combine merges it like any other
  // part. Measured on the B=64, S=4096 decode: a 69-nat spike in one row
  // costs 1.4x the normal call; the redo path makes the normal call about
  // 1 % slower than a kernel without one, where a running maximum kept in
  // the tile loop cost 3 %. Below 64 (log2 units) above m_ref the weights,
  // sums and outputs stay far inside the range of bf16 and fp32.
  int le = lane;  // per-lane values of the epilogue stay here (see the tile loop)
  opaque(le);
  float lse_v[2] = {0.f, 0.f};
  if (owner) {
    bool over = false, inf = false;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float l = lsum[hb];
      l += shfl_xor(l, le, 16);
      l += shfl_xor(l, le, 32);
      over |= !(l < SLACK);  // also catches inf and NaN
      inf |= !(l < INFINITY);
      lse_v[hb] = (m_ref[hb] + __log2f(l)) * kLn2;
      if (le < 16) {
        inv_s[wv * 32 + hb * 16 + le] = 1.0f / l;
        m_fix_s[wv * 32 + hb * 16 + le] = lse_v[hb];  // a redo's reference is m_ref + log2 l + 1
      }
    }
    const bool any_inf = __any(inf);
    if (__any(over) && le == 0) atomicOr(seg_flag, any_inf ? 3 : 1);
  }
  __syncthreads();
  if (*seg_flag) {
    const int st = (*seg_flag & 2) ? 2 : 1;
    if (st == 1 && threadIdx.x == 0) seg_flag[1] = 1;  // read by every thread before the barrier above
    return st;
  }

  // ---- finish: normalise, write the final row or this worker's partial (bf16)
  if (owner && le < 16) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = wv * 32 + hb * 16 + le;
      if (full) {
        if (a.lse) a.lse[(size_t)r * H + h] = lse_v[hb];
      } else {
        a.pl.part_lse[(size_t)slot * H + h] = lse_v[hb];
      }
    }
  }
  // The output is staged through LDS (the tile ring is free now) so that
  // every global store writes whole 1 KiB rows: the accumulator layout holds
  // 4 dims of 32 heads per store, which would write partial cache lines.
  // Head blocks are staged two at a time (64 rows of OROW bytes).
  const int g = le >> 5;
  bf16* const dst = full ? a.out + (size_t)r * H * DC : (bf16*)a.pl.part_o + (size_t)slot * H * DC;
  constexpr int OROW = DC * 2 + 16;  // 16 bytes of padding spread a column's rows over the banks
  static_assert(64 * OROW <= NBUF * TILE_BYTES, "output staging fits the tile ring");
#pragma unroll
  for (int half = 0; half < (NHB + 1) / 2; ++half) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int hb = 2 * half + h2;
      if (hb >= NHB) break;
      const int hh = 32 * hb + (le & 31);
      const float inv = inv_s[hh];
      char* lrow = smem + (32 * h2 + (le & 31)) * OROW + 2 * DW * wv;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          bf16x4 v;
          v[0] = f32_to_bf16(o[hb][d][4 * rq + 0] * inv);
          v[1] = f32_to_bf16(o[hb][d][4 * rq + 1] * inv);
          v[2] = f32_to_bf16(o[hb][d][4 * rq + 2] * inv);
          v[3] = f32_to_bf16(o[hb][d][4 * rq + 3] * inv);
          *(MLA_LDS bf16x4*)(lrow + 2 * (d * 32 + 8 * rq + 4 * g)) = v;
        }
    }
    __syncthreads();
    const int nrows = H - 64 * half < 64 ? H - 64 * half : 64;
    for (int i = wv; i < nrows; i += NW)
      *(bf16x8*)(dst + (size_t)(64 * half + i) * DC + 8 * le) = *(const MLA_LDS bf16x8*)(smem + i * OROW + 16 * le);
    __syncthreads();  // the staging rows are read before the next half overwrites them
  }
  return 0;
}

// SELF: the workgroup plans for itself (self_plan) instead of reading the
// planning kernel's results.
template <int NHB, bool STREAM, bool SELF>
__global__ __launch_bounds__(NW * 64, 1) void attn_mfma_kernel(Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[SMEM_BYTES];
  __shared__ int seg_flag[2];  // [0] overflow of this pass, [1] the pass is a redo
  __shared__ int cum_s[SELF ? SELF_MAX_R + 1 : 1], len_s[SELF ? SELF_MAX_R : 1];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int G = a.pl.G, R = a.pl.R;
  const int w = xcd_worker(blockIdx.x, G);
  if (threadIdx.x == 0) seg_flag[1] = 0;  // published by the first segment's opening barrier
  int total, seg_cost;
  if constexpr (SELF) {
    self_plan(a.map, R, G, TILE, cum_s, len_s, seg_cost, total);
    if (blockIdx.x == 0) {  // the combine kernel reads the plan of the rows from here
      for (int r = threadIdx.x; r <= R; r += blockDim.x) {
        a.pl.cum[r] = cum_s[r];
        if (r < R) a.pl.len[r] = len_s[r];
      }
      if (threadIdx.x == 0) a.pl.split[1] = seg_cost;
    }
  } else {
    total = a.pl.cum[R];
    seg_cost = a.pl.split[1];
  }
  const int per = plan_per_worker(total, G);
  const int t_begin = w * per;
  if (t_begin >= total) return;
  const int t_end = min(t_begin + per, total);
  int first;  // the row holding unit t_begin
  if constexpr (SELF) {
    int lo = 0, hi = R;  // largest r with cum_s[r] <= t_begin
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cum_s[mid] <= t_begin) lo = mid;
      else hi = mid - 1;
    }
    first = __builtin_amdgcn_readfirstlane(lo);  // LDS values are the same in every lane
  } else {
    first = a.pl.wrow[w];
  }
  for (int r = first; r < R; ++r) {
    const int c0 = SELF ? __builtin_amdgcn_readfirstlane(cum_s[r]) : a.pl.cum[r];
    const int c1 = SELF ? __builtin_amdgcn_readfirstlane(cum_s[r + 1]) : a.pl.cum[r + 1];
    if (c0 >= t_end) break;
    Segment sg;
    if (!plan_segment(c0, c1, seg_cost, t_begin, t_end, w, per, sg)) continue;
    const int len = SELF ? __builtin_amdgcn_readfirstlane(len_s[r]) : a.pl.len[r];
    // a redo with the bound from the sum of weights, or the generic code
    // (also for a second overflow, possible only for non-finite inputs); two
    // call sites measured faster than one inside a loop
    int st = attend_segment<NHB, STREAM>(a, r, len, sg.lt0, sg.lt1, sg.full, sg.slot, smem, seg_flag, lane, wv);
    if (st == 1)
      st = attend_segment<NHB, STREAM>(a, r, len, sg.lt0, sg.lt1, sg.full, sg.slot, smem, seg_flag, lane, wv);
    if (st != 0) generic_segment(a, r, len, sg.lt0, sg.lt1, sg.full, sg.slot, smem);
    if (threadIdx.x == 0) seg_flag[1] = 0;  // its last reads precede the segment's final barrier
  }
}
}  // namespace mf

// ===========================================================================
// log-sum-exp combine
// ===========================================================================
// Merge n normalised partial results of one (row, head): lse = log sum e^lse_p,
// out = sum_p e^(lse_p - lse) o_p. Parts with lse_p = -inf are skipped (never
// read). Threads of the block split d_c.
template <typename PT>
struct PartRef {
  const PT* o;
  float lse;
};

template <typename OutT, typename PartFn>
__device__ void combine_head(int n, PartFn part, int d_c, OutT* out, float* lse_out) {
  float mx = -INFINITY;
  for (int p = 0; p < n; ++p) mx = fmaxf(mx, part(p).lse);
  for (int d = threadIdx.x; d < d_c; d += blockDim.x) {
    float acc = 0.f, wsum = 0.f;
    for (int p = 0; p < n; ++p) {
      auto pp = part(p);
      if (pp.lse == -INFINITY) continue;
      const float e = __expf(pp.lse - mx);
      wsum += e;
      acc += e * load_f32(pp.o + d);
    }
    store_f32(out + d, wsum > 0.f ? acc / wsum : 0.f);
  }
  if (threadIdx.x == 0 && lse_out) {
    float ws = 0.f;
    for (int p = 0; p < n; ++p) {
      float l = part(p).lse;
      if (l != -INFINITY) ws += __expf(l - mx);
    }
    *lse_out = ws > 0.f ? mx + __logf(ws) : -INFINITY;
  }
}

// Split rows: workgroup (x, k) merges items 256x .. 256x+255 of the k-th row
// of the plan's split list, an item being VEC consecutive dims of one head
// (16 bytes of the output). The list entry gives the row and its parts: part
// 0 in slot s0, part i > 0 in slot 2(w0 + i) (the row started before those
// workers' ranges). Each thread issues the lse and partial loads of up to NP
// parts at once, then merges them with a running maximum, so a workgroup
// waits for memory twice (list entry, then data).
// Merge of the n parts of split row r for one item (VEC dims d.. of head h):
// part 0 in slot s0, part i > 0 in slot 2(w0 + i).
template <typename OutT, int VEC>
__device__ __forceinline__ void merge_item(const Plan& pl, int H, int d_c, int r, int s0, int w0, int n, int h,
                                           int d, OutT* out, float* lse) {
  constexpr int NP = 4;
  typedef OutT vec_t __attribute__((ext_vector_type(VEC)));
  float mx = -INFINITY, ws = 0.f;
  float acc[VEC];
#pragma unroll
  for (int x = 0; x < VEC; ++x) acc[x] = 0.f;
  for (int p0 = 0; p0 < n; p0 += NP) {
    float l[NP];
    vec_t v[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int i = p0 + j < n ? p0 + j : n - 1;
      const int slot = i == 0 ? s0 : 2 * (w0 + i);
      l[j] = p0 + j < n ? pl.part_lse[(size_t)slot * H + h] : -INFINITY;
      v[j] = *(const vec_t*)((const OutT*)pl.part_o + ((size_t)slot * H + h) * d_c + d);
    }
    float m2 = mx;
#pragma unroll
    for (int j = 0; j < NP; ++j) m2 = fmaxf(m2, l[j]);
    if (m2 == -INFINITY) continue;  // every part so far empty
    const float sc = __expf(mx - m2);
    ws *= sc;
#pragma unroll
    for (int x = 0; x < VEC; ++x) acc[x] *= sc;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const float w = __expf(l[j] - m2);
      ws += w;
#pragma unroll
      for (int x = 0; x < VEC; ++x) acc[x] += w * (float)v[j][x];
    }
    mx = m2;
  }
  const float inv = ws > 0.f ? 1.0f / ws : 0.f;
  vec_t o;
#pragma unroll
  for (int x = 0; x < VEC; ++x) {
    if constexpr (sizeof(OutT) == 2)
      o[x] = f32_to_bf16(acc[x] * inv);
    else
      o[x] = acc[x] * inv;
  }
  *(vec_t*)(out + ((size_t)r * H + h) * d_c + d) = o;
  if (lse && d == 0) lse[(size_t)r * H + h] = ws > 0.f ? mx + __logf(ws) : -INFINITY;
}

template <typename OutT, int VEC>
__global__ __launch_bounds__(256) void plan_combine_kernel(Plan pl, int H, int d_c, OutT* out, float* lse) {
  const int k = blockIdx.y;
  const int4 e = *(const int4*)(pl.split + 4 + 4 * k);
  if (k >= pl.split[0]) return;
  const int nq = d_c / VEC;
  const int item = blockIdx.x * 256 + threadIdx.x;
  if (item >= H * nq) return;
  const int h = item / nq, d = (item - h * nq) * VEC;
  merge_item<OutT, VEC>(pl, H, d_c, e.x, e.y, e.z, e.w, h, d, out, lse);
}

// Combine of a self-planned call: workgroup (x, r) reads row r's plan, which
// the first attention workgroup stored (prefix sums, length, fixed cost), and
// handles items 256x .. 256x+255 of the row: zeros and lse = -inf for an empty
// row, the merge for a row cut by worker boundaries, nothing for a row one
// worker finished.
template <typename OutT, int VEC>
__global__ __launch_bounds__(256) void self_combine_kernel(Plan pl, int H, int d_c, OutT* out, float* lse) {
  typedef OutT vec_t __attribute__((ext_vector_type(VEC)));
  const int r = blockIdx.y;
  const int nq = d_c / VEC;
  const int item = blockIdx.x * 256 + threadIdx.x;
  if (item >= H * nq) return;
  const int h = item / nq, d = (item - h * nq) * VEC;
  const int base = pl.cum[r], n = pl.cum[r + 1] - base, total = pl.cum[pl.R], seg_cost = pl.split[1];
  if (pl.len[r] == 0) {
    vec_t z;
#pragma unroll
    for (int x = 0; x < VEC; ++x) z[x] = (OutT)0.f;
    *(vec_t*)(out + ((size_t)r * H + h) * d_c + d) = z;
    if (lse && d == 0) lse[(size_t)r * H + h] = -INFINITY;
    return;
  }
  const int per = plan_per_worker(total, pl.G);
  const int s0 = base + seg_cost;  // first unit of the row's tiles
  const int w0 = s0 / per, w1 = (base + n - 1) / per;
  if (w0 == w1) return;  // finished by one worker
  merge_item<OutT, VEC>(pl, H, d_c, r, plan_slot(w0, s0, per), w0, w1 - w0 + 1, h, d, out, lse);
}

template <typename OutT>
__global__ __launch_bounds__(256) void lse_combine_kernel(const float* o_parts, const float* lse_parts, int n,
                                                          int64_t rows, int H, int d_c, OutT* out, float* lse) {
  const int64_t r = blockIdx.x;
  const int h = blockIdx.y;
  auto part = [&](int p) {
    const size_t idx = ((size_t)p * rows + r) * H + h;
    return PartRef<float>{o_parts + idx * d_c, lse_parts[idx]};
  };
  combine_head<OutT>(n, part, d_c, out + ((size_t)r * H + h) * d_c, lse ? lse + (size_t)r * H + h : nullptr);
}


// ===========================================================================
// host launchers
// ===========================================================================
static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

static bool use_mfma(const AttnCall& c) {
  if (c.dtype != MLA_BF16 || c.d_c != mf::DC || c.d_r != mf::DR) return false;
  if (c.H % 32 != 0 || c.H > 32 * mf::NW) return false;
  if (c.map.mode == 1 && c.map.page_size % mf::TILE != 0) return false;
  return aligned16(c.q) && aligned16(c.cache) && aligned16(c.out);
}

int attn_tile_size(const AttnCall& c) { return use_mfma(c) ? mf::TILE : gn::TT; }

#define MLA_LAUNCH_CHECK()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP; \
  } while (0)

// Launch of the attention kernel. With timing events the launch carries them
// (no marker commands on the stream): they take the start and end times of
// the kernel's dispatch.
template <typename K, typename A>
static void launch_timed(const AttnCall& c, K kernel, dim3 grid, dim3 block, const A& a) {
  if (c.timing_events)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, c.stream, (hipEvent_t)c.timing_events[0],
                          (hipEvent_t)c.timing_events[1], 0, a);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, c.stream, a);
}

template <typename T>
static void launch_generic(const AttnCall& c, const Plan& pl) {
  gn::Args<T> a;
  a.q = (const T*)c.q;
  a.cache = (const T*)c.cache;
  a.map = c.map;
  a.pl = pl;
  a.H = c.H;
  a.d_c = c.d_c;
  a.d_r = c.d_r;
  a.scale_log2 = c.kq_scale * kLog2e;
  a.out = (T*)c.out;
  a.lse = c.lse;
  dim3 grid(c.G, (c.H + gn::HGK - 1) / gn::HGK);
  launch_timed(c, gn::attn_generic_kernel<T>, grid, dim3(gn::NT), a);
}

template <typename T>
static int launch_attention_t(const AttnCall& c) {
  const bool mfma = use_mfma(c);
  const int tile = mfma ? mf::TILE : gn::TT;
  Plan pl = plan_layout(c.ws, c.R, c.G, c.H, c.d_c, tile, c.part_esize);
  constexpr int VEC = 16 / (int)sizeof(T);
  const bool vec_out = c.d_c % VEC == 0 && aligned16(c.out);
  // decode batches of up to SELF_MAX_R rows on the MFMA kernel plan inside
  // the attention and combine kernels (no planning kernel)
  const bool self = mfma && c.map.mode != 2 && c.R <= SELF_MAX_R && vec_out;
  if (!self) {
    hipLaunchKernelGGL(plan_kernel<T>, dim3(1), dim3(1024), 0, c.stream, c.map, pl, c.H, c.d_c, (T*)c.out, c.lse);
    MLA_LAUNCH_CHECK();
  }
  if (mfma) {
    mf::Args a;
    a.q = (const bf16*)c.q;
    a.cache = (const bf16*)c.cache;
    a.map = c.map;
    a.pl = pl;
    a.H = c.H;
    a.scale_log2 = c.kq_scale * kLog2e;
    a.out = (bf16*)c.out;
    a.lse = c.lse;
    const dim3 grid(c.G), block(mf::NW * 64);
    if (self) {  // decode: every cache row read once
      switch (c.H / 32) {
        case 1: launch_timed(c, mf::attn_mfma_kernel<1, true, true>, grid, block, a); break;
        case 2: launch_timed(c, mf::attn_mfma_kernel<2, true, true>, grid, block, a); break;
        case 3: launch_timed(c, mf::attn_mfma_kernel<3, true, true>, grid, block, a); break;
        default: launch_timed(c, mf::attn_mfma_kernel<4, true, true>, grid, block, a); break;
      }
    } else if (c.map.mode != 2) {
      switch (c.H / 32) {
        case 1: launch_timed(c, mf::attn_mfma_kernel<1, true, false>, grid, block, a); break;
        case 2: launch_timed(c, mf::attn_mfma_kernel<2, true, false>, grid, block, a); break;
        case 3: launch_timed(c, mf::attn_mfma_kernel<3, true, false>, grid, block, a); break;
        default: launch_timed(c, mf::attn_mfma_kernel<4, true, false>, grid, block, a); break;
      }
    } else {  // causal prefill: rows re-read by every later query
      switch (c.H / 32) {
        case 1: launch_timed(c, mf::attn_mfma_kernel<1, false, false>, grid, block, a); break;
        case 2: launch_timed(c, mf::attn_mfma_kernel<2, false, false>, grid, block, a); break;
        case 3: launch_timed(c, mf::attn_mfma_kernel<3, false, false>, grid, block, a); break;
        default: launch_timed(c, mf::attn_mfma_kernel<4, false, false>, grid, block, a); break;
      }
    }
  } else {
    launch_generic<T>(c, pl);
  }
  MLA_LAUNCH_CHECK();
  // decode with the up-projection: merge and W_UV in one kernel (bf16, d_c = 512, d_v = 128)
  if (c.w_uv && mfma && c.map.mode != 2 && upv_merge_fits(c.d_c, c.d_v, c.w_uv, c.v))
    return launch_upv_merge(pl, c.R, c.H, c.out, c.w_uv, c.v, c.lse, c.stream);
  if (self) {
    dim3 cgrid((unsigned)((c.H * (c.d_c / VEC) + 255) / 256), (unsigned)c.R);
    hipLaunchKernelGGL((self_combine_kernel<T, VEC>), cgrid, dim3(256), 0, c.stream, pl, c.H, c.d_c, (T*)c.out,
                       c.lse);
  } else {
    // at most min(R, G - 1) rows are cut by the G - 1 worker boundaries
    const unsigned max_split = (unsigned)(c.R < c.G ? c.R : c.G);
    if (vec_out) {
      dim3 cgrid((unsigned)((c.H * (c.d_c / VEC) + 255) / 256), max_split);
      hipLaunchKernelGGL((plan_combine_kernel<T, VEC>), cgrid, dim3(256), 0, c.stream, pl, c.H, c.d_c, (T*)c.out,
                         c.lse);
    } else {
      dim3 cgrid((unsigned)((c.H * c.d_c + 255) / 256), max_split);
      hipLaunchKernelGGL((plan_combine_kernel<T, 1>), cgrid, dim3(256), 0, c.stream, pl, c.H, c.d_c, (T*)c.out,
                         c.lse);
    }
  }
  MLA_LAUNCH_CHECK();
  if (c.w_uv) return launch_up_v(c.out, c.w_uv, c.v, c.R, c.H, c.d_c, c.d_v, c.dtype, c.stream);
  return MLA_OK;
}

int launch_attention(const AttnCall& c) {
  return c.dtype == MLA_BF16 ? launch_attention_t<bf16>(c) : launch_attention_t<float>(c);
}

int launch_lse_combine(const float* o_parts, const float* lse_parts, int n_parts, int64_t rows, int H, int d_c,
                       int dtype, void* out, float* lse, hipStream_t stream) {
  dim3 grid((unsigned)rows, H);
  if (dtype == MLA_BF16)
    hipLaunchKernelGGL(lse_combine_kernel<bf16>, grid, dim3(256), 0, stream, o_parts, lse_parts, n_parts, rows, H,
                       d_c, (bf16*)out, lse);
  else
    hipLaunchKernelGGL(lse_combine_kernel<float>, grid, dim3(256), 0, stream, o_parts, lse_parts, n_parts, rows, H,
                       d_c, (float*)out, lse);
  MLA_LAUNCH_CHECK();
  return MLA_OK;
}

}  // namespace mla
