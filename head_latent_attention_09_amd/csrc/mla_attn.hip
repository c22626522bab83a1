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

#include <math.h>

namespace mla {

// ===========================================================================
// planning: visible length and tile prefix sum of every row, the list of
// rows cut by worker boundaries, and the (final) output of empty rows
// ===========================================================================
__device__ __forceinline__ int row_len(const RowMap& m, int r) {
  if (m.mode == 2) {  // prefill, bottom-right causal alignment: t <= i + s_kv - s_q
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
  __shared__ int sums[1024];
  __shared__ int nsplit;
  const int tid = threadIdx.x;
  const int R = pl.R, tile = pl.tile;
  const int chunk = (R + 1023) / 1024;
  const int r0 = min(tid * chunk, R), r1 = min(r0 + chunk, R);
  if (tid == 0) nsplit = 0;
  int s = 0;
  for (int r = r0; r < r1; ++r) {
    int n = row_len(m, r);
    pl.len[r] = n;
    pl.flags[r] = 0;
    s += (n + tile - 1) / tile;
  }
  sums[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan
    int v = tid >= off ? sums[tid - off] : 0;
    __syncthreads();
    sums[tid] += v;
    __syncthreads();
  }
  const int total = sums[1023];
  const int per = plan_per_worker(total, pl.G);
  int base = tid == 0 ? 0 : sums[tid - 1];
  for (int r = r0; r < r1; ++r) {
    const int n = (pl.len[r] + tile - 1) / tile;
    pl.cum[r] = base;
    if (n > 0 && base / per != (base + n - 1) / per) pl.split[1 + atomicAdd(&nsplit, 1)] = r;
    base += n;
  }
  if (tid == 1023) pl.cum[R] = total;
  __syncthreads();
  if (tid == 0) pl.split[0] = nsplit;
  // rows with nothing visible: zeros and lse = -inf (no later kernel touches
  // them). Each thread checks its own rows; the rare empty rows are written
  // by the whole workgroup.
  __shared__ int nzero;
  __shared__ int zrows[256];
  if (tid == 0) nzero = 0;
  __syncthreads();
  for (int r = r0; r < r1; ++r)
    if (pl.len[r] == 0) {
      const int i = atomicAdd(&nzero, 1);
      if (i < 256) zrows[i] = r;
    }
  __syncthreads();
  const int nz = nzero;
  for (int j = 0; j < (nz < 256 ? nz : 256); ++j) {
    const int r = zrows[j];
    for (int i = tid; i < H * d_c; i += 1024) store_f32(out + (size_t)r * H * d_c + i, 0.f);
    if (lse)
      for (int h = tid; h < H; h += 1024) lse[(size_t)r * H + h] = -INFINITY;
  }
  if (nz > 256) {  // more empty rows than the list holds: each thread writes its own
    for (int r = r0; r < r1; ++r)
      if (pl.len[r] == 0) {
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

// ===========================================================================
// generic attention (fp32 or bf16 storage, any d_c <= 1024, d_c + d_r <= 1152)
// fp32 arithmetic on the vector ALUs; 8 heads per workgroup, 16-position tiles.
// ===========================================================================
namespace gn {
constexpr int TT = 16, HG = 8, WMAX = 1152, DCMAX = 1024, NT = 256;

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

template <typename T>
__device__ void attend_segment(const Args<T>& a, int r, int lt0, int lt1, bool full, int slot, int h0,
                               float* tile, float* qs, float* ps, float* alpha_s, float* stat_s,
                               float& m_run, float& l_run) {
  const int tid = threadIdx.x;
  const int W = a.d_c + a.d_r, WP = W + 1, H = a.H, d_c = a.d_c;
  const int nh = min(HG, H - h0);
  const int len = a.pl.len[r];
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
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    if (hh >= nh) break;
    const int h = h0 + hh;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = tid + k * NT;
      if (d < d_c) {
        float v = acc[hh][k] * stat_s[hh];
        if (full) store_f32(a.out + ((size_t)r * H + h) * d_c + d, v);
        else a.pl.part_o[((size_t)slot * H + h) * d_c + d] = v;
      }
    }
    if (tid == 0) {
      if (full) { if (a.lse) a.lse[(size_t)r * H + h] = stat_s[HG + hh]; }
      else a.pl.part_lse[(size_t)slot * H + h] = stat_s[HG + hh];
    }
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void attn_generic_kernel(Args<T> a) {
  __shared__ float tile[TT * (WMAX + 1)];
  __shared__ float qs[HG * WMAX];
  __shared__ float ps[HG * TT];
  __shared__ float alpha_s[HG];
  __shared__ float stat_s[2 * HG];
  float m_run = -INFINITY, l_run = 0.f;
  const int G = a.pl.G;
  const int w = xcd_worker(blockIdx.x, G);
  const int h0 = blockIdx.y * HG;
  const int total = a.pl.cum[a.pl.R];
  const int per = plan_per_worker(total, G);
  const int t_begin = w * per;
  if (t_begin >= total) return;
  const int t_end = min(t_begin + per, total);
  for (int r = plan_row_of(a.pl.cum, a.pl.R, t_begin); r < a.pl.R; ++r) {
    const int c0 = a.pl.cum[r], c1 = a.pl.cum[r + 1];
    if (c0 >= t_end) break;
    if (c1 <= t_begin || c1 == c0) continue;
    const int lt0 = max(t_begin, c0) - c0, lt1 = min(t_end, c1) - c0;
    const bool full = c0 >= t_begin && c1 <= t_end;
    attend_segment<T>(a, r, lt0, lt1, full, plan_slot(w, c0, per), h0, tile, qs, ps, alpha_s, stat_s,
                      m_run, l_run);
  }
}
}  // namespace gn

// ===========================================================================
// bf16 MFMA attention: d_c = 512, d_r = 64, 4 waves x 32 heads
// ===========================================================================
namespace mf {
constexpr int DC = 512, DR = 64, WD = 576;
constexpr int TILE = 32;                   // positions per tile
constexpr int C_BYTES = TILE * DC * 2;     // latent part of a tile: 32 rows x 1024 B
constexpr int TILE_BYTES = TILE * WD * 2;  // + rope part: 32 rows x 128 B = 36 KiB
constexpr int NSTAGE = 3;                  // tiles in the LDS ring
constexpr int KQR = 24;                    // query k-steps held in registers (dims 0..383)
constexpr int QLW = WD - 16 * KQR;         // query dims kept in LDS (384..575)
constexpr int QL_ROW = QLW * 2;            // bytes per head row of that block (24 chunks)
constexpr int QL_BYTES = 128 * QL_ROW;     // 48 KiB for the 128 query rows
constexpr int RING = 4;                    // LDS operand reads in flight per wave
constexpr int NW = 4;                      // waves per workgroup (32 heads each)
constexpr int LPW = 36 / NW;               // tile loads per wave
constexpr float SLACK = 64.0f;             // log2 units a score may exceed the reference max

// LDS tile layout. Latent region: row r at r*1024, its 16-byte chunk c at
// position c ^ sC(r) (XOR inside aligned groups of 16 chunks). Rope region:
// row r at C_BYTES + r*128, chunk c at c ^ sR(r). The XOR patterns make the
// two read patterns conflict-free for a 128- or 256-byte-wide LDS:
//  (a) QK operand: 32 rows, one chunk each (sC, sR distinct over 8/16 rows);
//  (b) PV operand, transposing loads: 4 consecutive rows x 4 chunks
//      (sC's bits 1-3 spread the 4 rows over distinct chunk pairs/quads).
__device__ __forceinline__ int sC(int r) {
  return (((r & 1) ? 6 : 0) ^ ((r & 2) ? 10 : 0)) ^ ((r >> 2) & 3);
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

// S^T accumulation with the accumulator pinned to VGPRs: the 256 AGPRs hold
// the output accumulator, and the compiler otherwise puts S there too and
// evicts the query fragments to scratch. Consecutive MFMAs accumulating into
// the same registers need no wait states between them.
__device__ __forceinline__ void mfma_vacc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vacc_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
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
  static_assert(N >= 0, "");
  constexpr int n = N > 63 ? 63 : N;
  // vmcnt in bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15) left unconstrained
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Issue the direct global->LDS loads of one tile (positions t0 .. t0+31 of
// batch entry b). 36 loads of 64 lanes x 16 B: load ld < 32 fills latent row
// ld (1 KiB, one row); load 32 + j fills the rope chunks of rows 8j .. 8j+7.
// Wave wv issues loads wv, wv + NW, ... Rows at or past `len` re-read row
// len-1 (finite data; their scores are masked to -inf).
__device__ __forceinline__ void issue_tile(const Args& a, char* buf, int b, int t0, int len, int lane, int wv) {
  const RowMap& m = a.map;
  const char* tile;
  if (m.mode == 1) {
    const int pg = page_of(m, b, t0);
    tile = (const char*)(a.cache + ((size_t)pg * m.page_size + (t0 % m.page_size)) * WD);
  } else {
    tile = (const char*)(a.cache + dense_row(m, b, t0, WD));
  }
  const int last = len - 1 - t0;  // last valid row of this tile (wave-uniform)
  // Latent rows ld = wv + 4k (k < 8): sC(ld) = f(wv) ^ (k & 3), so the lane's
  // chunk is (lane ^ f(wv)) ^ (k & 3); the row pointer is wave-uniform.
  int lx = lane ^ sC(wv);
  opaque(lx);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int ld = wv + NW * k;
    const int row = ld < last ? ld : last;
    dma16(tile + (size_t)row * (WD * 2), (uint32_t)((lx ^ (k & 3)) << 4), lds_addr(buf + ld * 1024));
  }
  // rope chunks of rows 8wv .. 8wv+7: lane -> row 8wv + lane/8, chunk (lane%8) ^ sR(row)
  {
    const int rl = NW * 2 * wv + (lane >> 3);
    const int row = rl < last ? rl : last;
    dma16(tile, (uint32_t)(row * (WD * 2) + DC * 2 + (((lane & 7) ^ sR(rl)) << 4)),
          lds_addr(buf + C_BYTES + wv * 1024));
  }
}

// Whole-row recompute with the generic kernel (running max with rescaling),
// writing the final result; the tile ring is reused as its scratch.
__device__ void recompute_row(const Args& a, int r, char* smem) {
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
  float m_run = -INFINITY, l_run = 0.f;
  const int len = a.pl.len[r];
  for (int h0 = 0; h0 < a.H; h0 += gn::HG)
    gn::attend_segment<bf16>(ga, r, 0, (len + gn::TT - 1) / gn::TT, true, 0, h0, tile, qs, ps, alpha_s, stat_s,
                             m_run, l_run);
  __syncthreads();
}

__device__ __forceinline__ void attend_segment(const Args& a, int r, int lt0, int lt1, bool full, int slot,
                                               char* smem, int* seg_flag, int lane, int wv) {
  const int H = a.H;
  const int len = a.pl.len[r];
  const int b = row_batch(a.map, r);
  const int g = lane >> 5;              // half of the wave
  const int h = wv * 32 + (lane & 31);  // this lane's head (MFMA column)
  const bool active = wv * 32 < H;      // waves past the last head only help load tiles
  const int ntiles = lt1 - lt0;

  // every wave must be done with the previous segment's LDS tiles (and flag)
  block_barrier();
  if (threadIdx.x == 0) *seg_flag = 0;

  // prologue: first NSTAGE-1 tiles, then this wave's 32 query rows as the
  // B operand of S^T = K Q^T (lane: head h, dims 16ks + 8g .. +7)
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < ntiles) issue_tile(a, smem + s * TILE_BYTES, b, (lt0 + s) * TILE, len, lane, wv);
  // this wave's 32 query rows: dims 0..383 (24 k-steps) in registers as the
  // B operand of S^T = K Q^T (lane: head h, dims 16ks + 8g .. +7); dims
  // 384..575 go to LDS, head row hr at ql + hr*QL_ROW, chunk c (of 24) at
  // c ^ sR(hr), one 12 KiB block per wave.
  const int hq = h < H ? h : H - 1;  // waves past the last head compute on a copy and write nothing
  char* ql = smem + NSTAGE * TILE_BYTES + wv * (32 * QL_ROW);
#pragma unroll
  for (int k = 0; k < 32 * QL_ROW / 1024; ++k) {
    const int p = k * 64 + lane;     // 16-byte chunk position in this wave's block
    const int hr = p / (QL_ROW / 16);
    const int pc = p - hr * (QL_ROW / 16);
    const int hsrc = wv * 32 + hr < H ? wv * 32 + hr : H - 1;
    const char* qbase = (const char*)(a.q + (size_t)r * H * WD + 16 * KQR);
    dma16(qbase, (uint32_t)(hsrc * (WD * 2) + ((pc ^ sR(hr)) << 4)), lds_addr(ql + k * 1024));
  }
  bf16x8 qf[KQR];
  {
    const bf16* qrow = a.q + ((size_t)r * H + hq) * WD + g * 8;
#pragma unroll
    for (int ks = 0; ks < KQR; ++ks) qf[ks] = *(const bf16x8*)(qrow + ks * 16);
  }
  wait_vmcnt<0>();  // query rows (and the prologue) complete before the loop

  // Softmax reference. Each head's reference max m_ref is the largest score
  // of the segment's first tile and the weights are 2^(x - m_ref). Keeping
  // the reference fixed keeps the output accumulator free of data-dependent
  // rescaling (a conditional rescale moves it out of the accumulation
  // registers). If a later score exceeds m_ref by more than SLACK the
  // exponent is clamped and the row is flagged; a fix-up pass recomputes
  // flagged rows with the generic kernel. Scores would have to grow by more
  // than 2^64 within one segment for that to happen.
  float m_ref = -INFINITY;
  float l_run = 0.f;  // running denominator over this lane's half of the positions
  f32x16 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f32x16{};
  bool overflow = false;
  for (int it = 0; it < ntiles; ++it) {
    if (it + NSTAGE - 2 < ntiles) wait_vmcnt<(NSTAGE - 2) * LPW>();
    else wait_vmcnt<0>();
    block_barrier();  // tile it visible; tile it-1's buffer free for reuse
    if (it + NSTAGE - 1 < ntiles)
      issue_tile(a, smem + ((it + NSTAGE - 1) % NSTAGE) * TILE_BYTES, b, (lt0 + it + NSTAGE - 1) * TILE, len,
                 lane, wv);
    const char* buf = smem + (it % NSTAGE) * TILE_BYTES;
    const int t0 = (lt0 + it) * TILE;

    // Per-lane LDS offsets, rebuilt every tile from an opaque copy of the lane
    // id: values live across the loop get spilled, and a spill reload in front
    // of the loop makes the compiler wait for all in-flight tile loads.
    // Forms are base + 32 * (j ^ x) (QK) and base + 64 * (u ^ x) (PV); the
    // remaining terms are immediates.
    int ln = lane;
    opaque(ln);
    const int mrow = ln & 31;  // QK: this lane's A-operand row (position) and head row
    const int sCm = sC(mrow), sRm = sR(mrow);
    const int gg = ln >> 5;
    const int baseC = mrow * 1024 + ((gg ^ (sCm & 1)) << 4);
    const int baseR = C_BYTES + mrow * 128 + ((gg ^ (sRm & 1)) << 4);
    const int baseQ = mrow * QL_ROW + ((gg ^ (sRm & 1)) << 4);
    const int xC = sCm >> 1, xR = sRm >> 1;
    const int q16 = ln & 15;
    const int rowA = 4 * gg + (q16 >> 2);  // PV: rows of the first transposing load (k-step 0)
    const int rowB = rowA + 8;
    const int cb = 2 * ((ln >> 4) & 1) + ((q16 & 3) >> 1);
    const int sA = sC(rowA), sB = sC(rowB);
    const int baseA = rowA * 1024 + ((cb ^ (sA & 3)) << 4) + (q16 & 1) * 8;
    const int baseB = rowB * 1024 + ((cb ^ (sB & 3)) << 4) + (q16 & 1) * 8;
    const int xA = sA >> 2, xB = sB >> 2;

    // ---- S^T[position][head] = K_tile . Q^T, 36 k-steps of 16 dims. LDS
    // operands are read RING k-steps ahead of their MFMA; the compiler
    // barriers keep reads in this order (neither hoisted nor sunk).
    f32x16 sacc;
    {
      // A operand (K tile rows) of k-step ks
      auto kread = [&](int ks) -> bf16x8 {
        const char* p = ks < 32 ? buf + baseC + (((ks & 7) ^ xC) << 5) + 256 * (ks >> 3)
                                : buf + baseR + (((ks - 32) ^ xR) << 5);
        return *(const MLA_LDS bf16x8*)p;
      };
      // B operand of k-steps ks >= KQR (query dims kept in LDS)
      auto qread = [&](int ks) -> bf16x8 {
        const int kq = ks - KQR;
        return *(const MLA_LDS bf16x8*)(ql + baseQ + 128 * (kq >> 2) + (((kq & 3) ^ xR) << 5));
      };
      bf16x8 kr[RING], qr[RING];
#pragma unroll
      for (int i = 0; i < RING; ++i) {
        kr[i] = kread(i);
        if (i >= KQR) qr[i] = qread(i);
      }
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        const bf16x8 a_op = kr[ks % RING];
        const bf16x8 b_op = ks < KQR ? qf[ks] : qr[ks % RING];
        if (ks + RING < 36) {
          kr[ks % RING] = kread(ks + RING);
          if (ks + RING >= KQR) qr[ks % RING] = qread(ks + RING);
        }
        asm volatile("" ::: "memory");
        if (ks == 0) mfma_vacc_first(sacc, a_op, b_op);
        else mfma_vacc(sacc, a_op, b_op);
      }
    }
    // the last QK MFMA's result is read by VALU next: 8-pass XDL -> VALU read
    // needs 11 wait states (the asm MFMA is invisible to the hazard checker)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");

    // ---- softmax weights (lane = head; 16 positions here, 16 in lane^32)
    const int nvalid = len - t0;  // positions i < nvalid are visible
    float tmax = -INFINITY;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int i = 8 * (rr >> 2) + 4 * g + (rr & 3);
      tmax = fmaxf(tmax, i < nvalid ? sacc[rr] * a.scale_log2 : -INFINITY);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    m_ref = m_ref == -INFINITY ? tmax : m_ref;  // first tile of the segment
    overflow |= tmax > m_ref + SLACK;
    bf16x8 pb[2];
    float psum = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int i = 8 * (rr >> 2) + 4 * g + (rr & 3);
      const float e = fminf(sacc[rr] * a.scale_log2 - m_ref, SLACK);
      const bf16 p = f32_to_bf16(i < nvalid ? __builtin_amdgcn_exp2f(e) : 0.f);
      pb[rr >> 3][rr & 7] = p;
      psum += bf16_to_f32(p);  // the denominator sums exactly the weights the MFMA uses
    }
    l_run += psum;

    // ---- O^T[dim][head] += V^T . P^T ; V^T fragments via transposing LDS loads.
    // Slot s of k-step kk holds position 16kk + 8(s/4) + 4g + s%4 (the order of
    // the S accumulators): lane group (l/16) reads positions 16kk + 4g + {0..3}
    // and the same +8, 16 dims each.
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    // 32 PV steps j = 16 kk + db; transposing reads run RING steps ahead
    auto vread = [&](int j, bool second) -> s16x4 {
      const int kk = j >> 4, db = j & 15;
      const char* p = buf + (second ? baseB + (((db & 3) ^ xB) << 6) : baseA + (((db & 3) ^ xA) << 6)) +
                      256 * (db >> 2) + kk * 16 * 1024;
      return __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)p);
    };
    s16x4 va[RING], vb[RING];
#pragma unroll
    for (int i = 0; i < RING; ++i) {
      va[i] = vread(i, false);
      vb[i] = vread(i, true);
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const s16x8 v8 = __builtin_shufflevector(va[j % RING], vb[j % RING], 0, 1, 2, 3, 4, 5, 6, 7);
      if (j + RING < 32) {
        va[j % RING] = vread(j + RING, false);
        vb[j % RING] = vread(j + RING, true);
      }
      asm volatile("" ::: "memory");
      o[j & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8), pb[j >> 4], o[j & 15], 0, 0, 0);
    }
  }
  // Overflow of the fixed reference (see above): the first workgroup to flag
  // row r recomputes the whole row with the generic running-max kernel into
  // the final output; the combine skips flagged rows.
  if (active && __any(overflow) && lane == 0) atomicOr(seg_flag, 1);
  block_barrier();
  if (*seg_flag) {
    __shared__ int claim;
    if (threadIdx.x == 0) claim = atomicOr(a.pl.flags + r, 1) == 0;
    __syncthreads();
    if (claim) recompute_row(a, r, smem);
    return;
  }
  if (!active) return;

  // ---- finish: full denominator, normalise, write final or partial result
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  const float lse_v = (m_ref + __log2f(l_tot)) * kLn2;
  if (full) {
    bf16* orow = a.out + ((size_t)r * H + h) * DC;
#pragma unroll
    for (int db = 0; db < 16; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 v;
        v[0] = f32_to_bf16(o[db][4 * rq + 0] * inv);
        v[1] = f32_to_bf16(o[db][4 * rq + 1] * inv);
        v[2] = f32_to_bf16(o[db][4 * rq + 2] * inv);
        v[3] = f32_to_bf16(o[db][4 * rq + 3] * inv);
        *(bf16x4*)(orow + db * 32 + 8 * rq + 4 * g) = v;
      }
    if (a.lse && g == 0) a.lse[(size_t)r * H + h] = lse_v;
  } else {
    float* prow = a.pl.part_o + ((size_t)slot * H + h) * DC;
#pragma unroll
    for (int db = 0; db < 16; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4 v;
        v[0] = o[db][4 * rq + 0] * inv;
        v[1] = o[db][4 * rq + 1] * inv;
        v[2] = o[db][4 * rq + 2] * inv;
        v[3] = o[db][4 * rq + 3] * inv;
        *(f32x4*)(prow + db * 32 + 8 * rq + 4 * g) = v;
      }
    if (g == 0) a.pl.part_lse[(size_t)slot * H + h] = lse_v;
  }
}

__global__ __launch_bounds__(NW * 64, 1) void attn_mfma_kernel(Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * TILE_BYTES + QL_BYTES];
  __shared__ int seg_flag;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int G = a.pl.G;
  const int w = xcd_worker(blockIdx.x, G);
  const int total = a.pl.cum[a.pl.R];
  const int per = plan_per_worker(total, G);
  const int t_begin = w * per;
  if (t_begin >= total) return;
  const int t_end = min(t_begin + per, total);
  for (int r = plan_row_of(a.pl.cum, a.pl.R, t_begin); r < a.pl.R; ++r) {
    const int c0 = a.pl.cum[r], c1 = a.pl.cum[r + 1];
    if (c0 >= t_end) break;
    if (c1 <= t_begin || c1 == c0) continue;
    const int lt0 = max(t_begin, c0) - c0, lt1 = min(t_end, c1) - c0;
    const bool full = c0 >= t_begin && c1 <= t_end;
    attend_segment(a, r, lt0, lt1, full, plan_slot(w, c0, per), smem, &seg_flag, lane, wv);
  }
}
}  // namespace mf

// ===========================================================================
// log-sum-exp combine
// ===========================================================================
// Merge n normalised partial results of one (row, head): lse = log sum e^lse_p,
// out = sum_p e^(lse_p - lse) o_p. Parts with lse_p = -inf are skipped (never
// read). Threads of the block split d_c.
struct PartRef {
  const float* o;
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
      acc += e * pp.o[d];
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

// Split rows: workgroup (k, hb) merges heads 8hb .. 8hb+7 of the k-th row of
// the plan's split list from its partial slots (one per worker it spans).
// Rows the attention kernel recomputed (flagged) are already final.
constexpr int CHB = 8;  // heads per combine workgroup
template <typename OutT>
__global__ __launch_bounds__(256) void plan_combine_kernel(Plan pl, int H, int d_c, OutT* out, float* lse) {
  __shared__ float w_s[CHB][64];
  __shared__ float inv_s[CHB];
  const int k = blockIdx.x;
  if (k >= pl.split[0]) return;
  const int r = pl.split[1 + k];
  if (pl.flags[r]) return;
  const int total = pl.cum[pl.R];
  const int per = plan_per_worker(total, pl.G);
  const int c0 = pl.cum[r], c1 = pl.cum[r + 1];
  const int w0 = c0 / per;
  const int n = (c1 - 1) / per - w0 + 1;
  const int h0 = blockIdx.y * CHB;
  const int nh = min(CHB, H - h0);
  if (n > 64) {  // very long rows: one head at a time
    for (int hh = 0; hh < nh; ++hh) {
      const int h = h0 + hh;
      auto part = [&](int i) {
        const int slot = plan_slot(w0 + i, c0, per);
        return PartRef{pl.part_o + ((size_t)slot * H + h) * d_c, pl.part_lse[(size_t)slot * H + h]};
      };
      combine_head<OutT>(n, part, d_c, out + ((size_t)r * H + h) * d_c, lse ? lse + (size_t)r * H + h : nullptr);
      __syncthreads();
    }
    return;
  }
  // weights e^(lse_i - lse) per (part, head), normalised
  if (threadIdx.x < nh) {
    const int h = h0 + threadIdx.x;
    float mx = -INFINITY;
    for (int i = 0; i < n; ++i) mx = fmaxf(mx, pl.part_lse[(size_t)plan_slot(w0 + i, c0, per) * H + h]);
    float ws = 0.f;
    for (int i = 0; i < n; ++i) {
      const float e = __expf(pl.part_lse[(size_t)plan_slot(w0 + i, c0, per) * H + h] - mx);
      w_s[threadIdx.x][i] = e;
      ws += e;
    }
    inv_s[threadIdx.x] = 1.0f / ws;
    if (lse) lse[(size_t)r * H + h] = mx + __logf(ws);
  }
  __syncthreads();
  if ((d_c & 3) == 0) {
    const int q4 = d_c >> 2;
    for (int idx = threadIdx.x; idx < nh * q4; idx += blockDim.x) {
      const int hh = idx / q4, d = (idx - hh * q4) * 4;
      const int h = h0 + hh;
      f32x4 acc = f32x4{};
      for (int i = 0; i < n; ++i) {
        const int slot = plan_slot(w0 + i, c0, per);
        const f32x4 v = *(const f32x4*)(pl.part_o + ((size_t)slot * H + h) * d_c + d);
        acc += w_s[hh][i] * v;
      }
      OutT* o = out + ((size_t)r * H + h) * d_c + d;
      const float sc = inv_s[hh];
      store_f32(o + 0, acc[0] * sc);
      store_f32(o + 1, acc[1] * sc);
      store_f32(o + 2, acc[2] * sc);
      store_f32(o + 3, acc[3] * sc);
    }
  } else {
    for (int idx = threadIdx.x; idx < nh * d_c; idx += blockDim.x) {
      const int hh = idx / d_c, d = idx - hh * d_c;
      const int h = h0 + hh;
      float acc = 0.f;
      for (int i = 0; i < n; ++i)
        acc += w_s[hh][i] * pl.part_o[((size_t)plan_slot(w0 + i, c0, per) * H + h) * d_c + d];
      store_f32(out + ((size_t)r * H + h) * d_c + d, acc * inv_s[hh]);
    }
  }
}

template <typename OutT>
__global__ __launch_bounds__(256) void lse_combine_kernel(const float* o_parts, const float* lse_parts, int n,
                                                          int64_t rows, int H, int d_c, OutT* out, float* lse) {
  const int64_t r = blockIdx.x;
  const int h = blockIdx.y;
  auto part = [&](int p) {
    const size_t idx = ((size_t)p * rows + r) * H + h;
    return PartRef{o_parts + idx * d_c, lse_parts[idx]};
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
  dim3 grid(c.G, (c.H + gn::HG - 1) / gn::HG);
  hipLaunchKernelGGL(gn::attn_generic_kernel<T>, grid, dim3(gn::NT), 0, c.stream, a);
}

template <typename T>
static int launch_attention_t(const AttnCall& c) {
  const bool mfma = use_mfma(c);
  const int tile = mfma ? mf::TILE : gn::TT;
  Plan pl = plan_layout(c.ws, c.R, c.G, c.H, c.d_c, tile);
  hipLaunchKernelGGL(plan_kernel<T>, dim3(1), dim3(1024), 0, c.stream, c.map, pl, c.H, c.d_c, (T*)c.out, c.lse);
  MLA_LAUNCH_CHECK();
  if (c.timing_events && hipEventRecord((hipEvent_t)c.timing_events[0], c.stream) != hipSuccess) return MLA_ERR_HIP;
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
    hipLaunchKernelGGL(mf::attn_mfma_kernel, dim3(c.G), dim3(mf::NW * 64), 0, c.stream, a);
  } else {
    launch_generic<T>(c, pl);
  }
  MLA_LAUNCH_CHECK();
  if (c.timing_events && hipEventRecord((hipEvent_t)c.timing_events[1], c.stream) != hipSuccess) return MLA_ERR_HIP;
  dim3 cgrid(c.G, (c.H + CHB - 1) / CHB);
  hipLaunchKernelGGL(plan_combine_kernel<T>, cgrid, dim3(256), 0, c.stream, pl, c.H, c.d_c, (T*)c.out, c.lse);
  MLA_LAUNCH_CHECK();
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
