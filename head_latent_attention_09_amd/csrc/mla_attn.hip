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
// planning: visible length and tile prefix sum of every row
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

__global__ __launch_bounds__(1024) void plan_kernel(RowMap m, Plan pl) {
  __shared__ int sums[1024];
  const int tid = threadIdx.x;
  const int R = pl.R, tile = pl.tile;
  const int chunk = (R + 1023) / 1024;
  const int r0 = min(tid * chunk, R), r1 = min(r0 + chunk, R);
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
  int base = tid == 0 ? 0 : sums[tid - 1];
  for (int r = r0; r < r1; ++r) {
    pl.cum[r] = base;
    base += (pl.len[r] + tile - 1) / tile;
  }
  if (tid == 1023) pl.cum[R] = sums[1023];
}

__device__ __forceinline__ int row_batch(const RowMap& m, int r) { return m.mode == 2 ? r / m.s_q : r; }

// element offset of cache position t of batch entry b (dense and prefill layouts)
__device__ __forceinline__ size_t dense_row(const RowMap& m, int b, int t, int width) {
  size_t stride = m.mode == 2 ? (size_t)m.s_kv : (size_t)m.cache_stride;
  return ((size_t)b * stride + t) * width;
}

__device__ __forceinline__ int page_of(const RowMap& m, int b, int t) {
  int p = m.block_table[(size_t)b * m.max_pages + t / m.page_size];
  return p < 0 ? 0 : (p >= m.num_pages ? m.num_pages - 1 : p);
}

// ===========================================================================
// bf16 MFMA attention: d_c = 512, d_r = 64, NW waves x 32 heads
// ===========================================================================
namespace mf {
constexpr int DC = 512, DR = 64, WD = 576;
constexpr int TILE = 32;                   // positions per tile
constexpr int C_BYTES = TILE * DC * 2;     // latent part of a tile: 32 rows x 1024 B
constexpr int TILE_BYTES = TILE * WD * 2;  // + rope part: 32 rows x 128 B = 36 KiB
constexpr int NSTAGE = 4;                  // tiles in the LDS ring
constexpr float SLACK = 32.0f;             // log2 units a score may exceed the reference max

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
template <int NW>
__device__ __forceinline__ void issue_tile(const Args& a, char* buf, int b, int t0, int len, int lane, int wv) {
  constexpr int LPW = 36 / NW;
  const RowMap& m = a.map;
  const bf16* tile;
  if (m.mode == 1) {
    const int pg = page_of(m, b, t0);
    tile = a.cache + ((size_t)pg * m.page_size + (t0 % m.page_size)) * WD;
  } else {
    tile = a.cache + dense_row(m, b, t0, WD);
  }
  const int last = len - 1 - t0;  // last valid row of this tile
#pragma unroll
  for (int k = 0; k < LPW; ++k) {
    const int ld = wv + NW * k;
    if (ld < 32) {
      const int row = ld < last ? ld : last;
      const char* src = (const char*)(tile + (size_t)row * WD) + ((lane ^ sC(ld)) << 4);
      __builtin_amdgcn_global_load_lds((const void*)src, (MLA_LDS void*)(buf + ld * 1024), 16, 0, 0);
    } else {
      const int j = ld - 32;
      const int rl = 8 * j + (lane >> 3);
      const int row = rl < last ? rl : last;
      const char* src = (const char*)(tile + (size_t)row * WD + DC) + (((lane & 7) ^ sR(rl)) << 4);
      __builtin_amdgcn_global_load_lds((const void*)src, (MLA_LDS void*)(buf + C_BYTES + j * 1024), 16, 0, 0);
    }
  }
}

template <int NW>
__device__ __forceinline__ void attend_segment(const Args& a, int r, int lt0, int lt1, bool full, int slot,
                                               char* smem, int lane, int wv) {
  constexpr int LPW = 36 / NW;
  const int H = a.H;
  const int len = a.pl.len[r];
  const int b = row_batch(a.map, r);
  const int g = lane >> 5;              // half of the wave
  const int h = wv * 32 + (lane & 31);  // this lane's head (MFMA column)
  const int ntiles = lt1 - lt0;

  // every wave must be done with the previous segment's LDS tiles
  block_barrier();

  // prologue: first NSTAGE-1 tiles, then this wave's 32 query rows as the
  // B operand of S^T = K Q^T (lane: head h, dims 16ks + 8g .. +7)
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < ntiles) issue_tile<NW>(a, smem + s * TILE_BYTES, b, (lt0 + s) * TILE, len, lane, wv);
  bf16x8 qf[36];
  {
    const bf16* qrow = a.q + ((size_t)r * H + h) * WD + g * 8;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) qf[ks] = *(const bf16x8*)(qrow + ks * 16);
  }
  wait_vmcnt<0>();  // query rows (and the prologue) complete before the loop

  // per-lane LDS byte offsets (tile-relative); remaining terms are immediates
  const int mrow = lane & 31;  // QK: this lane's A-operand row (position)
  int offC[8], offR[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) offC[j] = mrow * 1024 + (((2 * j + g) ^ sC(mrow)) << 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) offR[j] = C_BYTES + mrow * 128 + (((2 * j + g) ^ sR(mrow)) << 4);
  const int q16 = lane & 15;
  const int hf = (lane >> 4) & 1;
  const int rowA = 4 * g + (q16 >> 2);  // PV: rows of the first transposing load (k-step 0)
  const int rowB = rowA + 8;
  const int cb = 2 * hf + ((q16 & 3) >> 1);
  int offA[4], offB[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    offA[u] = rowA * 1024 + (((4 * u + cb) ^ sC(rowA)) << 4) + (q16 & 1) * 8;
    offB[u] = rowB * 1024 + (((4 * u + cb) ^ sC(rowB)) << 4) + (q16 & 1) * 8;
  }

  // Softmax reference. Each head's reference max m_ref is the largest score
  // of the segment's first tile and the weights are 2^(x - m_ref). Keeping
  // the reference fixed keeps the output accumulator free of data-dependent
  // rescaling (a conditional rescale moves it out of the accumulation
  // registers). If a later score exceeds m_ref by more than SLACK the
  // exponent is clamped and the row is flagged; a fix-up pass recomputes
  // flagged rows with the generic kernel. Scores would have to grow by more
  // than 2^32 within one segment for that to happen.
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
      issue_tile<NW>(a, smem + ((it + NSTAGE - 1) % NSTAGE) * TILE_BYTES, b, (lt0 + it + NSTAGE - 1) * TILE,
                     len, lane, wv);
    const char* buf = smem + (it % NSTAGE) * TILE_BYTES;
    const int t0 = (lt0 + it) * TILE;

    // ---- S^T[position][head] = K_tile . Q^T, 36 k-steps of 16 dims. Operand
    // reads run one k-step pair ahead of the MFMAs; the compiler barriers
    // keep the scheduler from hoisting every read (and its registers) up front.
    f32x16 sacc = f32x16{};
    {
      auto kread = [&](int ks) -> bf16x8 {
        const char* p = ks < 32 ? buf + offC[ks & 7] + 256 * (ks >> 3) : buf + offR[ks - 32];
        return *(const MLA_LDS bf16x8*)p;
      };
      bf16x8 k0 = kread(0), k1 = kread(1);
      asm volatile("s_nop 4" ::: "memory");  // VALU write of the zeroed accumulator -> MFMA SrcC
#pragma unroll
      for (int ks = 0; ks < 36; ks += 2) {
        bf16x8 n0 = k0, n1 = k1;
        if (ks + 2 < 36) {
          n0 = kread(ks + 2);
          n1 = kread(ks + 3);
        }
        asm volatile("" ::: "memory");
        mfma_vacc(sacc, k0, qf[ks]);
        mfma_vacc(sacc, k1, qf[ks + 1]);
        k0 = n0;
        k1 = n1;
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
    if (m_ref == -INFINITY) m_ref = tmax;  // first tile of the segment
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
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      auto vread = [&](int db, bool second) -> s16x4 {
        const char* p = buf + (second ? offB[db & 3] : offA[db & 3]) + 256 * (db >> 2) + kk * 16 * 1024;
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)p);
      };
      s16x4 va = vread(0, false), vb = vread(0, true);
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        s16x4 na = va, nb = vb;
        if (db + 1 < 16) {
          na = vread(db + 1, false);
          nb = vread(db + 1, true);
        }
        asm volatile("" ::: "memory");
        s16x8 v8 = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8), pb[kk], o[db], 0, 0, 0);
        va = na;
        vb = nb;
      }
    }
  }
  if (__any(overflow) && lane == 0) atomicOr(a.pl.flags + r, 1);

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

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void attn_mfma_kernel(Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * TILE_BYTES];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
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
    attend_segment<NW>(a, r, lt0, lt1, full, plan_slot(w, c0, per), smem, lane, wv);
  }
}
}  // namespace mf

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
// Recompute rows the MFMA kernel flagged (a score exceeded its fixed softmax
// reference by more than 2^32): the whole row, with a running max, written
// as the final result. Rows are strided over the grid; unflagged rows cost
// one flag read.
template <typename T>
__global__ __launch_bounds__(NT) void fixup_kernel(Args<T> a) {
  __shared__ float tile[TT * (WMAX + 1)];
  __shared__ float qs[HG * WMAX];
  __shared__ float ps[HG * TT];
  __shared__ float alpha_s[HG];
  __shared__ float stat_s[2 * HG];
  float m_run = -INFINITY, l_run = 0.f;
  const int h0 = blockIdx.y * HG;
  for (int r = blockIdx.x; r < a.pl.R; r += gridDim.x) {
    if (a.pl.flags[r] == 0) continue;
    const int len = a.pl.len[r];
    attend_segment<T>(a, r, 0, (len + TT - 1) / TT, true, 0, h0, tile, qs, ps, alpha_s, stat_s, m_run, l_run);
  }
}
}  // namespace gn

// ===========================================================================
// log-sum-exp combine
// ===========================================================================
// Merge n normalised partial results of one (row, head): lse = log sum e^lse_p,
// out = sum_p e^(lse_p - lse) o_p. Parts with lse_p = -inf are skipped (never
// read). Threads of the block split d_c.
template <typename OutT, typename PartFn>
__device__ void combine_head(int n, PartFn part, int d_c, OutT* out, float* lse_out) {
  float mx = -INFINITY;
  for (int p = 0; p < n; ++p) mx = fmaxf(mx, part(p).lse);
  float wsum = 0.f;
  for (int d = threadIdx.x; d < d_c; d += blockDim.x) {
    float acc = 0.f;
    wsum = 0.f;
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

struct PartRef {
  const float* o;
  float lse;
};

template <typename OutT>
__global__ __launch_bounds__(256) void plan_combine_kernel(Plan pl, int H, int d_c, OutT* out, float* lse) {
  const int k = blockIdx.x, h = blockIdx.y;
  const int G = pl.G;
  const int total = pl.cum[pl.R];
  const int per = plan_per_worker(total, G);
  // rows cut by worker boundary (k+1)*per; the row's first boundary handles it
  const int t = (k + 1) * per;
  if (t < total) {
    const int r = plan_row_of(pl.cum, pl.R, t);
    const int c0 = pl.cum[r], c1 = pl.cum[r + 1];
    if (c0 < t && t == (c0 / per + 1) * per) {
      const int w0 = c0 / per, w1 = (c1 - 1) / per;
      auto part = [&](int i) {
        const int w = w0 + i;
        const int slot = plan_slot(w, c0, per);
        return PartRef{pl.part_o + ((size_t)slot * H + h) * d_c, pl.part_lse[(size_t)slot * H + h]};
      };
      combine_head<OutT>(w1 - w0 + 1, part, d_c, out + ((size_t)r * H + h) * d_c,
                         lse ? lse + (size_t)r * H + h : nullptr);
    }
  }
  // rows with nothing visible: zeros and lse = -inf
  for (int r = k; r < pl.R; r += G) {
    if (pl.len[r] != 0) continue;
    for (int d = threadIdx.x; d < d_c; d += blockDim.x) store_f32(out + ((size_t)r * H + h) * d_c + d, 0.f);
    if (threadIdx.x == 0 && lse) lse[(size_t)r * H + h] = -INFINITY;
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
  if (c.H % 32 != 0 || c.H > 128) return false;
  if (c.map.mode == 1 && c.map.page_size % mf::TILE != 0) return false;
  return aligned16(c.q) && aligned16(c.cache) && aligned16(c.out);
}

int attn_tile_size(const AttnCall& c) { return use_mfma(c) ? mf::TILE : gn::TT; }

#define MLA_LAUNCH_CHECK()                                \
  do {                                                    \
    if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP; \
  } while (0)

template <typename T>
static int launch_generic(const AttnCall& c, const Plan& pl) {
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
  return MLA_OK;
}

int launch_attention(const AttnCall& c) {
  const bool mfma = use_mfma(c);
  const int tile = mfma ? mf::TILE : gn::TT;
  Plan pl = plan_layout(c.ws, c.R, c.G, c.H, c.d_c, tile);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, c.stream, c.map, pl);
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
    switch (c.H / 32) {
      case 1: hipLaunchKernelGGL(mf::attn_mfma_kernel<1>, dim3(c.G), dim3(64), 0, c.stream, a); break;
      case 2: hipLaunchKernelGGL(mf::attn_mfma_kernel<2>, dim3(c.G), dim3(128), 0, c.stream, a); break;
      case 3: hipLaunchKernelGGL(mf::attn_mfma_kernel<3>, dim3(c.G), dim3(192), 0, c.stream, a); break;
      default: hipLaunchKernelGGL(mf::attn_mfma_kernel<4>, dim3(c.G), dim3(256), 0, c.stream, a); break;
    }
  } else if (c.dtype == MLA_BF16) {
    launch_generic<bf16>(c, pl);
  } else {
    launch_generic<float>(c, pl);
  }
  MLA_LAUNCH_CHECK();
  if (c.timing_events && hipEventRecord((hipEvent_t)c.timing_events[1], c.stream) != hipSuccess) return MLA_ERR_HIP;
  dim3 cgrid(c.G, c.H);
  if (c.dtype == MLA_BF16)
    hipLaunchKernelGGL(plan_combine_kernel<bf16>, cgrid, dim3(256), 0, c.stream, pl, c.H, c.d_c, (bf16*)c.out, c.lse);
  else
    hipLaunchKernelGGL(plan_combine_kernel<float>, cgrid, dim3(256), 0, c.stream, pl, c.H, c.d_c, (float*)c.out, c.lse);
  MLA_LAUNCH_CHECK();
  if (mfma) {
    gn::Args<bf16> a;
    a.q = (const bf16*)c.q;
    a.cache = (const bf16*)c.cache;
    a.map = c.map;
    a.pl = pl;
    a.H = c.H;
    a.d_c = c.d_c;
    a.d_r = c.d_r;
    a.scale_log2 = c.kq_scale * kLog2e;
    a.out = (bf16*)c.out;
    a.lse = c.lse;
    const int rows_grid = c.R < c.G ? c.R : c.G;
    hipLaunchKernelGGL(gn::fixup_kernel<bf16>, dim3(rows_grid, (c.H + gn::HG - 1) / gn::HG), dim3(gn::NT), 0,
                       c.stream, a);
    MLA_LAUNCH_CHECK();
  }
  return MLA_OK;
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
