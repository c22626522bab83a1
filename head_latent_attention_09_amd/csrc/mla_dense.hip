// Dense products and row kernels around the latent attention, for gfx950:
//
//  * gemm_nt: C[m, n] = sum_k A[m, k] B[n, k] with row strides, batch strides
//    and split-K. Every projection of the steps around the path is this
//    product with the weight stored output-major (a row per output channel):
//    the new token's latent and rope key (tutorial, training form:
//    c = x W_c, x W_kr), the per-head expansion k = W_UK[h] c, v = W_UV[h] c
//    (ferrox-core test, naive branch), the fully absorbed query and output
//    products (notebook: W_aQK, W_aVO and the head sum), and the gated
//    variant's projections (tensortonic Gated MLA: X W^T).
//  * transpose of per-batch matrices (to bring weights stored input-major
//    into the output-major form above);
//  * split-K reduction;
//  * the cache-row epilogue: RMS normalisation of the latent part, rotary
//    rotation of the rope part at the token's position, and the write into a
//    dense or paged cache (ferrox-core: the cached latent is RMS-normed, the
//    rope key roped; notebook: the new row is appended before the query
//    attends);
//  * rotary rotation of query rope parts into the absorbed query rows.
//
// The bf16 product tiles 128 x 128 outputs per workgroup (4 waves of 64 x 64,
// 32x32x16 MFMA), stages 64-wide K slices of A and B in LDS with direct
// global->LDS loads (two slices in flight) and stages the bf16 output through
// LDS so every store writes 16 bytes per lane.
#include "mla_internal.h"

#include <math.h>

namespace mla {

namespace dn {
constexpr int BM = 128, BN = 128, BK = 64, NT = 256;
constexpr int A_BYTES = BM * BK * 2;  // 16 KiB
constexpr int B_BYTES = BN * BK * 2;  // 16 KiB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;

// 16-byte chunk swizzle inside a 128-byte row (8 chunks)
__device__ __forceinline__ int swz8(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename OutT>
struct GemmArgs {
  const bf16* A;   // A[batch * a_batch + m * lda + k]
  const bf16* B;   // B[batch * b_batch + n * ldb + k] for n < n1,
  const bf16* B2;  // B2[batch * b_batch + (n - n1) * ldb + k] for n >= n1 (two weights read as one)
  int n1;
  OutT* C;        // C[batch * c_batch + split * c_split + m * ldc + n]
  int64_t lda, ldb, ldc, a_batch, b_batch, c_batch, c_split;
  int M, N, K;
  int splits, kps;  // split-K: number of splits, K slices (of BK) per split
};

// Loads of one stage: A and B 128 rows x 8 chunks each, 4 + 4 loads of 64
// lanes per wave. Rows past M (N) re-read the last valid row (finite data;
// those outputs are not stored).
// Loads of one stage: A and B 128 rows x 8 chunks each, 4 + 4 loads of 64
// lanes per wave. Rows past M (N) re-read the last valid row (finite data;
// those outputs are not stored). Rows from n1 on come from base2.
__device__ __forceinline__ void issue_rows(const bf16* base, const bf16* base2, int n1, int64_t ld, int row0,
                                           int nrows, int k0, char* dst, int lane, int wv) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ld_i = wv * 4 + i;
    const int p = ld_i * 64 + lane;
    const int row = p >> 3;
    const int c = (p & 7) ^ swz8(row);
    int r = row0 + row;
    r = r < nrows ? r : nrows - 1;
    const bf16* src = (r < n1 ? base + (int64_t)r * ld : base2 + (int64_t)(r - n1) * ld) + k0 + c * 8;
    __builtin_amdgcn_global_load_lds((const void*)src, (MLA_LDS void*)(dst + ld_i * 1024), 16, 0, 0);
  }
}

template <typename OutT>
__global__ __launch_bounds__(NT, 2) void gemm_nt_kernel(GemmArgs<OutT> a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 5;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int batch = blockIdx.z / a.splits, split = blockIdx.z - batch * a.splits;
  const int wm = wv >> 1, wn = wv & 1;
  const int nk_all = a.K / BK;
  const int kc0 = split * a.kps;
  const int nk = min(nk_all - kc0, a.kps);
  const bf16* A = a.A + batch * a.a_batch;
  const bf16* B = a.B + batch * a.b_batch;
  const bf16* B2 = a.B2 + batch * a.b_batch;
  OutT* C = a.C + batch * a.c_batch + split * a.c_split;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  auto issue = [&](int kc, char* st) {
    issue_rows(A, A, a.M, a.lda, m0, a.M, (kc0 + kc) * BK, st, lane, wv);
    issue_rows(B, B2, a.n1, a.ldb, n0, a.N, (kc0 + kc) * BK, st + A_BYTES, lane, wv);
  };
  if (nk > 0) issue(0, smem);
  if (nk > 1) issue(1, smem + STAGE_BYTES);
  for (int kc = 0; kc < nk; ++kc) {
    // this wave's 8 loads of slice kc have landed (the next slice's 8 may be in flight) ...
    if (kc + 1 < nk) __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    barrier();  // ... and every other wave's
    const char* sa = smem + (kc & 1) * STAGE_BYTES;
    const char* sb = sa + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + (lane & 31);
        af[i] = *(const MLA_LDS bf16x8*)(sa + row * 128 + (((2 * ks + g) ^ swz8(row)) * 16));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + j * 32 + (lane & 31);
        bfr[j] = *(const MLA_LDS bf16x8*)(sb + row * 128 + (((2 * ks + g) ^ swz8(row)) * 16));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kc + 2 < nk) {
      barrier();  // every wave is done with this buffer
      issue(kc + 2, smem + (kc & 1) * STAGE_BYTES);
    }
  }

  if constexpr (sizeof(OutT) == 2) {
    // bf16 output staged through LDS: 16-byte stores of whole row segments
    constexpr int OROW = BN * 2 + 16;
    static_assert(BM * OROW <= 2 * STAGE_BYTES, "output tile fits the stage buffers");
    barrier();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          *(MLA_LDS bf16*)(smem + row * OROW + col * 2) = f32_to_bf16(acc[i][j][r]);
        }
      }
    barrier();
#pragma unroll
    for (int it = 0; it < BM * (BN / 8) / NT; ++it) {
      const int idx = it * NT + threadIdx.x;
      const int row = idx >> 4, ch = idx & 15;
      const int m = m0 + row, n = n0 + ch * 8;
      if (m < a.M && n < a.N)
        *(bf16x8*)(C + (int64_t)m * a.ldc + n) = *(const MLA_LDS bf16x8*)(smem + row * OROW + ch * 16);
    }
  } else {
    // fp32 output (split-K partials): 32 consecutive columns per half-wave store
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (m < a.M && n < a.N) C[(int64_t)m * a.ldc + n] = acc[i][j][r];
        }
      }
  }
}

// generic strided product (any sizes, fp32 or bf16 storage, fp32 accumulation):
// one thread per output element
template <typename T, typename OutT>
__global__ __launch_bounds__(256) void gemm_nt_generic_kernel(const T* A, const T* B, OutT* C, int64_t lda,
                                                              int64_t ldb, int64_t ldc, int64_t a_batch,
                                                              int64_t b_batch, int64_t c_batch, int M, int N, int K) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int batch = blockIdx.y;
  if (idx >= (int64_t)M * N) return;
  const int m = (int)(idx / N), n = (int)(idx - (int64_t)m * N);
  const T* a = A + batch * a_batch + (int64_t)m * lda;
  const T* b = B + batch * b_batch + (int64_t)n * ldb;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc += load_f32(a + k) * load_f32(b + k);
  store_f32(C + batch * c_batch + (int64_t)m * ldc + n, acc);
}

// sum of split-K partials [splits][M][ldp] (fp32) into C (ldc), any dtype
template <typename OutT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* P, int splits, int64_t split_stride,
                                                            int64_t ldp, OutT* C, int64_t ldc, int M, int N) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * N) return;
  const int m = (int)(idx / N), n = (int)(idx - (int64_t)m * N);
  float s = 0.f;
  for (int k = 0; k < splits; ++k) s += P[k * split_stride + (int64_t)m * ldp + n];
  store_f32(C + (int64_t)m * ldc + n, s);
}

// out[b][j][i] = in[b][i][j] for [rows x cols] matrices, 32 x 32 tiles through LDS
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* in, T* out, int rows, int cols, int64_t in_batch,
                                                        int64_t out_batch) {
  __shared__ T t[32][33];
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const T* src = in + b * in_batch;
  T* dst = out + b * out_batch;
  for (int y = ty; y < 32; y += 8) {
    const int r = r0 + y, c = c0 + tx;
    if (r < rows && c < cols) t[y][tx] = src[(int64_t)r * cols + c];
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int c = c0 + y, r = r0 + tx;
    if (r < rows && c < cols) dst[(int64_t)c * rows + r] = t[tx][y];
  }
}

// ---------------------------------------------------------------------------
// rotary angles: pair i of a d-wide rope part turns by pos * base^(-2i/d).
// The angle is formed and reduced modulo 2 pi in double precision (positions
// reach tens of thousands of radians, where a float product would lose
// about 1e-3 rad), then sin and cos are taken in float.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rope_angle(int pos, int i, int d, double log2_base, float& c, float& s) {
  const double inv = exp2(-2.0 * (double)i / (double)d * log2_base);
  double ang = (double)pos * inv;
  const double two_pi = 6.283185307179586;
  ang -= two_pi * floor(ang / two_pi);
  sincosf((float)ang, &s, &c);
}

// Cache rows of new tokens from the projections' fp32 partial sums:
// row n of P (summed over splits) is [z_c (d_c) | z_r (d_r)];
//   c   = z_c / sqrt(mean(z_c^2) + eps) * gain
//   k_pe = rotation of z_r at positions[n]
// written to the cache slot of (seq_ids[n], positions[n]). A token whose
// sequence, position or page lies outside the cache is skipped (nothing is
// written for it). One workgroup of 256 threads per token; thread t holds
// elements t, t + 256, ... of the row in registers (the row is at most
// CR_EPT * 256 wide), summing the splits with independent loads.
constexpr int CR_EPT = 20;  // d_c + d_r <= 5120

template <typename T>
__global__ __launch_bounds__(256) void cache_rows_kernel(const float* P, int splits, int64_t split_stride,
                                                         const T* gain, float eps, double log2_base,
                                                         const int32_t* seq_ids, const int32_t* positions, T* cache,
                                                         RowMap map, int n_seqs, int d_c, int d_r) {
  __shared__ float red[4];
  __shared__ float rope_in[1024];
  const int n = blockIdx.x;
  const int W = d_c + d_r;
  const int b = seq_ids[n], pos = positions[n];
  int64_t slot;
  if (b < 0 || b >= n_seqs || pos < 0) return;
  if (map.mode == 1) {
    if (pos >= map.max_pages * map.page_size) return;
    const int pg = map.block_table[(int64_t)b * map.max_pages + pos / map.page_size];
    if (pg < 0 || pg >= map.num_pages) return;
    slot = (int64_t)pg * map.page_size + pos % map.page_size;
  } else {
    if (pos >= map.cache_stride) return;
    slot = (int64_t)b * map.cache_stride + pos;
  }
  T* dst = cache + slot * W;
  const float* src = P + (int64_t)n * W;
  float v[CR_EPT];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < CR_EPT; ++e) {
    const int j = threadIdx.x + 256 * e;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    if (j < W) {
      int k = 0;
      for (; k + 4 <= splits; k += 4) {
        a0 += src[(int64_t)k * split_stride + j];
        a1 += src[(int64_t)(k + 1) * split_stride + j];
        a2 += src[(int64_t)(k + 2) * split_stride + j];
        a3 += src[(int64_t)(k + 3) * split_stride + j];
      }
      for (; k < splits; ++k) a0 += src[(int64_t)k * split_stride + j];
    }
    v[e] = (a0 + a1) + (a2 + a3);
    if (j < d_c) ss += v[e] * v[e];
    else if (j < W) rope_in[j - d_c] = v[e];
  }
  // latent part: sum of squares over the block, then normalise
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(tot / (float)d_c + eps);
#pragma unroll
  for (int e = 0; e < CR_EPT; ++e) {
    const int j = threadIdx.x + 256 * e;
    if (j < d_c) {
      float x = v[e] * inv;
      if (gain) x *= load_f32(gain + j);
      store_f32(dst + j, x);
    }
  }
  // rope part, one pair per thread (the summed values passed through LDS)
  for (int i = threadIdx.x; i < d_r / 2; i += 256) {
    float c, s;
    rope_angle(pos, i, d_r, log2_base, c, s);
    const float x0 = rope_in[2 * i], x1 = rope_in[2 * i + 1];
    store_f32(dst + d_c + 2 * i, x0 * c - x1 * s);
    store_f32(dst + d_c + 2 * i + 1, x0 * s + x1 * c);
  }
}

// The same rows with one wave per token (four tokens per workgroup of 256),
// for rows at most 1024 wide with an even latent width and many tokens: lane l holds
// elements l, l + 64, ... of the row, the sum of squares is a wave reduction,
// and the two elements of a rope pair sit in lanes l and l ^ 1 of the same
// register, so the kernel needs no barrier and no LDS.
constexpr int CRW_EPT = 16;
template <typename T>
__global__ __launch_bounds__(256) void cache_rows_wave_kernel(const float* P, int splits, int64_t split_stride,
                                                              const T* gain, float eps, double log2_base,
                                                              const int32_t* seq_ids, const int32_t* positions,
                                                              T* cache, RowMap map, int n_seqs, int n_tokens, int d_c,
                                                              int d_r) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= n_tokens) return;  // wave-uniform from here on: one token per wave
  const int W = d_c + d_r;
  const int b = seq_ids[n], pos = positions[n];
  int64_t slot;
  if (b < 0 || b >= n_seqs || pos < 0) return;
  if (map.mode == 1) {
    if (pos >= map.max_pages * map.page_size) return;
    const int pg = map.block_table[(int64_t)b * map.max_pages + pos / map.page_size];
    if (pg < 0 || pg >= map.num_pages) return;
    slot = (int64_t)pg * map.page_size + pos % map.page_size;
  } else {
    if (pos >= map.cache_stride) return;
    slot = (int64_t)b * map.cache_stride + pos;
  }
  T* dst = cache + slot * W;
  const float* src = P + (int64_t)n * W;
  float v[CRW_EPT];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < CRW_EPT; ++e) {
    const int j = lane + 64 * e;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    if (j < W) {
      int k = 0;
      for (; k + 4 <= splits; k += 4) {
        a0 += src[(int64_t)k * split_stride + j];
        a1 += src[(int64_t)(k + 1) * split_stride + j];
        a2 += src[(int64_t)(k + 2) * split_stride + j];
        a3 += src[(int64_t)(k + 3) * split_stride + j];
      }
      for (; k < splits; ++k) a0 += src[(int64_t)k * split_stride + j];
    }
    v[e] = (a0 + a1) + (a2 + a3);
    if (j < d_c) ss += v[e] * v[e];
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float inv = 1.0f / sqrtf(ss / (float)d_c + eps);
#pragma unroll
  for (int e = 0; e < CRW_EPT; ++e) {
    const int j = lane + 64 * e;
    const float pv = __shfl_xor(v[e], 1);  // the pair partner (every lane takes part)
    if (j < d_c) {
      float x = v[e] * inv;
      if (gain) x *= load_f32(gain + j);
      store_f32(dst + j, x);
    } else if (j < W) {
      // rope element ri = j - d_c of pair i = ri / 2 (d_c even: the partner is element j ^ 1)
      const int ri = j - d_c;
      float c, sn;
      rope_angle(pos, ri >> 1, d_r, log2_base, c, sn);
      const float y = (ri & 1) ? pv * sn + v[e] * c : v[e] * c - pv * sn;
      store_f32(dst + j, y);
    }
  }
}

// q[n, h, col0 + 2i .. +1] = rotation of q_pe[n, h, 2i .. +1] at positions[n]
template <typename T>
__global__ __launch_bounds__(256) void rope_rows_kernel(const T* src, T* dst, const int32_t* positions, int64_t rows,
                                                        int H, int d_r, int ldd, int col0, double log2_base) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int half = d_r / 2;
  if (idx >= rows * H * half) return;
  const int i = (int)(idx % half);
  const int64_t nh = idx / half;
  const int64_t n = nh / H;
  const float x0 = load_f32(src + nh * d_r + 2 * i), x1 = load_f32(src + nh * d_r + 2 * i + 1);
  T* o = dst + nh * ldd + col0 + 2 * i;
  if (!positions) {  // plain copy
    store_f32(o, x0);
    store_f32(o + 1, x1);
    return;
  }
  float c, s;
  rope_angle(positions[n], i, d_r, log2_base, c, s);
  store_f32(o, x0 * c - x1 * s);
  store_f32(o + 1, x0 * s + x1 * c);
}

template <typename T>
__global__ __launch_bounds__(256) void gate_kernel(T* x, const T* gt, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float gv = load_f32(gt + i);
  store_f32(x + i, load_f32(x + i) * (1.0f / (1.0f + __expf(-gv))));
}

// ---------------------------------------------------------------------------
// Large product with B rows gathered from two matrices: C[m, n] = sum_k
// A[m, k] B(n)[k] (bf16 in and out), where row n of B belongs to group
// g = n / (n1 + n2): its first n1 rows are rows g n1 .. of B1, the next n2
// rows g n2 .. of B2. The per-head key and value expansions of the latent
// rows (k[t,h] = W_UK[h] c_t, v[t,h] = W_UV[h] c_t) run as ONE product whose
// output row holds [k_nope | v] for every head, instead of one product per
// head and tensor that re-reads the latent rows each time.
// 256 x 256 outputs per workgroup of 8 waves (2 x 4, each 128 x 64), 64-wide
// K slices of A and B in LDS (two stages of 64 KiB, direct loads). The MFMA
// takes the B rows as its first operand, so each lane's accumulator holds 4
// consecutive output columns of one row: the bf16 output goes to the LDS
// staging area as 8-byte runs and to HBM as whole 16-byte chunks.
// ---------------------------------------------------------------------------
constexpr int PM = 256, PN = 256, PNT = 512;
constexpr int PA_BYTES = PM * BK * 2;        // 32 KiB
constexpr int PB_BYTES = PN * BK * 2;        // 32 KiB
constexpr int PSTAGE = PA_BYTES + PB_BYTES;  // 64 KiB

struct PairArgs {
  const bf16* A;
  int64_t lda;
  const bf16* B1;
  const bf16* B2;
  int64_t ldb;
  int n1, n2;
  bf16* C;
  int64_t ldc;
  int M, N, K;
  int band, ntn;  // M tiles per XCD, N tiles
};

// Workgroups are dealt to the 8 XCDs round-robin by index; workgroup i runs
// on XCD i % 8. Each XCD takes a band of M tiles (its A rows stay in that
// XCD's L2) and walks every N tile, so A is read from memory about once and
// each B tile once per XCD.
__global__ __launch_bounds__(PNT, 1) void gemm_pair_kernel(PairArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * PSTAGE];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 5;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int mt = xcd * a.band + local % a.band, nt = local / a.band;
  if (mt * PM >= a.M || nt >= a.ntn) return;  // past the last tile (whole workgroup)
  const int m0 = mt * PM, n0 = nt * PN;
  const int wm = wv >> 2, wn = wv & 3;
  const int nk = a.K / BK;

  // the rows this lane loads (fixed over the K slices): loads i = 0..3 of A
  // and of B, 64 lanes x 16 bytes each, cover rows (4 wv + i) * 8 + lane / 8
  const bf16* arow[4];
  const bf16* brow[4];
  int coff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = (wv * 4 + i) * 64 + lane;
    const int row = p >> 3;
    coff[i] = ((p & 7) ^ swz8(row)) * 8;
    int m = m0 + row;
    m = m < a.M ? m : a.M - 1;
    arow[i] = a.A + (int64_t)m * a.lda;
    int n = n0 + row;
    n = n < a.N ? n : a.N - 1;
    const int gs = a.n1 + a.n2;
    const int grp = n / gs, j = n - grp * gs;
    brow[i] = j < a.n1 ? a.B1 + ((int64_t)grp * a.n1 + j) * a.ldb
                       : a.B2 + ((int64_t)grp * a.n2 + (j - a.n1)) * a.ldb;
  }
  auto issue = [&](int kc, char* st) {
    const int k0 = kc * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(arow[i] + k0 + coff[i]),
                                       (MLA_LDS void*)(st + (wv * 4 + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(brow[i] + k0 + coff[i]),
                                       (MLA_LDS void*)(st + PA_BYTES + (wv * 4 + i) * 1024), 16, 0, 0);
  };

  f32x16 acc[4][2];  // [m block][n block], C^T layout: lane l = row m, registers = 4 consecutive n
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  if (nk > 0) issue(0, smem);
  if (nk > 1) issue(1, smem + PSTAGE);
  for (int kc = 0; kc < nk; ++kc) {
    // this wave's 8 loads of slice kc have landed (the next slice's 8 may be in flight) ...
    if (kc + 1 < nk) __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    barrier();  // ... and every other wave's
    const char* sa = smem + (kc & 1) * PSTAGE;
    const char* sb = sa + PA_BYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + (lane & 31);
        af[i] = *(const MLA_LDS bf16x8*)(sa + row * 128 + (((2 * ks + g) ^ swz8(row)) * 16));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + j * 32 + (lane & 31);
        bfr[j] = *(const MLA_LDS bf16x8*)(sb + row * 128 + (((2 * ks + g) ^ swz8(row)) * 16));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (kc + 2 < nk) {
      barrier();  // every wave is done with this buffer
      issue(kc + 2, smem + (kc & 1) * PSTAGE);
    }
  }

  // output, 128 rows at a time through LDS (rows of 256 bf16 + 16 bytes of padding)
  constexpr int OROW = PN * 2 + 16;
  static_assert(128 * OROW <= 2 * PSTAGE, "half the output tile fits the stage buffers");
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    barrier();  // the stage buffers (or the previous half) are free
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int row = i * 32 + (lane & 31);  // within the half
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = wn * 64 + j * 32 + 8 * q + 4 * g;
            bf16x4 v;
            v[0] = f32_to_bf16(acc[i][j][4 * q + 0]);
            v[1] = f32_to_bf16(acc[i][j][4 * q + 1]);
            v[2] = f32_to_bf16(acc[i][j][4 * q + 2]);
            v[3] = f32_to_bf16(acc[i][j][4 * q + 3]);
            *(MLA_LDS bf16x4*)(smem + row * OROW + col * 2) = v;
          }
        }
    }
    barrier();
#pragma unroll
    for (int it = 0; it < 128 * (PN / 8) / PNT; ++it) {
      const int idx = it * PNT + threadIdx.x;
      const int row = idx >> 5, ch = idx & 31;
      const int m = m0 + half * 128 + row, n = n0 + ch * 8;
      if (m < a.M && n < a.N)
        *(bf16x8*)(a.C + (int64_t)m * a.ldc + n) = *(const MLA_LDS bf16x8*)(smem + row * OROW + ch * 16);
    }
  }
}
}  // namespace dn

// ===========================================================================
// host side
// ===========================================================================
static bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

bool gemm_nt_mfma_ok(const GemmDesc& g) {
  return g.dtype == MLA_BF16 && g.K % dn::BK == 0 && g.K > 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
         g.a_batch % 8 == 0 && g.b_batch % 8 == 0 && al16(g.A) && al16(g.B) && (!g.B2 || al16(g.B2)) &&
         (g.out_f32 || (g.N % 8 == 0 && g.ldc % 8 == 0 && g.c_batch % 8 == 0 && al16(g.C)));
}

int launch_gemm_pair(const void* A, int64_t lda, const void* B1, const void* B2, int64_t ldb, int n1, int n2,
                     void* C, int64_t ldc, int M, int N, int K, hipStream_t s) {
  if (M <= 0 || N <= 0) return MLA_OK;
  if (K % dn::BK != 0 || K <= 0 || lda % 8 || ldb % 8 || ldc % 8 || N % 8 || n1 <= 0 || n2 < 0 || !al16(A) ||
      !al16(B1) || (n2 > 0 && !al16(B2)) || !al16(C))
    return MLA_ERR_UNSUPPORTED;
  const int mtiles = (M + dn::PM - 1) / dn::PM, ntiles = (N + dn::PN - 1) / dn::PN;
  const int band = (mtiles + 7) / 8;
  if ((int64_t)8 * band * ntiles > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  dn::PairArgs a{(const bf16*)A, lda, (const bf16*)B1, (const bf16*)B2, ldb, n1, n2, (bf16*)C, ldc, M, N, K,
                 band, ntiles};
  dim3 grid((unsigned)(8 * band * ntiles));
  hipLaunchKernelGGL(dn::gemm_pair_kernel, grid, dim3(dn::PNT), 0, s, a);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int launch_gemm_nt(const GemmDesc& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return MLA_OK;
  // a second weight (rows from n1 on) only on the MFMA path
  if (g.B2 && (g.n1 < 0 || !gemm_nt_mfma_ok(g))) return MLA_ERR_UNSUPPORTED;
  const bf16* B2 = g.B2 ? (const bf16*)g.B2 : (const bf16*)g.B;
  const int n1 = g.B2 ? g.n1 : g.N;
  if (gemm_nt_mfma_ok(g)) {
    const int nk = g.K / dn::BK;
    const int splits = g.splits < 1 ? 1 : (g.splits > nk ? nk : g.splits);
    const int kps = (nk + splits - 1) / splits;
    dim3 grid((unsigned)((g.M + dn::BM - 1) / dn::BM), (unsigned)((g.N + dn::BN - 1) / dn::BN),
              (unsigned)(g.batch * splits));
    if (g.out_f32) {
      dn::GemmArgs<float> a{(const bf16*)g.A, (const bf16*)g.B, B2, n1, (float*)g.C, g.lda, g.ldb, g.ldc,
                            g.a_batch, g.b_batch, g.c_batch, g.c_split, g.M, g.N, g.K, splits, kps};
      hipLaunchKernelGGL(dn::gemm_nt_kernel<float>, grid, dim3(dn::NT), 0, s, a);
    } else {
      if (splits != 1) return MLA_ERR_UNSUPPORTED;
      dn::GemmArgs<bf16> a{(const bf16*)g.A, (const bf16*)g.B, B2, n1, (bf16*)g.C, g.lda, g.ldb, g.ldc,
                           g.a_batch, g.b_batch, g.c_batch, 0, g.M, g.N, g.K, 1, kps};
      hipLaunchKernelGGL(dn::gemm_nt_kernel<bf16>, grid, dim3(dn::NT), 0, s, a);
    }
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  }
  // generic path: one split only (a split-K caller gets its partial in split 0, others zero-free:
  // callers of the generic path pass splits = 1)
  const int64_t total = (int64_t)g.M * g.N;
  dim3 grid((unsigned)((total + 255) / 256), (unsigned)g.batch);
  if (g.dtype == MLA_BF16) {
    if (g.out_f32)
      hipLaunchKernelGGL((dn::gemm_nt_generic_kernel<bf16, float>), grid, dim3(256), 0, s, (const bf16*)g.A,
                         (const bf16*)g.B, (float*)g.C, g.lda, g.ldb, g.ldc, g.a_batch, g.b_batch, g.c_batch, g.M,
                         g.N, g.K);
    else
      hipLaunchKernelGGL((dn::gemm_nt_generic_kernel<bf16, bf16>), grid, dim3(256), 0, s, (const bf16*)g.A,
                         (const bf16*)g.B, (bf16*)g.C, g.lda, g.ldb, g.ldc, g.a_batch, g.b_batch, g.c_batch, g.M,
                         g.N, g.K);
  } else {
    hipLaunchKernelGGL((dn::gemm_nt_generic_kernel<float, float>), grid, dim3(256), 0, s, (const float*)g.A,
                       (const float*)g.B, (float*)g.C, g.lda, g.ldb, g.ldc, g.a_batch, g.b_batch, g.c_batch, g.M,
                       g.N, g.K);
  }
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// number of split-K parts the bf16 product uses for C = A B^T of this size
// (enough workgroups to cover the chip twice), 1 on the generic path
int gemm_nt_splits(const GemmDesc& g, int cus, int max_splits) {
  if (!gemm_nt_mfma_ok(g)) return 1;
  const int64_t tiles = (int64_t)((g.M + dn::BM - 1) / dn::BM) * ((g.N + dn::BN - 1) / dn::BN) * g.batch;
  const int nk = g.K / dn::BK;
  int s = 1;
  while (tiles * s < 2 * (int64_t)cus && s * 2 <= nk && s * 2 <= max_splits) s *= 2;
  const int kps = (nk + s - 1) / s;  // slices per split; no split left empty
  return (nk + kps - 1) / kps;
}

int launch_splitk_reduce(const float* P, int splits, int64_t split_stride, int64_t ldp, void* C, int64_t ldc, int M,
                         int N, int dtype, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  if (total == 0) return MLA_OK;
  dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == MLA_BF16)
    hipLaunchKernelGGL(dn::splitk_reduce_kernel<bf16>, grid, dim3(256), 0, s, P, splits, split_stride, ldp,
                       (bf16*)C, ldc, M, N);
  else
    hipLaunchKernelGGL(dn::splitk_reduce_kernel<float>, grid, dim3(256), 0, s, P, splits, split_stride, ldp,
                       (float*)C, ldc, M, N);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int launch_transpose(const void* in, void* out, int rows, int cols, int batch, int64_t in_batch, int64_t out_batch,
                     int dtype, hipStream_t s) {
  if (rows <= 0 || cols <= 0 || batch <= 0) return MLA_OK;
  dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32), (unsigned)batch);
  if (dtype == MLA_BF16)
    hipLaunchKernelGGL(dn::transpose_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)in, (bf16*)out, rows, cols,
                       in_batch, out_batch);
  else
    hipLaunchKernelGGL(dn::transpose_kernel<float>, grid, dim3(256), 0, s, (const float*)in, (float*)out, rows,
                       cols, in_batch, out_batch);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int launch_cache_rows(const float* P, int splits, int64_t split_stride, const void* gain, float eps, float rope_base,
                      const int32_t* seq_ids, const int32_t* positions, void* cache, const RowMap& map, int n_seqs,
                      int n_tokens, int d_c, int d_r, int dtype, hipStream_t s) {
  if (n_tokens <= 0) return MLA_OK;
  const double lb = log2((double)rope_base);
  // one wave per token once the tokens fill the chip (8192 tokens, 2 splits: 104 -> 96 us);
  // few tokens with many splits (decode) keep 256 threads per token, whose split sums run
  // in parallel (64 tokens, 16 splits: 16 against 24 us)
  if (d_c + d_r <= 64 * dn::CRW_EPT && d_c % 2 == 0 && n_tokens >= 1024) {
    const dim3 grid((unsigned)((n_tokens + 3) / 4));
    if (dtype == MLA_BF16)
      hipLaunchKernelGGL(dn::cache_rows_wave_kernel<bf16>, grid, dim3(256), 0, s, P, splits, split_stride,
                         (const bf16*)gain, eps, lb, seq_ids, positions, (bf16*)cache, map, n_seqs, n_tokens, d_c,
                         d_r);
    else
      hipLaunchKernelGGL(dn::cache_rows_wave_kernel<float>, grid, dim3(256), 0, s, P, splits, split_stride,
                         (const float*)gain, eps, lb, seq_ids, positions, (float*)cache, map, n_seqs, n_tokens, d_c,
                         d_r);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  }
  if (dtype == MLA_BF16)
    hipLaunchKernelGGL(dn::cache_rows_kernel<bf16>, dim3((unsigned)n_tokens), dim3(256), 0, s, P, splits,
                       split_stride, (const bf16*)gain, eps, lb, seq_ids, positions, (bf16*)cache, map, n_seqs, d_c,
                       d_r);
  else
    hipLaunchKernelGGL(dn::cache_rows_kernel<float>, dim3((unsigned)n_tokens), dim3(256), 0, s, P, splits,
                       split_stride, (const float*)gain, eps, lb, seq_ids, positions, (float*)cache, map, n_seqs,
                       d_c, d_r);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int launch_rope_rows(const void* src, void* dst, const int32_t* positions, int64_t rows, int H, int d_r, int ldd,
                     int col0, float rope_base, int dtype, hipStream_t s) {
  const int64_t total = rows * H * (d_r / 2);
  if (total == 0) return MLA_OK;
  if (d_r % 2) return MLA_ERR_SHAPE;
  const double lb = log2((double)rope_base);
  dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == MLA_BF16)
    hipLaunchKernelGGL(dn::rope_rows_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)src, (bf16*)dst, positions,
                       rows, H, d_r, ldd, col0, lb);
  else
    hipLaunchKernelGGL(dn::rope_rows_kernel<float>, grid, dim3(256), 0, s, (const float*)src, (float*)dst,
                       positions, rows, H, d_r, ldd, col0, lb);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int launch_gate(void* x, const void* g, int64_t n, int dtype, hipStream_t s) {
  if (n <= 0) return MLA_OK;
  dim3 grid((unsigned)((n + 255) / 256));
  if (dtype == MLA_BF16)
    hipLaunchKernelGGL(dn::gate_kernel<bf16>, grid, dim3(256), 0, s, (bf16*)x, (const bf16*)g, n);
  else
    hipLaunchKernelGGL(dn::gate_kernel<float>, grid, dim3(256), 0, s, (float*)x, (const float*)g, n);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace mla
