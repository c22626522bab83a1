// Per-head products around the latent attention, for gfx950.
//
//  absorb: q[n,h,j] = sum_i W_UK[h,i,j] q_nope[n,h,i]   (W_UK[h] is [d_nope, d_c];
//          ferrox-core test, absorbed branch; lab Bloque B; MLA_tutorial q W_qc W_kc^T)
//          and q[n,h,d_c:] = q_pe[n,h,:]
//  up_v:   out[n,h,i] = sum_j W_UV[h,i,j] lat[n,h,j]     (W_UV[h] is [d_v, d_c];
//          ferrox-core module doc v[h] = wv_b[h] . out_lat[h])
//
// Both are, per head, C_h = A_h . op(W_h) with A_h the rows [n, h, :] of a
// [N, H, K] tensor. The bf16 path tiles 128 rows x 128 output columns per
// workgroup, stages 64-wide K slices of A and W in LDS with direct
// global->LDS loads (double-buffered), and runs 32x32x16 bf16 MFMA. When W_h
// is stored [K, D] (absorb) its B-operand fragments come from transposing
// LDS loads; when stored [D, K] (up_v) they are plain 16-byte LDS reads.
#include "mla_internal.h"

namespace mla {

namespace gm {
constexpr int BM = 128, BN = 128, BK = 64, NT = 256;
constexpr int A_BYTES = BM * BK * 2;  // 16 KiB
constexpr int B_BYTES = BN * BK * 2;  // 16 KiB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;

// rows of 8 chunks (128 B): A tile and [D,K]-stored W tile
__device__ __forceinline__ int swz8(int r) { return (r ^ (r >> 3)) & 7; }
// rows of 16 chunks (256 B): [K,D]-stored W tile read by 4-row transposing loads
__device__ __forceinline__ int swz16(int r) {
  return (0xCA60 >> (4 * (r & 3))) & 15;  // 0, 6, 10, 12 for r % 4 = 0..3 (a shift, not a branch)
}

struct Args {
  const bf16* A;   // [N, H, K]
  const bf16* W;   // TRANS_W: [H, D, K]; else [H, K, D]
  bf16* out;       // [N, H, ldo], columns 0..D-1 written
  const bf16* tail_src;  // absorb: q_pe [N, H, tail]; else null
  int64_t N;
  int H, K, D, ldo, tail;
};

__device__ __forceinline__ void wait_all_vm() { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); }
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool TRANS_W>
__device__ __forceinline__ void issue_stage(const Args& a, char* st, int64_t n0, int h, int j0, int k0, int lane,
                                            int wv) {
  // A: 128 rows x 8 chunks = 16 loads of 64 lanes (4 per wave)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ld = wv * 4 + i;
    const int p = ld * 64 + lane;
    const int row = p >> 3;
    const int c = (p & 7) ^ swz8(row);
    int64_t n = n0 + row;
    n = n < a.N ? n : a.N - 1;
    const bf16* src = a.A + ((size_t)n * a.H + h) * a.K + k0 + c * 8;
    __builtin_amdgcn_global_load_lds((const void*)src, (MLA_LDS void*)(st + ld * 1024), 16, 0, 0);
  }
  char* sb = st + A_BYTES;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ld = wv * 4 + i;
    const int p = ld * 64 + lane;
    const bf16* src;
    if (TRANS_W) {  // 128 output columns x 8 chunks along K
      const int row = p >> 3;
      const int c = (p & 7) ^ swz8(row);
      src = a.W + ((size_t)h * a.D + j0 + row) * a.K + k0 + c * 8;
    } else {        // 64 K rows x 16 chunks along the output columns
      const int row = p >> 4;
      const int c = (p & 15) ^ swz16(row);
      src = a.W + ((size_t)h * a.K + k0 + row) * a.D + j0 + c * 8;
    }
    __builtin_amdgcn_global_load_lds((const void*)src, (MLA_LDS void*)(sb + ld * 1024), 16, 0, 0);
  }
}

template <bool TRANS_W>
__global__ __launch_bounds__(NT, 2) void gemm_mfma_kernel(Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 5;
  const int64_t n0 = (int64_t)blockIdx.x * BM;
  const int j0 = blockIdx.y * BN;
  const int h = blockIdx.z;
  const int wm = wv >> 1, wn = wv & 1;  // wave tile: rows wm*64.., cols wn*64..
  const int nk = a.K / BK;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // two K slices in flight: both stage buffers are filled up front, and a
  // buffer is refilled as soon as every wave has read it
  issue_stage<TRANS_W>(a, smem, n0, h, j0, 0, lane, wv);
  if (nk > 1) issue_stage<TRANS_W>(a, smem + STAGE_BYTES, n0, h, j0, BK, lane, wv);
  for (int kc = 0; kc < nk; ++kc) {
    // this wave's loads of slice kc have landed (8 per slice, issued in order) ...
    if (kc + 1 < nk) __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8));
    else wait_all_vm();
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
        if (TRANS_W) {
          const int row = wn * 64 + j * 32 + (lane & 31);
          bfr[j] = *(const MLA_LDS bf16x8*)(sb + row * 128 + (((2 * ks + g) ^ swz8(row)) * 16));
        } else {
          // B lane: output column wn*64 + j*32 + lane%32, K slots 16ks + 8g + 0..7;
          // 16-lane group reads 4 K-rows x 16 columns per transposing load.
          const int q16 = lane & 15, hf = (lane >> 4) & 1;
          const int krow = 16 * ks + 8 * g + (q16 >> 2);
          const int c = (wn * 64 + j * 32 + 16 * hf + (q16 & 3) * 4) >> 3;
          const char* pa = sb + krow * 256 + ((c ^ swz16(krow)) * 16) + (q16 & 1) * 8;
          const char* pb = sb + (krow + 4) * 256 + ((c ^ swz16(krow + 4)) * 16) + (q16 & 1) * 8;
          s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)pa);
          s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)pb);
          typedef short s16x8 __attribute__((ext_vector_type(8)));
          s16x8 v8 = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
          bfr[j] = __builtin_bit_cast(bf16x8, v8);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kc + 2 < nk) {
      barrier();  // every wave is done with this buffer
      issue_stage<TRANS_W>(a, smem + (kc & 1) * STAGE_BYTES, n0, h, j0, (kc + 2) * BK, lane, wv);
    }
  }

  // Output through LDS: the accumulator layout (lane column lane%32, rows
  // 8(r/4) + 4g + r%4) would write 2 bytes per lane and store; staged, every
  // store writes 16 bytes per lane and four whole 256-byte row segments per
  // wave.
  constexpr int OROW = BN * 2 + 16;  // 16 bytes of padding per row
  static_assert(BM * OROW <= 2 * STAGE_BYTES, "output tile fits the stage buffers");
  barrier();  // every wave is done reading the stage buffers
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
    const int64_t n = n0 + row;
    if (n < a.N)
      *(bf16x8*)(a.out + ((size_t)n * a.H + h) * a.ldo + j0 + ch * 8) =
          *(const MLA_LDS bf16x8*)(smem + row * OROW + ch * 16);
  }
  // absorb: copy q_pe into the tail of the query rows (once per row block),
  // 16 bytes at a time when the tail is a multiple of 8 values
  if (a.tail_src && blockIdx.y == 0) {
    if ((a.tail & 7) == 0 && ((uintptr_t)a.tail_src & 15) == 0) {
      const int tc = a.tail >> 3;
      for (int idx = threadIdx.x; idx < BM * tc; idx += NT) {
        const int row = idx / tc, c = idx - row * tc;
        const int64_t n = n0 + row;
        if (n < a.N)
          *(bf16x8*)(a.out + ((size_t)n * a.H + h) * a.ldo + a.D + c * 8) =
              *(const bf16x8*)(a.tail_src + ((size_t)n * a.H + h) * a.tail + c * 8);
      }
    } else {
      for (int idx = threadIdx.x; idx < BM * a.tail; idx += NT) {
        const int row = idx / a.tail, k = idx - row * a.tail;
        const int64_t n = n0 + row;
        if (n < a.N) a.out[((size_t)n * a.H + h) * a.ldo + a.D + k] = a.tail_src[((size_t)n * a.H + h) * a.tail + k];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small-row-count up-projection (decode: one row per sequence). The 128x128
// tiles above leave most compute units idle when N is small (N=64, H=128 is
// 128 workgroups), and their two-stage pipeline keeps only one 64-wide K
// slice in flight per workgroup. Here a workgroup owns a 64-row x 64-column
// tile with the whole K extent resident in LDS (NS slices of 64; 128 KiB at
// K=512): every load of the tile is issued up front, and slice s is consumed
// as soon as its loads have landed. Wave (wm, wn) computes rows 32wm..,
// columns 32wn.. with one 32x32x16 MFMA per 16-wide k-step.
// Workgroups are numbered so that the column blocks of one (row block, head)
// run on the same XCD (the dispatcher deals workgroups to the 8 XCDs round
// robin), where they share the A rows in L2.
// ---------------------------------------------------------------------------
constexpr int SM = 64, SN = 64;
constexpr int S_SLICE = (SM + SN) * BK * 2;  // 16 KiB per 64-wide K slice

template <int NS>
__global__ __launch_bounds__(NT, 1) void upv_resident_kernel(Args a, int ncb, int units) {
  __shared__ __attribute__((aligned(1024))) char smem[NS * S_SLICE];
  const int L = blockIdx.x;
  const int unit = (L / (8 * ncb)) * 8 + (L & 7);  // (row block, head)
  if (unit >= units) return;
  const int cb = (L >> 3) % ncb;
  const int h = unit % a.H;
  const int64_t n0 = (int64_t)(unit / a.H) * SM;
  const int j0 = cb * SN;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 5;
  const int wm = wv >> 1, wn = wv & 1;

  // loads: per slice 8 of A (64 rows x 8 chunks) and 8 of W, two of each per wave
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    char* st = smem + sl * S_SLICE;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ld = wv * 2 + i;
      const int p = ld * 64 + lane;
      const int row = p >> 3;
      const int c = (p & 7) ^ swz8(row);
      int64_t n = n0 + row;
      n = n < a.N ? n : a.N - 1;
      __builtin_amdgcn_global_load_lds((const void*)(a.A + ((size_t)n * a.H + h) * a.K + sl * BK + c * 8),
                                       (MLA_LDS void*)(st + ld * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ld = wv * 2 + i;
      const int p = ld * 64 + lane;
      const int row = p >> 3;
      const int c = (p & 7) ^ swz8(row);
      __builtin_amdgcn_global_load_lds((const void*)(a.W + ((size_t)h * a.D + j0 + row) * a.K + sl * BK + c * 8),
                                       (MLA_LDS void*)(st + SM * 128 + ld * 1024), 16, 0, 0);
    }
  }

  f32x16 acc = f32x16{};
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    // this wave's loads of slices 0..sl have landed (4 per slice, issued in order)
    switch (NS - 1 - sl) {  // a constant once the loop is unrolled
#define MLA_VM(K_)                                                                   \
  case K_:                                                                         \
    __builtin_amdgcn_s_waitcnt(((4 * K_) & 15) | (((4 * K_) >> 4) << 14) | (7 << 4) | (15 << 8)); \
    break;
      MLA_VM(0) MLA_VM(1) MLA_VM(2) MLA_VM(3) MLA_VM(4) MLA_VM(5) MLA_VM(6) MLA_VM(7)
#undef MLA_VM
    }
    barrier();  // ... and every other wave's
    const char* sa = smem + sl * S_SLICE;
    const char* sb = sa + SM * 128;
    const int ra = wm * 32 + (lane & 31), rb = wn * 32 + (lane & 31);
    bf16x8 af[BK / 16], bfr[BK / 16];  // all fragments of the slice first: one LDS latency per slice
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      af[ks] = *(const MLA_LDS bf16x8*)(sa + ra * 128 + (((2 * ks + g) ^ swz8(ra)) * 16));
      bfr[ks] = *(const MLA_LDS bf16x8*)(sb + rb * 128 + (((2 * ks + g) ^ swz8(rb)) * 16));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], bfr[ks], acc, 0, 0, 0);
  }
  const int col = j0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t n = n0 + wm * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
    if (n < a.N) a.out[((size_t)n * a.H + h) * a.ldo + col] = f32_to_bf16(acc[r]);
  }
}

// ---------------------------------------------------------------------------
// Query absorption with a short contraction (d_nope <= 128): a workgroup owns
// one (head, 128-column block). Its W_UK block (K x 128) passes through LDS
// once into registers (each wave keeps the B fragments of its 64 columns: 64
// VGPRs at K=128), so the whole LDS serves a five-buffer ring of 64-row
// q_nope blocks with four blocks in flight. Each 64x128 output block is
// staged through the consumed ring buffer and stored as whole 256-byte row
// segments. The q_pe tail of the query rows is copied at the end, split over
// the column-block workgroups of a head. With K this short the per-tile
// kernel waits for its first loads most of the time; streaming keeps loads
// in flight across row blocks.
// ---------------------------------------------------------------------------
constexpr int ABM = 64;                        // rows per streamed block
constexpr int ANB = 5;                         // ring buffers (four blocks in flight)
constexpr int A_SLICE = ABM * BK * 2;          // 8 KiB: 64 rows x 64 K
constexpr int A_BLOCK = 2 * A_SLICE;           // room for K <= 128
constexpr int W_SLICE = BK * BN * 2;           // 16 KiB: 64 K rows x 128 columns
constexpr int ABS_SMEM = ANB * A_BLOCK;        // 80 KiB: two workgroups per CU
static_assert(ABM * BN * 2 <= A_BLOCK, "output block staged in a ring buffer");
static_assert(2 * W_SLICE <= ABS_SMEM, "W_UK block passes through the ring");

// vmcnt wait with a run-time count (a jump table of immediate waits)
__device__ __forceinline__ void wait_vm_n(int n) {
  switch (n) {
#define MLA_G(k) \
  case k:        \
    __builtin_amdgcn_s_waitcnt(((k) & 15) | (7 << 4) | (15 << 8) | (((k) >> 4) << 14)); \
    break;
#define MLA_G8(k) MLA_G(k) MLA_G(k + 1) MLA_G(k + 2) MLA_G(k + 3) MLA_G(k + 4) MLA_G(k + 5) MLA_G(k + 6) MLA_G(k + 7)
    MLA_G8(0) MLA_G8(8) MLA_G8(16) MLA_G8(24) MLA_G(32)
#undef MLA_G8
#undef MLA_G
    default: __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  }
}

// Direct global->LDS load of 64 lanes x 16 bytes (lane l: gbase + voff to
// LDS lds + 16 l), issued from inline asm: for the builtin the compiler waits
// for every such load in flight before any LDS read, which would drain the
// loads prefetched for later blocks. Completion is waited for explicitly.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(gbase), "s"(lds) : "memory");
}
__device__ __forceinline__ uint32_t lds_u32(const void* p) { return (uint32_t)(uintptr_t)(const MLA_LDS char*)p; }

// output staging: chunk c (8 columns) of row r at chunk c ^ (r & 15)
__device__ __forceinline__ int ostage(int r, int col) {
  return r * (BN * 2) + ((((col >> 3) ^ (r & 15))) << 4) + (col & 7) * 2;
}

__global__ __launch_bounds__(NT, 2) void absorb_stream_kernel(Args a, int parts) {
  __shared__ __attribute__((aligned(1024))) char smem[ABS_SMEM];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 5;
  const int ncb = a.D / BN;
  const int unit = blockIdx.x / parts, part = blockIdx.x - unit * parts;
  const int h = unit / ncb, cb = unit - h * ncb;
  const int j0 = cb * BN;
  const int ns = a.K / BK;                // 1 or 2 K slices
  const int64_t nrb = (a.N + ABM - 1) / ABM;
  const int nt = (int)((nrb - part + parts - 1) / parts);  // row blocks of this workgroup: part + parts * i
  const int wm = wv >> 1, wn = wv & 1;    // wave tile: rows 32wm.., columns 64wn..

  // W_UK[h][k][j0 ..] through LDS (per slice 64 rows x 16 chunks, 4 loads per
  // wave) into registers: B fragments of this wave's columns for every k-step
#pragma unroll
  for (int sl = 0; sl < 2; ++sl)
    if (sl < ns)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ld = wv * 4 + i;
        const int p = ld * 64 + lane;
        const int row = p >> 4;
        const int c = (p & 15) ^ swz16(row);
        dma16(a.W + ((size_t)h * a.K + sl * BK) * a.D + j0, (uint32_t)((row * a.D + c * 8) * 2),
              lds_u32(smem + sl * W_SLICE + ld * 1024));
      }
  wait_all_vm();
  barrier();
  bf16x8 bw[2][BK / 16][2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl)
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (sl >= ns) {
          bw[sl][ks][j] = bf16x8{};
          continue;
        }
        const char* sb = smem + sl * W_SLICE;
        const int q16 = lane & 15, hf = (lane >> 4) & 1;
        const int krow = 16 * ks + 8 * g + (q16 >> 2);
        const int c = (wn * 64 + j * 32 + 16 * hf + (q16 & 3) * 4) >> 3;
        const char* pa = sb + krow * 256 + ((c ^ swz16(krow)) * 16) + (q16 & 1) * 8;
        const char* pb = sb + (krow + 4) * 256 + ((c ^ swz16(krow + 4)) * 16) + (q16 & 1) * 8;
        s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)pa);
        s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)pb);
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        s16x8 v8 = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
        bw[sl][ks][j] = __builtin_bit_cast(bf16x8, v8);
      }
  barrier();  // every wave holds its fragments: the ring may be overwritten

  // A block t into ring buffer t % ANB: per slice 64 rows x 8 chunks, 2 loads per wave
  auto issue_a = [&](int t) {
    const int64_t r0 = (int64_t)(part + (int64_t)parts * t) * ABM;
    char* st = smem + (t % ANB) * A_BLOCK;
    const bf16* base = a.A + ((size_t)r0 * a.H + h) * a.K;  // row r0 of head h
    const int64_t last = a.N - 1 - r0;                       // rows past the end re-read the last row
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
      if (sl < ns)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int ld = wv * 2 + i;
          const int p = ld * 64 + lane;
          const int row0 = p >> 3;
          const int c = (p & 7) ^ swz8(row0);
          const int row = row0 < last ? row0 : (int)last;
          dma16(base, (uint32_t)(((size_t)row * a.H * a.K + sl * BK + c * 8) * 2),
                lds_u32(st + sl * A_SLICE + ld * 1024));
        }
  };
  constexpr int AHEAD_A = ANB - 1;  // blocks in flight
  const int LA = 2 * ns;            // A loads per block and wave
  constexpr int LS = 4;             // output stores per block and wave (64 rows x 256 B)
  for (int t = 0; t < AHEAD_A && t < nt; ++t) issue_a(t);

  for (int t = 0; t < nt; ++t) {
    // every wave is done with the staging of block t-1 (ring buffer (t+4) % 5)
    barrier();
    if (t + AHEAD_A < nt) issue_a(t + AHEAD_A);
    // this wave's memory operations issued after block t's loads: blocks
    // t+1 .. t+4 that exist, and the stores of blocks max(0, t-4) .. t-1
    int after = 0;
#pragma unroll
    for (int k = 1; k <= AHEAD_A; ++k) after += (t + k < nt ? LA : 0) + (t - k >= 0 ? LS : 0);
    wait_vm_n(after);
    barrier();  // block t complete for every wave
    const char* sa = smem + (t % ANB) * A_BLOCK;
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    const int ra = wm * 32 + (lane & 31);
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
      if (sl < ns)
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
          const bf16x8 af = *(const MLA_LDS bf16x8*)(sa + sl * A_SLICE + ra * 128 + (((2 * ks + g) ^ swz8(ra)) * 16));
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bw[sl][ks][j], acc[j], 0, 0, 0);
        }
    barrier();  // every wave is done reading block t: its buffer stages the output
    char* so = smem + (t % ANB) * A_BLOCK;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        *(MLA_LDS bf16*)(so + ostage(row, col)) = f32_to_bf16(acc[j][r]);
      }
    }
    barrier();
    const int64_t r0 = (int64_t)(part + (int64_t)parts * t) * ABM;
#pragma unroll
    for (int it = 0; it < LS; ++it) {
      const int idx = it * NT + threadIdx.x;
      const int row = idx >> 4, ch = idx & 15;
      const int64_t n = r0 + row;
      const bf16x8 v = *(const MLA_LDS bf16x8*)(so + row * (BN * 2) + ((ch ^ (row & 15)) << 4));
      if (n < a.N) *(bf16x8*)(a.out + ((size_t)n * a.H + h) * a.ldo + j0 + ch * 8) = v;
    }
  }

  // q_pe into the tail of the query rows: the rows of this workgroup's row
  // blocks are dealt round robin to the head's column-block workgroups, each
  // row copied whole by consecutive threads (16 bytes each); four loads in
  // flight per thread before their stores
  if (a.tail_src) {
    const int tc = a.tail >> 3;  // chunks per row (the tail is a multiple of 8 values)
    const int64_t rows = (int64_t)nt * ABM;
    const int64_t mine = rows > cb ? (rows - cb + ncb - 1) / ncb : 0;  // rows cb, cb + ncb, ...
    const int64_t total = mine * tc;
    for (int64_t w0 = threadIdx.x; w0 < total; w0 += (int64_t)NT * 4) {
      bf16x8 v[4];
      int64_t nn[4];
      int cc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t w = w0 + (int64_t)NT * u;
        nn[u] = -1;
        if (w < total) {
          const int64_t j = w / tc;
          cc[u] = (int)(w - j * tc);
          const int64_t rr = cb + ncb * j;  // row of this workgroup's blocks
          const int64_t t = rr / ABM;
          const int64_t n = (int64_t)(part + (int64_t)parts * t) * ABM + (rr - t * ABM);
          if (n < a.N) {
            nn[u] = n;
            v[u] = *(const bf16x8*)(a.tail_src + ((size_t)n * a.H + h) * a.tail + cc[u] * 8);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (nn[u] >= 0) *(bf16x8*)(a.out + ((size_t)nn[u] * a.H + h) * a.ldo + a.D + cc[u] * 8) = v[u];
    }
  }
}
}  // namespace gm

// generic per-head product: one thread per output element, fp32 accumulation
template <typename T, bool TRANS_W>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const T* A, const T* W, T* out, int64_t N, int H, int K,
                                                           int D, int ldo) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = N * H * (int64_t)D;
  if (idx >= total) return;
  const int i = (int)(idx % D);
  const int64_t nh = idx / D;
  const int h = (int)(nh % H);
  const T* a = A + nh * K;
  float acc = 0.f;
  if (TRANS_W) {
    const T* w = W + ((size_t)h * D + i) * K;
    for (int k = 0; k < K; ++k) acc += load_f32(a + k) * load_f32(w + k);
  } else {
    const T* w = W + (size_t)h * K * D + i;
    for (int k = 0; k < K; ++k) acc += load_f32(a + k) * load_f32(w + (size_t)k * D);
  }
  store_f32(out + nh * ldo + i, acc);
}

template <typename T>
__global__ __launch_bounds__(256) void copy_tail_kernel(const T* src, T* out, int64_t rows, int tail, int ldo,
                                                        int col0) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * tail) return;
  const int64_t row = idx / tail;
  const int k = (int)(idx - row * tail);
  out[row * ldo + col0 + k] = src[idx];
}

static bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

template <typename T, bool TRANS_W>
static int run_generic(const void* A, const void* W, void* out, int64_t N, int H, int K, int D, int ldo,
                       hipStream_t s) {
  const int64_t total = N * H * (int64_t)D;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0)
    hipLaunchKernelGGL((gemm_generic_kernel<T, TRANS_W>), dim3((unsigned)blocks), dim3(256), 0, s, (const T*)A,
                       (const T*)W, (T*)out, N, H, K, D, ldo);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

static bool mfma_ok(int K, int D, int ldo, const void* A, const void* W, const void* out) {
  return K % gm::BK == 0 && D % gm::BN == 0 && ldo % 8 == 0 && al16(A) && al16(W) && al16(out);
}

int launch_absorb(const void* q_nope, const void* q_pe, const void* w_uk, void* q, int64_t N, int H, int d_nope,
                  int d_c, int d_r, int dtype, hipStream_t s) {
  const int ldo = d_c + d_r;
  if (dtype == MLA_BF16 && mfma_ok(d_nope, d_c, ldo, q_nope, w_uk, q)) {
    gm::Args a{(const bf16*)q_nope, (const bf16*)w_uk, (bf16*)q, d_r > 0 ? (const bf16*)q_pe : nullptr,
               N, H, d_nope, d_c, ldo, d_r};
    if (d_nope <= 2 * gm::BK && d_r % 8 == 0 && (d_r == 0 || al16(q_pe))) {
      // one workgroup per (head, column block), or several splitting the row
      // blocks when there are fewer than two per compute unit
      int cus = mla_default_workers();
      if (cus <= 0) cus = 256;
      const int64_t units = (int64_t)H * (d_c / gm::BN);
      const int64_t nrb = (N + gm::ABM - 1) / gm::ABM;
      int64_t parts = (2 * (int64_t)cus + units - 1) / units;
      if (parts > nrb) parts = nrb;
      if (parts < 1) parts = 1;
      if (units * parts <= INT32_MAX) {
        hipLaunchKernelGGL(gm::absorb_stream_kernel, dim3((unsigned)(units * parts)), dim3(gm::NT), 0, s, a,
                           (int)parts);
        return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
      }
    }
    dim3 grid((unsigned)((N + gm::BM - 1) / gm::BM), d_c / gm::BN, H);
    hipLaunchKernelGGL(gm::gemm_mfma_kernel<false>, grid, dim3(gm::NT), 0, s, a);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  }
  int st = dtype == MLA_BF16 ? run_generic<bf16, false>(q_nope, w_uk, q, N, H, d_nope, d_c, ldo, s)
                             : run_generic<float, false>(q_nope, w_uk, q, N, H, d_nope, d_c, ldo, s);
  if (st != MLA_OK || d_r == 0 || !q_pe) return st;  // no q_pe: the tail is written elsewhere
  const int64_t rows = N * H;
  const int64_t blocks = (rows * d_r + 255) / 256;
  if (dtype == MLA_BF16)
    hipLaunchKernelGGL(copy_tail_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, s, (const bf16*)q_pe, (bf16*)q,
                       rows, d_r, ldo, d_c);
  else
    hipLaunchKernelGGL(copy_tail_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, (const float*)q_pe,
                       (float*)q, rows, d_r, ldo, d_c);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int launch_up_v(const void* lat, const void* w_uv, void* out, int64_t N, int H, int d_c, int d_v, int dtype,
                hipStream_t s) {
  if (dtype == MLA_BF16 && mfma_ok(d_c, d_v, d_v, lat, w_uv, out)) {
    gm::Args a{(const bf16*)lat, (const bf16*)w_uv, (bf16*)out, nullptr, N, H, d_c, d_v, d_v, 0};
    const int64_t big_tiles = (N + gm::BM - 1) / gm::BM * (d_v / gm::BN) * H;
    const int ns = d_c / gm::BK;
    if (big_tiles < 512 && ns <= 8) {  // too few 128x128 tiles to fill the chip: 64x64, K resident
      const int ncb = d_v / gm::SN;
      const int64_t units = (N + gm::SM - 1) / gm::SM * H;
      const unsigned blocks = (unsigned)((units + 7) / 8 * 8 * ncb);
      switch (ns) {
#define MLA_UPV(NS_)                                                                              \
  case NS_:                                                                                     \
    hipLaunchKernelGGL(gm::upv_resident_kernel<NS_>, dim3(blocks), dim3(gm::NT), 0, s, a, ncb, (int)units); \
    break;
        MLA_UPV(1) MLA_UPV(2) MLA_UPV(3) MLA_UPV(4) MLA_UPV(5) MLA_UPV(6) MLA_UPV(7) MLA_UPV(8)
#undef MLA_UPV
      }
      return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
    }
    dim3 grid((unsigned)((N + gm::BM - 1) / gm::BM), d_v / gm::BN, H);
    hipLaunchKernelGGL(gm::gemm_mfma_kernel<true>, grid, dim3(gm::NT), 0, s, a);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  }
  return dtype == MLA_BF16 ? run_generic<bf16, true>(lat, w_uv, out, N, H, d_c, d_v, d_v, s)
                           : run_generic<float, true>(lat, w_uv, out, N, H, d_c, d_v, d_v, s);
}

}  // namespace mla
