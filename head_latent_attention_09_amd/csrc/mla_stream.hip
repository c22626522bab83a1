// Products of a few rows with a large weight matrix, for gfx950:
//
//   C[m, n] = sum_k X[m, k] W[n, k],  m < M <= 64.
//
// The decode step's head-summed output of the fully absorbed layer is this
// shape, out_n = W_aVO concat_h(o_n[h])
// (MLA_RoPE-less.ipynb, matrix absorption and the adding trick; MLA_tutorial
// formula.md Part 3, inference form): 64 tokens against a 5120 x 65536
// weight, read once (1,000 weight bytes per byte of X). The kernel is a
// weight stream:
//
//  * a workgroup owns 256 weight rows (8 waves of 32) over a contiguous K
//    range (split-K when there are too few row tiles to fill the chip);
//  * each wave loads its rows straight into registers in the 32x32x16 MFMA
//    A-operand layout and keeps a ring of 32 k-steps (32 KiB per wave) in
//    flight: a k-step's slot is reloaded right after the MFMAs that read it;
//  * X is staged in LDS in 256-wide K blocks (four-block ring, loaded three
//    blocks ahead through registers, one barrier per block) and read by every
//    wave as the B operand (64 rows = two 32-column MFMA blocks);
//  * the output is fp32 partials per K split, summed by the caller's next
//    kernel (the split-K reduction, or the cache-row epilogue).
//
// Measured on MI355X against the 128 x 128 tiled product: 0.155 against
// 0.161 ms for that output product (4.4 TB/s; a plain read of the same
// matrix reaches about 5.9 TB/s on the same parts), but slower for the
// absorbed query (6 K blocks per workgroup: the ring's fill and drain are a
// third of the work) and for the cache-append projection at 64 tokens (576
// rows), which stay on the tiled product.
#include "mla_internal.h"

#include <type_traits>

namespace mla {

namespace ws {
constexpr int NW = 8;               // waves per workgroup
constexpr int NT = 64 * NW;         // 512 threads
constexpr int TN = 32 * NW;         // weight rows per workgroup
constexpr int KB = 256;             // K per X block
constexpr int KS = KB / 16;         // 32x32x16 k-steps per block
constexpr int XB = 4;               // X blocks resident in LDS
constexpr int XROW = KB * 2 + 16;   // bytes of one X row in a block: 32 chunks of 16 B and one of padding
constexpr int XBLK = 64 * XROW;     // 33 KiB
constexpr int XLD = 64 * KB * 2 / (16 * NT);  // 16-byte X loads per thread per block (4)
constexpr int NS = 2 * KS;          // weight ring: k-steps in flight per wave

struct Args {
  const bf16* X;
  int64_t ldx;
  const bf16* W;
  int64_t ldw;
  float* P;  // fp32 partials [splits][M][N] (ld N)
  int64_t p_split;
  int M, N, K, splits, nblk;
};

// X row t, 16-byte chunk c of a block at t * XROW + 16 c: the padding chunk
// moves consecutive rows by four banks, so the 16 lanes of a B-operand read
// pass (16 rows, one chunk) fall on distinct banks, and a lane's address
// for k-step ks is its own base plus 32 ks (an immediate offset)
__device__ __forceinline__ int x_off(int t, int c) { return t * XROW + (c << 4); }

__global__ __launch_bounds__(NT, 1) void stream_gemm_kernel(Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[XB * XBLK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int ntile = __builtin_amdgcn_readfirstlane(blockIdx.x / a.splits);
  const int split = __builtin_amdgcn_readfirstlane(blockIdx.x - ntile * a.splits);
  const int b0 = (int)((int64_t)split * a.nblk / a.splits);
  const int nb = (int)((int64_t)(split + 1) * a.nblk / a.splits) - b0;
  const int64_t k0 = (int64_t)b0 * KB;
  const int nks = nb * KS;  // k-steps of this workgroup

  // Weight rows of this wave: row0 .. row0 + 31; rows past N re-read the last one (their
  // outputs are not stored). The address of a load is a wave-uniform base (first row, K
  // position) plus a 32-bit lane offset (row and K half), so that no 64-bit address is held
  // per load.
  const int row0 = ntile * TN + wv * 32;
  const int rb = min(row0, a.N - 1);
  const char* wbase = (const char*)(a.W + (int64_t)rb * a.ldw) + k0 * 2;
  const uint32_t woff = (uint32_t)((min(row0 + (lane & 31), a.N - 1) - rb) * a.ldw * 2 + 16 * g);
  // (default cache policy: a load reads a quarter of a 128-byte line, the next three k-steps
  // the rest of it, which a non-temporal policy would fetch again each time)
  auto w_load = [&](int t) -> bf16x8 {
    return *(const bf16x8*)(wbase + 32 * (int64_t)min(t, nks - 1) + woff);
  };

  // X loads of block b: thread tid, load i covers row p / 32, chunk p % 32 with p = i * NT + tid
  // (rows past M re-read the last one)
  const char* xbase = (const char*)a.X + k0 * 2;
  uint32_t xoff[XLD];
#pragma unroll
  for (int i = 0; i < XLD; ++i) {
    const int p = i * NT + tid;
    xoff[i] = (uint32_t)(min(p >> 5, a.M - 1) * a.ldx * 2 + (p & 31) * 16);
  }
  auto x_load = [&](int b, int i) -> bf16x8 {
    return *(const bf16x8*)(xbase + (int64_t)min(b, nb - 1) * (KB * 2) + xoff[i]);
  };
  auto x_put = [&](int slot, int i, const bf16x8& v) {
    const int p = i * NT + tid;
    *(MLA_LDS bf16x8*)(smem + slot * XBLK + x_off(p >> 5, p & 31)) = v;
  };

  // Every load is unconditional, so that the compiler's count of loads in flight (and the
  // waits it derives from it) is exact: k-steps and blocks past the end re-read the last one
  // (lines just read: cache hits), and what they bring is never used.
  // prologue: X blocks 0 and 1 into slots 0 and 1, block 2 in flight, the weight ring filled.
  // Block 2 is loaded before the second half of the ring, as every later X block is loaded
  // before the 16 weight reloads of a block, so that its wait at the end of block 0 is as
  // deep as the loop's (the compiler takes the shallower of the two).
  bf16x8 wr[NS];
  bf16x8 xa[XLD], xb[XLD];
  {
#pragma unroll
    for (int t = 0; t < KS; ++t) wr[t] = w_load(t);
    bf16x8 xr[2][XLD];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < XLD; ++i) xr[b][i] = x_load(b, i);
#pragma unroll
    for (int i = 0; i < XLD; ++i) xa[i] = x_load(2, i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = KS; t < NS; ++t) wr[t] = w_load(t);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < XLD; ++i) x_put(b, i, xr[b][i]);
  }
  __syncthreads();

  f32x16 acc[2] = {f32x16{}, f32x16{}};
  // One X block: its k-steps use ring slots HALF * KS .. HALF * KS + KS - 1. X block b + 3 is
  // loaded at its start and block b + 2 (loaded at the start of block b - 1) written to LDS at
  // its end, so that the wait for an X load lies as far behind its issue as a weight slot's
  // (two blocks): under a saturated memory system a load takes about as long as the whole
  // ring, and a shallower wait would drain the ring at every block.
  auto block = [&](int b, auto half_c, bf16x8 (&xin)[XLD], bf16x8 (&xout)[XLD]) {
    constexpr int HALF = decltype(half_c)::value;
#pragma unroll
    for (int i = 0; i < XLD; ++i) xout[i] = x_load(b + 3, i);
    // the order of loads fixes the waits the compiler derives: keep it as written (X first,
    // then one weight reload per k-step, right after the MFMAs that read its slot)
    __builtin_amdgcn_sched_barrier(0);
    const char* xs = smem + (b & (XB - 1)) * XBLK + (lane & 31) * XROW + 16 * g;
    const int t0 = b * KS;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 x0 = *(const MLA_LDS bf16x8*)(xs + 32 * ks);
      const bf16x8 x1 = *(const MLA_LDS bf16x8*)(xs + 32 * XROW + 32 * ks);
      bf16x8& w = wr[HALF * KS + ks];
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, x0, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, x1, acc[1], 0, 0, 0);
      w = w_load(t0 + ks + NS);
      __builtin_amdgcn_sched_barrier(0);
    }
    // block b + 2 into the slot block b - 2 used (every wave passed the barrier that ended it);
    // past the end this writes a slot no later block reads
    const int slot = (b + 2) & (XB - 1);
#pragma unroll
    for (int i = 0; i < XLD; ++i) x_put(slot, i, xin[i]);
    __syncthreads();
  };
  int b = 0;
  for (; b + 1 < nb; b += 2) {
    block(b, std::integral_constant<int, 0>{}, xa, xb);
    block(b + 1, std::integral_constant<int, 1>{}, xb, xa);
  }
  if (b < nb) block(b, std::integral_constant<int, 0>{}, xa, xb);

  // D layout: lane l holds column (X row) 32 j + l % 32 and weight rows 8 (q / 4) + 4 g + q % 4
  const int nbase = ntile * TN + wv * 32 + 4 * g;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = 32 * j + (lane & 31);
    if (m >= a.M) continue;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int c = nbase + 8 * q4;
      if (c >= a.N) continue;
      *(f32x4*)(a.P + (int64_t)split * a.p_split + (int64_t)m * a.N + c) =
          f32x4{acc[j][4 * q4], acc[j][4 * q4 + 1], acc[j][4 * q4 + 2], acc[j][4 * q4 + 3]};
    }
  }
}
}  // namespace ws

bool stream_gemm_ok(const StreamDesc& d) {
  auto al = [](const void* p, int b) { return p == nullptr || ((uintptr_t)p & (b - 1)) == 0; };
  if (d.M < 1 || d.M > 64 || d.N < 1 || d.K < ws::KB || d.K % ws::KB) return false;
  if (d.N % 4 || d.ldx % 8 || d.ldw % 8) return false;
  // 32-bit lane offsets: 256 weight rows and 64 X rows of a workgroup within 2 GiB
  if (d.ldw > (1 << 22) || d.ldx > (1 << 24)) return false;
  if (!d.X || !d.W || !al(d.X, 16) || !al(d.W, 16)) return false;
  return d.P && al(d.P, 16) && d.p_split >= (int64_t)d.M * d.N;
}

int stream_gemm_splits(int N, int K, int cus, int max_splits) {
  const int tiles = (N + ws::TN - 1) / ws::TN;
  const int nblk = K / ws::KB;
  int s = cus / tiles;  // at most one workgroup per CU: no second, partly filled round
  s = s < 1 ? 1 : s;
  s = s > nblk ? nblk : s;
  return s > max_splits ? max_splits : s;
}

int launch_stream_gemm(const StreamDesc& d, hipStream_t s) {
  if (!stream_gemm_ok(d)) return MLA_ERR_UNSUPPORTED;
  if (d.splits < 1 || d.splits > d.K / ws::KB) return MLA_ERR_UNSUPPORTED;
  const int tiles = (d.N + ws::TN - 1) / ws::TN;
  ws::Args a{(const bf16*)d.X, d.ldx, (const bf16*)d.W, d.ldw, d.P, d.p_split, d.M, d.N, d.K, d.splits,
             d.K / ws::KB};
  hipLaunchKernelGGL(ws::stream_gemm_kernel, dim3((unsigned)(tiles * d.splits)), dim3(ws::NT), 0, s, a);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace mla
