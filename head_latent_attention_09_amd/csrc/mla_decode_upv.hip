// Decode: the merge of rows cut over several workers fused with the W_UV
// up-projection, for bf16 calls with d_c = 512 and d_v = 128.
//
// Method: the parts of a split row are merged by log-sum-exp (the result is
// the softmax-weighted sum over the whole row, up to rounding), then
// v[h] = W_UV[h] out_lat[h] (ferrox-core 0.23.0
// mla_absorbed.rs module documentation, the value up-projection after the
// latent attention; MLA_tutorial formula.md Part 3, inference form).
#include "mla_internal.h"

namespace mla {

// Workgroup (row block, head): A = the 32 rows' latent outputs of head h,
// built in LDS from the attention kernel's results -- a row one worker
// finished is read from `lat`, a cut row is merged from its
// partial outputs (the combine's merge), an empty row is zero -- then
// v[rows, h, :] = A W_UV[h]^T with 32x32x16 bf16 MFMA. Saves the combine
// kernel and the round trip of the merged rows through HBM.
//
// Eight waves in two roles, so that neither role's loads queue behind the
// other's (a wave's loads complete in issue order): waves 0-3 build A (row
// information with eight lanes per row, then the rows' partial outputs, two
// rows and up to eight parts each per batch of loads); waves 4-7 load their
// W_UV[h] operands straight into registers and own the MFMA, one 32-column
// block of v each.
namespace fu {
constexpr int FR = 32;                        // rows per workgroup
constexpr int FK = 512;                       // d_c
constexpr int FV = 128;                       // d_v (one 32-column block per MFMA wave)
constexpr int FPW = 8;                        // part weights kept per row (more parts: weights from HBM)
constexpr int A_ROW = FK * 2;                 // 1 KiB per A row
constexpr int FSMEM = FR * A_ROW;             // the A tile (32 KiB), then the output staging

// A row r, 16-byte chunk c at chunk c ^ (r & 7) (MFMA operand reads of 32 rows spread over the banks)
__device__ __forceinline__ int a_off(int r, int c) { return r * A_ROW + ((c ^ (r & 7)) << 4); }
__global__ __launch_bounds__(512, 1) void upv_merge_kernel(Plan pl, int H, const bf16* lat, const bf16* w_uv,
                                                           bf16* v, float* lse) {
  __shared__ __attribute__((aligned(1024))) char smem[FSMEM];
  __shared__ int rk[FR], rs0[FR], rw0[FR], rn[FR];  // row kind (0 empty, 1 read, 2 merge), its parts
  __shared__ float rl[FR], rwt[FR][FPW];             // merged lse of a cut row, its parts' weights
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = __builtin_amdgcn_readfirstlane(blockIdx.x % H);  // the division runs on the vector ALUs
  const int n0 = __builtin_amdgcn_readfirstlane((blockIdx.x / H) * FR);
  const int R = pl.R;
  const bool mw = wv >= 4;  // MFMA / W wave
  const int mwv = wv - 4;

  // MFMA waves: the W_UV[h] operands of their 32 columns over the whole K extent go straight
  // to registers (32 loads of 16 bytes per lane, all issued before anything waits), in the
  // 32x32x16 B layout: lane l holds column 32 mwv + l % 32, K 16 ks + 8 (l / 32) .. + 7
  bf16x8 bw[FK / 16];
  if (mw) {
    const bf16* wc = w_uv + ((size_t)h * FV + mwv * 32 + (lane & 31)) * FK + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < FK / 16; ++ks) bw[ks] = *(const bf16x8*)(wc + 16 * ks);
  } else {
    // row information: eight lanes per row, lane k reads the lse of parts k, k + 8, ...
    const int row = tid >> 3, k = tid & 7, r = n0 + row;
    int kind = 0, s0 = 0, w0 = 0, np = 0;
    float mx = -INFINITY, ws = 0.f, l_first = -INFINITY;
    // every plan entry in one round of loads (rows past the batch read the last row's)
    const int rc = r < R ? r : R - 1;
    const int len = pl.len[rc], base = pl.cum[rc], n = pl.cum[rc + 1] - base, total = pl.cum[R], c = pl.split[1];
    asm volatile("" ::"v"(len), "v"(base), "v"(n), "s"(total), "s"(c));  // keeps the loads ahead of the branch on len
    if (r < R && len > 0) {
      const int per = plan_per_worker(total, pl.G);
      const int sf = base + c;
      w0 = sf / per;
      const int w1 = (base + n - 1) / per;
      kind = 1;
      if (w0 != w1) {
        np = w1 - w0 + 1;
        s0 = plan_slot(w0, sf, per);
        for (int i = k; i < np; i += FPW) {
          const float l = pl.part_lse[(size_t)(i == 0 ? s0 : 2 * (w0 + i)) * H + h];
          if (i == k) l_first = l;
          if (l > mx) {
            ws = ws * __expf(mx - l) + 1.f;
            mx = l;
          } else if (l != -INFINITY) {
            ws += __expf(l - mx);
          }
        }
      }
    }
#pragma unroll
    for (int off = 1; off < FPW; off <<= 1) {
      const float om = __shfl_xor(mx, off), ow = __shfl_xor(ws, off);
      const float m2 = fmaxf(mx, om);
      ws = (mx == -INFINITY ? 0.f : ws * __expf(mx - m2)) + (om == -INFINITY ? 0.f : ow * __expf(om - m2));
      mx = m2;
    }
    float l_tot = -INFINITY;
    if (kind == 1 && np > 0) {
      kind = 2;
      l_tot = ws > 0.f ? mx + __logf(ws) : -INFINITY;
    }
    if (k < np) rwt[row][k] = (l_first == -INFINITY || l_tot == -INFINITY) ? 0.f : __expf(l_first - l_tot);
    if (k == 0) {
      rk[row] = kind;
      rs0[row] = s0;
      rw0[row] = w0;
      rn[row] = np;
      rl[row] = l_tot;
      if (r < R && lse && kind != 1) lse[(size_t)r * H + h] = l_tot;  // empty rows -inf, cut rows merged
    }
  }
  __syncthreads();

  if (!mw) {
    // A tile: wave wv builds rows 8 wv .. 8 wv + 7, lane = 16-byte chunk. Per batch of two
    // rows: their plan entries into scalar registers first, then the loads of up to eight
    // sources per row back to back (into zeroed registers, so that no skipped load leaves a
    // register the compiler could reuse while another load is in flight), then the sums.
    const bf16* po = (const bf16*)pl.part_o;
    constexpr int RB = 2;
#pragma unroll
    for (int rr = 0; rr < 8; rr += RB) {
      int kind[RB], s0[RB], w0[RB], n[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int row = wv * 8 + rr + i;
        kind[i] = __builtin_amdgcn_readfirstlane(rk[row]);
        s0[i] = __builtin_amdgcn_readfirstlane(rs0[row]);
        w0[i] = __builtin_amdgcn_readfirstlane(rw0[row]);
        n[i] = kind[i] == 0 ? 0 : kind[i] == 1 ? 1 : __builtin_amdgcn_readfirstlane(rn[row]);
      }
      auto src = [&](int i, int j) -> const bf16* {
        if (kind[i] == 1) return lat + ((size_t)(n0 + wv * 8 + rr + i) * H + h) * FK;
        return po + ((size_t)(j == 0 ? s0[i] : 2 * (w0[i] + j)) * H + h) * FK;
      };
      bf16x8 pv[RB][FPW];
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < FPW; ++j)
#pragma unroll
          for (int x = 0; x < 8; ++x) pv[i][j][x] = (bf16)0.f;
#pragma unroll
      for (int j = 0; j < FPW; ++j)
#pragma unroll
        for (int i = 0; i < RB; ++i)
          if (j < n[i]) pv[i][j] = *(const bf16x8*)(src(i, j) + lane * 8);
      float acc[RB][8];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int row = wv * 8 + rr + i;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[i][x] = 0.f;
#pragma unroll
        for (int j = 0; j < FPW; ++j) {
          const float w = j >= n[i] ? 0.f : kind[i] == 1 ? 1.f : rwt[row][j];
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[i][x] += w * (float)pv[i][j][x];
        }
        // parts beyond the first eight (rows cut over many workers): one at a time,
        // weights from their lse in HBM
        for (int j = FPW; j < n[i]; ++j) {
          const float l = pl.part_lse[(size_t)(2 * (w0[i] + j)) * H + h];
          const float w = l == -INFINITY ? 0.f : __expf(l - rl[row]);
          const bf16x8 v = *(const bf16x8*)(src(i, j) + lane * 8);
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[i][x] += w * (float)v[x];
        }
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        bf16x8 o;
#pragma unroll
        for (int x = 0; x < 8; ++x) o[x] = f32_to_bf16(acc[i][x]);
        *(MLA_LDS bf16x8*)(smem + a_off(wv * 8 + rr + i, lane)) = o;
      }
    }
  }

  // v^T block: MFMA wave mwv owns columns 32 mwv .. 32 mwv + 31 of all 32 rows
  f32x16 acc = f32x16{};
  const int g = lane >> 5;
  __syncthreads();  // the A tile is complete
  if (mw) {
#pragma unroll
    for (int ks = 0; ks < FK / 16; ++ks) {
      const bf16x8 af = *(const MLA_LDS bf16x8*)(smem + a_off(lane & 31, 2 * ks + g));  // row, K chunk
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bw[ks], acc, 0, 0, 0);
    }
  }
  __syncthreads();  // every MFMA wave is done with the A tile

  // output: stage the 32 x 128 block in the A tile, store whole 256-byte rows
  // (D layout: column lane % 32, rows 8 (q / 4) + 4 g + q % 4)
  if (mw) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 8 * (q >> 2) + 4 * g + (q & 3);
      *(MLA_LDS bf16*)(smem + row * 256 + (mwv * 32 + (lane & 31)) * 2) = f32_to_bf16(acc[q]);
    }
  }
  __syncthreads();
  {
    const int row = tid >> 4, c = tid & 15;
    const int r = n0 + row;
    if (r < R) *(bf16x8*)(v + ((size_t)r * H + h) * FV + c * 8) = *(const MLA_LDS bf16x8*)(smem + row * 256 + c * 16);
  }
}
}  // namespace fu

bool upv_merge_fits(int d_c, int d_v, const void* w_uv, const void* v) {
  return d_c == fu::FK && d_v == fu::FV && ((uintptr_t)w_uv & 15) == 0 && ((uintptr_t)v & 15) == 0;
}

int launch_upv_merge(const Plan& pl, int R, int H, const void* lat, const void* w_uv, void* v, float* lse,
                     hipStream_t stream) {
  const unsigned blocks = (unsigned)(((int64_t)R + fu::FR - 1) / fu::FR * H);
  hipLaunchKernelGGL(fu::upv_merge_kernel, dim3(blocks), dim3(512), 0, stream, pl, H, (const bf16*)lat,
                     (const bf16*)w_uv, (bf16*)v, lse);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace mla
