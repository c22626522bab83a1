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
// Twelve waves in two roles, so that neither role's loads queue behind the
// other's (a wave's loads complete in issue order): waves 0-7 build A, four
// rows each, every step of a row inside the wave that owns it (row
// information with sixteen lanes per row, then the rows' partial outputs), so
// that a row costs two rounds of dependent loads: the plan entries, then the
// parts' lse together with all parts' outputs; waves 8-11 load their W_UV[h]
// operands straight into registers and own the MFMA, one 32-column block of v
// each.
namespace fu {
constexpr int FR = 32;                        // rows per workgroup
constexpr int FK = 512;                       // d_c
constexpr int FV = 128;                       // d_v (one 32-column block per MFMA wave)
constexpr int AW = 8;                         // A waves
constexpr int RPW = FR / AW;                  // rows per A wave (4)
constexpr int LPR = 64 / RPW;                 // lanes per row for the row information (16)
constexpr int FPW = 8;                        // parts per row loaded in one round (more: one at a time)
constexpr int NT = 64 * (AW + 4);             // 768 threads
constexpr int A_ROW = FK * 2;                 // 1 KiB per A row
constexpr int FSMEM = FR * A_ROW;             // the A tile (32 KiB), then the output staging

// A row r, 16-byte chunk c at chunk c ^ (r & 7) (MFMA operand reads of 32 rows spread over the banks)
__device__ __forceinline__ int a_off(int r, int c) { return r * A_ROW + ((c ^ (r & 7)) << 4); }
__device__ __forceinline__ int rdl(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float rdlf(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__global__ __launch_bounds__(NT, 1) void upv_merge_kernel(Plan pl, int H, const bf16* lat, const bf16* w_uv,
                                                          bf16* v, float* lse) {
  __shared__ __attribute__((aligned(1024))) char smem[FSMEM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = __builtin_amdgcn_readfirstlane(blockIdx.x % H);  // the division runs on the vector ALUs
  const int n0 = __builtin_amdgcn_readfirstlane((blockIdx.x / H) * FR);
  const int R = pl.R;
  const bool mw = wv >= AW;  // MFMA / W wave
  const int mwv = wv - AW;

  // The two roles run in separate branches, each with the same two barriers, so that the
  // W_UV operands and the partial outputs never hold registers at the same time.
  if (mw) {
    // W_UV[h] operands of 32 columns over the whole K extent straight to registers (32 loads
    // of 16 bytes per lane, all issued before anything waits), in the 32x32x16 B layout:
    // lane l holds column 32 mwv + l % 32, K 16 ks + 8 (l / 32) .. + 7
    bf16x8 bw[FK / 16];
    const bf16* wc = w_uv + ((size_t)h * FV + mwv * 32 + (lane & 31)) * FK + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < FK / 16; ++ks) bw[ks] = *(const bf16x8*)(wc + 16 * ks);
    // v^T block: columns 32 mwv .. 32 mwv + 31 of all 32 rows
    f32x16 acc = f32x16{};
    const int g = lane >> 5;
    __syncthreads();  // the A tile is complete
#pragma unroll
    for (int ks = 0; ks < FK / 16; ++ks) {
      const bf16x8 af = *(const MLA_LDS bf16x8*)(smem + a_off(lane & 31, 2 * ks + g));  // row, K chunk
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bw[ks], acc, 0, 0, 0);
    }
    __syncthreads();  // every MFMA wave is done with the A tile
    // stage the 32 x 128 block in the A tile (D layout: column lane % 32, rows
    // 8 (q / 4) + 4 g + q % 4)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 8 * (q >> 2) + 4 * g + (q & 3);
      *(MLA_LDS bf16*)(smem + row * 256 + (mwv * 32 + (lane & 31)) * 2) = f32_to_bf16(acc[q]);
    }
  } else {
    // row information: lanes 16 i .. 16 i + 15 describe row 4 wv + i
    const int ri = lane / LPR, k = lane % LPR, r = n0 + wv * RPW + ri;
    const int rc = r < R ? r : R - 1;  // rows past the batch read the last row's entries
    const int len = pl.len[rc], base = pl.cum[rc], n = pl.cum[rc + 1] - base, total = pl.cum[R], c = pl.split[1];
    asm volatile("" ::"v"(len), "v"(base), "v"(n), "s"(total), "s"(c));  // keeps the loads ahead of the branch on len
    int kind = 0, s0 = 0, w0 = 0, np = 0;
    if (r < R && len > 0) {
      const int per = plan_per_worker(total, pl.G);
      const int sf = base + c;
      w0 = sf / per;
      const int w1 = (base + n - 1) / per;
      kind = 1;
      if (w0 != w1) {
        kind = 2;
        np = w1 - w0 + 1;
        s0 = plan_slot(w0, sf, per);
      }
    }
    // the four rows' descriptions as wave-uniform values
    int rkind[RPW], rs0[RPW], rw0[RPW], rn[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      rkind[i] = rdl(kind, LPR * i);
      rs0[i] = rdl(s0, LPR * i);
      rw0[i] = rdl(w0, LPR * i);
      rn[i] = rkind[i] == 0 ? 0 : rkind[i] == 1 ? 1 : rdl(np, LPR * i);
    }
    const bf16* po = (const bf16*)pl.part_o;
    auto src = [&](int i, int j) -> const bf16* {
      if (rkind[i] == 1) return lat + ((size_t)(n0 + wv * RPW + i) * H + h) * FK;
      return po + ((size_t)(j == 0 ? rs0[i] : 2 * (rw0[i] + j)) * H + h) * FK;
    };
    // one round: this lane's part lse, then up to eight parts of every row, lane = 16-byte chunk
    // (a part that is not loaded is never read: the same wave-uniform test guards both, and
    // leaving it unset lets every load target its own register without a copy that would wait)
    float l_first = -INFINITY;
    if (k < np) l_first = pl.part_lse[(size_t)(k == 0 ? s0 : 2 * (w0 + k)) * H + h];
    bf16x8 pv[RPW][FPW];
#pragma unroll
    for (int j = 0; j < FPW; ++j)
#pragma unroll
      for (int i = 0; i < RPW; ++i)
        if (j < rn[i]) pv[i][j] = *(const bf16x8*)(src(i, j) + lane * 8);

    // merged lse of each cut row: lane k folds parts k, k + 16, ..., then the row's 16 lanes combine
    float mx = l_first, ws = l_first == -INFINITY ? 0.f : 1.f;
    for (int i = k + LPR; i < np; i += LPR) {
      const float l = pl.part_lse[(size_t)(2 * (w0 + i)) * H + h];
      if (l > mx) {
        ws = ws * __expf(mx - l) + 1.f;
        mx = l;
      } else if (l != -INFINITY) {
        ws += __expf(l - mx);
      }
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) {
      const float om = __shfl_xor(mx, off), ow = __shfl_xor(ws, off);
      const float m2 = fmaxf(mx, om);
      ws = (mx == -INFINITY ? 0.f : ws * __expf(mx - m2)) + (om == -INFINITY ? 0.f : ow * __expf(om - m2));
      mx = m2;
    }
    const float l_tot = (kind == 2 && ws > 0.f) ? mx + __logf(ws) : -INFINITY;
    const float wk = (l_first == -INFINITY || l_tot == -INFINITY) ? 0.f : __expf(l_first - l_tot);
    if (k == 0 && r < R && lse && kind != 1) lse[(size_t)r * H + h] = l_tot;  // empty rows -inf, cut rows merged

#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      float acc[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[x] = 0.f;
#pragma unroll
      for (int j = 0; j < FPW; ++j) {
        if (j < rn[i]) {
          const float w = rkind[i] == 1 ? 1.f : rdlf(wk, LPR * i + j);
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[x] += w * (float)pv[i][j][x];
        }
      }
      // parts beyond the first eight (rows cut over many workers): one at a time, the weights of
      // parts below sixteen from their lanes, the rest from their lse in HBM
      if (rn[i] > FPW) {
        const float lt = rdlf(l_tot, LPR * i);
        for (int j = FPW; j < rn[i]; ++j) {
          float w;
          if (j < LPR) {
            w = rdlf(wk, LPR * i + j);
          } else {
            const float l = pl.part_lse[(size_t)(2 * (rw0[i] + j)) * H + h];
            w = l == -INFINITY ? 0.f : __expf(l - lt);
          }
          const bf16x8 pj = *(const bf16x8*)(src(i, j) + lane * 8);
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[x] += w * (float)pj[x];
        }
      }
      bf16x8 o;
#pragma unroll
      for (int x = 0; x < 8; ++x) o[x] = f32_to_bf16(acc[x]);
      *(MLA_LDS bf16x8*)(smem + a_off(wv * RPW + i, lane)) = o;
    }
    __syncthreads();  // the A tile is complete
    __syncthreads();  // the MFMA waves are done with it
  }
  __syncthreads();  // the output block is staged
  // store whole 256-byte rows
  if (tid < FR * 16) {
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
  hipLaunchKernelGGL(fu::upv_merge_kernel, dim3(blocks), dim3(fu::NT), 0, stream, pl, H, (const bf16*)lat,
                     (const bf16*)w_uv, (bf16*)v, lse);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace mla
