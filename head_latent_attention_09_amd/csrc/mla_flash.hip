// Standard (per-head) softmax attention for gfx950, bf16 storage, fp32
// accumulation: the unabsorbed form of MLA prefill, where every head has its
// own keys [W_UK[h] c_t | k_pe_t] (the rope key shared by all heads) and
// values W_UV[h] c_t (MLA_tutorial formula.md Part 3, training form; the
// ferrox-core test's naive branch), and the gated variant's attention
// (tensortonic "Kimi K3 step 2: Gated MLA": softmax(Q K^T / sqrt(D_h) + M)
// with an optional causal mask, then the sigmoid channel gate). The tutorial
// notes that absorption widens the query/key head to d_c + d_r and the value
// to d_c, so for prefill, which is compute-bound, the expanded form does about
// 3.4x fewer operations per attended pair (640 against 2176 at DeepSeek-V2
// sizes).
//
// One workgroup = 4 waves = 128 queries of one (sequence, head); wave w owns
// queries 32w .. 32w+31. Keys stream in blocks of 64 through a two-stage LDS
// ring (direct global->LDS loads), shared by the four waves. Per block and
// wave:
//   scores S^T = K Q^T (keys as M, queries as N): 2 key halves x (d_k / 16)
//     k-steps of v_mfma_f32_32x32x16_bf16, Q resident in registers;
//   online softmax in registers: each lane holds 32 keys of one query (the
//     two lanes of a query combine with one cross-lane step);
//   values O^T += V^T P^T (dims as M, queries as N): the score accumulators
//     ARE the B operand of the value MFMA once rounded to bf16 -- the keys of
//     each 16-key k-step are taken in the order the score layout holds them,
//     and the V^T operand (transposing LDS reads) uses the same order, so the
//     weights never go through LDS.
#include "mla_internal.h"

#include <math.h>

#include <type_traits>

namespace mla {
namespace fa {

constexpr int QB = 128, KB = 64, DN = 128, DV = 128, NT = 256, NW = 4;
static_assert(NT == 64 * NW && QB == 32 * NW, "four waves of 32 queries each");
typedef short s16x8 __attribute__((ext_vector_type(8)));

template <int DR>
struct L {
  static constexpr int KN = 0;                   // key nope rows: 64 x 256 B
  static constexpr int KR = KB * DN * 2;         // key rope rows: 64 x 2*DR B
  static constexpr int VO = KR + KB * DR * 2;    // value rows: 64 x 256 B
  static constexpr int STAGE = VO + KB * DV * 2; // 40 KiB (DR = 64) or 32 KiB (DR = 0)
};

struct Args {
  const bf16* q;
  int64_t q_row, q_head;
  const bf16* qr;
  int64_t qr_row, qr_head;
  const bf16* k;
  int64_t k_row, k_head;
  const bf16* kr;
  int64_t kr_row;
  const bf16* v;
  int64_t v_row, v_head;
  bf16* o;
  int64_t o_row, o_head;
  float* lse;
  const bf16* gate;
  int64_t g_row, g_head;
  int B, S_q, S_kv, H, nqb;
  float scale_log2;
};

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global->LDS load of 64 lanes x 16 bytes (lane l: gbase + voff to LDS
// lds + 16 l). Issued from inline asm so the compiler does not wait for it
// before unrelated LDS reads; completion is waited for with vmcnt.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(gbase), "s"(lds) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const MLA_LDS char*)p; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// LDS swizzles (16-byte chunk index within a row):
//   key nope rows (256 B): chunk c of row r at c ^ (r & 15): the score
//     operand reads 16 consecutive rows at one chunk;
//   key rope rows (128 B): chunk c at c ^ ((r >> 1) & 7);
//   value rows (256 B): chunk c at c ^ (4 (r & 3)): a transposing read takes
//     4 consecutive rows x 2 chunks per 16 lanes.
__device__ __forceinline__ int swk(int r) { return r & 15; }
__device__ __forceinline__ int swr(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swv(int r) { return 4 * (r & 3); }

template <int DR, bool CAUSAL, bool GATE>
__global__ __launch_bounds__(NT, 2) void flash_kernel(Args a) {
  using Lay = L<DR>;
  constexpr int KS = (DN + DR) / 16;  // score k-steps
  __shared__ __attribute__((aligned(1024))) char smem[2 * Lay::STAGE];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;

  // Workgroup i runs on XCD i % 8. With many (sequence, head) pairs (a multiple of 8, at
  // least 16 per XCD), every query block of one pair goes to the same XCD and they are
  // dispatched back to back (heaviest first), so the blocks that stream that pair's keys and
  // values run together and share them through that XCD's L2 (measured 4.6 % faster at
  // B=2, H=128, S=4096). With few pairs (their keys and values fit the last-level cache
  // anyway) that order leaves XCDs unevenly loaded at the end (3 % slower at B=2, H=16):
  // heaviest query blocks first, (sequence, head) fastest.
  const int BH = a.B * a.H;
  const int id = blockIdx.x;
  int qb, bh;
  if (BH % 8 == 0 && BH >= 128) {
    const int xcd = id & 7, local = id >> 3;
    qb = a.nqb - 1 - local % a.nqb;
    bh = (local / a.nqb) * 8 + xcd;
  } else {
    qb = a.nqb - 1 - id / BH;
    bh = id % BH;
  }
  const int b = bh / a.H, h = bh - b * a.H;
  const int q0 = qb * QB;
  const int off = a.S_kv - a.S_q;  // query i sees keys t <= i + off (causal)
  const int qw0 = q0 + 32 * wv;    // this wave's first query
  const int qi = qw0 + l32;        // this lane's query
  const int64_t qrow = (int64_t)b * a.S_q + (qi < a.S_q ? qi : a.S_q - 1);

  int kend = a.S_kv;  // keys the workgroup needs
  if (CAUSAL) {
    const int qlast = min(q0 + QB, a.S_q) - 1;
    kend = min(kend, qlast + off + 1);
  }
  const int nblk = kend > 0 ? (kend + KB - 1) / KB : 0;
  // keys this wave needs (causal: up to its last query)
  int wend = a.S_kv;
  if (CAUSAL) wend = min(wend, min(qw0 + 31, a.S_q - 1) + off + 1);

  // ---- query fragments (B operand of the score MFMA: lane = query l32,
  // dims 16 ks + 8 g .. +7)
  bf16x8 qf[KS];
  {
    const bf16* qp = a.q + qrow * a.q_row + (int64_t)h * a.q_head + 8 * g;
#pragma unroll
    for (int ks = 0; ks < DN / 16; ++ks) qf[ks] = *(const bf16x8*)(qp + 16 * ks);
    if constexpr (DR > 0) {
      const bf16* qq = a.qr + qrow * a.qr_row + (int64_t)h * a.qr_head + 8 * g;
#pragma unroll
      for (int ks = 0; ks < DR / 16; ++ks) qf[DN / 16 + ks] = *(const bf16x8*)(qq + 16 * ks);
    }
  }

  // ---- block loads: per wave 4 key-nope, DR/32 key-rope and 4 value loads of 1 KiB
  const int64_t krow0 = (int64_t)b * a.S_kv;
  auto issue = [&](int kb, char* st) {
    const int k0 = kb * KB;
    const int last = a.S_kv - 1 - k0;  // rows past the end re-read the last key (weights are 0)
    const char* kbase = (const char*)(a.k + (krow0 + k0) * a.k_row + (int64_t)h * a.k_head);
    const char* vbase = (const char*)(a.v + (krow0 + k0) * a.v_row + (int64_t)h * a.v_head);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ld = wv * 4 + i;  // rows 4 ld .. 4 ld + 3
      int r = 4 * ld + (lane >> 4);
      const int c = (lane & 15) ^ swk(r);
      r = r < last ? r : last;
      dma16(kbase, (uint32_t)(r * a.k_row * 2 + c * 16), lds_addr(st + Lay::KN + ld * 1024));
    }
    if constexpr (DR > 0) {
      const char* rbase = (const char*)(a.kr + (krow0 + k0) * a.kr_row);
#pragma unroll
      for (int i = 0; i < DR / 32; ++i) {
        const int ld = wv * (DR / 32) + i;  // rows 8 ld .. 8 ld + 7 (128 B each)
        int r = 8 * ld + (lane >> 3);
        const int c = (lane & 7) ^ swr(r);
        r = r < last ? r : last;
        dma16(rbase, (uint32_t)(r * a.kr_row * 2 + c * 16), lds_addr(st + Lay::KR + ld * 1024));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ld = wv * 4 + i;
      int r = 4 * ld + (lane >> 4);
      const int c = (lane & 15) ^ swv(r);
      r = r < last ? r : last;
      dma16(vbase, (uint32_t)(r * a.v_row * 2 + c * 16), lds_addr(st + Lay::VO + ld * 1024));
    }
  };

  float m_run = -INFINITY;  // running max of this lane's query (log2 units), same in both lanes of a query
  float l_run = 0.f;        // this lane's part of the denominator (its 32 keys per block)
  f32x16 o[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) o[d] = f32x16{};

  // two stages, one barrier per block: the barrier that publishes block kb
  // also proves every wave is done with block kb - 1, whose stage then takes
  // block kb + 1 while block kb is used
  if (nblk > 0) issue(0, smem);
  for (int kb = 0; kb < nblk; ++kb) {
    wait_vmcnt<0>();
    barrier();  // block kb is in LDS for every wave; block kb - 1 is no longer read
    if (kb + 1 < nblk) issue(kb + 1, smem + ((kb + 1) & 1) * Lay::STAGE);
    const char* st = smem + (kb & 1) * Lay::STAGE;
    const int k0 = kb * KB;
    if (k0 < wend) {  // wave-uniform: the wave sees some key of this block
      // ---- scores S^T[key][query] for keys k0 .. k0 + 63
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = 32 * mb + l32;
        s[mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          bf16x8 kf;
          if (ks < DN / 16) {
            const int c = 2 * ks + g;
            kf = *(const MLA_LDS bf16x8*)(st + Lay::KN + row * 256 + ((c ^ swk(row)) << 4));
          } else {
            const int c = 2 * (ks - DN / 16) + g;
            kf = *(const MLA_LDS bf16x8*)(st + Lay::KR + row * (2 * DR) + ((c ^ swr(row)) << 4));
          }
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[mb], 0, 0, 0);
        }
      }
      // ---- online softmax. Lane holds key 32 mb + 8 (r / 4) + 4 g + r % 4 of
      // its query. The scores are never rewritten (a rewrite on some blocks
      // only makes the compiler copy all 32 of them on every block): a full
      // block (every key visible) with a positive scale takes the maximum of
      // the raw scores and scales it; other blocks take the maximum of the
      // scaled visible scores; the scale is folded into the exponent's
      // multiply-add, and on those blocks invisible keys get weight 0.
      const bool full = k0 + KB <= a.S_kv && (!CAUSAL || k0 + KB - 1 <= qw0 + off);
      const bool fast = full && a.scale_log2 > 0.f;  // wave-uniform
      const float sc = a.scale_log2;
      auto visible = [&](int mb, int r) {
        const int kk = k0 + 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
        return kk < a.S_kv && (!CAUSAL || kk <= qi + off);
      };
      float mx;
      if (fast) {
        float m0 = fmaxf(s[0][0], s[0][1]), m1 = fmaxf(s[1][0], s[1][1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) {
          m0 = fmaxf(m0, fmaxf(s[0][r], s[0][r + 1]));
          m1 = fmaxf(m1, fmaxf(s[1][r], s[1][r + 1]));
        }
        mx = fmaxf(m0, m1) * sc;
      } else {
        mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (visible(mb, r)) mx = fmaxf(mx, s[mb][r] * sc);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // The reference moves only when the maximum rises by more than 8 (log2
      // units): weights stay below 2^8, and the output is rescaled (64
      // multiplies per lane) only in the blocks where a reference moves.
      const float m_new = fmaxf(m_run, mx);
      const bool bump = m_new > m_run + 8.f;  // also true for the first visible block
      const float m_next = bump ? m_new : m_run;
      const float m_use = m_next == -INFINITY ? 0.f : m_next;
      const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
      m_run = m_next;
      bf16x8 pf[4];  // B operand of the value MFMA for key k-steps 0..3
      float psum = 0.f;
      // two copies of the weight loop, chosen once per block: without and with the mask
      auto weights = [&](auto mask_c) {
        constexpr bool MASK = decltype(mask_c)::value;
        const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            bf16x8 p8;
#pragma unroll
            for (int t = 0; t < 8; t += 2) {
              const int r0 = 8 * jj + t, r1 = r0 + 1;
              float w0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][r0], sc, -m_use));
              float w1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][r1], sc, -m_use));
              if (MASK) {
                w0 = visible(mb, r0) ? w0 : 0.f;
                w1 = visible(mb, r1) ? w1 : 0.f;
              }
              bf16x2 q2;
              q2[0] = f32_to_bf16(w0);
              q2[1] = f32_to_bf16(w1);
              p8[t] = q2[0];
              p8[t + 1] = q2[1];
              // the denominator sums exactly the rounded weights the MFMA uses
              psum = __builtin_amdgcn_fdot2_f32_bf16(q2, ones, psum, false);
            }
            pf[2 * mb + jj] = p8;
          }
      };
      if (fast) weights(std::false_type{});
      else weights(std::true_type{});
      l_run = l_run * alpha + psum;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int d = 0; d < DV / 32; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      }
      // ---- values: O^T[dim][query] += V^T P^T. k-step ks2 takes keys
      // 16 ks2 + 4 g + 0..3 (slots 0-3) and 16 ks2 + 8 + 4 g + 0..3 (slots 4-7).
      const int q16 = lane & 15, hf = (lane >> 4) & 1;
#pragma unroll
      for (int ks2 = 0; ks2 < 4; ++ks2) {
        const int ra = 16 * ks2 + 4 * g + (q16 >> 2), rb = ra + 8;
#pragma unroll
        for (int d = 0; d < DV / 32; ++d) {
          const int c = 4 * d + 2 * hf + ((q16 & 3) >> 1);
          const char* pa = st + Lay::VO + ra * 256 + ((c ^ swv(ra)) << 4) + (q16 & 1) * 8;
          const char* pb = st + Lay::VO + rb * 256 + ((c ^ swv(rb)) << 4) + (q16 & 1) * 8;
          const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)pa);
          const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)pb);
          const s16x8 v8 = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8), pf[ks2], o[d], 0, 0, 0);
        }
      }
    }
  }
  barrier();  // every wave is done with the last block before the stage buffers are reused

  // ---- epilogue: normalise, gate, stage through LDS, store whole rows
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (a.lse && g == 0 && qi < a.S_q)
    a.lse[((int64_t)b * a.S_q + qi) * a.H + h] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  // wave w stages its 32 queries x 128 dims (8 KiB) at w * 8 KiB; row q16 of
  // the stage: chunk c at c ^ (q & 15)
  // (the barrier after the loop ended every read of the stage buffers)
  char* sw = smem + wv * 8192;
#pragma unroll
  for (int d = 0; d < DV / 32; ++d)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      // dims 32 d + 8 rq + 4 g + 0..3: chunk 4 d + rq, bytes 8 g ..
      bf16x4 v4;
#pragma unroll
      for (int t = 0; t < 4; ++t) v4[t] = f32_to_bf16(o[d][4 * rq + t] * inv);
      const int c = 4 * d + rq;
      *(MLA_LDS bf16x4*)(sw + l32 * 256 + ((c ^ (l32 & 15)) << 4) + 8 * g) = v4;
    }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int idx = it * 64 + lane;
    const int qr = idx >> 4, c = idx & 15;
    const int qq = qw0 + qr;
    bf16x8 v = *(const MLA_LDS bf16x8*)(sw + qr * 256 + ((c ^ (qr & 15)) << 4));
    if (qq < a.S_q) {
      const int64_t row = (int64_t)b * a.S_q + qq;
      if constexpr (GATE) {
        const bf16x8 gv = *(const bf16x8*)(a.gate + row * a.g_row + (int64_t)h * a.g_head + 8 * c);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float gs = 1.0f / (1.0f + __expf(-(float)gv[t]));
          v[t] = f32_to_bf16((float)v[t] * gs);
        }
      }
      *(bf16x8*)(a.o + row * a.o_row + (int64_t)h * a.o_head + 8 * c) = v;
    }
  }
}
}  // namespace fa

// ===========================================================================
bool flash_fits(int d_nope, int d_r, int d_v) { return d_nope == fa::DN && d_v == fa::DV && (d_r == 0 || d_r == 64); }

int launch_flash(const FlashDesc& f, hipStream_t s) {
  if (f.B <= 0 || f.S_q <= 0 || f.H <= 0) return MLA_OK;
  fa::Args a;
  a.q = (const bf16*)f.q;
  a.q_row = f.q_row;
  a.q_head = f.q_head;
  a.qr = (const bf16*)f.qr;
  a.qr_row = f.qr_row;
  a.qr_head = f.qr_head;
  a.k = (const bf16*)f.k;
  a.k_row = f.k_row;
  a.k_head = f.k_head;
  a.kr = (const bf16*)f.kr;
  a.kr_row = f.kr_row;
  a.v = (const bf16*)f.v;
  a.v_row = f.v_row;
  a.v_head = f.v_head;
  a.o = (bf16*)f.o;
  a.o_row = f.o_row;
  a.o_head = f.o_head;
  a.lse = f.lse;
  a.gate = (const bf16*)f.gate;
  a.g_row = f.g_row;
  a.g_head = f.g_head;
  a.B = f.B;
  a.S_q = f.S_q;
  a.S_kv = f.S_kv;
  a.H = f.H;
  a.nqb = (f.S_q + fa::QB - 1) / fa::QB;
  a.scale_log2 = f.scale * kLog2e;
  const int64_t nwg = (int64_t)a.nqb * f.B * f.H;
  if (nwg > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)nwg), block(fa::NT);
#define MLA_FA(DR_, C_, G_) hipLaunchKernelGGL((fa::flash_kernel<DR_, C_, G_>), grid, block, 0, s, a)
  if (f.d_r == 64) {
    if (f.causal) { if (f.gate) MLA_FA(64, true, true); else MLA_FA(64, true, false); }
    else { if (f.gate) MLA_FA(64, false, true); else MLA_FA(64, false, false); }
  } else {
    if (f.causal) { if (f.gate) MLA_FA(0, true, true); else MLA_FA(0, true, false); }
    else { if (f.gate) MLA_FA(0, false, true); else MLA_FA(0, false, false); }
  }
#undef MLA_FA
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace mla
