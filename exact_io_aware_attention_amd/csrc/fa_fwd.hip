// fa_fwd.hip - forward pass of exact attention, bf16 tensors, fp32 arithmetic (gfx950).
//
// One workgroup per (sequence, head, 128-query tile), so one head is spread over many
// compute units ("FlashAttention-2 (PT)", "2. Paralelismo aprimorado"). Four waves; each
// wave owns 32 query rows whose Q fragments stay in registers for the whole kernel.
// Key/value tiles of 64 rows are staged through LDS ("Tiling" in the AI Atlas summary;
// "Aperçu technique" on aiunderstanding.org) and each wave computes
//     S^T = K Q^T          (v_mfma_f32_32x32x16_bf16, fp32 accumulators)
//     online softmax        (running max m and sum l per query row, "Softmax en línea")
//     O^T += V^T P^T        (P converted to bf16 straight from the S^T registers)
// Computing S transposed puts one query per MFMA output column, so each query's
// softmax state sits in one lane and its mirror lane: a row reduction is in-register
// work plus one lane swap, with no LDS round trip ("3. Divisão de trabalho otimizada
// dentro do bloco"). The scale is folded into the exponent, c = scale * log2(e), and
// the division by l happens once at the end ("1. Minimização de operações não
// matriciais"). Only O and the logsumexp ever reach HBM.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

struct FwdParams {
  const u16* q;
  const u16* k;
  const u16* v;
  u16* o;
  float* lse;
  const int32_t* cu;
  int B, H, N, T;
  int n_qtiles;
  float scale;
  float c;  // scale * log2(e)
};

constexpr int kFwdWaves = 4;
constexpr int kFwdThreads = 64 * kFwdWaves;
constexpr int kFwdBR = 32 * kFwdWaves;  // queries per workgroup
constexpr int kFwdBC = 64;              // keys per tile
constexpr int kPadK = 8;                // bf16 padding per LDS row of K
constexpr int kPadV = 8;                // bf16 padding per LDS row of V^T

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_bf16_kernel(FwdParams p) {
  constexpr int BR = kFwdBR, BC = kFwdBC, NT = kFwdThreads;
  constexpr int NB = D / 32;    // 32-wide head-dim blocks of O^T
  constexpr int NS = D / 16;    // MFMA k-steps over the head dim
  constexpr int NJ = BC / 32;   // 32-key blocks of S^T per tile
  constexpr int NTK = BC / 16;  // MFMA k-steps over the keys of a tile
  constexpr int KPITCH = D + kPadK;
  constexpr int VPITCH = BC + kPadV;

  __shared__ __attribute__((aligned(16))) u16 Ks[BC * KPITCH];
  __shared__ __attribute__((aligned(16))) u16 Vt[D * VPITCH];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;

  // Workgroup -> (sequence, head, query tile). Causal tiles near the end of a sequence
  // have the most keys to visit, so they are issued first.
  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH;
  int qt = blockIdx.x / BH;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;
  const int b = bh / p.H, h = bh % p.H;
  int start, len;
  if (VARLEN) {
    start = p.cu[b];
    len = p.cu[b + 1] - start;
  } else {
    start = b * p.N;
    len = p.N;
  }
  const int q0 = qt * BR;
  if (q0 >= len) return;

  const size_t stride = (size_t)p.H * D;
  const size_t base = ((size_t)start * p.H + h) * D;
  const u16* __restrict__ Qg = p.q + base;
  const u16* __restrict__ Kg = p.k + base;
  const u16* __restrict__ Vg = p.v + base;

  const int wq0 = q0 + 32 * w;  // first query row of this wave
  const int qi = wq0 + lr;      // this lane's query row
  const int wq_last = min(wq0 + 31, len - 1);

  bf16x8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    qf[s] = qi < len ? ld16(Qg + (size_t)qi * stride + 16 * s + 8 * g) : zero_bf16x8();

  const int kv_end = CAUSAL ? min(q0 + BR, len) : len;
  const int n_kt = (kv_end + BC - 1) / BC;

  float m_run = -INFINITY;  // running max of raw scores q.k for this query row
  float l_run = 0.f;        // this lane's share of the running sum
  f32x16 oacc[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) oacc[bb] = f32x16{};

  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * BC;
    if (kt > 0) __syncthreads();  // every wave is done reading the previous tile
    stage_rows<BC, D, kPadK, NT>(Ks, Kg, k0, len, stride, tid);
    stage_transposed<BC, D, kPadV, NT>(Vt, Vg, k0, len, stride, tid);
    __syncthreads();

    const bool active = wq0 < len && (!CAUSAL || k0 <= wq_last);
    if (!active) continue;  // wave-uniform: this tile is entirely masked for the wave

    // S^T = K Q^T for the 64 keys of the tile: register r of block j (lane group g)
    // holds key k0 + 32j + crow_of_reg(r, g) against query qi.
    f32x16 sacc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      sacc[j] = f32x16{};
      const u16* arow = Ks + (32 * j + perm_rows(lr)) * KPITCH + 8 * g;
#pragma unroll
      for (int s = 0; s < NS; ++s) sacc[j] = mfma32(ld16(arow + 16 * s), qf[s], sacc[j]);
    }

    const bool need_mask = (k0 + BC > len) || (CAUSAL && k0 + BC - 1 > wq0);
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (need_mask) {
          const int key = k0 + 32 * j + crow_of_reg(r, g);
          if (key >= len || (CAUSAL && key > qi)) sacc[j][r] = -INFINITY;
        }
        mx = fmaxf(mx, sacc[j][r]);
      }
    }
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // row with no visible key yet
    const float alpha = fast_exp2((m_run - m_use) * p.c);
    const float nb = -m_use * p.c;
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(sacc[j][r], p.c, nb));
        sacc[j][r] = e;
        ls += e;
      }
    }
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) oacc[bb] *= alpha;

    bf16x8 pb[NTK];
#pragma unroll
    for (int t = 0; t < NTK; ++t) pb[t] = to_bf16x8(half_of(sacc[t >> 1], t & 1));

    // O^T += V^T P^T: A row m of block bb is head-dim entry 32*bb + perm_cols(m); the
    // 8 k-slots of lane group g at step t are keys 16t + 8g .. 16t + 8g + 7.
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const u16* arow = Vt + (32 * bb + perm_cols(lr)) * VPITCH + 8 * g;
#pragma unroll
      for (int t = 0; t < NTK; ++t) oacc[bb] = mfma32(ld16(arow + 16 * t), pb[t], oacc[bb]);
    }
  }

  if (qi >= len) return;
  const float l_tot = pair_sum(l_run);
  const float inv = 1.f / l_tot;
  u16* __restrict__ Og = p.o + base + (size_t)qi * stride;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    // lane group g holds head-dim entries 32bb + 16g + r, r = 0..15
    const bf16x8 lo = to_bf16x8(half_of(oacc[bb], 0) * inv);
    const bf16x8 hi = to_bf16x8(half_of(oacc[bb], 1) * inv);
    *reinterpret_cast<bf16x8*>(Og + 32 * bb + 16 * g) = lo;
    *reinterpret_cast<bf16x8*>(Og + 32 * bb + 16 * g + 8) = hi;
  }
  if (g == 0) {
    const size_t li = VARLEN ? (size_t)h * p.T + start + qi : ((size_t)b * p.H + h) * p.N + qi;
    p.lse[li] = m_run * p.scale + logf(l_tot);
  }
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_fwd_t(const Problem& pr) {
  FwdParams p;
  p.q = static_cast<const u16*>(pr.q);
  p.k = static_cast<const u16*>(pr.k);
  p.v = static_cast<const u16*>(pr.v);
  p.o = static_cast<u16*>(pr.o_out);
  p.lse = pr.lse_out;
  p.cu = pr.cu_seqlens;
  p.B = pr.batch;
  p.H = pr.heads;
  p.N = pr.seqlen;
  p.T = pr.total_tokens;
  p.n_qtiles = (pr.seqlen + kFwdBR - 1) / kFwdBR;
  p.scale = pr.scale;
  p.c = pr.scale * kLog2e;
  const dim3 grid((unsigned)(p.n_qtiles * pr.batch * pr.heads));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, VARLEN>), grid, dim3(kFwdThreads), 0, pr.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const Problem& p) { FA_DISPATCH(launch_fwd_t, p); }

}  // namespace fa
