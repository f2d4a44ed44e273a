// fa_fwd.hip - forward pass of exact attention, bf16 tensors, fp32 arithmetic (gfx950).
//
// One workgroup per (sequence, head, query tile), so one head is spread over many
// compute units ("FlashAttention-2 (PT)", "2. Paralelismo aprimorado"). Four waves;
// each wave owns QB blocks of 32 query rows whose Q fragments stay in registers for
// the whole kernel. Key/value tiles of 64 rows are staged through LDS ("Tiling" in the
// AI Atlas summary; "Aperçu technique" on aiunderstanding.org) and each wave computes
//     S^T = K Q^T          (v_mfma_f32_32x32x16_bf16, fp32 accumulators)
//     online softmax        (running max m and sum l per query row, "Softmax en línea")
//     O^T += V^T P^T        (P converted to bf16 straight from the S^T registers)
// Computing S transposed puts one query per MFMA output column, so each query's
// softmax state sits in one lane and its mirror lane: a row reduction is in-register
// work plus one lane swap, with no LDS round trip ("3. Divisão de trabalho otimizada
// dentro do bloco"). Non-matmul work is kept small ("1. Minimização de operações não
// matriciais"): the scale is folded into the exponent, c = scale * log2(e); the
// division by l happens once at the end; and the output is rescaled only when some
// row's running maximum has grown by more than 2^8 since the last rescale (until then
// the stale maximum keeps every exponent <= 2^8, so nothing overflows and O and l keep
// one common reference, which is all exactness needs).
//
// Data movement: K and V tiles are copied row-major into LDS by the global->LDS DMA
// path (global_load_lds_dwordx4: no registers, no LDS write instructions); the copy of
// the next tile runs while the current one is used, in the other of two LDS buffers,
// so each tile costs one barrier. K rows feed the A operand of S^T directly; V^T is
// read with ds_read_b64_tr_b16, which transposes 16 x 4 blocks on the way out of LDS.
// Row pitches are padded so both read patterns hit distinct LDS banks.
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
constexpr int kFwdBC = 64;        // keys per tile
constexpr float kRescaleTau = 8.f;  // log2 growth of the row max tolerated before rescaling

template <int D>
struct FwdLds {
  static constexpr int KP = pitch_rows<D>();  // K: read row-wise (A operand of S^T)
  static constexpr int VP = pitch_tr<D>();    // V: read with transpose reads (A of O^T)
  static constexpr int KSZ = kFwdBC * KP;
  static constexpr int VSZ = kFwdBC * VP;
  static constexpr int BUF = KSZ + VSZ;
};

template <int D, int QB>
struct FwdState {
  static constexpr int NB = D / 32;
  bf16x8 qf[QB][D / 16];
  f32x16 oacc[QB][NB];
  float m_run[QB];  // reference maximum of the raw scores q.k of this lane's query
  float l_run[QB];  // this lane's share of sum_j exp2(c * (s_j - m_run))
};

// One key tile for one wave: S^T, softmax update, O^T += V^T P^T.
template <int D, int QB, bool CAUSAL>
__device__ __forceinline__ void fwd_tile(FwdState<D, QB>& st, const u16* Ks, const u16* Vs, int k0, int len,
                                         int wq0, int lane, float c, bool mask) {
  constexpr int NS = D / 16, NJ = kFwdBC / 32, NTK = kFwdBC / 16, NB = D / 32;
  constexpr int KP = FwdLds<D>::KP, VP = FwdLds<D>::VP;
  const int lr = lane & 31, g = lane >> 5;

  f32x16 sacc[QB][NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int n = 0; n < QB; ++n) sacc[n][j] = f32x16{};
    const u16* arow = Ks + (32 * j + lr) * KP + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 a = ld16(arow + 16 * s);
#pragma unroll
      for (int n = 0; n < QB; ++n) sacc[n][j] = mfma32(a, st.qf[n][s], sacc[n][j]);
    }
  }

  bf16x8 pb[QB][NTK];
#pragma unroll
  for (int n = 0; n < QB; ++n) {
    const int qi = wq0 + 32 * n + lr;
    if (mask) {  // wave-uniform: a diagonal or tail tile
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * j + crow_nat(r, g);
          const bool hide = key >= len || (CAUSAL && key > qi);
          sacc[n][j][r] = hide ? -INFINITY : sacc[n][j][r];
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[n][j][r]);
    mx = pair_max(mx);
    const float m_new = fmaxf(st.m_run[n], mx);
    // Rescale when this row's maximum grew by more than 2^tau (always on the first
    // visible tile, where m_run is -inf); the decision is taken for the whole wave.
    const bool grow = (m_new - st.m_run[n]) * c > kRescaleTau;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_to = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2((st.m_run[n] - m_to) * c);
      st.m_run[n] = m_new;
      st.l_run[n] *= alpha;
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) st.oacc[n][bb] *= alpha;
    }
    const float nb = st.m_run[n] == -INFINITY ? 0.f : -st.m_run[n] * c;
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(sacc[n][j][r], c, nb));
        sacc[n][j][r] = e;
        ls += e;
      }
    }
    st.l_run[n] += ls;
#pragma unroll
    for (int t = 0; t < NTK; ++t) pb[n][t] = to_bf16x8(half_of(sacc[n][t >> 1], t & 1));
  }

  // O^T += V^T P^T: A row m of block bb is head-dim entry 32bb + m; the k-slots of lane
  // group g at step t are keys 16t + 4g + {0..3, 8..11}, matching the P registers.
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
    for (int t = 0; t < NTK; ++t) {
      const bf16x8 a = lds_tr_operand(Vs, VP, 16 * t, 32 * bb, lane);
#pragma unroll
      for (int n = 0; n < QB; ++n) st.oacc[n][bb] = mfma32(a, pb[n][t], st.oacc[n][bb]);
    }
  }
}

// Two query blocks per wave need the whole register file (one workgroup per compute
// unit); so does the non-causal head_dim 128 variant, which spills at two.
template <int D, bool CAUSAL, bool VARLEN, int QB>
__global__ __launch_bounds__(kFwdThreads, (QB == 1 && (CAUSAL || D == 64)) ? 2 : 1) void fwd_bf16_kernel(FwdParams p) {
  constexpr int BR = 32 * QB * kFwdWaves, BC = kFwdBC, NT = kFwdThreads;
  constexpr int NB = D / 32, NS = D / 16;
  using L = FwdLds<D>;
  __shared__ __attribute__((aligned(16))) u16 buf0[L::BUF];
  __shared__ __attribute__((aligned(16))) u16 buf1[L::BUF];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;

  // Workgroup -> (sequence, head, query tile), tile-major; causal tiles near the end of
  // a sequence have the most keys to visit, so they are issued first.
  int bh, qt;
  xcd_tile_map(blockIdx.x, p.B * p.H, p.n_qtiles, CAUSAL, false, bh, qt);
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

  const int wq0 = q0 + 32 * QB * w;  // first query row of this wave
  const int wq_last = min(wq0 + 32 * QB - 1, len - 1);

  FwdState<D, QB> st;
#pragma unroll
  for (int n = 0; n < QB; ++n) {
    const int qi = wq0 + 32 * n + lr;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      st.qf[n][s] = qi < len ? ld16(Qg + (size_t)qi * stride + 16 * s + 8 * g) : zero_bf16x8();
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) st.oacc[n][bb] = f32x16{};
    st.m_run[n] = -INFINITY;
    st.l_run[n] = 0.f;
  }

  const int kv_end = CAUSAL ? min(q0 + BR, len) : len;
  const int n_kt = (kv_end + BC - 1) / BC;

  TileDma<BC, D, L::KP, kFwdWaves> kdma;
  TileDma<BC, D, L::VP, kFwdWaves> vdma;
  kdma.init(stride, w, lane);
  vdma.init(stride, w, lane);
  auto issue = [&](int kt, u16* buf) {
    kdma.issue(buf, Kg, kt * BC, len, stride, w, lane);
    vdma.issue(buf + L::KSZ, Vg, kt * BC, len, stride, w, lane);
  };
  auto compute = [&](int kt, const u16* buf) {
    const int k0 = kt * BC;
    // wave-uniform: skip tiles that are entirely masked for this wave
    if (wq0 < len && (!CAUSAL || k0 <= wq_last)) {
      const bool mask = k0 + BC > len || (CAUSAL && k0 + BC - 1 > wq0);
      fwd_tile<D, QB, CAUSAL>(st, buf, buf + L::KSZ, k0, len, wq0, lane, p.c, mask);
    }
  };
  // Two LDS buffers in turn: the copy of tile kt+1 is in flight while tile kt is used.
  issue(0, buf0);
  wait_vmem();
  __syncthreads();
  for (int kt = 0; kt < n_kt; kt += 2) {
    if (kt + 1 < n_kt) issue(kt + 1, buf1);
    compute(kt, buf0);
    wait_vmem();
    __syncthreads();
    if (kt + 1 >= n_kt) break;
    if (kt + 2 < n_kt) issue(kt + 2, buf0);
    compute(kt + 1, buf1);
    wait_vmem();
    __syncthreads();
  }

#pragma unroll
  for (int n = 0; n < QB; ++n) {
    const int qi = wq0 + 32 * n + lr;
    const float l_tot = pair_sum(st.l_run[n]);
    if (qi >= len) continue;
    const float inv = 1.f / l_tot;
    u16* __restrict__ Og = p.o + base + (size_t)qi * stride;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      // lane group g holds head-dim entries 32bb + 8a + 4g + {0..3} in registers 4a..4a+3
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float x0 = st.oacc[n][bb][4 * a] * inv, x1 = st.oacc[n][bb][4 * a + 1] * inv;
        const float x2 = st.oacc[n][bb][4 * a + 2] * inv, x3 = st.oacc[n][bb][4 * a + 3] * inv;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        typedef float f32x4_ __attribute__((ext_vector_type(4)));
        *reinterpret_cast<bf16x4*>(Og + 32 * bb + 8 * a + 4 * g) =
            __builtin_convertvector(f32x4_{x0, x1, x2, x3}, bf16x4);
      }
    }
    if (g == 0) {
      const size_t li = VARLEN ? (size_t)h * p.T + start + qi : ((size_t)b * p.H + h) * p.N + qi;
      p.lse[li] = st.m_run[n] * p.scale + logf(l_tot);
    }
  }
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_fwd_t(const Problem& pr) {
  // Two query blocks per wave halve the LDS reads per MFMA; at head_dim 128 their
  // accumulators no longer fit the register file, so one block is used there.
  constexpr int QB = D == 64 ? 2 : 1;
  constexpr int BR = 32 * QB * kFwdWaves;
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
  p.n_qtiles = (pr.seqlen + BR - 1) / BR;
  p.scale = pr.scale;
  p.c = pr.scale * kLog2e;
  const dim3 grid((unsigned)(p.n_qtiles * pr.batch * pr.heads));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, VARLEN, QB>), grid, dim3(kFwdThreads), 0, pr.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const Problem& p) { FA_DISPATCH(launch_fwd_t, p); }

}  // namespace fa
