// fa_fp32.hip - exact attention with fp32 tensors and fp32 arithmetic throughout.
//
// The same tiled algorithm as the bf16 path (tiles staged through LDS, running row
// max and sum with rescaling, "Softmax en línea"; P recomputed from the logsumexp in
// the backward pass, "Recalcular en vez de guardar"), but every product is an fp32
// fused multiply-add on the vector ALUs: no reduced-precision operands anywhere.
// Two lanes share one row (query or key), each holding half of the head dimension, so
// the per-row accumulators fit in registers; partial dot products meet with one lane
// exchange. Workgroups: 2 waves, 64 rows.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kF32Threads = 128;
constexpr int kF32Rows = 64;   // rows (queries or keys) per workgroup
constexpr int kF32Tile = 16;   // rows of the streamed tile

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  const float* dout;
  const float* lse;
  const float* dvec;
  float* o;
  float* lse_out;
  float* dq;
  float* dk;
  float* dv;
  const int32_t* cu;
  int B, H, N, T;
  int n_tiles;
  float scale, c;
};

template <bool VARLEN>
__device__ __forceinline__ void seq_range(const F32Params& p, int b, int& start, int& len) {
  if (VARLEN) {
    start = p.cu[b];
    len = p.cu[b + 1] - start;
  } else {
    start = b * p.N;
    len = p.N;
  }
}

template <bool VARLEN>
__device__ __forceinline__ size_t stat_idx(const F32Params& p, int b, int h, int start, int n) {
  return VARLEN ? (size_t)h * p.T + start + n : ((size_t)b * p.H + h) * p.N + n;
}

// Copy rows [r0, r0 + ROWS) x D of a strided matrix into dst[ROWS][PITCH]; rows past
// `len` become zero.
template <int ROWS, int D, int PITCH>
__device__ __forceinline__ void stage_f32(float* dst, const float* __restrict__ src, int r0, int len,
                                          size_t stride, int tid) {
  for (int c = tid; c < ROWS * D; c += kF32Threads) {
    const int row = c / D, col = c % D;
    dst[row * PITCH + col] = r0 + row < len ? src[(size_t)(r0 + row) * stride + col] : 0.f;
  }
}

__device__ __forceinline__ float pair_reduce(float x) { return x + __shfl_xor(x, 1); }

// ---------------------------------------------------------------------------- forward

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kF32Threads) void fwd_fp32_kernel(F32Params p) {
  constexpr int HD = D / 2, BC = kF32Tile, QP = D + 1;
  __shared__ float Qs[kF32Rows * QP];
  __shared__ float Ks[BC * D];
  __shared__ float Vs[BC * D];

  const int tid = threadIdx.x, row = tid >> 1, half = tid & 1;
  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH;
  int qt = blockIdx.x / BH;
  if (CAUSAL) qt = p.n_tiles - 1 - qt;
  const int b = bh / p.H, h = bh % p.H;
  int start, len;
  seq_range<VARLEN>(p, b, start, len);
  const int q0 = qt * kF32Rows;
  if (q0 >= len) return;
  const size_t stride = (size_t)p.H * D, base = ((size_t)start * p.H + h) * D;
  const int qi = q0 + row;

  stage_f32<kF32Rows, D, QP>(Qs, p.q + base, q0, len, stride, tid);
  float acc[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) acc[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int kv_end = CAUSAL ? min(q0 + kF32Rows, len) : len;

  for (int k0 = 0; k0 < kv_end; k0 += BC) {
    __syncthreads();
    stage_f32<BC, D, D>(Ks, p.k + base, k0, len, stride, tid);
    stage_f32<BC, D, D>(Vs, p.v + base, k0, len, stride, tid);
    __syncthreads();
    float s[BC];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) part = fmaf(Qs[row * QP + half * HD + d], Ks[j * D + half * HD + d], part);
      float sj = pair_reduce(part);
      const int key = k0 + j;
      if (key >= len || (CAUSAL && key > qi)) sj = -INFINITY;
      s[j] = sj;
      mx = fmaxf(mx, sj);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f((m_run - m_use) * p.c);
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      s[j] = exp2f(s[j] * p.c - m_use * p.c);
      ls += s[j];
    }
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < HD; ++d) {
      float a = acc[d] * alpha;
#pragma unroll
      for (int j = 0; j < BC; ++j) a = fmaf(s[j], Vs[j * D + half * HD + d], a);
      acc[d] = a;
    }
  }
  if (qi >= len) return;
  float* __restrict__ og = p.o + base + (size_t)qi * stride + half * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) og[d] = acc[d] / l_run;
  if (half == 0) p.lse_out[stat_idx<VARLEN>(p, b, h, start, qi)] = m_run * p.scale + logf(l_run);
}

// ---------------------------------------------------------------------------- dK, dV

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kF32Threads) void dkdv_fp32_kernel(F32Params p) {
  constexpr int HD = D / 2, BQ = kF32Tile, KP = D + 1;
  __shared__ float Ks[kF32Rows * KP];
  __shared__ float Vs[kF32Rows * KP];
  __shared__ float Qt[BQ * D];
  __shared__ float dOt[BQ * D];
  __shared__ float lse_t[BQ];
  __shared__ float dd_t[BQ];

  const int tid = threadIdx.x, row = tid >> 1, half = tid & 1;
  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH;
  const int kt = blockIdx.x / BH;
  const int b = bh / p.H, h = bh % p.H;
  int start, len;
  seq_range<VARLEN>(p, b, start, len);
  const int k0 = kt * kF32Rows;
  if (k0 >= len) return;
  const size_t stride = (size_t)p.H * D, base = ((size_t)start * p.H + h) * D;
  const int kj = k0 + row;

  stage_f32<kF32Rows, D, KP>(Ks, p.k + base, k0, len, stride, tid);
  stage_f32<kF32Rows, D, KP>(Vs, p.v + base, k0, len, stride, tid);
  float dk[HD], dv[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) dk[d] = dv[d] = 0.f;

  const int q_begin = CAUSAL ? k0 : 0;
  for (int q0 = (q_begin / BQ) * BQ; q0 < len; q0 += BQ) {
    __syncthreads();
    stage_f32<BQ, D, D>(Qt, p.q + base, q0, len, stride, tid);
    stage_f32<BQ, D, D>(dOt, p.dout + base, q0, len, stride, tid);
    if (tid < BQ) {
      const int qq = q0 + tid;
      lse_t[tid] = qq < len ? p.lse[stat_idx<VARLEN>(p, b, h, start, qq)] * kLog2e : INFINITY;
      dd_t[tid] = qq < len ? p.dvec[stat_idx<VARLEN>(p, b, h, start, qq)] : 0.f;
    }
    __syncthreads();
    for (int i = 0; i < BQ; ++i) {
      float sp = 0.f, dpp = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) {
        sp = fmaf(Qt[i * D + half * HD + d], Ks[row * KP + half * HD + d], sp);
        dpp = fmaf(dOt[i * D + half * HD + d], Vs[row * KP + half * HD + d], dpp);
      }
      const float s = pair_reduce(sp), dp = pair_reduce(dpp);
      float pv = exp2f(s * p.c - lse_t[i]);
      if (CAUSAL && kj > q0 + i) pv = 0.f;
      const float ds = pv * (dp - dd_t[i]);
#pragma unroll
      for (int d = 0; d < HD; ++d) {
        dv[d] = fmaf(pv, dOt[i * D + half * HD + d], dv[d]);
        dk[d] = fmaf(ds, Qt[i * D + half * HD + d], dk[d]);
      }
    }
  }
  if (kj >= len) return;
  float* __restrict__ dkg = p.dk + base + (size_t)kj * stride + half * HD;
  float* __restrict__ dvg = p.dv + base + (size_t)kj * stride + half * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    dkg[d] = dk[d] * p.scale;
    dvg[d] = dv[d];
  }
}

// ---------------------------------------------------------------------------- dQ

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kF32Threads) void dq_fp32_kernel(F32Params p) {
  constexpr int HD = D / 2, BC = kF32Tile, QP = D + 1;
  __shared__ float Qs[kF32Rows * QP];
  __shared__ float dOs[kF32Rows * QP];
  __shared__ float Kt[BC * D];
  __shared__ float Vt[BC * D];

  const int tid = threadIdx.x, row = tid >> 1, half = tid & 1;
  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH;
  int qt = blockIdx.x / BH;
  if (CAUSAL) qt = p.n_tiles - 1 - qt;
  const int b = bh / p.H, h = bh % p.H;
  int start, len;
  seq_range<VARLEN>(p, b, start, len);
  const int q0 = qt * kF32Rows;
  if (q0 >= len) return;
  const size_t stride = (size_t)p.H * D, base = ((size_t)start * p.H + h) * D;
  const int qi = q0 + row;

  stage_f32<kF32Rows, D, QP>(Qs, p.q + base, q0, len, stride, tid);
  stage_f32<kF32Rows, D, QP>(dOs, p.dout + base, q0, len, stride, tid);
  const float lse_i = qi < len ? p.lse[stat_idx<VARLEN>(p, b, h, start, qi)] * kLog2e : INFINITY;
  const float d_i = qi < len ? p.dvec[stat_idx<VARLEN>(p, b, h, start, qi)] : 0.f;
  float dq[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) dq[d] = 0.f;
  const int kv_end = CAUSAL ? min(q0 + kF32Rows, len) : len;

  for (int k0 = 0; k0 < kv_end; k0 += BC) {
    __syncthreads();
    stage_f32<BC, D, D>(Kt, p.k + base, k0, len, stride, tid);
    stage_f32<BC, D, D>(Vt, p.v + base, k0, len, stride, tid);
    __syncthreads();
    for (int j = 0; j < BC; ++j) {
      float sp = 0.f, dpp = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) {
        sp = fmaf(Qs[row * QP + half * HD + d], Kt[j * D + half * HD + d], sp);
        dpp = fmaf(dOs[row * QP + half * HD + d], Vt[j * D + half * HD + d], dpp);
      }
      const float s = pair_reduce(sp), dp = pair_reduce(dpp);
      const int key = k0 + j;
      float pv = exp2f(s * p.c - lse_i);
      if (key >= len || (CAUSAL && key > qi)) pv = 0.f;
      const float ds = pv * (dp - d_i);
#pragma unroll
      for (int d = 0; d < HD; ++d) dq[d] = fmaf(ds, Kt[j * D + half * HD + d], dq[d]);
    }
  }
  if (qi >= len) return;
  float* __restrict__ dqg = p.dq + base + (size_t)qi * stride + half * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) dqg[d] = dq[d] * p.scale;
}

// ---------------------------------------------------------------------------- launch

F32Params make_f32(const Problem& pr) {
  F32Params p;
  p.q = static_cast<const float*>(pr.q);
  p.k = static_cast<const float*>(pr.k);
  p.v = static_cast<const float*>(pr.v);
  p.dout = static_cast<const float*>(pr.dout);
  p.lse = pr.lse;
  p.dvec = pr.dvec;
  p.o = static_cast<float*>(pr.o_out);
  p.lse_out = pr.lse_out;
  p.dq = static_cast<float*>(pr.dq);
  p.dk = static_cast<float*>(pr.dk);
  p.dv = static_cast<float*>(pr.dv);
  p.cu = pr.cu_seqlens;
  p.B = pr.batch;
  p.H = pr.heads;
  p.N = pr.seqlen;
  p.T = pr.total_tokens;
  p.n_tiles = (pr.seqlen + kF32Rows - 1) / kF32Rows;
  p.scale = pr.scale;
  p.c = pr.scale * kLog2e;
  return p;
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t fwd_t(const Problem& pr) {
  const F32Params p = make_f32(pr);
  hipLaunchKernelGGL((fwd_fp32_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)(p.n_tiles * p.B * p.H)),
                     dim3(kF32Threads), 0, pr.stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t dkdv_t(const Problem& pr) {
  const F32Params p = make_f32(pr);
  hipLaunchKernelGGL((dkdv_fp32_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)(p.n_tiles * p.B * p.H)),
                     dim3(kF32Threads), 0, pr.stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t dq_t(const Problem& pr) {
  const F32Params p = make_f32(pr);
  hipLaunchKernelGGL((dq_fp32_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)(p.n_tiles * p.B * p.H)),
                     dim3(kF32Threads), 0, pr.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp32(const Problem& p) { FA_DISPATCH(fwd_t, p); }

hipError_t launch_bwd_dkdv_fp32(const Problem& p) { FA_DISPATCH(dkdv_t, p); }

hipError_t launch_bwd_dq_fp32(const Problem& p) { FA_DISPATCH(dq_t, p); }

}  // namespace fa
