// fa_bwd.hip - backward pass of exact attention, bf16 tensors, fp32 arithmetic (gfx950).
//
// P is never read from memory: every kernel recomputes it tile by tile from Q, K and
// the saved logsumexp, P = exp2(c * q.k - LSE * log2(e)) with c = scale * log2(e)
// ("Recalcular en vez de guardar" in the AI Atlas summary of the FlashAttention paper).
// Three kernels:
//   bwd_pre   D_i = sum_k dO_ik * O_ik for every query row (fp32), from the stored O,
//             and -LSE_i / scale, the starting value of the S accumulation in bwd_dkdv.
//   bwd_dkdv  one (sequence, head, 128-key tile) at a time per workgroup (at head_dim
//             128 one persistent workgroup per compute unit takes a list of them); each
//             wave owns 32 keys and keeps K, V fragments and the dK^T, dV^T
//             accumulators in registers while it walks the 64-query tiles:
//                 S  = Q K^T,  P = exp2(c S - LSE log2e)
//                 dP = dO V^T, dS = P * (dP - D)
//                 dV^T += dO^T P,  dK^T += Q^T dS
//             S and dP are computed with one key per MFMA column, so P and dS feed the
//             next products' B operands straight from registers; Q and dO are staged
//             in LDS and read both row-wise and through transpose reads. At head_dim
//             128 the 32-query blocks run in a software pipeline (the next block's S
//             and dP on the matrix pipe while the vector ALUs do this block's softmax)
//             over four LDS buffers; at 64 two waves share each SIMD instead.
//   bwd_dq    the dQ accumulation pass: one workgroup per (sequence, head, 128-query
//             tile), dQ^T += K^T dS^T over the key tiles, with one query per MFMA column.
//             Its STATS form also computes the row statistics of bwd_pre for its own
//             queries (it loads their dO rows anyway) and runs first, so the backward
//             is two kernels: the dQ pass with the statistics, then bwd_dkdv.
// There are no atomics, so the result is bitwise reproducible run to run.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

struct BwdParams {
  const u16* q;
  const u16* k;
  const u16* v;
  const u16* o;
  const u16* dout;
  const float* lse;
  const float* dvec;
  const float* mneg;  // -LSE / scale (lse layout)
  float* dvec_out;  // the dQ pass that forms the statistics writes D here ...
  float* mneg_out;  // ... and -LSE / scale here
  float* dqacc;     // fused backward: fp32 dQ accumulator, (stat rows + 64) x D
  int* kvctr;       // work counters of the persistent dK/dV kernel (kKvCounters)
  u16* dq;
  u16* dk;
  u16* dv;
  const int32_t* cu;
  int B, H, N, T;
  int n_tiles;  // workgroups per (sequence, head): key tiles (dkdv) or query-tile slots (dq)
  float scale;
  float c;      // scale * log2(e)
};

// Index of (sequence b, head h, sequence-relative row n) in the lse / D layout:
// (B, H, N) for padded batches, (H, T) for packed ones.
template <bool VARLEN>
__device__ __forceinline__ size_t stat_index(const BwdParams& p, int b, int h, int start, int n) {
  return VARLEN ? (size_t)h * p.T + start + n : ((size_t)b * p.H + h) * p.N + n;
}

// ------------------------------------------------------------------------ bwd_pre

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* out);

template <>
__device__ __forceinline__ void load8<u16>(const u16* p, float* out) {
  const u32x4 x = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(x[i] << 16);
    out[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float* out) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[i] = a[i];
    out[4 + i] = b[i];
  }
}

// Sum over aligned groups of LANES (8 or 16) lanes, the result in every lane of the group,
// with DPP lane permutations: swap neighbours, swap pairs, then mirror within 8 and 16.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 8 || LANES == 16, "groups of 8 or 16 lanes");
  x += dpp_f32<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f32<0x141>(x);  // row_half_mirror
  if constexpr (LANES == 16) x += dpp_f32<0x140>(x);  // row_mirror
  return x;
}

// D = rowsum(dO * O) and -LSE / scale for 64 consecutive tokens of one (sequence, head)
// per workgroup (a packed batch is one sequence of total_tokens here: its statistics are
// laid out (H, total_tokens), those of a padded batch (B, H, N), so in both the 64 values
// are contiguous). D / 8 lanes reduce one row (8 elements each, a row is contiguous in
// memory); every load of the workgroup's rows is issued before the first reduction, so
// each wave keeps all of its rows in flight, and the results leave through LDS as two
// contiguous 256-byte stores.
constexpr int kPreTokens = 64;

template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                      const float* __restrict__ lse, float* __restrict__ dvec,
                                                      float* __restrict__ mneg, float* __restrict__ zacc,
                                                      int* __restrict__ kvctr, float scale, int H, int n_seq,
                                                      int n_tiles) {
  constexpr int LPR = D / 8;               // lanes per row
  constexpr int RPP = 256 / LPR;           // rows per pass
  constexpr int PASSES = kPreTokens / RPP;
  __shared__ float sd[kPreTokens];
  if (kvctr != nullptr && blockIdx.x == 0 && threadIdx.x < kKvCounters) kvctr[threadIdx.x] = 0;  // see bwd_dkdv
  // Heads vary fastest: consecutive workgroups read the rows of the same tokens, which
  // are adjacent in memory (token-major layout), so together they stream it in order.
  const int h = blockIdx.x % H;
  const int tile = (blockIdx.x / H) % n_tiles;
  const int s = blockIdx.x / H / n_tiles;
  const int sh = s * H + h;                // sequence * H + head
  const int n0 = tile * kPreTokens;
  const int sub = threadIdx.x % LPR;
  float a[PASSES][8], b[PASSES][8];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    // Rows past the end re-read the last row (no branch around the loads, so all of them
    // are in flight together); their sums are never stored.
    const int n = min(n0 + ps * RPP + (int)threadIdx.x / LPR, n_seq - 1);
    const size_t off = (((size_t)s * n_seq + n) * H + h) * D + 8 * sub;
    load8<T>(o + off, a[ps]);
    load8<T>(dout + off, b[ps]);
  }
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(a[ps][i], b[ps][i], acc);
    acc = group_sum<LPR>(acc);
    if (sub == 0) sd[ps * RPP + threadIdx.x / LPR] = acc;
  }
  __syncthreads();
  const size_t base = (size_t)sh * n_seq + n0;
  const int t = threadIdx.x % kPreTokens;
  if (n0 + t < n_seq) {
    if (threadIdx.x < kPreTokens)
      dvec[base + t] = sd[t];
    else if (threadIdx.x < 2 * kPreTokens)
      mneg[base + t] = -lse[base + t] / scale;
  }
  if (zacc != nullptr) {
    // The fused backward's dQ accumulator rows of these tokens start at zero (same row
    // order as the statistics, D floats per row).
    const int rows = min(kPreTokens, n_seq - n0);
    f32x4* z = reinterpret_cast<f32x4*>(zacc + base * D);
    for (int i = threadIdx.x; i < rows * (D / 4); i += 256) z[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// ------------------------------------------------------------------------ bwd_dkdv

constexpr int kKvWaves = 4;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKvBK = 32 * kKvWaves;  // keys per workgroup
constexpr int kKvBQ = 64;             // queries per tile: two 32-query blocks
constexpr int kKvPf = 2;              // operand reads run this many MFMA steps ahead
// LDS buffers of the head_dim-128 kernel: four (two tiles in flight while one is read;
// they fill the 160 KB).
constexpr int kKvStages = 4;

// One LDS buffer: Q and dO tiles (swizzled rows; read row-wise for S and dP and through
// transpose reads for dK and dV), all copied in by DMA. The per-query statistics sit in
// the pads of the Q tile: -LSE / scale of queries 16i .. 16i + 15 in the pad of row i,
// D in the pad of row 4 + i (i = 0..3).
template <int D>
struct KvLds {
  static constexpr int P = swz_pitch<D>();
  static constexpr int TSZ = kKvBQ * P;  // elements of one tile, pads included
  static constexpr int BUF = 2 * TSZ;
  // u16 element offset of the 16 statistics `which` (0: -LSE / scale, 1: D) of queries
  // 16 i .. 16 i + 15
  static constexpr int stat_pad(int which, int i) { return (4 * which + i) * P + D; }
};

// Row pitch of the K and V rows the head_dim-128 dK/dV kernel stages in LDS buffers 2 and
// 3 on their way into registers (conflict-free row reads).
template <int D>
constexpr int kv_rows_pitch() { return D + 8; }

template <int D>
struct KvState {
  static constexpr int NB = D / 32, NS = D / 16;
  bf16x8 kf[NS], vf[NS];    // this lane's key row and negated value row, as B operands
  f32x16 dvT[NB], dkT[NB];  // dV^T and -dK^T
};

// One 32-query block in flight, one key per C column: register r of lane group g holds
// query q + crow_nat(r, g). The S product starts from -LSE / scale, so that
// P = exp2(c s) with c = scale log2(e); with the value rows negated, the dP product
// starts from D and yields D - dP. The softmax step turns s into P and dp into
// P (D - dP) = -dS.
struct KvBlock {
  f32x16 s, dp;
};

// Statistics of the block at rows r0 of tile buffer buf, register set r4 (rows
// q = r0 + 8 r4 + 4 g + 0..3, in the pad for queries 16 (q / 16) ..): -LSE / scale
// (which = 0) or D (which = 1).
template <int D>
__device__ __forceinline__ f32x4 kv_stat4(const u16* buf, int which, int r0, int r4, int g) {
  const u16* pad = buf + KvLds<D>::stat_pad(which, (r0 >> 4) + (r4 >> 1));
  return *reinterpret_cast<const f32x4*>(pad + 16 * (r4 & 1) + 8 * g);
}

template <int D>
__device__ __forceinline__ void kv_init_s(KvBlock& b, const u16* buf, int r0, int r4, int g) {
  const f32x4 m4 = kv_stat4<D>(buf, 0, r0, r4, g);
#pragma unroll
  for (int e = 0; e < 4; ++e) b.s[4 * r4 + e] = m4[e];
}

template <int D>
__device__ __forceinline__ void kv_init_dp(KvBlock& b, const u16* buf, int r0, int r4, int g) {
  const f32x4 d4 = kv_stat4<D>(buf, 1, r0, r4, g);
#pragma unroll
  for (int e = 0; e < 4; ++e) b.dp[4 * r4 + e] = d4[e];
}

// dV^T / dK^T accumulation step. At head_dim 128 the accumulators (128 registers) are
// pinned in AGPRs, leaving the VGPRs to the score arithmetic; at 64 they fit anyway.
template <int D>
__device__ __forceinline__ void kv_acc_mfma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (D == 128) {
    mfma32_agpr(acc, a, b);
  } else {
    acc = mfma32(a, b, acc);
  }
}

template <int D>
__device__ __forceinline__ void kv_acc_fence(f32x16& acc) {
  if constexpr (D == 128) agpr_acc_fence(acc);
}

// Row-wise operand of step j of the S / dP products of the block at rows r0 of tile
// buffer `buf`: the two products alternate (even steps: Q slice j / 2 for S, odd
// steps: dO slice j / 2 for dP), so that no MFMA waits for the one just before it.
template <int D>
__device__ __forceinline__ bf16x8 kv_row_operand(const u16* buf, int r0, int j, int lane) {
  return swz_row_operand<D>((j & 1) ? buf + KvLds<D>::TSZ : buf, r0, j >> 1, lane);
}

// Transposed operand of step j of the dV / dK products of the block at rows r0: dO^T
// (for dV^T += dO^T P) in steps 0 .. NT-1, then Q^T (for dK^T += Q^T dS). Within a
// product, step jj covers head-dim columns 32 (jj % NB) .. (accumulator jj % NB) and
// query rows 16 (jj / NB) .. (k-slots in C-row order), so consecutive MFMAs update
// different accumulators.
template <int D>
__device__ __forceinline__ bf16x8 kv_tr_operand(const u16* buf, int r0, int j, int lane) {
  constexpr int NT = D / 16, NB = D / 32;  // operands per product, accumulators
  const int jj = j % NT;
  return swz_tr_operand<D>(j < NT ? buf + KvLds<D>::TSZ : buf, r0 + 16 * (jj / NB), 32 * (jj % NB), lane);
}

// Softmax of element r of block b (query qc + crow_nat(r, g)) in two parts, one step
// apart: the exponential P = exp2(c (S - LSE / scale)), then (next step) the mask, -dS =
// P (D - dP) and, every eighth element, eight of each converted to bf16 as half of a B
// operand. Done in one step, the multiply would wait on the exponential (a transcendental
// result needs a wait state before its first use, here an s_nop).
__device__ __forceinline__ void kv_softmax_exp(KvBlock& b, int r, float c) {
  float e = fast_exp2(b.s[r] * c);
  // Pin the exponential to this step (the compiler would otherwise sink the softmax
  // towards its first use, out of the matrix-pipe phase it is meant to overlap).
  asm volatile("" : "+v"(e));
  b.s[r] = e;
}

template <bool CAUSAL, bool MASK>
__device__ __forceinline__ void kv_softmax_finish(KvBlock& b, bf16x8 (&pb)[2], bf16x8 (&db)[2], int r, int qc,
                                                  int kj, int len, int g) {
  float e = b.s[r];
  if constexpr (MASK) {
    const int qq = qc + crow_nat(r, g);
    e = (qq >= len || (CAUSAL && kj > qq)) ? 0.f : e;
    b.s[r] = e;
  }
  b.dp[r] *= e;
  if (r % 8 == 7) {
    pb[r / 8] = to_bf16x8(half_of(b.s, r / 8));
    db[r / 8] = to_bf16x8(half_of(b.dp, r / 8));
    // keep the conversions in this step too (they would sink to phase Y's first MFMA)
    asm volatile("" : "+v"(pb[r / 8]), "+v"(db[r / 8]));
  }
}

// Phase X. The matrix pipe computes S and D - dP of block nx (rows rn of tile buffer
// bn; when NXT) while the vector ALUs run the softmax step of block cu (query rows
// qc.., tile buffer bc, rows rc; when CUR). rop holds the first kKvPf row operands of
// nx, and nx.s and nx.dp their starting values, read beforehand; the last steps read
// the first kKvPf transposed operands of phase Y for cu into top.
template <int D, bool CAUSAL, bool NXT, bool CUR, bool MASK>
__device__ __forceinline__ void kv_phase_x(const KvState<D>& st, KvBlock& nx, const u16* bn, int rn,
                                           bf16x8 (&rop)[kKvPf], KvBlock& cu, bf16x8 (&pb)[2], bf16x8 (&db)[2],
                                           const u16* bc, int rc, bf16x8 (&top)[kKvPf], int qc, int kj, int len,
                                           float c, int lane) {
  constexpr int NS = D / 16, NX = 2 * NS, EPS = 16 / NX;
  const int g = lane >> 5;
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    if constexpr (NXT) {
      const bf16x8 a = rop[j % kKvPf];
      if (j + kKvPf < NX) rop[j % kKvPf] = kv_row_operand<D>(bn, rn, j + kKvPf, lane);
      if ((j & 1) == 0)
        nx.s = mfma32(a, st.kf[j >> 1], nx.s);
      else
        nx.dp = mfma32(a, st.vf[j >> 1], nx.dp);
    }
    if constexpr (CUR) {
#pragma unroll
      for (int u = 0; u < EPS; ++u) kv_softmax_exp(cu, EPS * j + u, c);
      if (j > 0) {
#pragma unroll
        for (int u = 0; u < EPS; ++u) kv_softmax_finish<CAUSAL, MASK>(cu, pb, db, EPS * (j - 1) + u, qc, kj, len, g);
      }
      if (j >= NX - kKvPf) top[j - (NX - kKvPf)] = kv_tr_operand<D>(bc, rc, j - (NX - kKvPf), lane);
    }
    step_fence();
  }
  if constexpr (CUR) {
#pragma unroll
    for (int u = 0; u < EPS; ++u) kv_softmax_finish<CAUSAL, MASK>(cu, pb, db, EPS * (NX - 1) + u, qc, kj, len, g);
  }
}

// Phase Y for block cu (rows rc of tile buffer bc): dV^T += dO^T P, then
// -dK^T += Q^T (-dS), with the transposed operands read kKvPf steps ahead (the first
// ones in phase X). When NXT, the last steps read the first row operands and the
// starting values of S and dP of the block the next phase X computes (nx: rows rn of
// tile buffer bn).
template <int D, bool NXT>
__device__ __forceinline__ void kv_phase_y(KvState<D>& st, const u16* bc, int rc, const bf16x8 (&pb)[2],
                                           const bf16x8 (&db)[2], bf16x8 (&top)[kKvPf], const u16* bn, int rn,
                                           bf16x8 (&rop)[kKvPf], KvBlock& nx, int lane) {
  constexpr int NT = D / 16, NB = D / 32, NY = 2 * NT;
  static_assert(NY >= 8 && NY >= kKvPf, "the prefetches need eight steps");
#pragma unroll
  for (int j = 0; j < NY; ++j) {
    const bf16x8 a = top[j % kKvPf];
    if (j + kKvPf < NY) top[j % kKvPf] = kv_tr_operand<D>(bc, rc, j + kKvPf, lane);
    const int jj = j % NT;
    if (j < NT)
      kv_acc_mfma<D>(st.dvT[jj % NB], a, pb[jj / NB]);
    else
      kv_acc_mfma<D>(st.dkT[jj % NB], a, db[jj / NB]);
    if constexpr (NXT) {
      if (j >= NY - kKvPf) rop[j - (NY - kKvPf)] = kv_row_operand<D>(bn, rn, j - (NY - kKvPf), lane);
      if (j >= NY - 8 && j < NY - 4) kv_init_dp<D>(nx, bn, rn, j - (NY - 8), lane >> 5);
      if (j >= NY - 4) kv_init_s<D>(nx, bn, rn, j - (NY - 4), lane >> 5);
    }
    step_fence();
  }
}

// Phase X dispatch on the wave-uniform flags (each combination is its own straight-line
// code).
template <int D, bool CAUSAL>
__device__ __forceinline__ void kv_x(bool nxt, bool cur, bool mask, const KvState<D>& st, KvBlock& nx,
                                     const u16* bn, int rn, bf16x8 (&rop)[kKvPf], KvBlock& cu, bf16x8 (&pb)[2],
                                     bf16x8 (&db)[2], const u16* bc, int rc, bf16x8 (&top)[kKvPf], int qc, int kj,
                                     int len, float c, int lane) {
#define FA_KV_X(N, C, M) \
  kv_phase_x<D, CAUSAL, N, C, M>(st, nx, bn, rn, rop, cu, pb, db, bc, rc, top, qc, kj, len, c, lane)
  if (cur) {
    if (nxt) {
      if (mask) FA_KV_X(true, true, true); else FA_KV_X(true, true, false);
    } else {
      if (mask) FA_KV_X(false, true, true); else FA_KV_X(false, true, false);
    }
  } else if (nxt) {
    FA_KV_X(true, false, false);
  }
#undef FA_KV_X
}

// One (sequence, head, 128-key tile) for one workgroup; wave w owns keys k0 + 32w .. + 31
// and walks the 64-query tiles from the diagonal on, two 32-query blocks per tile, in a
// software pipeline across blocks and tiles:
//   X(t,0) [S, dP of (t,1) | softmax of (t,0)]  barrier  Y(t,0) [dV, dK of (t,0)]
//   X(t,1) [S, dP of (t+1,0) | softmax of (t,1)]  Y(t,1) [dV, dK of (t,1)]
// The barrier in tile t follows the wait for tile t+1 and precedes the copy of tile
// t+3 into the buffer tile t-1 used; a wave's last read of tile t-1 (in Y(t-1,1))
// comes before it.
template <int D, bool CAUSAL, bool VARLEN>
__device__ __forceinline__ void dkdv_ktile(const BwdParams& p, int bh, int kt, u16* lds, int nxt, int* nxt_slot) {
  constexpr int BK = kKvBK, BQ = kKvBQ, NS = D / 16, NB = D / 32;
  constexpr int S = kKvStages;
  using L = KvLds<D>;
  using Dma = TileDma<BQ, D, L::P, kKvWaves, true, 8, false>;  // statistics in the pads of Q rows 0..7

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int b = bh / p.H, h = bh % p.H;
  int start, len;
  if (VARLEN) {
    start = p.cu[b];
    len = p.cu[b + 1] - start;
  } else {
    start = b * p.N;
    len = p.N;
  }
  const int k0 = kt * BK;
  if (k0 >= len) {
    if (VARLEN && threadIdx.x == 0) *nxt_slot = nxt;
    return;
  }

  const size_t stride = (size_t)p.H * D;
  const size_t base = ((size_t)start * p.H + h) * D;
  const u16* __restrict__ Qg = p.q + base;
  const u16* __restrict__ dOg = p.dout + base;

  const int wk0 = k0 + 32 * w;  // first key of this wave
  const int kj = wk0 + lr;      // this lane's key

  KvState<D> st;  // K and V rows are read in the prologue
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    st.dvT[bb] = f32x16{};
    st.dkT[bb] = f32x16{};
  }

  const int qt_begin = CAUSAL ? k0 / BQ : 0;
  const int n_qt = (len + BQ - 1) / BQ;
  // First tile this wave computes (wave-uniform): under causal the first one whose last
  // query reaches the wave's first key; none when the wave's keys are all past the end.
  const int qt_w = wk0 >= len ? n_qt : (CAUSAL ? max(qt_begin, wk0 / BQ) : 0);

  Dma tdma;
  tdma.init(stride, w, lane);
  auto bufp = [&](int qt) -> u16* { return lds + ((unsigned)(qt - qt_begin) % S) * L::BUF; };
  // Every wave issues the same number of copies per tile (its share of the Q and dO
  // tiles, and two 16-query statistics copies: wave w copies -LSE / scale and D of
  // queries 16w .. 16w + 15 into their pads), so a wave can wait for "all but the
  // newest k tiles" with one vmcnt.
  static_assert(BQ == 64 && kKvWaves == 4, "statistics copies assume 16 queries per wave");
  constexpr int CNT = 2 * Dma::PER_WAVE + 2;
  auto issue = [&](int qt) {
    u16* buf = bufp(qt);
    const int q0 = qt * BQ;
    tdma.issue(buf, Qg, q0, len, stride, w, lane);
    tdma.issue(buf + L::TSZ, dOg, q0, len, stride, w, lane, false);
#if __HIP_DEVICE_COMPILE__
    // lane 16w + t lands at dst + 4 (16w + t) bytes: dst = pad - 64w bytes puts it at pad + 4t
    const int qq = min(q0 + lane, len - 1);  // rows past the end are masked in the tile
    const size_t si = stat_index<VARLEN>(p, b, h, start, qq);
    if ((lane >> 4) == w) {
      dma_lds_b32(p.mneg + si, buf + L::stat_pad(0, w) - 32 * w);
      dma_lds_b32(p.dvec + si, buf + L::stat_pad(1, w) - 32 * w);
    }
#endif
  };
  // Wait until the tiles issued after the wanted one (younger of them: 0 .. 2) are the
  // only copies this wave still has in flight.
  auto wait_tiles = [&](int younger) {
    if (younger >= 2)
      wait_vmem_count<2 * CNT>();
    else if (younger == 1)
      wait_vmem_count<CNT>();
    else
      wait_vmem();
  };

  // Prologue. This key tile's K and V rows come in through LDS buffers 2 and 3, whole
  // rows per copy instruction (loaded straight into registers, every load instruction
  // would gather 32 bytes from each of 32 rows), while tiles qt_begin and qt_begin + 1
  // land in buffers 0 and 1. Every wave takes its rows into registers before tile
  // qt_begin + 2 refills buffer 2; tile qt_begin + 3 goes to buffer 3 after the barrier
  // of tile qt_begin.
  static_assert(S == 4, "the K/V rows pass through buffers 2 and 3");
  constexpr int KVP = kv_rows_pitch<D>();
  static_assert(BK * KVP <= L::BUF, "a K or V tile fits in one buffer");
  {
    TileDma<BK, D, KVP, kKvWaves> kvdma;
    kvdma.init(stride, w, lane);
    kvdma.issue(lds + 2 * L::BUF, p.k + base, k0, len, stride, w, lane);
    kvdma.issue(lds + 3 * L::BUF, p.v + base, k0, len, stride, w, lane);
  }
  issue(qt_begin);
  if (qt_begin + 1 < n_qt) issue(qt_begin + 1);
  wait_tiles(min(1, n_qt - qt_begin - 1));  // the K/V rows and tile qt_begin (older copies)
  lds_barrier();
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int e = (32 * w + lr) * KVP + 16 * s + 8 * g;  // this lane's key row, head-dim 16 s + 8 g
    st.kf[s] = kj < len ? ld16(lds + 2 * L::BUF + e) : zero_bf16x8();
    const bf16x8 v = kj < len ? ld16(lds + 3 * L::BUF + e) : zero_bf16x8();
    st.vf[s] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, v) ^ 0x80008000u);
  }
  lds_barrier();
  if (qt_begin + 2 < n_qt) issue(qt_begin + 2);

  KvBlock blk0, blk1;
  bf16x8 rop[kKvPf], top[kKvPf], pb[2], db[2];
  // A wave's first block: S and D - dP alone, then the row operands of the next block.
  auto first_block = [&](int qt) {
    const u16* bf = bufp(qt);
#pragma unroll
    for (int j = 0; j < kKvPf; ++j) rop[j] = kv_row_operand<D>(bf, 0, j, lane);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      kv_init_s<D>(blk0, bf, 0, r4, g);
      kv_init_dp<D>(blk0, bf, 0, r4, g);
    }
    kv_phase_x<D, CAUSAL, true, false, false>(st, blk0, bf, 0, rop, blk1, pb, db, bf, 0, top, 0, kj, len, p.c,
                                              lane);
#pragma unroll
    for (int j = 0; j < kKvPf; ++j) rop[j] = kv_row_operand<D>(bf, 32, j, lane);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      kv_init_s<D>(blk1, bf, 32, r4, g);
      kv_init_dp<D>(blk1, bf, 32, r4, g);
    }
  };
  // The collective step between the two blocks of tile qt: wait for tile qt + 1 (tiles
  // up to qt + S - 2 may still be in flight), barrier, then refill the buffer of tile
  // qt - 1 with tile qt + S - 1.
  auto next_tile_sync = [&](int qt) {
    wait_tiles(max(0, min(S - 3, n_qt - qt - 2)));
    lds_barrier();
    if (qt + S - 1 < n_qt) issue(qt + S - 1);
  };
  auto mask_of = [&](int q0) { return q0 + BQ > len || (CAUSAL && q0 < wk0 + 31); };  // wave-uniform

  // Tiles before this wave's first: only the collective part.
  const int qs = min(qt_w, n_qt);
  if (qs == qt_begin && qs < n_qt) first_block(qs);
  for (int qt = qt_begin; qt < qs; ++qt) {
    if (qt + 1 < n_qt) next_tile_sync(qt);
    if (qt + 1 == qs && qs < n_qt) first_block(qs);
  }
  // Every tile but the last: the full pipeline. Each buffer slot has its own copy of
  // the code, so that LDS addresses are per-lane offsets plus constants.
  auto tile_step = [&](int qt) {
    const u16* bc = bufp(qt);
    const u16* bn = bufp(qt + 1);
    const int q0 = qt * BQ;
    const bool mask = mask_of(q0);
    kv_x<D, CAUSAL>(true, true, mask, st, blk1, bc, 32, rop, blk0, pb, db, bc, 0, top, q0, kj, len, p.c, lane);
    next_tile_sync(qt);
    kv_phase_y<D, true>(st, bc, 0, pb, db, top, bn, 0, rop, blk0, lane);
    kv_x<D, CAUSAL>(true, true, mask, st, blk0, bn, 0, rop, blk1, pb, db, bc, 32, top, q0 + 32, kj, len, p.c, lane);
    kv_phase_y<D, true>(st, bc, 32, pb, db, top, bn, 32, rop, blk1, lane);
  };
  for (int qt = qs; qt < n_qt - 1; ++qt) tile_step(qt);
  // The last tile.
  if (qs < n_qt) {
    const int qt = n_qt - 1;
    const u16* bc = bufp(qt);
    const int q0 = qt * BQ;
    const bool mask = mask_of(q0);
    kv_x<D, CAUSAL>(true, true, mask, st, blk1, bc, 32, rop, blk0, pb, db, bc, 0, top, q0, kj, len, p.c, lane);
    kv_phase_y<D, false>(st, bc, 0, pb, db, top, bc, 0, rop, blk0, lane);
    kv_x<D, CAUSAL>(false, true, mask, st, blk0, bc, 0, rop, blk1, pb, db, bc, 32, top, q0 + 32, kj, len, p.c, lane);
    kv_phase_y<D, false>(st, bc, 32, pb, db, top, bc, 32, rop, blk1, lane);
  }

#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    kv_acc_fence<D>(st.dvT[bb]);
    kv_acc_fence<D>(st.dkT[bb]);
  }
  // Every wave is past its last tile read: the LDS now stages this wave's dK and dV rows
  // (32 keys each) so that they leave as whole rows.
  static_assert(kKvWaves * 64 * stage_pitch<D>() <= S * L::BUF, "staging fits in the tile buffers");
  lds_barrier();
  // Packed batches: the next work item, drawn when this one started; by now no copy is in
  // flight, so the wait for the atomic's result costs nothing (the stores come after it).
  if (VARLEN && threadIdx.x == 0) *nxt_slot = nxt;
  u16* stg = lds + w * 64 * stage_pitch<D>();
  stage_acc_rows<D>(stg, st.dkT, -p.scale, lr, g);  // the accumulator holds -dK^T / scale
  stage_acc_rows<D>(stg + 32 * stage_pitch<D>(), st.dvT, 1.f, lr, g);
  const int valid = len - wk0;
  store_staged_rows<D, 32>(stg, p.dk + base + (size_t)wk0 * stride, stride, valid, lane);
  store_staged_rows<D, 32>(stg + 32 * stage_pitch<D>(), p.dv + base + (size_t)wk0 * stride, stride, valid, lane);
}

// Persistent: gridDim.x = 8 C workgroups, one per compute unit. Workgroup 8 c + x serves
// XCD x (the dispatcher places workgroup i on XCD i % 8), whose work items are the mapped
// tiles 8 k + x, k = 0, 1, ...: the key tiles of one head after another, heaviest first
// under causal masking. A workgroup's final stores drain while it starts its next item.
//  - Padded batches (every head alike): workgroup c takes k = n C + c in even rounds n
//    and n C + C - 1 - c in odd ones, so that a heavy and a light key tile alternate on
//    each compute unit and the XCD's workgroups move from head to head together (measured
//    3-7 % faster than drawing items as below, which spreads them over more heads).
//  - Packed batches (sequence lengths differ, and key tiles past a sequence's end are
//    empty): each workgroup draws the next k from its XCD's counter (kvctr[x], an atomic
//    add) when it starts an item, skipping empty ones, so a workgroup that drew light
//    tiles draws more (measured 6 % faster than the fixed order at 16384 packed tokens).
//    The statistics kernel that runs first sets the counters to zero; the last workgroup
//    to finish sets them back (kvctr[8] counts the finished ones), so that the workspace
//    is left as it was found.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kKvThreads, 1) void bwd_dkdv_bf16_kernel(BwdParams p) {
  static_assert(D == 128, "head_dim 64 has its own kernel (bwd_dkdv_rows_kernel)");
  __shared__ __attribute__((aligned(16))) u16 lds[kKvStages * KvLds<D>::BUF];
  // The item of iteration n goes to next_k[n % 2], in buffer 2 past its staged K rows:
  // written after a key tile's last read of the buffers (or at an empty item), read before
  // the next item's first copies, none of which reach it (tiles go to buffers 0 and 1,
  // the rows to the head of buffers 2 and 3; tile 2 refills buffer 2 only after a barrier).
  static_assert(kKvBK * kv_rows_pitch<D>() + 4 <= KvLds<D>::BUF, "room for the item slots");
  int* next_k = reinterpret_cast<int*>(lds + 2 * KvLds<D>::BUF + kKvBK * kv_rows_pitch<D>());
  const int total = p.B * p.H * p.n_tiles;
  const int xcd = blockIdx.x % 8, c = blockIdx.x / 8, C = gridDim.x / 8;
  const int count = (total - xcd + 7) / 8;  // work items of XCD xcd
  if constexpr (!VARLEN) {
    for (int n = 0;; ++n) {
      const int k = n * C + ((n & 1) ? C - 1 - c : c);
      if (k >= count) break;
      int bh, kt;
      xcd_tile_map(8 * k + xcd, p.B * p.H, p.n_tiles, false, true, bh, kt);
      if (n > 0) __syncthreads();  // every wave has read its staged rows of the previous tile
      dkdv_ktile<D, CAUSAL, VARLEN>(p, bh, kt, lds, 0, next_k);
    }
  } else {
    // Thread 0 draws items until one has keys or the XCD's list is used up (at most
    // count + 1 draws).
    auto draw = [&]() {
      int k;
      for (;;) {
        k = atomicAdd(p.kvctr + xcd, 1);
        if (k >= count) break;
        int bh, kt;
        xcd_tile_map(8 * k + xcd, p.B * p.H, p.n_tiles, false, true, bh, kt);
        const int b = bh / p.H;
        if (kt * kKvBK < p.cu[b + 1] - p.cu[b]) break;
      }
      return k;
    };
    if (threadIdx.x == 0) next_k[0] = draw();
    __syncthreads();
    for (int n = 0;; ++n) {
      const int k = next_k[n & 1];
      if (k >= count) break;
      int nxt = 0;
      if (threadIdx.x == 0) nxt = draw();
      int bh, kt;
      xcd_tile_map(8 * k + xcd, p.B * p.H, p.n_tiles, false, true, bh, kt);
      dkdv_ktile<D, CAUSAL, VARLEN>(p, bh, kt, lds, nxt, &next_k[(n + 1) & 1]);
      __syncthreads();  // the next item is visible; every wave has read its staged rows
    }
    if (threadIdx.x == 0) {
      __threadfence();  // this workgroup's last draw happens before it counts as finished
      if (atomicAdd(p.kvctr + 8, 1) == (int)gridDim.x - 1)
        for (int x = 0; x < kKvCounters; ++x) p.kvctr[x] = 0;
    }
  }
}

// ------------------------------------------------------------------------ bwd_fused
//
// The head_dim-128 dK/dV kernel with the dQ product folded in: one pass over the key
// tiles computes all five products (S, dP, dV, dK and dQ; the recomputation of P by
// blocks in "Recalcular en vez de guardar", AI Atlas summary of the FlashAttention
// paper), against seven in the two-kernel backward, at the price of fp32 atomics whose
// order makes dQ reproducible only up to rounding.
//
// The dQ product contracts over keys, which a wave holds one per lane, so -dS changes
// hands through LDS: after its softmax step every wave writes its 32 keys x 32 queries
// of -dS (bf16, the values its own dK product uses) into an exchange tile, and after the
// next workgroup barrier each wave computes -dQ / scale for the block's 32 queries and
// its own 32-wide slice of head_dim over all 128 keys (8 MFMAs; one query per C row, one
// head-dim column per lane, the K operands held in AGPRs since the prologue). The result
// is added into an fp32 accumulator in global memory (B, H, N, D) / (H, T, D) with
// global_atomic_add_f32, 128 contiguous bytes per half-wave; bwd_dq_convert scales it
// and writes dQ. The accumulator is zeroed by the statistics kernel (bwd_pre) that runs
// first.
//
// Schedule per 64-query tile t (blocks (t,0) and (t,1)), with X and Y the phases of the
// dK/dV kernel:
//   X(t,0)  write -dS(t,0) to E0[t % 2]   barrier t   Y(t,0) + atomics of dQ(t-2,1), dQ(t-1,0)
//   X(t,1)  write -dS(t,1) to E1[t % 2]               Y(t,1) + MFMAs of dQ(t-1,1), dQ(t,0)
// Each exchange slot is read between the barrier after its write and the one after that,
// and rewritten only after the latter. Three Q/dO buffers (not four) leave room for the
// four 8 KB exchange tiles; with three, the wait at every barrier is for all copies in
// flight, so the atomics, issued right after the barrier, have a whole tile to complete
// before the next wait.

constexpr int kFzStages = 3;
constexpr int kXq = 32;                 // queries per exchange-tile row
constexpr int kXTile = kKvBK * kXq;     // elements of one exchange tile (8 KB)

// Element offset of 4-element run `run` (queries 4 run .. 4 run + 3) of key row kk in an
// exchange tile. Runs are swizzled by key, run ^ ((kk >> 2) & 7): a wave's writes (one
// run per lane, 32 keys) and the transpose reads of the dQ product (4 keys x 32 queries
// per 32 lanes) both fall on distinct banks.
__device__ __forceinline__ int xch_elem(int kk, int run) { return kk * kXq + 4 * (run ^ ((kk >> 2) & 7)); }

// This lane's -dS (db: key kk, queries 8 r4 + 4 g + 0..3 in registers 4 r4 .. 4 r4 + 3)
// into exchange tile x, one 8-byte write per r4.
__device__ __forceinline__ void xch_write(u16* x, const bf16x8 (&db)[2], int kk, int g) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const u32x4 u = __builtin_bit_cast(u32x4, db[r4 >> 1]);
    *reinterpret_cast<u32x2*>(x + xch_elem(kk, 2 * r4 + g)) = u32x2{u[2 * (r4 & 1)], u[2 * (r4 & 1) + 1]};
  }
}

// A operand of step s of a dQ product from exchange tile x: row m = query m of the block,
// k-slots = keys 16 s + 4 g + {0..3, 8..11}, in the order of lds_tr_operand. The lane's
// addresses depend on s only through 512 s and the swizzle bit s % 2: xo holds the
// lane's element offsets for (s % 2, lo / hi read), set once by xch_lane_offsets.
struct XchLane {
  int o[4];
};

__device__ __forceinline__ XchLane xch_lane_offsets(int lane) {
  const int i = lane & 15, G = lane >> 4;
  const int kl = 4 * (G >> 1) + (i >> 2);  // key within the 16-key slice (lo read)
  const int run = 4 * (G & 1) + (i & 3);
  XchLane x;
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    x.o[2 * par] = xch_elem(16 * par + kl, run);
    x.o[2 * par + 1] = xch_elem(16 * par + kl + 8, run);
  }
  return x;
}

__device__ __forceinline__ bf16x8 xch_operand(const u16* x, const XchLane& xo, int s) {
  const u16* t = x + 16 * kXq * (s & ~1);
  const i16x4 lo = ds_read_tr16(t + xo.o[2 * (s & 1)]);
  const i16x4 hi = ds_read_tr16(t + xo.o[2 * (s & 1) + 1]);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// dQ MFMAs on AGPR accumulators with the K operand (B) in AGPRs too; the first step of a
// block starts from zero. The wait states are those of mfma32_agpr.
__device__ __forceinline__ void dq_mfma_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&a"(acc) : "v"(a), "a"(b));
}

__device__ __forceinline__ void dq_mfma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "a"(b));
}

__device__ __forceinline__ bf16x8 to_agpr(const bf16x8& x) {
  bf16x8 y;
  asm volatile("; K operand to AGPRs" : "=a"(y) : "0"(x));
  return y;
}

__device__ __forceinline__ void agpr_acc_fence2(f32x16& a, f32x16& b) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" : "+a"(a), "+a"(b));
}

// Adds v at byte offset off (this lane's, 32-bit) from the wave-uniform address base: the
// uniform part stays in SGPRs (the atomic's scalar base), the lane part in one VGPR.
__device__ __forceinline__ void atomic_add_f32(const char* base, uint32_t off, float v) {
  __builtin_amdgcn_global_atomic_fadd_f32((__attribute__((address_space(1))) float*)(base + (uint64_t)off), v);
}

// Byte offset of register r's row from a dQ block's first row (C row crow_nat(r, g) minus
// the lane group's 4 g, which is in the lane offset).
template <int D>
constexpr uint32_t dq_row_bytes(int r) { return (uint32_t)((8 * (r >> 2) + (r & 3)) * D * 4); }

// Phase Y(t,0) of the fused kernel: kv_phase_y's 16 MFMAs for block cu, and the atomics
// that add the two finished dQ blocks qa (first row at ga) and qb (at gb) into the
// accumulator, two per step. Register r of lane group g holds query row crow_nat(r, g),
// head-dim column 32 w + lr: byte offset dq_row_bytes(r) + loff from the block's first
// row, with loff = 4 (4 g D + 32 w + lr).
template <int D, bool NXT>
__device__ __forceinline__ void fz_phase_y_atomics(KvState<D>& st, const u16* bc, int rc, const bf16x8 (&pb)[2],
                                                   const bf16x8 (&db)[2], bf16x8 (&top)[kKvPf], const u16* bn, int rn,
                                                   bf16x8 (&rop)[kKvPf], KvBlock& nx, f32x16& qa, const char* ga,
                                                   f32x16& qb, const char* gb, uint32_t loff, int lane) {
  constexpr int NT = D / 16, NB = D / 32, NY = 2 * NT;
  static_assert(NY == 16, "two atomics per step cover the 16 registers of each block");
  agpr_acc_fence2(qa, qb);
#pragma unroll
  for (int j = 0; j < NY; ++j) {
    const bf16x8 a = top[j % kKvPf];
    if (j + kKvPf < NY) top[j % kKvPf] = kv_tr_operand<D>(bc, rc, j + kKvPf, lane);
    const int jj = j % NT;
    if (j < NT)
      kv_acc_mfma<D>(st.dvT[jj % NB], a, pb[jj / NB]);
    else
      kv_acc_mfma<D>(st.dkT[jj % NB], a, db[jj / NB]);
    atomic_add_f32(ga + dq_row_bytes<D>(j), loff, qa[j]);
    atomic_add_f32(gb + dq_row_bytes<D>(j), loff, qb[j]);
    if constexpr (NXT) {
      if (j >= NY - kKvPf) rop[j - (NY - kKvPf)] = kv_row_operand<D>(bn, rn, j - (NY - kKvPf), lane);
      if (j >= NY - 8 && j < NY - 4) kv_init_dp<D>(nx, bn, rn, j - (NY - 8), lane >> 5);
      if (j >= NY - 4) kv_init_s<D>(nx, bn, rn, j - (NY - 4), lane >> 5);
    }
    step_fence();
  }
}

// Phase Y(t,1) of the fused kernel: kv_phase_y's 16 MFMAs for block cu interleaved with
// the 16 MFMAs of two dQ blocks, qa from exchange tile xa and qb from xb (dQ step u:
// block u % 2, key slice u / 2). Order: kv0 kv1 dq0 kv2 dq1 kv3 ... kv15 dq14 dq15, so
// each dQ accumulator is updated every fourth MFMA; the dQ operands are read two dQ steps
// ahead.
template <int D, bool NXT>
__device__ __forceinline__ void fz_phase_y_dq(KvState<D>& st, const u16* bc, int rc, const bf16x8 (&pb)[2],
                                              const bf16x8 (&db)[2], bf16x8 (&top)[kKvPf], const u16* bn, int rn,
                                              bf16x8 (&rop)[kKvPf], KvBlock& nx, const u16* xa, const u16* xb,
                                              const XchLane& xo, const bf16x8 (&kq)[8], f32x16& qa, f32x16& qb,
                                              int lane) {
  constexpr int NT = D / 16, NB = D / 32, NY = 2 * NT;
  static_assert(NY == 16, "16 dQ steps pair with the 16 dV / dK steps");
  bf16x8 xop[2];
  auto kv_step = [&](int j) {
    const bf16x8 a = top[j % kKvPf];
    if (j + kKvPf < NY) top[j % kKvPf] = kv_tr_operand<D>(bc, rc, j + kKvPf, lane);
    const int jj = j % NT;
    if (j < NT)
      kv_acc_mfma<D>(st.dvT[jj % NB], a, pb[jj / NB]);
    else
      kv_acc_mfma<D>(st.dkT[jj % NB], a, db[jj / NB]);
    if constexpr (NXT) {
      if (j >= NY - kKvPf) rop[j - (NY - kKvPf)] = kv_row_operand<D>(bn, rn, j - (NY - kKvPf), lane);
      if (j >= NY - 8 && j < NY - 4) kv_init_dp<D>(nx, bn, rn, j - (NY - 8), lane >> 5);
      if (j >= NY - 4) kv_init_s<D>(nx, bn, rn, j - (NY - 4), lane >> 5);
    }
    step_fence();
  };
  auto dq_step = [&](int u) {
    const bf16x8 a = xop[u & 1];
    if (u + 2 < 16) xop[u & 1] = xch_operand(((u + 2) & 1) ? xb : xa, xo, (u + 2) >> 1);
    f32x16& acc = (u & 1) ? qb : qa;
    if (u < 2)
      dq_mfma_first(acc, a, kq[u >> 1]);
    else
      dq_mfma(acc, a, kq[u >> 1]);
    step_fence();
  };
  xop[0] = xch_operand(xa, xo, 0);
  xop[1] = xch_operand(xb, xo, 0);
  kv_step(0);
#pragma unroll
  for (int i = 1; i < NY; ++i) {
    kv_step(i);
    dq_step(i - 1);
  }
  dq_step(15);
}

// One workgroup per (sequence, head, 128-key tile); every wave walks the 64-query tiles
// from the workgroup's first (under causal, the one holding its first key) to the last.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kKvThreads, 1) void bwd_fused_bf16_kernel(BwdParams p) {
  static_assert(D == 128, "the fused backward is built for head_dim 128");
  constexpr int BK = kKvBK, BQ = kKvBQ, NS = D / 16, NB = D / 32;
  constexpr int S = kFzStages;
  using L = KvLds<D>;
  using Dma = TileDma<BQ, D, L::P, kKvWaves, true, 8, false>;  // statistics in the pads of Q rows 0..7
  constexpr int KVP = D + 8;  // row pitch of the staged K/V rows: conflict-free row reads
  // LDS: S tile buffers, then the four exchange tiles (E0[0], E0[1], E1[0], E1[1]). In the
  // prologue K is staged in buffer 2 and V over the exchange tiles (and beyond).
  constexpr int XOFF = S * L::BUF;
  constexpr int LDS_ELEMS = XOFF + (4 * kXTile > BK * KVP ? 4 * kXTile : BK * KVP);
  static_assert(BK * KVP <= L::BUF, "K is staged in one tile buffer");
  __shared__ __attribute__((aligned(16))) u16 lds[LDS_ELEMS];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;

  int bh, kt;
  xcd_tile_map(blockIdx.x, p.B * p.H, p.n_tiles, false, true, bh, kt);
  const int b = bh / p.H, h = bh % p.H;
  int start, len;
  if (VARLEN) {
    start = p.cu[b];
    len = p.cu[b + 1] - start;
  } else {
    start = b * p.N;
    len = p.N;
  }
  const int k0 = kt * BK;
  if (k0 >= len) return;

  const size_t stride = (size_t)p.H * D;
  const size_t base = ((size_t)start * p.H + h) * D;
  const u16* __restrict__ Qg = p.q + base;
  const u16* __restrict__ dOg = p.dout + base;

  const int wk0 = k0 + 32 * w;
  const int kj = wk0 + lr;
  const int kk = 32 * w + lr;  // this lane's key within the tile: its exchange row

  KvState<D> st;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    st.dvT[bb] = f32x16{};
    st.dkT[bb] = f32x16{};
  }

  const int qt_begin = CAUSAL ? k0 / BQ : 0;
  const int n_qt = (len + BQ - 1) / BQ;

  Dma tdma;
  tdma.init(stride, w, lane);
  auto bufp = [&](int qt) -> u16* { return lds + ((unsigned)(qt - qt_begin) % S) * L::BUF; };
  u16* const xch = lds + XOFF;
  auto e0 = [&](int qt) -> u16* { return xch + (qt & 1) * kXTile; };
  auto e1 = [&](int qt) -> u16* { return xch + (2 + (qt & 1)) * kXTile; };
  static_assert(BQ == 64 && kKvWaves == 4, "statistics copies assume 16 queries per wave");
  auto issue = [&](int qt) {
    u16* buf = bufp(qt);
    const int q0 = qt * BQ;
    tdma.issue(buf, Qg, q0, len, stride, w, lane);
    tdma.issue(buf + L::TSZ, dOg, q0, len, stride, w, lane, false);
#if __HIP_DEVICE_COMPILE__
    const int qq = min(q0 + lane, len - 1);
    const size_t si = stat_index<VARLEN>(p, b, h, start, qq);
    if ((lane >> 4) == w) {
      dma_lds_b32(p.mneg + si, buf + L::stat_pad(0, w) - 32 * w);
      dma_lds_b32(p.dvec + si, buf + L::stat_pad(1, w) - 32 * w);
    }
#endif
  };
  constexpr int CNT = 2 * Dma::PER_WAVE + 2;

  // Prologue: K rows through buffer 2, V rows through the exchange area, tiles qt_begin
  // and qt_begin + 1 into buffers 0 and 1.
  {
    TileDma<BK, D, KVP, kKvWaves> kvdma;
    kvdma.init(stride, w, lane);
    kvdma.issue(lds + 2 * L::BUF, p.k + base, k0, len, stride, w, lane);
    kvdma.issue(xch, p.v + base, k0, len, stride, w, lane);
  }
  issue(qt_begin);
  if (qt_begin + 1 < n_qt) {
    issue(qt_begin + 1);
    wait_vmem_count<CNT>();
  } else {
    wait_vmem();
  }
  lds_barrier();
  bf16x8 kq[8];  // K operands of the dQ product: head-dim column 32 w + lr, keys 16 s + ...
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int e = (32 * w + lr) * KVP + 16 * s + 8 * g;
    st.kf[s] = kj < len ? ld16(lds + 2 * L::BUF + e) : zero_bf16x8();
    const bf16x8 v = kj < len ? ld16(xch + e) : zero_bf16x8();
    st.vf[s] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, v) ^ 0x80008000u);
  }
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    bf16x8 x = lds_tr_operand(lds + 2 * L::BUF, KVP, 16 * s, 32 * w, lane);
    if (k0 + BK > len) {  // the staged rows past the end repeat row len - 1: zero those keys
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k0 + 16 * s + 4 * g + (e & 3) + 8 * (e >> 2) >= len) x[e] = (__bf16)0.f;
    }
    kq[s] = to_agpr(x);
  }
  lds_barrier();
  // Every wave clears its own rows of the four exchange tiles (the slots of the tiles
  // before the first hold zeros, so the first dQ steps add nothing).
  {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<u32x4_t*>(xch + x * kXTile + (32 * w) * kXq + 8 * (64 * i + lane)) = u32x4_t{0u, 0u, 0u, 0u};
  }

  // dQ accumulator rows: query row n of this (sequence, head) is row stat_index(n). The
  // two blocks whose atomics are pending start as zeros aimed at valid rows.
  const uint32_t loff = (uint32_t)(4 * (4 * g * D + 32 * w + lr));
  auto grow = [&](int q0) -> const char* {
    return reinterpret_cast<const char*>(p.dqacc + stat_index<VARLEN>(p, b, h, start, max(q0, 0)) * D);
  };
  const XchLane xo = xch_lane_offsets(lane);
  f32x16 qa = f32x16{}, qb = f32x16{};

  KvBlock blk0, blk1;
  bf16x8 rop[kKvPf], top[kKvPf], pb[2], db[2];
  {
    const u16* bf = bufp(qt_begin);
#pragma unroll
    for (int j = 0; j < kKvPf; ++j) rop[j] = kv_row_operand<D>(bf, 0, j, lane);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      kv_init_s<D>(blk0, bf, 0, r4, g);
      kv_init_dp<D>(blk0, bf, 0, r4, g);
    }
    kv_phase_x<D, CAUSAL, true, false, false>(st, blk0, bf, 0, rop, blk1, pb, db, bf, 0, top, 0, kj, len, p.c, lane);
#pragma unroll
    for (int j = 0; j < kKvPf; ++j) rop[j] = kv_row_operand<D>(bf, 32, j, lane);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      kv_init_s<D>(blk1, bf, 32, r4, g);
      kv_init_dp<D>(blk1, bf, 32, r4, g);
    }
  }
  // (Keys past the end get finite -dS; their dQ terms vanish with the zeroed K operands,
  // and their dK, dV rows are not stored.)
  auto mask_of = [&](int q0) { return q0 + BQ > len || (CAUSAL && q0 < wk0 + 31); };

  auto tile_step = [&](int qt) {
    const u16* bc = bufp(qt);
    const u16* bn = bufp(qt + 1);
    const int q0 = qt * BQ;
    const bool mask = mask_of(q0);
    kv_x<D, CAUSAL>(true, true, mask, st, blk1, bc, 32, rop, blk0, pb, db, bc, 0, top, q0, kj, len, p.c, lane);
    xch_write(e0(qt), db, kk, g);
    wait_vmem();  // tile qt + 1 (the only copies in flight) and the atomics of the last tile
    lds_barrier();
    if (qt + S - 1 < n_qt) issue(qt + S - 1);
    fz_phase_y_atomics<D, true>(st, bc, 0, pb, db, top, bn, 0, rop, blk0, qa, grow(q0 - 96), qb, grow(q0 - 64),
                                loff, lane);
    kv_x<D, CAUSAL>(true, true, mask, st, blk0, bn, 0, rop, blk1, pb, db, bc, 32, top, q0 + 32, kj, len, p.c, lane);
    xch_write(e1(qt), db, kk, g);
    fz_phase_y_dq<D, true>(st, bc, 32, pb, db, top, bn, 32, rop, blk1, e1(qt - 1), e0(qt), xo, kq, qa, qb, lane);
  };
  for (int qt = qt_begin; qt < n_qt - 1; ++qt) tile_step(qt);
  {
    const int qt = n_qt - 1;
    const u16* bc = bufp(qt);
    const int q0 = qt * BQ;
    const bool mask = mask_of(q0);
    kv_x<D, CAUSAL>(true, true, mask, st, blk1, bc, 32, rop, blk0, pb, db, bc, 0, top, q0, kj, len, p.c, lane);
    xch_write(e0(qt), db, kk, g);
    lds_barrier();
    fz_phase_y_atomics<D, false>(st, bc, 0, pb, db, top, bc, 0, rop, blk0, qa, grow(q0 - 96), qb, grow(q0 - 64),
                                 loff, lane);
    kv_x<D, CAUSAL>(false, true, mask, st, blk0, bc, 0, rop, blk1, pb, db, bc, 32, top, q0 + 32, kj, len, p.c, lane);
    xch_write(e1(qt), db, kk, g);
    fz_phase_y_dq<D, false>(st, bc, 32, pb, db, top, bc, 32, rop, blk1, e1(qt - 1), e0(qt), xo, kq, qa, qb, lane);
  }
  const int ql = (n_qt - 1) * BQ;  // the last tile's first query

#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    kv_acc_fence<D>(st.dvT[bb]);
    kv_acc_fence<D>(st.dkT[bb]);
  }
  static_assert(kKvWaves * 64 * stage_pitch<D>() <= XOFF, "staging stays clear of the exchange tiles");
  lds_barrier();
  // The last block's dQ (its -dS was written after the last barrier of the loop).
  f32x16 qc;
  {
    const u16* xl = e1(n_qt - 1);
    bf16x8 xn = xch_operand(xl, xo, 0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 a = xn;
      if (s + 1 < 8) xn = xch_operand(xl, xo, s + 1);
      if (s == 0)
        dq_mfma_first(qc, a, kq[0]);
      else
        dq_mfma(qc, a, kq[s]);
    }
  }
  u16* stg = lds + w * 64 * stage_pitch<D>();
  stage_acc_rows<D>(stg, st.dkT, -p.scale, lr, g);
  stage_acc_rows<D>(stg + 32 * stage_pitch<D>(), st.dvT, 1.f, lr, g);
  agpr_acc_fence2(qa, qb);
  agpr_acc_fence(qc);
  {
    const char* ga = grow(ql - 32);
    const char* gb = grow(ql);
    const char* gc = grow(ql + 32);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      atomic_add_f32(ga + dq_row_bytes<D>(r), loff, qa[r]);
      atomic_add_f32(gb + dq_row_bytes<D>(r), loff, qb[r]);
      atomic_add_f32(gc + dq_row_bytes<D>(r), loff, qc[r]);
    }
  }
  const int valid = len - wk0;
  store_staged_rows<D, 32>(stg, p.dk + base + (size_t)wk0 * stride, stride, valid, lane);
  store_staged_rows<D, 32>(stg + 32 * stage_pitch<D>(), p.dv + base + (size_t)wk0 * stride, stride, valid, lane);
}

// dQ = -scale * (accumulator) as bf16 in the caller's layout, for 64 consecutive tokens
// of one (sequence, head) per workgroup (a packed batch is one sequence of total_tokens);
// 16 lanes per row, 8 values each: 512 contiguous bytes read and 256 written per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float* __restrict__ acc, u16* __restrict__ dq,
                                                             float mul, int H, int n_seq, int n_tiles) {
  constexpr int LPR = D / 8, RPP = 256 / LPR, PASSES = kPreTokens / RPP;
  const int h = blockIdx.x % H;
  const int tile = (blockIdx.x / H) % n_tiles;
  const int s = blockIdx.x / H / n_tiles;
  const int n0 = tile * kPreTokens;
  const int sub = threadIdx.x % LPR;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int n = n0 + ps * RPP + (int)threadIdx.x / LPR;
    if (n < n_seq) {
      const float* src = acc + (((size_t)s * H + h) * n_seq + n) * D + 8 * sub;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 c = *reinterpret_cast<const f32x4*>(src + 4);
      const f32x8 x = {a[0] * mul, a[1] * mul, a[2] * mul, a[3] * mul, c[0] * mul, c[1] * mul, c[2] * mul, c[3] * mul};
      *reinterpret_cast<bf16x8*>(dq + (((size_t)s * n_seq + n) * H + h) * D + 8 * sub) = to_bf16x8(x);
    }
  }
}

// ------------------------------------------------------------------------ bwd_dkdv, head_dim 64
//
// At head_dim 64 a block has half the matrix work of head_dim 128 against the same
// softmax arithmetic, and the dK/dV state fits in 256 registers, so two waves share each
// SIMD and overlap one another's vector and matrix work; this kernel does the blocks in
// order, without the cross-block pipeline of the head_dim-128 kernel. Each wave owns
// 32 keys; Q and dO tiles sit in LDS with padded rows (pitch_both), read row-wise for
// S and dP and through transpose reads for dV and dK; LSE and D are copied per tile.

// Queries per tile: 128 halves the barriers and copies per query; under causal masking
// 64, since the first tile of each key range is partly above the diagonal and a larger
// tile wastes more there (a per-block skip would break the interleaving of blocks).
template <bool CAUSAL> constexpr int rk_bq() { return CAUSAL ? 64 : 128; }
// LDS buffers in the query-tile pipeline: with three, the copies of the next two tiles
// are in flight while one is used (64-query tiles fit three times in LDS, 128 twice).
template <int BQ> constexpr int rk_stages() { return BQ == 64 ? 3 : 2; }

// One LDS buffer: Q and dO tiles (row-major; read both row-wise for S and dP and through
// transpose reads for dK and dV), then LSE and D per query (all copied in by DMA).
template <int D, int BQ>
struct RkLds {
  static constexpr int P = pitch_both<D>();
  static constexpr int TSZ = BQ * P;               // elements of one tile
  static constexpr int STAT = 2 * TSZ;             // u16 offset of the fp32 statistics
  static constexpr int BUF = 2 * TSZ + 4 * BQ;     // + lse and D (2 x BQ floats)
};

template <int D>
struct RkState {
  static constexpr int NB = D / 32, NS = D / 16;
  bf16x8 kf[NS], vf[NS];  // this lane's key and value rows as B operands
  f32x16 dvT[NB], dkT[NB];
};

// One query tile for one wave, one 32-query block at a time (keeps the live score
// registers to one block):
//   S = Q K^T and dP = dO V^T with one key per column: register r of lane group g
//   holds query q0 + 32a + crow_nat(r, g) against key kj;
//   P = exp2(c S - LSE log2e) (exact, normalised), dS = P (dP - D);
//   dV^T += dO^T P and dK^T += Q^T dS, whose A rows (head-dim entries) are read
//   transposed from the row-major tiles with k-slots queries 16t + 4g + {0..3, 8..11}.
template <int D, bool CAUSAL>
__device__ __forceinline__ void rk_tile(RkState<D>& st, const u16* buf, int q0, int kj, int len, bool mask,
                                          int lane, float c) {
  constexpr int BQ = rk_bq<CAUSAL>();
  using L = RkLds<D, BQ>;
  constexpr int NB = D / 32, NS = D / 16, NA = BQ / 32;
  constexpr int P = L::P;
  const u16* Qs = buf;
  const u16* dOs = buf + L::TSZ;
  const float* lse_s = reinterpret_cast<const float*>(buf + L::STAT);
  const float* dd_s = lse_s + BQ;
  const int lr = lane & 31, g = lane >> 5;

#pragma unroll
  for (int a = 0; a < NA; ++a) {
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
    {
      const int off = (32 * a + lr) * P + 8 * g;
      bf16x8 aq = ld16(Qs + off), ad = ld16(dOs + off);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        bf16x8 nq = aq, nd = ad;
        if (s + 1 < NS) {
          nq = ld16(Qs + off + 16 * (s + 1));
          nd = ld16(dOs + off + 16 * (s + 1));
        }
        sacc = mfma32(aq, st.kf[s], sacc);
        dpacc = mfma32(ad, st.vf[s], dpacc);
        aq = nq;
        ad = nd;
      }
    }
    // The transposed A operands of dV += P^T dO do not depend on the softmax arithmetic:
    // fetch them now, so that their LDS latency hides under it.
    bf16x8 aot[2 * NB];
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) aot[i] = lds_tr_operand(dOs, P, 32 * a + 16 * (i & 1), 32 * (i >> 1), lane);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int qrow = 32 * a + 8 * r4 + 4 * g;  // registers 4r4..4r4+3: queries qrow..qrow+3
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + qrow);
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc[4 * r4 + e] = fast_exp2(fmaf(sacc[4 * r4 + e], c, -l4[e] * kLog2e));
    }
    if (mask) {  // wave-uniform: a diagonal or tail tile; hide keys after their query
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qq = q0 + 32 * a + crow_nat(r, g);
        sacc[r] = (qq >= len || (CAUSAL && kj > qq)) ? 0.f : sacc[r];
      }
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(dd_s + 32 * a + 8 * r4 + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) dpacc[4 * r4 + e] = sacc[4 * r4 + e] * (dpacc[4 * r4 + e] - d4[e]);
    }
    const bf16x8 pb0 = to_bf16x8(half_of(sacc, 0)), pb1 = to_bf16x8(half_of(sacc, 1));
    // dV += P^T dO, fetching the transposed Q operands of dK += dS^T Q meanwhile.
    bf16x8 aqt[2 * NB];
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) {
      aqt[i] = lds_tr_operand(Qs, P, 32 * a + 16 * (i & 1), 32 * (i >> 1), lane);
      kv_acc_mfma<D>(st.dvT[i >> 1], aot[i], (i & 1) ? pb1 : pb0);
    }
    const bf16x8 ds0 = to_bf16x8(half_of(dpacc, 0)), ds1 = to_bf16x8(half_of(dpacc, 1));
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) kv_acc_mfma<D>(st.dkT[i >> 1], aqt[i], (i & 1) ? ds1 : ds0);
  }
}

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kKvThreads, 2) void bwd_dkdv_rows_kernel(BwdParams p) {
  constexpr int BK = kKvBK, BQ = rk_bq<CAUSAL>(), NT = kKvThreads;
  constexpr int NB = D / 32, NS = D / 16;
  using L = RkLds<D, BQ>;
  __shared__ __attribute__((aligned(16))) u16 buf0[L::BUF];
  __shared__ __attribute__((aligned(16))) u16 buf1[L::BUF];
  __shared__ __attribute__((aligned(16))) u16 buf2[rk_stages<BQ>() == 3 ? L::BUF : 8];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;

  // Workgroup -> (sequence, head, key tile), head-grouped per XCD (the head's Q and dO
  // stay in L2); under causal the first key tiles see the most queries and come first.
  int bh, kt;
  xcd_tile_map(blockIdx.x, p.B * p.H, p.n_tiles, false, true, bh, kt);
  const int b = bh / p.H, h = bh % p.H;
  int start, len;
  if (VARLEN) {
    start = p.cu[b];
    len = p.cu[b + 1] - start;
  } else {
    start = b * p.N;
    len = p.N;
  }
  const int k0 = kt * BK;
  if (k0 >= len) return;

  const size_t stride = (size_t)p.H * D;
  const size_t base = ((size_t)start * p.H + h) * D;
  const u16* __restrict__ Qg = p.q + base;
  const u16* __restrict__ dOg = p.dout + base;

  const int wk0 = k0 + 32 * w;  // first key of this wave
  const int kj = wk0 + lr;      // this lane's key

  RkState<D> st;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const size_t off = base + (size_t)kj * stride + 16 * s + 8 * g;
    st.kf[s] = kj < len ? ld16(p.k + off) : zero_bf16x8();
    st.vf[s] = kj < len ? ld16(p.v + off) : zero_bf16x8();
  }
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    st.dvT[bb] = f32x16{};
    st.dkT[bb] = f32x16{};
  }

  const int qt_begin = CAUSAL ? k0 / BQ : 0;
  const int n_qt = (len + BQ - 1) / BQ;

  TileDma<BQ, D, L::P, kKvWaves> tdma;
  tdma.init(stride, w, lane);
  // Every wave issues the same number of copies per tile (its share of the Q and dO
  // tiles, and one 64-row statistics copy: waves 0, 2 copy LSE, waves 1, 3 D; the
  // duplicates land the same bytes), so a wave can wait for "all but the newest tile"
  // with one vmcnt.
  static_assert(BQ % 64 == 0 && kKvWaves == 4, "statistics copies assume 64-row pieces and 4 waves");
  constexpr int CNT = 2 * TileDma<BQ, D, L::P, kKvWaves>::PER_WAVE + BQ / 64;
  auto issue = [&](int qt, u16* buf) {
    const int q0 = qt * BQ;
    tdma.issue(buf, Qg, q0, len, stride, w, lane);
    tdma.issue(buf + L::TSZ, dOg, q0, len, stride, w, lane);
#if __HIP_DEVICE_COMPILE__
    const float* src = (w & 1) ? p.dvec : p.lse;
    float* dst = reinterpret_cast<float*>(buf + L::STAT) + ((w & 1) ? BQ : 0);
#pragma unroll
    for (int j = 0; j < BQ / 64; ++j) {
      const int qq = min(q0 + 64 * j + lane, len - 1);  // rows past the end are masked in the tile
      dma_lds_b32(src + stat_index<VARLEN>(p, b, h, start, qq), dst + 64 * j);
    }
#endif
  };
  auto compute = [&](int qt, const u16* buf) {
    const int q0 = qt * BQ;
    // wave-uniform: skip tiles whose queries all precede this wave's keys
    if (wk0 < len && (!CAUSAL || q0 + BQ - 1 >= wk0)) {
      const bool mask = q0 + BQ > len || (CAUSAL && q0 < wk0 + 31);
      rk_tile<D, CAUSAL>(st, buf, q0, kj, len, mask, lane, p.c);
    }
  };
  if constexpr (rk_stages<BQ>() == 3) {
    // Three LDS buffers in turn. Stage t: wait until tile t has landed (tile t+1 may
    // still be in flight), barrier (every wave is past tile t-1 too), refill tile t-1's
    // buffer with tile t+2, compute tile t.
    auto wait_for = [&](int qt) {
      if (qt + 1 < n_qt)
        wait_vmem_count<CNT>();
      else
        wait_vmem();
    };
    issue(qt_begin, buf0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      settle(st.kf[s]);
      settle(st.vf[s]);
    }
    if (qt_begin + 1 < n_qt) issue(qt_begin + 1, buf1);
    for (int qt = qt_begin; qt < n_qt; qt += 3) {
      wait_for(qt);
      __syncthreads();
      if (qt + 2 < n_qt) issue(qt + 2, buf2);
      compute(qt, buf0);
      if (qt + 1 >= n_qt) break;
      wait_for(qt + 1);
      __syncthreads();
      if (qt + 3 < n_qt) issue(qt + 3, buf0);
      compute(qt + 1, buf1);
      if (qt + 2 >= n_qt) break;
      wait_for(qt + 2);
      __syncthreads();
      if (qt + 4 < n_qt) issue(qt + 4, buf1);
      compute(qt + 2, buf2);
    }
  } else {
    // Two LDS buffers in turn: the copy of the next query tile is in flight while the
    // current one is used.
    issue(qt_begin, buf0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      settle(st.kf[s]);
      settle(st.vf[s]);
    }
    wait_vmem();
    __syncthreads();
    for (int qt = qt_begin; qt < n_qt; qt += 2) {
      if (qt + 1 < n_qt) issue(qt + 1, buf1);
      compute(qt, buf0);
      wait_vmem();
      __syncthreads();
      if (qt + 1 >= n_qt) break;
      if (qt + 2 < n_qt) issue(qt + 2, buf0);
      compute(qt + 1, buf1);
      wait_vmem();
      __syncthreads();
    }
  }

#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    kv_acc_fence<D>(st.dvT[bb]);
    kv_acc_fence<D>(st.dkT[bb]);
  }
  // buf0 stages this wave's dK rows, then its dV rows, so that they leave as whole rows;
  // the three-buffer loop leaves right after its last tile, so every wave must be past
  // its reads of the tiles first.
  static_assert(kKvWaves * 32 * stage_pitch<D>() <= L::BUF, "staging fits in one tile buffer");
  lds_barrier();
  u16* stg = buf0 + w * 32 * stage_pitch<D>();
  const int valid = len - wk0;
  stage_acc_rows<D>(stg, st.dkT, p.scale, lr, g);
  store_staged_rows<D, 32>(stg, p.dk + base + (size_t)wk0 * stride, stride, valid, lane);
  stage_acc_rows<D>(stg, st.dvT, 1.f, lr, g);
  store_staged_rows<D, 32>(stg, p.dv + base + (size_t)wk0 * stride, stride, valid, lane);
}

// ------------------------------------------------------------------------ bwd_dq

constexpr int kDqWaves = 4;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqBR = 32 * kDqWaves;  // queries per workgroup
constexpr int kDqBC = 64;             // keys per tile

// One double-buffered half: K (read row-wise for S^T and transposed for dQ) and V
// (row-wise for dP^T), both swizzled tiles (conflict-free both ways; one layout for both
// lets a single set of copy offsets serve K and V; the pads are unused).
template <int D>
struct DqLds {
  static constexpr int KP = swz_pitch<D>();
  static constexpr int VP = swz_pitch<D>();
  static constexpr int KSZ = kDqBC * KP;
  static constexpr int BUF = KSZ + kDqBC * VP;
};

template <int D>
struct DqState {
  static constexpr int NB = D / 32, NS = D / 16;
  bf16x8 qf[NS], dof[NS];  // this lane's query and output-gradient rows as B operands
  f32x16 dqT[NB];
  float lse2;  // LSE * log2(e) of this lane's query (+inf past the end)
  float dd;    // D of this lane's query
};

// One key tile for one wave, one 32-key block at a time (keeps the live score
// registers to one block):
//   S^T = K Q^T and dP^T = V dO^T with one query per column: register r of lane group
//   g holds key k0 + 32j + crow_nat(r, g) against query qi;
//   P = exp2(c S - LSE log2e), dS = P (dP - D);
//   dQ^T += K^T dS^T, whose A rows (head-dim entries) are read transposed from the
//   (swizzled) K tile with k-slots keys 16t + 4g + {0..3, 8..11}.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_tile(DqState<D>& st, const u16* buf, int k0, int len, int qi, int lane,
                                        float c, bool mask) {
  constexpr int NB = D / 32, NS = D / 16, NJ = kDqBC / 32;
  const u16* Ks = buf;
  const u16* Vs = buf + DqLds<D>::KSZ;
  const int g = lane >> 5;

#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
    {
      bf16x8 ak = swz_row_operand<D>(Ks, 32 * j, 0, lane), av = swz_row_operand<D>(Vs, 32 * j, 0, lane);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        bf16x8 nk = ak, nv = av;
        if (s + 1 < NS) {
          nk = swz_row_operand<D>(Ks, 32 * j, s + 1, lane);
          nv = swz_row_operand<D>(Vs, 32 * j, s + 1, lane);
        }
        sacc = mfma32(ak, st.qf[s], sacc);
        dpacc = mfma32(av, st.dof[s], dpacc);
        ak = nk;
        av = nv;
      }
    }
    // the dQ products' first two K operands, read while the softmax below runs
    bf16x8 ta[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) ta[i] = swz_tr_operand<D>(Ks, 32 * j + 16 * (i / NB), 32 * (i % NB), lane);
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(fmaf(sacc[r], c, -st.lse2));
    if (mask) {  // wave-uniform: a diagonal or tail tile
      // hidden: keys past the last one this query sees (one compare per score)
      const int lim = (CAUSAL ? min(qi, len - 1) : len - 1) - k0 - 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 32 * j + crow_nat(r, 0) > lim ? 0.f : sacc[r];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) dpacc[r] = sacc[r] * (dpacc[r] - st.dd);
    const bf16x8 ds0 = to_bf16x8(half_of(dpacc, 0)), ds1 = to_bf16x8(half_of(dpacc, 1));
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) {
      const int bb = i % NB, h = i / NB;
      const bf16x8 a = ta[i % 2];
      if (i + 2 < 2 * NB) ta[i % 2] = swz_tr_operand<D>(Ks, 32 * j + 16 * ((i + 2) / NB), 32 * ((i + 2) % NB), lane);
      st.dqT[bb] = mfma32(a, h ? ds1 : ds0, st.dqT[bb]);
    }
  }
}

// One query tile of one (sequence, head) of the dQ pass. The two LDS buffers are free
// again when it returns (its last step ends in a barrier).
// Sum of the elementwise products of eight bf16 pairs, in fp32.
__device__ __forceinline__ float dot8_bf16(const bf16x8& x, const bf16x8& y, float acc) {
  const u32x4 a = __builtin_bit_cast(u32x4, x), b = __builtin_bit_cast(u32x4, y);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(__uint_as_float(a[i] << 16), __uint_as_float(b[i] << 16), acc);
    acc = fmaf(__uint_as_float(a[i] & 0xffff0000u), __uint_as_float(b[i] & 0xffff0000u), acc);
  }
  return acc;
}

// One query tile of the dQ pass. With STATS the tile also forms its queries' row
// statistics, D_i = sum_k dO_ik O_ik (from the stored O, whose row the lane pair loads
// beside dO) and -LSE_i / scale, and writes both to the workspace for the dK/dV kernel
// that runs next: every query row belongs to exactly one tile, so the separate
// statistics pass is not needed.
template <int D, bool CAUSAL, bool VARLEN, bool STATS, bool DESC = false>
__device__ __forceinline__ void dq_qtile(const BwdParams& p, int b, int h, int start, int len, int qt, u16* buf0,
                                         u16* buf1) {
#if __HIP_DEVICE_COMPILE__
  constexpr int BR = kDqBR, BC = kDqBC;
  constexpr int NB = D / 32, NS = D / 16;
  using L = DqLds<D>;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int q0 = qt * BR;

  const size_t stride = (size_t)p.H * D;
  const size_t base = ((size_t)start * p.H + h) * D;
  const u16* __restrict__ Kg = p.k + base;
  const u16* __restrict__ Vg = p.v + base;

  const int wq0 = q0 + 32 * w;
  const int qi = wq0 + lr;
  const int wq_last = min(wq0 + 31, len - 1);

  DqState<D> st;
  const int kv_end = CAUSAL ? min(q0 + BR, len) : len;
  const int n_kt = (kv_end + BC - 1) / BC;

  static_assert(L::KP == L::VP, "K and V tiles share their copy offsets");
  TileDma<BC, D, L::KP, kDqWaves, true> kvdma;
  kvdma.init(stride, w, lane);
  // Step i visits key tile i, or with DESC tile n_kt - 1 - i (the sum over key tiles
  // does not depend on their order).
  auto tile_at = [&](int i) { return DESC ? n_kt - 1 - i : i; };
  auto issue = [&](int i, u16* buf) {
    const int kt = tile_at(i);
    kvdma.issue(buf, Kg, kt * BC, len, stride, w, lane);
    kvdma.issue(buf + L::KSZ, Vg, kt * BC, len, stride, w, lane);
  };
  auto compute = [&](int i, const u16* buf) {
    const int k0 = tile_at(i) * BC;
    if (wq0 < len && (!CAUSAL || k0 <= wq_last)) {
      const bool mask = k0 + BC > len || (CAUSAL && k0 + BC - 1 > wq0);
      dq_tile<D, CAUSAL>(st, buf, k0, len, qi, lane, p.c, mask);
    }
  };

  // The tile's Q and dO rows (and for the statistics O's) come in through the LDS
  // buffers as whole-row copies: loaded straight into registers, every load instruction
  // would gather 32 bytes from each of 32 rows. The first barrier lets every wave finish
  // reading the previous query tile's staged dQ rows out of buf1.
  constexpr int QP = D + 8;  // row pitch of the staged rows: conflict-free row reads
  static_assert(BR * QP <= L::BUF, "a query tile's rows fit in one buffer");
  const int er = (32 * w + lr) * QP + 8 * g;  // this lane's row, head-dim 8 g
  TileDma<BR, D, QP, kDqWaves> rdma;
  rdma.init(stride, w, lane);
  __syncthreads();
  rdma.issue(buf1, p.q + base, q0, len, stride, w, lane);
  rdma.issue(buf0, p.dout + base, q0, len, stride, w, lane);
  const float lse = qi < len ? p.lse[stat_index<VARLEN>(p, b, h, start, qi)] : INFINITY;
  if constexpr (!STATS) st.dd = qi < len ? p.dvec[stat_index<VARLEN>(p, b, h, start, qi)] : 0.f;
  wait_vmem();
  __syncthreads();
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    st.qf[s] = qi < len ? ld16(buf1 + er + 16 * s) : zero_bf16x8();
    st.dof[s] = qi < len ? ld16(buf0 + er + 16 * s) : zero_bf16x8();
  }
  st.lse2 = lse * kLog2e;
  __syncthreads();  // both buffers read
  issue(0, buf0);
  if constexpr (STATS) rdma.issue(buf1, p.o + base, q0, len, stride, w, lane);
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) st.dqT[bb] = f32x16{};
  wait_vmem();
  __syncthreads();
  if constexpr (STATS) {
    // lanes l and l ^ 32 hold the two halves of the row (head-dim 16 s + 8 g + 0..7)
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 o8 = qi < len ? ld16(buf1 + er + 16 * s) : zero_bf16x8();
      part = dot8_bf16(st.dof[s], o8, part);
    }
    st.dd = pair_sum(part);
    if (g == 0 && qi < len) {
      const size_t si = stat_index<VARLEN>(p, b, h, start, qi);
      p.dvec_out[si] = st.dd;
      p.mneg_out[si] = -lse / p.scale;
    }
    __syncthreads();  // O read out of buf1 before tile 1 is copied there
  }
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

  // The tiles are consumed (the loop ends on a barrier): buf1 stages this wave's dQ rows
  // so that they leave as whole rows (a workgroup's next query tile copies into the
  // buffers only after its first barrier).
  static_assert(4 * 32 * stage_pitch<D>() <= L::BUF, "staging fits in one tile buffer");
  u16* stg = buf1 + w * 32 * stage_pitch<D>();
  stage_acc_rows<D>(stg, st.dqT, p.scale, lr, g);
  store_staged_rows<D, 32>(stg, p.dq + base + (size_t)wq0 * stride, stride, len - wq0, lane);
#endif
}

// Two workgroups per compute unit (two waves per SIMD) keep the matrix pipe busy while
// the other wave waits on LDS or does its softmax arithmetic. Workgroup -> (sequence,
// head, slot) as in the forward: head-grouped per XCD; under causal masking slot i takes
// query tiles nt-1-i and i, so every workgroup visits the same number of key tiles, the
// second tile's keys in descending order (co-resident workgroups then read the same key
// tile at the same step; see the forward kernel).
template <int D, bool CAUSAL, bool VARLEN, bool STATS>
__global__ __launch_bounds__(kDqThreads, 2) void bwd_dq_bf16_kernel(BwdParams p) {
  using L = DqLds<D>;
  __shared__ __attribute__((aligned(16))) u16 buf0[L::BUF];
  __shared__ __attribute__((aligned(16))) u16 buf1[L::BUF];
  // The statistics form runs before bwd_dkdv and starts its work counters at zero.
  if (STATS && p.kvctr != nullptr && blockIdx.x == 0 && threadIdx.x < kKvCounters) p.kvctr[threadIdx.x] = 0;

  int bh, slot;
  xcd_tile_map(blockIdx.x, p.B * p.H, p.n_tiles, false, true, bh, slot);
  const int b = bh / p.H, h = bh % p.H;
  int start, len;
  if (VARLEN) {
    start = p.cu[b];
    len = p.cu[b + 1] - start;
  } else {
    start = b * p.N;
    len = p.N;
  }
  const int nt = (len + kDqBR - 1) / kDqBR;
  if (CAUSAL) {
    const int t_hi = nt - 1 - slot;
    if (t_hi < slot) return;
    dq_qtile<D, CAUSAL, VARLEN, STATS>(p, b, h, start, len, t_hi, buf0, buf1);
    if (slot < t_hi) dq_qtile<D, CAUSAL, VARLEN, STATS, true>(p, b, h, start, len, slot, buf0, buf1);
  } else {
    if (slot >= nt) return;
    dq_qtile<D, CAUSAL, VARLEN, STATS>(p, b, h, start, len, slot, buf0, buf1);
  }
}

// ------------------------------------------------------------------------ launch

// Compute units of the current device (cached per device).
int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

BwdParams make_params(const Problem& pr) {
  BwdParams p;
  p.q = static_cast<const u16*>(pr.q);
  p.k = static_cast<const u16*>(pr.k);
  p.v = static_cast<const u16*>(pr.v);
  p.o = static_cast<const u16*>(pr.o);
  p.dout = static_cast<const u16*>(pr.dout);
  p.lse = pr.lse;
  p.dvec = pr.dvec;
  p.mneg = pr.mneg;
  p.dvec_out = pr.dvec;
  p.mneg_out = pr.mneg;
  p.dqacc = pr.dqacc;
  p.kvctr = pr.kvctr;
  p.dq = static_cast<u16*>(pr.dq);
  p.dk = static_cast<u16*>(pr.dk);
  p.dv = static_cast<u16*>(pr.dv);
  p.cu = pr.cu_seqlens;
  p.B = pr.batch;
  p.H = pr.heads;
  p.N = pr.seqlen;
  p.T = pr.total_tokens;
  p.n_tiles = 0;
  p.scale = pr.scale;
  p.c = pr.scale * kLog2e;
  return p;
}

template <int D, typename T>
hipError_t launch_pre_t(const Problem& pr) {
  // A packed batch is one sequence of total_tokens tokens.
  const int n_seqs = pr.cu_seqlens ? 1 : pr.batch;
  const int n_seq = pr.cu_seqlens ? pr.total_tokens : pr.seqlen;
  const int n_tiles = (n_seq + kPreTokens - 1) / kPreTokens;
  const dim3 grid((unsigned)((long long)n_tiles * n_seqs * pr.heads));
  hipLaunchKernelGGL((bwd_pre_kernel<D, T>), grid, dim3(256), 0, pr.stream, static_cast<const T*>(pr.o),
                     static_cast<const T*>(pr.dout), pr.lse, pr.dvec, pr.mneg, pr.dqacc, pr.kvctr, pr.scale, pr.heads,
                     n_seq, n_tiles);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_dkdv_t(const Problem& pr) {
  BwdParams p = make_params(pr);
  p.n_tiles = (pr.seqlen + kKvBK - 1) / kKvBK;
  const dim3 grid((unsigned)(p.n_tiles * pr.batch * pr.heads));
  if constexpr (D == 64) {
    hipLaunchKernelGGL((bwd_dkdv_rows_kernel<D, CAUSAL, VARLEN>), grid, dim3(kKvThreads), 0, pr.stream, p);
  } else {
    const int ncu = device_cu_count();
    const unsigned g = (unsigned)(ncu >= 8 ? ncu / 8 * 8 : 8);
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, CAUSAL, VARLEN>), dim3(g), dim3(kKvThreads), 0, pr.stream, p);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_fused_t(const Problem& pr) {
  if constexpr (D != 128) {
    return hipErrorInvalidValue;
  } else {
    BwdParams p = make_params(pr);
    p.n_tiles = (pr.seqlen + kKvBK - 1) / kKvBK;
    const dim3 grid((unsigned)(p.n_tiles * pr.batch * pr.heads));
    hipLaunchKernelGGL((bwd_fused_bf16_kernel<D, CAUSAL, VARLEN>), grid, dim3(kKvThreads), 0, pr.stream, p);
    return hipGetLastError();
  }
}

template <int D>
hipError_t launch_convert_t(const Problem& pr) {
  const int n_seqs = pr.cu_seqlens ? 1 : pr.batch;
  const int n_seq = pr.cu_seqlens ? pr.total_tokens : pr.seqlen;
  const int n_tiles = (n_seq + kPreTokens - 1) / kPreTokens;
  const dim3 grid((unsigned)((long long)n_tiles * n_seqs * pr.heads));
  hipLaunchKernelGGL((bwd_dq_convert_kernel<D>), grid, dim3(256), 0, pr.stream, pr.dqacc, static_cast<u16*>(pr.dq),
                     -pr.scale, pr.heads, n_seq, n_tiles);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN, bool STATS>
hipError_t launch_dq_any(const Problem& pr) {
  BwdParams p = make_params(pr);
  const int n_qtiles = (pr.seqlen + kDqBR - 1) / kDqBR;
  p.n_tiles = CAUSAL ? (n_qtiles + 1) / 2 : n_qtiles;  // workgroup slots per (sequence, head)
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, CAUSAL, VARLEN, STATS>),
                     dim3((unsigned)(p.n_tiles * pr.batch * pr.heads)), dim3(kDqThreads), 0, pr.stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_dq_t(const Problem& pr) { return launch_dq_any<D, CAUSAL, VARLEN, false>(pr); }

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_dq_stats_t(const Problem& pr) { return launch_dq_any<D, CAUSAL, VARLEN, true>(pr); }

}  // namespace

hipError_t launch_bwd_pre(const Problem& pr, bool fp32) {
  if (fp32) return pr.head_dim == 64 ? launch_pre_t<64, float>(pr) : launch_pre_t<128, float>(pr);
  return pr.head_dim == 64 ? launch_pre_t<64, u16>(pr) : launch_pre_t<128, u16>(pr);
}

hipError_t launch_bwd_dkdv_bf16(const Problem& p) { FA_DISPATCH(launch_dkdv_t, p); }

hipError_t launch_bwd_dq_bf16(const Problem& p) { FA_DISPATCH(launch_dq_t, p); }

hipError_t launch_bwd_dq_stats_bf16(const Problem& p) { FA_DISPATCH(launch_dq_stats_t, p); }

hipError_t launch_bwd_fused_bf16(const Problem& p) {
  if (p.head_dim != 128) return hipErrorInvalidValue;
  FA_DISPATCH(launch_fused_t, p);
}

hipError_t launch_bwd_dq_convert(const Problem& p) {
  return p.head_dim == 64 ? launch_convert_t<64>(p) : launch_convert_t<128>(p);
}

}  // namespace fa
