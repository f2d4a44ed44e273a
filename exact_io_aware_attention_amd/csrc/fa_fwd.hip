// fa_fwd.hip - forward pass of exact attention, bf16 tensors, fp32 arithmetic (gfx950).
//
// One workgroup per (sequence, head, query tile), so one head is spread over many
// compute units ("FlashAttention-2 (PT)", "2. Paralelismo aprimorado"). Four waves;
// each wave owns one block of 32 query rows whose Q fragments stay in registers for
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
// division by l happens once at the end; and the output is rescaled only when a key
// block's exponentials, formed under the current reference maximum, would grow too
// large (a lane's share of a row sum above 2^8; until then nothing overflows and O and
// l keep one common reference, which is all exactness needs).
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
  int n_slots;  // workgroups per (sequence, head)
  float scale;
  float c;  // scale * log2(e)
};

// Four waves per workgroup, one 32-query block per wave. Workgroups per compute unit:
// two at head_dim 128 (256 registers per wave), three at 64, whose Q and O fragments
// fit 168. (Two query blocks per wave at one wave per SIMD, which halves the LDS reads
// per MFMA, measured 6-23 % slower at head_dim 64: no other wave covers the waits
// between the score MFMAs, the softmax and P.V.)
constexpr int kFwdWaves = 4;
template <int D> constexpr int fwd_occupancy() { return D == 64 ? 3 : 2; }
constexpr int kFwdBC = 64;        // keys per tile
constexpr float kKeepSum = 256.f;  // 2^8: bound on a lane's share of a block's row sum

template <int D>
struct FwdLds {
  static constexpr int KP = pitch_rows<D>();  // K: read row-wise (A operand of S^T)
  static constexpr int VP = pitch_tr<D>();    // V: read with transpose reads (A of O^T)
  static constexpr int KSZ = kFwdBC * KP;
  static constexpr int VSZ = kFwdBC * VP;
  static constexpr int BUF = KSZ + VSZ;
};

template <int D>
struct FwdState {
  static constexpr int NB = D / 32;
  bf16x8 qf[D / 16];
  f32x16 oacc[NB];
  float m_run;  // reference maximum of the raw scores q.k of this lane's query
  float l_run;  // this lane's share of sum_j exp2(c * (s_j - m_run))
};

// The tile loop is software-pipelined by hand. A 64-key tile is two 32-key blocks, and
// under the lazy rescale each block's softmax update stands on its own, so the
// exponentials of one block run while the matrix pipe works on the other:
//   S_0 | S_1 with exp(S_0) | P_0 V_0 with exp(S_1) | P_1 V_1
// Operand reads run kFwdPf steps ahead of the MFMA that uses them, across the phase
// boundaries, and a scheduling barrier (step_fence) closes every step, so the compiler
// neither sinks a read next to its use (exposing the LDS latency) nor hoists all of
// them (a register per read).

constexpr int kFwdPf = 3;

// K operand of S step s for key block j: row 32j + lane % 32 of the tile, head-dim
// entries 16s + 8(lane / 32) + 0..7.
template <int D>
__device__ __forceinline__ bf16x8 fwd_k_operand(const u16* Ks, int j, int s, int lane) {
  return ld16(Ks + (32 * j + (lane & 31)) * FwdLds<D>::KP + 8 * (lane >> 5) + 16 * s);
}

// V^T operand of PV step (bb, t): head-dim block bb, key slice 16t..16t+15 of the tile;
// its k-slots are keys 16t + 4g + {0..3, 8..11}, matching the registers of P.
template <int D>
__device__ __forceinline__ bf16x8 fwd_v_operand(const u16* Vs, int bb, int t, int lane) {
  return lds_tr_operand(Vs, FwdLds<D>::VP, 16 * t, 32 * bb, lane);
}

// ---- The row-sum check instead of row maxima.
// The exponentials of a 32-key block are formed under the current reference without
// looking for the block's maximum first, and kept when every lane's share of each row sum
// is at most 2^8: then so is every single P, whatever the block's true maximum, which is
// all the lazy rescale needs (O and l on one common reference, nothing overflows).
// Only before a query's first visible key, or when the check fails, does the reference
// move to the block's exact maximum and the exponentials get formed again. The row sums
// are formed anyway, so the common case trades a 16-value maximum, a lane swap and a
// serial section per block for one compare.

__device__ __forceinline__ float row_max16(const f32x16& x) {
  float mx = x[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
  return mx;
}

// Hide the scores of block j (keys kb0 .. kb0 + 31) that the query does not see.
template <bool CAUSAL>
__device__ __forceinline__ void fwd_mask(f32x16& sj, int kb0, int len, int wq0, int lane) {
  const int qi = wq0 + (lane & 31), g = lane >> 5;
  // Key kb0 + crow_nat(r, g) is hidden when it lies past the last key this query sees
  // (the sequence's last, and under causal masking the query's own position): one
  // compare of the register's lane-independent row offset against a per-lane bound.
  const int last = CAUSAL ? min(qi, len - 1) : len - 1;
  const int lim = last - kb0 - 4 * g;
#pragma unroll
  for (int r = 0; r < 16; ++r) sj[r] = crow_nat(r, 0) > lim ? -INFINITY : sj[r];
}

// Exponential r of the block (the raw scores stay), its share of the row sum and, every
// eighth, the bf16 conversion of eight of them into P.
__device__ __forceinline__ void fwd_exp_one(const f32x16& sj, f32x8& ev, bf16x8 (&pj)[2], float (&ls)[4], float nb,
                                             float c, int r) {
  float e = fast_exp2(fmaf(sj[r], c, nb));
  // Pin the exponential (and below the conversion) to this step: the compiler would sink
  // them out of the matrix-pipe phase they are meant to overlap.
  asm volatile("" : "+v"(e));
  ev[r & 7] = e;
  // the first four start the partial sums (0 + e would cost an add: e may be -0)
  if (r < 4)
    ls[r & 3] = e;
  else
    ls[r & 3] += e;
  if (r % 8 == 7) {
    pj[r / 8] = to_bf16x8(ev);
    asm volatile("" : "+v"(pj[r / 8]));
  }
}

// Whether the block's exponentials stand (see above); decided for the whole wave.
__device__ __forceinline__ bool fwd_keep(float m_run, const f32x16& sj, float bsum) {
  bool redo = !(bsum <= kKeepSum);
  if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0)  // before some query's first visible key
    redo |= m_run == -INFINITY && row_max16(sj) > -INFINITY;
  return __builtin_amdgcn_ballot_w64(redo) == 0;
}

// The uncommon path: the reference moves to the block's exact row maximum, l and O
// (which holds only products formed under the old reference) are scaled to match, and
// the block's exponentials are formed again.
template <int D>
__device__ __forceinline__ void fwd_redo(FwdState<D>& st, const f32x16& sj, bf16x8 (&pj)[2], float& bsum, float c) {
  const float m_new = fmaxf(st.m_run, pair_max(row_max16(sj)));
  const float m_to = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = fast_exp2((st.m_run - m_to) * c);
  st.m_run = m_new;
  st.l_run *= alpha;
#pragma unroll
  for (int bb = 0; bb < D / 32; ++bb) st.oacc[bb] *= alpha;
  const float nb = -m_to * c;
  f32x8 ev;
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    ev[r & 7] = fast_exp2(fmaf(sj[r], c, nb));
    sum = r == 0 ? ev[0] : sum + ev[r & 7];
    if (r % 8 == 7) pj[r / 8] = to_bf16x8(ev);
  }
  bsum = sum;
}

// One key tile for one wave: S^T = K Q^T, softmax update, O^T += V^T P^T.
template <int D, bool CAUSAL>
__device__ __forceinline__ void fwd_tile(FwdState<D>& st, const u16* Ks, const u16* Vs, int k0, int len, int wq0,
                                         int lane, float c, bool mask) {
  constexpr int NS = D / 16, NB = D / 32;
  constexpr int TP = 2 * NB;  // PV steps per key block
  constexpr int NSTEP = 2 * NS + 2 * TP;
  static_assert(16 % NS == 0 && 16 % TP == 0, "exponentials must split evenly over the steps");
  // The tile's 2 NS + 2 TP MFMA operands from LDS, in step order (S_0, S_1, P_0 V_0,
  // P_1 V_1) as one stream read kFwdPf steps ahead across the phase boundaries, so that
  // no phase starts by waiting for its first reads.
  auto op = [&](int n) {
    if (n < NS) return fwd_k_operand<D>(Ks, 0, n, lane);
    if (n < 2 * NS) return fwd_k_operand<D>(Ks, 1, n - NS, lane);
    if (n < 2 * NS + TP) return fwd_v_operand<D>(Vs, (n - 2 * NS) % NB, (n - 2 * NS) / NB, lane);
    return fwd_v_operand<D>(Vs, (n - 2 * NS - TP) % NB, 2 + (n - 2 * NS - TP) / NB, lane);
  };
  bf16x8 ring[kFwdPf];
#pragma unroll
  for (int n = 0; n < kFwdPf; ++n) ring[n] = op(n);
  auto next = [&](int n) {
    const bf16x8 a = ring[n % kFwdPf];
    if (n + kFwdPf < NSTEP) ring[n % kFwdPf] = op(n + kFwdPf);
    return a;
  };
  f32x16 s0 = f32x16{}, s1 = f32x16{};
  // S_0
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bf16x8 a = next(s);
    s0 = mfma32(a, st.qf[s], s0);
    step_fence();
  }
  if (mask) fwd_mask<CAUSAL>(s0, k0, len, wq0, lane);  // wave-uniform: a diagonal or tail tile

  // S_1 with exp(S_0)
  bf16x8 p0[2], p1[2];
  f32x8 ev;
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
  float nb = st.m_run == -INFINITY ? 0.f : -st.m_run * c;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bf16x8 a = next(NS + s);
    s1 = mfma32(a, st.qf[s], s1);
#pragma unroll
    for (int u = 0; u < 16 / NS; ++u) fwd_exp_one(s0, ev, p0, ls, nb, c, s * (16 / NS) + u);
    step_fence();
  }
  float bsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
  if (!fwd_keep(st.m_run, s0, bsum)) fwd_redo<D>(st, s0, p0, bsum, c);
  st.l_run += bsum;
  if (mask) fwd_mask<CAUSAL>(s1, k0 + 32, len, wq0, lane);

  // P_0 V_0 with exp(S_1). If block 1 then moves the reference, P_0 (formed under the
  // old one) has joined O already and is scaled with the rest of it. Step i accumulates
  // output block i % NB over key half i / NB: consecutive MFMAs never share an
  // accumulator, so none waits for the result of the one before it.
  ls[0] = ls[1] = ls[2] = ls[3] = 0.f;
  nb = st.m_run == -INFINITY ? 0.f : -st.m_run * c;
#pragma unroll
  for (int i = 0; i < TP; ++i) {
    const bf16x8 a = next(2 * NS + i);
    st.oacc[i % NB] = mfma32(a, p0[i / NB], st.oacc[i % NB]);
#pragma unroll
    for (int u = 0; u < 16 / TP; ++u) fwd_exp_one(s1, ev, p1, ls, nb, c, i * (16 / TP) + u);
    step_fence();
  }
  bsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
  if (!fwd_keep(st.m_run, s1, bsum)) fwd_redo<D>(st, s1, p1, bsum, c);
  st.l_run += bsum;

  // P_1 V_1
#pragma unroll
  for (int i = 0; i < TP; ++i) {
    const bf16x8 a = next(2 * NS + TP + i);
    st.oacc[i % NB] = mfma32(a, p1[i / NB], st.oacc[i % NB]);
    step_fence();
  }
}

// One query tile of one (sequence, head): the key loop and the epilogue. The two LDS
// buffers are free again when it returns (its last step ends in a barrier).
template <int D, bool CAUSAL, bool VARLEN, bool DESC = false>
__device__ __forceinline__ void fwd_qtile(const FwdParams& p, int b, int h, int start, int len, int qt, u16* buf0,
                                          u16* buf1) {
#if __HIP_DEVICE_COMPILE__
  constexpr int NW = kFwdWaves;
  constexpr int BR = 32 * NW, BC = kFwdBC;
  constexpr int NB = D / 32, NS = D / 16;
  using L = FwdLds<D>;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int q0 = qt * BR;

  const size_t stride = (size_t)p.H * D;
  const size_t base = ((size_t)start * p.H + h) * D;
  const u16* __restrict__ Qg = p.q + base;
  const u16* __restrict__ Kg = p.k + base;
  const u16* __restrict__ Vg = p.v + base;

  const int wq0 = q0 + 32 * w;  // first query row of this wave
  const int wq_last = min(wq0 + 31, len - 1);

  FwdState<D> st;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) st.oacc[bb] = f32x16{};
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  const int kv_end = CAUSAL ? min(q0 + BR, len) : len;
  const int n_kt = (kv_end + BC - 1) / BC;

  TileDma<BC, D, L::KP, NW> kdma;
  TileDma<BC, D, L::VP, NW> vdma;
  kdma.init(stride, w, lane);
  vdma.init(stride, w, lane);
  // Step i of the key loop visits key tile i, or with DESC tile n_kt - 1 - i: the
  // online softmax combines the blocks in any order.
  auto tile_at = [&](int i) { return DESC ? n_kt - 1 - i : i; };
  auto issue = [&](int i, u16* buf) {
    const int kt = tile_at(i);
    kdma.issue(buf, Kg, kt * BC, len, stride, w, lane);
    vdma.issue(buf + L::KSZ, Vg, kt * BC, len, stride, w, lane);
  };
  auto compute = [&](int i, const u16* buf) {
    const int k0 = tile_at(i) * BC;
    // wave-uniform: skip tiles that are entirely masked for this wave
    if (wq0 < len && (!CAUSAL || k0 <= wq_last)) {
      const bool mask = k0 + BC > len || (CAUSAL && k0 + BC - 1 > wq0);
      fwd_tile<D, CAUSAL>(st, buf, buf + L::KSZ, k0, len, wq0, lane, p.c, mask);
    }
  };
  // The tile's Q rows come in through buf1 (whole-row copies; loaded straight into
  // registers, every load instruction would gather 32 bytes from each of 32 rows) while
  // K/V tile 0 lands in buf0; every wave takes its rows before tile 1 refills buf1.
  // The first barrier lets every wave finish reading the previous query tile's O rows
  // out of buf1.
  {
    constexpr int QP = D + 8;  // row pitch of the staged Q rows: conflict-free row reads
    static_assert(BR * QP <= L::BUF, "the Q tile fits in one buffer");
    __syncthreads();
    TileDma<BR, D, QP, NW> qdma;
    qdma.init(stride, w, lane);
    qdma.issue(buf1, Qg, q0, len, stride, w, lane);
    issue(0, buf0);
    wait_vmem();
    __syncthreads();
    const int qi = wq0 + lr;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      st.qf[s] = qi < len ? ld16(buf1 + (32 * w + lr) * QP + 16 * s + 8 * g) : zero_bf16x8();
    __syncthreads();
  }
  // Two LDS buffers in turn: the copy of tile kt+1 is in flight while tile kt is used.
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

  // The tiles being consumed (the loop ends on a barrier), buf1 stages O so that its rows
  // leave whole (buf1, since a workgroup's next query tile starts by copying into buf0;
  // its first barrier comes after these reads).
  static_assert(NW * 32 * stage_pitch<D>() <= L::BUF, "staging fits in one tile buffer");
  u16* stg = buf1 + w * 32 * stage_pitch<D>();
  const int qi = wq0 + lr;
  const float l_tot = pair_sum(st.l_run);
  stage_acc_rows<D>(stg, st.oacc, 1.f / l_tot, lr, g);
  store_staged_rows<D, 32>(stg, p.o + base + (size_t)wq0 * stride, stride, len - wq0, lane);
  if (g == 0 && qi < len) {
    const size_t li = VARLEN ? (size_t)h * p.T + start + qi : ((size_t)b * p.H + h) * p.N + qi;
    p.lse[li] = st.m_run * p.scale + logf(l_tot);
  }
#endif
}

// Workgroup -> (sequence, head, slot): head-grouped per XCD, so the workgroups
// resident on one XCD share few heads and stream the same K/V rows through its L2 (this
// keeps the fabric traffic near the O(N d) operand bytes at long sequences). Without
// masking a slot is one query tile; under causal masking tile t visits t + 1 key tiles,
// so slot i takes tiles nt-1-i and i and every workgroup does the same work. The first
// tile walks the keys upwards from 0, the second downwards from its diagonal: workgroup
// i reaches its second tile after nt - i steps and key tile j of it at step nt - j, the
// same step for every workgroup, so at any moment the co-resident workgroups of a head
// read two key tiles between them (one in each direction) and the head's K/V passes
// through L2 about once, however long the sequence.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(64 * kFwdWaves, fwd_occupancy<D>()) void fwd_bf16_kernel(FwdParams p) {
  constexpr int BR = 32 * kFwdWaves;
  using L = FwdLds<D>;
  __shared__ __attribute__((aligned(16))) u16 buf0[L::BUF];
  __shared__ __attribute__((aligned(16))) u16 buf1[L::BUF];

  int bh, slot;
  xcd_tile_map(blockIdx.x, p.B * p.H, p.n_slots, false, true, bh, slot);
  const int b = bh / p.H, h = bh % p.H;
  int start, len;
  if (VARLEN) {
    start = p.cu[b];
    len = p.cu[b + 1] - start;
  } else {
    start = b * p.N;
    len = p.N;
  }
  const int nt = (len + BR - 1) / BR;
  if (CAUSAL) {
    const int t_hi = nt - 1 - slot;
    if (t_hi < slot) return;
    fwd_qtile<D, CAUSAL, VARLEN>(p, b, h, start, len, t_hi, buf0, buf1);
    if (slot < t_hi) fwd_qtile<D, CAUSAL, VARLEN, true>(p, b, h, start, len, slot, buf0, buf1);
  } else {
    if (slot >= nt) return;
    fwd_qtile<D, CAUSAL, VARLEN>(p, b, h, start, len, slot, buf0, buf1);
  }
}

// ------------------------------------------------------------------------ decode
//
// Few new queries (seqlen_q <= 32, one MFMA column block) against a long key cache:
// the work is reading K and V once, so the key range is cut into splits and each split
// is one single-wave workgroup (two per compute unit, each with its own double-buffered
// LDS tiles), which runs the forward tile loop over its keys for all the queries at
// once. Each split leaves its O (normalised by its own sum, fp32) and logsumexp; a
// second kernel merges them with weights exp(lse_s - lse) ("Softmax en línea" in the AI
// Atlas summary: softmax blocks combine exactly through their maxima and sums). Causal
// masking is bottom-right aligned: query i is at position seqlen_k - seqlen_q + i.
struct DecParams {
  const u16* q;
  const u16* k;
  const u16* v;
  u16* o;
  float* lse;
  float* part_o;
  float* part_lse;
  int B, H, Nq, Nk, n_splits, split_len;
  float scale;
  float c;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64, 1) void decode_split_kernel(DecParams p) {
  constexpr int BC = kFwdBC, NB = D / 32, NS = D / 16;
  using L = FwdLds<D>;
  __shared__ __attribute__((aligned(16))) u16 buf0[L::BUF];
  __shared__ __attribute__((aligned(16))) u16 buf1[L::BUF];
  const int lane = threadIdx.x, lr = lane & 31, g = lane >> 5;
  const int split = blockIdx.x % p.n_splits, bh = blockIdx.x / p.n_splits;
  const int b = bh / p.H, h = bh % p.H;
  const int ks = split * p.split_len;
  const int ke = min(ks + p.split_len, p.Nk);  // the split sizing keeps ks < ke
  const int qpos0 = p.Nk - p.Nq;                // position of query 0 in the sequence
  const size_t stride = (size_t)p.H * D;
  const u16* __restrict__ Qg = p.q + ((size_t)b * p.Nq * p.H + h) * D;
  const u16* __restrict__ Kg = p.k + ((size_t)b * p.Nk * p.H + h) * D + (size_t)ks * stride;
  const u16* __restrict__ Vg = p.v + ((size_t)b * p.Nk * p.H + h) * D + (size_t)ks * stride;
  const int len = ke - ks;  // keys of this split, rows 0..len-1 of Kg / Vg

  FwdState<D> st;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    st.qf[s] = lr < p.Nq ? ld16(Qg + (size_t)lr * stride + 16 * s + 8 * g) : zero_bf16x8();
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) st.oacc[bb] = f32x16{};
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  TileDma<BC, D, L::KP, 1> kdma;
  TileDma<BC, D, L::VP, 1> vdma;
  // The wave index (0) is read from the hardware rather than written as a constant: with
  // a literal the LDS destinations fold into constant address-space casts that this
  // compiler's instruction selection rejects.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  kdma.init(stride, w, lane);
  vdma.init(stride, w, lane);
  const int n_kt = (len + BC - 1) / BC;
  // The tile loop works in split-relative key indices; a query's position relative to
  // the split is qpos0 + i - ks.
  const int wq0 = qpos0 - ks;
  auto step = [&](int kt, const u16* buf) {
    const int k0 = kt * BC;
    const bool mask = k0 + BC > len || (CAUSAL && k0 + BC - 1 > wq0);  // wave-uniform
    fwd_tile<D, CAUSAL>(st, buf, buf + L::KSZ, k0, len, wq0, lane, p.c, mask);
  };
  kdma.issue(buf0, Kg, 0, len, stride, w, lane);
  vdma.issue(buf0 + L::KSZ, Vg, 0, len, stride, w, lane);
#pragma unroll
  for (int s = 0; s < NS; ++s) settle(st.qf[s]);
  wait_vmem();
  for (int kt = 0; kt < n_kt; kt += 2) {
    // One wave: its LDS reads of a buffer are consumed by its MFMAs before the next
    // copy into that buffer is issued, and its own copies are awaited with vmcnt.
    if (kt + 1 < n_kt) {
      kdma.issue(buf1, Kg, (kt + 1) * BC, len, stride, w, lane);
      vdma.issue(buf1 + L::KSZ, Vg, (kt + 1) * BC, len, stride, w, lane);
    }
    step(kt, buf0);
    wait_vmem();
    if (kt + 1 >= n_kt) break;
    if (kt + 2 < n_kt) {
      kdma.issue(buf0, Kg, (kt + 2) * BC, len, stride, w, lane);
      vdma.issue(buf0 + L::KSZ, Vg, (kt + 2) * BC, len, stride, w, lane);
    }
    step(kt + 1, buf1);
    wait_vmem();
  }

  const float l_tot = pair_sum(st.l_run);
  if (lr >= p.Nq) return;
  // A split can hold no key a query sees (causal): its weight in the merge is then 0.
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  float* __restrict__ Po = p.part_o + (((size_t)bh * p.n_splits + split) * p.Nq + lr) * D;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      // lane group g holds head-dim entries 32bb + 8a + 4g + {0..3} in registers 4a..4a+3
      *reinterpret_cast<f32x4*>(Po + 32 * bb + 8 * a + 4 * g) =
          f32x4{st.oacc[bb][4 * a] * inv, st.oacc[bb][4 * a + 1] * inv, st.oacc[bb][4 * a + 2] * inv,
                st.oacc[bb][4 * a + 3] * inv};
    }
  }
  if (g == 0)
    p.part_lse[((size_t)bh * p.n_splits + split) * p.Nq + lr] =
        empty ? -INFINITY : st.m_run * p.scale + logf(l_tot);
}

// One wave per (sequence, head, query): lse = log sum_s exp(lse_s), O = sum_s
// exp(lse_s - lse) O_s, each lane owning head-dim entries lane and lane + 64.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecParams p) {
  constexpr int NJ = D / 64;
  const int lane = threadIdx.x;
  const int i = blockIdx.x % p.Nq, bh = blockIdx.x / p.Nq;
  const int b = bh / p.H, h = bh % p.H;
  const float* pl = p.part_lse + (size_t)bh * p.n_splits * p.Nq + i;
  const float* po = p.part_o + ((size_t)bh * p.n_splits * p.Nq + i) * D;
  float m = -INFINITY;
  for (int s = 0; s < p.n_splits; ++s) m = fmaxf(m, pl[(size_t)s * p.Nq]);
  float den = 0.f, acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < p.n_splits; ++s) {
      const float wgt = expf(pl[(size_t)s * p.Nq] - m);
      den += wgt;
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = fmaf(wgt, po[(size_t)s * p.Nq * D + lane + 64 * j], acc[j]);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  u16* __restrict__ Og = p.o + (((size_t)b * p.Nq + i) * p.H + h) * D;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const __bf16 x = (__bf16)(acc[j] * inv);
    Og[lane + 64 * j] = __builtin_bit_cast(u16, x);
  }
  if (lane == 0) p.lse[((size_t)b * p.H + h) * p.Nq + i] = den > 0.f ? m + logf(den) : -INFINITY;
}

template <int D, bool CAUSAL>
hipError_t launch_decode_t(const DecodeProblem& pr) {
  DecParams p;
  p.q = static_cast<const u16*>(pr.q);
  p.k = static_cast<const u16*>(pr.k);
  p.v = static_cast<const u16*>(pr.v);
  p.o = static_cast<u16*>(pr.o);
  p.lse = pr.lse;
  p.part_o = pr.part_o;
  p.part_lse = pr.part_lse;
  p.B = pr.batch;
  p.H = pr.heads;
  p.Nq = pr.seqlen_q;
  p.Nk = pr.seqlen_k;
  p.n_splits = pr.num_splits;
  p.split_len = pr.split_len;
  p.scale = pr.scale;
  p.c = pr.scale * kLog2e;
  const unsigned bh = (unsigned)(pr.batch * pr.heads);
  hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL>), dim3(bh * (unsigned)pr.num_splits), dim3(64), 0, pr.stream,
                     p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(bh * (unsigned)pr.seqlen_q), dim3(64), 0, pr.stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_fwd_t(const Problem& pr) {
  constexpr int BR = 32 * kFwdWaves;
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
  const int n_qtiles = (pr.seqlen + BR - 1) / BR;
  p.n_slots = CAUSAL ? (n_qtiles + 1) / 2 : n_qtiles;
  p.scale = pr.scale;
  p.c = pr.scale * kLog2e;
  const dim3 grid((unsigned)(p.n_slots * pr.batch * pr.heads));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, VARLEN>), grid, dim3(64 * kFwdWaves), 0, pr.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const Problem& p) { FA_DISPATCH(launch_fwd_t, p); }

hipError_t launch_decode_bf16(const DecodeProblem& p) {
  if (p.head_dim == 64) return p.causal ? launch_decode_t<64, true>(p) : launch_decode_t<64, false>(p);
  return p.causal ? launch_decode_t<128, true>(p) : launch_decode_t<128, false>(p);
}

}  // namespace fa
