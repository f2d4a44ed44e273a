// fa_fwd_fp8.hip - forward pass with FP8 (OCP E4M3) Q, K, V on gfx950's 8-bit MFMA.
//
// The 8-bit variant named for FlashAttention-3 ([SA] "FlashAttention-2 (PT)", section
// "Comparação com versões subsequentes"): Q, K and V are E4M3 codes with one fp32
// descale factor each (real value = descale * code value); O is bf16, LSE fp32 (natural
// log), as in the bf16 forward. Both products run on v_mfma_scale_f32_32x32x64_f8f6f4
// (64-deep contraction, twice the bf16 MFMA rate):
//   S^T = K Q^T    A = K rows from LDS (32 bytes of head dim per lane), B = Q in VGPRs;
//   O^T += V^T P^T A = V^T read from the row-major V tile with ds_read_b64_tr_b8,
//                  B = P rounded to E4M3 from the S^T registers.
// One query per MFMA column as in the bf16 kernels: the S^T registers of a lane are one
// query's scores, 16 keys per 32-key block. A 64-key tile makes one P^T operand (its 32
// bytes per lane are the lane's 16 keys of each block), so the softmax reference is
// updated once per tile (lazy: only when the tile's maximum exceeds it by more than
// 2^8 in exp2 units; P then lies in [0, 256], inside E4M3's range, and the stale
// reference cancels between O and l).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kF8Waves = 4;
constexpr int kF8Threads = 64 * kF8Waves;
constexpr int kF8BR = 32 * kF8Waves;  // queries per workgroup
constexpr int kF8BC = 64;             // keys per tile
constexpr int kF8Pitch = 144;         // LDS row pitch in bytes (128 + 16: conflict-free reads)
constexpr float kF8Tau = 8.f;         // lazy-rescale threshold (exp2 units)

struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  u16* o;
  float* lse;
  int B, H, N;
  int n_qtiles;
  float c;          // softmax_scale * descale_q * descale_k * log2(e)
  float scale_eff;  // softmax_scale * descale_q * descale_k
  float descale_v;
};

// C = A B (+ C) on E4M3 operands (cbsz = blgp = 0), block scales 2^0.
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// LDS tiles: rows of kF8Pitch bytes, head-dim bytes 0 .. D-1 (the rest is pad).
template <int D>
struct F8Lds {
  static constexpr int TILE = kF8BC * kF8Pitch;  // bytes of one K or V tile
  static constexpr int BUF = 2 * TILE;           // K then V
};

// A operand of S^T = K Q^T for 32-key block j and head-dim slice t (64 bytes): lane l
// reads key row 32j + l % 32, bytes 64t + 32g .. + 31 (g = l / 32).
__device__ __forceinline__ i32x8 f8_k_operand(const uint8_t* Ks, int j, int t, int lane) {
  const uint8_t* p = Ks + (32 * j + (lane & 31)) * kF8Pitch + 64 * t + 32 * (lane >> 5);
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// A operand of O^T += V^T P^T for head-dim rows 32 mt .. + 31: lane l is row
// d = 32 mt + l % 32, and its byte 8t + kk (t = 0..3, kk = 0..7) is V[key][d] for
// key = 32 (t / 2) + 16 (t % 2) + 8 (kk / 4) + 4 g + kk % 4, the order in which the
// lane's P^T operand holds its keys (byte 16 j + r = C register r of block j). With
// ds_read_b64_tr_b8, output lane i of a 16-lane group receives byte i % 8 of the 8-byte
// run addressed by lane 2 kk + i / 8 as its byte kk; lane 2 kk + p therefore addresses
// key kk's row at head-dim d0 + 8 p, d0 = 32 mt + 16 ((l / 16) % 2).
__device__ __forceinline__ i32x8 f8_vt_operand(const uint8_t* Vs, int mt, int lane) {
  const int i = lane & 15, G = lane >> 4, g = lane >> 5;
  const int kk = i >> 1, p = i & 1;
  const int key_lane = 8 * (kk >> 2) + 4 * g + (kk & 3);
  const uint8_t* base = Vs + key_lane * kF8Pitch + 32 * mt + 16 * (G & 1) + 8 * p;
  i32x8 r;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int key_t = 32 * (t >> 1) + 16 * (t & 1);
    const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_i32x2*)(__attribute__((address_space(3))) uint8_t*)(base + key_t * kF8Pitch));
    r[2 * t] = x[0];
    r[2 * t + 1] = x[1];
  }
  return r;
}

// Wait states between the 64-cycle 8-bit MFMA that last wrote acc and any vector read of
// it. The compiler's own count (about 19) proved too short for the last registers of the
// accumulator (measured: a copy placed right after read them stale), so reads that can
// follow the final P V closely go behind this fence.
__device__ __forceinline__ void f8_acc_fence(f32x16& acc) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" : "+v"(acc));
}

template <int D>
struct F8State {
  static constexpr int NT = D / 64, NM = D / 32;
  i32x8 qf[NT];      // this lane's query row as the B operand of S^T (per 64-byte slice)
  f32x16 oacc[NM];   // O^T, one query per column
  float m_ref;       // reference maximum of the raw scores (-inf before the first key)
  float l_run;       // this lane's share of the row sum (16 of the 32 keys per block)
};

// One 64-key tile for one wave.
template <int D, bool CAUSAL>
__device__ __forceinline__ void f8_tile(F8State<D>& st, const uint8_t* Ks, const uint8_t* Vs, int k0, int len,
                                        int qi, int lane, float c, bool mask) {
  constexpr int NT = D / 64, NM = D / 32;
  const int g = lane >> 5;
  f32x16 s[2] = {f32x16{}, f32x16{}};
  // the two blocks' products alternate, so no MFMA waits for the one just before it
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 2; ++j) s[j] = mfma_fp8(f8_k_operand(Ks, j, t, lane), st.qf[t], s[j]);
  if (mask) {  // wave-uniform: a diagonal or tail tile
    // hidden: keys past the last one this query sees (one compare per score)
    const int lim = (CAUSAL ? min(qi, len - 1) : len - 1) - k0 - 4 * g;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[j][r] = 32 * j + crow_nat(r, 0) > lim ? -INFINITY : s[j][r];
  }
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  // Move the reference when the tile's maximum exceeds it by more than kF8Tau (in exp2
  // units): then O and l are scaled to the new one. mx is the same in both lanes of a
  // query, so the decision is per query.
  if (mx > -INFINITY && (st.m_ref == -INFINITY || (mx - st.m_ref) * c > kF8Tau)) {
    const float alpha = st.m_ref == -INFINITY ? 0.f : fast_exp2((st.m_ref - mx) * c);
    st.m_ref = mx;
    st.l_run *= alpha;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) st.oacc[mt] *= alpha;
  }
  const float nb = st.m_ref == -INFINITY ? 0.f : -st.m_ref * c;
  i32x8 pf;
  float ls[4] = {0.f, 0.f, 0.f, 0.f};  // four partial row sums: no chain of 32 dependent adds
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      float e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        e[u] = fast_exp2(fmaf(s[j][r + u], c, nb));  // exp2(-inf) = 0 for masked keys
        ls[u] += e[u];
      }
      // the low word's old value is e[0]'s own register (both halves are written)
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], __float_as_int(e[0]), false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], w, true);
      pf[4 * j + r / 4] = w;  // bytes 16 j + r .. + 3
    }
  }
  st.l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#pragma unroll
  for (int mt = 0; mt < NM; ++mt) st.oacc[mt] = mfma_fp8(f8_vt_operand(Vs, mt, lane), pf, st.oacc[mt]);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF8Threads, 2) void fwd_fp8_kernel(Fp8Params p) {
#if __HIP_DEVICE_COMPILE__
  constexpr int BR = kF8BR, BC = kF8BC, NT = D / 64, NM = D / 32;
  using L = F8Lds<D>;
  __shared__ __attribute__((aligned(16))) uint8_t buf0[L::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[L::BUF];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;

  // Workgroup -> (sequence, head, query tile), head-grouped per XCD; under causal the
  // longest rows (last query tiles) first.
  int bh, qt;
  xcd_tile_map(blockIdx.x, p.B * p.H, p.n_qtiles, CAUSAL, true, bh, qt);
  const int b = bh / p.H, h = bh % p.H;
  const int len = p.N;
  const int q0 = qt * BR;
  const size_t stride = (size_t)p.H * D;  // bytes between consecutive tokens
  const size_t base = ((size_t)b * p.N * p.H + h) * D;
  const uint8_t* __restrict__ Kg = p.k + base;
  const uint8_t* __restrict__ Vg = p.v + base;

  const int wq0 = q0 + 32 * w;
  const int qi = wq0 + lr;
  const int wq_last = min(wq0 + 31, len - 1);

  F8State<D> st;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    i32x8 x = i32x8{};
    if (qi < len) {
      const uint8_t* qp = p.q + base + (size_t)qi * stride + 64 * t + 32 * g;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(qp);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(qp + 16);
      x = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    st.qf[t] = x;
  }
#pragma unroll
  for (int mt = 0; mt < NM; ++mt) st.oacc[mt] = f32x16{};
  st.m_ref = -INFINITY;
  st.l_run = 0.f;

  const int kv_end = CAUSAL ? min(q0 + BR, len) : len;
  const int n_kt = (kv_end + BC - 1) / BC;

  // The tiles are copied as rows of D / 2 u16 (the bytes are moved, not read as bf16).
  TileDma<BC, D / 2, kF8Pitch / 2, kF8Waves> dma;
  dma.init(stride / 2, w, lane);
  auto issue = [&](int kt, uint8_t* buf) {
    dma.issue(reinterpret_cast<u16*>(buf), reinterpret_cast<const u16*>(Kg), kt * BC, len, stride / 2, w, lane);
    dma.issue(reinterpret_cast<u16*>(buf + L::TILE), reinterpret_cast<const u16*>(Vg), kt * BC, len, stride / 2,
              w, lane);
  };
  auto compute = [&](int kt, const uint8_t* buf) {
    const int k0 = kt * BC;
    if (wq0 < len && (!CAUSAL || k0 <= wq_last)) {  // wave-uniform
      const bool mask = k0 + BC > len || (CAUSAL && k0 + BC - 1 > wq0);
      f8_tile<D, CAUSAL>(st, buf, buf + L::TILE, k0, len, qi, lane, p.c, mask);
    }
  };
  issue(0, buf0);
#pragma unroll
  for (int t = 0; t < NT; ++t) settle(st.qf[t]);
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

  // The tiles are consumed (the loop ends on a barrier): the two buffers stage the O rows
  // (waves 0, 1 in buf0, waves 2, 3 in buf1) so that they leave whole. O rows are D bf16
  // apart by token (stride counts the 8-bit inputs' bytes).
  constexpr int SROWS = 32 * stage_pitch<D>();  // u16 elements of one wave's staging
  static_assert(2 * SROWS * 2 <= L::BUF, "two waves' staging fits in one tile buffer");
  u16* stg = reinterpret_cast<u16*>(w < 2 ? buf0 : buf1) + (w & 1) * SROWS;
  // the barrier above can pass at once for the last wave to arrive, right after its P V
  f8_acc_fence(st.oacc[NM - 1]);
  const float l_tot = pair_sum(st.l_run);
  stage_acc_rows<D>(stg, st.oacc, p.descale_v / l_tot, lr, g);
  store_staged_rows<D, 32>(stg, p.o + base + (size_t)wq0 * stride, stride, len - wq0, lane);
  if (g == 0 && qi < len) p.lse[((size_t)b * p.H + h) * p.N + qi] = st.m_ref * p.scale_eff + logf(l_tot);
#endif
}

template <int D, bool CAUSAL>
hipError_t launch_fp8_t(const Fp8Problem& pr) {
  Fp8Params p;
  p.q = static_cast<const uint8_t*>(pr.q);
  p.k = static_cast<const uint8_t*>(pr.k);
  p.v = static_cast<const uint8_t*>(pr.v);
  p.o = static_cast<u16*>(pr.o);
  p.lse = pr.lse;
  p.B = pr.batch;
  p.H = pr.heads;
  p.N = pr.seqlen;
  p.n_qtiles = (pr.seqlen + kF8BR - 1) / kF8BR;
  p.scale_eff = pr.scale * pr.descale_q * pr.descale_k;
  p.c = p.scale_eff * kLog2e;
  p.descale_v = pr.descale_v;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)(p.n_qtiles * pr.batch * pr.heads)),
                     dim3(kF8Threads), 0, pr.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Problem& p) {
  if (p.head_dim == 64) return p.causal ? launch_fp8_t<64, true>(p) : launch_fp8_t<64, false>(p);
  return p.causal ? launch_fp8_t<128, true>(p) : launch_fp8_t<128, false>(p);
}

}  // namespace fa
