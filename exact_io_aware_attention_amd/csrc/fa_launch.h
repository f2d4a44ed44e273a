// fa_launch.h - internal interface between the C ABI (fa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// One call's arguments, already checked on the host. Pointers are device pointers.
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  const void* o;       // forward: written; backward: read
  const void* dout;
  const float* lse;    // forward: written through lse_out; backward: read
  float* lse_out;
  void* o_out;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;         // backward workspace: D_i = rowsum(dO * O), same layout as lse
  float* mneg;         // backward workspace: -LSE_i / scale, same layout as lse
  float* dqacc;        // fused backward workspace: fp32 dQ accumulator (lse rows + 64) x head_dim,
                       // zeroed by launch_bwd_pre when set
  int* kvctr;          // backward workspace: kKvCounters work counters of the head_dim-128 dK/dV
                       // kernel, zeroed by the statistics kernels (launch_bwd_pre, the dQ pass
                       // with statistics) and left zero by the dK/dV kernel when it ends
  const int32_t* cu_seqlens;  // NULL: padded batch
  int batch, heads, seqlen, head_dim;
  int total_tokens;    // batch * seqlen, or the packed token count
  float scale;
  bool causal;
  hipStream_t stream;
};

// Work counters of the persistent dK/dV kernel: one per XCD and one of finished workgroups.
constexpr int kKvCounters = 9;

// Each launcher enqueues one kernel on p.stream and returns hipGetLastError().
hipError_t launch_fwd_bf16(const Problem& p);
hipError_t launch_fwd_fp32(const Problem& p);
hipError_t launch_bwd_pre(const Problem& p, bool fp32);   // D = rowsum(dO * O), -LSE / scale
hipError_t launch_bwd_dkdv_bf16(const Problem& p);
hipError_t launch_bwd_dq_bf16(const Problem& p);
// The dQ pass that also writes the row statistics (p.dvec, p.mneg) from p.o, p.dout, p.lse.
hipError_t launch_bwd_dq_stats_bf16(const Problem& p);
// The fused backward (head_dim 128, bf16): dK, dV, and dQ added into p.dqacc by fp32
// atomics; then the conversion dq = -scale * dqacc.
hipError_t launch_bwd_fused_bf16(const Problem& p);
hipError_t launch_bwd_dq_convert(const Problem& p);
hipError_t launch_bwd_dkdv_fp32(const Problem& p);
hipError_t launch_bwd_dq_fp32(const Problem& p);

// Decoding: seqlen_q (1..32) new queries against seqlen_k cached keys, the key range cut
// into num_splits splits of split_len keys (a multiple of 64) whose partial results
// (O normalised by its own sum, fp32, and the split's logsumexp) go to the workspace and
// are merged by logsumexp weights.
// Forward pass on OCP FP8 E4M3 inputs with per-tensor descale factors (bf16 O).
struct Fp8Problem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int batch, heads, seqlen, head_dim;
  float scale, descale_q, descale_k, descale_v;
  bool causal;
  hipStream_t stream;
};

hipError_t launch_fwd_fp8(const Fp8Problem& p);

struct DecodeProblem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* part_o;    // (batch, heads, num_splits, seqlen_q, head_dim)
  float* part_lse;  // (batch, heads, num_splits, seqlen_q)
  int batch, heads, seqlen_q, seqlen_k, head_dim;
  int num_splits, split_len;
  float scale;
  bool causal;
  hipStream_t stream;
};

constexpr int kDecodeMaxQ = 32;

// Number of key splits and their length for a decode launch: `requested` (> 0) or, with
// 0, enough splits for about 1024 single-wave workgroups, each at least 256 keys long.
inline void decode_splits(int batch, int heads, int seqlen_k, int requested, int* num_splits, int* split_len) {
  const long long bh = (long long)batch * heads;
  long long want = requested > 0 ? requested : (1024 + bh - 1) / bh;
  const long long max_by_len = requested > 0 ? (seqlen_k + 63) / 64 : (seqlen_k + 255) / 256;
  if (want > max_by_len) want = max_by_len;
  if (want < 1) want = 1;
  long long len = (seqlen_k + want - 1) / want;
  len = (len + 63) / 64 * 64;
  *split_len = (int)len;
  *num_splits = (int)((seqlen_k + len - 1) / len);
}

// Enqueues the split kernel and the merge kernel on p.stream.
hipError_t launch_decode_bf16(const DecodeProblem& p);

// Calls fn<head_dim, causal, varlen>(p) for the instantiation matching p.
#define FA_DISPATCH(fn, p)                                                         \
  do {                                                                             \
    const bool vl_ = (p).cu_seqlens != nullptr;                                    \
    if ((p).head_dim == 64) {                                                      \
      if ((p).causal) return vl_ ? fn<64, true, true>(p) : fn<64, true, false>(p); \
      return vl_ ? fn<64, false, true>(p) : fn<64, false, false>(p);               \
    }                                                                              \
    if ((p).causal) return vl_ ? fn<128, true, true>(p) : fn<128, true, false>(p); \
    return vl_ ? fn<128, false, true>(p) : fn<128, false, false>(p);               \
  } while (0)

}  // namespace fa
