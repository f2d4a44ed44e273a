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
  const int32_t* cu_seqlens;  // NULL: padded batch
  int batch, heads, seqlen, head_dim;
  int total_tokens;    // batch * seqlen, or the packed token count
  float scale;
  bool causal;
  hipStream_t stream;
};

// Each launcher enqueues one kernel on p.stream and returns hipGetLastError().
hipError_t launch_fwd_bf16(const Problem& p);
hipError_t launch_fwd_fp32(const Problem& p);
hipError_t launch_bwd_pre(const Problem& p, bool fp32);   // D = rowsum(dO * O)
hipError_t launch_bwd_dkdv_bf16(const Problem& p);
hipError_t launch_bwd_dq_bf16(const Problem& p);
hipError_t launch_bwd_dkdv_fp32(const Problem& p);
hipError_t launch_bwd_dq_fp32(const Problem& p);

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
