// fa_api.hip - the C ABI of libfa.so: argument checks on the host, then kernel launches
// on the caller's stream. Declarations and conventions: include/fa.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "fa_launch.h"

namespace {

constexpr size_t kAlign = 16;

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

// The kernels track the running maximum of the raw scores q.k and exponentiate
// c * (s - m) with c = scale * log2(e): that is the maximum of the scaled scores only when
// c > 0, so the scale must be positive (and finite).
bool scale_ok(float scale) { return isfinite(scale) && scale > 0.f; }

// Common checks of fa_fwd and fa_bwd; fills the sizes of `pr`.
int check_common(int batch, int heads, int seqlen, int head_dim, float scale, int causal,
                 const int32_t* cu_seqlens, int total_tokens, int dtype, fa::Problem& pr) {
  if (batch < 1 || heads < 1 || seqlen < 1) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
  if (cu_seqlens != nullptr) {
    if (total_tokens < 0) return FA_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(cu_seqlens) % sizeof(int32_t) != 0) return FA_ERR_INVALID_ARG;
  }
  const long long tokens = cu_seqlens ? (long long)total_tokens : (long long)batch * seqlen;
  // Element offsets are computed in 64 bits; the lse/D index (heads * tokens) and the
  // launch grid (sequences * heads * tiles) must fit the kernels' 32-bit work counters.
  if ((long long)heads * tokens > INT32_MAX) return FA_ERR_INVALID_ARG;
  if ((long long)batch * heads * ((seqlen + 63) / 64) > INT32_MAX) return FA_ERR_INVALID_ARG;
  if (!cu_seqlens && tokens > INT32_MAX) return FA_ERR_INVALID_ARG;
  pr.batch = batch;
  pr.heads = heads;
  pr.seqlen = seqlen;
  pr.head_dim = head_dim;
  pr.total_tokens = (int)tokens;
  pr.scale = scale;
  pr.causal = causal != 0;
  pr.cu_seqlens = cu_seqlens;
  return FA_OK;
}

// D and -LSE / scale: one fp32 each per (head, token), each array rounded up to 256 bytes,
// then 256 bytes of work counters for the dK/dV kernel.
size_t stat_bytes_for(int heads, long long tokens) {
  const size_t bytes = (size_t)heads * (size_t)tokens * sizeof(float);
  return ((bytes + 255) / 256) * 256;
}
constexpr size_t kCounterBytes = 256;
static_assert(fa::kKvCounters * sizeof(int) <= kCounterBytes, "the counters fit their block");
size_t workspace_bytes_for(int heads, long long tokens) { return 2 * stat_bytes_for(heads, tokens) + kCounterBytes; }

// Checks shared by the backward entry points; sets pr.dvec to the workspace.
int check_bwd(fa::Problem& pr, void* workspace, size_t workspace_bytes, int batch, int heads, int seqlen,
              int head_dim, float scale, int causal, const int32_t* cu_seqlens, int total_tokens, int dtype) {
  const int st = check_common(batch, heads, seqlen, head_dim, scale, causal, cu_seqlens, total_tokens, dtype, pr);
  if (st != FA_OK) return st;
  const size_t need = workspace_bytes_for(heads, pr.total_tokens);
  if (workspace == nullptr || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return FA_ERR_WORKSPACE;
  pr.dvec = static_cast<float*>(workspace);
  pr.mneg = reinterpret_cast<float*>(static_cast<char*>(workspace) + stat_bytes_for(heads, pr.total_tokens));
  pr.kvctr = reinterpret_cast<int*>(static_cast<char*>(workspace) + 2 * stat_bytes_for(heads, pr.total_tokens));
  return FA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Checks of the decode entry points; fills the sizes and the split choice of `pr` and
// the workspace it needs.
int check_decode(int batch, int heads, int seqlen_q, int seqlen_k, int head_dim, float scale, int causal,
                 int num_splits, int dtype, fa::DecodeProblem& pr, size_t* need) {
  if (batch < 1 || heads < 1 || seqlen_q < 1 || seqlen_k < 1 || num_splits < 0) return FA_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (causal && seqlen_q > seqlen_k) return FA_ERR_INVALID_ARG;
  if (seqlen_q > fa::kDecodeMaxQ) return FA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (num_splits > (seqlen_k + 63) / 64) return FA_ERR_INVALID_ARG;
  if ((long long)batch * seqlen_k * heads * head_dim > INT32_MAX * 8LL) return FA_ERR_INVALID_ARG;
  int splits = 0, split_len = 0;
  fa::decode_splits(batch, heads, seqlen_k, num_splits, &splits, &split_len);
  const long long items = (long long)batch * heads * splits;
  if (items > INT32_MAX || (long long)batch * heads * seqlen_q > INT32_MAX) return FA_ERR_INVALID_ARG;
  const size_t part_o = (size_t)items * seqlen_q * head_dim * sizeof(float);
  const size_t part_lse = (size_t)items * seqlen_q * sizeof(float);
  *need = ((part_o + part_lse + 255) / 256) * 256;
  pr.batch = batch;
  pr.heads = heads;
  pr.seqlen_q = seqlen_q;
  pr.seqlen_k = seqlen_k;
  pr.head_dim = head_dim;
  pr.num_splits = splits;
  pr.split_len = split_len;
  pr.scale = scale;
  pr.causal = causal != 0;
  return FA_OK;
}

// Scratch memory of fa_bwd_noalloc: the backward's row statistics (D and -LSE / scale)
// in a fixed device array, for callers that cannot allocate. Each GPU the library runs
// on holds its own copy until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is used.
constexpr size_t kScratchBytes = FA_BWD_NOALLOC_MAX_SCRATCH;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, or nullptr with *err set.
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || ptr == nullptr) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

#define FA_EXPORT __attribute__((visibility("default")))

extern "C" {

FA_EXPORT int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int heads,
           int seqlen, int head_dim, float softmax_scale, int causal, const int32_t* cu_seqlens,
           int total_tokens, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o) || !aligned(lse)) return FA_ERR_INVALID_ARG;
  fa::Problem pr{};
  const int st = check_common(batch, heads, seqlen, head_dim, softmax_scale, causal, cu_seqlens,
                              total_tokens, dtype, pr);
  if (st != FA_OK) return st;
  if (pr.total_tokens == 0) return FA_OK;  // a packed batch of empty sequences
  pr.q = q;
  pr.k = k;
  pr.v = v;
  pr.o_out = o;
  pr.lse_out = lse;
  pr.stream = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == FA_DTYPE_BF16 ? fa::launch_fwd_bf16(pr) : fa::launch_fwd_fp32(pr);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_EXPORT int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int heads,
                         int seqlen, int head_dim, float softmax_scale, float descale_q, float descale_k,
                         float descale_v, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o) || !aligned(lse)) return FA_ERR_INVALID_ARG;
  // The 8-bit kernel's scores are scaled by scale * descale_q * descale_k (see scale_ok).
  if (!isfinite(descale_v) || !scale_ok(descale_q) || !scale_ok(descale_k)) return FA_ERR_INVALID_ARG;
  if (!scale_ok(softmax_scale * descale_q * descale_k)) return FA_ERR_INVALID_ARG;
  fa::Problem chk{};
  const int st = check_common(batch, heads, seqlen, head_dim, softmax_scale, causal, nullptr, 0, FA_DTYPE_BF16,
                              chk);
  if (st != FA_OK) return st;
  fa::Fp8Problem pr{};
  pr.q = q;
  pr.k = k;
  pr.v = v;
  pr.o = o;
  pr.lse = lse;
  pr.batch = batch;
  pr.heads = heads;
  pr.seqlen = seqlen;
  pr.head_dim = head_dim;
  pr.scale = softmax_scale;
  pr.descale_q = descale_q;
  pr.descale_k = descale_k;
  pr.descale_v = descale_v;
  pr.causal = causal != 0;
  pr.stream = static_cast<hipStream_t>(stream);
  return status_of(fa::launch_fwd_fp8(pr));
}

FA_EXPORT size_t fa_bwd_workspace_bytes(int batch, int heads, int seqlen, int head_dim, int varlen, int total_tokens) {
  if (batch < 1 || heads < 1 || seqlen < 1) return 0;
  if (head_dim != 64 && head_dim != 128) return 0;
  if (varlen && total_tokens < 0) return 0;
  const long long tokens = varlen ? (long long)total_tokens : (long long)batch * seqlen;
  return workspace_bytes_for(heads, tokens);
}


FA_EXPORT int fa_bwd_preprocess(const void* o, const void* dout, const float* lse, void* workspace,
                                size_t workspace_bytes, int batch, int heads, int seqlen, int head_dim,
                                float softmax_scale, const int32_t* cu_seqlens, int total_tokens, int dtype,
                                void* stream) {
  if (!o || !dout || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned(o) || !aligned(dout) || !aligned(lse)) return FA_ERR_INVALID_ARG;
  fa::Problem pr{};
  const int st = check_bwd(pr, workspace, workspace_bytes, batch, heads, seqlen, head_dim, softmax_scale, 0,
                           cu_seqlens, total_tokens, dtype);
  if (st != FA_OK || pr.total_tokens == 0) return st;
  pr.o = o;
  pr.dout = dout;
  pr.lse = lse;
  pr.stream = static_cast<hipStream_t>(stream);
  return status_of(fa::launch_bwd_pre(pr, dtype == FA_DTYPE_FP32));
}

FA_EXPORT int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                const void* workspace, size_t workspace_bytes, void* dk, void* dv, int batch, int heads,
                int seqlen, int head_dim, float softmax_scale, int causal, const int32_t* cu_seqlens,
                int total_tokens, int dtype, void* stream) {
  if (!q || !k || !v || !dout || !lse || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(dout) || !aligned(lse) || !aligned(dk) ||
      !aligned(dv))
    return FA_ERR_INVALID_ARG;
  fa::Problem pr{};
  const int st = check_bwd(pr, const_cast<void*>(workspace), workspace_bytes, batch, heads, seqlen, head_dim,
                           softmax_scale, causal, cu_seqlens, total_tokens, dtype);
  if (st != FA_OK || pr.total_tokens == 0) return st;
  pr.q = q;
  pr.k = k;
  pr.v = v;
  pr.dout = dout;
  pr.lse = lse;
  pr.dk = dk;
  pr.dv = dv;
  pr.stream = static_cast<hipStream_t>(stream);
  return status_of(dtype == FA_DTYPE_BF16 ? fa::launch_bwd_dkdv_bf16(pr) : fa::launch_bwd_dkdv_fp32(pr));
}

FA_EXPORT int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
              const void* workspace, size_t workspace_bytes, void* dq, int batch, int heads, int seqlen,
              int head_dim, float softmax_scale, int causal, const int32_t* cu_seqlens, int total_tokens,
              int dtype, void* stream) {
  if (!q || !k || !v || !dout || !lse || !dq) return FA_ERR_INVALID_ARG;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(dout) || !aligned(lse) || !aligned(dq))
    return FA_ERR_INVALID_ARG;
  fa::Problem pr{};
  const int st = check_bwd(pr, const_cast<void*>(workspace), workspace_bytes, batch, heads, seqlen, head_dim,
                           softmax_scale, causal, cu_seqlens, total_tokens, dtype);
  if (st != FA_OK || pr.total_tokens == 0) return st;
  pr.q = q;
  pr.k = k;
  pr.v = v;
  pr.dout = dout;
  pr.lse = lse;
  pr.dq = dq;
  pr.stream = static_cast<hipStream_t>(stream);
  return status_of(dtype == FA_DTYPE_BF16 ? fa::launch_bwd_dq_bf16(pr) : fa::launch_bwd_dq_fp32(pr));
}

FA_EXPORT int fa_bwd_dq_stats(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* workspace, size_t workspace_bytes, void* dq, int batch,
                              int heads, int seqlen, int head_dim, float softmax_scale, int causal,
                              const int32_t* cu_seqlens, int total_tokens, int dtype, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq) return FA_ERR_INVALID_ARG;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o) || !aligned(dout) || !aligned(lse) || !aligned(dq))
    return FA_ERR_INVALID_ARG;
  fa::Problem pr{};
  const int st = check_bwd(pr, workspace, workspace_bytes, batch, heads, seqlen, head_dim, softmax_scale, causal,
                           cu_seqlens, total_tokens, dtype);
  if (st != FA_OK || pr.total_tokens == 0) return st;
  if (dtype == FA_DTYPE_FP32) {
    // fp32: the statistics pass, then the dQ pass that reads them
    const int r = fa_bwd_preprocess(o, dout, lse, workspace, workspace_bytes, batch, heads, seqlen, head_dim,
                                    softmax_scale, cu_seqlens, total_tokens, dtype, stream);
    if (r != FA_OK) return r;
    return fa_bwd_dq(q, k, v, dout, lse, workspace, workspace_bytes, dq, batch, heads, seqlen, head_dim,
                     softmax_scale, causal, cu_seqlens, total_tokens, dtype, stream);
  }
  pr.q = q;
  pr.k = k;
  pr.v = v;
  pr.o = o;
  pr.dout = dout;
  pr.lse = lse;
  pr.dq = dq;
  pr.stream = static_cast<hipStream_t>(stream);
  return status_of(fa::launch_bwd_dq_stats_bf16(pr));
}

FA_EXPORT int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int batch, int heads,
           int seqlen, int head_dim, float softmax_scale, int causal, const int32_t* cu_seqlens,
           int total_tokens, int dtype, void* stream) {
  // Check everything before enqueueing anything, so a bad argument launches nothing.
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o) || !aligned(dout) || !aligned(lse) ||
      !aligned(dq) || !aligned(dk) || !aligned(dv))
    return FA_ERR_INVALID_ARG;
  fa::Problem pr{};
  const int st = check_bwd(pr, workspace, workspace_bytes, batch, heads, seqlen, head_dim, softmax_scale,
                           causal, cu_seqlens, total_tokens, dtype);
  if (st != FA_OK || pr.total_tokens == 0) return st;
  // The dQ pass forms the row statistics as it goes; the dK/dV kernel reads them.
  const int r = fa_bwd_dq_stats(q, k, v, o, dout, lse, workspace, workspace_bytes, dq, batch, heads, seqlen,
                                head_dim, softmax_scale, causal, cu_seqlens, total_tokens, dtype, stream);
  if (r != FA_OK) return r;
  return fa_bwd_dkdv(q, k, v, dout, lse, workspace, workspace_bytes, dk, dv, batch, heads, seqlen, head_dim,
                     softmax_scale, causal, cu_seqlens, total_tokens, dtype, stream);
}

// fa_bwd_atomic's workspace: the statistics as in fa_bwd, then the fp32 dQ accumulator,
// (heads * tokens + 64) rows of head_dim (the 64 extra rows take the zero terms of the
// last query tile's rows past the end).
size_t dqacc_bytes_for(int heads, long long tokens, int head_dim) {
  return ((size_t)heads * (size_t)tokens + 64) * (size_t)head_dim * sizeof(float);
}

FA_EXPORT size_t fa_bwd_atomic_workspace_bytes(int batch, int heads, int seqlen, int head_dim, int varlen,
                                               int total_tokens) {
  const size_t stats = fa_bwd_workspace_bytes(batch, heads, seqlen, head_dim, varlen, total_tokens);
  if (stats == 0) return 0;
  const long long tokens = varlen ? (long long)total_tokens : (long long)batch * seqlen;
  return stats + dqacc_bytes_for(heads, tokens, head_dim);
}

FA_EXPORT int fa_bwd_atomic(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                            int batch, int heads, int seqlen, int head_dim, float softmax_scale, int causal,
                            const int32_t* cu_seqlens, int total_tokens, int dtype, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o) || !aligned(dout) || !aligned(lse) ||
      !aligned(dq) || !aligned(dk) || !aligned(dv))
    return FA_ERR_INVALID_ARG;
  fa::Problem pr{};
  const int st = check_bwd(pr, workspace, workspace_bytes, batch, heads, seqlen, head_dim, softmax_scale,
                           causal, cu_seqlens, total_tokens, dtype);
  if (st != FA_OK) return st;
  if (head_dim != 128 || dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  const size_t stats = workspace_bytes_for(heads, pr.total_tokens);
  if (workspace_bytes < stats + dqacc_bytes_for(heads, pr.total_tokens, head_dim)) return FA_ERR_WORKSPACE;
  if (pr.total_tokens == 0) return FA_OK;
  pr.q = q;
  pr.k = k;
  pr.v = v;
  pr.o = o;
  pr.dout = dout;
  pr.lse = lse;
  pr.dq = dq;
  pr.dk = dk;
  pr.dv = dv;
  pr.dqacc = reinterpret_cast<float*>(static_cast<char*>(workspace) + stats);
  pr.stream = static_cast<hipStream_t>(stream);
  // Statistics (and the accumulator cleared), the fused kernel, then dQ from the accumulator.
  hipError_t e = fa::launch_bwd_pre(pr, false);
  if (e == hipSuccess) e = fa::launch_bwd_fused_bf16(pr);
  if (e == hipSuccess) e = fa::launch_bwd_dq_convert(pr);
  return status_of(e);
}

FA_EXPORT int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, void* dq, void* dk, void* dv, int batch, int heads, int seqlen,
                             int head_dim, float softmax_scale, int causal, const int32_t* cu_seqlens,
                             int total_tokens, int dtype, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o) || !aligned(dout) || !aligned(lse) ||
      !aligned(dq) || !aligned(dk) || !aligned(dv))
    return FA_ERR_INVALID_ARG;
  fa::Problem chk{};
  const int st = check_common(batch, heads, seqlen, head_dim, softmax_scale, causal, cu_seqlens, total_tokens,
                              dtype, chk);
  if (st != FA_OK) return st;
  const size_t need = workspace_bytes_for(heads, chk.total_tokens);
  if (need > kScratchBytes) return FA_ERR_SCRATCH;
  if (chk.total_tokens == 0) return FA_OK;
  hipError_t err = hipSuccess;
  void* ws = scratch_on_current_device(&err);
  if (ws == nullptr) return FA_ERR_HIP;
  // The same three kernels as fa_bwd, with the scratch array as the workspace. Nothing in
  // it needs clearing: the preprocess writes every statistic the later kernels read.
  return fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, kScratchBytes, batch, heads, seqlen, head_dim,
                softmax_scale, causal, cu_seqlens, total_tokens, dtype, stream);
}

FA_EXPORT size_t fa_fwd_decode_workspace_bytes(int batch, int heads, int seqlen_q, int seqlen_k, int head_dim,
                                               int num_splits) {
  fa::DecodeProblem pr{};
  size_t need = 0;
  if (check_decode(batch, heads, seqlen_q, seqlen_k, head_dim, 1.f, 0, num_splits, FA_DTYPE_BF16, pr, &need) != FA_OK)
    return 0;
  return need;
}

FA_EXPORT int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int heads,
                            int seqlen_q, int seqlen_k, int head_dim, float softmax_scale, int causal,
                            int num_splits, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o) || !aligned(lse)) return FA_ERR_INVALID_ARG;
  fa::DecodeProblem pr{};
  size_t need = 0;
  const int st = check_decode(batch, heads, seqlen_q, seqlen_k, head_dim, softmax_scale, causal, num_splits, dtype,
                              pr, &need);
  if (st != FA_OK) return st;
  if (workspace == nullptr || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return FA_ERR_WORKSPACE;
  const size_t items = (size_t)batch * heads * pr.num_splits;
  pr.q = q;
  pr.k = k;
  pr.v = v;
  pr.o = o;
  pr.lse = lse;
  pr.part_o = static_cast<float*>(workspace);
  pr.part_lse = pr.part_o + items * seqlen_q * head_dim;
  pr.stream = static_cast<hipStream_t>(stream);
  return status_of(fa::launch_decode_bf16(pr));
}

FA_EXPORT const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or flag)";
    case FA_ERR_UNSUPPORTED: return "unsupported head_dim or dtype (head_dim 64 or 128; bf16 or fp32)";
    case FA_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than fa_bwd_workspace_bytes()";
    case FA_ERR_HIP: return "HIP kernel launch failed";
    case FA_ERR_SCRATCH:
      return "problem needs more scratch than fa_bwd_noalloc's fixed device array holds "
             "(8 * heads * tokens bytes > FA_BWD_NOALLOC_MAX_SCRATCH); use fa_bwd with a workspace";
    default: return "unknown status code";
  }
}

}  // extern "C"
