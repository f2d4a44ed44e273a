// fa_ubench.hip - device facts and ceiling measurements for the roofline of the attention
// kernels: the compute-unit count and clock the device reports, and three loops that
// measure what the chip sustains (bf16 MFMA throughput, vector-ALU exponential and FMA
// rates, HBM copy bandwidth). Declarations: include/fa_ubench.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "fa_common.h"
#include "fa_ubench.h"

namespace fa {
namespace {

constexpr int kUbThreads = 256;

// Four independent 32x32x16 bf16 MFMA chains per wave: the matrix pipe never waits for
// a result, so the loop runs at the pipe's issue rate. The operands depend on the lane
// so nothing folds; the accumulators are summed into `out` at the end.
__global__ __launch_bounds__(kUbThreads) void ub_mfma_kernel(float* __restrict__ out, int iters) {
  const int tid = threadIdx.x;
  const u32x4 bits = {0x3f803f80u ^ (uint32_t)tid, 0x3f003f00u, 0x3e803e80u, 0x3f403f40u ^ (uint32_t)blockIdx.x};
  const bf16x8 a = __builtin_bit_cast(bf16x8, bits);
  const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{bits[3], bits[2], bits[1], bits[0]});
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(b, a, c1);
    c2 = mfma32(a, a, c2);
    c3 = mfma32(b, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(size_t)blockIdx.x * kUbThreads + tid] = s;
}

// Eight independent chains per lane of one vector operation: op 0 the exponential the
// attention kernels use (v_exp_f32, x <- 2^-x stays in (0, 1]), op 1 an fp32 FMA.
__global__ __launch_bounds__(kUbThreads) void ub_valu_kernel(float* __restrict__ out, int iters, int op) {
  const int tid = threadIdx.x;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.25f + 0.01f * j + 1e-4f * (tid & 63);
  if (op == 0) {
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  } else {
    const float m = 0.999f, a = 1e-3f;
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = fmaf(x[j], m, a);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  out[(size_t)blockIdx.x * kUbThreads + tid] = s;
}

// LDS operand reads as the attention kernels issue them, eight per step in every wave:
// op 0 row-wise 16-byte reads (ds_read_b128: lane l reads row l % 32, chunk l / 32, of a
// tile with a 68-dword pitch, conflict-free), op 1 transpose reads (ds_read_b64_tr_b16 in
// the operand pattern of lds_tr_operand on a tile with an 80-dword pitch). The rows read
// move by 16 each step so the loads stay in the loop; their bits are folded into `out`.
constexpr int kUbLdsElems = 32768;  // 64 KiB of bf16

__global__ __launch_bounds__(kUbThreads) void ub_lds_kernel(float* __restrict__ out, int iters, int op) {
  __shared__ __attribute__((aligned(16))) u16 lds[kUbLdsElems];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < kUbLdsElems; i += kUbThreads) lds[i] = (u16)(i * 2654435761u >> 16);
  __syncthreads();
  uint32_t acc = 0;
  if (op == 0) {
    constexpr int P = 136;  // pitch_rows<128>()
    const u16* base = lds + (lane & 31) * P + 8 * (lane >> 5);
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(base + (((i * 3 + j) & 7) * 16) * P + 16 * (j & 3));
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
  } else {
    constexpr int P = 160;  // pitch_tr<128>()
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x8 v = lds_tr_operand(lds, P, ((i * 3 + j) & 7) * 16, 32 * (j & 3), lane);
        const u32x4 u = __builtin_bit_cast(u32x4, v);
        acc ^= u[0] ^ u[1] ^ u[2] ^ u[3];
      }
  }
  out[(size_t)blockIdx.x * kUbThreads + tid] = __uint_as_float(acc);
}

// dst = src, 16 bytes per lane per access, grid-stride.
__global__ __launch_bounds__(kUbThreads) void ub_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                             size_t n) {
  const size_t step = (size_t)gridDim.x * kUbThreads;
  for (size_t i = (size_t)blockIdx.x * kUbThreads + threadIdx.x; i < n; i += step) dst[i] = src[i];
}

}  // namespace
}  // namespace fa

#define FA_EXPORT __attribute__((visibility("default")))

extern "C" {

FA_EXPORT int fa_device_info(int device, int* compute_units, int* max_clock_khz, int* l2_bytes, char* arch,
                             int arch_len) {
  if (!compute_units || !max_clock_khz || !l2_bytes || (arch_len > 0 && !arch)) return FA_UB_ERR_INVALID_ARG;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return FA_UB_ERR_HIP;
  *compute_units = prop.multiProcessorCount;
  *max_clock_khz = prop.clockRate;
  *l2_bytes = prop.l2CacheSize;
  if (arch_len > 0) {
    strncpy(arch, prop.gcnArchName, (size_t)arch_len - 1);
    arch[arch_len - 1] = '\0';
  }
  return FA_UB_OK;
}

FA_EXPORT int fa_ubench_mfma_bf16(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return FA_UB_ERR_INVALID_ARG;
  hipLaunchKernelGGL(fa::ub_mfma_kernel, dim3(blocks), dim3(fa::kUbThreads), 0, static_cast<hipStream_t>(stream),
                     out, iters);
  return hipGetLastError() == hipSuccess ? FA_UB_OK : FA_UB_ERR_HIP;
}

FA_EXPORT int fa_ubench_valu(float* out, int blocks, int iters, int op, void* stream) {
  if (!out || blocks < 1 || iters < 1 || (op != 0 && op != 1)) return FA_UB_ERR_INVALID_ARG;
  hipLaunchKernelGGL(fa::ub_valu_kernel, dim3(blocks), dim3(fa::kUbThreads), 0, static_cast<hipStream_t>(stream),
                     out, iters, op);
  return hipGetLastError() == hipSuccess ? FA_UB_OK : FA_UB_ERR_HIP;
}

FA_EXPORT int fa_ubench_lds(float* out, int blocks, int iters, int op, void* stream) {
  if (!out || blocks < 1 || iters < 1 || (op != 0 && op != 1)) return FA_UB_ERR_INVALID_ARG;
  hipLaunchKernelGGL(fa::ub_lds_kernel, dim3(blocks), dim3(fa::kUbThreads), 0, static_cast<hipStream_t>(stream),
                     out, iters, op);
  return hipGetLastError() == hipSuccess ? FA_UB_OK : FA_UB_ERR_HIP;
}

FA_EXPORT int fa_ubench_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 != 0 || blocks < 1) return FA_UB_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0) return FA_UB_ERR_INVALID_ARG;
  hipLaunchKernelGGL(fa::ub_copy_kernel, dim3(blocks), dim3(fa::kUbThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const fa::u32x4*>(src), static_cast<fa::u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? FA_UB_OK : FA_UB_ERR_HIP;
}

}  // extern "C"
