// fa_ubench.hip - device facts and ceiling measurements for the roofline of the attention
// kernels: the compute-unit count and clock the device reports, and loops that measure
// what the chip sustains (bf16 MFMA throughput, vector-ALU exponential and FMA rates, LDS
// operand reads, HBM copy bandwidth). Declarations: include/fa_ubench.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "fa_common.h"
#include "fa_ubench.h"

namespace fa {
namespace {

constexpr int kUbThreads = 256;

// Four independent 32x32x16 bf16 MFMA chains per wave, two rounds per step (8 MFMAs): the
// matrix pipe never waits for a result, so the loop runs at the pipe's issue rate. The
// operands depend on the lane so nothing folds; the accumulators are summed into `out`.
__global__ __launch_bounds__(kUbThreads) void ub_mfma_kernel(float* __restrict__ out, int iters) {
  const int tid = threadIdx.x;
  const u32x4 bits = {0x3f803f80u ^ (uint32_t)tid, 0x3f003f00u, 0x3e803e80u, 0x3f403f40u ^ (uint32_t)blockIdx.x};
  const bf16x8 a = __builtin_bit_cast(bf16x8, bits);
  const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{bits[3], bits[2], bits[1], bits[0]});
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      c0 = mfma32(a, b, c0);
      c1 = mfma32(b, a, c1);
      c2 = mfma32(a, a, c2);
      c3 = mfma32(b, b, c3);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(size_t)blockIdx.x * kUbThreads + tid] = s;
}

// The same for the 8-bit MFMA of the FP8 forward (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3
// operands, block scales 2^0, 131072 FLOP each). Every operand byte is 0x30 .. 0x3f
// (E4M3 0.5 .. 0.94), so no NaN code occurs.
__global__ __launch_bounds__(kUbThreads) void ub_mfma_fp8_kernel(float* __restrict__ out, int iters) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const int tid = threadIdx.x;
  const int x = (int)(0x38383838u ^ (uint32_t)(tid & 15) * 0x01010101u);
  const int y = (int)(0x3a3a3a3au ^ (uint32_t)(blockIdx.x & 15) * 0x01010101u);
  const i32x8 a = {x, y, x, y, x, y, x, y};
  const i32x8 b = {y, x, y, x, y, x, y, x};
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 0, 0, 0, 127, 0, 127);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 127, 0, 127);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 0, 0, 0, 127, 0, 127);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(size_t)blockIdx.x * kUbThreads + tid] = s;
}

// One dependent MFMA chain per wave with NV independent vector operations after each MFMA
// (in eight chains of their own: fp32 FMAs, or exponentials when EXP), the MFMA's
// accumulator in VGPRs (the compiler's form) or in AGPRs (inline asm, as the attention
// kernels pin their output accumulators): how much vector work hides under the matrix
// pipe at a given occupancy, which is what the attention kernels' softmax needs.
template <int NV, bool AGPR, bool EXP>
__global__ __launch_bounds__(kUbThreads) void ub_coexec_kernel(float* __restrict__ out, int iters) {
  const int tid = threadIdx.x;
  const u32x4 bits = {0x3f803f80u ^ (uint32_t)tid, 0x3f003f00u, 0x3e803e80u, 0x3f403f40u ^ (uint32_t)blockIdx.x};
  const bf16x8 a = __builtin_bit_cast(bf16x8, bits);
  const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{bits[3], bits[2], bits[1], bits[0]});
  f32x16 c = f32x16{};
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = 0.25f + 0.01f * k + 1e-4f * (tid & 63);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (AGPR)
        mfma32_agpr(c, a, b);
      else
        c = mfma32(a, b, c);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        if constexpr (EXP)
          x[k & 7] = __builtin_amdgcn_exp2f(-x[k & 7]);
        else
          x[k & 7] = fmaf(x[k & 7], 0.999f, 1e-3f);
      }
      step_fence();
    }
  }
  if constexpr (AGPR) agpr_acc_fence(c);
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c[r];
#pragma unroll
  for (int k = 0; k < 8; ++k) s += x[k];
  out[(size_t)blockIdx.x * kUbThreads + tid] = s;
}

template <int NV>
hipError_t launch_coexec(float* out, int blocks, int iters, bool agpr, bool ex, hipStream_t st) {
  if (agpr) {
    if (ex)
      hipLaunchKernelGGL((ub_coexec_kernel<NV, true, true>), dim3(blocks), dim3(kUbThreads), 0, st, out, iters);
    else
      hipLaunchKernelGGL((ub_coexec_kernel<NV, true, false>), dim3(blocks), dim3(kUbThreads), 0, st, out, iters);
  } else {
    if (ex)
      hipLaunchKernelGGL((ub_coexec_kernel<NV, false, true>), dim3(blocks), dim3(kUbThreads), 0, st, out, iters);
    else
      hipLaunchKernelGGL((ub_coexec_kernel<NV, false, false>), dim3(blocks), dim3(kUbThreads), 0, st, out, iters);
  }
  return hipGetLastError();
}

// The forward's mix of work with none of its dependences: per wave, four independent
// 32x32x16 bf16 MFMA chains, and with MIX after every MFMA one exponential and three FMAs
// on independent vector chains (the forward issues about one exponential and three other
// vector instructions per MFMA), each MFMA and its vector work closed by a scheduling
// barrier as in the kernels. No LDS, no copies, no barriers, no data flow from the MFMAs
// to the vector work: the MFMA rate this reaches at one or two workgroups per SIMD bounds
// what a schedule of the forward's instruction mix can reach.
template <bool MIX>
__global__ __launch_bounds__(kUbThreads) void ub_mix_kernel(float* __restrict__ out, int iters) {
  const int tid = threadIdx.x;
  const u32x4 bits = {0x3f803f80u ^ (uint32_t)tid, 0x3f003f00u, 0x3e803e80u, 0x3f403f40u ^ (uint32_t)blockIdx.x};
  const bf16x8 a = __builtin_bit_cast(bf16x8, bits);
  const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{bits[3], bits[2], bits[1], bits[0]});
  float x[8], y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[k] = 0.25f + 0.01f * k + 1e-4f * (tid & 63);
    y[k] = x[k];
  }
  f32x16 c[4] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      c[m] = mfma32(a, b, c[m]);
      if constexpr (MIX) {
        x[(2 * m) & 7] = __builtin_amdgcn_exp2f(-x[(2 * m) & 7]);
#pragma unroll
        for (int f = 0; f < 3; ++f) y[(3 * m + f) & 7] = fmaf(y[(3 * m + f) & 7], 0.999f, 1e-3f);
      }
      step_fence();
    }
  }
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[m][r];
#pragma unroll
  for (int k = 0; k < 8; ++k) s += x[k] + y[k];
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

// LDS operand reads as the attention kernels issue them: eight 1 KiB operands per step in
// every wave, all eight in flight before their values are consumed (by an empty asm use:
// no arithmetic), at constant offsets from a base that alternates between the two halves
// of the tile each step (one address add, and the loads stay in the loop). op 0: row-wise
// reads of a swizzled 64-row tile (swz_row_operand, one ds_read_b128 per operand); op 1:
// transpose reads of the same tile (swz_tr_operand, two ds_read_b64_tr_b16 per operand).
// The first dword of each step's first operand is folded into `out`.
constexpr int kUbLdsElems = 32768;  // 64 KiB of bf16

__global__ __launch_bounds__(kUbThreads) void ub_lds_kernel(float* __restrict__ out, int iters, int op) {
  __shared__ __attribute__((aligned(16))) u16 lds[kUbLdsElems];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < kUbLdsElems; i += kUbThreads) lds[i] = (u16)(i * 2654435761u >> 16);
  __syncthreads();
  constexpr int HALF = 64 * swz_pitch<128>();  // one 64-row tile
  uint32_t acc = 0;
  bf16x8 x[8];
  if (op == 0) {
    for (int i = 0; i < iters; ++i) {
      const u16* t = lds + (i & 1) * HALF;
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = swz_row_operand<128>(t, 32 * (j & 1), j >> 1, lane);
      asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
      acc ^= __builtin_bit_cast(u32x4, x[0])[0];
    }
  } else {
    for (int i = 0; i < iters; ++i) {
      const u16* t = lds + (i & 1) * HALF;
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = swz_tr_operand<128>(t, 16 * (j & 3), 32 * (j >> 2), lane);
      asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
      acc ^= __builtin_bit_cast(u32x4, x[0])[0];
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

FA_EXPORT int fa_ubench_mfma_fp8(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return FA_UB_ERR_INVALID_ARG;
  hipLaunchKernelGGL(fa::ub_mfma_fp8_kernel, dim3(blocks), dim3(fa::kUbThreads), 0,
                     static_cast<hipStream_t>(stream), out, iters);
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

FA_EXPORT int fa_ubench_mfma_valu(float* out, int blocks, int iters, int nvalu, int agpr, int op, void* stream) {
  if (!out || blocks < 1 || iters < 1 || (agpr != 0 && agpr != 1) || (op != 0 && op != 1)) return FA_UB_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool ag = agpr == 1, ex = op == 0;
  hipError_t e;
  switch (nvalu) {
    case 0: e = fa::launch_coexec<0>(out, blocks, iters, ag, ex, st); break;
    case 2: e = fa::launch_coexec<2>(out, blocks, iters, ag, ex, st); break;
    case 4: e = fa::launch_coexec<4>(out, blocks, iters, ag, ex, st); break;
    case 8: e = fa::launch_coexec<8>(out, blocks, iters, ag, ex, st); break;
    default: return FA_UB_ERR_INVALID_ARG;
  }
  return e == hipSuccess ? FA_UB_OK : FA_UB_ERR_HIP;
}

FA_EXPORT int fa_ubench_mfma_mix(float* out, int blocks, int iters, int mix, void* stream) {
  if (!out || blocks < 1 || iters < 1 || (mix != 0 && mix != 1)) return FA_UB_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (mix)
    hipLaunchKernelGGL(fa::ub_mix_kernel<true>, dim3(blocks), dim3(fa::kUbThreads), 0, st, out, iters);
  else
    hipLaunchKernelGGL(fa::ub_mix_kernel<false>, dim3(blocks), dim3(fa::kUbThreads), 0, st, out, iters);
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
