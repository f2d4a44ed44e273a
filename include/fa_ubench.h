/*
 * fa_ubench.h - device facts and measured ceilings for the roofline of libfa's kernels
 * (part of libfa.so; not part of the attention path itself).
 *
 * The attention kernels are bounded by the matrix cores (the pages' point that GEMM
 * units do most of the FLOPs: "FlashAttention-2 (PT)", "1. Minimização de operações não
 * matriciais"), with the vector ALUs' exponentials and the HBM bandwidth as secondary
 * ceilings ("Pensar en la E/S" in the AI Atlas summary). These calls report the device's
 * compute-unit count and clock, from which the dense MFMA peak follows, and run loops
 * that measure what the chip sustains for each ceiling.
 *
 * Conventions: pointers are device pointers owned by the caller; work is enqueued on
 * `stream` (a hipStream_t passed as void*) and timed by the caller around the call.
 * Return FA_UB_OK, FA_UB_ERR_INVALID_ARG (checked on the host before any launch) or
 * FA_UB_ERR_HIP (a HIP call or launch failed).
 */
#ifndef FA_UBENCH_H_
#define FA_UBENCH_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { FA_UB_OK = 0, FA_UB_ERR_INVALID_ARG = 1, FA_UB_ERR_HIP = 4 };

/* Compute units, maximum engine clock (kHz) and L2 size (bytes) of `device` as the HIP
 * runtime reports them, and its architecture name (NUL-terminated, truncated to
 * arch_len - 1 characters; arch may be NULL when arch_len is 0). Host pointers. */
int fa_device_info(int device, int* compute_units, int* max_clock_khz, int* l2_bytes, char* arch,
                   int arch_len);

/* `blocks` workgroups of four waves; each wave issues 8 * iters v_mfma_f32_32x32x16_bf16
 * (32768 FLOP each) in four independent chains. out: blocks * 256 floats (written). */
int fa_ubench_mfma_bf16(float* out, int blocks, int iters, void* stream);

/* The same with the 8-bit MFMA of the FP8 forward: each wave issues 8 * iters
 * v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, unit block scales, 131072 FLOP each)
 * in four independent chains. out: blocks * 256 floats (written). */
int fa_ubench_mfma_fp8(float* out, int blocks, int iters, void* stream);

/* `blocks` workgroups of 256 lanes; each lane runs 8 * iters vector operations in eight
 * independent chains: op 0 the exponential v_exp_f32, op 1 an fp32 FMA (2 FLOP).
 * out: blocks * 256 floats (written). */
int fa_ubench_valu(float* out, int blocks, int iters, int op, void* stream);

/* `blocks` workgroups of four waves, each with a 64 KiB LDS tile; every wave reads
 * 8 * iters operands of 1 KiB (32 x 16 bf16) in the forms the attention kernels use,
 * eight in flight at a time: op 0 row-wise (one ds_read_b128 each), op 1 transposed (two
 * ds_read_b64_tr_b16 each), from a swizzled tile without bank conflicts.
 * out: blocks * 256 floats (written). */
int fa_ubench_lds(float* out, int blocks, int iters, int op, void* stream);

/* `blocks` workgroups of four waves; each wave runs one dependent chain of 4 * iters
 * v_mfma_f32_32x32x16_bf16 with nvalu (0, 2, 4 or 8) independent vector operations after
 * each MFMA: op 0 the exponential v_exp_f32, op 1 an fp32 FMA. agpr 1 keeps the MFMA's
 * accumulator in AGPRs, 0 in VGPRs. The time per MFMA at one or two workgroups per SIMD
 * (blocks = 1 or 2 per SIMD) measures how much vector work the matrix pipe hides.
 * out: blocks * 256 floats (written). */
int fa_ubench_mfma_valu(float* out, int blocks, int iters, int nvalu, int agpr, int op, void* stream);

/* `blocks` workgroups of four waves; each wave issues 4 * iters v_mfma_f32_32x32x16_bf16
 * in four independent chains. With mix 1, every MFMA is followed by one v_exp_f32 and
 * three fp32 FMAs on independent vector chains (the forward's instruction mix per MFMA,
 * without its dependences, LDS reads, copies or barriers); mix 0 issues the MFMAs alone.
 * At blocks = 1 or 2 per SIMD the MFMA rate bounds what a schedule of that mix can reach
 * at that occupancy. out: blocks * 256 floats (written). */
int fa_ubench_mfma_mix(float* out, int blocks, int iters, int mix, void* stream);

/* Copies `bytes` (a multiple of 16; src and dst 16-byte aligned, not overlapping) from
 * src to dst with `blocks` workgroups of 256 lanes, 16 bytes per lane per access. */
int fa_ubench_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_UBENCH_H_ */
