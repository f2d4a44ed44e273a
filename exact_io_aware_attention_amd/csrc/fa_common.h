// fa_common.h - device helpers shared by the gfx950 attention kernels.
//
// MFMA operand layout used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16): lane l supplies row m = l % 32 and the 8 k-slots of lane group
//                g = l / 32; B (16 x 32): lane l supplies column n = l % 32 and the
//                same 8 k-slots of group g. A and B pair up slot by slot, so which
//                real index sits in which slot is ours to choose, as long as A and B
//                choose alike.
//   C (32 x 32): lane l, register r holds row m = 8*(r/4) + 4*g + (r%4), column
//                n = l % 32 (crow_nat below).
// The kernels put one query (or one key) per C column, so per-row state lives in one
// lane and its mirror lane l ^ 32. The C registers of a first product (rows = keys or
// queries of a tile) then serve directly as the B operand of a second product that
// contracts over those rows: registers 8h .. 8h + 7 of lane group g hold rows
// 16h + 4g + {0..3, 8..11}, and the matching A operand is fetched from the row-major
// LDS tile with transpose reads (lds_tr_operand) in exactly that row order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// O^T += A B on accumulators held in AGPRs. Under a 512-register budget (one wave per
// SIMD) the output accumulators live in AGPRs for a whole kernel and are touched only by
// these MFMAs, while everything else (compiled with VGPR-form MFMAs) stays in VGPRs. The
// compiler cannot see hazards through inline asm, so the two wait states that a
// VALU-written A/B operand needs before an MFMA read are padded here, and
// agpr_acc_fence must separate the last of these MFMAs from any VALU or v_accvgpr_read
// access to the accumulator.
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Closes one step of a software-pipelined phase: the scheduler moves no instruction
// across it, so each step keeps the reads, MFMAs and vector work it was written with.
__device__ __forceinline__ void step_fence() { __builtin_amdgcn_sched_barrier(0); }

// Wait states between an MFMA writing `acc` and VALU / v_accvgpr_read reads of it.
__device__ __forceinline__ void agpr_acc_fence(f32x16& acc) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" : "+a"(acc));
}

// Workgroup index -> (sequence*head index bh, tile index t) for a grid of BH x NT
// workgroups. Workgroups are dispatched to the 8 XCDs round-robin (workgroup i runs on
// XCD i % 8) and each XCD has its own L2.
//  - tile-major (xcd_group = false): workgroup L is head L % BH, tile L / BH. When BH
//    is a multiple of 8, every tile of a head still lands on one XCD, and under causal
//    masking (rev = true: tile order reversed) the longest rows of all heads are issued
//    first, which balances the causal work best.
//  - head-grouped (xcd_group = true, BH a multiple of 8): the k-th workgroup an XCD
//    receives is head (k / NT) * 8 + xcd, tile k % NT, so an XCD works through all tiles
//    of one head before the next and the head's operands stay in that XCD's L2.
__device__ __forceinline__ void xcd_tile_map(int L, int BH, int NT, bool rev, bool xcd_group, int& bh, int& t) {
  constexpr int kXcds = 8;
  if (xcd_group && BH % kXcds == 0) {
    const int xcd = L % kXcds, k = L / kXcds;
    bh = (k / NT) * kXcds + xcd;
    t = k % NT;
  } else {
    bh = L % BH;
    t = L / BH;
  }
  if (rev) t = NT - 1 - t;
}

__device__ __forceinline__ bf16x8 ld16(const u16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// Eight fp32 -> eight bf16, round to nearest even.
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x8& x) {
  return __builtin_convertvector(x, bf16x8);
}

// Four fp32 -> four bf16 (round to nearest even) stored as one 8-byte write.
__device__ __forceinline__ void store_bf16x4(u16* dst, float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<bf16x4*>(dst) = __builtin_convertvector(f32x4{a, b, c, d}, bf16x4);
}

// Output rows leave through LDS so that each row is written whole. The lane holding
// row lr (0..31) in lane group g has head-dim entries 32 bb + 8 a + 4 g + {0..3} of
// accumulator bb in its registers 4a..4a+3 (the C layout of a 32x32 MFMA with one row
// per column lane); stored directly, every store instruction would put 8 bytes into
// each of 32 rows. Staged as bf16 rows (pitch D + 8 elements: 16-byte aligned rows), the
// tile is read back so that D / 8 lanes write one row with 16-byte stores.
template <int D>
constexpr int stage_pitch() { return D + 8; }

template <int D>
__device__ __forceinline__ void stage_acc_rows(u16* stg, const f32x16 (&acc)[D / 32], float mul, int lr, int g) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int bb = 0; bb < D / 32; ++bb)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<bf16x4*>(stg + lr * stage_pitch<D>() + 32 * bb + 8 * a + 4 * g) = __builtin_convertvector(
          f32x4{acc[bb][4 * a] * mul, acc[bb][4 * a + 1] * mul, acc[bb][4 * a + 2] * mul, acc[bb][4 * a + 3] * mul},
          bf16x4);
}

// Writes staged rows 0 .. ROWS-1 that are below `valid`: row r goes to dst + r * stride
// (16-byte aligned rows of D bf16).
template <int D, int ROWS>
__device__ __forceinline__ void store_staged_rows(const u16* stg, u16* __restrict__ dst, size_t stride, int valid,
                                                  int lane) {
  constexpr int LPR = D / 8, RPI = 64 / LPR;  // lanes per row, rows per store instruction
  static_assert(ROWS % RPI == 0, "whole store instructions");
  const int c = lane % LPR, r0 = lane / LPR;
#pragma unroll
  for (int i = 0; i < ROWS / RPI; ++i) {
    const int r = RPI * i + r0;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * stage_pitch<D>() + 8 * c);
    if (r < valid) *reinterpret_cast<u32x4*>(dst + (size_t)r * stride + 8 * c) = v;
  }
}

__device__ __forceinline__ f32x8 half_of(const f32x16& x, int h) {
  return h == 0 ? f32x8{x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]}
                : f32x8{x[8], x[9], x[10], x[11], x[12], x[13], x[14], x[15]};
}

// Reductions over a lane and its mirror lane (l ^ 32). v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second; fed the same
// value twice, its two results hold {x_lo, x_lo} and {x_hi, x_hi}, so combining them
// gives the pair's reduction in every lane.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------------------
// LDS transpose reads (ds_read_b64_tr_b16).
// Within each group of 16 lanes, lane 4k + j supplies the address of an 8-byte run
// (4 bf16) and output lane i receives element (i % 4) of the run supplied by lane
// 4k + i / 4, for k = 0..3. When lane 4k + j points at row (r0 + k), columns
// c0 + 4j .. c0 + 4j + 3 of a row-major tile, output lane i therefore holds column
// c0 + i at rows r0 .. r0 + 3: a 16 x 4 block, transposed.
// ---------------------------------------------------------------------------------------

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ i16x4 ds_read_tr16(const u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(__attribute__((address_space(3))) u16*)p);
}

// A operand (32 rows x 16 k-slots) of an MFMA whose k index runs along the rows of a
// row-major LDS tile `t` (pitch in elements): A row m = tile column c0 + m, and the
// 8 k-slots of lane group g are tile rows {r0 + 4g + 0..3, r0 + 8 + 4g + 0..3}, which
// is exactly the order in which a 32x32 C register file (natural row order) holds
// rows r0 .. r0 + 15 for lane group g in registers 8h .. 8h + 7 (h = r0 / 16 parity).
__device__ __forceinline__ bf16x8 lds_tr_operand(const u16* t, int pitch, int r0, int c0, int lane) {
  const int i = lane & 15;
  const int G = lane >> 4;  // 16-lane group: (lane group g = G / 2, column half G % 2)
  const u16* base = t + (r0 + 4 * (G >> 1) + (i >> 2)) * pitch + c0 + 16 * (G & 1) + 4 * (i & 3);
  const i16x4 lo = ds_read_tr16(base);
  const i16x4 hi = ds_read_tr16(base + 8 * pitch);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// LDS row pitches (in bf16 elements). Row-wise A-operand reads (ds_read_b128) are
// serviced 16 lanes at a time, 16 consecutive rows x 16 bytes: a pitch of 4 (mod 64)
// dwords puts them on distinct banks. Transpose reads (ds_read_b64_tr_b16) are serviced
// 32 lanes at a time, 4 consecutive rows x 64 bytes: a pitch of 16 (mod 64) dwords
// does. (Measured with the LDS bank-conflict counter.) A tile read both ways cannot
// satisfy both and uses pitch_both, which favours the row-wise reads.
template <int D> constexpr int pitch_rows() { return D + 8; }
template <int D> constexpr int pitch_tr() { return D + 32; }
template <int D> constexpr int pitch_both() { return D == 64 ? D + 8 : D + 24; }

// Row (within a 32-row block) held by C register r of lane group g, natural order.
__device__ __forceinline__ int crow_nat(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// ---------------------------------------------------------------------------------------
// Swizzled LDS tiles, for operands read both row-wise and through transpose reads: rows
// of D + 32 bf16 (the D elements, then a 64-byte pad), with 16-byte chunk c of row r
// stored at chunk position c ^ swz_j(r), swz_j(r) = (r >> 2) & 3. Counted in 16-byte
// chunks, the 64 banks are 16 positions, and each row starts 4 (D = 128: 20 chunks per
// row) or 12 (D = 64: 12 chunks) positions after the previous one. Hence
//   row-wise operand reads, 16 lanes = one chunk of 16 consecutive rows (16-aligned):
//     within each group of 4 rows the pitch puts the rows on distinct multiples of 4
//     (bits 2-3), and across the 4 groups the XOR gives distinct low bits;
//   transpose reads, 32 lanes = chunks 4m .. 4m + 3 of 4 consecutive rows (4-aligned):
//     the pitch separates the rows (bits 2-3) and the XOR permutes within the 4 chunks;
// so neither shape has bank conflicts. The XOR never leaves a group of 4 chunks, so data
// stays out of the pads, which are free for other use. The pattern depends on r % 16
// only: tiles whose first row is a multiple of 16 share it. Every address splits into a
// per-lane part that does not depend on the row block or the slice, and a constant.
// ---------------------------------------------------------------------------------------
template <int D>
constexpr int swz_pitch() {
  static_assert(D == 64 || D == 128, "swizzled tiles are 64 or 128 elements wide");
  return D + 32;
}

__device__ __forceinline__ int swz_j(int r) { return (r >> 2) & 3; }

// Row-wise A or B operand from a swizzled tile: lane l reads row r0 + l % 32, elements
// 16 s + 8 g .. + 7 (g = l / 32), i.e. chunk 2 s + g = 4 (s / 2) + (2 (s % 2) + g).
// r0 must be a multiple of 16.
template <int D>
__device__ __forceinline__ bf16x8 swz_row_operand(const u16* t, int r0, int s, int lane) {
  constexpr int P = swz_pitch<D>();
  const int lr = lane & 31, g = lane >> 5;
  const int lane_part = lr * P + 8 * (((2 * (s & 1)) | g) ^ swz_j(lr));
  return *reinterpret_cast<const bf16x8*>(t + lane_part + r0 * P + 32 * (s >> 1));
}

// lds_tr_operand on a swizzled tile. r0 must be a multiple of 16 and c0 of 32.
template <int D>
__device__ __forceinline__ bf16x8 swz_tr_operand(const u16* t, int r0, int c0, int lane) {
  constexpr int P = swz_pitch<D>();
  const int i = lane & 15;
  const int G = lane >> 4;
  const int rl = 4 * (G >> 1) + (i >> 2);            // row within the 16-row group (lo read)
  const int u = 2 * (G & 1) + ((i & 3) >> 1);        // chunk within the group of 4
  const int e = 4 * (i & 1);                         // element within the chunk
  const int lo = rl * P + 8 * (u ^ swz_j(rl)) + e;
  const int hi = (rl + 8) * P + 8 * (u ^ swz_j(rl + 8)) + e;
  const int cst = r0 * P + c0;                       // chunk group c0 / 32 starts at element c0
  const i16x4 a = ds_read_tr16(t + lo + cst);
  const i16x4 b = ds_read_tr16(t + hi + cst);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------------------------------
// Global -> LDS tile staging. `src` points at row 0 of a matrix whose rows are
// `stride` elements apart; rows [r0, r0 + ROWS) are staged and rows >= `len` are
// zero-filled. All NT threads of the workgroup call these together.
// ---------------------------------------------------------------------------------------

// Global -> LDS copies of a tile with global_load_lds_dwordx4: each instruction moves
// 64 lanes x 16 bytes straight into 1 KB of consecutive LDS, with no registers and no
// LDS write instructions, and completes asynchronously (vmcnt). The LDS tile keeps its
// padded row pitch: linear 16-byte chunk L of the tile is row L / CPP, chunk L % CPP
// (CPP = PITCH / 8 chunks per row); lanes that land on a padding chunk copy the row's
// first chunk there, which is never read. Rows at or past `len` are clamped to row
// len - 1: the data is finite and every consumer masks those rows out.
// Global -> LDS copies (global_load_lds_dword / _dwordx4), written as inline asm. Lane i
// of a wave lands its 4 or 16 bytes at LDS address dst + 4 i or dst + 16 i (dst, a
// wave-uniform LDS address, goes to M0). Issued through the compiler builtin instead,
// a copy counts as a pending LDS write that the compiler cannot tell apart from the
// tiles being read: it then waits for every copy in flight (vmcnt(0)) before the next
// LDS read, which undoes a multi-buffer pipeline. Callers wait for the copies
// themselves (wait_vmem, wait_vmem_count) before a barrier that publishes the tile.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// (The s_nop is the wait state an M0 write needs before the copy reads it.)
__device__ __forceinline__ void dma_lds_b128(const void* src, const void* dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_addr(dst)) : "memory");
}

__device__ __forceinline__ void dma_lds_b32(const void* src, const void* dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(src), "{m0}"(lds_addr(dst)) : "memory");
}

// The same copy from a wave-uniform base address plus a per-lane 32-bit byte offset: the
// address add happens in the load, so no 64-bit vector add per copy. The base must be
// the same in every lane; it is read from the first one (where the compiler cannot
// prove it uniform it holds it in VGPRs, and v_readfirstlane moves it to SGPRs). The
// load reads the base from SGPRs that an s_mov in the same asm block has just written:
// an SGPR written by a vector instruction (such as v_readfirstlane) needs five wait
// states before a memory instruction may read it, which the compiler cannot see to
// insert here, while one written by a scalar instruction needs none. The s_mov also
// provides the wait state after the M0 write.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void dma_lds_b128(const void* sbase, uint32_t voff, const void* dst) {
  uint64_t base;
  asm volatile("s_mov_b64 %0, %2\n\tglobal_load_lds_dwordx4 %1, %0"
               : "=&s"(base)
               : "v"(voff), "s"(uniform_ptr(sbase)), "{m0}"(lds_addr(dst))
               : "memory");
}

// A use of x that makes the compiler wait here for the loads that produced it. The
// compiler's own waits are vmcnt(0) (it does not count the asm copies above), so a
// register loaded before a tile loop and first read inside it would cost a wait inside
// the loop, on every trip, for every tile copy in flight. Called once, right after the
// first tile's copy is issued, the wait overlaps that copy instead.
template <typename T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" : : "v"(x));
}

// Workgroup barrier without a memory fence: unlike __syncthreads it does not make the
// compiler wait for outstanding copies; it only keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// With SWZ the tile is a swizzled one (PITCH == swz_pitch<D>()): each lane fetches the
// chunk whose swizzled position is the slot it writes. The pads of rows below
// FREE_PAD_ROWS hold other data: a copy into such a tile (issue with free_pads) skips
// those pad chunks (only the copies that reach these rows carry a lane mask); every
// other pad chunk receives the row's first chunk.
template <int ROWS, int D, int PITCH, int NWAVES, bool SWZ = false, int FREE_PAD_ROWS = 0, bool SADDR = true>
struct TileDma {
  static_assert(PITCH % 8 == 0, "pitch must be a whole number of 16-byte chunks");
  static_assert(!SWZ || (PITCH == D + 32 && ROWS % 16 == 0), "swizzled tiles: pitch D + 32, 16-row aligned");
  static constexpr int CPP = PITCH / 8;
  static constexpr int TOTAL = ROWS * CPP;
  static_assert(TOTAL % 64 == 0, "a tile must be a whole number of 64-chunk copies");
  static constexpr int NINST = TOTAL / 64;
  static constexpr int PER_WAVE = (NINST + NWAVES - 1) / NWAVES;
  static constexpr int MASK_COPIES = (FREE_PAD_ROWS * CPP + 63) / 64;  // copies that reach those rows
  static_assert(!FREE_PAD_ROWS || SWZ, "free pads exist in swizzled tiles only");

  // Byte offset, from the tile's first row in global memory, of the chunk this lane
  // copies in each of its instructions. It does not depend on the tile, so it is
  // computed once. Wave w issues copies w, w + NWAVES, ...; a wave with one copy
  // fewer repeats the last one (same bytes to the same place), which keeps the issue
  // free of branches.
  uint32_t off[PER_WAVE];
  uint32_t pad_bits;  // bit i set when this lane's chunk in copy i is a free pad chunk

  __device__ __forceinline__ static int copy_index(int w, int i) { return min(w + i * NWAVES, NINST - 1); }

  // Chunk of global row `row` that lands in chunk slot c of the LDS row.
  __device__ __forceinline__ static int src_chunk(int row, int c) {
    if constexpr (SWZ)
      return c < D / 8 ? c ^ swz_j(row) : 0;
    else
      return c < D / 8 ? c : 0;
  }

  __device__ __forceinline__ void init(size_t stride, int w, int lane) {
    pad_bits = 0;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int L = 64 * copy_index(w, i) + lane;
      const int row = L / CPP, c = L % CPP;
      off[i] = (uint32_t)(((size_t)row * stride + 8 * src_chunk(row, c)) * sizeof(u16));
      if (c >= D / 8 && row < FREE_PAD_ROWS) pad_bits |= 1u << i;
    }
  }

  // Copy i of a full tile: from the SGPR base plus this lane's offset, or (SADDR false)
  // from a 64-bit vector address (measured faster in the dK/dV kernel, whose copies sit
  // among scalar-heavy code; the others gain from the address add leaving the VALU).
  __device__ __forceinline__ void copy_full(const char* base, int i, u16* dst) const {
    if constexpr (SADDR)
      dma_lds_b128(base, off[i], dst);
    else
      dma_lds_b128(base + off[i], dst);
  }

  // Copy rows [r0, r0 + ROWS) of `src` into `dst` (w: the wave index, uniform). Rows at
  // or past `len` are copies of row len - 1 (the consumer masks them). The body is
  // compiled for the device only: hipcc's host pass otherwise drops (without a
  // diagnostic) the launch stubs of kernels that inline this control flow.
  __device__ __forceinline__ void issue(u16* dst, const u16* __restrict__ src, int r0, int len, size_t stride,
                                        int w, int lane, bool free_pads = true) const {
#if __HIP_DEVICE_COMPILE__
    if (r0 + ROWS <= len) {  // wave-uniform: a full tile
      const char* base = reinterpret_cast<const char*>(src + (size_t)r0 * stride);
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int k = copy_index(w, i);
        // i * NWAVES is copy i's smallest index: later copies never reach the free pads
        if (free_pads && i * NWAVES < MASK_COPIES && k < MASK_COPIES) {  // wave-uniform
          if (!((pad_bits >> i) & 1)) copy_full(base, i, dst + 512 * k);
        } else {
          copy_full(base, i, dst + 512 * k);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int k = copy_index(w, i);
        const int L = 64 * k + lane;
        const int row = L / CPP, c = L % CPP;
        const int grow = min(r0 + row, len - 1);
        const u16* g = src + (size_t)grow * stride + 8 * src_chunk(row, c);
        if (!(free_pads && c >= D / 8 && row < FREE_PAD_ROWS)) dma_lds_b128(g, dst + 512 * k);
      }
    }
#endif
  }
};

// Wait for this wave's outstanding global loads (including LDS DMA) to land.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N of this wave's global loads are outstanding (they complete in
// issue order, so everything issued before the newest N has landed).
template <int N>
__device__ __forceinline__ void wait_vmem_count() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace fa
