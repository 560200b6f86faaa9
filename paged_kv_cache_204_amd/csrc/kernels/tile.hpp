// MFMA tile helpers shared by the attention kernels of this library:
// pool addressing, LDS DMA and transposing LDS reads, explicit load-counter
// waits and the swizzled K/V tile layout in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../kernels.hpp"

namespace pkv {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;


// K or V of layer p.layer, kv head h, as 16-byte chunks: token slot `off` of
// block `blk` starts at chunk blk * (Hkv * B * D / 8) + off * D / 8.  The pool
// creation keeps a layer under 2^32 chunks and a block under 2^24 chunks, so
// the index is one 24-bit multiply-add in 32 bits.
__host__ __device__ inline const uint4* layer_head_base(const AttnParams& p, const uint16_t* pool,
                                                        int h, int D) {
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * p.B * D;
  return reinterpret_cast<const uint4*>(pool + static_cast<size_t>(p.layer) * p.N * blk_stride +
                                        static_cast<size_t>(h) * p.B * D);
}

__device__ __forceinline__ uint32_t chunk_index(int32_t blk, uint32_t blk_chunks, int32_t within) {
  return __umul24(static_cast<uint32_t>(blk), blk_chunks) + static_cast<uint32_t>(within);
}

// Row r of an item belongs to row group r / G (query head r % G of the kv
// head's group).  G is a run-time value of at most 16 and r stays below
// 1024, so r * ceil(2^16 / G) >> 16 is exactly r / G (the rounding of the
// multiplier adds less than 1/64 to a quotient whose fraction is at most
// 15/16), one multiply instead of an integer division sequence.
struct RowOf {
  int grp, head;
};
__device__ __forceinline__ RowOf row_of(const AttnParams& p, int r) {
  const int grp = static_cast<int>((static_cast<uint32_t>(r) * p.g_magic) >> 16);
  return {grp, r - grp * p.G};
}

// ---------------------------------------------------------------- MFMA path
constexpr int kStep = 32;          // key tokens per step (two 16-token tiles)
constexpr float kSlack = 8.f;      // log2 headroom of P above the reference max

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// global_load_lds_dwordx4: lane i copies the 16 bytes at `src` to LDS byte
// lds + 16 i (lds wave-uniform, through M0).  Issued as inline assembly so
// the compiler's wait insertion, which would treat the LDS write as aliasing
// every later LDS read and drain all loads before them, leaves it alone: its
// completion is awaited explicitly with wait_vmcnt.  (A load the compiler
// tracks is still awaited correctly: these only add younger entries to the
// in-order count.)
__device__ __forceinline__ void lds_dma16(const uint4* src, const void* lds) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_ptr)(lds)));
  uint32_t saved;
  // M0 is put back as it was, so the compiler's own use of it is undisturbed
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(m0)
      : "memory");
}

// The same copy from a wave-uniform base address plus a 32-bit per-lane
// byte offset (the SGPR-base form of the instruction): no 64-bit address
// arithmetic per lane.
__device__ __forceinline__ void lds_dma16_at(const void* base, uint32_t off, const void* lds) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_ptr)(lds)));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(m0)
      : "memory");
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 4-element rows named by lanes 4k + i / 4, for k = 0..3.
__device__ __forceinline__ v4i16 lds_read_tr16(const void* at) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(at));
}

// s_waitcnt vmcnt(N), the other counters left alone (vmcnt sits in bits
// 3:0 and 15:14 of the immediate, expcnt in 6:4, lgkmcnt in 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// s_waitcnt vmcnt(STEP * n) for 0 <= n <= MAXN (n a constant once unrolled;
// a larger n waits for STEP * MAXN).
template <int STEP, int MAXN>
__device__ __forceinline__ void wait_vmcnt_steps(int n) {
  if constexpr (MAXN > 0) {
    if (n >= MAXN) {
      wait_vmcnt<STEP * MAXN>();
      return;
    }
    wait_vmcnt_steps<STEP, MAXN - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// A step's K or V tile in LDS: 32 token rows of D bf16 without padding.  The
// 16-byte chunk c of row r sits in chunk slot c ^ tile_swz(r), so the 16 rows
// that one MFMA operand read touches fall on distinct banks.
template <int D>
__device__ __forceinline__ int tile_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int tile_byte(int r, int c) { return r * (2 * D) + ((c ^ tile_swz<D>(r)) << 4); }

// Orders this wave's LDS writes before its later LDS reads (no other wave
// takes part, so no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

}  // namespace pkv
