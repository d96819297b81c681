// Device helpers shared by the MFMA kernels of libtpmlp.so (gemm.hip,
// skinny.hip): buffer resources and buffer-to-LDS DMA of operand tiles, the
// swizzled LDS layouts and the fragment reads that go with them.
//
// Operand tiles are 64 deep in k.  A k-contiguous tile [R rows][64 k] is
// stored as 128-byte rows of 16-byte chunks, chunk c of row r at slot
// c ^ (r & 7), and read with ds_read_b128.  An m/n-contiguous tile
// [64 k][RW cols] is stored as k-rows of RW/8 chunks, chunk c of k-row r at
// slot c ^ mn_swz(r), and read with ds_read_b64_tr_b16, the gfx950 LDS
// transpose read (two per 8-k fragment).  One MFMA operand fragment covers 16
// rows (or columns) x 32 k: lane l holds index l % 16, k = 8*(l/16) .. +7.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.h"

namespace tpmlp {

constexpr uint32_t OOB = 0xFFFFFFF0u;         // past the end of any accepted buffer
constexpr int RSRC_FLAGS = 0x00020000;        // raw buffer, 32-bit data

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RSRC_FLAGS);
}
__device__ __forceinline__ void dma16(rsrc_t r, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, 0, 0, 0);
}
// s_waitcnt with only the vector-memory counter constrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// A bare barrier: no implied waits (outstanding DMA stays in flight), and a
// compiler barrier for memory operations.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// DMA of a k-contiguous operand tile: R rows x 64 k into [row][8 chunks].
// One wave instruction fills 1 KiB = 8 rows; lane i of instruction j of wave
// q holds LDS chunk p = (q + 4j)*64 + i: row p/8, slot p%8, which holds the
// logical chunk slot ^ (row & 7) -- the same chunk for every j.
// ---------------------------------------------------------------------------
template <int R>
struct DmaK {
  static constexpr int NI = R / 32;  // instructions per wave per tile
  uint32_t voff[NI];                 // row*ld*2 + chunk*16 (bytes from the tile's first k), or OOB
  int kc;                            // element offset of the lane's chunk in the tile
  __device__ __forceinline__ void init(int row0, int rows, int64_t ld, int lane, int q) {
    kc = ((lane & 7) ^ ((lane >> 3) & 7)) * 8;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = (q + 4 * j) * 8 + (lane >> 3);
      const int grow = row0 + r;
      voff[j] = grow < rows ? (uint32_t)((int64_t)grow * ld * 2) + (uint32_t)kc * 2u : OOB;
    }
  }
  // instruction J of a tile; rs addresses the operand from the tile's first
  // k; chunks at or past kvalid (elements from the tile's first k) read zeros
  template <int J>
  __device__ __forceinline__ void issue(rsrc_t rs, uint8_t* region, int kvalid, int q) const {
    dma16(rs, region + (q + 4 * J) * 1024, kc < kvalid ? voff[J] : OOB);
  }
};

// ---------------------------------------------------------------------------
// DMA of an m/n-contiguous operand tile: 64 k-rows x RW columns into
// [k][RW/8 chunks]; chunk c of k-row r at slot c ^ mn_swz(r).
//
// The transposed fragment read has each 16-lane group read 32 bytes from each
// of 4 k-rows (8g + 0..3, g = lane / 16), and 32 lanes are served per pass
// over the 64 four-byte banks.  2(r&3) spreads one group's 4 rows over 128
// bytes of banks; bit 3 of r (g odd) moves the other group of the pass to the
// other 128 bytes: XOR 8 chunks when a k-row is a multiple of 256 bytes long,
// XOR 2 chunks when it is an odd multiple of 128 bytes (rows then alternate
// bank halves by themselves).
// ---------------------------------------------------------------------------
template <int RW>
__device__ __forceinline__ int mn_swz(int r) {
  static_assert((RW * 2) % 128 == 0, "k-row length");
  constexpr int X = ((RW * 2) % 256 == 0) ? 8 : 2;
  return (2 * (r & 3)) ^ (X * ((r >> 3) & 1));
}
template <int RW>
struct DmaMN {
  static constexpr int CPR = RW / 8;
  static constexpr int NI = RW / 32;
  static_assert(CPR % 8 == 0, "tile width");
  uint32_t voff[NI];  // krow*ld*2 + col*2 (bytes from the tile's first k row), or OOB
  __device__ __forceinline__ void init(int col0, int cols, int64_t ld, int lane, int q) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int p = (q + 4 * j) * 64 + lane;
      const int kr = p / CPR;
      const int chunk = (p % CPR) ^ mn_swz<RW>(kr);
      const int col = col0 + chunk * 8;
      voff[j] = col < cols ? (uint32_t)((int64_t)kr * ld * 2) + (uint32_t)col * 2u : OOB;
    }
  }
  // instruction J of a tile; rs addresses the operand from the tile's first k
  // row and ends with the operand, so k rows past the end read zeros
  template <int J>
  __device__ __forceinline__ void issue(rsrc_t rs, uint8_t* region, int q) const {
    dma16(rs, region + (q + 4 * J) * 1024, voff[J]);
  }
};

// ---------------------------------------------------------------------------
// Fragment reads (16 rows/columns x 32 k of one MFMA operand, 8 bf16 per lane:
// lane l holds index l%16, k = 8*(l/16) .. +7 of the k-step).
// ---------------------------------------------------------------------------
// k-contiguous region: byte offset of the lane's fragment for block row base
// rb, k-step s; block i adds i*2048.
__device__ __forceinline__ int kfrag_off(int rb, int s, int lane) {
  const int l16 = lane & 15, lq = lane >> 4;
  return (rb + l16) * 128 + (((s * 4 + lq) ^ (l16 & 7)) << 4);
}
// m/n-contiguous region of width RW: per-lane k-row byte base and the column
// part of block i (columns cb + 16 i .. +15).
template <int RW>
__device__ __forceinline__ int mn_kbase(int lane) {
  const int g = lane >> 4, src = lane & 15;
  return (8 * g + (src >> 2)) * (RW * 2);
}
// (the lane's k-row is 8*(lane/16) + (lane%16)/4 plus multiples of 4 and 32,
// which leave its low two bits and bit 3 unchanged)
template <int RW>
__device__ __forceinline__ int mn_coloff(int cb, int i, int lane) {
  const int src = lane & 15;
  const int chunk = (cb + 16 * i + 4 * (src & 3)) >> 3;
  const int r = 8 * (lane >> 4) + (src >> 2);
  return ((chunk ^ mn_swz<RW>(r)) << 4) + (src & 1) * 8;
}
// The LDS reads and MFMAs are volatile inline asm: they issue in source
// order, and the compiler inserts no waits for the buffer-to-LDS loads in
// flight (it cannot tell the regions apart).  LDS read results are consumed
// only after an explicit lgkmcnt(0) wait.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <int OFF>
__device__ __forceinline__ bf16x8 ld_b128(uint32_t addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ v4i16 tr16(uint32_t addr) {
  v4i16 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
template <int OFF0, int OFF1>
__device__ __forceinline__ bf16x8 ld_tr2(uint32_t addr) {
  const v4i16 lo = tr16<OFF0>(addr);
  const v4i16 hi = tr16<OFF1>(addr);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl<0, N>(f); }

}  // namespace tpmlp
