// Buffer loads straight into LDS (gfx950 "buffer_load ... lds"), shared by
// the forward and backward kernels.  A tile is filled in 1 KB segments: one
// wave-wide load writes 16 bytes per lane at consecutive LDS addresses, so a
// padded row layout is produced by giving each lane the source offset of
// the element that belongs at its LDS position (padding positions get an
// offset past the buffer's range and read zeros).
#pragma once
#include "device.hpp"

namespace pn {

// Byte offset, inside one tile, that lane `lane` of segment `seg` fills, as
// a source offset relative to the tile's first key row (or ~0 for padding
// slots, which the bounds-checked load turns into a harmless zero fill).
__device__ __forceinline__ uint32_t seg_src_offset(int seg, int lane, int row_bytes, int stride) {
  const int pos = (seg * 64 + lane) * 16;
  const int row = pos / stride, col = pos % stride;
  return col < row_bytes ? (uint32_t)(row * row_bytes + col) : 0x7ffffff0u;
}

// Buffer resource descriptor (V#) over `bytes` bytes at `base`: loads at
// offsets >= bytes return zeros (the hardware range check), which is how key
// rows past the end of the sequence arrive as zeros.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)((a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

__device__ __forceinline__ i32x4 uniform(i32x4 x) {
  return i32x4{__builtin_amdgcn_readfirstlane(x[0]), __builtin_amdgcn_readfirstlane(x[1]),
               __builtin_amdgcn_readfirstlane(x[2]), __builtin_amdgcn_readfirstlane(x[3])};
}

// One wave-wide buffer load of 16 (or 4) bytes per lane straight into LDS at
// lds_addr + 16*lane (4*lane).  Issued through inline asm on purpose: the
// compiler's wait-count pass cannot tell which LDS bytes such a load writes,
// so it would make the next LDS read of ANY tile wait for it, serialising
// the prefetch.  Every wait these loads need is explicit in the kernel
// (s_waitcnt vmcnt(0) before the barrier that publishes a tile); compiler-
// generated waits for other memory operations only become more conservative.
template <int IMM = 0>
__device__ __forceinline__ void lds_load16(i32x4 rsrc, uint32_t voff, uint32_t soff,
                                           uint32_t lds_base) {
  // M0 carries the LDS destination, lds_base + IMM, formed inside the asm so
  // the compiler keeps one base instead of one register per destination;
  // M0 is declared clobbered, so the compiler re-establishes any value of
  // its own after the load.  The scalar operands are wave-uniform; the
  // read-first-lanes only tell the register allocator so (it may otherwise
  // have moved a uniform value into vector registers).
  rsrc = uniform(rsrc);
  soff = __builtin_amdgcn_readfirstlane(soff);
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile(
      "s_add_u32 m0, %3, %4\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_base), "i"(IMM)
      : "memory", "m0", "scc");
}
__device__ __forceinline__ void lds_load4(i32x4 rsrc, uint32_t voff, uint32_t soff,
                                          uint32_t lds_addr) {
  rsrc = uniform(rsrc);
  soff = __builtin_amdgcn_readfirstlane(soff);
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile(
      "s_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "buffer_load_dword %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_addr)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

}  // namespace pn
