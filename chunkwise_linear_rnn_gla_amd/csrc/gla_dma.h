// gla_dma.h -- asynchronous global -> LDS copies (LDS-DMA through buffer
// resources) and the memory-counter waits the staging loops use (gfx950).
#pragma once

#include "gla_common.h"

namespace gla {

// Asynchronous global -> LDS copy through a buffer resource: 16 bytes at
// rsrc base + soff + voff (voff per lane, soff wave-uniform) into LDS at
// lds_wave_base + 16 * lane.
// The copy is issued from inline assembly: the instruction writes no
// register, and the compiler, which cannot tell which LDS bytes a copy
// writes, would otherwise wait for every outstanding copy (including the
// prefetch of a later chunk) before the next LDS read.  Completion is waited
// for explicitly (wait_vm) before a staged buffer is read.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
__device__ inline i32x4 make_rsrc(const void* base) {
  // raw buffer: stride 0, range 2 GiB, 32-bit data format
  const unsigned long long a = (unsigned long long)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32) & 0xffff);
  r[2] = 0x7fffffff;
  r[3] = 0x00020000;
  return r;
}
// lds_wave_base: LDS byte address (wave-uniform).  The instruction takes it
// in M0, which the "{m0}" operand asks the compiler to load: the compiler
// then knows M0's contents at this point and keeps any value of its own
// there safe, so the statement has no hidden effect on registers.
__device__ inline void dma16b(const i32x4& r, unsigned voff, unsigned soff, unsigned lds_wave_base) {
  asm volatile("buffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "{m0}"(__builtin_amdgcn_readfirstlane(lds_wave_base)), "v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}
// LDS byte address of a __shared__ object.
template <typename P>
__device__ inline unsigned lds_addr(P* p) {
  return (unsigned)(size_t)(__attribute__((address_space(3))) void*)p;
}
// Wait until at most N of this wave's global memory operations are
// outstanding.  Loads complete in issue order, so in a wave that issues only
// loads this waits for all but the last N.
template <int N>
__device__ inline void wait_vm_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory"); }
// Wait for this wave's outstanding global memory operations (LDS copies too).
__device__ inline void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Prefetch into the caches: a 4-byte asynchronous LDS copy per lane from byte
// 128 l of [base, base + bytes) (lanes past the end read nothing), one per
// 128-byte line of an 8 KB piece.  The LDS bytes written at lds_dummy +
// 4 * lane are never read.
__device__ inline void touch_lines(const void* base, int bytes, int l, unsigned lds_dummy) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const unsigned long long a = (unsigned long long)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32) & 0xffff);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000;
  // M0 (the LDS address) is an operand the compiler loads ("{m0}"), not a
  // register the statement sets behind its back
  asm volatile("buffer_load_dword %1, %2, %3 offen lds"
               :
               : "{m0}"(__builtin_amdgcn_readfirstlane(lds_dummy)), "v"((unsigned)l * 128u), "s"(r),
                 "s"(0u)
               : "memory");
}

}  // namespace gla
