// Direct loads from memory into LDS for the multi-query kernel's staging
// ring: gfx950's buffer loads with the lds bit, issued from inline assembly
// and ordered by explicit vmcnt waits and barriers.
#ifndef PA_LDS_DMA_H_
#define PA_LDS_DMA_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef int i32x4_t __attribute__((ext_vector_type(4)));  // a buffer descriptor (V#)

// Descriptor of `bytes` bytes at `base` (both wave-uniform): raw (stride 0,
// no swizzle), 32-bit data format.  Each word goes through readfirstlane so
// that the descriptor is built in SGPRs, as the instruction requires, even
// where the compiler computed a uniform value in a VGPR.
__device__ __forceinline__ i32x4_t raw_buffer(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from memory straight into LDS through a raw buffer
// descriptor (buffer_load_dwordx4 with the lds bit): lane i reads byte offset
// voffset of the buffer and writes lds_base + 16 i, lds_base being
// wave-uniform.  Lanes whose offset lies at or past the descriptor's record
// count read nothing and write zeros (both checked on the hardware).  The
// load counts in vmcnt like any vector load.  It is issued from assembly so
// that the compiler, which cannot tell which LDS bytes such a load writes,
// does not put a full vmcnt wait before every later LDS read; callers order
// it with vm_wait and block_barrier.  lds_base is an M0 operand, so the
// compiler writes M0 right before the instruction and knows it holds that
// value; the nop is the wait state an M0 write needs before such a load.
template <bool kNonTemporal>
__device__ __forceinline__ void buffer_load_lds16(uint32_t voffset, i32x4_t rsrc, uint32_t lds_base) {
  if constexpr (kNonTemporal)
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :: "v"(voffset), "s"(rsrc), "{m0}"(lds_base) : "memory");
  else
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voffset), "s"(rsrc), "{m0}"(lds_base) : "memory");
}

// The same with a wave-uniform byte offset in the scalar offset operand:
// lanes read base + soffset + voffset, and soffset + voffset is what the
// range check compares with the record count (checked on the hardware: with
// a one-page record count every lane past the first page read zeros).
template <bool kNonTemporal>
__device__ __forceinline__ void buffer_load_lds16(uint32_t voffset, i32x4_t rsrc, uint32_t soffset, uint32_t lds_base) {
  if constexpr (kNonTemporal)
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds"
                 :: "v"(voffset), "s"(rsrc), "s"(soffset), "{m0}"(lds_base) : "memory");
  else
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voffset), "s"(rsrc), "s"(soffset), "{m0}"(lds_base) : "memory");
}

// LDS byte address of a pointer into __shared__ memory, made wave-uniform.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p)));
}

// Waits until at most N of this wave's vector memory loads are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier after this wave's LDS reads have completed; no vmcnt
// wait (loads still in flight into other LDS buffers stay in flight).
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace pa

#endif  // PA_LDS_DMA_H_
