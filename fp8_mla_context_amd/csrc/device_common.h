// Device helpers shared by the attention kernels: global->LDS DMA with explicit
// completion waits, a bare workgroup barrier and wave-uniform pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {
namespace dev {

// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_address(const uint8_t* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p));
}

// global_load_lds_dwordx4 from base + off (base wave-uniform, off per lane) to LDS
// address lds_addr + 16 * lane. Issued as inline assembly so that the compiler does not
// wait for it before unrelated LDS reads; completion is tracked with wait_vmcnt. The LDS
// address goes in through an m0 operand, so the compiler writes m0 itself and knows it
// (m0 cannot be declared clobbered); the nop is the wait state between that write and
// the DMA.
__device__ __forceinline__ void dma_load16(const uint8_t* base, uint32_t off, uint32_t lds_addr) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "{m0}"(lds_addr)
      : "memory");
}

// wait until at most n (wave-uniform, 0..15) vector-memory loads of this wave are outstanding
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
  }
}

// workgroup barrier without the blanket memory wait of __syncthreads (every LDS read
// before it has been consumed by an MFMA, so it has completed)
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// a pointer that is the same in every lane, kept in scalar registers
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ float vmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

}  // namespace dev
}  // namespace mla
