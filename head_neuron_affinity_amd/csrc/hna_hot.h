// Device helpers of the hot affinity kernels (gfx950): explicit vector-memory
// waits, untracked buffer loads into accumulation registers, asynchronous
// buffer -> LDS copies, raw buffer resources and compile-time loops.
#pragma once

#include <utility>

#include "hna_internal.h"

namespace hna {
namespace hot {

constexpr int pow2_slots(int cpr) { return cpr <= 8 ? 8 : (cpr <= 16 ? 16 : 32); }

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (LGKM and export counters untouched).
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Untracked 16-byte buffer load into four accumulation registers (MFMA
// operands may come from them): dst = the 16 bytes at voff of resource rs.
// The compiler does not count it; the caller waits for it with an explicit
// vmcnt that names dst as an operand (so dst is neither read nor reused
// before the data has landed).
__device__ inline void bload16(u32x4& dst, __amdgpu_buffer_rsrc_t rs, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=a"(dst) : "v"(voff), "s"(rs));
}
// The same at voff + OFF, OFF a compile-time byte offset: the multiple of 4096
// goes in the scalar offset, the rest in the instruction's offset field.  (The
// range check covers voff only: for reads that are in range by construction.)
template <int OFF>
__device__ inline void bload16_at(u32x4& dst, __amdgpu_buffer_rsrc_t rs, uint32_t voff) {
  constexpr uint32_t hi = OFF & ~4095u, lo = OFF & 4095u;
  if constexpr (hi == 0)
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen offset:%3"
                 : "=a"(dst) : "v"(voff), "s"(rs), "n"(lo));
  else
    asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen offset:%4"
                 : "=a"(dst) : "v"(voff), "s"(rs), "s"(hi), "n"(lo));
}

// s_waitcnt vmcnt(N) that also names the registers it guards as operands, so
// the compiler cannot move their uses (or reuse them) ahead of the wait.
template <int N>
__device__ inline void vm_wait_tied(u32x4& x, u32x4& y) {
  asm volatile("s_waitcnt vmcnt(%2)" : "+a"(x), "+a"(y) : "n"(N));
}
template <int N>
__device__ inline void vm_wait_tied(u32x4& x, u32x4& y, u32x4& z, u32x4& w) {
  asm volatile("s_waitcnt vmcnt(%4)" : "+a"(x), "+a"(y), "+a"(z), "+a"(w) : "n"(N));
}

// Empty statement that names x as read and written: uses of x placed after it
// cannot move above an earlier volatile statement (such as a wait), and x is
// not reused before it.
__device__ inline void tie(u32x4& x) { asm volatile("" : "+a"(x)); }

// Calls f(IC<B>), f(IC<B+1>), ..., f(IC<E-1>) (a loop with a compile-time index).
template <int B, int E, typename F>
__device__ inline __attribute__((always_inline)) void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zeros (hardware range check), so tile edges need no clamping.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000 /* 32-bit data format, no swizzle */);
}
constexpr uint32_t kOutOfRange = 0x7ffffff0u;   // offset past any resource: reads zeros

// Asynchronous 16-byte buffer -> LDS copy: lane l copies the 16 bytes at
// voff of resource rs (voff is what the range check covers) and writes them
// at LDS address lds_base + OFF + 16 l (lds_base wave-uniform).  Issued as
// inline assembly on purpose: the compiler then does not track the LDS write,
// so it adds no vmcnt wait before reads of the other buffer (the kernel orders
// every copy itself with explicit vmcnt waits and barriers).
template <int OFF>
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds"
               :: "s"(lds_base), "n"(OFF), "v"(voff), "s"(rs) : "memory", "scc");
}
// LDS address of a workgroup-shared object
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr)const_cast<void*>(p);
}


}  // namespace hot
}  // namespace hna
