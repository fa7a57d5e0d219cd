// Global -> LDS DMA on gfx950 (buffer_load ... lds), shared by the bf16 GEMM
// and the column projection.
//
// One instruction moves 16 bytes per lane from a buffer (descriptor + per-lane
// byte offset + uniform byte offset) to LDS at M0 + 16 * lane, so a wave fills
// 1 KB of LDS linearly and any layout swizzle is applied by choosing which
// global chunk each lane fetches. Offsets at or past the descriptor's
// num_records read as zero, which is how tails and out-of-range rows are
// filled without branches.
//
// The instruction is issued from a one-instruction asm block: it writes no
// register (only LDS), so the compiler tracks nothing for it. Issued through
// the builtin, the compiler would make every later LDS read wait for all DMA
// in flight, because it cannot tell the stages of a ring apart; that drains
// the ring at each fragment read. Callers therefore wait explicitly
// (wait_vmcnt, then a barrier) before reading a stage, and drain with
// wait_vmcnt<0>() before the workgroup exits. A kernel that issues DMA must
// not mix in compiler-tracked vector memory loads whose results it waits for
// while DMA is in flight: the compiler would count only its own loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmlp {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));

constexpr uint32_t DMA_OOB = 0x80000000u;  // a buffer offset that fails the range check

// buffer descriptor: base address, stride 0, num_records = nbytes, raw-buffer flags
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  rsrc_t r;
  r.x = static_cast<uint32_t>(a);
  r.y = static_cast<uint32_t>(a >> 32) & 0xFFFFu;
  r.z = nbytes;
  r.w = 0x00020000u;
  return r;
}

// 16 bytes per lane from (r, voff + soff) to LDS at lds + 16 * lane. M0
// carries the LDS address; s_nop 0 covers the M0-write-to-LDS-DMA hazard.
__device__ __forceinline__ void dma16(rsrc_t r, const void* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)lds));
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(r), "s"(soff), "{m0}"(m0)
      : "memory");
}

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Swizzle of 16-byte chunk positions in an N-major [k][256 n] bf16 tile row
// (512 bytes): chunk c of row k sits at position c ^ nn_swz(k). The rows one
// transposing read touches (4 consecutive k, and k + 4) then map a pair of
// chunks to 8 distinct pairs of bank groups.
__device__ __forceinline__ int nn_swz(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }

}  // namespace lmlp
