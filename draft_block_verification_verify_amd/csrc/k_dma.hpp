// Direct global -> LDS copies on gfx950 (buffer_load ... lds) and the
// explicit wait that goes with them.  Shared by the attention and projection
// kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

// ----------------------------------------------------------------------------
// Direct global -> LDS copies (gfx950 buffer_load ... lds).  A wavefront
// writes 64 x 16 B = 1 KB of LDS per instruction, lane l at byte 16 l of the
// wave's destination; the global address of each lane is free, so a tile is
// laid out XOR-swizzled in LDS by choosing which 16-B chunk a lane fetches.
// Rows past the end of a tensor are outside the buffer's range and read 0.
// ----------------------------------------------------------------------------

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor: base, no stride, `bytes` in range (raw-buffer bounds
// check on the per-lane offset), default data format.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = int(uint32_t(a));
  r.y = int(uint32_t(a >> 32) & 0xFFFFu);
  r.z = int(bytes);
  r.w = 0x00020000;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return uint32_t(reinterpret_cast<uintptr_t>(p));
}

// 16 B per lane from base(rsrc) + soff + voff into LDS at m0 + 16 * lane.
// Issued through inline asm so that the compiler does not add its own
// whole-queue waits; completion is tracked with wait_and_barrier.
__device__ __forceinline__ i32x4 uniform(i32x4 r) {
  r.x = __builtin_amdgcn_readfirstlane(r.x);
  r.y = __builtin_amdgcn_readfirstlane(r.y);
  r.z = __builtin_amdgcn_readfirstlane(r.z);
  r.w = __builtin_amdgcn_readfirstlane(r.w);
  return r;
}

// NT: the non-temporal hint, for data streamed once per step (weights, KV)
template <bool NT = false>
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_wave_dst, int voff, int soff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_wave_dst);
  const i32x4 rs = uniform(rsrc);
  const int so = __builtin_amdgcn_readfirstlane(soff);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :
                 : "s"(m0v), "v"(voff), "s"(rs), "s"(so)
                 : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0v), "v"(voff), "s"(rs), "s"(so)
                 : "memory");
}

// Streams read once per step (the projection weights, the KV cache) carry
// the non-temporal hint.  Measured with the caches flushed by 512 MB of
// writes before each step, it takes an 8-row LM head over 151936 x 4096 fp16
// weights from 266 to 197 us, and attention over 32 sequences of 1k-16k
// cached tokens (1.2 GB of K and V) from 280 to 230 us: the stream no longer
// displaces, and forces the write-back of, the lines other data left behind.
constexpr bool kNtStream = true;

// Wait until at most N vector-memory operations of this wave are pending,
// then a workgroup barrier (no other memory fence).
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

}  // namespace sv
