// Cross-workgroup hand-over of the decode kernels' rank-space intermediate:
// the workspace header, device-coherent loads and stores, and the call tag.
#pragma once

#include "lb_common.h"

// workspace header (bytes): one 64-bit call counter per workgroup of the
// single launch, then an error word set when a poll gives up.
#define LB_SYNC_CTR 0  // + 8 * workgroup
#define LB_SYNC_ERR 2048
#define LB_SPIN_LIMIT (1 << 20)  // polls of one wait before it gives up

__device__ inline uint32_t ld32c(const void* p) {
  return __hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st32c(void* p, uint32_t v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st64c(void* p, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void add64c_noret(void* p, uint64_t v) {
  (void)__hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Raw buffer resource over `bytes` bytes (loads beyond return 0).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// 16 bytes (two tagged z words) with a device-coherent (sc1) load.
__device__ inline u32x4 ld_tagged2(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 16 /* sc1 */);
}

// The z tag of a single-launch call from the workgroup's call counter: the
// counter + 1, skipping 0 when the 32-bit value wraps.  Tag 0 marks z stored
// by the two-launch path (phase A alone), so no poll ever accepts it.
__device__ inline uint32_t call_tag(uint32_t ctr) {
  const uint32_t t = ctr + 1u;
  return t + (t == 0u ? 1u : 0u);
}

// Compiler-only barrier: memory may have changed here, so loads after it are
// neither hoisted above it nor merged with loads before it.
__device__ inline void compiler_memory_barrier() { __asm__ volatile("" ::: "memory"); }

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Hands `v` to the compiler as if modified here, so work that depends on it
// (and the wait for the load that produced it) is not hoisted above this point.
__device__ inline uint32_t late(uint32_t v) {
  __asm__ volatile("" : "+v"(v));
  return v;
}
