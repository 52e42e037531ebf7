// Buffer-resource loads on gfx950: bounds-checked global reads that return 0
// beyond the resource's byte range, either into registers or straight into LDS
// (buffer_load_dword{,x4} ... lds).  Measured placement of the LDS form: lane i
// of a wave writes its 4 or 16 bytes at the wave-uniform LDS address + i*size.
#pragma once
#include "common.h"

namespace slope {

typedef __attribute__((address_space(3))) void lds_void;

// Byte offset that is always beyond a resource (resources are kept below 2 GiB).
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // raw (stride 0) resource; num_records in bytes, clamped below 2 GiB
  const int n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// 16 bytes from resource offset `off` to LDS at `lds_wave_base + lane*16`.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 16, off, 0, 0, 0);
}
// 4 bytes from resource offset `off` to LDS at `lds_wave_base + lane*4`.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 4, off, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Compiler-only fence (emits no instruction): no load, store or LDS access of
// this wave is moved across it.  The waits and the barrier below are not
// memory operations to the compiler, so a kernel whose loads must stay on one
// side of them (register loads counted by a following wait_vmcnt, LDS reads
// that must follow a barrier with nothing in between to pin them) places one.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Wait until this wave's LDS reads (and other LGKM operations) have completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

// Workgroup barrier without the memory fence of __syncthreads(): the LDS
// traffic it orders is waited for explicitly with wait_vmcnt / lgkmcnt.
__device__ __forceinline__ void barrier() { __builtin_amdgcn_s_barrier(); }

}  // namespace slope
