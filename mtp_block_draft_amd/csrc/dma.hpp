// Building blocks of the LDS-ring matrix kernels: 16-byte global -> LDS copies
// (global_load_lds_dwordx4, which writes lane i's 16 bytes at the LDS base +
// 16 i), the explicit memory-counter waits that pipeline them, the XOR swizzle
// of the staged tiles and the 32 x 32 x 16 bf16 MFMA.
#pragma once

#include "common.hpp"

namespace dmtp {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16).  Lane l supplies row
// (l % 32) of A and column (l % 32) of B, k values 8 (l / 32) .. + 7; element i
// of D sits at row 8 (i / 4) + 4 (l / 32) + (i % 4), column l % 32.
__device__ __forceinline__ f32x16_t mfma32(const u32x4& a, const u32x4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Position of 16-byte chunk c of row r in a [rows][BK] bf16 tile (an
// involution: it also gives the chunk stored at position c).  The XOR keeps the
// 16 rows that one LDS read pass touches on distinct 16-byte positions of the
// 256-byte bank window: (r >> 2) & 3 for 64-byte rows, (r >> 1) & 7 for
// 128-byte rows.
template <int BK>
__device__ __forceinline__ int swz_chunk(int r, int c) {
  static_assert(BK == 32 || BK == 64, "row width");
  return BK == 32 ? (c ^ ((r >> 2) & 3)) : (c ^ ((r >> 1) & 7));
}

// Element offset of 16-byte chunk c of row r in a [rows][BK] bf16 tile.
template <int BK>
__device__ __forceinline__ int swz_row(int r, int c) { return r * BK + (swz_chunk<BK>(r, c) << 3); }

__device__ __forceinline__ int swz_k32(int r, int c) { return swz_row<32>(r, c); }

// Copy 16 bytes per lane from src to LDS at dst + 16 * lane.  AUX is the
// cache-policy field of the instruction (2: non-temporal, for data read once).
template <int AUX = 0>
__device__ __forceinline__ void lds_dma16(const void* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, AUX);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// and all of its LDS reads have returned.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// wait_vm_lgkm0<PW * newer>() for a run-time newer in [0, MAXN].
template <int PW, int MAXN>
__device__ __forceinline__ void wait_newer(int newer) {
  if constexpr (MAXN <= 0) {
    wait_vm_lgkm0<0>();
  } else {
    if (newer >= MAXN)
      wait_vm_lgkm0<PW * MAXN>();
    else
      wait_newer<PW, MAXN - 1>(newer);
  }
}

// wait_vm_lgkm0<n>() for a run-time n in [0, N].
template <int N>
__device__ __forceinline__ void wait_vm_dyn(int n) {
  if constexpr (N <= 0) {
    wait_vm_lgkm0<0>();
  } else {
    if (n >= N)
      wait_vm_lgkm0<N>();
    else
      wait_vm_dyn<N - 1>(n);
  }
}

// Workgroup barrier for the LDS ring: no memory fence (the waits above order
// this wave's own copies), and a compiler barrier so that no LDS access moves
// across it.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace dmtp
