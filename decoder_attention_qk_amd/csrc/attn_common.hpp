// Helpers shared by the attention kernels (forward and backward): direct
// global->LDS DMA through buffer resources, and the wait on vector memory.
#pragma once

#include "device_common.hpp"

namespace muse {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// Buffer resource over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

// 16 bytes per lane at byte offset voff of the buffer, straight into LDS at
// dst + 16 * lane (dst must be the same for the whole wave).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voff, lds_char *dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, 0, 0, 0);
}

// 4 bytes per lane at byte offset voff, into LDS at dst + 4 * lane.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rsrc, int voff, lds_char *dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 4, voff, 0, 0, 0);
}

// x of the lower-half lane and of the upper-half lane of this lane's pair
// (l, l ^ 32), by one VALU lane swap (no LDS round trip).
__device__ __forceinline__ void swap32(float x, float &lo, float &hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

__device__ __forceinline__ void vmem_wait_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt untouched
}

// Sum of per-wave accumulators over the parts of one split work item.  Each
// part stores this wave's R x C accumulators to its slot (floats, [element]
// [lane]) with device-coherent stores -- a store completes only once it is
// visible device-wide, so waiting for them orders them before the arrival --
// and counts its arrival; the wave that arrives last resets the counter to
// zero, replaces acc by the sum of every part's slot in part order (the same
// bits whichever part arrives last) and returns true.  No wave waits for
// another.  Release/acquire fences would write back and invalidate the XCD's
// whole L2 instead, which its other workgroups pay for in refetches.
template <int R, int C>
__device__ __forceinline__ bool split_sum(f32x16 (&acc)[R][C], float *slot0, int64_t part_stride, int part,
                                          int nparts, uint32_t *cnt) {
  const int lane = threadIdx.x & 63;
  float *mine = slot0 + part * part_stride + lane;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __hip_atomic_store(mine + ((r * C + c) * 16 + i) * 64, acc[r][c][i], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  // the signal fences keep the compiler from moving the relaxed atomics to
  // other addresses across the wait (they emit no instruction)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  uint32_t prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (prev != (uint32_t)(nparts - 1)) return false;
  if (lane == 0) *cnt = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[r][c] = f32x16{};
  for (int p = 0; p < nparts; ++p) {
    const float *src = slot0 + p * part_stride + lane;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[r][c][i] += __hip_atomic_load(src + ((r * C + c) * 16 + i) * 64, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  }
  return true;
}

// LDS layout of a tile of 64 rows of D bf16 values with its 16-byte chunks
// XOR-swizzled per row (the swizzle is applied on the DMA source side).
template <int D>
struct Tile {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CHUNKS = D / 8;                    // 16-byte chunks per row
  static constexpr int TILE_BYTES = 64 * ROW_BYTES;       // one tile
  static constexpr int ROWS_PER_256B = 256 / ROW_BYTES;
  // Row-fragment reads (16 rows x one chunk per 16-lane group): spread 16
  // rows over 16 slots.
  static __device__ __forceinline__ int swz_k(int row) { return (row / ROWS_PER_256B) % CHUNKS; }
  // Transposed reads (4 rows x 32 columns per half-wave): give each row its
  // own quarter of the 256-byte bank window (XOR on 4-chunk groups).
  static __device__ __forceinline__ int swz_v(int row) {
    return 4 * ((row / ROWS_PER_256B) & (CHUNKS / 4 - 1));
  }
  // Both patterns on one tile: the 4-chunk group follows the row as in swz_v,
  // the chunk inside the group follows the next row bits, so 16 consecutive
  // rows still land on 16 distinct slots.  Adding 16 rows leaves it
  // unchanged; adding 8 rows flips bit 1.
  static __device__ __forceinline__ int swz_kv(int row) {
    const int m = row / ROWS_PER_256B;
    return 4 * (m & (CHUNKS / 4 - 1)) + ((m / (CHUNKS / 4)) & 3);
  }
};

}  // namespace muse
