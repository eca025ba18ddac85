// Storage order of keys and values in the T0 pool, the T1 window and the T1
// staging buffer (internal; the C ABI documents it as "K-tiles" / "V-tiles").
//
// Every (sequence, layer, KV head) block of `cap` slots (cap a multiple of 32)
// is cut into 32-slot blocks of 32*D elements.  Inside a block the elements are
// ordered so that one wave's 16-byte loads, lane after lane, are exactly the
// operands of v_mfma_f32_16x16x32_bf16 -- each operand load of the attention
// kernel is one contiguous 1 KB access:
//
//  K-tiles: two tiles of 16 rows; slot r of the block (r = 8j + 4u + i) is row
//           4j + i of tile u (the token order that makes the S^T accumulator the
//           A operand of P.V); a tile stores [D/8 chunks][16 rows][8 elements].
//  V-tiles: [D/16][4 panels of 8 slots][16 dims][8 slots]: the 8 slots of a
//           panel for one dimension are contiguous (a B operand of P.V).
#pragma once

namespace tkv {

__host__ __device__ inline long k_off(long slot, int d, int D) {
  const int r = (int)(slot & 31);
  const int u = (r >> 2) & 1;
  const int row = ((r >> 3) << 2) | (r & 3);
  return (slot >> 5) * 32L * D + (long)u * 16 * D + ((long)(d >> 3) * 16 + row) * 8 + (d & 7);
}

__host__ __device__ inline long v_off(long slot, int d, int D) {
  const int r = (int)(slot & 31);
  return (slot >> 5) * 32L * D + ((long)((d >> 4) << 2) + (r >> 3)) * 128 + (d & 15) * 8 + (r & 7);
}

}  // namespace tkv
