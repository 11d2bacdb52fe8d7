// gkd_device.hpp - device-side helpers shared by the libgkdhead kernels
// (gfx950, wave64). Nothing here is used by the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gkd {

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// float32 -> bfloat16 bits, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Argmax order: larger value first, then the lower flat index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Wave64 (value desc, index asc) reduction; every lane gets the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off, kWave);
    const int oi = __shfl_xor(i, off, kWave);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Workgroup id -> (crop, item within crop) so that every item of one crop
// lands on the same XCD (sharing its L2 for the crop's feature re-reads)
// and the items of a crop are dispatched back to back.
struct ItemCoord {
  int crop;
  int item;
};
__device__ __forceinline__ ItemCoord xcd_item(int wg, int items_per_crop) {
  const int xcd = wg % kXcds;
  const int slot = wg / kXcds;
  ItemCoord c;
  c.crop = (slot / items_per_crop) * kXcds + xcd;
  c.item = slot % items_per_crop;
  return c;
}

// Valid-row bookkeeping for one crop, done by wave 0 of the workgroup.
// Rows are "valid" when any of up to two masks is set. The crop's valid
// rows are split into nblk near-equal blocks by rank; block `blk` gets the
// ranks [lo, hi). Writes the selected row ids to rows[0..hi-lo) and returns
// (total valid count) in *n_valid. Runs on wave 0 only; the caller syncs.
__device__ __forceinline__ void select_rows(const uint8_t* m0, const uint8_t* m1,
                                            int R, int lane, int blk,
                                            int rows_per_blk, int* rows,
                                            uint8_t* sel_m0, uint8_t* sel_m1,
                                            int* n_valid, int* n_sel) {
  int total = 0;
  for (int base = 0; base < R; base += kWave) {
    const int r = base + lane;
    const bool v = r < R && ((m0 && m0[r]) || (m1 && m1[r]));
    total += __popcll(__ballot(v));
  }
  const int nb = (total + rows_per_blk - 1) / rows_per_blk;
  const int lo = nb ? (int)((long long)blk * total / nb) : 0;
  const int hi = nb ? (int)((long long)(blk + 1) * total / nb) : 0;
  int seen = 0;
  for (int base = 0; base < R; base += kWave) {
    const int r = base + lane;
    const bool a = r < R && m0 && m0[r];
    const bool t = r < R && m1 && m1[r];
    const bool v = a || t;
    const uint64_t bal = __ballot(v);
    const int rank = seen + __popcll(bal & ((1ull << lane) - 1ull));
    if (v && rank >= lo && rank < hi) {
      rows[rank - lo] = r;
      sel_m0[rank - lo] = a;
      sel_m1[rank - lo] = t;
    }
    seen += __popcll(bal);
  }
  if (lane == 0) {
    *n_valid = total;
    *n_sel = (blk < nb) ? hi - lo : 0;
  }
}

}  // namespace gkd
