// gkd_device.hpp - device-side helpers shared by the libgkdhead kernels
// (gfx950, wave64). Nothing here is used by the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gkd {

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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

// The -1..1 coordinate of index x of n along one axis: the cell centre
// (2x + 1)/n - 1, or with corners the corner-aligned 2x/(n - 1) - 1 (0 for
// n == 1).
__device__ __forceinline__ float keypoint_coord(int x, int n, bool corners) {
  if (!corners) return (float)(2 * x + 1) / (float)n - 1.f;
  return n > 1 ? (float)(2 * x) / (float)(n - 1) - 1.f : 0.f;
}

// Taps of output o on the align_corners=True grid of a 4x upsample of n
// samples: source position o (n - 1) / (4n - 1), from an exact integer
// ratio (the upper tap clamps at the last sample; n == 1 has one).
__device__ __forceinline__ void corner_taps(int o, int n, int& i0, int& i1, float& lam) {
  if (n == 1) {
    i0 = i1 = 0;
    lam = 0.f;
    return;
  }
  const int num = o * (n - 1), den = 4 * n - 1;
  i0 = num / den;
  lam = (float)(num - i0 * den) / (float)den;
  i1 = i0 + 1 < n ? i0 + 1 : n - 1;
}

// Argmax order: larger value first, then the lower flat index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// One exchange step of the argmax reduction through a DPP lane pattern.
template <int CTRL>
__device__ __forceinline__ void argmax_dpp_step(float& v, int& i) {
  const float ov = __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xf, 0xf, false);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// Wave64 (value desc, index asc) reduction; every lane gets the winner.
// Within each 16-lane row: quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// half-row mirror, row mirror (register-level lane moves, no LDS); then the
// four row results are combined from readlane values.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_dpp_step<0xB1>(v, i);   // quad_perm(1,0,3,2)
  argmax_dpp_step<0x4E>(v, i);   // quad_perm(2,3,0,1)
  argmax_dpp_step<0x141>(v, i);  // row_half_mirror
  argmax_dpp_step<0x140>(v, i);  // row_mirror
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
    const int ri = __builtin_amdgcn_readlane(i, 16 * r);
    if (better(rv, ri, bv, bi)) {
      bv = rv;
      bi = ri;
    }
  }
  v = bv;
  i = bi;
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
// The masks of the first 128 rows are requested together and held in
// registers for both passes (one memory round trip for R <= 128).
__device__ __forceinline__ void select_rows(const uint8_t* m0, const uint8_t* m1,
                                            int R, int lane, int blk,
                                            int rows_per_blk, int* rows,
                                            uint8_t* sel_m0, uint8_t* sel_m1,
                                            int* n_valid, int* n_sel) {
  constexpr int kHeld = 2;  // 64-row blocks held in registers
  uint32_t held[kHeld];     // bit 0: m0 set, bit 1: m1 set
#pragma unroll
  for (int i = 0; i < kHeld; ++i) {
    const int r = i * kWave + lane;
    const bool in = r < R;
    held[i] = ((in && m0 && m0[r]) ? 1u : 0u) | ((in && m1 && m1[r]) ? 2u : 0u);
  }
  auto load_flags = [&](int r) -> uint32_t {
    return ((r < R && m0 && m0[r]) ? 1u : 0u) | ((r < R && m1 && m1[r]) ? 2u : 0u);
  };
  int total = 0;
#pragma unroll
  for (int i = 0; i < kHeld; ++i) total += __popcll(__ballot(held[i] != 0));
  for (int base = kHeld * kWave; base < R; base += kWave)
    total += __popcll(__ballot(load_flags(base + lane) != 0));
  const int nb = (total + rows_per_blk - 1) / rows_per_blk;
  const int lo = nb ? (int)((long long)blk * total / nb) : 0;
  const int hi = nb ? (int)((long long)(blk + 1) * total / nb) : 0;
  int seen = 0;
  auto place = [&](uint32_t f, int r) {
    const bool v = f != 0;
    const uint64_t bal = __ballot(v);
    const int rank = seen + __popcll(bal & ((1ull << lane) - 1ull));
    if (v && rank >= lo && rank < hi) {
      rows[rank - lo] = r;
      sel_m0[rank - lo] = f & 1u;
      sel_m1[rank - lo] = (f >> 1) & 1u;
    }
    seen += __popcll(bal);
  };
#pragma unroll
  for (int i = 0; i < kHeld; ++i) place(held[i], i * kWave + lane);
  for (int base = kHeld * kWave; base < R; base += kWave) place(load_flags(base + lane), base + lane);
  if (lane == 0) {
    *n_valid = total;
    *n_sel = (blk < nb) ? hi - lo : 0;
  }
}

// ---------------------------------------------------------------------------
// 4x bilinear expand of one low-res cell (half-pixel centres, edge clamp).
// Output sample 4i + d reads source rows (lo, hi) with weights (wl, wh):
//   d=0: (i-1, i) (3/8, 5/8)   d=1: (i-1, i) (1/8, 7/8)
//   d=2: (i, i+1) (7/8, 1/8)   d=3: (i, i+1) (5/8, 3/8)
// and at a clamped border (1, 0) on the cell itself, which reproduces the
// border duplicates bit for bit.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void bilinear_taps4(int i, int n, float (&wl)[4], float (&wh)[4]) {
  const bool lo_ok = i > 0, hi_ok = i < n - 1;
  wl[0] = lo_ok ? 0.375f : 1.f;  wh[0] = lo_ok ? 0.625f : 0.f;
  wl[1] = lo_ok ? 0.125f : 1.f;  wh[1] = lo_ok ? 0.875f : 0.f;
  wl[2] = hi_ok ? 0.875f : 1.f;  wh[2] = hi_ok ? 0.125f : 0.f;
  wl[3] = hi_ok ? 0.625f : 1.f;  wh[3] = hi_ok ? 0.375f : 0.f;
}

// h[d] for one source row r: horizontal taps around column j.
__device__ __forceinline__ void bilinear_hrow(const float* __restrict__ Pr, int j, int jm, int jp,
                                     const float (&wl)[4], const float (&wh)[4],
                                     float (&h)[4]) {
  const float a = Pr[jm], c = Pr[j], e = Pr[jp];
  h[0] = fmaf(wh[0], c, wl[0] * a);
  h[1] = fmaf(wh[1], c, wl[1] * a);
  h[2] = fmaf(wh[2], e, wl[2] * c);
  h[3] = fmaf(wh[3], e, wl[3] * c);
}

}  // namespace gkd
