// heatmap.hip - gkd_kernel_heatmap on gfx950.
//
// The head's 1x1 "conv" of L2-normalised kernels against the 4x bilinearly
// upsampled query features (GKDT-L GGUF model card, section "Model") is a
// linear map, and so is the upsample; this kernel contracts at LOW
// resolution first (16x fewer MACs and 16x fewer feature bytes than
// upsampling first) and expands afterwards, fusing the modality mean, the
// 4x expand, the heatmap store and the per-row argmax into one pass.
//
// Work item = (crop b, block of <= 16 valid rows). One workgroup of 9 waves
// per item:
//   1. wave 0 selects the block's rows from the masks;
//   2. the raw kernel rows of both modalities (16 x C each) are staged in
//      LDS; per-row 1/||k|| is taken in fp32 from the stored values;
//   3. contraction P[m, s] = sum_c k[m, c] F[c, s] on MFMA. Each wave owns
//      64-pixel super-tiles; a lane streams 4 consecutive pixels of 8 (bf16)
//      or 1 (f32) channels per load straight from HBM in the layout the MFMA
//      B operand needs (4 N-tiles interleaved by pixel), so the feature map
//      makes one trip HBM -> VGPR with no LDS round trip; the A operand
//      comes from LDS;
//   4. epilogue: P_row = a * P_vis + b * P_txt (a, b = mask / (||k|| n)),
//      written to LDS (aliasing the kernel tile, which is dead by then);
//   5. each thread expands one low-res cell into its 4x4 output block,
//      stores it with non-temporal 16-byte stores (full 128-byte lines) and
//      keeps a running (value desc, index asc) best; wave + workgroup
//      reductions give the row's peak.
// Workgroups are mapped so all items of one crop run back to back on one
// XCD: the crop's feature map is fetched from HBM once and re-read from
// that XCD's L2 by the crop's other row blocks.
#include "gkd_device.hpp"
#include "launch.hpp"

#include <climits>
#include <cmath>

namespace gkd {
namespace {

constexpr int kWaves = 9;
constexpr int kThreads = kWaves * kWave;  // 576
constexpr int kMT = 16;                   // MFMA M tile = max rows per item
constexpr int kST = 64;                   // pixels per super-tile

struct HmParams {
  const void* query;
  const void* kv;
  const uint8_t* mv;
  const void* kt;
  const uint8_t* mt;
  int B, C, H, W, R, S;
  int rows_per_item;  // <= kMT
  int items_per_crop;
  int cp;             // C rounded up to the K step
  int ldk;            // LDS row stride of the kernel tile (elements)
  int p_offset;       // byte offset of the fused maps in LDS (0 = aliased)
  float* heat;
  int32_t* idx;
  float* xy;
  float* score;
};

// ---------------------------------------------------------------------------
// Contraction, bf16: v_mfma_f32_16x16x32_bf16. K step = 32 channels.
// Lane (n = lane & 15, g = lane >> 4) supplies channels c0 + 8g + e,
// e = 0..7, for pixels px = 64 st + 4n + t of N-tile t (t = 0..3).
// ---------------------------------------------------------------------------
struct Bf16Loads {
  u32x2 v[8];  // v[e] = 4 pixels (bf16) of channel c0 + 8g + e
};

template <bool FAST>
__device__ __forceinline__ void load_bf16(Bf16Loads& L, const uint16_t* __restrict__ F,
                                          int C, int S, int c0, int g, int px) {
  if (FAST) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      L.v[e] = *reinterpret_cast<const u32x2*>(F + (size_t)(c0 + 8 * g + e) * S + px);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c0 + 8 * g + e;
      uint32_t h[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        h[t] = (c < C && px + t < S) ? F[(size_t)c * S + px + t] : 0u;
      L.v[e].x = h[0] | (h[1] << 16);
      L.v[e].y = h[2] | (h[3] << 16);
    }
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// 8 channels x 4 pixels -> 4 B operands (8 channels each), one per N-tile.
__device__ __forceinline__ void transpose_bf16(const Bf16Loads& L, bf16x8 (&b)[4]) {
  u32x4 t0, t1, t2, t3;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t ex = L.v[2 * d].x, ox = L.v[2 * d + 1].x;
    const uint32_t ey = L.v[2 * d].y, oy = L.v[2 * d + 1].y;
    t0[d] = __builtin_amdgcn_perm(ox, ex, 0x05040100u);  // pixel 0
    t1[d] = __builtin_amdgcn_perm(ox, ex, 0x07060302u);  // pixel 1
    t2[d] = __builtin_amdgcn_perm(oy, ey, 0x05040100u);  // pixel 2
    t3[d] = __builtin_amdgcn_perm(oy, ey, 0x07060302u);  // pixel 3
  }
  b[0] = as_bf16x8(t0);
  b[1] = as_bf16x8(t1);
  b[2] = as_bf16x8(t2);
  b[3] = as_bf16x8(t3);
}

__device__ __forceinline__ void mfma_step_bf16(const Bf16Loads& L, const uint16_t* __restrict__ A,
                                               int ldk, int c0, int m, int g, bool has_v,
                                               bool has_t, f32x4 (&acc)[2][4]) {
  bf16x8 av, at;
  if (has_v) av = *reinterpret_cast<const bf16x8*>(A + (size_t)m * ldk + c0 + 8 * g);
  if (has_t) at = *reinterpret_cast<const bf16x8*>(A + (size_t)(kMT + m) * ldk + c0 + 8 * g);
  bf16x8 b[4];
  transpose_bf16(L, b);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (has_v) acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[t], acc[0][t], 0, 0, 0);
    if (has_t) acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at, b[t], acc[1][t], 0, 0, 0);
  }
}

// One 64-pixel super-tile, all channels. Two register stages: the loads of
// K step k+1 are in flight while step k runs on the matrix cores.
template <bool FAST>
__device__ __forceinline__ void contract_tile_bf16(const HmParams& p, const uint16_t* __restrict__ F,
                                                   const uint16_t* __restrict__ A, int px,
                                                   int lane, bool has_v, bool has_t,
                                                   f32x4 (&acc)[2][4]) {
  const int n = lane & 15, g = lane >> 4;
  constexpr int KS = 32;
  Bf16Loads a, b;
  load_bf16<FAST>(a, F, p.C, p.S, 0, g, px);
  int c0 = 0;
  for (; c0 + 2 * KS <= p.cp; c0 += 2 * KS) {
    load_bf16<FAST>(b, F, p.C, p.S, c0 + KS, g, px);
    mfma_step_bf16(a, A, p.ldk, c0, n, g, has_v, has_t, acc);
    if (c0 + 2 * KS < p.cp) load_bf16<FAST>(a, F, p.C, p.S, c0 + 2 * KS, g, px);
    mfma_step_bf16(b, A, p.ldk, c0 + KS, n, g, has_v, has_t, acc);
  }
  if (c0 < p.cp) mfma_step_bf16(a, A, p.ldk, c0, n, g, has_v, has_t, acc);
}

// ---------------------------------------------------------------------------
// Contraction, f32: v_mfma_f32_16x16x4_f32. Macro step = 16 channels =
// 4 MFMA k-steps. At k-step e lane (n, g) supplies channel c0 + 4g + e for
// the 4 pixels px..px+3 (one float4 load), i.e. 4 N-tiles at once.
// ---------------------------------------------------------------------------
struct F32Loads {
  f32x4 v[4];  // v[e] = 4 pixels of channel c0 + 4g + e
};

template <bool FAST>
__device__ __forceinline__ void load_f32(F32Loads& L, const float* __restrict__ F, int C,
                                         int S, int c0, int g, int px) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = c0 + 4 * g + e;
    if (FAST) {
      L.v[e] = *reinterpret_cast<const f32x4*>(F + (size_t)c * S + px);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        L.v[e][t] = (c < C && px + t < S) ? F[(size_t)c * S + px + t] : 0.f;
    }
  }
}

__device__ __forceinline__ void mfma_step_f32(const F32Loads& L, const float* __restrict__ A,
                                              int ldk, int c0, int m, int g, bool has_v,
                                              bool has_t, f32x4 (&acc)[2][4]) {
  f32x4 av, at;
  if (has_v) av = *reinterpret_cast<const f32x4*>(A + (size_t)m * ldk + c0 + 4 * g);
  if (has_t) at = *reinterpret_cast<const f32x4*>(A + (size_t)(kMT + m) * ldk + c0 + 4 * g);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (has_v) acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], L.v[e][t], acc[0][t], 0, 0, 0);
      if (has_t) acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(at[e], L.v[e][t], acc[1][t], 0, 0, 0);
    }
  }
}

template <bool FAST>
__device__ __forceinline__ void contract_tile_f32(const HmParams& p, const float* __restrict__ F,
                                                  const float* __restrict__ A, int px, int lane,
                                                  bool has_v, bool has_t, f32x4 (&acc)[2][4]) {
  const int n = lane & 15, g = lane >> 4;
  constexpr int KS = 16;
  F32Loads a, b;
  load_f32<FAST>(a, F, p.C, p.S, 0, g, px);
  int c0 = 0;
  for (; c0 + 2 * KS <= p.cp; c0 += 2 * KS) {
    load_f32<FAST>(b, F, p.C, p.S, c0 + KS, g, px);
    mfma_step_f32(a, A, p.ldk, c0, n, g, has_v, has_t, acc);
    if (c0 + 2 * KS < p.cp) load_f32<FAST>(a, F, p.C, p.S, c0 + 2 * KS, g, px);
    mfma_step_f32(b, A, p.ldk, c0 + KS, n, g, has_v, has_t, acc);
  }
  if (c0 < p.cp) mfma_step_f32(a, A, p.ldk, c0, n, g, has_v, has_t, acc);
}

// Rows 4g..4g+3 x pixels px..px+3 of the fused low-res maps -> LDS.
template <bool FAST>
__device__ __forceinline__ void store_fused(float* P, const float (&f)[4][4], int S, int px,
                                            int g, int nsel) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = 4 * g + i;
    if (slot >= nsel) continue;
    float* dst = P + (size_t)slot * S + px;
    if (FAST) {
      *reinterpret_cast<f32x4*>(dst) = f32x4{f[i][0], f[i][1], f[i][2], f[i][3]};
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (px + t < S) dst[t] = f[i][t];
    }
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
__device__ __forceinline__ void taps4(int i, int n, float (&wl)[4], float (&wh)[4]) {
  const bool lo_ok = i > 0, hi_ok = i < n - 1;
  wl[0] = lo_ok ? 0.375f : 1.f;  wh[0] = lo_ok ? 0.625f : 0.f;
  wl[1] = lo_ok ? 0.125f : 1.f;  wh[1] = lo_ok ? 0.875f : 0.f;
  wl[2] = hi_ok ? 0.875f : 1.f;  wh[2] = hi_ok ? 0.125f : 0.f;
  wl[3] = hi_ok ? 0.625f : 1.f;  wh[3] = hi_ok ? 0.375f : 0.f;
}

// h[d] for one source row r: horizontal taps around column j.
__device__ __forceinline__ void hrow(const float* __restrict__ Pr, int j, int jm, int jp,
                                     const float (&wl)[4], const float (&wh)[4],
                                     float (&h)[4]) {
  const float a = Pr[jm], c = Pr[j], e = Pr[jp];
  h[0] = fmaf(wh[0], c, wl[0] * a);
  h[1] = fmaf(wh[1], c, wl[1] * a);
  h[2] = fmaf(wh[2], e, wl[2] * c);
  h[3] = fmaf(wh[3], e, wl[3] * c);
}

// Waves per SIMD the register allocator must leave room for.
template <typename T, int NSTW>
constexpr int hm_waves_per_eu() {
  return (sizeof(T) == 2 && NSTW == 1) ? 4 : 3;
}

// NSTW: super-tiles per wave. ALIAS: the fused low-res maps reuse the
// kernel tile's LDS (kept in registers until the tile is dead); otherwise
// they have their own LDS region and each super-tile is written as soon as
// it is done (large maps, where registers cannot hold them).
template <typename T, int NSTW, bool ALIAS, bool FAST>
__global__ __attribute__((amdgpu_flat_work_group_size(1, kThreads),
                          amdgpu_waves_per_eu(hm_waves_per_eu<T, NSTW>())))
void heatmap_kernel(HmParams p) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int s_rows[kMT];
  __shared__ uint8_t s_mv[kMT], s_mt[kMT];
  __shared__ int s_nvalid, s_nsel;
  __shared__ float s_inv[2 * kMT];
  __shared__ float s_redv[kMT][kWaves];
  __shared__ int s_redi[kMT][kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const ItemCoord ic = xcd_item(blockIdx.x, p.items_per_crop);
  const int b = ic.crop;
  if (b >= p.B) return;

  const uint8_t* mv = p.mv ? p.mv + (size_t)b * p.R : nullptr;
  const uint8_t* mt = p.mt ? p.mt + (size_t)b * p.R : nullptr;

  // 1. rows of this item
  if (wave == 0)
    select_rows(mv, mt, p.R, lane, ic.item, p.rows_per_item, s_rows, s_mv, s_mt,
                &s_nvalid, &s_nsel);
  // decode sentinels for the crop's rows without any prompt (first item)
  if (ic.item == 0 && p.idx) {
    for (int r = tid; r < p.R; r += kThreads) {
      if (!((mv && mv[r]) || (mt && mt[r]))) {
        const size_t o = (size_t)b * p.R + r;
        p.idx[o] = -1;
        p.xy[2 * o] = __builtin_nanf("");
        p.xy[2 * o + 1] = __builtin_nanf("");
        p.score[o] = -INFINITY;
      }
    }
  }
  __syncthreads();
  const int nsel = s_nsel;
  if (nsel == 0) return;

  // 2. stage raw kernel rows [2][kMT][ldk] (zero rows where masked/absent)
  T* A = reinterpret_cast<T*>(lds);
  {
    constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte chunk
    const int cpr = p.cp / EPV;          // chunks per row
    const T* kv = static_cast<const T*>(p.kv);
    const T* kt = static_cast<const T*>(p.kt);
    for (int q = tid; q < 2 * kMT * cpr; q += kThreads) {
      const int row = q / cpr, ch = q - row * cpr;
      const int mod = row / kMT, slot = row - mod * kMT;
      const bool on = slot < nsel && (mod == 0 ? s_mv[slot] : s_mt[slot]);
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (on) {
        const T* src = (mod == 0 ? kv : kt) + ((size_t)b * p.R + s_rows[slot]) * p.C;
        const int c = ch * EPV;
        if (FAST) {
          v = *reinterpret_cast<const u32x4*>(src + c);
        } else {
          T tmp[EPV];
#pragma unroll
          for (int e = 0; e < EPV; ++e) tmp[e] = (c + e < p.C) ? src[c + e] : T(0);
          __builtin_memcpy(&v, tmp, 16);
        }
      }
      *reinterpret_cast<u32x4*>(A + (size_t)row * p.ldk + ch * EPV) = v;
    }
  }
  __syncthreads();

  // 1/||k|| per (modality, slot) in fp32 from the stored values
  for (int row = wave; row < 2 * kMT; row += kWaves) {
    float ss = 0.f;
    for (int c = lane; c < p.C; c += kWave) {
      float v;
      if constexpr (sizeof(T) == 2) v = bf16_bits_to_f32(A[(size_t)row * p.ldk + c]);
      else v = A[(size_t)row * p.ldk + c];
      ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) s_inv[row] = 1.f / fmaxf(sqrtf(ss), 1e-12f);
  }
  __syncthreads();
  bool has_v = false, has_t = false;
  for (int s = 0; s < nsel; ++s) {
    has_v |= s_mv[s] != 0;
    has_t |= s_mt[s] != 0;
  }

  // 3. contraction at low resolution, one super-tile at a time; each
  //    tile's fused rows are kept in registers until the kernel tile in LDS
  //    is dead. Lane (n, g) ends up holding rows 4g..4g+3; their fusion
  //    weights a = m_vis / (n ||k_vis||), c = m_txt / (n ||k_txt||).
  const int n16 = lane & 15, g4 = lane >> 4;
  float cv[4], ct[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = 4 * g4 + i;
    cv[i] = ct[i] = 0.f;
    if (slot < nsel) {
      const float n = (float)((int)s_mv[slot] + (int)s_mt[slot]);
      cv[i] = s_mv[slot] ? s_inv[slot] / n : 0.f;
      ct[i] = s_mt[slot] ? s_inv[kMT + slot] / n : 0.f;
    }
  }
  float fused[ALIAS ? NSTW : 1][4][4];  // [tile][row 4g+i][pixel 4n+t]
  float* P = reinterpret_cast<float*>(lds + (ALIAS ? 0 : p.p_offset));
#pragma unroll
  for (int w = 0; w < NSTW; ++w) {
    const int st = wave + w * kWaves;
    if (st * kST >= p.S) break;
    const int px = st * kST + 4 * n16;
    f32x4 acc[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (sizeof(T) == 2) {
      const uint16_t* F = static_cast<const uint16_t*>(p.query) + (size_t)b * p.C * p.S;
      contract_tile_bf16<FAST>(p, F, reinterpret_cast<const uint16_t*>(A), px, lane, has_v,
                               has_t, acc);
    } else {
      const float* F = static_cast<const float*>(p.query) + (size_t)b * p.C * p.S;
      contract_tile_f32<FAST>(p, F, reinterpret_cast<const float*>(A), px, lane, has_v, has_t,
                              acc);
    }
    const int wi = ALIAS ? w : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) fused[wi][i][t] = fmaf(ct[i], acc[1][t][i], cv[i] * acc[0][t][i]);
    if constexpr (!ALIAS) store_fused<FAST>(P, fused[0], p.S, px, g4, nsel);
  }
  // 4. fused, scaled low-res maps -> LDS P[slot][S]
  if constexpr (ALIAS) {
    __syncthreads();  // the kernel tile is dead; P aliases it
#pragma unroll
    for (int w = 0; w < NSTW; ++w) {
      const int st = wave + w * kWaves;
      if (st * kST >= p.S) break;
      store_fused<FAST>(P, fused[w], p.S, st * kST + 4 * n16, g4, nsel);
    }
  }
  __syncthreads();

  // 5. 4x expand + non-temporal stores + running argmax
  const int Ho = 4 * p.H, Wo = 4 * p.W;
  for (int s = 0; s < nsel; ++s) {
    const float* Pr = P + (size_t)s * p.S;
    float* out = p.heat + ((size_t)b * p.R + s_rows[s]) * (size_t)Ho * Wo;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int cell = tid; cell < p.S; cell += kThreads) {
      const int i = cell / p.W, j = cell - i * p.W;
      const int im = i > 0 ? i - 1 : 0, ip = i < p.H - 1 ? i + 1 : i;
      const int jm = j > 0 ? j - 1 : 0, jp = j < p.W - 1 ? j + 1 : j;
      float xl[4], xh[4], yl[4], yh[4];
      taps4(j, p.W, xl, xh);
      taps4(i, p.H, yl, yh);
      float hm[4], h0[4], hp[4];
      hrow(Pr + (size_t)im * p.W, j, jm, jp, xl, xh, hm);
      hrow(Pr + (size_t)i * p.W, j, jm, jp, xl, xh, h0);
      hrow(Pr + (size_t)ip * p.W, j, jm, jp, xl, xh, hp);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float* lo = d < 2 ? hm : h0;
        const float* hi = d < 2 ? h0 : hp;
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fmaf(yh[d], hi[e], yl[d] * lo[e]);
        const int y = 4 * i + d;
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(out + (size_t)y * Wo + 4 * j));
        const int base = y * Wo + 4 * j;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (better(o[e], base + e, bv, bi)) {
            bv = o[e];
            bi = base + e;
          }
      }
    }
    if (p.idx) {
      wave_argmax(bv, bi);
      if (lane == 0) {
        s_redv[s][wave] = bv;
        s_redi[s][wave] = bi;
      }
    }
  }
  if (!p.idx) return;
  __syncthreads();
  if (tid < nsel) {
    float bv = s_redv[tid][0];
    int bi = s_redi[tid][0];
    for (int w = 1; w < kWaves; ++w)
      if (better(s_redv[tid][w], s_redi[tid][w], bv, bi)) {
        bv = s_redv[tid][w];
        bi = s_redi[tid][w];
      }
    const size_t o = (size_t)b * p.R + s_rows[tid];
    const int y = bi / Wo, x = bi - y * Wo;
    p.idx[o] = bi;
    p.xy[2 * o] = (float)(2 * x + 1) / (float)Wo - 1.f;
    p.xy[2 * o + 1] = (float)(2 * y + 1) / (float)Ho - 1.f;
    p.score[o] = bv;
  }
}

template <typename T, int NSTW, bool ALIAS, bool FAST>
hipError_t launch_t(const HmParams& p, size_t lds, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((heatmap_kernel<T, NSTW, ALIAS, FAST>), dim3(grid), dim3(kThreads), lds,
                     stream, p);
  return hipGetLastError();
}

template <typename T, bool FAST>
hipError_t dispatch_nstw(const HmParams& p, int nstw, size_t lds, int grid,
                         hipStream_t stream) {
  switch (nstw) {
    case 1: return launch_t<T, 1, true, FAST>(p, lds, grid, stream);
    case 2: return launch_t<T, 2, true, FAST>(p, lds, grid, stream);
    default: return launch_t<T, 4, false, FAST>(p, lds, grid, stream);
  }
}

}  // namespace

HeatmapPlan plan_heatmap(int C, int S, bool bf16) {
  HeatmapPlan pl;
  const size_t esz = bf16 ? 2 : 4;
  const int kstep = bf16 ? 32 : 16;
  pl.cp = (C + kstep - 1) / kstep * kstep;
  pl.ldk = pl.cp + (bf16 ? 8 : 4);  // 16-byte pad: conflict-free A reads
  const size_t a_bytes = (size_t)2 * kMT * pl.ldk * esz;
  const int nst = (S + kST - 1) / kST;
  pl.nstw = (nst + kWaves - 1) / kWaves;
  if (pl.nstw <= 2) {
    // fused maps alias the kernel tile; 16 rows fit when S <= 1152
    int rb = kMT;
    const size_t budget = a_bytes > (size_t)74 * 1024 ? a_bytes : (size_t)74 * 1024;
    while (rb > 1 && (size_t)rb * S * 4 > budget) rb >>= 1;
    const size_t p_bytes = (size_t)rb * S * 4;
    pl.rows_per_item = rb;
    pl.p_offset = 0;
    pl.lds_bytes = a_bytes > p_bytes ? a_bytes : p_bytes;
  } else {
    // separate region after the kernel tile
    int rb = kMT;
    while (rb >= 1 && a_bytes + (size_t)rb * S * 4 > kLdsBudget) rb >>= 1;
    pl.rows_per_item = rb;
    pl.p_offset = (int)a_bytes;
    pl.lds_bytes = a_bytes + (size_t)(rb > 0 ? rb : 0) * S * 4;
  }
  if (pl.lds_bytes > kLdsBudget) pl.rows_per_item = 0;
  return pl;
}

hipError_t launch_heatmap(const HeatmapArgs& a, hipStream_t stream) {
  HmParams p;
  p.query = a.query;
  p.kv = a.kv;
  p.mv = a.mv;
  p.kt = a.kt;
  p.mt = a.mt;
  p.B = a.B;
  p.C = a.C;
  p.H = a.H;
  p.W = a.W;
  p.R = a.R;
  p.S = a.H * a.W;
  p.heat = a.heat;
  p.idx = a.idx;
  p.xy = a.xy;
  p.score = a.score;

  const HeatmapPlan plan = plan_heatmap(a.C, p.S, a.bf16);
  if (plan.rows_per_item < 1) return hipErrorInvalidValue;
  p.cp = plan.cp;
  p.ldk = plan.ldk;
  p.p_offset = plan.p_offset;
  p.rows_per_item = plan.rows_per_item;
  p.items_per_crop = (a.R + plan.rows_per_item - 1) / plan.rows_per_item;
  const size_t lds = plan.lds_bytes;
  const int nstw = plan.nstw;
  const int kstep = a.bf16 ? 32 : 16;
  const int crops_pad = (a.B + kXcds - 1) / kXcds * kXcds;
  const long long grid = (long long)crops_pad * p.items_per_crop;
  if (grid > INT_MAX) return hipErrorInvalidConfiguration;

  const bool fast = (a.C % kstep == 0) && (p.S % kST == 0);
  if (a.bf16)
    return fast ? dispatch_nstw<uint16_t, true>(p, nstw, lds, (int)grid, stream)
                : dispatch_nstw<uint16_t, false>(p, nstw, lds, (int)grid, stream);
  return fast ? dispatch_nstw<float, true>(p, nstw, lds, (int)grid, stream)
              : dispatch_nstw<float, false>(p, nstw, lds, (int)grid, stream);
}

}  // namespace gkd
