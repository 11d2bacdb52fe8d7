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
//   2. contraction P[m, s] = sum_c k[m, c] F[c, s] on MFMA. Each wave owns
//      64-pixel super-tiles; per K step a lane streams 4 consecutive pixels
//      of 8 (bf16) or 4 (f32) channels straight from HBM in the layout the
//      MFMA B operand needs (4 N-tiles interleaved by pixel), and its slice
//      of the raw kernel rows (A operand) from L2. The K loop keeps NS
//      steps of loads in flight with no branch inside it, so the wait
//      counters always leave the newer stages outstanding. The squared row
//      norms accumulate from the same A fragments in float32;
//   3. epilogue: P_row = a * P_vis + c * P_txt with a, c = mask / (n ||k||),
//      written to LDS;
//   4. each thread expands one low-res cell into its 4x4 output block,
//      stores it with non-temporal 16-byte stores (full 128-byte lines) and
//      keeps a running (value desc, index asc) best; wave + workgroup
//      reductions give the row's peak.
// LDS holds only the fused low-res maps (<= 74 KiB per workgroup).
// Workgroups are mapped so all items of one crop run back to back on one
// XCD: the crop's feature map is fetched from HBM once and re-read from
// that XCD's L2 by the crop's other row blocks.
#include "gkd_device.hpp"
#include "launch.hpp"

#include <climits>
#include <cmath>
#include <type_traits>

namespace gkd {
namespace {

constexpr int kWaves = 9;
constexpr int kThreads = kWaves * kWave;  // 576
constexpr int kMT = 16;                   // MFMA M tile = max rows per item
constexpr int kST = 64;                   // pixels per super-tile
constexpr int kVis = 1, kTxt = 2;         // modality mask of an item

struct HmParams {
  const void* query;
  const void* kv;
  const uint8_t* mv;
  const void* kt;
  const uint8_t* mt;
  int B, C, H, W, R, S;
  int rows_per_item;  // <= kMT
  int items_per_crop;
  int nsteps;         // K steps: ceil(C / 32) for bf16, ceil(C / 16) for f32
  void* heat;      // [B,R,4H,4W] float32, or bfloat16 when heat_bf16
  bool heat_bf16;
  int32_t* idx;
  float* xy;
  float* score;
  bool corners;    // corner-aligned keypoint coordinates
  bool up_corners; // upsample on the align_corners=True grid
};

// ---------------------------------------------------------------------------
// One K step of loads. bf16: v_mfma_f32_16x16x32_bf16, 32 channels per step;
// lane (n = lane & 15, g = lane >> 4) supplies channels c0 + 8g + e,
// e = 0..7, for pixels px + t of N-tile t (t = 0..3), and A = 8 channels
// c0 + 8g .. +7 of its row n. f32: v_mfma_f32_16x16x4_f32, 16 channels per
// step as 4 MFMA k-steps; at k-step e lane (n, g) supplies channel
// c0 + 4g + e for the 4 pixels (one float4) and A = channels c0 + 4g .. +3.
// ---------------------------------------------------------------------------
struct StageBf16 {
  u32x2 f[8];
  u32x4 av, at;
};
struct StageF32 {
  f32x4 f[4];
  f32x4 av, at;
};

template <int MODE, bool FAST>
__device__ __forceinline__ void issue(StageBf16& st, const uint16_t* __restrict__ F, int C, int S,
                                      int step, int g, int px, const uint16_t* rv,
                                      const uint16_t* rt) {
  const int c0 = step * 32 + 8 * g;
  if (FAST) {
    const uint16_t* base = F + (size_t)c0 * S + px;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.f[e] = *reinterpret_cast<const u32x2*>(base + (size_t)e * S);
    if (MODE & kVis) st.av = *reinterpret_cast<const u32x4*>(rv + c0);
    if (MODE & kTxt) st.at = *reinterpret_cast<const u32x4*>(rt + c0);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c0 + e;
      uint32_t h[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) h[t] = (c < C && px + t < S) ? F[(size_t)c * S + px + t] : 0u;
      st.f[e].x = h[0] | (h[1] << 16);
      st.f[e].y = h[2] | (h[3] << 16);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint16_t* r = m == 0 ? rv : rt;
      if (!(MODE & (m == 0 ? kVis : kTxt))) continue;
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (c0 + e < C) ? r[c0 + e] : 0u;
      u32x4 v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                      h[6] | (h[7] << 16)};
      if (m == 0) st.av = v;
      else st.at = v;
    }
  }
}

template <int MODE, bool FAST>
__device__ __forceinline__ void issue(StageF32& st, const float* __restrict__ F, int C, int S,
                                      int step, int g, int px, const float* rv,
                                      const float* rt) {
  const int c0 = step * 16 + 4 * g;
  if (FAST) {
    const float* base = F + (size_t)c0 * S + px;
#pragma unroll
    for (int e = 0; e < 4; ++e) st.f[e] = *reinterpret_cast<const f32x4*>(base + (size_t)e * S);
    if (MODE & kVis) st.av = *reinterpret_cast<const f32x4*>(rv + c0);
    if (MODE & kTxt) st.at = *reinterpret_cast<const f32x4*>(rt + c0);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = c0 + e;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        st.f[e][t] = (c < C && px + t < S) ? F[(size_t)c * S + px + t] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (MODE & kVis) st.av[e] = (c0 + e < C) ? rv[c0 + e] : 0.f;
      if (MODE & kTxt) st.at[e] = (c0 + e < C) ? rt[c0 + e] : 0.f;
    }
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Sum of squares of 8 bfloat16 values (two per dword) in float32.
__device__ __forceinline__ float sumsq_bf16(u32x4 v, float acc) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float lo = __uint_as_float(v[d] << 16);
    const float hi = __uint_as_float(v[d] & 0xffff0000u);
    acc = fmaf(lo, lo, acc);
    acc = fmaf(hi, hi, acc);
  }
  return acc;
}

// Consume one K step. A lanes whose row slot is masked loaded some other
// valid row (so the load is unconditional); `onv` / `ont` zero them here,
// as does `live` for the padding steps past C. Selects, not branches.
template <int MODE>
__device__ __forceinline__ void compute(const StageBf16& st, bool live, bool onv, bool ont,
                                        f32x4 (&acc)[2][4], float& ssv, float& sst) {
  const u32x4 z = u32x4{0u, 0u, 0u, 0u};
  const u32x4 av = (live && onv) ? st.av : z;
  const u32x4 at = (live && ont) ? st.at : z;
  if (MODE & kVis) ssv = sumsq_bf16(av, ssv);
  if (MODE & kTxt) sst = sumsq_bf16(at, sst);
  // 8 channels x 4 pixels -> one B operand (8 channels) per N-tile
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
    u32x4 bt;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = (t < 2) ? st.f[2 * d].x : st.f[2 * d].y;
      const uint32_t hi = (t < 2) ? st.f[2 * d + 1].x : st.f[2 * d + 1].y;
      bt[d] = __builtin_amdgcn_perm(hi, lo, sel);
    }
    const bf16x8 b = as_bf16x8(bt);
    if (MODE & kVis)
      acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), b, acc[0][t], 0, 0, 0);
    if (MODE & kTxt)
      acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(at), b, acc[1][t], 0, 0, 0);
  }
}

template <int MODE>
__device__ __forceinline__ void compute(const StageF32& st, bool live, bool onv, bool ont,
                                        f32x4 (&acc)[2][4], float& ssv, float& sst) {
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 av = (live && onv) ? st.av : z;
  const f32x4 at = (live && ont) ? st.at : z;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (MODE & kVis) ssv = fmaf(av[e], av[e], ssv);
    if (MODE & kTxt) sst = fmaf(at[e], at[e], sst);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (MODE & kVis)
        acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], st.f[e][t], acc[0][t], 0, 0, 0);
      if (MODE & kTxt)
        acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(at[e], st.f[e][t], acc[1][t], 0, 0, 0);
    }
  }
}

// Whole K loop for one 64-pixel super-tile: a ring of NS stages, issued
// NS-1 steps ahead. Past the last step the issue index is clamped (a
// harmless reload) and the step is consumed with a zero A operand, so the
// loop body has no branch and every wait leaves NS-1 stages in flight.
template <typename Stage, typename T, int MODE, bool FAST, int NS>
__device__ __forceinline__ void contract_tile(const T* __restrict__ F, int C, int S, int nsteps,
                                              int px, int lane, const T* rv, const T* rt,
                                              bool onv, bool ont, f32x4 (&acc)[2][4],
                                              float& ssv, float& sst) {
  const int g = lane >> 4;
  Stage st[NS];
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    issue<MODE, FAST>(st[j], F, C, S, j < nsteps ? j : nsteps - 1, g, px, rv, rt);
  for (int k0 = 0; k0 < nsteps; k0 += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int k = k0 + j;
      const int ahead = k + NS - 1 < nsteps ? k + NS - 1 : nsteps - 1;
      issue<MODE, FAST>(st[(j + NS - 1) % NS], F, C, S, ahead, g, px, rv, rt);
      // keep program order: the wait before compute() must leave the
      // stages issued after st[j] in flight
      __builtin_amdgcn_sched_barrier(0);
      compute<MODE>(st[j], k < nsteps, onv, ont, acc, ssv, sst);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
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

// Register budget per wave: 128 VGPRs for two stages, 168 for deeper rings.
template <int NS>
constexpr int hm_waves_per_eu() {
  return NS <= 2 ? 4 : 3;
}

template <typename T, bool FAST, int NS>
__global__ __attribute__((amdgpu_flat_work_group_size(1, kThreads),
                          amdgpu_waves_per_eu(hm_waves_per_eu<NS>())))
void heatmap_kernel(HmParams p) {
  extern __shared__ __align__(16) float P[];  // fused low-res maps [rows][S]
  __shared__ int s_rows[kMT];
  __shared__ uint8_t s_mv[kMT], s_mt[kMT];
  __shared__ int s_nvalid, s_nsel;
  __shared__ float s_redv[kMT][kWaves];
  __shared__ int s_redi[kMT][kWaves];
  typedef typename std::conditional<sizeof(T) == 2, StageBf16, StageF32>::type Stage;

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
  bool has_v = false, has_t = false;
  for (int s = 0; s < nsel; ++s) {
    has_v |= s_mv[s] != 0;
    has_t |= s_mt[s] != 0;
  }

  // 2. contraction, one 64-pixel super-tile at a time
  const int n16 = lane & 15, g4 = lane >> 4;
  const T* F = static_cast<const T*>(p.query) + (size_t)b * p.C * p.S;
  // this lane's A rows: row slot n16 of each modality. A lane whose slot
  // is empty or masked reads the first row that carries the modality (a
  // valid address) and zeroes it in compute().
  int first_v = 0, first_t = 0;
  for (int s = nsel - 1; s >= 0; --s) {
    if (s_mv[s]) first_v = s;
    if (s_mt[s]) first_t = s;
  }
  const bool onv = n16 < nsel && s_mv[n16];
  const bool ont = n16 < nsel && s_mt[n16];
  const T* rv = static_cast<const T*>(p.kv) +
                ((size_t)b * p.R + s_rows[onv ? n16 : first_v]) * p.C;
  const T* rt = static_cast<const T*>(p.kt) +
                ((size_t)b * p.R + s_rows[ont ? n16 : first_t]) * p.C;
  const int nst = (p.S + kST - 1) / kST;
  for (int st = wave; st < nst; st += kWaves) {
    const int px = st * kST + 4 * n16;
    f32x4 acc[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float ssv = 0.f, sst = 0.f;
    if (has_v && has_t)
      contract_tile<Stage, T, kVis | kTxt, FAST, NS>(F, p.C, p.S, p.nsteps, px, lane, rv, rt,
                                                     onv, ont, acc, ssv, sst);
    else if (has_v)
      contract_tile<Stage, T, kVis, FAST, NS>(F, p.C, p.S, p.nsteps, px, lane, rv, rt, onv,
                                              ont, acc, ssv, sst);
    else
      contract_tile<Stage, T, kTxt, FAST, NS>(F, p.C, p.S, p.nsteps, px, lane, rv, rt, onv,
                                              ont, acc, ssv, sst);

    // 3. norms: lanes n16, n16+16, n16+32, n16+48 hold quarter sums of
    //    row n16; fusion weight of row slot m: mask / (n ||k||)
    ssv += __shfl_xor(ssv, 16, kWave);
    ssv += __shfl_xor(ssv, 32, kWave);
    sst += __shfl_xor(sst, 16, kWave);
    sst += __shfl_xor(sst, 32, kWave);
    float wv = 0.f, wt = 0.f;
    if (n16 < nsel) {
      const float n = (float)((int)s_mv[n16] + (int)s_mt[n16]);
      if (s_mv[n16]) wv = 1.f / (fmaxf(sqrtf(ssv), 1e-12f) * n);
      if (s_mt[n16]) wt = 1.f / (fmaxf(sqrtf(sst), 1e-12f) * n);
    }
    float fused[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float cv = __shfl(wv, 4 * g4 + i, kWave);
      const float ct = __shfl(wt, 4 * g4 + i, kWave);
#pragma unroll
      for (int t = 0; t < 4; ++t) fused[i][t] = fmaf(ct, acc[1][t][i], cv * acc[0][t][i]);
    }
    store_fused<FAST>(P, fused, p.S, px, g4, nsel);
  }
  __syncthreads();

  // 4. 4x expand + non-temporal stores + running argmax
  const int Ho = 4 * p.H, Wo = 4 * p.W;
  for (int s = 0; s < nsel; ++s) {
    const float* Pr = P + (size_t)s * p.S;
    const size_t out_e = ((size_t)b * p.R + s_rows[s]) * (size_t)Ho * Wo;  // row's first element
    float bv = -INFINITY;
    int bi = INT_MAX;
    if (p.up_corners) {
      // align_corners=True grid: thread takes 4-output chunks of the map
      // in raster order (one output row, columns 4x .. 4x + 3)
      for (int q = tid; q < Ho * p.W; q += kThreads) {
        const int y = q / p.W, x4 = q - y * p.W;
        int i0, i1;
        float ly;
        corner_taps(y, p.H, i0, i1, ly);
        const float* p0 = Pr + (size_t)i0 * p.W;
        const float* p1 = Pr + (size_t)i1 * p.W;
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int j0, j1;
          float lx;
          corner_taps(4 * x4 + e, p.W, j0, j1, lx);
          const float top = fmaf(lx, p0[j1] - p0[j0], p0[j0]);
          const float bot = fmaf(lx, p1[j1] - p1[j0], p1[j0]);
          o[e] = fmaf(ly, bot - top, top);
        }
        const size_t e0 = out_e + 4 * (size_t)q;
        if (p.heat == nullptr) {
          // keypoints only: nothing is stored
        } else if (p.heat_bf16) {
          const u32x2 v = {
              __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[0], o[1]}, bf16x2)),
              __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[2], o[3]}, bf16x2))};
          __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.heat) + e0));
        } else {
          __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(static_cast<float*>(p.heat) + e0));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (better(o[e], 4 * q + e, bv, bi)) {
            bv = o[e];
            bi = 4 * q + e;
          }
      }
    } else
    for (int cell = tid; cell < p.S; cell += kThreads) {
      const int i = cell / p.W, j = cell - i * p.W;
      const int im = i > 0 ? i - 1 : 0, ip = i < p.H - 1 ? i + 1 : i;
      const int jm = j > 0 ? j - 1 : 0, jp = j < p.W - 1 ? j + 1 : j;
      float xl[4], xh[4], yl[4], yh[4];
      bilinear_taps4(j, p.W, xl, xh);
      bilinear_taps4(i, p.H, yl, yh);
      float hm[4], h0[4], hp[4];
      bilinear_hrow(Pr + (size_t)im * p.W, j, jm, jp, xl, xh, hm);
      bilinear_hrow(Pr + (size_t)i * p.W, j, jm, jp, xl, xh, h0);
      bilinear_hrow(Pr + (size_t)ip * p.W, j, jm, jp, xl, xh, hp);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float* lo = d < 2 ? hm : h0;
        const float* hi = d < 2 ? h0 : hp;
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fmaf(yh[d], hi[e], yl[d] * lo[e]);
        const int y = 4 * i + d;
        const size_t e = out_e + (size_t)y * Wo + 4 * j;
        if (p.heat == nullptr) {
          // keypoints only: nothing is stored
        } else if (p.heat_bf16) {
          // round to nearest even; the peak below still uses the float32 values
          const u32x2 v = {
              __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[0], o[1]}, bf16x2)),
              __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[2], o[3]}, bf16x2))};
          __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.heat) + e));
        } else {
          __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(static_cast<float*>(p.heat) + e));
        }
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
    p.xy[2 * o] = keypoint_coord(x, Wo, p.corners);
    p.xy[2 * o + 1] = keypoint_coord(y, Ho, p.corners);
    p.score[o] = bv;
  }
}

#ifndef GKD_HEATMAP_STAGES
#define GKD_HEATMAP_STAGES 2
#endif

template <typename T, bool FAST>
hipError_t launch_t(const HmParams& p, size_t lds, int grid, hipStream_t stream) {
  constexpr int NS = GKD_HEATMAP_STAGES;
  hipLaunchKernelGGL((heatmap_kernel<T, FAST, NS>), dim3(grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

HeatmapPlan plan_heatmap(int C, int S, bool bf16) {
  HeatmapPlan pl;
  const int kstep = bf16 ? 32 : 16;
  pl.nsteps = (C + kstep - 1) / kstep;
  // rows per item: 16 unless the fused maps would crowd LDS (keep two
  // workgroups per CU: <= 74 KiB)
  int rb = kMT;
  while (rb > 1 && (size_t)rb * S * 4 > (size_t)74 * 1024) rb >>= 1;
  pl.rows_per_item = rb;
  pl.lds_bytes = (size_t)rb * S * 4;
  if (pl.lds_bytes > kLdsBudget) pl.rows_per_item = 0;
  return pl;
}

hipError_t launch_heatmap(const HeatmapArgs& a, hipStream_t stream) {
  if (heatmap_stream_applicable(a.C, a.H * a.W, a.bf16, a.heat == nullptr))
    return launch_heatmap_stream(a, stream);
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
  p.heat_bf16 = a.heat_bf16;
  p.idx = a.idx;
  p.corners = a.corners;
  p.up_corners = a.up_corners;
  p.xy = a.xy;
  p.score = a.score;

  const HeatmapPlan plan = plan_heatmap(a.C, p.S, a.bf16);
  if (plan.rows_per_item < 1) return hipErrorInvalidValue;
  p.nsteps = plan.nsteps;
  p.rows_per_item = plan.rows_per_item;
  p.items_per_crop = (a.R + plan.rows_per_item - 1) / plan.rows_per_item;
  const int crops_pad = (a.B + kXcds - 1) / kXcds * kXcds;
  const long long grid = (long long)crops_pad * p.items_per_crop;
  if (grid > INT_MAX) return hipErrorInvalidConfiguration;

  const int kstep = a.bf16 ? 32 : 16;
  // fast path: whole K steps, whole super-tiles (aligned vector loads)
  const bool fast = (a.C % kstep == 0) && (p.S % kST == 0);
  if (a.bf16)
    return fast ? launch_t<uint16_t, true>(p, plan.lds_bytes, (int)grid, stream)
                : launch_t<uint16_t, false>(p, plan.lds_bytes, (int)grid, stream);
  return fast ? launch_t<float, true>(p, plan.lds_bytes, (int)grid, stream)
              : launch_t<float, false>(p, plan.lds_bytes, (int)grid, stream);
}

}  // namespace gkd
