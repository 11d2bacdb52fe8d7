// vkp.hip - gkd_vkp_pool on gfx950: visual keypoint prototypes.
//
// Each prototype is the Gaussian-weighted mean of the support feature
// fibres around one support keypoint (GKDT-L GGUF model card, section
// "Model", "Prompts" bullet: soft Gaussian pooling over feature fibres at
// sigma = 14 px; reading notes, paper.gecl.asia, "Method": support features
// near the annotated point are aggregated into the prototype).
//
// As a contraction: protos[r, c] = sum_s w[r, s] F[c, s] / sum_s w[r, s]
// with M = rows, N = channels, K = pixels. In NCHW the pixel axis is the
// contiguous one, so a lane's K run is one 16-byte load; no transpose.
// Work item = (crop, block of <= 16 valid rows, block of 256 channels);
// 4 waves x 4 N-tiles of 16 channels.
//
// The Gaussian weights are generated on the fly into LDS, separable:
// w = wy(i) * wx(j), each factor taken relative to the nearest cell centre
// (exp(-(d^2 - d_min^2) / 2 sigma^2)); the common factor cancels in the
// weighted mean and keeps the largest weight at 1 so tiny sigmas cannot
// underflow every weight. For bf16 the weight is split into hi + lo
// bfloat16 parts (two MFMAs), which keeps ~16 significant bits of w; the
// fp32 path uses v_mfma_f32_16x16x4_f32 with fp32 weights.
#include "gkd_device.hpp"
#include "launch.hpp"

#include <climits>
#include <cmath>

namespace gkd {
namespace {

constexpr int kVWaves = 4;
constexpr int kVThreads = kVWaves * kWave;  // 256
constexpr int kVRows = 16;                  // rows per item (one M tile)
constexpr int kVCh = 256;                   // channels per item
constexpr int kVChunk = 576;                // pixels per weight tile in LDS

struct VkParams {
  const void* support;
  const float* kpts;
  const uint8_t* valid;
  int B, C, H, W, R, S;
  float stride, inv2s2;
  int cblocks, items_per_crop;
  int ldw;  // LDS row stride of the weight tile (elements)
  void* protos;
};

__device__ __forceinline__ float nearest_centre_offset(float x, float stride, int n) {
  int j = (int)floorf(x / stride);
  j = j < 0 ? 0 : (j > n - 1 ? n - 1 : j);
  return ((float)j + 0.5f) * stride - x;
}

template <typename T, bool FAST>
__global__ __launch_bounds__(kVThreads) void vkp_kernel(VkParams p) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int s_rows[kVRows];
  __shared__ uint8_t s_dummy0[kVRows], s_dummy1[kVRows];
  __shared__ int s_nvalid, s_nsel;
  __shared__ float s_x[kVRows], s_y[kVRows], s_dx0[kVRows], s_dy0[kVRows];
  __shared__ float s_wsum[kVRows];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const ItemCoord ic = xcd_item(blockIdx.x, p.items_per_crop);
  const int b = ic.crop;
  if (b >= p.B) return;
  const int rblk = ic.item / p.cblocks, cblk = ic.item - rblk * p.cblocks;

  if (wave == 0)
    select_rows(p.valid + (size_t)b * p.R, nullptr, p.R, lane, rblk, kVRows, s_rows,
                s_dummy0, s_dummy1, &s_nvalid, &s_nsel);
  __syncthreads();
  const int nsel = s_nsel;
  if (nsel == 0) return;

  if (tid < kVRows) {
    float x = 0.f, y = 0.f;
    if (tid < nsel) {
      const float* k = p.kpts + 2 * ((size_t)b * p.R + s_rows[tid]);
      x = k[0];
      y = k[1];
    }
    const float dx0 = nearest_centre_offset(x, p.stride, p.W);
    const float dy0 = nearest_centre_offset(y, p.stride, p.H);
    s_x[tid] = x;
    s_y[tid] = y;
    s_dx0[tid] = dx0 * dx0;
    s_dy0[tid] = dy0 * dy0;
    // normaliser: sum_ij wy(i) wx(j) = (sum_i wy)(sum_j wx)
    float sx = 0.f, sy = 0.f;
    for (int j = 0; j < p.W; ++j) {
      const float d = ((float)j + 0.5f) * p.stride - x;
      sx += expf(-(d * d - dx0 * dx0) * p.inv2s2);
    }
    for (int i = 0; i < p.H; ++i) {
      const float d = ((float)i + 0.5f) * p.stride - y;
      sy += expf(-(d * d - dy0 * dy0) * p.inv2s2);
    }
    s_wsum[tid] = sx * sy;
  }

  const int n = lane & 15, g = lane >> 4;
  const int ch0 = cblk * kVCh + wave * 64;  // first channel of this wave
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const T* Fb = static_cast<const T*>(p.support) + (size_t)b * p.C * p.S;
  constexpr bool kBf16 = sizeof(T) == 2;

  for (int s0 = 0; s0 < p.S; s0 += kVChunk) {
    const int len = (p.S - s0) < kVChunk ? (p.S - s0) : kVChunk;
    const int lenp = kBf16 ? (len + 31) / 32 * 32 : (len + 15) / 16 * 16;
    __syncthreads();  // previous tile consumed; s_* visible
    // weight tile for rows 0..15, pixels s0 .. s0+lenp (zero past S / rows)
    for (int q = tid; q < kVRows * lenp; q += kVThreads) {
      const int m = q / lenp, k = q - m * lenp, s = s0 + k;
      float w = 0.f;
      if (m < nsel && s < p.S) {
        const int i = s / p.W, j = s - i * p.W;
        const float dx = ((float)j + 0.5f) * p.stride - s_x[m];
        const float dy = ((float)i + 0.5f) * p.stride - s_y[m];
        w = expf(-(dx * dx - s_dx0[m]) * p.inv2s2) * expf(-(dy * dy - s_dy0[m]) * p.inv2s2);
      }
      if constexpr (kBf16) {
        uint16_t* Wl = reinterpret_cast<uint16_t*>(lds);
        const uint16_t hi = f32_to_bf16_bits(w);
        const uint16_t lo = f32_to_bf16_bits(w - bf16_bits_to_f32(hi));
        Wl[(size_t)m * p.ldw + k] = hi;
        Wl[(size_t)(kVRows + m) * p.ldw + k] = lo;
      } else {
        reinterpret_cast<float*>(lds)[(size_t)m * p.ldw + k] = w;
      }
    }
    __syncthreads();

    if constexpr (kBf16) {
      const uint16_t* Wl = reinterpret_cast<const uint16_t*>(lds);
      const uint16_t* F = reinterpret_cast<const uint16_t*>(Fb);
      for (int k0 = 0; k0 < lenp; k0 += 32) {
        const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(Wl + (size_t)n * p.ldw + k0 + 8 * g);
        const bf16x8 alo =
            *reinterpret_cast<const bf16x8*>(Wl + (size_t)(kVRows + n) * p.ldw + k0 + 8 * g);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int c = ch0 + 16 * t + n;
          const int s = s0 + k0 + 8 * g;
          u32x4 v = u32x4{0u, 0u, 0u, 0u};
          if (c < p.C) {
            if (FAST) {
              v = *reinterpret_cast<const u32x4*>(F + (size_t)c * p.S + s);
            } else {
              uint16_t h[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) h[e] = (s + e < p.S) ? F[(size_t)c * p.S + s + e] : 0;
              __builtin_memcpy(&v, h, 16);
            }
          }
          const bf16x8 bv = __builtin_bit_cast(bf16x8, v);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bv, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bv, acc[t], 0, 0, 0);
        }
      }
    } else {
      const float* Wl = reinterpret_cast<const float*>(lds);
      const float* F = reinterpret_cast<const float*>(Fb);
      for (int k0 = 0; k0 < lenp; k0 += 16) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(Wl + (size_t)n * p.ldw + k0 + 4 * g);
        f32x4 bv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int c = ch0 + 16 * t + n;
          const int s = s0 + k0 + 4 * g;
          bv[t] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (c < p.C) {
            if (FAST) {
              bv[t] = *reinterpret_cast<const f32x4*>(F + (size_t)c * p.S + s);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) bv[t][e] = (s + e < p.S) ? F[(size_t)c * p.S + s + e] : 0.f;
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], bv[t][e], acc[t], 0, 0, 0);
      }
    }
  }

  // D layout: lane (n, g) holds rows 4g + i, channel ch0 + 16t + n
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * g + i;
    if (m >= nsel) continue;
    const float inv = 1.f / s_wsum[m];
    const size_t row = ((size_t)b * p.R + s_rows[m]) * p.C;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = ch0 + 16 * t + n;
      if (c >= p.C) continue;
      const float v = acc[t][i] * inv;
      if constexpr (kBf16) static_cast<uint16_t*>(p.protos)[row + c] = f32_to_bf16_bits(v);
      else static_cast<float*>(p.protos)[row + c] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 fast path: the weights are separable, so
//   protos[r, c] = sum_i wy(r, i) * (sum_j wx(r, j) F[c, i, j]) / (sum wx)(sum wy)
// The inner sum is one MFMA per image row with K = j (W <= 32 columns, one
// 16-byte load of 8 pixels per lane, straight from HBM), A = wx as hi + lo
// bfloat16 parts (constant over the whole item, held in registers); the
// outer sum is an fp32 fma per row. One workgroup = (crop, 256 channels,
// all of the crop's valid rows up to 80): every support byte is read once.
// Wave w owns channel tile w (16 channels) for every M tile.
// ---------------------------------------------------------------------------
constexpr int kFWaves = 8;
constexpr int kFThreads = kFWaves * kWave;  // 512
constexpr int kFRows = 80;                  // valid rows per item
constexpr int kFMaxMT = kFRows / 16;
constexpr int kFMaxHW = 32;                 // H, W <= 32
constexpr int kFCh = kFWaves * 16;          // channels per item
constexpr int kFDepth = 6;                  // image rows loaded ahead per wave
constexpr int kFMaxR = 256;                 // R <= 256 (masks and keypoints staged in LDS)

struct VkFastParams {
  const uint16_t* support;
  const float* kpts;
  const uint8_t* valid;
  int B, C, H, W, R, S;
  float stride, inv2s2;
  int cblocks, items_per_crop;
  uint16_t* protos;
};

// Workgroup barrier without a memory fence: the row loads already in
// flight keep streaming (this wave's LDS writes are completed first).
__device__ __forceinline__ void lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int MT>
__device__ __forceinline__ void vkp_fast_item(const VkFastParams& p, int b, int c0, int nsel,
                                              int lane, const uint16_t* src, bool col_ok,
                                              u32x4 (&ring)[kFDepth], const int* s_rows,
                                              const uint16_t (*s_wxh)[kFMaxHW],
                                              const uint16_t (*s_wxl)[kFMaxHW],
                                              const float (*s_wy)[kFRows], const float* s_inv) {
  const int n16 = lane & 15, g4 = lane >> 4;
  // A: wx of row 16 h + n16 at columns 8 g4 .. 8 g4 + 7, hi and lo parts
  bf16x8 ahi[MT], alo[MT];
#pragma unroll
  for (int h = 0; h < MT; ++h) {
    ahi[h] = *reinterpret_cast<const bf16x8*>(&s_wxh[16 * h + n16][8 * g4]);
    alo[h] = *reinterpret_cast<const bf16x8*>(&s_wxl[16 * h + n16][8 * g4]);
  }
  f32x4 acc[MT];
#pragma unroll
  for (int h = 0; h < MT; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i0 = 0; i0 < p.H; i0 += kFDepth) {
#pragma unroll
    for (int d = 0; d < kFDepth; ++d) {
      const int i = i0 + d;
      if (i < p.H) {
        const u32x4 v = col_ok ? ring[d] : u32x4{0u, 0u, 0u, 0u};
        const int in = i + kFDepth < p.H ? i + kFDepth : p.H - 1;
        ring[d] = *reinterpret_cast<const u32x4*>(src + (size_t)in * p.W);
        const bf16x8 bv = __builtin_bit_cast(bf16x8, v);
#pragma unroll
        for (int h = 0; h < MT; ++h) {
          f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[h], bv, f32x4{0.f, 0.f, 0.f, 0.f},
                                                            0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[h], bv, t, 0, 0, 0);
          const f32x4 wy = *reinterpret_cast<const f32x4*>(&s_wy[i][16 * h + 4 * g4]);
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[h][k] = fmaf(wy[k], t[k], acc[h][k]);
        }
      }
    }
  }
  // D layout: lane (n16, g4) holds rows 16 h + 4 g4 + k of channel c0 + n16
#pragma unroll
  for (int h = 0; h < MT; ++h) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int m = 16 * h + 4 * g4 + k;
      if (m < nsel)
        p.protos[((size_t)b * p.R + s_rows[m]) * p.C + c0 + n16] =
            f32_to_bf16_bits(acc[h][k] * s_inv[m]);
    }
  }
}

__global__ __launch_bounds__(kFThreads, 2) void vkp_fast_kernel(VkFastParams p) {
  __shared__ int s_rows[kFRows];
  __shared__ uint8_t s_dummy0[kFRows], s_dummy1[kFRows];
  __shared__ int s_nvalid, s_nsel;
  __shared__ uint8_t s_valid[kFMaxR];
  __shared__ float s_kx[kFMaxR], s_ky[kFMaxR];
  __shared__ __align__(16) uint16_t s_wxh[kFRows][kFMaxHW];
  __shared__ __align__(16) uint16_t s_wxl[kFRows][kFMaxHW];
  __shared__ __align__(16) float s_wy[kFMaxHW][kFRows];
  __shared__ float s_x[kFRows], s_y[kFRows], s_dx0[kFRows], s_dy0[kFRows], s_inv[kFRows];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const ItemCoord ic = xcd_item(blockIdx.x, p.items_per_crop);
  const int b = ic.crop;
  if (b >= p.B) return;
  const int rblk = ic.item / p.cblocks, cblk = ic.item - rblk * p.cblocks;

  // the crop's masks and keypoints in one round trip, then rows from LDS
  if (tid < p.R) {
    const size_t o = (size_t)b * p.R + tid;
    s_valid[tid] = p.valid[o];
    s_kx[tid] = p.kpts[2 * o];
    s_ky[tid] = p.kpts[2 * o + 1];
  }
  lds_sync();
  if (wave == 0)
    select_rows(s_valid, nullptr, p.R, lane, rblk, kFRows, s_rows, s_dummy0, s_dummy1, &s_nvalid,
                &s_nsel);
  lds_sync();
  const int nsel = s_nsel;
  if (nsel == 0) return;
  const int MT = (nsel + 15) / 16;

  // B of wave w: channel c0 + n16, image row i, columns 8 g4 .. 8 g4 + 7
  // (lanes past the row's columns carry zeros). The first kFDepth rows are
  // requested now, ahead of the weight set-up.
  const int c0 = cblk * kFCh + 16 * wave;
  const bool wave_on = c0 < p.C;
  const int g4 = lane >> 4;
  const bool col_ok = 8 * g4 < p.W;
  const uint16_t* src =
      p.support + ((size_t)b * p.C + (wave_on ? c0 : 0) + (lane & 15)) * p.S + (col_ok ? 8 * g4 : 0);
  u32x4 ring[kFDepth];
  if (wave_on) {
#pragma unroll
    for (int d = 0; d < kFDepth; ++d) {
      const int i = d < p.H ? d : p.H - 1;
      ring[d] = *reinterpret_cast<const u32x4*>(src + (size_t)i * p.W);
    }
  }

  // per-row keypoint and nearest-centre offsets (rows past nsel: weight 0)
  if (tid < kFRows) {
    float x = 0.f, y = 0.f;
    if (tid < nsel) {
      x = s_kx[s_rows[tid]];
      y = s_ky[s_rows[tid]];
    }
    const float dx0 = nearest_centre_offset(x, p.stride, p.W);
    const float dy0 = nearest_centre_offset(y, p.stride, p.H);
    s_x[tid] = x;
    s_y[tid] = y;
    s_dx0[tid] = dx0 * dx0;
    s_dy0[tid] = dy0 * dy0;
  }
  lds_sync();
  // separable weight factors, each relative to the nearest cell centre
  for (int q = tid; q < kFRows * kFMaxHW; q += kFThreads) {
    const int m = q / kFMaxHW, j = q - m * kFMaxHW;
    float wx = 0.f, wy = 0.f;
    if (m < nsel) {
      if (j < p.W) {
        const float d = ((float)j + 0.5f) * p.stride - s_x[m];
        wx = expf(-(d * d - s_dx0[m]) * p.inv2s2);
      }
      if (j < p.H) {
        const float d = ((float)j + 0.5f) * p.stride - s_y[m];
        wy = expf(-(d * d - s_dy0[m]) * p.inv2s2);
      }
    }
    const uint16_t hi = f32_to_bf16_bits(wx);
    s_wxh[m][j] = hi;
    s_wxl[m][j] = f32_to_bf16_bits(wx - bf16_bits_to_f32(hi));
    s_wy[j][m] = wy;
  }
  lds_sync();
  // normaliser: sum_ij wy(i) wx(j) = (sum_i wy)(sum_j wx), with wx as the
  // hi + lo parts the MFMA sees
  if (tid < nsel) {
    float sx = 0.f, sy = 0.f;
    for (int j = 0; j < p.W; ++j)
      sx += bf16_bits_to_f32(s_wxh[tid][j]) + bf16_bits_to_f32(s_wxl[tid][j]);
    for (int i = 0; i < p.H; ++i) sy += s_wy[i][tid];
    s_inv[tid] = 1.f / (sx * sy);
  }
  lds_sync();
  if (!wave_on) return;
  switch (MT) {
    case 1: vkp_fast_item<1>(p, b, c0, nsel, lane, src, col_ok, ring, s_rows, s_wxh, s_wxl, s_wy, s_inv); break;
    case 2: vkp_fast_item<2>(p, b, c0, nsel, lane, src, col_ok, ring, s_rows, s_wxh, s_wxl, s_wy, s_inv); break;
    case 3: vkp_fast_item<3>(p, b, c0, nsel, lane, src, col_ok, ring, s_rows, s_wxh, s_wxl, s_wy, s_inv); break;
    case 4: vkp_fast_item<4>(p, b, c0, nsel, lane, src, col_ok, ring, s_rows, s_wxh, s_wxl, s_wy, s_inv); break;
    default: vkp_fast_item<5>(p, b, c0, nsel, lane, src, col_ok, ring, s_rows, s_wxh, s_wxl, s_wy, s_inv); break;
  }
}

template <typename T, bool FAST>
hipError_t launch_t(const VkParams& p, size_t lds, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((vkp_kernel<T, FAST>), dim3(grid), dim3(kVThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vkp(const VkpArgs& a, hipStream_t stream) {
  if (a.bf16 && a.W <= kFMaxHW && a.H <= kFMaxHW && a.W % 8 == 0 && a.C % 16 == 0 &&
      a.R <= kFMaxR) {
    VkFastParams f;
    f.support = static_cast<const uint16_t*>(a.support);
    f.kpts = a.kpts;
    f.valid = a.valid;
    f.B = a.B;
    f.C = a.C;
    f.H = a.H;
    f.W = a.W;
    f.R = a.R;
    f.S = a.H * a.W;
    f.stride = a.stride;
    f.inv2s2 = 1.f / (2.f * a.sigma * a.sigma);
    f.protos = static_cast<uint16_t*>(a.protos);
    f.cblocks = (a.C + kFCh - 1) / kFCh;
    f.items_per_crop = ((a.R + kFRows - 1) / kFRows) * f.cblocks;
    const int crops_pad = (a.B + kXcds - 1) / kXcds * kXcds;
    const long long grid = (long long)crops_pad * f.items_per_crop;
    if (grid > INT_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(vkp_fast_kernel, dim3((unsigned)grid), dim3(kFThreads), 0, stream, f);
    return hipGetLastError();
  }
  VkParams p;
  p.support = a.support;
  p.kpts = a.kpts;
  p.valid = a.valid;
  p.B = a.B;
  p.C = a.C;
  p.H = a.H;
  p.W = a.W;
  p.R = a.R;
  p.S = a.H * a.W;
  p.stride = a.stride;
  p.inv2s2 = 1.f / (2.f * a.sigma * a.sigma);
  p.protos = a.protos;
  p.cblocks = (a.C + kVCh - 1) / kVCh;
  const int rblocks = (a.R + kVRows - 1) / kVRows;
  p.items_per_crop = rblocks * p.cblocks;
  const int chunk = p.S < kVChunk ? p.S : kVChunk;
  size_t lds;
  if (a.bf16) {
    p.ldw = (chunk + 31) / 32 * 32 + 8;
    lds = (size_t)2 * kVRows * p.ldw * 2;
  } else {
    p.ldw = (chunk + 15) / 16 * 16 + 4;
    lds = (size_t)kVRows * p.ldw * 4;
  }
  const int crops_pad = (a.B + kXcds - 1) / kXcds * kXcds;
  const long long grid = (long long)crops_pad * p.items_per_crop;
  if (grid > INT_MAX) return hipErrorInvalidConfiguration;
  if (a.bf16)
    return (p.S % 32 == 0) ? launch_t<uint16_t, true>(p, lds, (int)grid, stream)
                           : launch_t<uint16_t, false>(p, lds, (int)grid, stream);
  return (p.S % 16 == 0) ? launch_t<float, true>(p, lds, (int)grid, stream)
                         : launch_t<float, false>(p, lds, (int)grid, stream);
}

}  // namespace gkd
