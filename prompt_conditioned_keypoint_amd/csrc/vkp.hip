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

template <typename T, bool FAST>
hipError_t launch_t(const VkParams& p, size_t lds, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((vkp_kernel<T, FAST>), dim3(grid), dim3(kVThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vkp(const VkpArgs& a, hipStream_t stream) {
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
