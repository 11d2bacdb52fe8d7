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
  int tok_T, tok_skip;  // support as tokens [B, tok_T, C], pixel s at token tok_skip + s
                        //   (tok_T == 0: [B, C, H, W]; FAST is then never used)
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

  const bool tok = p.tok_T > 0;
  const T* Fb = static_cast<const T*>(p.support) +
                (tok ? ((size_t)b * p.tok_T + p.tok_skip) * p.C : (size_t)b * p.C * p.S);
  // element (channel c, pixel s) of the crop's map
  auto at = [&](int c, int s) { return tok ? (size_t)s * p.C + c : (size_t)c * p.S + s; };
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
              for (int e = 0; e < 8; ++e) h[e] = (s + e < p.S) ? F[at(c, s + e)] : 0;
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
              for (int e = 0; e < 4; ++e) bv[t][e] = (s + e < p.S) ? F[at(c, s + e)] : 0.f;
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
// outer sum is an fp32 fma per row. Item = (crop, block of up to 80 valid
// rows, 128 channels); wave w owns channel tile w (16 channels) for every
// M tile, so every support byte is read once.
//
// Persistent and pipelined: the grid is two workgroups per CU. Each
// workgroup first lists the (crop, row block) pairs that hold valid rows
// (crops without a visual prompt cost nothing after that), then walks the
// items k = blockIdx.x, + gridDim.x, ... While item k streams, the masks
// and keypoints of the next item are in flight, and the last ring refills
// of item k already fetch the first image rows of the next one, so the
// row selection and weight set-up between items overlap the HBM stream.
// ---------------------------------------------------------------------------
constexpr int kFWaves = 8;
constexpr int kFThreads = kFWaves * kWave;  // 512
constexpr int kFRows = 80;                  // valid rows per item
constexpr int kFMaxHW = 32;                 // H, W <= 32 (one half wave per weight row)
constexpr int kFCh = kFWaves * 16;          // channels per item
constexpr int kFDepth = 4;                  // image rows loaded ahead per wave
constexpr int kFMaxR = 256;                 // R <= 256 (masks and keypoints staged in LDS)
constexpr int kFList = 4096;                // (crop, row block) pairs per launch
constexpr int kFWgPerCu = 2;                // resident workgroups per CU (4 waves per SIMD)

struct VkFastParams {
  const uint16_t* support;
  const float* kpts;
  const uint8_t* valid;
  int B, C, H, W, R, S;
  bool chain;  // H % kFDepth == 0: the ring runs on into the next item
  float stride, inv_stride;
  float nl2s2;      // -log2(e) / (2 sigma^2): w = 2^(d^2 nl2s2)
  int cblocks;
  bool mask_words;  // R % 4 == 0 and the mask base 4-byte aligned
  uint16_t* protos;
  int tok_T, tok_skip;  // TOK kernels: support as tokens [B, tok_T, C], pixel s at tok_skip + s
};

// Token layout (TOK): a wave's row load brings 8 channels of one pixel per
// lane (lane = 2 j + half: pixel j, channels 8 half .. + 7 of the wave's 16);
// the row goes through the wave's LDS slice (pixel rows of kFTokRow bytes)
// and comes back through transposing reads as 8 pixels of one channel.
constexpr int kFTokRow = 48;  // 16 channels (32 B) + one pad slot

// Workgroup barrier without a memory fence: the row loads already in
// flight keep streaming (this wave's LDS writes are completed first).
__device__ __forceinline__ void lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Offset from x to the centre of the cell it falls in (clamped to the
// grid), with the cell index from a product by 1 / stride: near a cell
// border this may pick the neighbouring centre, which only changes the
// common factor that the weighted mean divides out.
__device__ __forceinline__ float centre_offset_fast(float x, float stride, float inv_stride, int n) {
  int j = (int)floorf(x * inv_stride);
  j = j < 0 ? 0 : (j > n - 1 ? n - 1 : j);
  return ((float)j + 0.5f) * stride - x;
}

// Sum over each half wave (lanes 0-31, 32-63), complete in its last lane:
// shifts by 1, 2, 4, 8 within each 16-lane row, then row 1 (3) adds the
// total of row 0 (2) broadcast from its lane 15.
__device__ __forceinline__ float dpp_add(float x, int v) { return x + __int_as_float(v); }
__device__ __forceinline__ float half_wave_sum(float x) {
  int v = __float_as_int(x);
  x = dpp_add(x, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true));  // row_shr:1
  v = __float_as_int(x);
  x = dpp_add(x, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true));  // row_shr:2
  v = __float_as_int(x);
  x = dpp_add(x, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true));  // row_shr:4
  v = __float_as_int(x);
  x = dpp_add(x, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true));  // row_shr:8
  v = __float_as_int(x);
  x = dpp_add(x, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false)); // row_bcast:15
  return x;
}

// Number of set mask bytes of one crop.
__device__ __forceinline__ int count_valid(const VkFastParams& p, int b) {
  int cnt = 0;
  if (p.mask_words) {
    const uint32_t* v = reinterpret_cast<const uint32_t*>(p.valid + (size_t)b * p.R);
#pragma unroll 4
    for (int q = 0; q < p.R / 4; ++q) {
      const uint32_t w = v[q];
      // high bit of each byte set iff that byte is nonzero
      const uint32_t t = (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
      cnt += __popc(t);
    }
  } else {
    const uint8_t* v = p.valid + (size_t)b * p.R;
#pragma unroll 8
    for (int r = 0; r < p.R; ++r) cnt += v[r] != 0;
  }
  return cnt;
}

// One item's image rows: the wave's 16 channels start at a wave-uniform
// base; lane (n16, g4) adds a fixed byte offset for channel n16 and columns
// 8 g4 .. 8 g4 + 7 (lanes past the row's columns re-read column 0 and
// contribute zeros).
template <bool TOK>
__device__ __forceinline__ const char* item_base(const VkFastParams& p, int b, int c0) {
  if constexpr (TOK)
    return reinterpret_cast<const char*>(p.support + ((size_t)b * p.tok_T + p.tok_skip) * p.C + c0);
  return reinterpret_cast<const char*>(p.support + ((size_t)b * p.C + c0) * p.S);
}
__device__ __forceinline__ u32x4 load_row(const char* base, uint32_t loff) {
  return *reinterpret_cast<const u32x4*>(base + loff);
}

// Streams one item through the ring and writes its prototypes. The ring
// enters holding rows 0 .. kFDepth-1 of this item (slot = row mod kFDepth)
// and, when nsrc is set (H a multiple of kFDepth), leaves holding rows
// 0 .. kFDepth-1 of the next item: the refill of slot d in the last period
// is exactly the next item's row d. Without nsrc the tail refills re-read
// the last row and the caller loads the next ring itself.
template <int MT, bool TOK>
__device__ __forceinline__ void vkp_fast_item(const VkFastParams& p, int b, int c0, int nsel,
                                              const char* src, uint32_t loff,
                                              bool col_ok, const char* nsrc,
                                              u32x4 (&ring)[kFDepth],
                                              const int* s_rows,
                                              const uint16_t (*s_wxh)[kFMaxHW],
                                              const uint16_t (*s_wxl)[kFMaxHW],
                                              const float (*s_wy)[kFRows], const float* s_inv,
                                              int lane_in, unsigned char* tok_slice) {
  // the lane-derived LDS addresses are built here, per item, rather than
  // hoisted out of the item loop and held live across it
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
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
        const int ni = i + kFDepth;
        const size_t rowb = TOK ? (size_t)p.W * p.C * 2 : (size_t)p.W * 2;
        const char* a = ni < p.H ? src + ni * rowb
                        : nsrc   ? nsrc + (ni - p.H) * rowb
                                 : src + (p.H - 1) * rowb;
        ring[d] = load_row(a, loff);
        bf16x8 bv;
        if constexpr (TOK) {
          // pixel j = lane / 2 of the row, channels 8 (lane % 2) .. + 7, to the
          // slice; back as pixels 8 g4 .. 8 g4 + 7 of channel n16 (rows
          // 8 g4 + n16 / 4 and + 4, columns 4 (n16 % 4) .. + 3)
          *reinterpret_cast<u32x4*>(tok_slice + (lane >> 1) * kFTokRow + 16 * (lane & 1)) = v;
          const uint32_t lo_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(
              tok_slice + (8 * g4 + (n16 >> 2)) * kFTokRow + 8 * (n16 & 3));
          u32x2 lo, hi;
          asm volatile(
              "ds_read_b64_tr_b16 %0, %2\n"
              "ds_read_b64_tr_b16 %1, %2 offset:%3\n"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(lo), "=&v"(hi)
              : "v"(lo_addr), "i"(4 * kFTokRow)
              : "memory");
          bv = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        } else {
          bv = __builtin_bit_cast(bf16x8, v);
        }
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

template <bool TOK>
__global__ __launch_bounds__(kFThreads, kFWgPerCu * kFWaves / 4) void vkp_fast_kernel(VkFastParams p) {
  __shared__ __align__(16) unsigned char s_tok[TOK ? kFWaves * 32 * kFTokRow : 16];
  __shared__ int s_list[kFList];  // crop << 2 | row block
  __shared__ int s_wsum[kFWaves];
  __shared__ int s_rows[kFRows];
  __shared__ uint8_t s_dummy0[kFRows], s_dummy1[kFRows];
  __shared__ int s_nvalid, s_nsel;
  __shared__ uint8_t s_valid[kFMaxR];
  __shared__ float s_kx[kFMaxR], s_ky[kFMaxR];
  __shared__ __align__(16) uint16_t s_wxh[kFRows][kFMaxHW];
  __shared__ __align__(16) uint16_t s_wxl[kFRows][kFMaxHW];
  __shared__ __align__(16) float s_wy[kFMaxHW][kFRows];
  __shared__ float s_inv[kFRows];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // (crop, row block) pairs with valid rows, in crop order: a crop with n
  // valid rows has ceil(n / kFRows) row blocks (the split select_rows uses)
  int nlist = 0;
  for (int base = 0; base < p.B; base += kFThreads) {
    const int bb = base + tid;
    const int nb = bb < p.B ? (count_valid(p, bb) + kFRows - 1) / kFRows : 0;
    int x = nb;  // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off, kWave);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) s_wsum[wave] = x;
    lds_sync();
    int first = nlist + x - nb;
    for (int w = 0; w < kFWaves; ++w) {
      const int s = s_wsum[w];
      if (w < wave) first += s;
      nlist += s;
    }
    for (int j = 0; j < nb; ++j) s_list[first + j] = (bb << 2) | j;
    lds_sync();
  }
  const int nitems = nlist * p.cblocks;
  int k = blockIdx.x;
  if (k >= nitems) return;

  const int g4 = lane >> 4;
  const bool col_ok = 8 * g4 < p.W;
  int b = 0, rblk = 0, c0 = 0;
  auto decode = [&](int kk, int& bo, int& ro, int& co) {
    const int e = kk / p.cblocks;
    const int ent = __builtin_amdgcn_readfirstlane(s_list[e]);
    bo = ent >> 2;
    ro = ent & 3;
    co = (kk - e * p.cblocks) * kFCh + 16 * wave;
  };
  decode(k, b, rblk, c0);
  bool on = c0 < p.C;
  // TOK: lane 2 j + h loads pixel j's channels 8 h .. + 7 (pixels past W
  // re-read pixel 0 and contribute zeros)
  const bool tok_ok = (lane >> 1) < p.W;
  const uint32_t loff =
      TOK ? (uint32_t)(((tok_ok ? (lane >> 1) : 0) * p.C + 8 * (lane & 1)) * 2)
          : (uint32_t)(((lane & 15) * p.S + (col_ok ? 8 * g4 : 0)) * 2);
  const bool row_ok = TOK ? tok_ok : col_ok;
  unsigned char* const tok_slice = s_tok + (TOK ? (size_t)wave * 32 * kFTokRow : 0);
  const char* src = item_base<TOK>(p, b, on ? c0 : 0);

  // masks and keypoints of the item's crop (registers until staged)
  uint8_t mv = 0;
  float mx = 0.f, my = 0.f;
  if (tid < p.R) {
    const size_t o = (size_t)b * p.R + tid;
    mv = p.valid[o];
    mx = p.kpts[2 * o];
    my = p.kpts[2 * o + 1];
  }
  u32x4 ring[kFDepth];
#pragma unroll
  for (int d = 0; d < kFDepth; ++d) {
    ring[d] = u32x4{0u, 0u, 0u, 0u};
    if (on && d < p.H) ring[d] = load_row(src + (size_t)d * (TOK ? p.W * p.C : p.W) * 2, loff);
  }

  for (;;) {
    // stage the crop's masks and keypoints, pick the item's rows
    if (tid < p.R) {
      s_valid[tid] = mv;
      s_kx[tid] = mx;
      s_ky[tid] = my;
    }
    lds_sync();
    if (wave == 0)
      select_rows(s_valid, nullptr, p.R, lane, rblk, kFRows, s_rows, s_dummy0, s_dummy1,
                  &s_nvalid, &s_nsel);
    lds_sync();
    const int nsel = s_nsel;
    // separable weight factors, each relative to the nearest cell centre,
    // for the M tiles the MFMAs read (rows past nsel, and columns past
    // W / H, get weight 0)
    const int rows16 = (nsel + 15) / 16 * 16;
#pragma nounroll
    for (int q = tid; q < rows16 * kFMaxHW; q += kFThreads) {
      const int m = q / kFMaxHW, j = q - m * kFMaxHW;
      float wx = 0.f, wy = 0.f;
      if (m < nsel) {
        const int r = s_rows[m];
        if (j < p.W) {
          const float x = s_kx[r];
          const float dx0 = centre_offset_fast(x, p.stride, p.inv_stride, p.W);
          const float d = ((float)j + 0.5f) * p.stride - x;
          wx = __builtin_amdgcn_exp2f((d * d - dx0 * dx0) * p.nl2s2);
        }
        if (j < p.H) {
          const float y = s_ky[r];
          const float dy0 = centre_offset_fast(y, p.stride, p.inv_stride, p.H);
          const float d = ((float)j + 0.5f) * p.stride - y;
          wy = __builtin_amdgcn_exp2f((d * d - dy0 * dy0) * p.nl2s2);
        }
      }
      const uint16_t hi = f32_to_bf16_bits(wx);
      const uint16_t lo = f32_to_bf16_bits(wx - bf16_bits_to_f32(hi));
      s_wxh[m][j] = hi;
      s_wxl[m][j] = lo;
      s_wy[j][m] = wy;
      // normaliser: sum_ij wy(i) wx(j) = (sum_i wy)(sum_j wx), with wx as
      // the hi + lo parts the MFMA sees; the 32 lanes of row m (a half
      // wave: kFMaxHW = 32 and q steps by whole waves) sum in registers
      const float sx = half_wave_sum(bf16_bits_to_f32(hi) + bf16_bits_to_f32(lo));
      const float sy = half_wave_sum(wy);
      if (j == kFMaxHW - 1 && m < nsel) s_inv[m] = 1.f / (sx * sy);
    }
    lds_sync();

    // the next item: its masks and keypoints are requested now, its first
    // rows by the last refills of this item's ring
    const int kn = k + (int)gridDim.x;
    const bool has_next = kn < nitems;
    int bn = 0, rn = 0, cn = 0;
    if (has_next) decode(kn, bn, rn, cn);
    const bool on_n = has_next && cn < p.C;
    const char* nsrc_all = on_n ? item_base<TOK>(p, bn, cn) : nullptr;
    const char* nsrc = p.chain ? nsrc_all : nullptr;
    if (has_next && tid < p.R) {
      const size_t o = (size_t)bn * p.R + tid;
      mv = p.valid[o];
      mx = p.kpts[2 * o];
      my = p.kpts[2 * o + 1];
    }
    if (on) {
      switch ((nsel + 15) / 16) {
        case 1: vkp_fast_item<1, TOK>(p, b, c0, nsel, src, loff, row_ok, nsrc, ring, s_rows, s_wxh, s_wxl, s_wy, s_inv, lane, tok_slice); break;
        case 2: vkp_fast_item<2, TOK>(p, b, c0, nsel, src, loff, row_ok, nsrc, ring, s_rows, s_wxh, s_wxl, s_wy, s_inv, lane, tok_slice); break;
        case 3: vkp_fast_item<3, TOK>(p, b, c0, nsel, src, loff, row_ok, nsrc, ring, s_rows, s_wxh, s_wxl, s_wy, s_inv, lane, tok_slice); break;
        case 4: vkp_fast_item<4, TOK>(p, b, c0, nsel, src, loff, row_ok, nsrc, ring, s_rows, s_wxh, s_wxl, s_wy, s_inv, lane, tok_slice); break;
        default: vkp_fast_item<5, TOK>(p, b, c0, nsel, src, loff, row_ok, nsrc, ring, s_rows, s_wxh, s_wxl, s_wy, s_inv, lane, tok_slice); break;
      }
    }
    if (on_n && !(on && p.chain)) {
#pragma unroll
      for (int d = 0; d < kFDepth; ++d)
        if (d < p.H) ring[d] = load_row(nsrc_all + (size_t)d * (TOK ? p.W * p.C : p.W) * 2, loff);
    }
    if (!has_next) break;
    k = kn;
    b = bn;
    rblk = rn;
    c0 = cn;
    on = on_n;
    src = on_n ? nsrc_all : src;
    // every wave is done with this item's rows, weights and normaliser
    // before the next set-up overwrites them
    lds_sync();
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
    f.C = a.C;
    f.H = a.H;
    f.W = a.W;
    f.R = a.R;
    f.S = a.H * a.W;
    f.chain = a.H % kFDepth == 0;
    f.stride = a.stride;
    f.inv_stride = 1.f / a.stride;
    f.nl2s2 = (float)(-1.4426950408889634 / (2.0 * (double)a.sigma * (double)a.sigma));
    f.cblocks = (a.C + kFCh - 1) / kFCh;
    f.mask_words = a.R % 4 == 0 && (reinterpret_cast<uintptr_t>(a.valid) & 3u) == 0;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int rblocks = (a.R + kFRows - 1) / kFRows;
    const int crops_per_launch = kFList / rblocks;
    // one launch per group of crops whose (crop, row block) list fits in LDS
    for (int b0 = 0; b0 < a.B; b0 += crops_per_launch) {
      const int nb = a.B - b0 < crops_per_launch ? a.B - b0 : crops_per_launch;
      const size_t rows0 = (size_t)b0 * a.R;
      f.tok_T = a.tokens ? a.tok_skip + f.S : 0;
      f.tok_skip = a.tokens ? a.tok_skip : 0;
      f.support = static_cast<const uint16_t*>(a.support) +
                  (size_t)b0 * a.C * (a.tokens ? (size_t)f.tok_T : (size_t)f.S);
      f.kpts = a.kpts + 2 * rows0;
      f.valid = a.valid + rows0;
      f.protos = static_cast<uint16_t*>(a.protos) + rows0 * a.C;
      f.B = nb;
      const long long items = (long long)nb * rblocks * f.cblocks;
      const long long cap = (long long)kFWgPerCu * (cus > 0 ? cus : 1);
      const int grid = (int)(items < cap ? items : cap);
      if (a.tokens)
        hipLaunchKernelGGL(vkp_fast_kernel<true>, dim3((unsigned)grid), dim3(kFThreads), 0, stream, f);
      else
        hipLaunchKernelGGL(vkp_fast_kernel<false>, dim3((unsigned)grid), dim3(kFThreads), 0, stream, f);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
  p.tok_T = a.tokens ? a.tok_skip + p.S : 0;
  p.tok_skip = a.tokens ? a.tok_skip : 0;
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
    return (p.S % 32 == 0 && !a.tokens) ? launch_t<uint16_t, true>(p, lds, (int)grid, stream)
                                        : launch_t<uint16_t, false>(p, lds, (int)grid, stream);
  return (p.S % 16 == 0 && !a.tokens) ? launch_t<float, true>(p, lds, (int)grid, stream)
                         : launch_t<float, false>(p, lds, (int)grid, stream);
}

}  // namespace gkd
