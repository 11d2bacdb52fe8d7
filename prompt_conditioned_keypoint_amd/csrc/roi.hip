// roi.hip - gkd_roi_preprocess / gkd_roi_backproject on gfx950: the ROI
// stage on either side of the head.
//
// GKDT-L GGUF model card, section "Model": the Input bullet resizes the
// image so that its longer side is the input size, centre-pads it to a
// square with the mean colour (124, 116, 104) and applies ImageNet
// normalisation; the Output bullet returns keypoints in the ROI's -1..1
// frame. In top-down use every detector box is one ROI. The conventions
// the card leaves open are fixed in include/gkdhead.h.
//
// Preprocess: one thread per (box, output row, 4 output columns). The box
// geometry is integer arithmetic; the bilinear taps and their fractions
// come from exact integer division ((2u + 1) * bw - nw over 2 * nw), so a
// tap never depends on a rounded float. The source image is small next to
// the output and stays in L2, so the taps are plain byte loads; the
// output planes take 16-byte (f32) or 8-byte (bf16) non-temporal stores.
#include "gkd_device.hpp"
#include "launch.hpp"

#include <cmath>

namespace gkd {
namespace {

constexpr int kRThreads = 256;

struct RoiGeom {
  int x0, y0, bw, bh;  // the box clamped to the image; bw == 0: empty
  int nw, nh, px, py;  // resized size and left / top pad
};

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

__device__ __forceinline__ RoiGeom roi_geom(const int32_t* box, int H, int W, int L) {
  RoiGeom g;
  const int x0 = clampi(box[0], 0, W), x1 = clampi(box[2], 0, W);
  const int y0 = clampi(box[1], 0, H), y1 = clampi(box[3], 0, H);
  g.x0 = x0;
  g.y0 = y0;
  g.bw = x1 > x0 ? x1 - x0 : 0;
  g.bh = y1 > y0 ? y1 - y0 : 0;
  if (g.bw == 0 || g.bh == 0) {
    g.bw = g.bh = g.nw = g.nh = g.px = g.py = 0;
    return g;
  }
  // the longer side becomes L; the shorter one round(side * L / longer),
  // halves up, at least 1
  const long long lng = g.bw > g.bh ? g.bw : g.bh;
  g.nw = (int)((2LL * g.bw * L + lng) / (2LL * lng));
  g.nh = (int)((2LL * g.bh * L + lng) / (2LL * lng));
  g.nw = g.nw < 1 ? 1 : g.nw;
  g.nh = g.nh < 1 ? 1 : g.nh;
  g.px = (L - g.nw) / 2;
  g.py = (L - g.nh) / 2;
  return g;
}

// Taps of output sample o (0 <= o < n_out) resized from n_in samples:
// source position (o + 1/2) n_in / n_out - 1/2 = num / den exactly,
// clamped below at 0; the upper tap clamps at the last sample.
__device__ __forceinline__ void roi_taps(int o, int n_in, int n_out, int& i0, int& i1, float& lam) {
  const int num = (2 * o + 1) * n_in - n_out, den = 2 * n_out;
  if (num <= 0) {
    i0 = 0;
    lam = 0.f;
  } else {
    i0 = num / den;
    lam = (float)(num - i0 * den) / (float)den;
  }
  i1 = i0 + 1 < n_in ? i0 + 1 : n_in - 1;
}

struct RoiNorm {
  float scale[3], bias[3], pad[3];  // value = v * scale + bias (v in 0..255)
};

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kRThreads) void roi_kernel(RoiArgs a, RoiNorm nm) {
  const int b = blockIdx.y;
  const int Q = (a.L + 3) / 4;  // column quads per output row
  const int t = blockIdx.x * kRThreads + threadIdx.x;
  if (t >= a.L * Q) return;
  const int v = t / Q, u0 = 4 * (t - v * Q);
  const RoiGeom g = roi_geom(a.boxes + 4 * (size_t)b, a.H, a.W, a.L);

  float o[3][4];
  const bool row_in = g.bw > 0 && v >= g.py && v < g.py + g.nh;
  int r0 = 0, r1 = 0;
  float ly = 0.f;
  if (row_in) roi_taps(v - g.py, g.bh, g.nh, r0, r1, ly);
  const uint8_t* row0 = a.image + ((size_t)(g.y0 + r0) * a.W + g.x0) * 3;
  const uint8_t* row1 = a.image + ((size_t)(g.y0 + r1) * a.W + g.x0) * 3;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int u = u0 + e;
    if (row_in && u >= g.px && u < g.px + g.nw) {
      int s0, s1;
      float lx;
      roi_taps(u - g.px, g.bw, g.nw, s0, s1, lx);
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        const float p00 = row0[3 * s0 + c], p01 = row0[3 * s1 + c];
        const float p10 = row1[3 * s0 + c], p11 = row1[3 * s1 + c];
        const float top = (1.f - lx) * p00 + lx * p01;
        const float bot = (1.f - lx) * p10 + lx * p11;
        o[c][e] = fmaf((1.f - ly) * top + ly * bot, nm.scale[c], nm.bias[c]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 3; ++c) o[c][e] = nm.pad[c];
    }
  }

  const size_t plane = (size_t)a.L * a.L;
  const size_t base = (size_t)b * 3 * plane + (size_t)v * a.L + u0;
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    if constexpr (BF16) {
      uint16_t* dst = static_cast<uint16_t*>(a.out) + base + c * plane;
      if constexpr (VEC) {
        const u32x2 w = {
            __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[c][0], o[c][1]}, bf16x2)),
            __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[c][2], o[c][3]}, bf16x2))};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(dst));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (u0 + e < a.L)
            dst[e] = (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(
                                                                 f32x2{o[c][e], 0.f}, bf16x2)) &
                                0xffffu);
      }
    } else {
      float* dst = static_cast<float*>(a.out) + base + c * plane;
      if constexpr (VEC) {
        __builtin_nontemporal_store(f32x4{o[c][0], o[c][1], o[c][2], o[c][3]},
                                    reinterpret_cast<f32x4*>(dst));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (u0 + e < a.L) dst[e] = o[c][e];
      }
    }
  }
}

__global__ __launch_bounds__(kRThreads) void backproject_kernel(BackprojectArgs a) {
  const size_t i = (size_t)blockIdx.x * kRThreads + threadIdx.x;
  if (i >= (size_t)a.B * a.R) return;
  const int b = (int)(i / (size_t)a.R);
  const RoiGeom g = roi_geom(a.boxes + 4 * (size_t)b, a.H, a.W, a.L);
  if (g.bw == 0) {
    a.out[2 * i] = __builtin_nanf("");
    a.out[2 * i + 1] = __builtin_nanf("");
    return;
  }
  // canvas position (x + 1) L / 2, less the pad, scaled back by the crop's
  // size over the resized size, plus the box origin (NaN stays NaN)
  const float half = 0.5f * (float)a.L;
  const float xc = (a.xy[2 * i] + 1.f) * half, yc = (a.xy[2 * i + 1] + 1.f) * half;
  a.out[2 * i] = (float)g.x0 + (xc - (float)g.px) * ((float)g.bw / (float)g.nw);
  a.out[2 * i + 1] = (float)g.y0 + (yc - (float)g.py) * ((float)g.bh / (float)g.nh);
}

}  // namespace

hipError_t launch_roi(const RoiArgs& a, hipStream_t stream) {
  // ImageNet statistics; the pad colour goes through the same map
  static const float kMean[3] = {0.485f, 0.456f, 0.406f};
  static const float kStd[3] = {0.229f, 0.224f, 0.225f};
  static const float kPad[3] = {124.f, 116.f, 104.f};
  RoiNorm nm;
  for (int c = 0; c < 3; ++c) {
    nm.scale[c] = 1.f / (255.f * kStd[c]);
    nm.bias[c] = -kMean[c] / kStd[c];
    nm.pad[c] = fmaf(kPad[c], nm.scale[c], nm.bias[c]);
  }
  const long long quads = (long long)a.L * ((a.L + 3) / 4);
  const dim3 grid((unsigned)((quads + kRThreads - 1) / kRThreads), (unsigned)a.B);
  const bool vec = a.L % 4 == 0;
  if (a.bf16) {
    if (vec)
      hipLaunchKernelGGL((roi_kernel<true, true>), grid, dim3(kRThreads), 0, stream, a, nm);
    else
      hipLaunchKernelGGL((roi_kernel<true, false>), grid, dim3(kRThreads), 0, stream, a, nm);
  } else {
    if (vec)
      hipLaunchKernelGGL((roi_kernel<false, true>), grid, dim3(kRThreads), 0, stream, a, nm);
    else
      hipLaunchKernelGGL((roi_kernel<false, false>), grid, dim3(kRThreads), 0, stream, a, nm);
  }
  return hipGetLastError();
}

hipError_t launch_backproject(const BackprojectArgs& a, hipStream_t stream) {
  const long long n = (long long)a.B * a.R;
  hipLaunchKernelGGL(backproject_kernel, dim3((unsigned)((n + kRThreads - 1) / kRThreads)),
                     dim3(kRThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gkd
