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
// Preprocess, direct form (float32 canvases, and bfloat16 ones wider than
// 2048): a workgroup per (box, 1024 quads of 4 output columns). The box
// geometry is integer arithmetic; the bilinear taps and their fractions
// come from exact integer division ((2u + 1) * bw - nw over 2 * nw), so a
// tap never depends on a rounded float, and the column taps are tabulated
// once per workgroup in LDS. The source image is small next to the output
// and is served from L2: each output pixel reads its two horizontally
// adjacent RGB taps of each source row as one 12-byte aligned window (6
// bytes at any offset fit in it) instead of twelve byte loads. The output
// planes take 16-byte (f32) or 8-byte (bf16) non-temporal stores.
// Separable form (bfloat16 canvases up to 2048): the same values with the
// horizontal step done once per source row (roi_win_kernel), which removes
// about half of the per-pixel VALU work that bounds the direct form.
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
  // halves up, at least 1 (2 * 65535 * 4096 < 2^31: 32-bit exact)
  const int lng = g.bw > g.bh ? g.bw : g.bh;
  g.nw = (2 * g.bw * L + lng) / (2 * lng);
  g.nh = (2 * g.bh * L + lng) / (2 * lng);
  g.nw = g.nw < 1 ? 1 : g.nw;
  g.nh = g.nh < 1 ? 1 : g.nh;
  g.px = (L - g.nw) / 2;
  g.py = (L - g.nh) / 2;
  return g;
}

// floor(n / d) for 0 <= n < 2^31, 0 < d < 2^14, with rd = 1/d in float:
// the float quotient is within 0.01 of n / d for quotients below 2^17, so
// one correction step makes it exact.
__device__ __forceinline__ int div_exact(int n, int d, float rd, int& rem) {
  int q = (int)((float)n * rd);
  int r = n - q * d;
  if (r < 0) {
    --q;
    r += d;
  } else if (r >= d) {
    ++q;
    r -= d;
  }
  rem = r;
  return q;
}

// Taps of output sample o (0 <= o < n_out) resized from n_in samples:
// source position (o + 1/2) n_in / n_out - 1/2 = num / den exactly,
// clamped below at 0; the upper tap clamps at the last sample.
// rden = 1 / (2 n_out).
__device__ __forceinline__ void roi_taps(int o, int n_in, int n_out, float rden, int& i0, int& i1,
                                         float& lam) {
  const int num = (2 * o + 1) * n_in - n_out, den = 2 * n_out;
  if (num <= 0) {
    i0 = 0;
    lam = 0.f;
  } else {
    int rem;
    i0 = div_exact(num, den, rden, rem);
    lam = (float)rem / (float)den;
  }
  i1 = i0 + 1 < n_in ? i0 + 1 : n_in - 1;
}

// The 8 image bytes from byte offset off (the image base is 4-byte
// aligned), as two dwords: from the aligned 12-byte window holding them,
// or, unless the caller has checked that the window stays inside the
// image (SAFE), byte by byte where it would pass the end of the image
// (total bytes; bytes past it read as 0).
template <bool SAFE>
__device__ __forceinline__ void load8(const uint8_t* img, size_t total, size_t off, uint32_t& lo,
                                      uint32_t& hi) {
  const size_t w = off & ~(size_t)3;
  if (SAFE || w + 12 <= total) {
    // three dwords through a 4-byte-aligned pointer (never a wider load)
    const uint32_t* wp = reinterpret_cast<const uint32_t*>(img + w);
    const uint32_t x0 = wp[0], x1 = wp[1], x2 = wp[2];
    const uint32_t sh = (uint32_t)(off - w);
    lo = __builtin_amdgcn_alignbyte(x1, x0, sh);  // bytes sh .. sh + 3
    hi = __builtin_amdgcn_alignbyte(x2, x1, sh);  // bytes sh + 4 .. sh + 7
  } else {
    uint32_t x[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 6; ++k)
      if (off + k < total) x[k >> 2] |= (uint32_t)img[off + k] << (8 * (k & 3));
    lo = x[0];
    hi = x[1];
  }
}

// Byte k (0..5) of the pair (lo, hi) as a float.
__device__ __forceinline__ float byte_f(uint32_t lo, uint32_t hi, int k) {
  return (float)(((k < 4 ? lo : hi) >> (8 * (k & 3))) & 0xffu);
}

struct RoiNorm {
  float scale[3], bias[3], pad[3];  // value = v * scale + bias (v in 0..255)
};

constexpr int kQuadsPerThread = 4;  // output quads (4 columns) per thread
constexpr int kQuadsPerBlock = kQuadsPerThread * kRThreads;

// One workgroup: one box, kQuadsPerBlock consecutive column quads of its
// canvas (several rows). The box geometry and the column taps of the whole
// canvas width (byte offset of the left tap in the crop row, and its
// fraction; -1 for pad columns) are set up once in LDS; a thread's quads
// are kRThreads apart, so each store instruction stays contiguous.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kRThreads) void roi_kernel(RoiArgs a, RoiNorm nm) {
  extern __shared__ __align__(16) int2 s_col[];  // [L]: (3 s0 or -1, lx bits)
  __shared__ RoiGeom sg;
  const int b = blockIdx.y;
  if (threadIdx.x == 0) sg = roi_geom(a.boxes + 4 * (size_t)b, a.H, a.W, a.L);
  __syncthreads();
  const RoiGeom g = sg;
  const float rw = 1.f / (float)(2 * g.nw), rh = 1.f / (float)(2 * g.nh);
  for (int u = threadIdx.x; u < a.L; u += kRThreads) {
    int2 e = {-1, 0};
    if (g.bw > 0 && u >= g.px && u < g.px + g.nw) {
      int s0, s1;
      float lx;
      roi_taps(u - g.px, g.bw, g.nw, rw, s0, s1, lx);
      // at the right edge both taps are the last pixel: weight 0 on the
      // second makes the value that pixel's
      e = {3 * s0, __float_as_int(s1 != s0 ? lx : 0.f)};
    }
    s_col[u] = e;
  }
  __syncthreads();

  const uint8_t* __restrict__ img = a.image;
  const size_t total = (size_t)a.H * a.W * 3;
  const int Q = (a.L + 3) / 4;  // column quads per output row
  const float rq = 1.f / (float)Q;
  const size_t plane = (size_t)a.L * a.L;
#pragma unroll
  for (int k = 0; k < kQuadsPerThread; ++k) {
    const int t = blockIdx.x * kQuadsPerBlock + k * kRThreads + (int)threadIdx.x;
    if (t >= a.L * Q) break;
    int rem;
    const int v = div_exact(t, Q, rq, rem), u0 = 4 * rem;
    float o[3][4];
    const bool row_in = g.bw > 0 && v >= g.py && v < g.py + g.nh;
    int r0 = 0, r1 = 0;
    float ly = 0.f;
    if (row_in) roi_taps(v - g.py, g.bh, g.nh, rh, r0, r1, ly);
    const size_t row0 = ((size_t)(g.y0 + r0) * a.W + g.x0) * 3;
    const size_t row1 = ((size_t)(g.y0 + r1) * a.W + g.x0) * 3;
    // every window of this row pair ends by byte row1 + 3 bw + 9 (r0 <= r1)
    const bool safe = row1 + 3 * (size_t)g.bw + 12 <= total;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int2 col = u0 + e < a.L ? s_col[u0 + e] : int2{-1, 0};
      if (row_in && col.x >= 0) {
        const float lx = __int_as_float(col.y);
        uint32_t a0, a1, c0, c1;  // taps s0, s0 + 1 of rows r0 and r1
        if (safe) {
          load8<true>(img, total, row0 + col.x, a0, a1);
          load8<true>(img, total, row1 + col.x, c0, c1);
        } else {
          load8<false>(img, total, row0 + col.x, a0, a1);
          load8<false>(img, total, row1 + col.x, c0, c1);
        }
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          const float p00 = byte_f(a0, a1, c), p01 = byte_f(a0, a1, 3 + c);
          const float p10 = byte_f(c0, c1, c), p11 = byte_f(c0, c1, 3 + c);
          const float top = fmaf(lx, p01 - p00, p00);
          const float bot = fmaf(lx, p11 - p10, p10);
          o[c][e] = fmaf(fmaf(ly, bot - top, top), nm.scale[c], nm.bias[c]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 3; ++c) o[c][e] = nm.pad[c];
      }
    }

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
}

// Separable form: a thread owns two canvas columns of one box and walks
// kRRows canvas rows down them, keeping the horizontal interpolation of the
// two source rows the current canvas row uses (its top and bottom taps) and
// computing one only when a canvas row moves to a source row it does not
// hold yet. The values are the direct form's, bit for bit (the same top and
// bottom, then the same vertical step), with the horizontal work and the
// image reads done about once per source row instead of twice per canvas
// row. All threads of a workgroup walk the same rows, so the reuse tests are
// uniform. A workgroup: one box, kRRows rows, all column pairs (up to
// kRWinMaxL columns).
constexpr int kRRows = 8;
constexpr int kRWinMaxL = 2048;  // 1024 threads of two columns

struct RoiCols {
  int off[2];    // 3 s0 of the left tap, -1: pad column
  float lx[2];
};

template <bool BF16, bool VEC>
__global__ __launch_bounds__(1024) void roi_win_kernel(RoiArgs a, RoiNorm nm) {
  const int b = blockIdx.y, v0 = blockIdx.x * kRRows, u0 = 2 * (int)threadIdx.x;
  const RoiGeom g = roi_geom(a.boxes + 4 * (size_t)b, a.H, a.W, a.L);
  const int L = a.L;
  if (u0 >= L) return;  // no barrier below
  const float rw = 1.f / (float)(2 * g.nw), rh = 1.f / (float)(2 * g.nh);
  RoiCols cols;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int u = u0 + e;
    cols.off[e] = -1;
    cols.lx[e] = 0.f;
    if (g.bw > 0 && u < L && u >= g.px && u < g.px + g.nw) {
      int s0, s1;
      float lx;
      roi_taps(u - g.px, g.bw, g.nw, rw, s0, s1, lx);
      // at the right edge both taps are the last pixel: weight 0 on the
      // second makes the value that pixel's
      cols.off[e] = 3 * s0;
      cols.lx[e] = s1 != s0 ? lx : 0.f;
    }
  }
  const uint8_t* __restrict__ img = a.image;
  const size_t total = (size_t)a.H * a.W * 3;
  // horizontal interpolation of source row r (in the crop) at this
  // thread's columns, the three channels
  auto hrow = [&](int r, float (&h)[3][2]) {
    const size_t row = ((size_t)(g.y0 + r) * a.W + g.x0) * 3;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (cols.off[e] >= 0) {
        uint32_t lo, hi;
        load8<false>(img, total, row + (size_t)cols.off[e], lo, hi);
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          const float p0 = byte_f(lo, hi, c), p1 = byte_f(lo, hi, 3 + c);
          h[c][e] = fmaf(cols.lx[e], p1 - p0, p0);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 3; ++c) h[c][e] = 0.f;
      }
    }
  };
  int ra = -1, rb = -1;  // source rows held in ha and hb
  float ha[3][2], hb[3][2];
#pragma unroll
  for (int c = 0; c < 3; ++c) ha[c][0] = ha[c][1] = hb[c][0] = hb[c][1] = 0.f;
  const size_t plane = (size_t)L * L;
  for (int k = 0; k < kRRows; ++k) {
    const int v = v0 + k;
    if (v >= L) break;
    float o[3][2];
    if (g.bw > 0 && v >= g.py && v < g.py + g.nh) {
      int r0, r1;
      float ly;
      roi_taps(v - g.py, g.bh, g.nh, rh, r0, r1, ly);
      // (ra, rb) <- (r0, r1), reusing what is held (r0 <= r1 <= r0 + 1, and
      // both move down with v)
      if (r0 != ra) {
        if (r0 == rb) {
#pragma unroll
          for (int c = 0; c < 3; ++c) ha[c][0] = hb[c][0], ha[c][1] = hb[c][1];
        } else {
          hrow(r0, ha);
        }
        ra = r0;
      }
      if (r1 != rb) {
        if (r1 == ra) {
#pragma unroll
          for (int c = 0; c < 3; ++c) hb[c][0] = ha[c][0], hb[c][1] = ha[c][1];
        } else {
          hrow(r1, hb);
        }
        rb = r1;
      }
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int c = 0; c < 3; ++c)
          o[c][e] = cols.off[e] >= 0
                        ? fmaf(fmaf(ly, hb[c][e] - ha[c][e], ha[c][e]), nm.scale[c], nm.bias[c])
                        : nm.pad[c];
    } else {
#pragma unroll
      for (int c = 0; c < 3; ++c) o[c][0] = o[c][1] = nm.pad[c];
    }
    const size_t base = (size_t)b * 3 * plane + (size_t)v * L + u0;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      if constexpr (BF16) {
        uint16_t* dst = static_cast<uint16_t*>(a.out) + base + c * plane;
        const uint32_t w =
            __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[c][0], o[c][1]}, bf16x2));
        if constexpr (VEC) {
          __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(dst));
        } else {
          dst[0] = (uint16_t)(w & 0xffffu);
          if (u0 + 1 < L) dst[1] = (uint16_t)(w >> 16);
        }
      } else {
        float* dst = static_cast<float*>(a.out) + base + c * plane;
        if constexpr (VEC) {
          __builtin_nontemporal_store(f32x2{o[c][0], o[c][1]}, reinterpret_cast<f32x2*>(dst));
        } else {
          dst[0] = o[c][0];
          if (u0 + 1 < L) dst[1] = o[c][1];
        }
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
  const bool vec = a.L % 4 == 0;
  // bfloat16 canvases: the separable form (its lower VALU count decides);
  // float32 ones: the direct form, whose 16-byte stores keep the write
  // stream at its rate
  if (a.bf16 && a.L <= kRWinMaxL) {
    const int threads = ((a.L + 1) / 2 + kWave - 1) / kWave * kWave;
    const dim3 grid((unsigned)((a.L + kRRows - 1) / kRRows), (unsigned)a.B);
    if (a.L % 2 == 0)
      hipLaunchKernelGGL((roi_win_kernel<true, true>), grid, dim3(threads), 0, stream, a, nm);
    else
      hipLaunchKernelGGL((roi_win_kernel<true, false>), grid, dim3(threads), 0, stream, a, nm);
    return hipGetLastError();
  }
  const long long quads = (long long)a.L * ((a.L + 3) / 4);
  const dim3 grid((unsigned)((quads + kQuadsPerBlock - 1) / kQuadsPerBlock), (unsigned)a.B);
  const size_t lds = (size_t)a.L * sizeof(int2);  // the column table
  if (a.bf16) {
    if (vec)
      hipLaunchKernelGGL((roi_kernel<true, true>), grid, dim3(kRThreads), lds, stream, a, nm);
    else
      hipLaunchKernelGGL((roi_kernel<true, false>), grid, dim3(kRThreads), lds, stream, a, nm);
  } else {
    if (vec)
      hipLaunchKernelGGL((roi_kernel<false, true>), grid, dim3(kRThreads), lds, stream, a, nm);
    else
      hipLaunchKernelGGL((roi_kernel<false, false>), grid, dim3(kRThreads), lds, stream, a, nm);
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
