// decode.hip - gkd_peak_decode on gfx950: per-row heatmap peak.
//
// GKDT-L GGUF model card, section "Model", "Output" bullet: each prompt's
// heatmap peak gives a keypoint in the crop's -1..1 frame plus a score.
// One workgroup per (crop, row) scans the map with 16-byte loads, keeps a
// per-thread (value desc, index asc) best, then reduces across the wave and
// the workgroup. The order of the reduction does not matter: the
// comparison is a total order on (value, index) for non-NaN values, so the
// lowest index of the maximum always wins.
#include "gkd_device.hpp"
#include "launch.hpp"

#include <climits>
#include <cmath>

namespace gkd {
namespace {

constexpr int kDThreads = 256;

template <bool VEC>
__global__ __launch_bounds__(kDThreads) void decode_kernel(DecodeArgs p) {
  __shared__ float s_v[kDThreads / kWave];
  __shared__ int s_i[kDThreads / kWave];
  const size_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (p.valid && !p.valid[row]) {
    if (tid == 0) {
      p.idx[row] = -1;
      p.xy[2 * row] = __builtin_nanf("");
      p.xy[2 * row + 1] = __builtin_nanf("");
      p.score[row] = -INFINITY;
    }
    return;
  }
  const int P = p.Ho * p.Wo;
  const float* h = p.heat + row * (size_t)P;
  float bv = -INFINITY;
  int bi = INT_MAX;
  if (VEC) {
    const f32x4* h4 = reinterpret_cast<const f32x4*>(h);
    for (int q = tid; q < P / 4; q += kDThreads) {
      const f32x4 v = __builtin_nontemporal_load(h4 + q);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (better(v[e], 4 * q + e, bv, bi)) {
          bv = v[e];
          bi = 4 * q + e;
        }
    }
  } else {
    for (int q = tid; q < P; q += kDThreads) {
      const float v = h[q];
      if (better(v, q, bv, bi)) {
        bv = v;
        bi = q;
      }
    }
  }
  wave_argmax(bv, bi);
  if (lane == 0) {
    s_v[wave] = bv;
    s_i[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kDThreads / kWave; ++w)
      if (better(s_v[w], s_i[w], bv, bi)) {
        bv = s_v[w];
        bi = s_i[w];
      }
    const int y = bi / p.Wo, x = bi - y * p.Wo;
    p.idx[row] = bi;
    p.xy[2 * row] = keypoint_coord(x, p.Wo, p.corners);
    p.xy[2 * row + 1] = keypoint_coord(y, p.Ho, p.corners);
    p.score[row] = bv;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.R;
  if (rows > INT_MAX) return hipErrorInvalidConfiguration;
  const bool vec = ((long long)a.Ho * a.Wo) % 4 == 0;
  if (vec)
    hipLaunchKernelGGL(decode_kernel<true>, dim3((unsigned)rows), dim3(kDThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_kernel<false>, dim3((unsigned)rows), dim3(kDThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gkd
