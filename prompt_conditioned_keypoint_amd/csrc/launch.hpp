// launch.hpp - internal interface between the C ABI (api.hip) and the
// kernel translation units. Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gkd {

struct HeatmapArgs {
  const void* query;
  const void* kv;
  const uint8_t* mv;
  const void* kt;
  const uint8_t* mt;
  int B, C, H, W, R;
  bool bf16;
  float* heat;
  int32_t* idx;
  float* xy;
  float* score;
};

struct VkpArgs {
  const void* support;
  const float* kpts;
  const uint8_t* valid;
  int B, C, H, W, R;
  float stride, sigma;
  bool bf16;
  void* protos;
};

struct DecodeArgs {
  const float* heat;
  const uint8_t* valid;
  int B, R, Ho, Wo;
  int32_t* idx;
  float* xy;
  float* score;
};

// Shape limits of the heatmap kernel. Its LDS holds the kernel rows of
// both modalities for all C channels plus the fused low-res maps of at least
// one row (aliased with the kernel rows for small maps).
constexpr int kHeatmapMaxS = 2304;
constexpr size_t kLdsBudget = 150 * 1024;  // of 160 KiB; the rest is static

struct HeatmapPlan {
  int cp = 0;             // C rounded up to the K step
  int ldk = 0;            // LDS row stride of the kernel tile (elements)
  int nstw = 0;           // 64-pixel super-tiles per wave
  int rows_per_item = 0;  // 0 = shape does not fit
  int p_offset = 0;       // LDS byte offset of the fused maps
  size_t lds_bytes = 0;   // dynamic LDS per workgroup
};
HeatmapPlan plan_heatmap(int C, int S, bool bf16);

hipError_t launch_heatmap(const HeatmapArgs& a, hipStream_t stream);
hipError_t launch_vkp(const VkpArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace gkd
