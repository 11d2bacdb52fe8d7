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
  void* heat;      // [B,R,4H,4W] float32, or bfloat16 when heat_bf16; null: keypoints only
  bool heat_bf16;
  int32_t* idx;
  float* xy;
  float* score;
  bool corners;    // decode: corner-aligned -1..1 coordinates
  bool up_corners; // upsample on the align_corners=True grid
  int tok_skip;    // query as tokens [B, tok_skip + H*W, C] (channels last)
  bool tokens;     //   when set; otherwise [B, C, H, W]
};

struct VkpArgs {
  const void* support;
  const float* kpts;
  const uint8_t* valid;
  int B, C, H, W, R;
  float stride, sigma;
  bool bf16;
  void* protos;
  int tok_skip;    // support as tokens [B, tok_skip + H*W, C] (channels last)
  bool tokens;     //   when set; otherwise [B, C, H, W]
};

struct DecodeArgs {
  const float* heat;
  const uint8_t* valid;
  int B, R, Ho, Wo;
  int32_t* idx;
  float* xy;
  float* score;
  bool corners;    // corner-aligned -1..1 coordinates
};

struct RoiArgs {
  const uint8_t* image;   // [H,W,3] RGB
  int H, W;
  const int32_t* boxes;   // [B,4] (x0, y0, x1, y1)
  int B, L;
  bool bf16;
  void* out;              // [B,3,L,L]
};

struct BackprojectArgs {
  const float* xy;        // [B,R,2] in the canvas's -1..1 frame
  const int32_t* boxes;
  int B, R, H, W, L;
  float* out;             // [B,R,2] image coordinates
};

// Shape limits of the heatmap kernel: its LDS holds the fused low-res maps
// of at least one row (S floats).
constexpr int kHeatmapMaxS = 16384;
constexpr size_t kLdsBudget = 156 * 1024;  // of 160 KiB; the rest is static

struct HeatmapPlan {
  int nsteps = 0;         // K steps over the channels
  int rows_per_item = 0;  // 0 = shape does not fit
  size_t lds_bytes = 0;   // dynamic LDS per workgroup
};
HeatmapPlan plan_heatmap(int C, int S, bool bf16);

hipError_t launch_heatmap(const HeatmapArgs& a, hipStream_t stream);
// bf16 path in two launches: contraction (all rows of a crop per
// workgroup, low-res maps parked in the heatmap rows), then expand + decode
// (one wave per valid row)
struct StreamPlan {
  int ng = 0, chunk_px = 0, nchunks = 0, rblocks = 0, wpg = 0;
  size_t contract_lds = 0, expand_lds = 0;
  bool ok = false;
};
// keypoints_only / whole_maps: no heatmaps are written and the decode runs
// in the contraction, so every item must cover whole maps
bool heatmap_stream_applicable(int C, int S, bool bf16, bool keypoints_only);
StreamPlan plan_heatmap_stream(int B, int C, int S, int R, bool whole_maps, bool tokens);
hipError_t launch_heatmap_stream(const HeatmapArgs& a, hipStream_t stream);
hipError_t launch_vkp(const VkpArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_roi(const RoiArgs& a, hipStream_t stream);
hipError_t launch_backproject(const BackprojectArgs& a, hipStream_t stream);

}  // namespace gkd
