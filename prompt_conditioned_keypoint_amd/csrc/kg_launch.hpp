// kg_launch.hpp - internal interface between the C ABI (api.hip) and the
// kernel-generation transformer (kg.hip). Arguments arrive here already
// validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gkd {

struct KgArgs {
  const void* vis;        // [B,R,C] bf16 or null
  const uint8_t* mv;      // [B,R] or null
  const void* txt;        // [B,R,C] bf16 or null
  const uint8_t* mt;      // [B,R] or null
  const void* query;      // [B,C,H,W] bf16, or tokens [B, tok_skip + H*W, C]
  int B, C, H, W, R;
  int tok_skip;
  bool tokens;
  const void* weights;    // flat bf16 array (mask token, then per block)
  int n_blocks, d_ff;
  void* out;              // [2,B,R,C] bf16: visual kernels, then text kernels
  void* ws;               // workspace of kg_workspace_bytes() bytes, 256-B aligned
};

size_t kg_workspace_bytes(int B, int C, int H, int W, int R, int d_ff, bool tokens);
hipError_t launch_kg(const KgArgs& a, hipStream_t stream);

}  // namespace gkd
