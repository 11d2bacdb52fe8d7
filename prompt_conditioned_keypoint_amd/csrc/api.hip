// api.hip - the C ABI of libgkdhead: argument validation, status codes,
// thread-local error text, and dispatch to the kernel launchers.
//
// Every check runs before the first HIP call, so an invalid call launches
// nothing, writes nothing and does not even touch the HIP runtime.
#include "gkdhead.h"
#include "launch.hpp"
#include "kg_launch.hpp"

#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

namespace {

thread_local char g_err[512] = "";

gkd_status fail(gkd_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

gkd_status ok() {
  g_err[0] = '\0';
  return GKD_OK;
}

constexpr long long kMaxElems = 0x7fffffffLL;  // element counts < 2^31

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

gkd_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(GKD_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int gkd_abi_version(void) { return GKD_ABI_VERSION; }

const char* gkd_status_string(int status) {
  switch (status) {
    case GKD_OK: return "GKD_OK";
    case GKD_ERR_NULL: return "GKD_ERR_NULL";
    case GKD_ERR_SHAPE: return "GKD_ERR_SHAPE";
    case GKD_ERR_DTYPE: return "GKD_ERR_DTYPE";
    case GKD_ERR_VALUE: return "GKD_ERR_VALUE";
    case GKD_ERR_UNSUPPORTED: return "GKD_ERR_UNSUPPORTED";
    case GKD_ERR_HIP: return "GKD_ERR_HIP";
    case GKD_ERR_ALIGN: return "GKD_ERR_ALIGN";
    default: return "GKD_ERR_UNKNOWN";
  }
}

const char* gkd_last_error(void) { return g_err; }

gkd_status gkd_vkp_pool(const void* support, const float* kpts_px, const uint8_t* kpt_valid,
                        int B, int C, int H, int W, int R, float stride_px, float sigma_px,
                        gkd_dtype dtype, uint32_t flags, void* protos, hipStream_t stream) {
  const bool tokens = (flags & GKD_QUERY_TOKENS) != 0;
  const int skip = (int)((flags >> 8) & 255u);
  if ((flags & ~(uint32_t)(GKD_QUERY_TOKENS | GKD_QUERY_SKIP(255))) != 0 || (!tokens && skip != 0))
    return fail(GKD_ERR_UNSUPPORTED, "gkd_vkp_pool: unknown flags 0x%x", (unsigned)flags);
  if (dtype != GKD_DTYPE_F32 && dtype != GKD_DTYPE_BF16)
    return fail(GKD_ERR_DTYPE, "gkd_vkp_pool: unknown dtype %d", (int)dtype);
  if (B < 0 || R < 0 || C < 1 || H < 1 || W < 1)
    return fail(GKD_ERR_SHAPE, "gkd_vkp_pool: bad shape B=%d C=%d H=%d W=%d R=%d", B, C, H, W, R);
  if (!std::isfinite(stride_px) || !(stride_px > 0.f))
    return fail(GKD_ERR_VALUE, "gkd_vkp_pool: stride_px must be finite and > 0");
  if (!std::isfinite(sigma_px) || !(sigma_px > 0.f))
    return fail(GKD_ERR_VALUE, "gkd_vkp_pool: sigma_px must be finite and > 0");
  if ((long long)C * H * W > kMaxElems || (long long)B * C * ((long long)H * W + skip) > kMaxElems ||
      (long long)B * R * C > kMaxElems || (long long)B * R * 2 > kMaxElems)
    return fail(GKD_ERR_SHAPE, "gkd_vkp_pool: an element count reaches 2^31");
  if (B == 0 || R == 0) return ok();
  if (!support || !kpts_px || !kpt_valid || !protos)
    return fail(GKD_ERR_NULL, "gkd_vkp_pool: NULL pointer argument");
  if (!aligned16(support) || !aligned16(protos) || !aligned4(kpts_px))
    return fail(GKD_ERR_ALIGN, "gkd_vkp_pool: support/protos need 16-byte, kpts 4-byte alignment");
  gkd::VkpArgs a;
  a.support = support;
  a.kpts = kpts_px;
  a.valid = kpt_valid;
  a.B = B;
  a.C = C;
  a.H = H;
  a.W = W;
  a.R = R;
  a.stride = stride_px;
  a.sigma = sigma_px;
  a.bf16 = dtype == GKD_DTYPE_BF16;
  a.protos = protos;
  a.tokens = tokens;
  a.tok_skip = skip;
  return hip_status(gkd::launch_vkp(a, stream), "gkd_vkp_pool");
}

gkd_status gkd_kernel_heatmap(const void* query, const void* kern_vis, const uint8_t* mask_vis,
                              const void* kern_txt, const uint8_t* mask_txt, int B, int C,
                              int H, int W, int R, gkd_dtype dtype, uint32_t flags,
                              void* heatmaps, int32_t* peak_idx, float* peak_xy,
                              float* peak_score, hipStream_t stream) {
  constexpr uint32_t kKnown = GKD_HEATMAP_BF16 | GKD_UPSAMPLE_CORNERS | GKD_COORDS_CORNERS |
                              GKD_QUERY_TOKENS | GKD_QUERY_SKIP(255);
  const bool tokens = (flags & GKD_QUERY_TOKENS) != 0;
  const int skip = (int)((flags >> 8) & 255u);
  if ((flags & ~kKnown) != 0 || (!tokens && skip != 0))
    return fail(GKD_ERR_UNSUPPORTED, "gkd_kernel_heatmap: unknown flags 0x%x", (unsigned)flags);
  if (dtype != GKD_DTYPE_F32 && dtype != GKD_DTYPE_BF16)
    return fail(GKD_ERR_DTYPE, "gkd_kernel_heatmap: unknown dtype %d", (int)dtype);
  if (B < 0 || R < 0 || C < 1 || H < 1 || W < 1)
    return fail(GKD_ERR_SHAPE, "gkd_kernel_heatmap: bad shape B=%d C=%d H=%d W=%d R=%d", B, C,
                H, W, R);
  if ((long long)B * C * ((long long)H * W + skip) > kMaxElems || (long long)B * R * C > kMaxElems ||
      (long long)B * R * 16 * H * W > kMaxElems || (long long)B * R * 2 > kMaxElems)
    return fail(GKD_ERR_SHAPE, "gkd_kernel_heatmap: an element count reaches 2^31");
  if ((long long)H * W > gkd::kHeatmapMaxS)
    return fail(GKD_ERR_UNSUPPORTED, "gkd_kernel_heatmap: H*W=%lld beyond the maximum %d",
                (long long)H * W, gkd::kHeatmapMaxS);
  {
    const bool bf16 = dtype == GKD_DTYPE_BF16;
    const bool kp = heatmaps == nullptr;
    const bool stream = gkd::heatmap_stream_applicable(C, H * W, bf16, kp);
    if (tokens && !stream)
      return fail(GKD_ERR_UNSUPPORTED,
                  "gkd_kernel_heatmap: token-layout queries need bfloat16 features, C %% 32 == 0 "
                  "and H*W %% 16 == 0 (H*W <= 576 for keypoints only)");
    const bool fits = stream ? gkd::plan_heatmap_stream(B, C, H * W, R, kp, tokens).ok
                             : gkd::plan_heatmap(C, H * W, bf16).rows_per_item >= 1;
    if (!fits)
      return fail(GKD_ERR_UNSUPPORTED,
                  "gkd_kernel_heatmap: H*W=%d does not fit the kernel's LDS budget", H * W);
  }
  if (B == 0 || R == 0) return ok();
  if (!query) return fail(GKD_ERR_NULL, "gkd_kernel_heatmap: NULL query");
  if ((kern_vis == nullptr) != (mask_vis == nullptr) ||
      (kern_txt == nullptr) != (mask_txt == nullptr))
    return fail(GKD_ERR_NULL, "gkd_kernel_heatmap: a kernel/mask pair is half NULL");
  if (!kern_vis && !kern_txt)
    return fail(GKD_ERR_NULL, "gkd_kernel_heatmap: no prompt modality given");
  const int ndec = (peak_idx != nullptr) + (peak_xy != nullptr) + (peak_score != nullptr);
  if (ndec != 0 && ndec != 3)
    return fail(GKD_ERR_NULL, "gkd_kernel_heatmap: decode outputs must be all NULL or all set");
  if (!heatmaps && ndec == 0)
    return fail(GKD_ERR_NULL, "gkd_kernel_heatmap: NULL heatmaps and no decode outputs");
  if (!aligned16(query) || (heatmaps && !aligned16(heatmaps)) ||
      (kern_vis && !aligned16(kern_vis)) ||
      (kern_txt && !aligned16(kern_txt)))
    return fail(GKD_ERR_ALIGN, "gkd_kernel_heatmap: query/kernels/heatmaps need 16-byte alignment");
  if (ndec && (!aligned4(peak_idx) || !aligned4(peak_xy) || !aligned4(peak_score)))
    return fail(GKD_ERR_ALIGN, "gkd_kernel_heatmap: decode outputs need 4-byte alignment");
  gkd::HeatmapArgs a;
  a.query = query;
  a.kv = kern_vis;
  a.mv = mask_vis;
  a.kt = kern_txt;
  a.mt = mask_txt;
  a.B = B;
  a.C = C;
  a.H = H;
  a.W = W;
  a.R = R;
  a.bf16 = dtype == GKD_DTYPE_BF16;
  a.heat = heatmaps;
  a.heat_bf16 = (flags & GKD_HEATMAP_BF16) != 0;
  a.corners = (flags & GKD_COORDS_CORNERS) != 0;
  a.up_corners = (flags & GKD_UPSAMPLE_CORNERS) != 0;
  a.tokens = tokens;
  a.tok_skip = skip;
  a.idx = peak_idx;
  a.xy = peak_xy;
  a.score = peak_score;
  return hip_status(gkd::launch_heatmap(a, stream), "gkd_kernel_heatmap");
}

gkd_status gkd_peak_decode(const float* heatmaps, const uint8_t* row_valid, int B, int R, int Ho,
                           int Wo, uint32_t flags, int32_t* peak_idx, float* peak_xy,
                           float* peak_score, hipStream_t stream) {
  if ((flags & ~(uint32_t)GKD_COORDS_CORNERS) != 0)
    return fail(GKD_ERR_UNSUPPORTED, "gkd_peak_decode: unknown flags 0x%x", (unsigned)flags);
  if (B < 0 || R < 0 || Ho < 1 || Wo < 1)
    return fail(GKD_ERR_SHAPE, "gkd_peak_decode: bad shape B=%d R=%d Ho=%d Wo=%d", B, R, Ho, Wo);
  if ((long long)B * R * Ho * Wo > kMaxElems || (long long)B * R * 2 > kMaxElems)
    return fail(GKD_ERR_SHAPE, "gkd_peak_decode: an element count reaches 2^31");
  if (B == 0 || R == 0) return ok();
  if (!heatmaps || !peak_idx || !peak_xy || !peak_score)
    return fail(GKD_ERR_NULL, "gkd_peak_decode: NULL pointer argument");
  if (!aligned16(heatmaps) || !aligned4(peak_idx) || !aligned4(peak_xy) || !aligned4(peak_score))
    return fail(GKD_ERR_ALIGN, "gkd_peak_decode: heatmaps need 16-byte, outputs 4-byte alignment");
  gkd::DecodeArgs a;
  a.heat = heatmaps;
  a.valid = row_valid;
  a.B = B;
  a.R = R;
  a.Ho = Ho;
  a.Wo = Wo;
  a.idx = peak_idx;
  a.xy = peak_xy;
  a.score = peak_score;
  a.corners = (flags & GKD_COORDS_CORNERS) != 0;
  return hip_status(gkd::launch_decode(a, stream), "gkd_peak_decode");
}

namespace {

gkd_status roi_shape(const char* fn, int H, int W, int B, int L) {
  if (H < 1 || W < 1 || H > 65535 || W > 65535 || B < 0 || B > 65535 || L < 1 || L > 4096)
    return fail(GKD_ERR_SHAPE, "%s: bad shape height=%d width=%d B=%d out_size=%d", fn, H, W, B,
                L);
  if ((long long)H * W * 3 > kMaxElems || (long long)B * 3 * L * L > kMaxElems)
    return fail(GKD_ERR_SHAPE, "%s: an element count reaches 2^31", fn);
  return GKD_OK;
}

}  // namespace

gkd_status gkd_roi_preprocess(const uint8_t* image, int height, int width, const int32_t* boxes,
                              int B, int out_size, gkd_dtype dtype, uint32_t flags, void* out,
                              hipStream_t stream) {
  if (flags != 0) return fail(GKD_ERR_UNSUPPORTED, "gkd_roi_preprocess: flags must be 0");
  if (dtype != GKD_DTYPE_F32 && dtype != GKD_DTYPE_BF16)
    return fail(GKD_ERR_DTYPE, "gkd_roi_preprocess: unknown dtype %d", (int)dtype);
  const gkd_status sh = roi_shape("gkd_roi_preprocess", height, width, B, out_size);
  if (sh != GKD_OK) return sh;
  if (B == 0) return ok();
  if (!image || !boxes || !out) return fail(GKD_ERR_NULL, "gkd_roi_preprocess: NULL pointer argument");
  if (!aligned4(image) || !aligned4(boxes) || !aligned16(out))
    return fail(GKD_ERR_ALIGN,
                "gkd_roi_preprocess: image and boxes need 4-byte, out 16-byte alignment");
  gkd::RoiArgs a;
  a.image = image;
  a.H = height;
  a.W = width;
  a.boxes = boxes;
  a.B = B;
  a.L = out_size;
  a.bf16 = dtype == GKD_DTYPE_BF16;
  a.out = out;
  return hip_status(gkd::launch_roi(a, stream), "gkd_roi_preprocess");
}

gkd_status gkd_roi_backproject(const float* xy, const int32_t* boxes, int B, int R, int height,
                               int width, int out_size, uint32_t flags, float* out_xy,
                               hipStream_t stream) {
  if (flags != 0) return fail(GKD_ERR_UNSUPPORTED, "gkd_roi_backproject: flags must be 0");
  const gkd_status sh = roi_shape("gkd_roi_backproject", height, width, B, out_size);
  if (sh != GKD_OK) return sh;
  if (R < 0) return fail(GKD_ERR_SHAPE, "gkd_roi_backproject: bad shape R=%d", R);
  if ((long long)B * R * 2 > kMaxElems)
    return fail(GKD_ERR_SHAPE, "gkd_roi_backproject: an element count reaches 2^31");
  if (B == 0 || R == 0) return ok();
  if (!xy || !boxes || !out_xy) return fail(GKD_ERR_NULL, "gkd_roi_backproject: NULL pointer argument");
  if (!aligned4(xy) || !aligned4(boxes) || !aligned4(out_xy))
    return fail(GKD_ERR_ALIGN, "gkd_roi_backproject: arrays need 4-byte alignment");
  gkd::BackprojectArgs a;
  a.xy = xy;
  a.boxes = boxes;
  a.B = B;
  a.R = R;
  a.H = height;
  a.W = width;
  a.L = out_size;
  a.out = out_xy;
  return hip_status(gkd::launch_backproject(a, stream), "gkd_roi_backproject");
}

size_t gkd_kg_workspace_size(int B, int C, int H, int W, int R, int d_ff, uint32_t flags) {
  if (B < 0 || R < 0 || C < 64 || H < 1 || W < 1 || d_ff < 64) return 0;
  return gkd::kg_workspace_bytes(B, C, H, W, R, d_ff, (flags & GKD_QUERY_TOKENS) != 0);
}

}  // extern "C"

namespace {

// Validation shared by gkd_kg_transformer and its no-allocation variant:
// everything but the workspace; fills `a` (workspace excluded) and the
// workspace size the call needs. On GKD_OK with B == 0 or R == 0 the call
// is empty (*empty set).
gkd_status kg_check(const char* fn, const void* kern_vis, const uint8_t* mask_vis,
                    const void* kern_txt, const uint8_t* mask_txt, const void* query, int B,
                    int C, int H, int W, int R, const void* weights, int n_blocks, int d_ff,
                    gkd_dtype dtype, uint32_t flags, void* out, gkd::KgArgs& a, size_t& need,
                    bool& empty) {
  const bool tokens = (flags & GKD_QUERY_TOKENS) != 0;
  const int skip = (int)((flags >> 8) & 255u);
  empty = false;
  if ((flags & ~(uint32_t)(GKD_QUERY_TOKENS | GKD_QUERY_SKIP(255))) != 0 || (!tokens && skip != 0))
    return fail(GKD_ERR_UNSUPPORTED, "%s: unknown flags 0x%x", fn, (unsigned)flags);
  if (dtype != GKD_DTYPE_F32 && dtype != GKD_DTYPE_BF16)
    return fail(GKD_ERR_DTYPE, "%s: unknown dtype %d", fn, (int)dtype);
  if (dtype != GKD_DTYPE_BF16)
    return fail(GKD_ERR_UNSUPPORTED, "%s: needs bfloat16 operands", fn);
  if (B < 0 || R < 0 || C < 1 || H < 1 || W < 1 || d_ff < 1 || n_blocks < 1)
    return fail(GKD_ERR_SHAPE, "%s: bad shape B=%d C=%d H=%d W=%d R=%d d_ff=%d "
                "n_blocks=%d", fn, B, C, H, W, R, d_ff, n_blocks);
  if (C % 64 != 0 || d_ff % 64 != 0 || n_blocks > 64 || 2LL * R > 576)
    return fail(GKD_ERR_UNSUPPORTED, "%s: needs C %% 64 == 0, d_ff %% 64 == 0, "
                "n_blocks <= 64 and 2R <= 576", fn);
  const long long HW = (long long)H * W, M = 2LL * B * R;
  if (M * (C > d_ff ? C : d_ff) > kMaxElems || B * (HW + skip) * C > kMaxElems ||
      (long long)C * C * 8 + 2LL * C * d_ff > kMaxElems / n_blocks)
    return fail(GKD_ERR_SHAPE, "%s: an element count reaches 2^31", fn);
  need = gkd::kg_workspace_bytes(B, C, H, W, R, d_ff, tokens);
  if (B == 0 || R == 0) {
    empty = true;
    return ok();
  }
  if (!query || !weights || !out)
    return fail(GKD_ERR_NULL, "%s: NULL pointer argument", fn);
  if (!mask_vis && !mask_txt)
    return fail(GKD_ERR_NULL, "%s: give mask_vis, mask_txt or both", fn);
  if ((mask_vis && !kern_vis) || (mask_txt && !kern_txt))
    return fail(GKD_ERR_NULL, "%s: a mask without its prototypes", fn);
  if (!aligned16(query) || !aligned16(weights) || !aligned16(out) ||
      (mask_vis && !aligned16(kern_vis)) || (mask_txt && !aligned16(kern_txt)))
    return fail(GKD_ERR_ALIGN, "%s: arrays need 16-byte alignment", fn);
  a.vis = mask_vis ? kern_vis : nullptr;
  a.mv = mask_vis;
  a.txt = mask_txt ? kern_txt : nullptr;
  a.mt = mask_txt;
  a.query = query;
  a.B = B;
  a.C = C;
  a.H = H;
  a.W = W;
  a.R = R;
  a.tok_skip = skip;
  a.tokens = tokens;
  a.weights = weights;
  a.n_blocks = n_blocks;
  a.d_ff = d_ff;
  a.out = out;
  a.ws = nullptr;
  return ok();
}

// The no-allocation variant's workspace: one array per GPU, in the
// library's device code object (placed on each GPU when the library loads
// there, held until the process ends). Its host-side name is not a device
// address: kernels get the address hipGetSymbolAddress returns for the
// current device, looked up once per device and kept in g_scratch_ptr.
constexpr size_t kKgStaticBytes = (size_t)GKD_KG_STATIC_WORKSPACE_BYTES;
static __device__ __align__(256) unsigned char scratch[kKgStaticBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// This device's address of `scratch` (the current device), or null with
// *err set.
void* scratch_on_current_device(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

gkd_status gkd_kg_transformer(const void* kern_vis, const uint8_t* mask_vis, const void* kern_txt,
                              const uint8_t* mask_txt, const void* query, int B, int C, int H,
                              int W, int R, const void* weights, int n_blocks, int d_ff,
                              gkd_dtype dtype, uint32_t flags, void* out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  gkd::KgArgs a;
  size_t need = 0;
  bool empty = false;
  const gkd_status st = kg_check("gkd_kg_transformer", kern_vis, mask_vis, kern_txt, mask_txt,
                                 query, B, C, H, W, R, weights, n_blocks, d_ff, dtype, flags, out,
                                 a, need, empty);
  if (st != GKD_OK || empty) return st;
  if (!workspace) return fail(GKD_ERR_NULL, "gkd_kg_transformer: NULL workspace");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(GKD_ERR_ALIGN, "gkd_kg_transformer: the workspace needs 256-byte alignment");
  if (workspace_bytes < need)
    return fail(GKD_ERR_VALUE, "gkd_kg_transformer: workspace of %zu bytes, needs %zu",
                workspace_bytes, need);
  a.ws = workspace;
  return hip_status(gkd::launch_kg(a, stream), "gkd_kg_transformer");
}

gkd_status gkd_kg_transformer_noalloc(const void* kern_vis, const uint8_t* mask_vis,
                                      const void* kern_txt, const uint8_t* mask_txt,
                                      const void* query, int B, int C, int H, int W, int R,
                                      const void* weights, int n_blocks, int d_ff,
                                      gkd_dtype dtype, uint32_t flags, void* out,
                                      hipStream_t stream) {
  gkd::KgArgs a;
  size_t need = 0;
  bool empty = false;
  const gkd_status st = kg_check("gkd_kg_transformer_noalloc", kern_vis, mask_vis, kern_txt,
                                 mask_txt, query, B, C, H, W, R, weights, n_blocks, d_ff, dtype,
                                 flags, out, a, need, empty);
  if (st != GKD_OK || empty) return st;
  if (need > kKgStaticBytes)
    return fail(GKD_ERR_VALUE, "gkd_kg_transformer_noalloc: this shape needs %zu bytes of "
                "workspace, the static workspace holds %zu (GKD_KG_STATIC_WORKSPACE_BYTES); "
                "use gkd_kg_transformer with a workspace of that size", need, kKgStaticBytes);
  hipError_t e = hipSuccess;
  void* ws = scratch_on_current_device(&e);
  if (ws == nullptr) return hip_status(e, "gkd_kg_transformer_noalloc: static workspace");
  a.ws = ws;
  return hip_status(gkd::launch_kg(a, stream), "gkd_kg_transformer_noalloc");
}

}  // extern "C"
