/*
 * gkdhead.h - C ABI of libgkdhead, the GKDT parameter-free detection head
 * on AMD Instinct MI355X (gfx950).
 *
 * The head turns prompt kernels and dense query features into heatmaps and
 * keypoints (GKDT-L GGUF model card, huggingface.co/Asher-1/GKD_GGUF,
 * section "Model"; GKDT paper summary, agihunt.info, pipeline paragraph):
 *   1. gkd_vkp_pool       Gaussian pooling of support feature fibres around
 *                         each support keypoint (visual keypoint prototypes);
 *   2. gkd_kernel_heatmap L2-normalised kernel rows applied as a 1x1
 *                         convolution to the 4x bilinearly upsampled query
 *                         features, fused per row over the prompt modalities,
 *                         optionally with the peak decode fused in;
 *   3. gkd_peak_decode    per-row argmax of a heatmap, mapped to -1..1, plus
 *                         the score;
 * and the ROI stage either side of the head in top-down use:
 *   4. gkd_roi_preprocess   crop, resize, centre-pad and normalise detector
 *                           boxes of an image into the backbone's input;
 *   5. gkd_roi_backproject  -1..1 keypoints back to image coordinates;
 * and the step that makes the kernels from the prototypes:
 *   6. gkd_kg_transformer   the kernel-generation transformer (with
 *                           gkd_kg_workspace_size for its workspace).
 *
 * Conventions shared by every call:
 *   - Every array argument is a DEVICE pointer owned by the caller, dense
 *     and row-major in the shape given. Feature maps, kernel rows,
 *     prototypes and heatmaps must be 16-byte aligned, keypoints and decode
 *     outputs 4-byte aligned (else GKD_ERR_ALIGN); masks have no
 *     alignment requirement. The library
 *     allocates no memory and keeps no state besides a thread-local error
 *     text, so calls are re-entrant.
 *   - Calls are asynchronous and ordered on `stream` (0 = the null stream).
 *     The library never synchronises. Faults inside a kernel surface at the
 *     caller's next synchronisation as a HIP error.
 *   - Arguments are validated before anything is launched: on any status
 *     other than GKD_OK nothing is launched and no output byte is written.
 *     gkd_last_error() then describes the failure.
 *   - Outputs must not overlap inputs or each other.
 *   - B == 0 or R == 0 is an empty batch: GKD_OK, nothing launched.
 *   - Every element count (e.g. B*R*4H*4W) must be below 2^31.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified results.
 *   - Kernel-row norms are taken in float32, so every kernel row of
 *     gkd_kernel_heatmap must have ||k||_2 < 2^64 (about 1.8e19; bfloat16
 *     rows reach it only with elements above about 5.8e17). Larger rows
 *     give unspecified results (their squared norm overflows to infinity
 *     and the row's map comes out zero). Rows with ||k||_2 below 1e-12,
 *     zero rows included, are scaled by 1e12 (the clamp of the norm).
 *   - `flags` must be 0 (else GKD_ERR_UNSUPPORTED), except for the
 *     heatmap output format, upsample grid and query layout flags of
 *     gkd_kernel_heatmap (GKD_HEATMAP_BF16, GKD_UPSAMPLE_CORNERS,
 *     GKD_QUERY_TOKENS with GKD_QUERY_SKIP, which gkd_vkp_pool and
 *     gkd_kg_transformer accept too) and the keypoint coordinate flag of
 *     gkd_kernel_heatmap and gkd_peak_decode (GKD_COORDS_CORNERS).
 *
 * ABI history: version 1 had float32 heatmaps only; version 2 adds
 * GKD_HEATMAP_BF16 (gkd_kernel_heatmap's heatmaps argument became void *,
 * which existing callers pass unchanged); version 3 adds the ROI stage
 * (gkd_roi_preprocess, gkd_roi_backproject); version 4 adds
 * GKD_COORDS_CORNERS; version 5 adds GKD_UPSAMPLE_CORNERS; version 6 adds
 * GKD_QUERY_TOKENS; version 7 accepts it in gkd_vkp_pool for the support
 * map; version 8 adds the kernel-generation transformer
 * (gkd_kg_workspace_size, gkd_kg_transformer); version 9 adds
 * gkd_kg_transformer_noalloc.
 */
#ifndef GKDHEAD_H
#define GKDHEAD_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GKD_ABI_VERSION 9

/* gkd_kernel_heatmap flag: store the heatmaps as bfloat16 instead of float32
 * (half the bytes of the dominant output stream). */
#define GKD_HEATMAP_BF16 0x1u
/* gkd_kernel_heatmap flag: upsample on the align_corners=True grid (first
 * and last outputs on the first and last low-res samples: source position
 * o (n - 1) / (4n - 1)) instead of half-pixel centres. */
#define GKD_UPSAMPLE_CORNERS 0x2u
/* gkd_kernel_heatmap and gkd_peak_decode flag: map the peak index to -1..1
 * corner-aligned, x = 2 col / (Wo - 1) - 1 (0 when Wo == 1), instead of
 * the cell centre (2 col + 1) / Wo - 1; likewise y. */
#define GKD_COORDS_CORNERS 0x4u
/* gkd_kernel_heatmap flag: the query arrives as the ViT's token sequence,
 * [B, skip + H*W, C] with channels last, pixel (y, x) at token
 * skip + y*W + x; skip (the leading class / storage tokens, 0..255) goes in
 * bits 8..15 via GKD_QUERY_SKIP. Needs bfloat16 features, C % 32 == 0 and
 * H*W % 16 == 0 (H*W <= 576 for keypoints only), else
 * GKD_ERR_UNSUPPORTED. The results equal, bit for bit, those of the same
 * call on the [B, C, H, W] layout. gkd_vkp_pool takes the same flag for its
 * support map, for any dtype and shape, and its prototypes equal those of
 * the same call on the [B, C, H, W] layout bit for bit: bfloat16 maps with
 * H, W <= 32, W % 8 == 0, C % 16 == 0 and R <= 256 take the fast VKP kernel
 * in either layout, all other shapes and float32 the general one. */
#define GKD_QUERY_TOKENS 0x8u
#define GKD_QUERY_SKIP(n) (((uint32_t)(n) & 255u) << 8)

#ifndef GKD_API
#define GKD_API __attribute__((visibility("default")))
#endif

typedef enum {
    GKD_OK = 0,
    GKD_ERR_NULL = 1,        /* required pointer NULL, or a pointer group half NULL */
    GKD_ERR_SHAPE = 2,       /* negative/zero size, or an element count >= 2^31   */
    GKD_ERR_DTYPE = 3,       /* dtype not one of gkd_dtype                         */
    GKD_ERR_VALUE = 4,       /* stride or sigma not finite and positive           */
    GKD_ERR_UNSUPPORTED = 5, /* nonzero flags, or a shape beyond the kernels' limits */
    GKD_ERR_HIP = 6,         /* the HIP runtime refused a launch                   */
    GKD_ERR_ALIGN = 7        /* a pointer is not 16-byte aligned                    */
} gkd_status;

typedef enum {
    GKD_DTYPE_F32 = 0,  /* IEEE float32 */
    GKD_DTYPE_BF16 = 1  /* bfloat16 (upper half of a float32) */
} gkd_dtype;

/* ABI version of the loaded library (GKD_ABI_VERSION). */
GKD_API int gkd_abi_version(void);

/* Static, never-NULL name of a status code (unknown codes included). */
GKD_API const char *gkd_status_string(int status);

/* Thread-local detail of the calling thread's last failed call ("" if the
 * last call succeeded). Valid until the thread's next gkd_* call. */
GKD_API const char *gkd_last_error(void);

/*
 * Visual keypoint prototypes (VKP).
 * GKDT-L GGUF model card, section "Model", "Prompts" bullet: a 1-shot visual
 * prompt is pooled from the support features with a soft Gaussian over the
 * feature fibres, sigma = 14 px; the paper summary (agihunt.info, pipeline
 * paragraph) takes the prototypes from Gaussian heatmaps on the support
 * image; the reading notes (paper.gecl.asia, "Method") aggregate the support
 * features near each annotated point.
 *
 * For every (b, r) with kpt_valid[b,r] != 0:
 *   w(i,j)  = exp(-((cx_j - x)^2 + (cy_i - y)^2) / (2 sigma^2)),
 *             cx_j = (j + 1/2) stride_px, cy_i = (i + 1/2) stride_px
 *   protos[b,r,c] = sum_ij w(i,j) support[b,c,i,j] / sum_ij w(i,j)
 * over the whole H x W grid, rounded to `dtype` (bf16: nearest, ties to
 * even). Rows with kpt_valid == 0 are not written.
 *
 *   support    [B,C,H,W] dtype   support feature map (or, with
 *                                GKD_QUERY_TOKENS, [B, skip + H*W, C] tokens)
 *   kpts_px    [B,R,2]   float32 (x, y) in input pixels; the input spans
 *                                [0, W*stride_px) x [0, H*stride_px)
 *   kpt_valid  [B,R]     uint8   nonzero = row has a keypoint
 *   stride_px  > 0, finite (16 for a ViT/16 backbone)
 *   sigma_px   > 0, finite (14 in the model card)
 *   protos     [B,R,C]   dtype   output
 * Limits: C >= 1, H >= 1, W >= 1.
 */
GKD_API gkd_status gkd_vkp_pool(const void *support, const float *kpts_px,
                        const uint8_t *kpt_valid, int B, int C, int H, int W,
                        int R, float stride_px, float sigma_px,
                        gkd_dtype dtype, uint32_t flags, void *protos,
                        hipStream_t stream);

/*
 * Kernel heatmaps, with the peak decode optionally fused.
 * GKDT-L GGUF model card, section "Model": the parameter-free head upsamples
 * the features 4x bilinearly, L2-normalises the kernels, applies them as a
 * 1x1 convolution and fuses the prompts row by row under a mask, prompt rows
 * padded to 80; its "Output" bullet takes the per-prompt peak of each
 * 4H x 4W map as a -1..1 keypoint plus a score. The reading notes
 * (paper.gecl.asia, "Method") call this a normalised convolution of the
 * generated kernels with the query features.
 *
 * For every (b, r) with mask_vis[b,r] or mask_txt[b,r] set (n = number of
 * set masks), with u = up4(query[b]) the half-pixel bilinear 4x upsample
 * (or, with GKD_UPSAMPLE_CORNERS, the align_corners=True one):
 *   heatmaps[b,r,y,x] = (1/n) sum_{m set} sum_c k_m[b,r,c] u[c,y,x] / ||k_m[b,r]||
 * (||k|| is clamped below at 1e-12). Computed at low resolution and then
 * expanded, which is the same linear map. Rows with no mask set are not
 * written.
 *
 *   query      [B,C,H,W] dtype   query feature map (or, with GKD_QUERY_TOKENS,
 *                                [B, skip + H*W, C] tokens)
 *   kern_vis   [B,R,C]   dtype   visual kernels; mask_vis [B,R] uint8.
 *                                Both NULL = no visual prompt in the batch.
 *   kern_txt   [B,R,C]   dtype   text kernels; mask_txt [B,R] uint8.
 *                                Both NULL = no text prompt in the batch.
 *                                At least one modality must be given.
 *   heatmaps   [B,R,4H,4W] output: float32, or with flags = GKD_HEATMAP_BF16
 *                                bfloat16 (each value rounded to nearest even
 *                                from its float32 result). The fused decode
 *                                takes the peak and score from the float32
 *                                values in both formats.
 *                                heatmaps NULL = keypoints only: with the
 *                                decode outputs set, only they are computed
 *                                (no heatmap byte is written anywhere; on
 *                                bf16 features with H*W <= 576 the peak is
 *                                found in the contraction's epilogue).
 *   peak_idx   [B,R]   int32     optional fused decode (see gkd_peak_decode);
 *   peak_xy    [B,R,2] float32   all three NULL = no decode, else all three
 *   peak_score [B,R]   float32   non-NULL. Rows with no mask get the sentinel.
 *                                heatmaps and the decode outputs cannot all
 *                                be NULL (GKD_ERR_NULL). GKD_COORDS_CORNERS
 *                                selects the corner-aligned coordinates.
 * Limits: C >= 1, H >= 1, W >= 1, H*W <= 16384 (else GKD_ERR_UNSUPPORTED).
 */
GKD_API gkd_status gkd_kernel_heatmap(const void *query, const void *kern_vis,
                              const uint8_t *mask_vis, const void *kern_txt,
                              const uint8_t *mask_txt, int B, int C, int H,
                              int W, int R, gkd_dtype dtype, uint32_t flags,
                              void *heatmaps, int32_t *peak_idx,
                              float *peak_xy, float *peak_score,
                              hipStream_t stream);

/*
 * Peak decode.
 * GKDT-L GGUF model card, section "Model", "Output" bullet: each prompt's
 * heatmap peak becomes a keypoint in the crop's normalised -1..1 frame plus
 * a confidence score.
 *
 * For every (b, r) with row_valid[b,r] != 0 (or every row if row_valid is
 * NULL): p = the lowest flat index y*Wo + x holding the row's maximum;
 *   peak_idx   = p
 *   peak_xy    = ((2x + 1)/Wo - 1, (2y + 1)/Ho - 1)   (cell centres), or with
 *                flags = GKD_COORDS_CORNERS (2x/(Wo - 1) - 1, 2y/(Ho - 1) - 1)
 *   peak_score = heatmaps[b,r,y,x]
 * Invalid rows get idx -1, xy NaN, score -inf.
 *
 *   heatmaps   [B,R,Ho,Wo] float32
 *   row_valid  [B,R] uint8 or NULL
 *   peak_idx [B,R] int32, peak_xy [B,R,2] float32, peak_score [B,R] float32
 * Limits: Ho >= 1, Wo >= 1.
 */
GKD_API gkd_status gkd_peak_decode(const float *heatmaps, const uint8_t *row_valid,
                           int B, int R, int Ho, int Wo, uint32_t flags,
                           int32_t *peak_idx, float *peak_xy,
                           float *peak_score, hipStream_t stream);

/*
 * ROI preprocessing.
 * GKDT-L GGUF model card, section "Model", "Input" bullet: the image is
 * resized so that its longer side is the input size, centre-padded to a
 * square with the mean colour (124, 116, 104), and ImageNet-normalised;
 * in top-down use (GKDT paper summary, agihunt.info: keypoints per
 * detected object) each detector box is cropped first. Conventions the
 * card leaves open:
 *   - a box is an integer pixel rectangle (x0, y0, x1, y1), x1 and y1
 *     exclusive, clamped to the image; an empty box (after clamping) gives
 *     a canvas of pad colour;
 *   - the box's longer side becomes out_size, the shorter one
 *     round(side * out_size / longer), halves up, at least 1;
 *   - the resized crop sits at ((out_size - nw) / 2, (out_size - nh) / 2)
 *     (integer division: an odd pixel of pad goes right / bottom);
 *   - the resize is bilinear with half-pixel centres (source position
 *     (u + 1/2) bw / nw - 1/2, clamped below at 0; the upper tap clamps at
 *     the crop's last pixel), without antialiasing and without rounding
 *     back to 8 bits;
 *   - every canvas value v (pad included) becomes
 *     (v / 255 - mean_c) / std_c, mean (0.485, 0.456, 0.406),
 *     std (0.229, 0.224, 0.225), c = R, G, B.
 * The arithmetic is float32; taps and their fractions come from exact
 * integer ratios.
 *
 *   image     [height,width,3] uint8 RGB, 4-byte aligned
 *   boxes     [B,4] int32, 4-byte aligned (any values: they are clamped)
 *   out       [B,3,out_size,out_size] dtype (float32 or bfloat16, rounded
 *             to nearest even), 16-byte aligned
 * Limits: 1 <= height, width <= 65535; 1 <= out_size <= 4096;
 * B <= 65535 (else GKD_ERR_SHAPE).
 */
GKD_API gkd_status gkd_roi_preprocess(const uint8_t *image, int height, int width,
                              const int32_t *boxes, int B, int out_size,
                              gkd_dtype dtype, uint32_t flags, void *out,
                              hipStream_t stream);

/*
 * ROI back-projection.
 * GKDT-L GGUF model card, section "Model", "Output" bullet: keypoints come
 * out in the ROI's normalised -1..1 frame. This maps them to the image:
 *   x_img = x0 + ((x + 1) out_size / 2 - px) * bw / nw
 * and the same along y, with the box geometry of gkd_roi_preprocess; image
 * coordinates are continuous (pixel i covers [i, i + 1)). NaN inputs (the
 * decode's invalid rows) stay NaN; empty boxes give NaN.
 *
 *   xy        [B,R,2] float32, 4-byte aligned
 *   boxes     [B,4] int32, the boxes given to gkd_roi_preprocess
 *   out_xy    [B,R,2] float32, 4-byte aligned
 * Limits: as gkd_roi_preprocess.
 */
GKD_API gkd_status gkd_roi_backproject(const float *xy, const int32_t *boxes, int B,
                               int R, int height, int width, int out_size,
                               uint32_t flags, float *out_xy, hipStream_t stream);

/*
 * gkd_kg_transformer - the kernel-generation (KG) transformer that turns
 * the visual and text keypoint prototypes into the kernels of the head
 * (GKDT model card, "Architecture" bullet: 2 blocks of self- and
 * cross-attention, d_ff = 1024, a mask token; paper summary, four-step
 * pipeline). Readings: the sequence of a crop is its 2R slots [visual rows
 * 0..R-1, text rows 0..R-1]; a slot whose row lacks that prompt holds the
 * mask token; self-attention keys are the slots of rows with any prompt;
 * cross-attention keys and
 * values are the H*W query feature tokens; each block is post-norm,
 * x = LN1(x + SA(x)), x = LN2(x + CA(x, F)), x = LN3(x + W2 relu(W1 x + b1)
 * + b2), LayerNorm eps 1e-5; heads are 64 wide (C/64 heads), scores scaled
 * by 1/8.
 *
 *   kern_vis, kern_txt [B,R,C] bf16  prototypes (NULL with their mask NULL)
 *   mask_vis, mask_txt [B,R] u8      nonzero: the row has that prompt; at
 *                                    least one mask must be given
 *   query      [B,C,H,W] bf16        query features (or, with
 *                                    GKD_QUERY_TOKENS, [B, skip + H*W, C])
 *   weights    flat bf16             mask token [C]; then per block: SA
 *                                    in_proj W [3C,C], b [3C]; SA out_proj
 *                                    W [C,C], b [C]; LN1 w, b [C]; CA
 *                                    in_proj W [3C,C], b [3C]; CA out_proj
 *                                    W [C,C], b [C]; LN2 w, b; FFN W1
 *                                    [d_ff,C], b1 [d_ff], W2 [C,d_ff], b2
 *                                    [C]; LN3 w, b (torch Linear layout,
 *                                    y = x W^T + b)
 *   out        [2,B,R,C] bf16 (out)  kernels: out[0] from the visual slots,
 *                                    out[1] from the text slots (the head's
 *                                    kern_vis and kern_txt as they stand).
 *                                    Rows with no prompt in either modality
 *                                    are not written: they are no
 *                                    self-attention keys, so they change no
 *                                    other row, and the head reads no
 *                                    kernel of a masked row. Only the
 *                                    2 n_b slots of crop b's n_b prompted
 *                                    rows are computed.
 *   workspace  device memory of at least gkd_kg_workspace_size() bytes,
 *              256-byte aligned, owned by the caller; its contents on entry
 *              do not matter and are left undefined. Calls that share a
 *              workspace must not overlap.
 * dtype must be GKD_DTYPE_BF16 (matrix operands in bfloat16, accumulation,
 * softmax, LayerNorm and the residual stream in float32). Limits: C % 64
 * == 0, d_ff % 64 == 0, 1 <= n_blocks <= 64, 2R <= 576 (the
 * self-attention holds all scores of a row in registers; the
 * cross-attention streams the H*W keys, so H*W is limited only by the
 * element counts below), else GKD_ERR_UNSUPPORTED. All arrays but the masks 16-byte aligned (else
 * GKD_ERR_ALIGN); workspace_bytes too small gives GKD_ERR_VALUE. flags: 0
 * or GKD_QUERY_TOKENS | GKD_QUERY_SKIP(n).
 */
GKD_API size_t gkd_kg_workspace_size(int B, int C, int H, int W, int R, int d_ff,
                                     uint32_t flags);
GKD_API gkd_status gkd_kg_transformer(const void *kern_vis, const uint8_t *mask_vis,
                                      const void *kern_txt, const uint8_t *mask_txt,
                                      const void *query, int B, int C, int H, int W, int R,
                                      const void *weights, int n_blocks, int d_ff,
                                      gkd_dtype dtype, uint32_t flags, void *out,
                                      void *workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * gkd_kg_transformer_noalloc - gkd_kg_transformer for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. It takes no workspace argument:
 * the workspace is an array of GKD_KG_STATIC_WORKSPACE_BYTES inside the
 * library's device code, one per GPU, placed when the library is loaded
 * on that GPU and held until the process ends. The call allocates nothing
 * (no hipMalloc, no allocating library routine); its first call on a GPU
 * looks up that GPU's copy of the array (hipGetSymbolAddress), with the
 * current device being the one `stream` runs on.
 *   - Arguments, results and errors are those of gkd_kg_transformer,
 *     which this call equals bit for bit; a shape whose
 *     gkd_kg_workspace_size() exceeds GKD_KG_STATIC_WORKSPACE_BYTES is
 *     rejected with GKD_ERR_VALUE before anything is launched (at C = 1024,
 *     H = W = 24, R = 80, d_ff = 1024: up to 10 crops per call, 12 with
 *     GKD_QUERY_TOKENS).
 *   - All calls on one GPU share its array and nothing in it needs to
 *     start at zero; two calls that overlap in time on one GPU (different
 *     streams, or host threads without stream ordering) race on it and
 *     give undefined results.
 */
#define GKD_KG_STATIC_WORKSPACE_BYTES (64u << 20)
GKD_API gkd_status gkd_kg_transformer_noalloc(const void *kern_vis, const uint8_t *mask_vis,
                                              const void *kern_txt, const uint8_t *mask_txt,
                                              const void *query, int B, int C, int H, int W,
                                              int R, const void *weights, int n_blocks,
                                              int d_ff, gkd_dtype dtype, uint32_t flags,
                                              void *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GKDHEAD_H */
