// heatmap_stream.hip - gkd_kernel_heatmap for bf16 features: up to three
// launches on the caller's stream, each shaped for one side of the memory
// system.
//
// The head (GKDT-L GGUF model card, section "Model": rows padded to 80
// with masks, L2 kernel norm, 1x1 kernel conv against 4x bilinearly
// upsampled dense features, per-row fusion of the prompt modalities,
// argmax read out as a -1..1 keypoint plus score) is linear up to the
// argmax, so the contraction runs at the features' own resolution and only
// its result is expanded.
//
// 0. row_prep_kernel (only when both prompt modalities are passed): for the
//    rows of crops that hold both, the fusion weights and, by linearity of
//    the per-row fusion, the single combined kernel w_v k_v + w_t k_t, split
//    into bfloat16 hi and lo parts and parked in the row's own heatmap.
// 1. contract_kernel (HBM reads): one workgroup per (crop, pixel chunk)
//    takes ALL valid rows of the crop (up to 80 per item, both
//    modalities), so every feature byte crosses HBM and the CU exactly
//    once. Feature tiles [32 channels][chunk pixels] and the rows' kernel
//    slices stream straight into a three-slot LDS ring
//    (global_load_lds_dwordx4); MFMA B operands come from transposing LDS
//    reads (ds_read_b64_tr_b16), A operands from plain 16-byte LDS reads.
//    Items with few kernel rows load one step ahead, the rest two, which
//    evens out the items' finishing times under shared bandwidth.
//    The fused low-resolution map of a row (float32, H*W values) is parked
//    in the first H*W floats of that row's own heatmap.
// 2. expand_kernel (HBM writes): one wave per valid row reads its parked
//    map into LDS, writes the 4x bilinear expansion with 16-byte
//    non-temporal stores and reduces the first-occurrence argmax in
//    registers. Waves are independent (no workgroup barrier), so a CU
//    keeps many rows' stores in flight.
// Everything parked in a heatmap row is read back before the expand pass
// overwrites that row.
#include "gkd_device.hpp"
#include "launch.hpp"

#include <climits>
#include <cmath>

namespace gkd {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// ---------------------------------------------------------------------------
// row expansion
// ---------------------------------------------------------------------------
// The 16 outputs of low-res cell (i, j): rows 4i .. 4i+3, columns 4j ..
// 4j+3, raster order. Half-pixel 4x bilinear weights: each output lies
// 3/8 or 1/8 of a cell from its own cell centre toward a neighbour, so it
// is centre + w * (neighbour - centre); at a clamped border the neighbour is
// the cell itself and the output is the centre exactly.
__device__ __forceinline__ void cell_values(const float* P, int i, int j, int H, int W,
                                            float (&o)[16]) {
  const int im = i > 0 ? i - 1 : 0, ip = i < H - 1 ? i + 1 : i;
  const int jm = j > 0 ? j - 1 : 0, jp = j < W - 1 ? j + 1 : j;
  float h[3][4];
  const int rows[3] = {im, i, ip};
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const float* pr = P + rows[r] * W;
    const float a = pr[jm], c = pr[j], e = pr[jp];
    const float dl = a - c, dr = e - c;
    h[r][0] = fmaf(dl, 0.375f, c);
    h[r][1] = fmaf(dl, 0.125f, c);
    h[r][2] = fmaf(dr, 0.125f, c);
    h[r][3] = fmaf(dr, 0.375f, c);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float c = h[1][e], du = h[0][e] - c, dd = h[2][e] - c;
    o[0 + e] = fmaf(du, 0.375f, c);
    o[4 + e] = fmaf(du, 0.125f, c);
    o[8 + e] = fmaf(dd, 0.125f, c);
    o[12 + e] = fmaf(dd, 0.375f, c);
  }
}

__device__ __forceinline__ float max16(const float (&o)[16]) {
  float m01 = fmaxf(fmaxf(o[0], o[1]), fmaxf(o[2], o[3]));
  float m23 = fmaxf(fmaxf(o[4], o[5]), fmaxf(o[6], o[7]));
  float m45 = fmaxf(fmaxf(o[8], o[9]), fmaxf(o[10], o[11]));
  float m67 = fmaxf(fmaxf(o[12], o[13]), fmaxf(o[14], o[15]));
  return fmaxf(fmaxf(m01, m23), fmaxf(m45, m67));
}

// first raster position of value m among o[0..15]
__device__ __forceinline__ int first_of(const float (&o)[16], float m) {
  int sel = 15;
#pragma unroll
  for (int q = 14; q >= 0; --q) sel = (o[q] == m) ? q : sel;
  return sel;
}

struct RowGeom {
  int H, W, S, Ho, Wo;
  uint64_t magic_w;  // ceil(2^32 / W): c / W == (c * magic_w) >> 32 for c * W < 2^32
};

// One wave expands the low-res map P (row-major H x W, in LDS) of one row
// into out ([4H][4W]) with 16-byte non-temporal stores and leaves the
// row's first-occurrence argmax (value, flat index) in every lane.
// SMALLW (W <= 64): a lane's cells c, c + 64, ... lie on increasing cell
// rows, so every output of a later cell has a larger flat index than any
// output of an earlier one; the lane keeps (best value, its cell) with a
// strict > and finds the position inside the cell once, at the end.
// OUT: kOutF32 stores float32; kOutBf16 stores bfloat16 (each value
// rounded to nearest even from the float32 result; the peak is still taken
// on the float32 values); kOutNone stores nothing and only finds the peak,
// with the same arithmetic.
constexpr int kOutNone = 0, kOutF32 = 1, kOutBf16 = 2;
template <bool SMALLW, int OUT>
__device__ __forceinline__ void expand_row(const float* P, void* out_row, const RowGeom& g,
                                           int lane, bool decode, float& best_v, int& best_i) {
  float bv = -INFINITY;
  int bi = INT_MAX;  // SMALLW: best cell; otherwise best flat index
  for (int c = lane; c < g.S; c += kWave) {
    const int i = (int)(((uint64_t)(uint32_t)c * g.magic_w) >> 32), j = c - i * g.W;
    float o[16];
    cell_values(P, i, j, g.H, g.W, o);
    const size_t e0 = (size_t)(4 * i) * g.Wo + 4 * j;  // element of output (4i, 4j)
    if constexpr (OUT == kOutBf16) {
      uint16_t* dst = static_cast<uint16_t*>(out_row) + e0;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const u32x2 v = {
            __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[4 * d], o[4 * d + 1]}, bf16x2)),
            __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[4 * d + 2], o[4 * d + 3]}, bf16x2))};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(dst + (size_t)d * g.Wo));
      }
    } else if constexpr (OUT == kOutF32) {
      float* dst = static_cast<float*>(out_row) + e0;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        __builtin_nontemporal_store(f32x4{o[4 * d], o[4 * d + 1], o[4 * d + 2], o[4 * d + 3]},
                                    reinterpret_cast<f32x4*>(dst + (size_t)d * g.Wo));
    }
    const float m = max16(o);
    if (SMALLW) {
      if (m > bv) {
        bv = m;
        bi = c;
      }
    } else {
      const int q = first_of(o, m);
      const int flat = (4 * i + (q >> 2)) * g.Wo + 4 * j + (q & 3);
      if (better(m, flat, bv, bi)) {
        bv = m;
        bi = flat;
      }
    }
  }
  if (!decode) return;
  if (SMALLW && bi != INT_MAX) {
    const int c = bi;
    const int i = (int)(((uint64_t)(uint32_t)c * g.magic_w) >> 32), j = c - i * g.W;
    float o[16];
    cell_values(P, i, j, g.H, g.W, o);
    const int q = first_of(o, bv);
    bi = (4 * i + (q >> 2)) * g.Wo + 4 * j + (q & 3);
  }
  wave_argmax(bv, bi);
  best_v = bv;
  best_i = bi;
}

// One wave expands P (H x W in LDS) on the align_corners=True grid into
// out ([4H][4W], OUT as for expand_row) in raster order: lane l takes the
// 4-output chunks l, l + 64, ... of the map (one output row, columns
// 4x .. 4x + 3), so a lane's outputs ascend in flat index and a strict >
// keeps the first peak. Every output is the bilinear mix of the four
// source samples around its position (corner_taps).
template <int OUT>
__device__ __forceinline__ void expand_row_corners(const float* P, void* out_row, const RowGeom& g,
                                                   int lane, bool decode, float& best_v,
                                                   int& best_i) {
  float bv = -INFINITY;
  int bi = INT_MAX;
  const int nq = g.Ho * g.W;
  for (int q = lane; q < nq; q += kWave) {
    const int y = (int)(((uint64_t)(uint32_t)q * g.magic_w) >> 32), x4 = q - y * g.W;
    int i0, i1;
    float ly;
    corner_taps(y, g.H, i0, i1, ly);
    const float* p0 = P + i0 * g.W;
    const float* p1 = P + i1 * g.W;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int j0, j1;
      float lx;
      corner_taps(4 * x4 + e, g.W, j0, j1, lx);
      const float top = fmaf(lx, p0[j1] - p0[j0], p0[j0]);
      const float bot = fmaf(lx, p1[j1] - p1[j0], p1[j0]);
      o[e] = fmaf(ly, bot - top, top);
    }
    if constexpr (OUT == kOutBf16) {
      const u32x2 v = {
          __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[0], o[1]}, bf16x2)),
          __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[2], o[3]}, bf16x2))};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out_row)) + q);
    } else if constexpr (OUT == kOutF32) {
      __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]},
                                  reinterpret_cast<f32x4*>(static_cast<float*>(out_row)) + q);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (o[e] > bv) {
        bv = o[e];
        bi = 4 * q + e;
      }
  }
  if (!decode) return;
  wave_argmax(bv, bi);
  best_v = bv;
  best_i = bi;
}

// Wave64 maximum (every lane gets it): the argmax lane pattern on values
// alone.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The first-occurrence peak of the 4x expansion of P (one wave; the same
// result, bit for bit, as expand_row's scan) without evaluating every cell.
// Each expanded value is a convex combination of at most four low-res
// values of its cell's 3x3 neighbourhood, computed in two fma stages whose
// rounding adds at most about 4 ulp of M = max |P|. With L the peak of the
// cell holding the maximum of P (a value of the expansion, so a lower bound
// of its peak) and T = L - M * 2^-20, every output >= L, the peak and all
// its ties included, lies in the 3x3 neighbourhood of a "hot" cell, one
// with P >= T. The hot cells are listed in hl (kMaxHot ints of this wave's
// LDS) and only their neighbourhoods are evaluated, seven hot cells at a
// time (lane = 9 * slot + neighbour). No hot cell (a NaN in the bound),
// more than kMaxHot (flat maps) or maps beyond kPeakChunks * 64 cells fall
// back to the full scan. A lane holds its cells of P in registers.
constexpr int kMaxHot = 64, kPeakChunks = 9;
template <bool SMALLW>
__device__ __forceinline__ void row_peak(const float* P, int* hl, const RowGeom& g, int lane,
                                         float& best_v, int& best_i) {
  constexpr int kPerPass = kWave / 9;
  if (g.S > kPeakChunks * kWave) {
    expand_row<SMALLW, kOutNone>(P, nullptr, g, lane, true, best_v, best_i);
    return;
  }
  float v[kPeakChunks];
#pragma unroll
  for (int k = 0; k < kPeakChunks; ++k) v[k] = k * kWave + lane < g.S ? P[k * kWave + lane] : 0.f;
  float pv = -INFINITY, amax = 0.f;
  int pc = INT_MAX;
#pragma unroll
  for (int k = 0; k < kPeakChunks; ++k) {
    const bool in = k * kWave + lane < g.S;
    amax = in ? fmaxf(amax, fabsf(v[k])) : amax;
    if (in && v[k] > pv) {  // a lane's cells ascend: strict > keeps the first
      pv = v[k];
      pc = k * kWave + lane;
    }
  }
  wave_argmax(pv, pc);
  amax = wave_max(amax);
  float o[16];
  float T = __int_as_float(0x7fc00000);  // NaN: no cell is hot
  if (pc != INT_MAX) {
    const int i = (int)(((uint64_t)(uint32_t)pc * g.magic_w) >> 32), j = pc - i * g.W;
    cell_values(P, i, j, g.H, g.W, o);
    T = max16(o) - amax * 0x1p-20f;
  }
  int nhot = 0;
#pragma unroll
  for (int k = 0; k < kPeakChunks; ++k) {
    const bool h = k * kWave + lane < g.S && v[k] >= T;
    const uint64_t m = __ballot(h);
    const int rank = nhot + (int)__builtin_amdgcn_mbcnt_hi(
                                (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (h && rank < kMaxHot) hl[rank] = k * kWave + lane;
    nhot += __popcll(m);
  }
  if (nhot == 0 || nhot > kMaxHot) {
    expand_row<SMALLW, kOutNone>(P, nullptr, g, lane, true, best_v, best_i);
    return;
  }
  __builtin_amdgcn_wave_barrier();  // the list is the wave's own: in-order LDS
  float bv = -INFINITY;
  int bi = INT_MAX;
  const int slot = lane / 9, nb = lane - 9 * slot;
  const int di = nb / 3 - 1, dj = nb % 3 - 1;
  for (int k0 = 0; k0 < nhot; k0 += kPerPass) {
    if (slot < kPerPass && k0 + slot < nhot) {
      const int h = hl[k0 + slot];
      const int hi = (int)(((uint64_t)(uint32_t)h * g.magic_w) >> 32), hj = h - hi * g.W;
      int ni = hi + di, nj = hj + dj;  // clamped: a repeated cell repeats a candidate
      ni = ni < 0 ? 0 : (ni > g.H - 1 ? g.H - 1 : ni);
      nj = nj < 0 ? 0 : (nj > g.W - 1 ? g.W - 1 : nj);
      cell_values(P, ni, nj, g.H, g.W, o);
      const float m = max16(o);
      const int q = first_of(o, m);
      const int flat = (4 * ni + (q >> 2)) * g.Wo + 4 * nj + (q & 3);
      if (better(m, flat, bv, bi)) {
        bv = m;
        bi = flat;
      }
    }
  }
  wave_argmax(bv, bi);
  best_v = bv;
  best_i = bi;
}

// keypoint record of one row: flat index, -1..1 coordinates (cell centres
// or corner-aligned), raw score
__device__ __forceinline__ void write_keypoint(int32_t* idx, float* xy, float* score, size_t o,
                                               float bv, int bi, int Ho, int Wo, bool corners) {
  const int y = bi / Wo, x = bi - y * Wo;
  idx[o] = bi;
  xy[2 * o] = keypoint_coord(x, Wo, corners);
  xy[2 * o + 1] = keypoint_coord(y, Ho, corners);
  score[o] = bv;
}

// ---------------------------------------------------------------------------
// contraction
// ---------------------------------------------------------------------------
constexpr int kCWaves = 12;
constexpr int kCThreads = kCWaves * kWave;  // 768
constexpr int kKS = 32;                     // channels per K step (one MFMA K)
constexpr int kStages = 3;                  // feature ring slots (loads run two steps ahead)
constexpr int kLightArows = 32;             // items with at most this many kernel rows load one step ahead
constexpr int kGroupPx = 48;                // one wave unit: 3 N tiles of 16 pixels
constexpr int kItemRows = 80;               // valid rows per item
constexpr int kMaxMH = kItemRows / 16;      // M tiles per modality
constexpr int kMaxDma = 5;                  // direct-to-LDS loads per wave per stage
constexpr int kRowSlots = 9;                // kernel row in LDS: 8 x 16 B (two K steps) + 1 pad
constexpr int kPairSlots = 2;               // kernel-row ring: two slots of two K steps each
constexpr size_t kContractLds = 158 * 1024; // dynamic LDS of a contraction workgroup
// item modes: rows of one modality, or both modalities present, in which
// case each row's two kernels enter as one pre-weighted combination, formed
// either step by step in LDS (kComb) or once per row by the row pass, which
// parks it in the row's own heatmap (kPre)
constexpr int kVis = 1, kTxt = 2, kComb = 3, kPre = 4;

// Where the row pass parks the combined kernel of a row (bfloat16 hi part,
// then lo part, C values each) inside that row's heatmap: float offsets,
// 128-byte aligned, past the H*W floats of the parked low-res map. Both are
// 0 when a heatmap row (row_f floats: 16 H*W for float32 heatmaps, 8 H*W
// for bfloat16 ones) is too short to hold them.
struct CombLayout {
  int hi = 0, lo = 0;
};
CombLayout comb_layout(int C, int S, long long row_f) {
  CombLayout l;
  const long long half = ((long long)C / 2 + 31) / 32 * 32;  // C bf16 in floats, rounded up
  const long long hi = ((long long)S + 31) / 32 * 32;
  if (hi + 2 * half <= row_f) {
    l.hi = (int)hi;
    l.lo = (int)(hi + half);
  }
  return l;
}

struct ContractParams {
  const uint16_t* query;
  const uint16_t* kv;
  const uint8_t* mv;
  const uint16_t* kt;
  const uint8_t* mt;
  int B, C, H, W, R, S;
  int ng;        // wave N groups per chunk (divides 12)
  int chunk_px;  // ng * 48
  int nchunks, rblocks, items_per_crop, nsteps;
  int comb_hi, comb_lo;  // CombLayout of the rows of two-modality crops (0: none)
  int light_arows;       // items staging at most this many kernel rows load one step ahead
  float* heat;           // heatmap rows, viewed as floats (parking space); null: keypoints only
  size_t row_f;          // floats per heatmap row: 16 H*W (float32) or 8 H*W (bfloat16)
  const float* wsrc;     // fusion weights (w_v, w_t) of row r at wsrc + r * w_stride, for the
  size_t w_stride;       //   step-by-step combination
  // keypoints only (heat null): the decode runs in the epilogue; every
  // item then covers whole maps (one pixel chunk)
  int32_t* idx;
  float* xy;
  float* score;
  bool corners;          // corner-aligned keypoint coordinates
  bool up_corners;       // upsample on the align_corners=True grid
  int tok_T, tok_skip;   // query as tokens [B, tok_T, C], pixel s at token tok_skip + s
                         //   (tok_T == 0: [B, C, H, W])
  uint64_t magic_w;      // ceil(2^32 / W)
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 layout:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 7]. The count is an
// immediate, so a three-level branch tree over the bits of n picks one of
// eight waits (a switch compiles to a structurized chain several times as
// long, on the K loop's critical path).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  asm volatile(
      "s_bitcmp1_b32 %0, 2\n\t"
      "s_cbranch_scc1 .Lw1_%=\n\t"
      "s_bitcmp1_b32 %0, 1\n\t"
      "s_cbranch_scc1 .Lw01_%=\n\t"
      "s_bitcmp1_b32 %0, 0\n\t"
      "s_cbranch_scc1 .Lw001_%=\n\t"
      "s_waitcnt vmcnt(0)\n\t"
      "s_branch .Lwe_%=\n"
      ".Lw001_%=:\n\t"
      "s_waitcnt vmcnt(1)\n\t"
      "s_branch .Lwe_%=\n"
      ".Lw01_%=:\n\t"
      "s_bitcmp1_b32 %0, 0\n\t"
      "s_cbranch_scc1 .Lw011_%=\n\t"
      "s_waitcnt vmcnt(2)\n\t"
      "s_branch .Lwe_%=\n"
      ".Lw011_%=:\n\t"
      "s_waitcnt vmcnt(3)\n\t"
      "s_branch .Lwe_%=\n"
      ".Lw1_%=:\n\t"
      "s_bitcmp1_b32 %0, 1\n\t"
      "s_cbranch_scc1 .Lw11_%=\n\t"
      "s_bitcmp1_b32 %0, 0\n\t"
      "s_cbranch_scc1 .Lw101_%=\n\t"
      "s_waitcnt vmcnt(4)\n\t"
      "s_branch .Lwe_%=\n"
      ".Lw101_%=:\n\t"
      "s_waitcnt vmcnt(5)\n\t"
      "s_branch .Lwe_%=\n"
      ".Lw11_%=:\n\t"
      "s_bitcmp1_b32 %0, 0\n\t"
      "s_cbranch_scc1 .Lw111_%=\n\t"
      "s_waitcnt vmcnt(6)\n\t"
      "s_branch .Lwe_%=\n"
      ".Lw111_%=:\n\t"
      "s_waitcnt vmcnt(7)\n"
      ".Lwe_%=:"
      :
      : "s"(n)
      : "memory", "scc");
}

// Workgroup barrier without a memory fence (a fence would also drain the
// direct-to-LDS loads in flight). This wave's own LDS accesses are
// completed first; its direct-to-LDS loads are the caller's business.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Each K step stages [32 feature rows x chunk] in the feature ring and
// [the item's kernel rows x 32 channels] in the kernel-row ring, both as
// whole 1 KiB blocks (one load instruction: 64 lanes x 16 B, lane order).
// Feature block q goes to wave q % 12; kernel-row blocks continue the same
// round robin after the feature blocks, so no wave issues more than
// ceil(blocks / 12) loads per step. Per lane and instruction: the source
// address of step 0 (features) or of steps 0 and 1 (kernel rows); a step
// adds one wave-uniform byte offset. Slots that are never read (row pads,
// past the plan) load the crop's first feature bytes plus that offset,
// which stay inside the crop's feature map at every step, so every lane
// issues every load with no exec masking and no per-step address selection.
struct DmaPlan {
  uint64_t src[kMaxDma];  // per-lane source address of instruction i at step 0
  uint32_t second;        // bit i: this lane's slot holds the pair's second step
  int nf;                 // feature loads of this wave per step (instructions 0 .. nf-1)
  int na;                 // kernel-row loads per step (instructions nf .. nf+na-1)
  int qa0;                // first kernel-row block of this wave
};
struct DmaBases {
  const uint16_t* F;   // the crop's feature map (also the stand-in source)
  size_t fstep_bytes;  // feature bytes per K step: 64 S (channel rows) or 64 (tokens)
};

// cache policy of the feature loads: non-temporal (each feature byte is
// read once, so the stream should not displace what the next passes reuse
// from L2 and the memory-side cache). Token-layout loads keep the default
// policy: a step reads half of each pixel's 128-byte line and the next
// step the other half, which then comes from L2.
constexpr int kFeatureCpol = 2;

// feature blocks of one step into feature slot fs (TOK: token layout)
template <bool TOK>
__device__ __forceinline__ void issue_features(const DmaPlan& pl, const DmaBases& bs,
                                               unsigned char* fs, int wave, int step) {
  const uint64_t so = (uint64_t)step * bs.fstep_bytes;
#pragma unroll
  for (int i = 0; i < kMaxDma; ++i)
    if (i < pl.nf) {
      glb_void* src = (glb_void*)(pl.src[i] + so);
      lds_void* dst = (lds_void*)(fs + (size_t)(wave + kCWaves * i) * 1024);
      if constexpr (TOK)
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, kFeatureCpol);
    }
}

// kernel-row blocks of two K steps (step, step + 1; step even) into
// kernel-row slot as; `last` when step + 1 is past the end
__device__ __forceinline__ void issue_rows(const DmaPlan& pl, const DmaBases& bs,
                                           unsigned char* as, int step, bool last) {
  const uint64_t so = (uint64_t)step * (kKS * 2);
#pragma unroll
  for (int i = 0; i < kMaxDma; ++i)
    if (i >= pl.nf && i < pl.nf + pl.na) {
      uint64_t src = pl.src[i] + so;
      // in a one-step pair, a second-step column would run past the row:
      // the lane loads the stand-in instead
      if (last && ((pl.second >> i) & 1u)) src = (uint64_t)bs.F;
      __builtin_amdgcn_global_load_lds((glb_void*)src,
                                       (lds_void*)(as + (size_t)(pl.qa0 + kCWaves * (i - pl.nf)) * 1024),
                                       16, 0, 0);
    }
}

// Two channels of the combination w_v k_v + w_t k_t (bf16 pairs, the lower
// channel in the low half) split into a bfloat16 hi part and the bfloat16
// rounding of the remainder, each pair rounded to nearest even by one
// packed conversion. hi + lo carries about 16 significant bits.
__device__ __forceinline__ void combine_pair(uint32_t v, uint32_t t, float wv, float wt,
                                             uint32_t& hi, uint32_t& lo) {
  const f32x2 x = {fmaf(wt, __uint_as_float(t << 16), wv * __uint_as_float(v << 16)),
                   fmaf(wt, __uint_as_float(t & 0xffff0000u), wv * __uint_as_float(v & 0xffff0000u))};
  const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  const f32x2 r = {x[0] - __uint_as_float(hb << 16), x[1] - __uint_as_float(hb & 0xffff0000u)};
  hi = hb;
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}

struct ItemShape {
  int ng;      // wave N groups of the item's chunk
  int chunk_px;
  int rs;      // 16-byte slots per LDS feature row: chunk_px / 8 + 1 (one pad)
  int nsel;    // valid rows of the item
  int MH;      // M tiles per modality
  int nmod;    // modalities present (1 or 2)
  int arows;   // kernel rows staged per step: nmod * MH * 16
  int fbytes;  // feature slot (whole 1 KiB blocks)
  int abytes;  // kernel-row slot (whole 1 KiB blocks)
  int px0;     // first pixel of the chunk
  bool has_v;
  int ahead;   // K steps the loads run ahead: 2, or 1 for light items
};

// K loop, row norms and epilogue for one item. MODE: kVis / kTxt (one
// modality: the row norms are summed along the K loop and the fusion weight
// is applied to the finished sums), kComb (both modalities: each pair of
// steps' kernel-row slices is first replaced in LDS by the weighted combination
// w_v k_v + w_t k_t, as a bfloat16 hi part over the visual rows and a lo
// part over the text rows, so a row needs one accumulator and two MFMAs) or
// kPre (the same hi and lo parts, formed once by the row pass and staged
// directly).
// UPW: wave units (one M tile x one 48-pixel group) a wave may own.
template <int MODE, int UPW, bool TOK>
__device__ __forceinline__ void contract_item(const ContractParams& p, unsigned char* lds,
                                              const DmaPlan& pl, const DmaBases& bs,
                                              const ItemShape& it, int b, int wave, int lane,
                                              const int* s_rows, const uint8_t* s_mv,
                                              const uint8_t* s_mt, float (*s_w)[kItemRows]) {
  constexpr bool COMB = MODE == kComb;
  constexpr bool TWO = COMB || MODE == kPre;  // rows carry hi and lo parts, weights applied
  constexpr int NM = TWO ? 2 : 1;  // A operands per unit (hi + lo, or the one modality)
  const int tid = wave * kWave + lane;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int gw = wave % it.ng;           // this wave's pixel group
  const int h0 = wave / it.ng;           // first M tile
  const int hstep = kCWaves / it.ng;
  const int gpx = gw * kGroupPx;         // group start within the chunk
  const int row_bytes = it.rs * 16;
  const int arow0 = it.MH * 16;          // kernel rows per modality in LDS

  // masked rows: zero A (one modality); in kComb their weights are 0
  bool on[UPW];
#pragma unroll
  for (int u = 0; u < UPW; ++u) {
    const int slot = 16 * (h0 + u * hstep) + n16;
    on[u] = TWO || (slot < it.nsel && (MODE == kVis ? s_mv[slot] : s_mt[slot]));
  }
  f32x4 acc[UPW][3];
#pragma unroll
  for (int u = 0; u < UPW; ++u)
#pragma unroll
    for (int t = 0; t < 3; ++t) acc[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // row norms (one modality): thread 4 a + c sums the squares of 16-byte
  // column c of staged kernel row a, step by step
  const bool norm_thread = !TWO && tid < 4 * it.arows;
  const int nrow = tid >> 2, ncol = tid & 3;
  // combination (kComb): thread 8 a + c rewrites 16-byte column c (both
  // steps of a pair) of row slot a; its weights are read once step 0 (and
  // the weights' DMA before it) landed
  const bool comb_thread = COMB && tid < 8 * arow0;
  const int crow = tid >> 3, ccol = tid & 7;
  float wv = 0.f, wt = 0.f;
  float ss = 0.f;

  unsigned char* const aring = lds + (size_t)kStages * it.fbytes;
  const int ahead = it.ahead;  // loads run this many steps ahead
  for (int k = 0; k < p.nsteps; ++k) {
    {
      // step k (features, and with an even step the kernel rows of it and
      // the next) has landed for this wave once at most the loads of the
      // younger steps issued so far remain: every wave issues its loads in
      // step order, the prologue included, so those are step k + 1's
      // (ahead is 1 or 2: at most the next step's loads, <= kMaxDma)
      static_assert(kStages == 3 && kMaxDma <= 7, "one younger step of at most 7 loads");
      const int younger = ahead == 2 && k + 1 < p.nsteps ? pl.nf + ((k & 1) ? pl.na : 0) : 0;
      wait_vmcnt_dyn(younger);
    }
    lds_barrier();  // everyone's step k landed; the slots of step k-1 are free
    if constexpr (COMB) {
      if (k == 0 && comb_thread && crow < it.nsel) {
        wv = s_w[0][crow];
        wt = s_w[1][crow];
      }
    }
    // the loads of step k + ahead go to the slots step k - 1 used
    if (k + ahead < p.nsteps) {
      const int s = k + ahead;
      issue_features<TOK>(pl, bs, lds + (size_t)(s % kStages) * it.fbytes, wave, s);
      if ((s & 1) == 0)
        issue_rows(pl, bs, aring + (size_t)((s >> 1) % kPairSlots) * it.abytes, s, s + 1 == p.nsteps);
    }

    const int cur = k % kStages;
    const unsigned char* sb = lds + (size_t)cur * it.fbytes;
    // this step's half (16-byte slots 4 (k & 1) .. + 3) of its pair's rows
    unsigned char* const sp = aring + (size_t)((k >> 1) % kPairSlots) * it.abytes;
    unsigned char* const sa = sp + 64 * (k & 1);
    if constexpr (COMB) {
      // an even step combines the whole pair (its own half and the next
      // step's), so only every other step waits on a second barrier
      if ((k & 1) == 0) {
        if (comb_thread) {
          u32x4* pv = reinterpret_cast<u32x4*>(sp + crow * (kRowSlots * 16) + 16 * ccol);
          u32x4* pt = reinterpret_cast<u32x4*>(sp + (arow0 + crow) * (kRowSlots * 16) + 16 * ccol);
          const u32x4 v = *pv, t = *pt;
          u32x4 hi, lo;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            uint32_t h, l;
            combine_pair(v[d], t[d], wv, wt, h, l);
            hi[d] = h;
            lo[d] = l;
          }
          *pv = hi;
          *pt = lo;
        }
        lds_barrier();  // the combined rows are in place
      }
    }
    // B: lane (n16, g4) of N tile t receives channels 8 g4 .. 8 g4 + 7 of
    // pixel gpx + 16 t + n16. Tokens: 16 contiguous bytes of the pixel's
    // slot (64 bytes a pixel); channel rows: two transposing 8-byte reads
    // (rows 8 g4 + n16/4 and +4, columns 4 (n16 % 4) .. +3 of the tile)
    u32x4 bw[3];
    if constexpr (TOK) {
      const uint32_t addr = (uint32_t)(uintptr_t)(lds_void*)(sb + (gpx + n16) * 64 + 16 * g4);
      asm volatile(
          "ds_read_b128 %0, %3\n"
          "ds_read_b128 %1, %3 offset:1024\n"
          "ds_read_b128 %2, %3 offset:2048\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(bw[0]), "=&v"(bw[1]), "=&v"(bw[2])
          : "v"(addr)
          : "memory");
    } else {
      const int r0 = 8 * g4 + (n16 >> 2);
      const uint32_t lo_addr =
          (uint32_t)(uintptr_t)(lds_void*)(sb + r0 * row_bytes + (gpx + 4 * (n16 & 3)) * 2);
      const uint32_t hi_addr = lo_addr + 4 * row_bytes;
      u32x2 blo[3], bhi[3];
      asm volatile(
          "ds_read_b64_tr_b16 %0, %6\n"
          "ds_read_b64_tr_b16 %1, %6 offset:32\n"
          "ds_read_b64_tr_b16 %2, %6 offset:64\n"
          "ds_read_b64_tr_b16 %3, %7\n"
          "ds_read_b64_tr_b16 %4, %7 offset:32\n"
          "ds_read_b64_tr_b16 %5, %7 offset:64\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(blo[0]), "=&v"(blo[1]), "=&v"(blo[2]), "=&v"(bhi[0]), "=&v"(bhi[1]),
            "=&v"(bhi[2])
          : "v"(lo_addr), "v"(hi_addr)
          : "memory");
#pragma unroll
      for (int t = 0; t < 3; ++t) bw[t] = u32x4{blo[t].x, blo[t].y, bhi[t].x, bhi[t].y};
    }
    bf16x8 bv[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) bv[t] = __builtin_bit_cast(bf16x8, bw[t]);
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
      const int h = h0 + u * hstep;
      if (h >= it.MH) break;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int ar = m * arow0 + 16 * h + n16;
        const u32x4 v = *reinterpret_cast<const u32x4*>(sa + ar * (kRowSlots * 16) + 16 * g4);
        const bf16x8 a = __builtin_bit_cast(bf16x8, on[u] ? v : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
        for (int t = 0; t < 3; ++t)
          acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv[t], acc[u][t], 0, 0, 0);
      }
    }
    if (norm_thread) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(sa + nrow * (kRowSlots * 16) + 16 * ncol);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float lo = __uint_as_float(v[d] << 16), hi = __uint_as_float(v[d] & 0xffff0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
    }
  }
  // fusion weights mask / (n ||k||) from the norms (one modality: n = 1)
  if constexpr (!TWO) {
    ss += __shfl_xor(ss, 1, kWave);
    ss += __shfl_xor(ss, 2, kWave);
    if (norm_thread && ncol == 0 && nrow < it.nsel) {
      const bool on_row = MODE == kVis ? s_mv[nrow] : s_mt[nrow];
      s_w[0][nrow] = on_row ? 1.f / fmaxf(sqrtf(ss), 1e-12f) : 0.f;
    }
  }
  lds_barrier();  // the ring is free; the weights are visible

  if (p.heat == nullptr) {
    // keypoints only: the fused low-res maps go to the (now free) ring in
    // passes of whole rows, and each wave finds the peak of the 4x
    // expansion of its rows with the expand pass's arithmetic (row_peak:
    // only the neighbourhoods that can hold it), storing nothing but the
    // keypoint
    // (the ring's last kCWaves * kMaxHot ints hold the waves' hot-cell lists)
    float* Pl = reinterpret_cast<float*>(lds);
    constexpr size_t kHotBytes = (size_t)kCWaves * kMaxHot * sizeof(int);
    int* hl = reinterpret_cast<int*>(lds + kContractLds - kHotBytes) + wave * kMaxHot;
    // rows at a pitch of S + 4 floats: the four row groups of a store land
    // in different banks
    const size_t pitch = (size_t)p.S + 4;
    const int rows_per_pass = (int)((kContractLds - kHotBytes) / (pitch * 4));
    const RowGeom g{p.H, p.W, p.S, 4 * p.H, 4 * p.W, p.magic_w};
    for (int base = 0; base < it.nsel; base += rows_per_pass) {
#pragma unroll
      for (int u = 0; u < UPW; ++u) {
        const int h = h0 + u * hstep;
        if (h >= it.MH) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = 16 * h + 4 * g4 + i;
          if (slot < base || slot >= base + rows_per_pass || slot >= it.nsel) continue;
          const float w = TWO ? 1.f : s_w[0][slot];
          float* dst = Pl + (size_t)(slot - base) * pitch + gpx + n16;
#pragma unroll
          for (int t = 0; t < 3; ++t)
            if (gpx + 16 * t + n16 < p.S) dst[16 * t] = TWO ? acc[u][t][i] : w * acc[u][t][i];
        }
      }
      lds_barrier();
      const int nrows = min(rows_per_pass, it.nsel - base);
      for (int r = wave; r < nrows; r += kCWaves) {
        float bv;
        int bi;
        if (p.up_corners)
          expand_row_corners<kOutNone>(Pl + (size_t)r * pitch, nullptr, g, lane, true, bv, bi);
        else if (p.W <= kWave)
          row_peak<true>(Pl + (size_t)r * pitch, hl, g, lane, bv, bi);
        else
          row_peak<false>(Pl + (size_t)r * pitch, hl, g, lane, bv, bi);
        if (lane == 0)
          write_keypoint(p.idx, p.xy, p.score, (size_t)b * p.R + s_rows[base + r], bv, bi, g.Ho,
                         g.Wo, p.corners);
      }
      lds_barrier();
    }
    return;
  }
  // fused low-res maps -> the first H*W floats of each row's heatmap,
  // straight from the accumulators: lane (n16, g4) holds rows 4 g4 + i of
  // each M tile at pixel 16 t + n16, so 16 lanes store 64 contiguous bytes
  // (no LDS staging and no barriers: an 80-row item's write-back no longer
  // waits on passes through the LDS, which held at most 69 rows at a time)
  const size_t hw_out = p.row_f;
#pragma unroll
  for (int u = 0; u < UPW; ++u) {
    const int h = h0 + u * hstep;
    if (h >= it.MH) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = 16 * h + 4 * g4 + i;
      if (slot >= it.nsel) continue;
      const float w = TWO ? 1.f : s_w[0][slot];
      float* dst = p.heat + ((size_t)b * p.R + s_rows[slot]) * hw_out + it.px0 + gpx + n16;
#pragma unroll
      for (int t = 0; t < 3; ++t)
        if (it.px0 + gpx + 16 * t + n16 < p.S) dst[16 * t] = TWO ? acc[u][t][i] : w * acc[u][t][i];
    }
  }
}

template <int MODE, int MAXU, bool TOK>
__device__ __forceinline__ void contract_dispatch(int upw, const ContractParams& p,
                                                  unsigned char* lds, const DmaPlan& pl,
                                                  const DmaBases& bs, const ItemShape& it, int b,
                                                  int wave, int lane, const int* s_rows,
                                                  const uint8_t* s_mv, const uint8_t* s_mt,
                                                  float (*s_w)[kItemRows]) {
#define GKD_CONTRACT(U) \
  contract_item<MODE, (U < MAXU ? U : MAXU), TOK>(p, lds, pl, bs, it, b, wave, lane, s_rows, s_mv, \
                                             s_mt, s_w)
  switch (upw) {
    case 1: GKD_CONTRACT(1); break;
    case 2: GKD_CONTRACT(2); break;
    case 3: GKD_CONTRACT(3); break;
    case 4: GKD_CONTRACT(4); break;
    default: GKD_CONTRACT(5); break;
  }
#undef GKD_CONTRACT
}

template <bool TOK>
__global__ __launch_bounds__(kCThreads) void contract_kernel(ContractParams p) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int s_rows[kItemRows];
  __shared__ uint8_t s_mv[kItemRows], s_mt[kItemRows];
  __shared__ int s_nvalid, s_nsel;
  __shared__ float s_w[2][kItemRows];  // fusion weights: mask / (n ||k||)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const ItemCoord ic = xcd_item(blockIdx.x, p.items_per_crop);
  const int b = ic.crop;
  if (b >= p.B) return;
  const int chunk = ic.item % p.nchunks, rblk = ic.item / p.nchunks;
  const uint8_t* mv = p.mv ? p.mv + (size_t)b * p.R : nullptr;
  const uint8_t* mt = p.mt ? p.mt + (size_t)b * p.R : nullptr;

  // a lane id the compiler cannot see through keeps the lane-dependent
  // set-up below from being hoisted and held across the K loop
  int lane_p = lane;
  asm volatile("" : "+v"(lane_p));
  constexpr bool tok = TOK;
  ItemShape it;
  it.ng = p.ng;
  it.chunk_px = it.ng * kGroupPx;
  it.rs = it.chunk_px / 8 + 1;
  it.px0 = chunk * p.chunk_px;
  // feature slots of a step: 32 channel rows of rs 16-byte columns, or with
  // tokens 4 16-byte pieces (32 channels) per pixel, pixel-major
  const int nF = tok ? 4 * it.chunk_px : kKS * it.rs;
  const int nfi = (nF + kWave - 1) / kWave;     // feature blocks
  it.fbytes = nfi * 1024;

  DmaBases bs;
  bs.F = tok ? p.query + ((size_t)b * p.tok_T + p.tok_skip) * p.C : p.query + (size_t)b * p.C * p.S;
  bs.fstep_bytes = tok ? (size_t)kKS * 2 : (size_t)kKS * p.S * 2;
  const uint64_t stand_in = (uint64_t)bs.F;

  // ---- DMA plan, feature part. Feature slot u < nF: feature row r = u /
  // rs (channel), 16-byte column u % rs (the last one pads the row); past
  // the map: the row's start. Pad slots and slots past the plan are never
  // read and load the stand-in. The feature prologue needs no row
  // information, so it is in flight while the item's rows are selected.
  DmaPlan pl;
  pl.nf = wave < nfi ? (nfi - wave + kCWaves - 1) / kCWaves : 0;
  pl.second = 0;
#pragma unroll
  for (int i = 0; i < kMaxDma; ++i) {
    pl.src[i] = stand_in;
    if (i >= pl.nf) continue;  // the kernel-row part fills its own below
    const int u = (wave + kCWaves * i) * kWave + lane_p;
    if (u < nF && tok) {
      // pixel px0 + u / 4, channels 8 (u % 4) .. + 7 of the step; past the
      // map: the stand-in (the pixels are never read)
      const int px = it.px0 + (u >> 2);
      if (px < p.S)
        pl.src[i] = stand_in + 2ull * ((uint32_t)px * (uint32_t)p.C + 8u * (uint32_t)(u & 3));
    } else if (u < nF) {
      const int r = u / it.rs, cc = u - r * it.rs;
      const int px = it.px0 + 8 * cc;
      if (cc < it.rs - 1) pl.src[i] = stand_in + 2ull * (uint32_t)(r * p.S + (px < p.S ? px : 0));
    }
  }
  issue_features<TOK>(pl, bs, lds, wave, 0);

  if (wave == 0)
    select_rows(mv, mt, p.R, lane, rblk, kItemRows, s_rows, s_mv, s_mt, &s_nvalid, &s_nsel);
  // keypoints only: the crop's first item writes the sentinels of its rows
  // with no mask set (the weights parked in peak_xy belong to valid rows)
  if (p.heat == nullptr && rblk == 0 && wave == kCWaves - 1) {
    for (int r = lane; r < p.R; r += kWave) {
      if (!((mv && mv[r]) || (mt && mt[r]))) {
        const size_t o = (size_t)b * p.R + r;
        p.idx[o] = -1;
        p.xy[2 * o] = __builtin_nanf("");
        p.xy[2 * o + 1] = __builtin_nanf("");
        p.score[o] = -INFINITY;
      }
    }
  }
  __syncthreads();
  it.nsel = s_nsel;
  if (it.nsel == 0) {
    wait_vmcnt<0>();  // the feature prologue lands before the LDS is released
    return;
  }
  // modalities present and the first slot of each: every wave scans the
  // item's slots (at most 80) with two ballots rather than a serial loop
  static_assert(kItemRows <= 2 * kWave, "two ballots cover an item");
  const uint64_t bv0 = __ballot(lane < it.nsel && s_mv[lane]);
  const uint64_t bt0 = __ballot(lane < it.nsel && s_mt[lane]);
  const uint64_t bv1 = __ballot(kWave + lane < it.nsel && s_mv[kWave + lane]);
  const uint64_t bt1 = __ballot(kWave + lane < it.nsel && s_mt[kWave + lane]);
  const bool has_v = (bv0 | bv1) != 0, has_t = (bt0 | bt1) != 0;
  const int first_v = bv0 ? __builtin_ctzll(bv0) : (bv1 ? kWave + __builtin_ctzll(bv1) : 0);
  const int first_t = bt0 ? __builtin_ctzll(bt0) : (bt1 ? kWave + __builtin_ctzll(bt1) : 0);
  it.has_v = has_v;
  it.MH = (it.nsel + 15) / 16;
  it.nmod = (int)has_v + (int)has_t;
  it.arows = it.nmod * it.MH * 16;
  // both modalities: the row pass either parked each row's combined kernel
  // in the row's heatmap (kPre) or parked the fusion weights w = 1 / (n
  // ||k||) there, just past the H*W floats this kernel writes. The weights
  // go straight to LDS ahead of the kernel-row prologue (entry 64 j + lane
  // of s_w from wave j), so the K loop's wait for step 0 covers them; slots
  // past nsel are never read.
  const bool comb = has_v && has_t;
  const bool pre = comb && p.comb_hi > 0;
  if (comb && !pre && wave * kWave < 2 * kItemRows) {
    const int e = wave * kWave + lane;
    const int wm = e / kItemRows, wslot = e - wm * kItemRows;
    if (e < 2 * kItemRows && wslot < it.nsel)
      __builtin_amdgcn_global_load_lds(
          (glb_void*)(p.wsrc + ((size_t)b * p.R + s_rows[wslot]) * p.w_stride + wm),
          (lds_void*)(&s_w[0][0] + wave * kWave), 4, 0, 0);
  }
  const int nA = it.arows * kRowSlots;          // kernel-row slots of a step pair
  const int nai = (nA + kWave - 1) / kWave;     // kernel-row blocks
  it.abytes = nai * 1024;

  // kernel rows: the prompt kernels (row pitch C), or the hi and lo parts
  // parked in the crop's heatmap rows (row pitch 2 row_f bf16 values)
  const uint16_t* const crop_heat =
      reinterpret_cast<const uint16_t*>(p.heat + (size_t)b * p.R * p.row_f);
  const uint16_t* const rows_v = pre ? crop_heat + 2 * (size_t)p.comb_hi
                                     : (has_v ? p.kv + (size_t)b * p.R * p.C : bs.F);
  const uint16_t* const rows_t = pre ? crop_heat + 2 * (size_t)p.comb_lo
                                     : (has_t ? p.kt + (size_t)b * p.R * p.C : bs.F);
  const uint32_t rpitch = pre ? 2u * (uint32_t)p.row_f : (uint32_t)p.C;

  // ---- DMA plan, kernel-row part. Kernel-row slot v < nA: kernel row
  // (modality index, slot) = v / 9, 16-byte column v % 9 of the step pair
  // (the ninth pads: a row's 64 channels of two steps are one 128-byte
  // line); masked or empty slots load the modality's first valid row
  // (finite) and are zeroed before the MFMA, or weighted by 0 in the
  // combination (kPre: every slot below nsel holds a combination; empty ones
  // load slot 0). Kernel-row blocks continue the feature blocks' round robin.
  pl.qa0 = (wave - nfi % kCWaves + kCWaves) % kCWaves;
  pl.na = pl.qa0 < nai ? (nai - pl.qa0 + kCWaves - 1) / kCWaves : 0;
#pragma unroll
  for (int i = 0; i < kMaxDma; ++i) {
    if (i < pl.nf || i >= pl.nf + pl.na) continue;
    const int v = (pl.qa0 + kCWaves * (i - pl.nf)) * kWave + lane_p;
    if (v < nA && v % kRowSlots < kRowSlots - 1) {
      const int ar = v / kRowSlots, ac = v - ar * kRowSlots;
      const int mi = ar / (it.MH * 16), slot = ar - mi * (it.MH * 16);
      const bool vis = has_v && mi == 0;
      const bool on = slot < it.nsel && (pre || (vis ? s_mv[slot] : s_mt[slot]));
      const int use = on ? slot : (pre ? 0 : (vis ? first_v : first_t));
      pl.src[i] = (uint64_t)(vis ? rows_v : rows_t) +
                  2ull * ((uint32_t)s_rows[use] * rpitch + 8 * ac);
      // a last pair with one step: the second step's columns are not read
      // (they would run past the row)
      if (ac >= 4) pl.second |= 1u << i;
    }
  }
  // the rest of the prologue: the kernel rows of steps 0 and 1, then the
  // features of step 1 (items that load two steps ahead), so step 0 waits
  // only for its own loads and is not queued behind step 1's. Items with
  // few kernel rows move fewer bytes per step; loading them only one step
  // ahead leaves the heavier items of the batch a larger share of the
  // memory bandwidth, so all items finish closer together.
  it.ahead = it.arows <= p.light_arows ? 1 : kStages - 1;
  unsigned char* const aring = lds + (size_t)kStages * it.fbytes;
  issue_rows(pl, bs, aring, 0, p.nsteps == 1);
  if (it.ahead > 1 && p.nsteps > 1) issue_features<TOK>(pl, bs, lds + (size_t)it.fbytes, wave, 1);

  const int upw = (it.MH * it.ng + kCWaves - 1) / kCWaves;
  if (pre)
    contract_dispatch<kPre, kMaxMH, TOK>(upw, p, lds, pl, bs, it, b, wave, lane_p, s_rows, s_mv, s_mt,
                                    s_w);
  else if (comb)
    contract_dispatch<kComb, kMaxMH, TOK>(upw, p, lds, pl, bs, it, b, wave, lane_p, s_rows, s_mv, s_mt,
                                     s_w);
  else if (has_v)
    contract_dispatch<kVis, kMaxMH, TOK>(upw, p, lds, pl, bs, it, b, wave, lane_p, s_rows, s_mv, s_mt,
                                    s_w);
  else
    contract_dispatch<kTxt, kMaxMH, TOK>(upw, p, lds, pl, bs, it, b, wave, lane_p, s_rows, s_mv, s_mt,
                                    s_w);
}

// ---------------------------------------------------------------------------
// row pass for the contraction's two-modality items
// ---------------------------------------------------------------------------
// One wave per (crop, row). In a crop that holds both modalities, every
// valid row gets its two fusion weights w_m = mask_m / (n ||k_m||)
// (||k|| clamped below at 1e-12, n = number of set masks) and, where its
// heatmap row has room (CombLayout), the combination w_v k_v + w_t k_t as
// bfloat16 hi and lo parts, parked there; otherwise the two weights are
// parked at floats H*W and H*W + 1 for the contraction to combine step by
// step. Either way the data lies past the low-res map that the contraction
// parks in the row, and the expand pass overwrites it.
constexpr int kPWaves = 4;

struct PrepParams {
  const uint16_t* kv;
  const uint8_t* mv;
  const uint16_t* kt;
  const uint8_t* mt;
  int B, C, R, S;
  int groups_per_crop;  // ceil(R / kPWaves)
  int comb_hi, comb_lo; // CombLayout (0: park the weights)
  float* heat;
  size_t row_f;         // floats per heatmap row
  float* wout;          // parked fusion weights of row r: wout + r * w_stride (+0 v, +1 t)
  size_t w_stride;
};

__device__ __forceinline__ float sum_squares8(u32x4 x) {
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float lo = __uint_as_float(x[d] << 16), hi = __uint_as_float(x[d] & 0xffff0000u);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}

__global__ __launch_bounds__(kPWaves * kWave) void row_prep_kernel(PrepParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x / p.groups_per_crop;
  const int r = (blockIdx.x - b * p.groups_per_crop) * kPWaves + wave;
  if (b >= p.B || r >= p.R) return;
  const uint8_t* mv = p.mv + (size_t)b * p.R;
  const uint8_t* mt = p.mt + (size_t)b * p.R;
  // one pass over the crop's masks gives both the crop scan and this row's
  // own masks; blocks of 4 x 64 rows with clamped indices, so every load of
  // a block is requested before the first wait
  uint32_t av = 0, at = 0, vr = 0, tr = 0;
  for (int base = 0; base < p.R; base += 4 * kWave) {
    uint32_t x[4], y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = min(base + i * kWave + lane, p.R - 1);
      x[i] = mv[q];
      y[i] = mt[q];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av |= x[i];
      at |= y[i];
      if (base + i * kWave + lane == r) {
        vr = x[i];
        tr = y[i];
      }
    }
  }
  const bool v = __ballot(vr != 0) != 0, t = __ballot(tr != 0) != 0;
  if (__ballot(av != 0) == 0 || __ballot(at != 0) == 0) return;
  if (!v && !t) return;
  const size_t row = ((size_t)b * p.R + r) * p.C;
  const uint16_t* kvr = p.kv + row;
  const uint16_t* ktr = p.kt + row;
  // the row's kernels in blocks of 512 channels (8 per lane); the first two
  // blocks are requested together and stay in registers for the
  // combination, the rest (C > 1024) are read again from cache
  auto load8 = [&](const uint16_t* k, bool on, int c) -> u32x4 {
    return (on && c < p.C) ? *reinterpret_cast<const u32x4*>(k + c) : u32x4{0u, 0u, 0u, 0u};
  };
  u32x4 a[2], e[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a[i] = load8(kvr, v, 8 * (i * kWave + lane));
    e[i] = load8(ktr, t, 8 * (i * kWave + lane));
  }
  float ssv = sum_squares8(a[0]) + sum_squares8(a[1]);
  float sst = sum_squares8(e[0]) + sum_squares8(e[1]);
  for (int c = 8 * (2 * kWave + lane); c < p.C; c += 8 * kWave) {
    ssv += sum_squares8(load8(kvr, v, c));
    sst += sum_squares8(load8(ktr, t, c));
  }
  ssv = wave_sum(ssv);
  sst = wave_sum(sst);
  const float n = (float)((int)v + (int)t);
  const float wv = v ? 1.f / (fmaxf(sqrtf(ssv), 1e-12f) * n) : 0.f;
  const float wt = t ? 1.f / (fmaxf(sqrtf(sst), 1e-12f) * n) : 0.f;
  if (p.comb_hi == 0) {
    if (lane == 0) {
      float* wd = p.wout + ((size_t)b * p.R + r) * p.w_stride;
      wd[0] = wv;
      wd[1] = wt;
    }
    return;
  }
  float* h = p.heat + ((size_t)b * p.R + r) * p.row_f;
  // the combination, 8 channels per lane and block; an absent modality
  // enters as zeros
  uint16_t* const hr = reinterpret_cast<uint16_t*>(h + p.comb_hi);
  uint16_t* const lr = reinterpret_cast<uint16_t*>(h + p.comb_lo);
  auto store8 = [&](u32x4 x, u32x4 y, int c) {
    u32x4 hi, lo;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t hd, ld;
      combine_pair(x[d], y[d], wv, wt, hd, ld);
      hi[d] = hd;
      lo[d] = ld;
    }
    // non-temporal: the parts go out to memory now instead of staying dirty
    // in L2 until the contraction's feature stream evicts them
    __builtin_nontemporal_store(hi, reinterpret_cast<u32x4*>(hr + c));
    __builtin_nontemporal_store(lo, reinterpret_cast<u32x4*>(lr + c));
  };
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = 8 * (i * kWave + lane);
    if (c < p.C) store8(a[i], e[i], c);
  }
  for (int c = 8 * (2 * kWave + lane); c < p.C; c += 8 * kWave)
    store8(load8(kvr, v, c), load8(ktr, t, c), c);
}

// ---------------------------------------------------------------------------
// expand + decode
// ---------------------------------------------------------------------------
constexpr int kEWaves = 4;
constexpr int kEThreads = kEWaves * kWave;
// A batch with many rows caps the expand workgroups resident on a CU by
// their LDS request (a CU holds 160 KiB). Each heatmap row is written by one
// wave, and fewer rows in flight at once store faster: three workgroups
// (twelve waves) a CU for rows up to 24 KB (96x96 bfloat16 maps), two for
// rows up to 96 KB, one for larger rows (the 192x192 float32 maps). A small
// batch keeps every row in flight.
constexpr long long kExpandCapRows = 8192;    // B * R from which the residency is capped
constexpr size_t kExpandLds3 = 52 * 1024;     // three workgroups fit a CU, four do not
constexpr size_t kExpandLds2 = 64 * 1024;     // two fit, three do not
constexpr size_t kExpandLds1 = 96 * 1024;     // one
constexpr size_t kExpandSmallRow = 24 * 1024; // heatmap row bytes up to which three are resident
constexpr size_t kExpandBigRow = 96 * 1024;   // row bytes above which one is

struct ExpandParams {
  const uint8_t* mv;
  const uint8_t* mt;
  int B, H, W, R, S, Ho, Wo;
  int wpg;               // rows (waves) per workgroup
  int groups_per_crop;   // ceil(R / wpg)
  uint64_t magic_w;      // ceil(2^32 / W)
  float* heat;           // heatmap rows viewed as floats (the parked maps)
  size_t row_f;          // floats per heatmap row
  int32_t* idx;
  float* xy;
  float* score;
  bool corners;          // corner-aligned keypoint coordinates
};

// One wave per valid row of the crop (by rank).
template <bool SMALLW, bool BF16, bool UPC>
__global__ __launch_bounds__(kEThreads) void expand_kernel(ExpandParams p) {
  extern __shared__ __align__(16) float lds_p[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const ItemCoord ic = xcd_item(blockIdx.x, p.groups_per_crop);
  const int b = ic.crop;
  if (b >= p.B || wave >= p.wpg) return;
  const uint8_t* mv = p.mv ? p.mv + (size_t)b * p.R : nullptr;
  const uint8_t* mt = p.mt ? p.mt + (size_t)b * p.R : nullptr;

  if (ic.item == 0 && wave == 0 && p.idx) {
    for (int r = lane; r < p.R; r += kWave) {
      if (!((mv && mv[r]) || (mt && mt[r]))) {
        const size_t o = (size_t)b * p.R + r;
        p.idx[o] = -1;
        p.xy[2 * o] = __builtin_nanf("");
        p.xy[2 * o + 1] = __builtin_nanf("");
        p.score[o] = -INFINITY;
      }
    }
  }

  // this wave's row: the rank-th valid row of the crop. The masks of two
  // 64-row chunks are requested together (clamped indices, so every load is
  // in bounds and in flight before the first ballot).
  int rank = ic.item * p.wpg + wave;
  int row = -1;
  for (int base = 0; base < p.R && row < 0; base += 2 * kWave) {
    uint8_t x[2], y[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = min(base + h * kWave + lane, p.R - 1);
      x[h] = mv ? mv[q] : 0;
      y[h] = mt ? mt[q] : 0;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c0 = base + h * kWave;
      const bool v = c0 + lane < p.R && (x[h] | y[h]);
      const uint64_t bal = __ballot(v);
      const int cnt = __popcll(bal);
      if (row < 0) {
        if (rank < cnt) {
          const int below = __popcll(bal & ((1ull << lane) - 1ull));
          const uint64_t hit = __ballot(v && below == rank);
          row = c0 + __builtin_ctzll(hit);
        } else {
          rank -= cnt;
        }
      }
    }
  }
  if (row < 0) return;

  float* out = p.heat + ((size_t)b * p.R + row) * p.row_f;
  float* P = lds_p + (size_t)wave * p.S;
  // the parked low-res map -> LDS (this wave only), four 16-byte loads per
  // lane in flight at a time; every load has returned before the first
  // store below can overwrite it
  const int nv = p.S / 4;
  for (int v0 = 0; v0 < nv; v0 += 4 * kWave) {
    f32x4 t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      t[i] = reinterpret_cast<const f32x4*>(out)[min(v0 + i * kWave + lane, nv - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (v0 + i * kWave + lane < nv) reinterpret_cast<f32x4*>(P)[v0 + i * kWave + lane] = t[i];
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

  const RowGeom g{p.H, p.W, p.S, p.Ho, p.Wo, p.magic_w};
  float bv;
  int bi;
  if constexpr (UPC)
    expand_row_corners<BF16 ? kOutBf16 : kOutF32>(P, out, g, lane, p.idx != nullptr, bv, bi);
  else
    expand_row<SMALLW, BF16 ? kOutBf16 : kOutF32>(P, out, g, lane, p.idx != nullptr, bv, bi);
  if (p.idx && lane == 0) write_keypoint(p.idx, p.xy, p.score, (size_t)b * p.R + row, bv, bi, p.Ho, p.Wo,
                                     p.corners);
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

bool heatmap_stream_applicable(int C, int S, bool bf16, bool keypoints_only) {
  // keypoints only: one workgroup's 12 wave groups must cover the whole map
  return bf16 && C % kKS == 0 && S % 16 == 0 && S <= kHeatmapMaxS &&
         (!keypoints_only || S <= kCWaves * kGroupPx);
}

StreamPlan plan_heatmap_stream(int B, int C, int S, int R, bool whole_maps, bool tokens) {
  StreamPlan sp;
  // wave groups per chunk: the fewest that still cover a small map in one
  // chunk, then fewer still while the batch leaves CUs idle (not when every
  // item must cover whole maps)
  static const int kNgSteps[] = {12, 6, 4, 3, 2, 1};
  int k = 0;
  while (k + 1 < 6 && kNgSteps[k + 1] * kGroupPx >= S) ++k;
  const int rblocks = ceil_div(R, kItemRows);
  while (!whole_maps && k + 1 < 6 &&
         (long long)B * ceil_div(S, kNgSteps[k] * kGroupPx) * rblocks < 240)
    ++k;
  sp.ng = kNgSteps[k];
  sp.chunk_px = sp.ng * kGroupPx;
  sp.nchunks = ceil_div(S, sp.chunk_px);
  sp.rblocks = rblocks;
  // LDS of an item: three feature slots and two kernel-row pair slots
  int max_instr = 0;
  size_t max_lds = 0;
  auto need = [&](int chunk_px, int arows) {
    const int nfi = ceil_div(tokens ? 4 * chunk_px : kKS * (chunk_px / 8 + 1), kWave);
    const int nai = ceil_div(arows * kRowSlots, kWave);
    if (nfi + nai > max_instr) max_instr = nfi + nai;
    const size_t lds = (size_t)(kStages * nfi + kPairSlots * nai) * 1024;
    if (lds > max_lds) max_lds = lds;
  };
  need(sp.chunk_px, 2 * kItemRows);
  need(sp.chunk_px, kItemRows);
  // one workgroup per CU whatever its LDS (registers decide that), so an
  // item may deepen its ring into the whole budget
  sp.contract_lds = max_lds <= kContractLds ? kContractLds : max_lds;
  sp.wpg = S <= 4096 ? kEWaves : 1;
  sp.expand_lds = (size_t)sp.wpg * S * sizeof(float);
  sp.ok = ceil_div(max_instr, kCWaves) <= kMaxDma && sp.contract_lds <= kContractLds &&
          sp.expand_lds <= 64 * 1024 && (!whole_maps || sp.nchunks == 1);
  return sp;
}

hipError_t launch_heatmap_stream(const HeatmapArgs& a, hipStream_t stream) {
  const int S = a.H * a.W;
  const bool kp = a.heat == nullptr;  // keypoints only
  const StreamPlan sp = plan_heatmap_stream(a.B, a.C, S, a.R, kp, a.tokens);
  if (!sp.ok) return hipErrorInvalidConfiguration;
  const long long crops_pad = (long long)(a.B + kXcds - 1) / kXcds * kXcds;
  float* const heat = static_cast<float*>(a.heat);
  const size_t row_f = kp ? 0 : (size_t)(a.heat_bf16 ? 8 : 16) * S;  // floats per heatmap row
  // no heatmap rows: the two-prompt rows combine step by step, with their
  // fusion weights parked in peak_xy (two floats per row, overwritten by
  // the decode)
  const CombLayout cl = kp ? CombLayout{} : comb_layout(a.C, S, (long long)row_f);
  float* const wpark = kp ? a.xy : heat + S;
  const size_t wstride = kp ? 2 : row_f;

  if (a.kv != nullptr && a.kt != nullptr) {
    PrepParams np;
    np.kv = static_cast<const uint16_t*>(a.kv);
    np.mv = a.mv;
    np.kt = static_cast<const uint16_t*>(a.kt);
    np.mt = a.mt;
    np.B = a.B;
    np.C = a.C;
    np.R = a.R;
    np.S = S;
    np.groups_per_crop = ceil_div(a.R, kPWaves);
    np.comb_hi = cl.hi;
    np.comb_lo = cl.lo;
    np.heat = heat;
    np.row_f = row_f;
    np.wout = wpark;
    np.w_stride = wstride;
    const long long ngrid = (long long)a.B * np.groups_per_crop;
    if (ngrid > INT_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(row_prep_kernel, dim3((unsigned)ngrid), dim3(kPWaves * kWave), 0, stream,
                       np);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  ContractParams cp;
  cp.query = static_cast<const uint16_t*>(a.query);
  cp.kv = static_cast<const uint16_t*>(a.kv);
  cp.mv = a.mv;
  cp.kt = static_cast<const uint16_t*>(a.kt);
  cp.mt = a.mt;
  cp.B = a.B;
  cp.C = a.C;
  cp.H = a.H;
  cp.W = a.W;
  cp.R = a.R;
  cp.S = S;
  cp.ng = sp.ng;
  cp.chunk_px = sp.chunk_px;
  cp.nchunks = sp.nchunks;
  cp.rblocks = sp.rblocks;
  cp.items_per_crop = sp.nchunks * sp.rblocks;
  cp.nsteps = a.C / kKS;
  cp.comb_hi = (a.kv != nullptr && a.kt != nullptr) ? cl.hi : 0;
  cp.comb_lo = (a.kv != nullptr && a.kt != nullptr) ? cl.lo : 0;
  cp.light_arows = kLightArows;
  cp.heat = heat;
  cp.row_f = row_f;
  cp.wsrc = wpark;
  cp.w_stride = wstride;
  cp.idx = a.idx;
  cp.xy = a.xy;
  cp.score = a.score;
  cp.corners = a.corners;
  cp.tok_T = a.tokens ? a.tok_skip + S : 0;
  cp.tok_skip = a.tokens ? a.tok_skip : 0;
  cp.up_corners = a.up_corners;
  cp.magic_w = (0x100000000ull + (uint64_t)a.W - 1) / (uint64_t)a.W;
  const long long cgrid = crops_pad * cp.items_per_crop;
  if (cgrid > INT_MAX) return hipErrorInvalidConfiguration;
  if (a.tokens)
    hipLaunchKernelGGL(contract_kernel<true>, dim3((unsigned)cgrid), dim3(kCThreads),
                       sp.contract_lds, stream, cp);
  else
    hipLaunchKernelGGL(contract_kernel<false>, dim3((unsigned)cgrid), dim3(kCThreads),
                       sp.contract_lds, stream, cp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || kp) return e;

  ExpandParams ep;
  ep.mv = a.mv;
  ep.mt = a.mt;
  ep.B = a.B;
  ep.H = a.H;
  ep.W = a.W;
  ep.R = a.R;
  ep.S = S;
  ep.Ho = 4 * a.H;
  ep.Wo = 4 * a.W;
  ep.wpg = sp.wpg;
  ep.groups_per_crop = ceil_div(a.R, sp.wpg);
  ep.magic_w = (0x100000000ull + (uint64_t)a.W - 1) / (uint64_t)a.W;
  ep.heat = heat;
  ep.row_f = row_f;
  ep.idx = a.idx;
  ep.corners = a.corners;
  ep.xy = a.xy;
  ep.score = a.score;
  size_t elds = sp.expand_lds;
  if ((long long)a.B * a.R >= kExpandCapRows) {
    const size_t row_bytes = row_f * sizeof(float);
    const size_t cap = row_bytes > kExpandBigRow     ? kExpandLds1
                       : row_bytes > kExpandSmallRow ? kExpandLds2
                                                     : kExpandLds3;
    if (elds < cap) elds = cap;
  }
  const long long egrid = crops_pad * ep.groups_per_crop;
  if (egrid > INT_MAX) return hipErrorInvalidConfiguration;
#define GKD_EXPAND(SW, BF, UPC)                                                              \
  hipLaunchKernelGGL((expand_kernel<SW, BF, UPC>), dim3((unsigned)egrid), dim3(kEThreads),   \
                     elds, stream, ep)
  if (a.up_corners) {
    if (a.heat_bf16) GKD_EXPAND(false, true, true);
    else GKD_EXPAND(false, false, true);
  } else if (a.W <= kWave) {
    if (a.heat_bf16) GKD_EXPAND(true, true, false);
    else GKD_EXPAND(true, false, false);
  } else {
    if (a.heat_bf16) GKD_EXPAND(false, true, false);
    else GKD_EXPAND(false, false, false);
  }
#undef GKD_EXPAND
  return hipGetLastError();
}

}  // namespace gkd
