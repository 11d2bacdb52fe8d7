// heatmap_lds.hip - gkd_kernel_heatmap, bf16 fast path on gfx950: the
// feature map streams HBM -> LDS with direct-to-LDS 16-byte loads and feeds
// the matrix cores through transposing LDS reads.
//
// Same computation as heatmap.hip (GKDT-L GGUF model card, section "Model":
// 4x bilinear upsample, L2 kernel norm, 1x1 kernel conv, per-row mask
// fusion, rows padded to 80; contracted at low resolution, then expanded),
// organised for the memory pipeline of a CU:
//   - a vector memory instruction costs the address unit about the same
//     time whatever its width, so every load here moves 16 bytes per lane;
//   - F is staged once per workgroup in LDS, so one item covers up to 32
//     rows (64 MFMA rows with both modalities) and a crop's feature map is
//     re-read from L2 at most ceil(rows / 32) times;
//   - the LDS tile keeps F's natural [channel][pixel] layout; the MFMA B
//     operand (8 channels of one pixel per lane) comes from two
//     ds_read_b64_tr_b16: within each 16-lane group, lane 4a + t receives
//     element t of the 8-byte rows read by lanes a, a+4, a+8, a+12, so a
//     lane pointing at channel row 4e + .. of column block a hands the
//     4 channels of pixel 4a + t to lane 4a + t.
//
// K loop: a ring of three LDS stages, each [F: 32 channels x S pixels,
// padded rows] + [A: 64 kernel rows x 32 channels, 80-byte rows]. Every
// wave issues exactly five global_load_lds_dwordx4 per stage, so after
// `s_waitcnt vmcnt(5)` its part of stage k has landed while stage k+1 stays
// in flight; a bare s_barrier (no fence, which would drain every
// outstanding load) then publishes stage k and frees stage k-1 for the
// loads of step k+2.
//
// Row norms are taken before the loop from global memory (float32 sums of
// the stored bf16 values). After the loop the fused low-res maps overwrite
// the stage buffers; the 4x expand, non-temporal stores and the argmax are
// as in heatmap.hip.
#include "gkd_device.hpp"
#include "launch.hpp"

#include <climits>
#include <cmath>

namespace gkd {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int kWaves = 9;
constexpr int kThreads = kWaves * kWave;  // 576
constexpr int kRB = 32;                   // max output rows per item
constexpr int kARows = 2 * kRB;           // kernel rows per stage (both modalities)
constexpr int kKS = 32;                   // channels per K step
constexpr int kStages = 3;
constexpr int kDmaPerWave = 5;            // global_load_lds per wave per stage
constexpr int kSlots = kDmaPerWave * kWaves * kWave;  // 16-byte slots per stage
constexpr int kVis = 1, kTxt = 2;
constexpr int kMaxS = 576;                // one pixel group: 9 waves x 64 px

struct LdsParams {
  const uint16_t* query;
  const uint16_t* kv;
  const uint8_t* mv;
  const uint16_t* kt;
  const uint8_t* mt;
  int B, C, H, W, R, S;
  int rows_per_item, items_per_crop, nsteps;
  int rs;          // 16-byte slots per LDS F row: S/8 + 1 (one pad slot)
  int stage_bytes;
  float* heat;
  int32_t* idx;
  float* xy;
  float* score;
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 layout:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence (a fence would also drain the
// direct-to-LDS loads in flight). This wave's own LDS writes are completed
// first (lgkmcnt(0)); its direct-to-LDS loads are the caller's business.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One lane's share of one stage: five 16-byte source addresses; the LDS
// destination of slot u is fixed at stage + 16 u by the instruction.
struct DmaPlan {
  const uint16_t* base[kDmaPerWave];
  int stride[kDmaPerWave];  // elements per channel step (S for F, 1 for A, 0 junk)
};

// K loop for one item and the fused low-res maps. MODE: modalities present
// in the item; MH: M tiles (16 rows) per modality. A fragments of rows
// that are empty or masked are zeroed in registers: their LDS rows hold a
// stand-in row (the load must have a valid address) that may be anything.
template <int MODE, int MH>
__device__ __forceinline__ void contract_item(const LdsParams& p, unsigned char* lds,
                                              const DmaPlan& plan, int nsel, int wave, int lane,
                                              const uint8_t* s_mv, const uint8_t* s_mt,
                                              const float (*s_w)[kRB]) {
  const int n16 = lane & 15, g4 = lane >> 4;
  const int nst = p.S / 64;  // super-tiles (<= 9)
  const bool computes = wave < nst;
  const int nF = kKS * p.rs;
  const int row_bytes = p.rs * 16;
  bool on[2][MH];
#pragma unroll
  for (int h = 0; h < MH; ++h) {
    const int slot = 16 * h + n16;
    on[0][h] = slot < nsel && s_mv[slot];
    on[1][h] = slot < nsel && s_mt[slot];
  }
  f32x4 acc[2 * MH][4];
#pragma unroll
  for (int m = 0; m < 2 * MH; ++m)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int stage, int step) {
    unsigned char* sb = lds + (size_t)stage * p.stage_bytes;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const uint16_t* src = plan.base[i] + (size_t)(step * kKS) * plan.stride[i];
      __builtin_amdgcn_global_load_lds(
          (glb_void*)src, (lds_void*)(sb + (size_t)(wave * kDmaPerWave + i) * 1024), 16, 0, 0);
    }
  };

  for (int k = 0; k < p.nsteps; ++k) {
    wait_vmcnt<kDmaPerWave>();  // this wave's stage k landed (stage k+1 may fly)
    lds_barrier();              // everyone's stage k landed; stage k-1 is free
    const int ahead = k + 2 < p.nsteps ? k + 2 : p.nsteps - 1;
    issue((k + 2) % kStages, ahead);
    if (computes) {
      const unsigned char* sb = lds + (size_t)(k % kStages) * p.stage_bytes;
      const unsigned char* sa = sb + (size_t)nF * 16;
      u32x4 a[2][MH];
#pragma unroll
      for (int mod = 0; mod < 2; ++mod) {
        if (!(MODE & (mod == 0 ? kVis : kTxt))) continue;
#pragma unroll
        for (int h = 0; h < MH; ++h) {
          const int ar = mod * kRB + 16 * h + n16;
          const u32x4 v = *reinterpret_cast<const u32x4*>(sa + ar * 80 + 16 * g4);
          a[mod][h] = on[mod][h] ? v : u32x4{0u, 0u, 0u, 0u};
        }
      }
      // B operands of the wave's 4 N-tiles: 8 transposing reads, issued
      // together and completed inside the same asm block (the compiler's
      // own wait for them would also drain the direct-to-LDS loads of the
      // next stages)
      const int px = wave * 64 + 4 * (n16 & 3);
      const int r0 = 8 * g4 + (n16 >> 2);
      const uint32_t lo_addr =
          (uint32_t)(uintptr_t)(lds_void*)(sb + r0 * row_bytes + px * 2);
      const uint32_t hi_addr = lo_addr + 4 * row_bytes;
      u32x2 blo[4], bhi[4];
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n"
          "ds_read_b64_tr_b16 %1, %8 offset:32\n"
          "ds_read_b64_tr_b16 %2, %8 offset:64\n"
          "ds_read_b64_tr_b16 %3, %8 offset:96\n"
          "ds_read_b64_tr_b16 %4, %9\n"
          "ds_read_b64_tr_b16 %5, %9 offset:32\n"
          "ds_read_b64_tr_b16 %6, %9 offset:64\n"
          "ds_read_b64_tr_b16 %7, %9 offset:96\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(blo[0]), "=&v"(blo[1]), "=&v"(blo[2]), "=&v"(blo[3]), "=&v"(bhi[0]),
            "=&v"(bhi[1]), "=&v"(bhi[2]), "=&v"(bhi[3])
          : "v"(lo_addr), "v"(hi_addr)
          : "memory");
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8 bv =
            __builtin_bit_cast(bf16x8, u32x4{blo[t].x, blo[t].y, bhi[t].x, bhi[t].y});
#pragma unroll
        for (int mod = 0; mod < 2; ++mod) {
          if (!(MODE & (mod == 0 ? kVis : kTxt))) continue;
#pragma unroll
          for (int h = 0; h < MH; ++h)
            acc[mod * MH + h][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a[mod][h]), bv, acc[mod * MH + h][t], 0, 0, 0);
        }
      }
    }
  }
  wait_vmcnt<0>();  // the ring's trailing reloads too: P overwrites the stages
  lds_barrier();

  // fused low-res maps -> LDS P[slot][S]; lane (n16, g4) holds rows
  // 4 g4 + i of each M tile at pixel 64 w + 16 t + n16
  float* P = reinterpret_cast<float*>(lds);
  if (computes) {
#pragma unroll
    for (int h = 0; h < MH; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = 16 * h + 4 * g4 + i;
        if (slot >= nsel) continue;
        const float wv = (MODE & kVis) ? s_w[0][slot] : 0.f;
        const float wt = (MODE & kTxt) ? s_w[1][slot] : 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float av = (MODE & kVis) ? acc[h][t][i] : 0.f;
          const float at = (MODE & kTxt) ? acc[MH + h][t][i] : 0.f;
          P[(size_t)slot * p.S + wave * 64 + 16 * t + n16] = fmaf(wt, at, wv * av);
        }
      }
    }
  }
}

template <int MH>
__global__ __launch_bounds__(kThreads) void heatmap_lds_kernel(LdsParams p) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int s_rows[kRB];
  __shared__ uint8_t s_mv[kRB], s_mt[kRB];
  __shared__ int s_nvalid, s_nsel;
  __shared__ float s_w[2][kRB];  // fusion weights: mask / (n ||k||)
  __shared__ float s_redv[kRB][kWaves];
  __shared__ int s_redi[kRB][kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const ItemCoord ic = xcd_item(blockIdx.x, p.items_per_crop);
  const int b = ic.crop;
  if (b >= p.B) return;
  const uint8_t* mv = p.mv ? p.mv + (size_t)b * p.R : nullptr;
  const uint8_t* mt = p.mt ? p.mt + (size_t)b * p.R : nullptr;

  if (wave == 0)
    select_rows(mv, mt, p.R, lane, ic.item, p.rows_per_item, s_rows, s_mv, s_mt, &s_nvalid,
                &s_nsel);
  if (ic.item == 0 && p.idx) {
    for (int r = tid; r < p.R; r += kThreads) {
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
  const int nsel = s_nsel;
  if (nsel == 0) return;
  bool has_v = false, has_t = false;
  int first_v = 0, first_t = 0;
  for (int s = nsel - 1; s >= 0; --s) {
    if (s_mv[s]) { has_v = true; first_v = s; }
    if (s_mt[s]) { has_t = true; first_t = s; }
  }

  const uint16_t* F = p.query + (size_t)b * p.C * p.S;

  // ---- DMA plan: slot u -> source (F row / kernel row / stand-in) -------
  const int nF = kKS * p.rs;  // F slots
  const int nA = kARows * 5;  // A slots: 4 data + 1 pad per row
  DmaPlan plan;
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int u = (wave * kDmaPerWave + i) * kWave + lane;
    const uint16_t* base = F;  // stand-in: any valid 16-byte source
    int stride = 0;
    if (u < nF) {
      const int r = u / p.rs, cc = u - r * p.rs;
      base = F + (size_t)r * p.S + (cc < p.rs - 1 ? 8 * cc : 0);
      stride = p.S;
    } else if (u < nF + nA) {
      const int v = u - nF, ar = v / 5, ac = v - ar * 5;
      const int mod = ar / kRB, slot = ar - mod * kRB;
      const bool present = mod == 0 ? has_v : has_t;
      if (present) {
        const bool on = slot < nsel && (mod == 0 ? s_mv[slot] : s_mt[slot]);
        const int use = on ? slot : (mod == 0 ? first_v : first_t);
        const uint16_t* kbase = mod == 0 ? p.kv : p.kt;
        base = kbase + ((size_t)b * p.R + s_rows[use]) * p.C + (ac < 4 ? 8 * ac : 0);
        stride = 1;
      }
    }
    plan.base[i] = base;
    plan.stride[i] = stride;
  }
  // prologue: stages 0 and 1 in flight ...
  {
    const int s1 = p.nsteps > 1 ? 1 : 0;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      unsigned char* sb = lds + (size_t)st * p.stage_bytes;
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i) {
        const uint16_t* src = plan.base[i] + (size_t)((st == 0 ? 0 : s1) * kKS) * plan.stride[i];
        __builtin_amdgcn_global_load_lds(
            (glb_void*)src, (lds_void*)(sb + (size_t)(wave * kDmaPerWave + i) * 1024), 16, 0, 0);
      }
    }
  }
  // ... while the row norms are taken from global memory (their loads
  // drain the counter once, before any compute)
  for (int row = wave; row < kARows; row += kWaves) {
    const int mod = row / kRB, slot = row - mod * kRB;
    const bool on = slot < nsel && (mod == 0 ? s_mv[slot] : s_mt[slot]);
    float ss = 0.f;
    if (on) {
      const uint16_t* k = (mod == 0 ? p.kv : p.kt) + ((size_t)b * p.R + s_rows[slot]) * p.C;
      for (int c = 8 * lane; c < p.C; c += 8 * kWave) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(k + c);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float lo = __uint_as_float(v[d] << 16), hi = __uint_as_float(v[d] & 0xffff0000u);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        }
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) {
      float w = 0.f;
      if (on) {
        const float n = (float)((int)s_mv[slot] + (int)s_mt[slot]);
        w = 1.f / (fmaxf(sqrtf(ss), 1e-12f) * n);
      }
      s_w[mod][slot] = w;
    }
  }
  wait_vmcnt<0>();

  if (has_v && has_t)
    contract_item<kVis | kTxt, MH>(p, lds, plan, nsel, wave, lane, s_mv, s_mt, s_w);
  else if (has_v)
    contract_item<kVis, MH>(p, lds, plan, nsel, wave, lane, s_mv, s_mt, s_w);
  else
    contract_item<kTxt, MH>(p, lds, plan, nsel, wave, lane, s_mv, s_mt, s_w);
  __syncthreads();
  float* P = reinterpret_cast<float*>(lds);

  // ---- 4x expand + non-temporal stores + running argmax -----------------
  const int Ho = 4 * p.H, Wo = 4 * p.W;
  for (int s = 0; s < nsel; ++s) {
    const float* Pr = P + (size_t)s * p.S;
    float* out = p.heat + ((size_t)b * p.R + s_rows[s]) * (size_t)Ho * Wo;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int cell = tid; cell < p.S; cell += kThreads) {
      const int i = cell / p.W, j = cell - i * p.W;
      const int im = i > 0 ? i - 1 : 0, ip = i < p.H - 1 ? i + 1 : i;
      const int jm = j > 0 ? j - 1 : 0, jp = j < p.W - 1 ? j + 1 : j;
      float xl[4], xh[4], yl[4], yh[4];
      bilinear_taps4(j, p.W, xl, xh);
      bilinear_taps4(i, p.H, yl, yh);
      float hm[4], h0[4], hp[4];
      bilinear_hrow(Pr + (size_t)im * p.W, j, jm, jp, xl, xh, hm);
      bilinear_hrow(Pr + (size_t)i * p.W, j, jm, jp, xl, xh, h0);
      bilinear_hrow(Pr + (size_t)ip * p.W, j, jm, jp, xl, xh, hp);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float* lo = d < 2 ? hm : h0;
        const float* hi = d < 2 ? h0 : hp;
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fmaf(yh[d], hi[e], yl[d] * lo[e]);
        const int y = 4 * i + d;
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(out + (size_t)y * Wo + 4 * j));
        const int base = y * Wo + 4 * j;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (better(o[e], base + e, bv, bi)) {
            bv = o[e];
            bi = base + e;
          }
      }
    }
    if (p.idx) {
      wave_argmax(bv, bi);
      if (lane == 0) {
        s_redv[s][wave] = bv;
        s_redi[s][wave] = bi;
      }
    }
  }
  if (!p.idx) return;
  __syncthreads();
  if (tid < nsel) {
    float bv = s_redv[tid][0];
    int bi = s_redi[tid][0];
    for (int w = 1; w < kWaves; ++w)
      if (better(s_redv[tid][w], s_redi[tid][w], bv, bi)) {
        bv = s_redv[tid][w];
        bi = s_redi[tid][w];
      }
    const size_t o = (size_t)b * p.R + s_rows[tid];
    const int y = bi / Wo, x = bi - y * Wo;
    p.idx[o] = bi;
    p.xy[2 * o] = (float)(2 * x + 1) / (float)Wo - 1.f;
    p.xy[2 * o + 1] = (float)(2 * y + 1) / (float)Ho - 1.f;
    p.score[o] = bv;
  }
}

hipError_t launch_mh(const LdsParams& p, int mh, size_t lds, int grid, hipStream_t stream) {
  if (mh == 1)
    hipLaunchKernelGGL((heatmap_lds_kernel<1>), dim3(grid), dim3(kThreads), lds, stream, p);
  else
    hipLaunchKernelGGL((heatmap_lds_kernel<2>), dim3(grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

bool heatmap_lds_applicable(int C, int S, bool bf16) {
  return bf16 && C % kKS == 0 && S % 64 == 0 && S <= kMaxS &&
         // F slots + A slots fit the five DMA instructions per wave
         kKS * (S / 8 + 1) + kARows * 5 <= kSlots;
}

hipError_t launch_heatmap_lds(const HeatmapArgs& a, hipStream_t stream) {
  LdsParams p;
  p.query = static_cast<const uint16_t*>(a.query);
  p.kv = static_cast<const uint16_t*>(a.kv);
  p.mv = a.mv;
  p.kt = static_cast<const uint16_t*>(a.kt);
  p.mt = a.mt;
  p.B = a.B;
  p.C = a.C;
  p.H = a.H;
  p.W = a.W;
  p.R = a.R;
  p.S = a.H * a.W;
  p.heat = a.heat;
  p.idx = a.idx;
  p.xy = a.xy;
  p.score = a.score;
  p.rs = p.S / 8 + 1;
  p.nsteps = a.C / kKS;
  p.stage_bytes = kSlots * 16;
  // rows per item: 32 (two M tiles per modality) unless a crop never has
  // more than 16 rows, where one M tile per modality suffices
  p.rows_per_item = a.R > 16 ? kRB : 16;
  const int mh = p.rows_per_item / 16;
  p.items_per_crop = (a.R + p.rows_per_item - 1) / p.rows_per_item;
  const size_t stages = (size_t)kStages * p.stage_bytes;
  const size_t pmaps = (size_t)p.rows_per_item * p.S * 4;
  const size_t lds = stages > pmaps ? stages : pmaps;
  const int crops_pad = (a.B + kXcds - 1) / kXcds * kXcds;
  const long long grid = (long long)crops_pad * p.items_per_crop;
  if (grid > INT_MAX) return hipErrorInvalidConfiguration;
  return launch_mh(p, mh, lds, (int)grid, stream);
}

}  // namespace gkd
