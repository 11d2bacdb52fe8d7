// kg.hip - the kernel-generation (KG) transformer: prototypes -> kernels.
//
// GKDT model card, "Architecture" bullet (2 blocks of self- and
// cross-attention, d_ff = 1024, a mask token); paper summary, four-step
// pipeline (the transformer rewrites the visual and text prototypes into
// the convolution kernels of the head). Readings: the sequence is the 2R
// slots [visual rows, text rows], a slot without a prompt holds the mask
// token, self-attention keys are the slots of prompted rows, blocks are
// post-norm (x = LN(x + SA(x)); LN(x + CA(x, F)); LN(x + FFN(x))) with ReLU,
// heads are 64 wide. The kernels come out as [2, B, R, C]: plane 0 the
// visual kernels, plane 1 the text kernels, as the head takes them.
//
// Only the slots of prompted rows are computed: a row without a prompt
// is no self-attention key, so it changes no other slot's output, and the
// head never reads its kernels. kg_compact_kernel lists the 2 n_b slots of
// the n_b prompted rows of crop b (visual slots, then text slots) as
// consecutive rows of a compact matrix starting at off[b]; every dense
// layer and both attentions run over those rows only, and the last
// LayerNorm scatters them to their [2, B, R, C] places (other rows are not
// written).
//
// bfloat16 throughout for matrix operands (weights, prototypes, features,
// and every activation that feeds a product), float32 for accumulation, the
// residual stream, softmax and LayerNorm. Per block:
//   gemm   x -> [Q|K|V] rows                      (SA in_proj)
//   attn   softmax(Q K^T / 8) V, scores in registers
//   gemm   out_proj + bias + residual (float32)    -> LayerNorm
//   gemm   x -> Q (CA), gemm F -> [K|V] rows       (CA in_proj)
//   attn, gemm + residual -> LayerNorm
//   gemm   W1 + bias, ReLU -> gemm W2 + bias + residual -> LayerNorm
// The products run on v_mfma_f32_16x16x32_bf16.
#include "gkd_device.hpp"
#include "kg_launch.hpp"

namespace gkd {
namespace {

constexpr int kHd = 64;          // head width
constexpr int kMaxKeys = 576;    // attention keys held in registers (36 tiles of 16)
constexpr int kKeyTiles = kMaxKeys / 16;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ float bf(const uint16_t* p, long long i) {
  return bf16_bits_to_f32(p[i]);
}
__host__ __device__ __forceinline__ int rup32(int n) { return (n + 31) & ~31; }

// ---------------------------------------------------------------------------
// C[m, n] = sum_k A[m, k] W[n, k] + bias[n], W a torch Linear weight [N, K].
// Row m of A sits at A + (m / a_rows) * a_bstride + (m % a_rows) * lda, so a
// token sequence with leading special tokens is read in place.
// Epilogues: kOutBf16 (optionally ReLU), columns >= tsplit row-major to
// out2 instead; kOutResF32: float32 acc + bias + res.
// ---------------------------------------------------------------------------
enum { kOutBf16 = 0, kOutBf16Relu = 1, kOutResF32 = 2 };

struct GemmParams {
  const uint16_t* A;
  long long a_bstride;
  int a_rows, lda;
  const uint16_t* W;
  const uint16_t* bias;
  int M, N, K;          // M: rows the grid covers
  const int* m_dev;     // or null: the actual row count (<= M) is *m_dev
  int mode;
  uint16_t* out_bf;
  float* out_f;
  const float* res;
  int ldo;
  int tsplit;
  uint16_t* out2;  // columns >= tsplit go here, row-major, ld2
  int ld2;
};

typedef __attribute__((address_space(3))) void kg_lds_void;
typedef __attribute__((address_space(1))) void kg_glb_void;

// Workgroup tile 256 x BN, K step BK (32 or 64), 8 waves: BN = 256 as
// 2 x 4 wave tiles of 128 x 64, BN = 128 as 4 x 2 wave tiles of 64 x 64
// (MT x 4 MFMA tiles of 16 x 16 per wave). Both operand tiles stream
// straight into LDS (global_load_lds, 16 bytes a lane) through a ring of NS
// stages, the loads of K step k + NS - 1 issued right after the barrier of
// step k. Row r of a tile is BK / 8 16-byte chunks; chunk c sits at chunk
// position c ^ sw(r), sw(r) = r & 7 for 8 chunks a row and (r >> 2) & 3 for
// 4, so the 16 rows an MFMA operand read touches fall in different banks.
constexpr int kGM = 256;
constexpr int kGemmBK = 64, kGemmNS = 2;

template <int BN, int BK, int NS>
__host__ __device__ constexpr size_t gemm_lds_bytes() {
  return (size_t)NS * (kGM + BN) * BK * 2;
}

template <int CPR>
__device__ __forceinline__ int gemm_sw(int r) {
  return CPR == 8 ? (r & 7) : ((r >> 2) & 3);
}

// s_waitcnt vmcnt(N) (N < 64), the other counters left alone
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt(0x0070 | 0x0f00 | (N & 15) | ((N >> 4) << 14));
}

template <int BN, int BK, int NS>
__global__ __launch_bounds__(512) void kg_gemm_kernel(GemmParams p) {
  constexpr int WM = BN == 256 ? 128 : 64;  // wave tile rows
  constexpr int MT = WM / 16;
  constexpr int NT = 4;                     // wave tile columns: 64
  constexpr int WN = BN / 64;               // waves across N
  constexpr int CPR = BK / 8;               // 16-byte chunks a row
  constexpr int A_BYTES = kGM * BK * 2;
  constexpr int STAGE = (kGM + BN) * BK * 2;
  constexpr int NA = kGM * CPR / 512;       // A loads per wave and step (64 lanes x 8 waves)
  constexpr int NB = BN * CPR / 512;
  constexpr int PS = NA + NB;               // loads per wave and stage
  static_assert(NS >= 2 && NS <= 4 && PS * (NS - 2) < 16, "ring shape");
  extern __shared__ __attribute__((aligned(16))) unsigned char glds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_n = (p.N + BN - 1) / BN;
  // With a device-side row count the grid covers the most rows there can
  // be and only the first `total` workgroups have tiles.
  if (p.m_dev != nullptr) p.M = *p.m_dev;
  const int total = ((p.M + kGM - 1) / kGM) * tiles_n;
  const int bid = blockIdx.x;
  if (bid >= total) return;
  // Workgroups are dealt round-robin over the 8 XCDs (XCD bid % 8); give
  // each XCD a contiguous run of the tiles, so the N-tiles of one A row
  // band share an L2: XCD x takes tiles s_x .. s_x + c_x - 1 with
  // c_x = total / 8 (+1 for the first total % 8).
  const int xcd = bid % kXcds, q = total / kXcds, rem = total % kXcds;
  const int lin = xcd * q + min(xcd, rem) + bid / kXcds;
  const int m0 = (lin / tiles_n) * kGM, n0 = (lin % tiles_n) * BN;

  // per-lane element offsets of the chunks this lane loads (step 0)
  uint32_t aoff[NA], woff[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int q = (wave + 8 * i) * 64 + lane, r = q / CPR, cs = (q % CPR) ^ gemm_sw<CPR>(r);
    const int m = min(m0 + r, p.M - 1);
    aoff[i] = (uint32_t)((long long)(m / p.a_rows) * p.a_bstride + (long long)(m % p.a_rows) * p.lda +
                         8 * cs);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int q = (wave + 8 * i) * 64 + lane, r = q / CPR, cs = (q % CPR) ^ gemm_sw<CPR>(r);
    const int n = min(n0 + r, p.N - 1);
    woff[i] = (uint32_t)((long long)n * p.K + 8 * cs);
  }
  auto issue = [&](int stage, int k0) {
    unsigned char* base = glds + (size_t)stage * STAGE;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      __builtin_amdgcn_global_load_lds((kg_glb_void*)(p.A + aoff[i] + k0),
                                       (kg_lds_void*)(base + (size_t)(wave + 8 * i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      __builtin_amdgcn_global_load_lds((kg_glb_void*)(p.W + woff[i] + k0),
                                       (kg_lds_void*)(base + A_BYTES + (size_t)(wave + 8 * i) * 1024),
                                       16, 0, 0);
  };

  const int wm0 = (wave / WN) * WM, wn0 = (wave % WN) * 64;
  const int fr = lane & 15, g = lane >> 4;
  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / BK;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s, s * BK);
  int slot = 0;  // kt % NS
  for (int kt = 0; kt < nk; ++kt) {
    // this step's loads landed; later steps' (up to NS - 2 of them) may fly
    const int later = min(NS - 2, nk - 1 - kt);
    if (NS > 3 && later >= 2) wait_vmcnt<2 * PS>();
    else if (NS > 2 && later >= 1) wait_vmcnt<PS>();
    else wait_vmcnt<0>();
    __syncthreads();  // everyone's; the slot step kt - 1 used is free
    if (kt + NS - 1 < nk) issue(slot == 0 ? NS - 1 : slot - 1, (kt + NS - 1) * BK);
    const unsigned char* sa = glds + (size_t)slot * STAGE;
    const unsigned char* sb = sa + A_BYTES;
    slot = slot + 1 == NS ? 0 : slot + 1;
    // Operand fragments run one group ahead of the MFMAs that use them: a
    // group is two A fragments (rows 16 i .. 16 i + 31 of the wave tile)
    // times the four B fragments of one 32-wide K half, and the loads for
    // group n + 1 are issued before the MFMAs of group n, so their LDS
    // latency hides behind those MFMAs.
    constexpr int GPH = MT / 2;         // groups a K half
    constexpr int NG = GPH * (BK / 32);
    auto lds16 = [&](const unsigned char* t, int r, int j) {
      return as_bf16x8(*reinterpret_cast<const u32x4*>(t + (r * CPR + (j ^ gemm_sw<CPR>(r))) * 16));
    };
    bf16x8 bq[BK / 32][NT];
    bf16x8 aq[2][2];
#pragma unroll
    for (int jn = 0; jn < NT; ++jn) bq[0][jn] = lds16(sb, wn0 + 16 * jn + fr, g);
#pragma unroll
    for (int u = 0; u < 2; ++u) aq[0][u] = lds16(sa, wm0 + 16 * u + fr, g);
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      const int h = n / GPH, i = 2 * (n % GPH);
      if (n + 1 < NG) {
        const int h1 = (n + 1) / GPH, i1 = 2 * ((n + 1) % GPH);
#pragma unroll
        for (int u = 0; u < 2; ++u) aq[(n + 1) & 1][u] = lds16(sa, wm0 + 16 * (i1 + u) + fr, 4 * h1 + g);
      }
      if (BK / 32 > 1 && n == 0) {
        // the second K half's B fragments, well ahead of their first use
#pragma unroll
        for (int jn = 0; jn < NT; ++jn) bq[BK / 32 - 1][jn] = lds16(sb, wn0 + 16 * jn + fr, 4 + g);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int jn = 0; jn < NT; ++jn)
          acc[i + u][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bq[h][jn], aq[n & 1][u], acc[i + u][jn], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // The MFMAs compute the transposed tile (W rows as the first operand), so
  // acc[i][j][e] holds C[m0 + wm0 + 16 i + fr][n0 + wn0 + 16 j + 4 g + e]:
  // four consecutive columns of one row, stored as one 8- or 16-byte piece
  // (N, tsplit and the leading dimensions are multiples of 64).
  const int mrow = m0 + wm0 + fr;
  const int nb = n0 + wn0 + 4 * g;
  if (p.mode == kOutResF32) {
#pragma unroll
    for (int jn = 0; jn < NT; ++jn) {
      const int n = nb + 16 * jn;
      if (n >= p.N) continue;
      // the column group's residual loads first, then its stores
      f32x4 r[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int m = mrow + 16 * i;
        r[i] = m < p.M ? *reinterpret_cast<const f32x4*>(p.res + (long long)m * p.ldo + n)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const f32x4 bias = {bf(p.bias, n), bf(p.bias, n + 1), bf(p.bias, n + 2), bf(p.bias, n + 3)};
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int m = mrow + 16 * i;
        if (m < p.M)
          *reinterpret_cast<f32x4*>(p.out_f + (long long)m * p.ldo + n) = acc[i][jn] + bias + r[i];
      }
    }
    return;
  }
  const bool relu = p.mode == kOutBf16Relu;
#pragma unroll
  for (int jn = 0; jn < NT; ++jn) {
    const int n = nb + 16 * jn;
    if (n >= p.N) continue;
    const f32x4 bias = {bf(p.bias, n), bf(p.bias, n + 1), bf(p.bias, n + 2), bf(p.bias, n + 3)};
    uint16_t* dst;
    int ld;
    if (n < p.tsplit) {
      dst = p.out_bf + n;
      ld = p.ldo;
    } else {
      dst = p.out2 + (n - p.tsplit);
      ld = p.ld2;
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = mrow + 16 * i;
      if (m >= p.M) continue;
      f32x4 v = acc[i][jn] + bias;
      if (relu) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], 0.f);
      }
      const uint32_t w0 = f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
      const uint32_t w1 = f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
      *reinterpret_cast<u32x2*>(dst + (long long)m * ld) = u32x2{w0, w1};
    }
  }
}

// ---------------------------------------------------------------------------
// Attention of the compact query rows of one crop (off[b] .. off[b+1]) over
// Tk <= 576 keys, one workgroup per (crop, head). Keys: the
// crop's own compact rows (self-attention) or the crop's Tk query-feature
// tokens (cross-attention); K and V are row-major in both cases. The
// launches take it for self-attention; cross-attention streams its keys
// (kg_xattn_kernel, below).
// The head's K and V rows (128 bytes each, keys past Tk repeat the last
// key, whose probability is 0) stream into LDS with global_load_lds, 16
// bytes a lane and no register round trip; 16-byte chunk c of key row r
// sits at chunk position c ^ (r & 7), so the 16 key rows one operand read
// touches spread over the banks. A wave takes 16 queries at a time and
// computes the transposed scores S^T = K Q^T, so lane (query n = lane & 15,
// group g = lane >> 4) holds keys 16 t + 4 g + e (e = 0..3) of its query
// in tile t: 36 tiles cover 576 keys in registers. Softmax (scale
// 1/sqrt(64)) reduces over e, t and the 4 lane groups. The product
// O^T = V^T P^T takes its P^T operand straight from those registers: an
// MFMA sums over its 32 k-slots in any order as long as both operands
// agree, so k-slots 8 g .. 8 g + 7 of a 32-key chunk c carry keys
// 32 c + 4 g + (0..3) and 32 c + 16 + 4 g + (0..3) on both sides; the V^T
// operand comes from row-major V through transposing LDS reads
// (ds_read_b64_tr_b16: the 16 lanes of a group each point at 4 dims of one
// of 4 key rows, and lane n receives the 4 keys of dim n). A crop without
// compact rows has nothing to do.
// ---------------------------------------------------------------------------
struct AttnParams {
  const uint16_t* q;
  int ldq;
  const uint16_t* k;      // K rows, head h at columns 64 h ..
  int ldk;
  const uint16_t* v;      // V rows, likewise
  int ldv;
  const int* off;         // compact rows of crop b: off[b] .. off[b+1]
  uint16_t* out;
  int ldo;
  int nh, Tk;             // Tk: cross-attention keys per crop; 0: self-attention
};

// Waves per workgroup: 8 where the key tiles leave room for two waves a
// SIMD (NT = 10), 4 for 576 keys, whose scores need most of a SIMD's registers.
template <int NT>
constexpr int attn_waves() { return NT <= 10 ? 8 : 4; }

__host__ __device__ inline size_t attn_lds_bytes(int tk_max) {
  return (size_t)rup32(tk_max) * kHd * 2 * 2;  // K and V rows
}

// bfloat16 bits of a float, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// NT: key tiles held in registers (10 covers 160 keys, 36 covers 576).
template <int NT>
__global__ __launch_bounds__(64 * attn_waves<NT>()) void kg_attn_kernel(AttnParams p) {
  constexpr int kAttnWaves = attn_waves<NT>();
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_kv[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x % p.nh, b = blockIdx.x / p.nh;
  const int fr = lane & 15, g = lane >> 4, fk = g * 8;
  const int qb = p.off[b], Tq = p.off[b + 1] - qb;
  if (Tq <= 0) return;
  const bool self = p.Tk == 0;
  const int Tk = self ? Tq : p.Tk;
  const long long kb = self ? (long long)qb : (long long)b * p.Tk;  // first key row
  const int nt = (Tk + 15) >> 4, kpad = rup32(Tk);
  unsigned char* sK = lds_kv;
  unsigned char* sV = lds_kv + (size_t)kpad * 128;

  // Stage K, then V: 1-KiB blocks of 8 key rows, one block per wave and
  // instruction.
  const int nblk = kpad / 8;
  for (int blk = wave; blk < 2 * nblk; blk += kAttnWaves) {
    const bool isv = blk >= nblk;
    const int bl = isv ? blk - nblk : blk;
    const int q = bl * 64 + lane, r = q >> 3, c = (q & 7) ^ (r & 7);
    const long long key = kb + min(r, Tk - 1);
    const uint16_t* src = (isv ? p.v + key * p.ldv : p.k + key * p.ldk) + h * kHd + 8 * c;
    __builtin_amdgcn_global_load_lds((kg_glb_void*)src, (kg_lds_void*)((isv ? sV : sK) + bl * 1024),
                                     16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0070 | 0x0f00);  // vmcnt(0): this wave's blocks landed
  __syncthreads();                              // and everyone's

  for (int q0 = wave * 16; q0 < Tq; q0 += 16 * kAttnWaves) {

  const uint16_t* qrow = p.q + (qb + min(q0 + fr, Tq - 1)) * (long long)p.ldq + h * kHd + fk;
  const bf16x8 qb0 = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow));
  const bf16x8 qb1 = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 32));

  f32x4 s[NT];
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if ((t & 3) == 0) __builtin_amdgcn_sched_barrier(0);  // K reads a few tiles ahead, not all
    if (t < nt) {
      const int key = t * 16 + fr;  // rows past Tk: masked below
      const unsigned char* krow = sK + key * 128;
      const bf16x8 k0 = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + ((g ^ (key & 7)) << 4)));
      const bf16x8 k1 = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + (((g + 4) ^ (key & 7)) << 4)));
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qb0, z, 0, 0, 0);
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb1, z, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = t * 16 + 4 * g + e;
        z[e] = kk < Tk ? z[e] : -INFINITY;
        mx = fmaxf(mx, z[e]);
      }
      s[t] = z;
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));

  // p = exp((s - max) / 8) = exp2((s - max) * log2(e) / 8); keys past Tk
  // hold -inf and give 0.
  constexpr float kScale = 0.125f * 1.4426950408889634f;
  const float base = mx == -INFINITY ? 0.f : mx;
  float sum = 0.f;
  uint32_t pk[NT + 1][2];  // bfloat16 pairs: keys (4g, 4g+1), (4g+2, 4g+3) of tile t
  pk[NT][0] = pk[NT][1] = 0u;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < nt) {
      uint32_t hb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // v_exp_f32 directly: arguments are <= 0 and results below 2^-126
        // are far under the bfloat16 rounding of the largest term.
        hb[e] = bf16_rne(__builtin_amdgcn_exp2f((s[t][e] - base) * kScale));
        sum += bf16_bits_to_f32(hb[e]);  // the sum of what the product uses
      }
      pk[t][0] = hb[0] | (hb[1] << 16);
      pk[t][1] = hb[2] | (hb[3] << 16);
    } else {
      pk[t][0] = pk[t][1] = 0u;
    }
  }
  sum += __shfl_xor(sum, 16);
  sum += __shfl_xor(sum, 32);

  f32x4 o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // lane (fr, g) points at key row 4 g + fr / 4 of the chunk, dims
  // 16 j + 4 (fr % 4) .. + 3; the keys 16 further share the row swizzle
  const int vkey = 4 * g + (fr >> 2);
#pragma unroll
  for (int c = 0; c < (NT + 1) / 2; ++c) {
    // keep the V reads of each chunk beside its MFMAs (hoisted, they would
    // sit in registers next to all of P)
    __builtin_amdgcn_sched_barrier(0);
    if (2 * c < nt) {
      const bf16x8 pb = as_bf16x8(u32x4{pk[2 * c][0], pk[2 * c][1], pk[2 * c + 1][0], pk[2 * c + 1][1]});
      const int key = 32 * c + vkey;
      const unsigned char* vrow = sV + key * 128 + (fr & 1) * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int chunk = 2 * j + ((fr & 3) >> 1);
        const unsigned char* a = vrow + ((chunk ^ (key & 7)) << 4);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 16 * 128));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const bf16x8 va = as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]});
        o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[j], 0, 0, 0);
      }
    }
  }
  // o[j][e] = O^T[dim 16 j + 4 g + e][query q0 + fr]
  const int qi = q0 + fr;
  if (qi < Tq) {
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    uint16_t* orow = p.out + (qb + qi) * (long long)p.ldo + h * kHd + 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w0 = f32_to_bf16_bits(o[j][0] * inv) | ((uint32_t)f32_to_bf16_bits(o[j][1] * inv) << 16);
      const uint32_t w1 = f32_to_bf16_bits(o[j][2] * inv) | ((uint32_t)f32_to_bf16_bits(o[j][3] * inv) << 16);
      *reinterpret_cast<u32x2*>(orow + 16 * j) = u32x2{w0, w1};
    }
  }
  }  // query groups
}

// ---------------------------------------------------------------------------
// Cross-attention with the keys streamed: the same product as above for
// Tk = HW keys (the crop's query-feature tokens), one workgroup of 8 waves
// per (crop, head), but K and V pass through a three-stage LDS ring in
// chunks of 64 keys (16 KiB a stage, global_load_lds, same swizzle), so a
// workgroup needs 48 KiB and several share a CU, one's loads overlapping
// another's products. Softmax runs online (Milakov and Gimelshein, "Online
// normalizer calculation for softmax"): per chunk the running maximum m of
// a query moves to max(m, chunk max), the sum l and the output O are scaled
// by exp((m_old - m_new) / 8) and the chunk's probabilities
// exp((s - m_new) / 8), rounded to bfloat16, are added to l and, through
// the MFMA, to O. Wave w owns query tile w of each pass of 128 queries
// (one tile a wave keeps two workgroups on a CU).
// ---------------------------------------------------------------------------
constexpr int kXaWaves = 8, kXaChunk = 64, kXaStages = 3;
constexpr int kXaStage = 2 * kXaChunk * 128;  // K rows, then V rows
constexpr int kXaQt = 1;                     // query tiles a wave holds

__global__ __launch_bounds__(64 * kXaWaves) void kg_xattn_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_ring[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x % p.nh, b = blockIdx.x / p.nh;
  const int fr = lane & 15, g = lane >> 4, fk = g * 8;
  const int qb = p.off[b], Tq = p.off[b + 1] - qb;
  if (Tq <= 0) return;
  const int Tk = p.Tk;
  const long long kb = (long long)b * Tk;
  const int nch = (Tk + kXaChunk - 1) / kXaChunk;
  const int nqt = (Tq + 15) >> 4;
  constexpr float kScale = 0.125f * 1.4426950408889634f;

  // wave w loads K rows 8 w .. 8 w + 7 and V rows 8 w .. 8 w + 7 of a chunk
  const int dr = 8 * wave + (lane >> 3), dc = (lane & 7) ^ (dr & 7);
  auto issue = [&](int ch) {
    unsigned char* st = lds_ring + (ch % kXaStages) * kXaStage;
    const long long key = kb + min(ch * kXaChunk + dr, Tk - 1);
    __builtin_amdgcn_global_load_lds((kg_glb_void*)(p.k + key * p.ldk + h * kHd + 8 * dc),
                                     (kg_lds_void*)(st + wave * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((kg_glb_void*)(p.v + key * p.ldv + h * kHd + 8 * dc),
                                     (kg_lds_void*)(st + kXaChunk * 128 + wave * 1024), 16, 0, 0);
  };

  for (int qt0 = 0; qt0 < nqt; qt0 += kXaWaves * kXaQt) {
    __syncthreads();  // the previous pass is done with the ring
    bf16x8 qf[kXaQt][2];
    f32x4 o[kXaQt][4];
    float m[kXaQt], l[kXaQt];
#pragma unroll
    for (int u = 0; u < kXaQt; ++u) {
      const int q0 = (qt0 + wave + kXaWaves * u) * 16;
      const uint16_t* qrow = p.q + (qb + min(q0 + fr, Tq - 1)) * (long long)p.ldq + h * kHd + fk;
      qf[u][0] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow));
      qf[u][1] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 32));
#pragma unroll
      for (int j = 0; j < 4; ++j) o[u][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[u] = -INFINITY;
      l[u] = 0.f;
    }
    issue(0);
    if (nch > 1) issue(1);
    for (int ch = 0; ch < nch; ++ch) {
      // this chunk's two loads landed (the next chunk's two may still fly)
      if (ch + 1 < nch)
        __builtin_amdgcn_s_waitcnt(0x0070 | 0x0f00 | 2);  // vmcnt(2)
      else
        __builtin_amdgcn_s_waitcnt(0x0070 | 0x0f00);      // vmcnt(0)
      __syncthreads();  // everyone's landed; stage (ch + 2) % 3 is free
      if (ch + 2 < nch) issue(ch + 2);
      const unsigned char* sK = lds_ring + (ch % kXaStages) * kXaStage;
      const unsigned char* sV = sK + kXaChunk * 128;
#pragma unroll
      for (int u = 0; u < kXaQt; ++u) {
        if (qt0 + wave + kXaWaves * u >= nqt) continue;  // wave-uniform
        f32x4 sc[4];
        float cm = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int kr = t * 16 + fr;
          const unsigned char* krow = sK + kr * 128;
          const bf16x8 k0 = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + ((g ^ (kr & 7)) << 4)));
          const bf16x8 k1 = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + (((g + 4) ^ (kr & 7)) << 4)));
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
          z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[u][0], z, 0, 0, 0);
          z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[u][1], z, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            z[e] = ch * kXaChunk + t * 16 + 4 * g + e < Tk ? z[e] : -INFINITY;
            cm = fmaxf(cm, z[e]);
          }
          sc[t] = z;
        }
        cm = fmaxf(cm, __shfl_xor(cm, 16));
        cm = fmaxf(cm, __shfl_xor(cm, 32));
        const float mn = fmaxf(m[u], cm);  // finite: every chunk has a key
        const float alpha = __builtin_amdgcn_exp2f((m[u] - mn) * kScale);  // 0 on the first chunk
        m[u] = mn;
        uint32_t pk[4][2];
        float ps = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          uint32_t hb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hb[e] = bf16_rne(__builtin_amdgcn_exp2f((sc[t][e] - mn) * kScale));
            ps += bf16_bits_to_f32(hb[e]);
          }
          pk[t][0] = hb[0] | (hb[1] << 16);
          pk[t][1] = hb[2] | (hb[3] << 16);
        }
        l[u] = l[u] * alpha + ps;  // this lane's share; the groups are summed at the end
#pragma unroll
        for (int j = 0; j < 4; ++j) o[u][j] *= alpha;
        const int vkey = 4 * g + (fr >> 2);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 pb = as_bf16x8(u32x4{pk[2 * c][0], pk[2 * c][1], pk[2 * c + 1][0], pk[2 * c + 1][1]});
          const int kr = 32 * c + vkey;
          const unsigned char* vrow = sV + kr * 128 + (fr & 1) * 8;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int chunk = 2 * j + ((fr & 3) >> 1);
            const unsigned char* a = vrow + ((chunk ^ (kr & 7)) << 4);
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 16 * 128));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            o[u][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]}),
                                                            pb, o[u][j], 0, 0, 0);
          }
        }
      }
    }
    // o[u][j][e] = O^T[dim 16 j + 4 g + e][query]: normalise and store
#pragma unroll
    for (int u = 0; u < kXaQt; ++u) {
      float sum = l[u];
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      const int qi = (qt0 + wave + kXaWaves * u) * 16 + fr;
      if (qi < Tq) {
        const float inv = sum > 0.f ? 1.f / sum : 0.f;
        uint16_t* orow = p.out + (qb + qi) * (long long)p.ldo + h * kHd + 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w0 = f32_to_bf16_bits(o[u][j][0] * inv) | ((uint32_t)f32_to_bf16_bits(o[u][j][1] * inv) << 16);
          const uint32_t w1 = f32_to_bf16_bits(o[u][j][2] * inv) | ((uint32_t)f32_to_bf16_bits(o[u][j][3] * inv) << 16);
          *reinterpret_cast<u32x2*>(orow + 16 * j) = u32x2{w0, w1};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// LayerNorm of the compact float32 rows m < *m_dev (one wave per row, eps
// 1e-5, biased variance): writes the float32 result (the residual stream)
// and its bfloat16 copy. With R > 0 the bfloat16 rows go to the two-plane
// output instead: compact row m (crop cmap[m], slot smap[m]) lands in row
// (slot / R) * B + b, slot % R of plane-major [2, B, R, C]. The row is read
// once, 16 bytes a lane, and kept in registers (V float4 a lane: C <= 256 V;
// wider rows take V = 0, three passes over the row).
// ---------------------------------------------------------------------------
template <int V>
__global__ __launch_bounds__(256) void kg_layernorm_kernel(const float* y, const uint16_t* w,
                                                           const uint16_t* bvec, const int* m_dev,
                                                           int C, int B, int R, const int* cmap,
                                                           const int* smap, float* x,
                                                           uint16_t* xb) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= *m_dev) return;
  const int n4 = C / 4;
  const f32x4* row = reinterpret_cast<const f32x4*>(y + (long long)m * C);
  long long drow = m;
  if (R > 0) {
    const int b = cmap[m], sl = smap[m];
    drow = ((long long)(sl >= R) * B + b) * R + (sl >= R ? sl - R : sl);
  }
  auto hsum = [](f32x4 v) { return (v[0] + v[1]) + (v[2] + v[3]); };
  auto wave_sum = [](float t) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) t += __shfl_xor(t, d);
    return t;
  };
  auto emit = [&](int c4, f32x4 v, float mu, float rs) {
    const u32x2 wv = *reinterpret_cast<const u32x2*>(w + 4 * c4);
    const u32x2 bv = *reinterpret_cast<const u32x2*>(bvec + 4 * c4);
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t ww = wv[e >> 1] >> (16 * (e & 1)), bb = bv[e >> 1] >> (16 * (e & 1));
      o[e] = fmaf((v[e] - mu) * rs, bf16_bits_to_f32((uint16_t)ww), bf16_bits_to_f32((uint16_t)bb));
    }
    if (x) reinterpret_cast<f32x4*>(x + (long long)m * C)[c4] = o;
    const uint32_t lo = f32_to_bf16_bits(o[0]) | ((uint32_t)f32_to_bf16_bits(o[1]) << 16);
    const uint32_t hi = f32_to_bf16_bits(o[2]) | ((uint32_t)f32_to_bf16_bits(o[3]) << 16);
    *reinterpret_cast<u32x2*>(xb + drow * C + 4 * c4) = u32x2{lo, hi};
  };
  if constexpr (V > 0) {
    f32x4 v[V];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int c4 = lane + 64 * i;
      v[i] = c4 < n4 ? row[c4] : f32x4{0.f, 0.f, 0.f, 0.f};
      s += hsum(v[i]);
    }
    const float mu = wave_sum(s) / (float)C;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      if (lane + 64 * i < n4) {
        const f32x4 t = v[i] - mu;
        q += hsum(t * t);
      }
    }
    const float rs = 1.f / sqrtf(wave_sum(q) / (float)C + 1e-5f);
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (lane + 64 * i < n4) emit(lane + 64 * i, v[i], mu, rs);
  } else {
    float s = 0.f;
    for (int c4 = lane; c4 < n4; c4 += 64) s += hsum(row[c4]);
    const float mu = wave_sum(s) / (float)C;
    float q = 0.f;
    for (int c4 = lane; c4 < n4; c4 += 64) {
      const f32x4 t = row[c4] - mu;
      q += hsum(t * t);
    }
    const float rs = 1.f / sqrtf(wave_sum(q) / (float)C + 1e-5f);
    for (int c4 = lane; c4 < n4; c4 += 64) emit(c4, row[c4], mu, rs);
  }
}

// The compact slot list: crop b's n_b prompted rows (any mask set) give the
// 2 n_b compact rows off[b] .. off[b+1] - 1, the visual slots (slot r) of
// those rows in row order, then their text slots (slot R + r); cmap and
// smap give each compact row's crop and slot, off[B] the row count. One
// workgroup of 16 waves: per-crop counts by wave ballots (kept in off[]),
// an exclusive scan over crops in chunks of 1024 with a running carry,
// then each wave lists its crops' rows in order (ballot prefix counts).
__global__ __launch_bounds__(1024) void kg_compact_kernel(const uint8_t* mv, const uint8_t* mt,
                                                          int B, int R, int* off, int* cmap,
                                                          int* smap) {
  __shared__ int s_scan[1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto prompted = [&](int b, int r) {
    const long long o = (long long)b * R + r;
    return r < R && ((mv && mv[o]) || (mt && mt[o]));
  };
  for (int b = wave; b < B; b += 16) {
    int n = 0;
    for (int r0 = 0; r0 < R; r0 += 64) n += __popcll(__ballot(prompted(b, r0 + lane)));
    if (lane == 0) off[b] = n;
  }
  __syncthreads();  // counts in off[] (workgroup-visible)
  int carry = 0;
  for (int b0 = 0; b0 < B; b0 += 1024) {
    const int b = b0 + tid;
    const int n = b < B ? off[b] : 0;
    s_scan[tid] = n;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int add = tid >= d ? s_scan[tid - d] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    if (b < B) off[b] = 2 * (carry + s_scan[tid] - n);
    carry += s_scan[1023];
    __syncthreads();  // s_scan is rewritten by the next chunk
  }
  if (tid == 0) off[B] = 2 * carry;
  __syncthreads();  // starts in off[]
  for (int b = wave; b < B; b += 16) {
    const int start = off[b], n = (off[b + 1] - start) / 2;
    int j = 0;
    for (int r0 = 0; r0 < R; r0 += 64) {
      const int r = r0 + lane;
      const bool pr = prompted(b, r);
      const unsigned long long msk = __ballot(pr);
      if (pr) {
        const int k = start + j + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(msk >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)msk, 0u));
        cmap[k] = b;
        smap[k] = r;
        cmap[k + n] = b;
        smap[k + n] = R + r;
      }
      j += __popcll(msk);
    }
  }
}

// The compact input rows, one wave a row: slot r < R of crop b holds its
// visual prototype (slot R + r its text prototype), or the mask token where
// the row has no prompt of that kind; 16 bytes (8 channels) a lane.
__global__ __launch_bounds__(256) void kg_assemble_kernel(const uint16_t* vis, const uint8_t* mv,
                                                          const uint16_t* txt, const uint8_t* mt,
                                                          const uint16_t* tok, int R, int C,
                                                          const int* m_dev, const int* cmap,
                                                          const int* smap, float* x,
                                                          uint16_t* xb) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= *m_dev) return;
  const int b = cmap[m], sl = smap[m];
  const int r = sl < R ? sl : sl - R;
  const long long row = (long long)b * R + r;
  const bool have = sl < R ? (mv && mv[row]) : (mt && mt[row]);
  const uint16_t* src = have ? (sl < R ? vis : txt) + row * C : tok;
  for (int c8 = lane; c8 < C / 8; c8 += 64) {
    const u32x4 v = reinterpret_cast<const u32x4*>(src)[c8];
    reinterpret_cast<u32x4*>(xb + (long long)m * C)[c8] = v;
    f32x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      lo[2 * e] = bf16_bits_to_f32((uint16_t)(v[e] & 0xffffu));
      lo[2 * e + 1] = bf16_bits_to_f32((uint16_t)(v[e] >> 16));
      hi[2 * e] = bf16_bits_to_f32((uint16_t)(v[e + 2] & 0xffffu));
      hi[2 * e + 1] = bf16_bits_to_f32((uint16_t)(v[e + 2] >> 16));
    }
    f32x4* xr = reinterpret_cast<f32x4*>(x + (long long)m * C) + 2 * c8;
    xr[0] = lo;
    xr[1] = hi;
  }
}

// [B, C, HW] -> [B, HW, C] (bfloat16), 64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void kg_tokens_kernel(const uint16_t* src, int C, int HW,
                                                        uint16_t* dst) {
  __shared__ uint16_t tile[64][66];
  const int p0 = blockIdx.x * 64, c0 = blockIdx.y * 64, b = blockIdx.z;
  const int t = threadIdx.x, col = t & 63, r0 = t >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int cl = 4 * i + r0;
    if (p0 + col < HW) tile[cl][col] = src[((long long)b * C + c0 + cl) * HW + p0 + col];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int pl = 4 * i + r0;
    if (p0 + pl < HW) dst[((long long)b * HW + p0 + pl) * C + c0 + col] = tile[col][pl];
  }
}

size_t al256(size_t n) { return (n + 255) & ~(size_t)255; }

struct KgWorkspace {
  int *off, *cmap, *smap;
  float *x, *y;
  uint16_t *xb, *qk, *kv, *ao, *hh, *fq;
  size_t bytes;
};

KgWorkspace carve(uint8_t* base, int B, int C, int HW, int R, int F, bool tokens) {
  const size_t M = (size_t)B * 2 * R;
  KgWorkspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += al256(bytes);
    return p;
  };
  w.off = reinterpret_cast<int*>(take(((size_t)B + 1) * 4));
  w.cmap = reinterpret_cast<int*>(take(M * 4));
  w.smap = reinterpret_cast<int*>(take(M * 4));
  w.x = reinterpret_cast<float*>(take(M * C * 4));
  w.y = reinterpret_cast<float*>(take(M * C * 4));
  w.xb = reinterpret_cast<uint16_t*>(take(M * C * 2));
  w.qk = reinterpret_cast<uint16_t*>(take(M * 2 * C * 2));
  w.kv = reinterpret_cast<uint16_t*>(take((size_t)B * HW * 2 * C * 2));
  w.ao = reinterpret_cast<uint16_t*>(take(M * C * 2));
  w.hh = reinterpret_cast<uint16_t*>(take(M * F * 2));
  w.fq = tokens ? nullptr : reinterpret_cast<uint16_t*>(take((size_t)B * HW * C * 2));
  w.bytes = off;
  return w;
}

hipError_t gemm(const uint16_t* A, long long a_bstride, int a_rows, int lda, const uint16_t* W,
                const uint16_t* bias, int M, const int* m_dev, int N, int K, int mode,
                uint16_t* out_bf, float* out_f, const float* res, int ldo, int tsplit,
                hipStream_t st, uint16_t* out2 = nullptr, int ld2 = 0) {
  GemmParams p{A, a_bstride, a_rows, lda, W, bias, M, N, K, m_dev, mode, out_bf, out_f, res, ldo,
               tsplit, out2, ld2};
  // the wide tile where N fills it, else 128 columns
  if (N % 256 == 0) {
    const int tiles = ((M + kGM - 1) / kGM) * (N / 256);
    hipLaunchKernelGGL((kg_gemm_kernel<256, kGemmBK, kGemmNS>), dim3(tiles), dim3(512),
                       (gemm_lds_bytes<256, kGemmBK, kGemmNS>()), st, p);
  } else {
    const int tiles = ((M + kGM - 1) / kGM) * ((N + 127) / 128);
    hipLaunchKernelGGL((kg_gemm_kernel<128, kGemmBK, kGemmNS>), dim3(tiles), dim3(512),
                       (gemm_lds_bytes<128, kGemmBK, kGemmNS>()), st, p);
  }
  return hipGetLastError();
}

// tk_max: the most keys a crop can have (self-attention: 2R; cross: HW)
hipError_t attn(const AttnParams& p, int B, int tk_max, hipStream_t st) {
  if (p.Tk > 0)
    hipLaunchKernelGGL(kg_xattn_kernel, dim3(B * p.nh), dim3(64 * kXaWaves),
                       kXaStages * kXaStage, st, p);
  else if (tk_max <= 160)
    hipLaunchKernelGGL(kg_attn_kernel<10>, dim3(B * p.nh), dim3(64 * attn_waves<10>()),
                       attn_lds_bytes(tk_max), st, p);
  else
    hipLaunchKernelGGL(kg_attn_kernel<kKeyTiles>, dim3(B * p.nh), dim3(64 * attn_waves<kKeyTiles>()),
                       attn_lds_bytes(tk_max), st, p);
  return hipGetLastError();
}

hipError_t layernorm(const float* y, const uint16_t* w, const uint16_t* b, int M,
                     const int* m_dev, int C, int B, int R, const int* cmap, const int* smap,
                     float* x, uint16_t* xb, hipStream_t st) {
  if (C <= 1024)
    hipLaunchKernelGGL(kg_layernorm_kernel<4>, dim3((M + 3) / 4), dim3(256), 0, st, y, w, b, m_dev,
                       C, B, R, cmap, smap, x, xb);
  else if (C <= 2048)
    hipLaunchKernelGGL(kg_layernorm_kernel<8>, dim3((M + 3) / 4), dim3(256), 0, st, y, w, b, m_dev,
                       C, B, R, cmap, smap, x, xb);
  else
    hipLaunchKernelGGL(kg_layernorm_kernel<0>, dim3((M + 3) / 4), dim3(256), 0, st, y, w, b, m_dev,
                       C, B, R, cmap, smap, x, xb);
  return hipGetLastError();
}

}  // namespace

size_t kg_workspace_bytes(int B, int C, int H, int W, int R, int d_ff, bool tokens) {
  return carve(nullptr, B, C, H * W, R, d_ff, tokens).bytes;
}

hipError_t launch_kg(const KgArgs& a, hipStream_t st) {
  const int C = a.C, F = a.d_ff, R = a.R, HW = a.H * a.W, T = 2 * R, nh = C / kHd;
  const int M = a.B * T;  // rows the grids cover; the compact count off[B] bounds the work
  const KgWorkspace w = carve(static_cast<uint8_t*>(a.ws), a.B, C, HW, R, F, a.tokens);
  const int* mc = w.off + a.B;
  const uint16_t* wts = static_cast<const uint16_t*>(a.weights);
  const uint16_t* tok = wts;
  const size_t blk = (size_t)8 * C * C + (size_t)2 * F * C + (size_t)15 * C + F;

  hipError_t e;
  hipLaunchKernelGGL(kg_compact_kernel, dim3(1), dim3(1024), 0, st, a.mv, a.mt, a.B, R, w.off,
                     w.cmap, w.smap);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    hipLaunchKernelGGL(kg_assemble_kernel, dim3((M + 3) / 4), dim3(256), 0, st,
                       static_cast<const uint16_t*>(a.vis), a.mv, static_cast<const uint16_t*>(a.txt),
                       a.mt, tok, R, C, mc, w.cmap, w.smap, w.x, w.xb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // The query features as a token matrix [B * HW, C] (read in place when
  // they already are tokens).
  const uint16_t* fq;
  long long fq_bstride;
  if (a.tokens) {
    fq = static_cast<const uint16_t*>(a.query) + (size_t)a.tok_skip * C;
    fq_bstride = (long long)(a.tok_skip + HW) * C;
  } else {
    hipLaunchKernelGGL(kg_tokens_kernel, dim3((HW + 63) / 64, C / 64, a.B), dim3(256), 0, st,
                       static_cast<const uint16_t*>(a.query), C, HW, w.fq);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    fq = w.fq;
    fq_bstride = (long long)HW * C;
  }

  for (int l = 0; l < a.n_blocks; ++l) {
    const uint16_t* p = wts + C + l * blk;
    const uint16_t* sa_in_w = p;          p += (size_t)3 * C * C;
    const uint16_t* sa_in_b = p;          p += 3 * C;
    const uint16_t* sa_out_w = p;         p += (size_t)C * C;
    const uint16_t* sa_out_b = p;         p += C;
    const uint16_t* ln1_w = p;            p += C;
    const uint16_t* ln1_b = p;            p += C;
    const uint16_t* ca_in_w = p;          p += (size_t)3 * C * C;
    const uint16_t* ca_in_b = p;          p += 3 * C;
    const uint16_t* ca_out_w = p;         p += (size_t)C * C;
    const uint16_t* ca_out_b = p;         p += C;
    const uint16_t* ln2_w = p;            p += C;
    const uint16_t* ln2_b = p;            p += C;
    const uint16_t* ff1_w = p;            p += (size_t)F * C;
    const uint16_t* ff1_b = p;            p += F;
    const uint16_t* ff2_w = p;            p += (size_t)C * F;
    const uint16_t* ff2_b = p;            p += C;
    const uint16_t* ln3_w = p;            p += C;
    const uint16_t* ln3_b = p;
    const bool last = l + 1 == a.n_blocks;

    // self-attention over the compact slots: [Q|K] rows, and V rows in the
    // attention output buffer (each (crop, head) workgroup stages its V
    // columns in LDS before it writes the same columns); keys = the crop's
    // own slots
    if ((e = gemm(w.xb, 0, M, C, sa_in_w, sa_in_b, M, mc, 3 * C, C, kOutBf16, w.qk, nullptr,
                  nullptr, 2 * C, 2 * C, st, w.ao, C)) != hipSuccess) return e;
    {
      AttnParams ap{w.qk, 2 * C, w.qk + C, 2 * C, w.ao, C, w.off, w.ao, C, nh, 0};
      if ((e = attn(ap, a.B, T, st)) != hipSuccess) return e;
    }
    if ((e = gemm(w.ao, 0, M, C, sa_out_w, sa_out_b, M, mc, C, C, kOutResF32, nullptr, w.y, w.x,
                  C, C, st)) != hipSuccess) return e;
    if ((e = layernorm(w.y, ln1_w, ln1_b, M, mc, C, a.B, 0, w.cmap, w.smap, w.x, w.xb, st)) !=
        hipSuccess) return e;
    // cross-attention to the query features: [K|V] rows of every token
    if ((e = gemm(w.xb, 0, M, C, ca_in_w, ca_in_b, M, mc, C, C, kOutBf16, w.qk, nullptr, nullptr,
                  C, C, st)) != hipSuccess) return e;
    if ((e = gemm(fq, fq_bstride, HW, C, ca_in_w + (size_t)C * C, ca_in_b + C, a.B * HW, nullptr,
                  2 * C, C, kOutBf16, w.kv, nullptr, nullptr, 2 * C, 2 * C, st)) != hipSuccess)
      return e;
    {
      AttnParams ap{w.qk, C, w.kv, 2 * C, w.kv + C, 2 * C, w.off, w.ao, C, nh, HW};
      if ((e = attn(ap, a.B, HW, st)) != hipSuccess) return e;
    }
    if ((e = gemm(w.ao, 0, M, C, ca_out_w, ca_out_b, M, mc, C, C, kOutResF32, nullptr, w.y, w.x,
                  C, C, st)) != hipSuccess) return e;
    if ((e = layernorm(w.y, ln2_w, ln2_b, M, mc, C, a.B, 0, w.cmap, w.smap, w.x, w.xb, st)) !=
        hipSuccess) return e;
    // feed-forward
    if ((e = gemm(w.xb, 0, M, C, ff1_w, ff1_b, M, mc, F, C, kOutBf16Relu, w.hh, nullptr, nullptr,
                  F, F, st)) != hipSuccess) return e;
    if ((e = gemm(w.hh, 0, M, F, ff2_w, ff2_b, M, mc, C, F, kOutResF32, nullptr, w.y, w.x, C, C,
                  st)) != hipSuccess) return e;
    if ((e = layernorm(w.y, ln3_w, ln3_b, M, mc, C, a.B, last ? R : 0, w.cmap, w.smap,
                       last ? nullptr : w.x, last ? static_cast<uint16_t*>(a.out) : w.xb, st)) !=
        hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gkd
