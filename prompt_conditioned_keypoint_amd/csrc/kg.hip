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
// bfloat16 throughout for matrix operands (weights, prototypes, features,
// and every activation that feeds a product), float32 for accumulation, the
// residual stream, softmax and LayerNorm. Per block:
//   gemm   x -> [Q|K] rows and V^T per head        (SA in_proj)
//   attn   softmax(Q K^T / 8) V, scores in registers
//   gemm   out_proj + bias + residual (float32)    -> LayerNorm
//   gemm   x -> Q (CA), gemm F -> [K] rows and V^T (CA in_proj)
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
constexpr int kGT = 128;         // GEMM tile (M and N)
constexpr int kGK = 64;          // GEMM K step
constexpr int kGPitch = kGK + 8; // bf16 per LDS tile row (16-B aligned, skewed banks)

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
// Epilogues: kOutBf16 (optionally ReLU); columns >= tsplit go to vt
// transposed per head, vt[((b * nh + h) * 64 + d) * vt_ld + p] with
// b = m / t_rows, p = m % t_rows; kOutResF32: float32 acc + bias + res.
// ---------------------------------------------------------------------------
enum { kOutBf16 = 0, kOutBf16Relu = 1, kOutResF32 = 2 };

struct GemmParams {
  const uint16_t* A;
  long long a_bstride;
  int a_rows, lda;
  const uint16_t* W;
  const uint16_t* bias;
  int M, N, K;
  int mode;
  uint16_t* out_bf;
  float* out_f;
  const float* res;
  int ldo;
  int tsplit;
  uint16_t* vt;
  int t_rows, vt_ld, nh;
};

__global__ __launch_bounds__(256) void kg_gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kGT * kGPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kGT * kGPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_n = (p.N + kGT - 1) / kGT;
  const int total = gridDim.x;
  int lin = blockIdx.x;
  // Workgroups are dealt round-robin over the 8 XCDs; give each XCD a
  // contiguous run of tiles so the N-tiles of one A row band share an L2.
  if ((total & (kXcds - 1)) == 0) lin = (lin % kXcds) * (total / kXcds) + lin / kXcds;
  const int m0 = (lin / tiles_n) * kGT, n0 = (lin % tiles_n) * kGT;

  // Each thread moves 4 A and 4 W chunks of 16 B per K step:
  // chunk c = tid + 256 i -> tile row c >> 3, 8-element column group c & 7.
  const uint16_t* arow[4];
  const uint16_t* wrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, r = c >> 3, cg = (c & 7) * 8;
    const int m = min(m0 + r, p.M - 1), n = min(n0 + r, p.N - 1);
    arow[i] = p.A + (long long)(m / p.a_rows) * p.a_bstride + (long long)(m % p.a_rows) * p.lda + cg;
    wrow[i] = p.W + (long long)n * p.K + cg;
  }
  u32x4 ra[4], rw[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const u32x4*>(arow[i] + k0);
      rw[i] = *reinterpret_cast<const u32x4*>(wrow[i] + k0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, off = (c >> 3) * kGPitch + (c & 7) * 8;
      *reinterpret_cast<u32x4*>(&sA[buf][off]) = ra[i];
      *reinterpret_cast<u32x4*>(&sB[buf][off]) = rw[i];
    }
  };

  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / kGK;
  load(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * kGK);
#pragma unroll
    for (int ks = 0; ks < kGK; ks += 32) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sA[cur][(wm + 16 * i + fr) * kGPitch + ks + fk]));
        b[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sB[cur][(wn + 16 * i + fr) * kGPitch + ks + fk]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) stash(cur ^ 1);
    __syncthreads();
  }

  // acc[i][j][e] holds C[m0 + wm + 16 i + 4 (lane >> 4) + e][n0 + wn + 16 j + (lane & 15)].
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn + 16 * j + fr;
    if (n >= p.N) continue;
    const float bias = bf(p.bias, n);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm + 16 * i + 4 * (lane >> 4) + e;
        if (m >= p.M) continue;
        float v = acc[i][j][e] + bias;
        if (p.mode == kOutResF32) {
          const long long o = (long long)m * p.ldo + n;
          p.out_f[o] = v + p.res[o];
        } else {
          if (p.mode == kOutBf16Relu) v = fmaxf(v, 0.f);
          if (n < p.tsplit) {
            p.out_bf[(long long)m * p.ldo + n] = f32_to_bf16_bits(v);
          } else {
            const int c = n - p.tsplit, b = m / p.t_rows, t = m % p.t_rows;
            p.vt[((long long)(b * p.nh + (c >> 6)) * kHd + (c & 63)) * p.vt_ld + t] =
                f32_to_bf16_bits(v);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Attention of Tq queries over Tk <= 576 keys for one (crop, head), one
// workgroup of 4 waves per (crop, head): K [Tk, 64] and V^T [64, Tk] of the
// head are staged in LDS once (keys past Tk read as 0) and every wave reads
// them there. A wave takes 16 queries at a time and computes the transposed scores S^T = K Q^T, so
// lane (query n = lane & 15, group g = lane >> 4) holds keys 16 t + 4 g + e
// (e = 0..3) of its query in tile t: 36 tiles cover 576 keys in registers.
// Softmax (scale 1/sqrt(64)) reduces over e, t and the 4 lane groups. The
// product O^T = V^T P^T then takes its P^T operand straight from those
// registers: an MFMA sums over its 32 k-slots in any order as long as both
// operands agree, so k-slots 8 g .. 8 g + 7 of a 32-key chunk c carry keys
// 32 c + 4 g + (0..3) and 32 c + 16 + 4 g + (0..3) on both sides. Keys with
// key_ok == 0 get probability 0; a query without an allowed key gives 0.
// ---------------------------------------------------------------------------
struct AttnParams {
  const uint16_t* q;
  int ldq;
  const uint16_t* k;
  int ldk;
  const uint16_t* vt;
  int vt_ld;
  const uint8_t* key_ok;  // [B, Tk], or null: every key
  uint16_t* out;
  int ldo;
  int nh, Tq, Tk;
};

constexpr int kAttnWaves = 4;
constexpr int kKPitch = kHd + 8;  // bf16 per LDS row of K (16-B rows, skewed banks)

__host__ __device__ inline int attn_vpitch(int Tk) { return rup32(Tk) + 8; }
__host__ __device__ inline size_t attn_lds_bytes(int Tk) {
  return (size_t)((Tk + 15) & ~15) * kKPitch * 2 + (size_t)kHd * attn_vpitch(Tk) * 2;
}

// bfloat16 bits of a float, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// NT: key tiles held in registers (10 covers 160 keys, 36 covers 576).
template <int NT>
__global__ __launch_bounds__(64 * kAttnWaves) void kg_attn_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_kv[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x % p.nh, b = blockIdx.x / p.nh;
  const int fr = lane & 15, g = lane >> 4, fk = g * 8;
  const int nt = (p.Tk + 15) >> 4, kpad = rup32(p.Tk), vp = attn_vpitch(p.Tk);
  uint16_t* sK = lds_kv;
  uint16_t* sV = lds_kv + (size_t)nt * 16 * kKPitch;

  // Stage K (rows of 8 16-byte pieces) and V^T (64 rows of kpad keys).
  for (int c = tid; c < p.Tk * 8; c += 64 * kAttnWaves) {
    const int key = c >> 3, piece = (c & 7) * 8;
    *reinterpret_cast<u32x4*>(&sK[key * kKPitch + piece]) = *reinterpret_cast<const u32x4*>(
        p.k + (long long)(b * p.Tk + key) * p.ldk + h * kHd + piece);
  }
  const uint16_t* vsrc = p.vt + (long long)(b * p.nh + h) * kHd * p.vt_ld;
  for (int c = tid; c < kHd * (kpad / 8); c += 64 * kAttnWaves) {
    const int d = c / (kpad / 8), k8 = (c % (kpad / 8)) * 8;
    const uint16_t* src = vsrc + (long long)d * p.vt_ld + k8;
    u32x4 v;
    if (k8 + 8 <= p.Tk) {
      v = *reinterpret_cast<const u32x4*>(src);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (k8 + 2 * e < p.Tk ? (uint32_t)src[2 * e] : 0u) |
               ((k8 + 2 * e + 1 < p.Tk ? (uint32_t)src[2 * e + 1] : 0u) << 16);
      v = u32x4{w[0], w[1], w[2], w[3]};
    }
    *reinterpret_cast<u32x4*>(&sV[d * vp + k8]) = v;
  }
  __syncthreads();

  for (int q0 = wave * 16; q0 < p.Tq; q0 += 16 * kAttnWaves) {

  const uint16_t* qrow = p.q + (long long)(b * p.Tq + min(q0 + fr, p.Tq - 1)) * p.ldq + h * kHd + fk;
  const bf16x8 qb0 = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow));
  const bf16x8 qb1 = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 32));
  const uint8_t* okrow = p.key_ok ? p.key_ok + (long long)b * p.Tk : nullptr;

  f32x4 s[NT];
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < nt) {
      const uint16_t* krow = sK + (t * 16 + fr) * kKPitch + fk;  // rows past Tk: masked below
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(krow)), qb0, z, 0, 0, 0);
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 32)), qb1, z, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = t * 16 + 4 * g + e;
        const bool ok = key < p.Tk && (!okrow || okrow[key]);
        z[e] = ok ? z[e] : -INFINITY;
        mx = fmaxf(mx, z[e]);
      }
      s[t] = z;
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));

  // p = exp((s - max) / 8) = exp2((s - max) * log2(e) / 8); masked keys hold
  // -inf and give 0, and so does every key of a query with no allowed key.
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
  const uint16_t* vbase = sV + 4 * g;
#pragma unroll
  for (int c = 0; c < (NT + 1) / 2; ++c) {
    if (2 * c < nt) {
      const bf16x8 pb = as_bf16x8(u32x4{pk[2 * c][0], pk[2 * c][1], pk[2 * c + 1][0], pk[2 * c + 1][1]});
      const int k0 = 32 * c;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint16_t* vrow = vbase + (16 * j + fr) * vp + k0;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
        const bf16x8 va = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[j], 0, 0, 0);
      }
    }
  }
  // o[j][e] = O^T[dim 16 j + 4 g + e][query q0 + fr]
  const int qi = q0 + fr;
  if (qi < p.Tq) {
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    uint16_t* orow = p.out + (long long)(b * p.Tq + qi) * p.ldo + h * kHd + 4 * g;
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
// LayerNorm of float32 rows (one wave per row, eps 1e-5, biased variance):
// writes the float32 result (the residual stream) and its bfloat16 copy.
// With R > 0 the bfloat16 rows go to the two-plane output instead: slot s
// of crop b lands in row (s / R) * B + b, s % R of plane-major [2, B, R, C].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kg_layernorm_kernel(const float* y, const uint16_t* w,
                                                           const uint16_t* bvec, int M, int C,
                                                           int B, int R, float* x, uint16_t* xb) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const float* row = y + (long long)m * C;
  float s = 0.f;
  for (int c = lane; c < C; c += 64) s += row[c];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) s += __shfl_xor(s, d);
  const float mu = s / (float)C;
  float v = 0.f;
  for (int c = lane; c < C; c += 64) {
    const float t = row[c] - mu;
    v = fmaf(t, t, v);
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d);
  const float rs = 1.f / sqrtf(v / (float)C + 1e-5f);
  long long drow = m;
  if (R > 0) {
    const int b = m / (2 * R), s = m % (2 * R);
    drow = ((long long)(s >= R) * B + b) * R + (s >= R ? s - R : s);
  }
  for (int c = lane; c < C; c += 64) {
    const float o = fmaf((row[c] - mu) * rs, bf(w, c), bf(bvec, c));
    if (x) x[(long long)m * C + c] = o;
    xb[drow * C + c] = f32_to_bf16_bits(o);
  }
}

// The 2R input slots of every crop (prototype or mask token) and the
// self-attention key mask (a slot is a key when its row has any prompt).
__global__ void kg_assemble_kernel(const uint16_t* vis, const uint8_t* mv, const uint16_t* txt,
                                   const uint8_t* mt, const uint16_t* tok, int B, int R, int C,
                                   float* x, uint16_t* xb, uint8_t* key_ok) {
  const long long n = (long long)B * 2 * R * C;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    const int c = (int)(i % C);
    const long long bs = i / C;
    const int s = (int)(bs % (2 * R)), b = (int)(bs / (2 * R));
    const int r = s < R ? s : s - R;
    const long long row = (long long)b * R + r;
    const bool v = mv && mv[row], t = mt && mt[row];
    const bool have = s < R ? v : t;
    const uint16_t h = have ? (s < R ? vis : txt)[row * C + c] : tok[c];
    x[i] = bf16_bits_to_f32(h);
    xb[i] = h;
    if (c == 0) key_ok[bs] = (v || t) ? 1 : 0;
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
  uint8_t* key_ok;
  float *x, *y;
  uint16_t *xb, *qk, *vt, *kc, *ao, *hh, *fq;
  size_t bytes;
};

KgWorkspace carve(uint8_t* base, int B, int C, int HW, int R, int F, bool tokens) {
  const size_t M = (size_t)B * 2 * R, T = (size_t)rup32(2 * R > HW ? 2 * R : HW);
  KgWorkspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += al256(bytes);
    return p;
  };
  w.key_ok = take(M);
  w.x = reinterpret_cast<float*>(take(M * C * 4));
  w.y = reinterpret_cast<float*>(take(M * C * 4));
  w.xb = reinterpret_cast<uint16_t*>(take(M * C * 2));
  w.qk = reinterpret_cast<uint16_t*>(take(M * 2 * C * 2));
  w.vt = reinterpret_cast<uint16_t*>(take((size_t)B * C * T * 2));
  w.kc = reinterpret_cast<uint16_t*>(take((size_t)B * HW * C * 2));
  w.ao = reinterpret_cast<uint16_t*>(take(M * C * 2));
  w.hh = reinterpret_cast<uint16_t*>(take(M * F * 2));
  w.fq = tokens ? nullptr : reinterpret_cast<uint16_t*>(take((size_t)B * HW * C * 2));
  w.bytes = off;
  return w;
}

hipError_t gemm(const uint16_t* A, long long a_bstride, int a_rows, int lda, const uint16_t* W,
                const uint16_t* bias, int M, int N, int K, int mode, uint16_t* out_bf,
                float* out_f, const float* res, int ldo, int tsplit, uint16_t* vt, int t_rows,
                int vt_ld, int nh, hipStream_t st) {
  GemmParams p{A, a_bstride, a_rows, lda, W, bias, M, N, K, mode, out_bf, out_f, res, ldo,
               tsplit, vt, t_rows, vt_ld, nh};
  const int tiles = ((M + kGT - 1) / kGT) * ((N + kGT - 1) / kGT);
  hipLaunchKernelGGL(kg_gemm_kernel, dim3(tiles), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t attn(const uint16_t* q, int ldq, const uint16_t* k, int ldk, const uint16_t* vt,
                int vt_ld, const uint8_t* key_ok, uint16_t* out, int ldo, int B, int nh, int Tq,
                int Tk, hipStream_t st) {
  AttnParams p{q, ldq, k, ldk, vt, vt_ld, key_ok, out, ldo, nh, Tq, Tk};
  if (Tk <= 160)
    hipLaunchKernelGGL(kg_attn_kernel<10>, dim3(B * nh), dim3(64 * kAttnWaves), attn_lds_bytes(Tk), st, p);
  else
    hipLaunchKernelGGL(kg_attn_kernel<kKeyTiles>, dim3(B * nh), dim3(64 * kAttnWaves), attn_lds_bytes(Tk), st, p);
  return hipGetLastError();
}

hipError_t layernorm(const float* y, const uint16_t* w, const uint16_t* b, int M, int C, int B,
                     int R, float* x, uint16_t* xb, hipStream_t st) {
  hipLaunchKernelGGL(kg_layernorm_kernel, dim3((M + 3) / 4), dim3(256), 0, st, y, w, b, M, C, B, R,
                     x, xb);
  return hipGetLastError();
}

}  // namespace

size_t kg_workspace_bytes(int B, int C, int H, int W, int R, int d_ff, bool tokens) {
  return carve(nullptr, B, C, H * W, R, d_ff, tokens).bytes;
}

hipError_t launch_kg(const KgArgs& a, hipStream_t st) {
  const int C = a.C, F = a.d_ff, R = a.R, HW = a.H * a.W, T = 2 * R, nh = C / kHd;
  const int M = a.B * T;
  const KgWorkspace w = carve(static_cast<uint8_t*>(a.ws), a.B, C, HW, R, F, a.tokens);
  const uint16_t* wts = static_cast<const uint16_t*>(a.weights);
  const uint16_t* tok = wts;
  const size_t blk = (size_t)8 * C * C + (size_t)2 * F * C + (size_t)15 * C + F;
  const int vt_sa = rup32(T), vt_ca = rup32(HW);

  hipError_t e;
  {
    const long long n = (long long)M * C;
    const int grid = (int)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
    hipLaunchKernelGGL(kg_assemble_kernel, dim3(grid), dim3(256), 0, st,
                       static_cast<const uint16_t*>(a.vis), a.mv, static_cast<const uint16_t*>(a.txt),
                       a.mt, tok, a.B, R, C, w.x, w.xb, w.key_ok);
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

    // self-attention
    if ((e = gemm(w.xb, 0, M, C, sa_in_w, sa_in_b, M, 3 * C, C, kOutBf16, w.qk, nullptr, nullptr,
                  2 * C, 2 * C, w.vt, T, vt_sa, nh, st)) != hipSuccess) return e;
    if ((e = attn(w.qk, 2 * C, w.qk + C, 2 * C, w.vt, vt_sa, w.key_ok, w.ao, C, a.B, nh, T, T,
                  st)) != hipSuccess) return e;
    if ((e = gemm(w.ao, 0, M, C, sa_out_w, sa_out_b, M, C, C, kOutResF32, nullptr, w.y, w.x, C,
                  C, nullptr, 1, 1, nh, st)) != hipSuccess) return e;
    if ((e = layernorm(w.y, ln1_w, ln1_b, M, C, a.B, 0, w.x, w.xb, st)) != hipSuccess) return e;
    // cross-attention to the query features
    if ((e = gemm(w.xb, 0, M, C, ca_in_w, ca_in_b, M, C, C, kOutBf16, w.qk, nullptr, nullptr, C,
                  C, nullptr, 1, 1, nh, st)) != hipSuccess) return e;
    if ((e = gemm(fq, fq_bstride, HW, C, ca_in_w + (size_t)C * C, ca_in_b + C, a.B * HW, 2 * C,
                  C, kOutBf16, w.kc, nullptr, nullptr, C, C, w.vt, HW, vt_ca, nh, st)) !=
        hipSuccess) return e;
    if ((e = attn(w.qk, C, w.kc, C, w.vt, vt_ca, nullptr, w.ao, C, a.B, nh, T, HW, st)) !=
        hipSuccess) return e;
    if ((e = gemm(w.ao, 0, M, C, ca_out_w, ca_out_b, M, C, C, kOutResF32, nullptr, w.y, w.x, C,
                  C, nullptr, 1, 1, nh, st)) != hipSuccess) return e;
    if ((e = layernorm(w.y, ln2_w, ln2_b, M, C, a.B, 0, w.x, w.xb, st)) != hipSuccess) return e;
    // feed-forward
    if ((e = gemm(w.xb, 0, M, C, ff1_w, ff1_b, M, F, C, kOutBf16Relu, w.hh, nullptr, nullptr, F,
                  F, nullptr, 1, 1, nh, st)) != hipSuccess) return e;
    if ((e = gemm(w.hh, 0, M, F, ff2_w, ff2_b, M, C, F, kOutResF32, nullptr, w.y, w.x, C, C,
                  nullptr, 1, 1, nh, st)) != hipSuccess) return e;
    if ((e = layernorm(w.y, ln3_w, ln3_b, M, C, a.B, last ? R : 0, last ? nullptr : w.x,
                       last ? static_cast<uint16_t*>(a.out) : w.xb, st)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gkd
