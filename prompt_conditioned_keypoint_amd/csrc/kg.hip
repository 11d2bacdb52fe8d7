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
#include "launch.hpp"

namespace gkd {
namespace {

constexpr int kHd = 64;          // head width
constexpr int kMaxKeys = 576;    // attention keys held in registers (36 tiles of 16)
constexpr int kKeyTiles = kMaxKeys / 16;
constexpr int kPPitch = kMaxKeys + 8;  // bf16 per LDS row of probabilities (16-B rows)
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
// Attention of Tq queries over Tk <= 576 keys for one (crop, head): each
// wave takes 16 queries, holds their 16 x Tk scores in registers (36 MFMA
// tiles), takes the softmax with the 1/sqrt(64) scale, writes the
// unnormalised probabilities to LDS in bfloat16, multiplies them by V^T and
// divides by the row sums. Keys with key_ok == 0 get probability 0; a row
// without an allowed key gives 0.
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
  int nh, Tq, Tk, qtiles;
};

__global__ __launch_bounds__(256) void kg_attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sP[4][16 * kPPitch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qt = blockIdx.x % p.qtiles, bh = blockIdx.x / p.qtiles;
  const int h = bh % p.nh, b = bh / p.nh;
  const int q0 = qt * 64 + wave * 16;
  const int fr = lane & 15, g = lane >> 4, fk = g * 8;
  const int nt = (p.Tk + 15) >> 4, kpad = rup32(p.Tk);

  const uint16_t* qrow = p.q + (long long)(b * p.Tq + min(q0 + fr, p.Tq - 1)) * p.ldq + h * kHd + fk;
  const bf16x8 qa0 = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow));
  const bf16x8 qa1 = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 32));

  f32x4 s[kKeyTiles];
  float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  uint32_t okbits[2] = {0u, 0u};  // bit t: this lane's key of tile t is allowed
#pragma unroll
  for (int t = 0; t < kKeyTiles; ++t) {
    if (t < nt) {
      const int key = t * 16 + fr;
      const uint16_t* krow = p.k + (long long)(b * p.Tk + min(key, p.Tk - 1)) * p.ldk + h * kHd + fk;
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa0, as_bf16x8(*reinterpret_cast<const u32x4*>(krow)), z, 0, 0, 0);
      s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa1, as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 32)), z, 0, 0, 0);
      const bool ok = key < p.Tk && (!p.key_ok || p.key_ok[(long long)b * p.Tk + key]);
      if (ok) {
        okbits[t >> 5] |= 1u << (t & 31);
#pragma unroll
        for (int e = 0; e < 4; ++e) mx[e] = fmaxf(mx[e], s[t][e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], d));

  // p = exp((s - max) / 8) = exp2((s - max) * log2(e) / 8)
  constexpr float kScale = 0.125f * 1.4426950408889634f;
  float sum[4] = {0.f, 0.f, 0.f, 0.f};
  uint16_t* myP = sP[wave];
#pragma unroll
  for (int t = 0; t < kKeyTiles; ++t) {
    if (t < nt) {
      const bool ok = (okbits[t >> 5] >> (t & 31)) & 1u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = ok ? exp2f((s[t][e] - mx[e]) * kScale) : 0.f;
        const uint16_t hb = f32_to_bf16_bits(v);
        sum[e] += bf16_bits_to_f32(hb);  // the sum of what the product uses
        myP[(4 * g + e) * kPPitch + t * 16 + fr] = hb;
      }
    } else if (t * 16 < kpad) {
#pragma unroll
      for (int e = 0; e < 4; ++e) myP[(4 * g + e) * kPPitch + t * 16 + fr] = 0;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) sum[e] += __shfl_xor(sum[e], d);
  __syncthreads();

  f32x4 o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* vbase = p.vt + (long long)(b * p.nh + h) * kHd * p.vt_ld;
  for (int k0 = 0; k0 < kpad; k0 += 32) {
    const bf16x8 pa = as_bf16x8(*reinterpret_cast<const u32x4*>(&myP[fr * kPPitch + k0 + fk]));
    const int kb = k0 + fk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t* vrow = vbase + (long long)(16 * j + fr) * p.vt_ld;
      u32x4 v;
      if (kb + 8 <= p.Tk) {
        v = *reinterpret_cast<const u32x4*>(vrow + kb);
      } else {  // ragged key tail: keys past Tk contribute 0 (their p is 0 too)
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = kb + 2 * e < p.Tk ? vrow[kb + 2 * e] : 0u;
          const uint32_t hi = kb + 2 * e + 1 < p.Tk ? vrow[kb + 2 * e + 1] : 0u;
          w[e] = lo | (hi << 16);
        }
        v = u32x4{w[0], w[1], w[2], w[3]};
      }
      o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf16x8(v), o[j], 0, 0, 0);
    }
  }
  // o[j][e] = O[query q0 + 4 g + e][dim 16 j + fr]
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int qi = q0 + 4 * g + e;
    if (qi >= p.Tq) continue;
    const float inv = sum[e] > 0.f ? 1.f / sum[e] : 0.f;
    uint16_t* orow = p.out + (long long)(b * p.Tq + qi) * p.ldo + h * kHd;
#pragma unroll
    for (int j = 0; j < 4; ++j) orow[16 * j + fr] = f32_to_bf16_bits(o[j][e] * inv);
  }
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
  const int qtiles = (Tq + 63) / 64;
  AttnParams p{q, ldq, k, ldk, vt, vt_ld, key_ok, out, ldo, nh, Tq, Tk, qtiles};
  hipLaunchKernelGGL(kg_attn_kernel, dim3(B * nh * qtiles), dim3(256), 0, st, p);
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
