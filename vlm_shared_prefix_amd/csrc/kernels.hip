// Device kernels for shared-prefix candidate scoring on gfx950 (CDNA4).
//
// Precision scheme (bf16 models): weights bfloat16; activations and the
// residual stream float32; GEMM activations enter the matrix cores as two
// bfloat16 terms (hi + lo, hi = bf16(a), lo = bf16(a - hi)), so a GEMM is
// W·hi + W·lo with float32 accumulation; q/k/v and the KV store are float16
// and attention runs on float16 MFMA with float32 softmax; norms, softmax
// merge and readout are float32.  float32 models run every step in float32.
#include <hip/hip_runtime.h>
#include <climits>
#include <stdint.h>
#include <math.h>

#include <algorithm>

#include "kernels.h"

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

#define NEG_INF (-__builtin_inff())

namespace jevk {

// ----------------------------------------------------------------------------
// scalar helpers
// ----------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(u16 b) { return __uint_as_float(((uint32_t)b) << 16); }

// round-to-nearest-even float32 -> bfloat16 bits (finite inputs)
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

template <typename WT> __device__ __forceinline__ float ldw(const WT* p, size_t i);
typedef u16 u16x8_t __attribute__((ext_vector_type(8)));
template <> __device__ __forceinline__ float ldw<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ldw<u16>(const u16* p, size_t i) { return bf16_to_f32(p[i]); }

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Range flag of the float16 activation planes: bit 0 of *flags is set when a value written
// to a float16 plane lies outside the float16 range (|v| > 65504) or is not finite.
__device__ __forceinline__ bool f16_out_of_range(float v) { return !(fabsf(v) <= 65504.f); }
__device__ __forceinline__ void flag_f16_range(int* flags, bool bad) {
  if (bad && flags) atomicOr(flags, 1);
}

// block of 256 threads: sum over the block, result broadcast to all threads
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// ----------------------------------------------------------------------------
// K1: embedding rows.  Row t with tok[t] >= 0 gathers E[tok[t]]; tok[t] = -1 - j copies
// the given embedding row vis[j] (a visual token).
// ----------------------------------------------------------------------------
template <typename WT>
__global__ void __launch_bounds__(256) embed_rows(const WT* __restrict__ E, const int* __restrict__ tok, int T,
                                                  int H, const WT* __restrict__ vis, float* __restrict__ x,
                                                  int* __restrict__ flags, int vec) {
  const int t = blockIdx.x;
  if (t == 0 && threadIdx.x == 0 && flags) *flags = 0;   // the forward's range flag starts clear
  if (t >= T) return;
  const int k = tok[t];
  const WT* src = (k < 0) ? vis + (size_t)(-1 - k) * H : E + (size_t)k * H;
  float* dst = x + (size_t)t * H;
  if constexpr (sizeof(WT) == 2) {
    if (vec) {   // H % 8 == 0, rows 16 B aligned: 8 elements per thread and step
      for (int i = threadIdx.x * 8; i < H; i += 256 * 8) {
        const u16x8_t w = *reinterpret_cast<const u16x8_t*>(src + i);
        *reinterpret_cast<float4*>(dst + i) =
            make_float4(bf16_to_f32(w[0]), bf16_to_f32(w[1]), bf16_to_f32(w[2]), bf16_to_f32(w[3]));
        *reinterpret_cast<float4*>(dst + i + 4) =
            make_float4(bf16_to_f32(w[4]), bf16_to_f32(w[5]), bf16_to_f32(w[6]), bf16_to_f32(w[7]));
      }
      return;
    }
  }
  for (int i = threadIdx.x; i < H; i += 256) dst[i] = ldw(src, i);
}

// ----------------------------------------------------------------------------
// K2: RMSNorm, y[i] = g * x[row_i] / sqrt(mean(x^2) + eps), one block per row.
// ----------------------------------------------------------------------------
template <typename WT>
__global__ void __launch_bounds__(256) rmsnorm_rows(const float* __restrict__ x, int ldx,
                                                    const int* __restrict__ rows, int n_rows, int H,
                                                    const WT* __restrict__ g, float eps,
                                                    float* __restrict__ y, u16* __restrict__ yh,
                                                    u16* __restrict__ yl, int ldy, int vec) {
  __shared__ float red[4];
  const int i = blockIdx.x;
  if (i >= n_rows) return;
  const int src = rows ? rows[i] : i;
  const float* xr = x + (size_t)src * ldx;
  float ss = 0.f;
  if (vec) {   // H, ldx, ldy % 4 == 0 and x, y, g aligned: 4 elements per thread and step
    const float4* x4 = reinterpret_cast<const float4*>(xr);
    const int H4 = H >> 2;
    for (int k = threadIdx.x; k < H4; k += 256) {
      const float4 v = x4[k];
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = block_sum256(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)H + eps);
    for (int k = threadIdx.x; k < H4; k += 256) {
      const float4 v = x4[k];
      const float xv[4] = {v.x, v.y, v.z, v.w};
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = ldw(g, 4 * k + e) * (xv[e] * r);
      if (y) *reinterpret_cast<float4*>(y + (size_t)i * ldy + 4 * k) = make_float4(o[0], o[1], o[2], o[3]);
      if (yh) {
        u16 hh[4], ll[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hh[e] = f32_to_bf16(o[e]);
          ll[e] = f32_to_bf16(o[e] - bf16_to_f32(hh[e]));
        }
        *reinterpret_cast<uint2*>(yh + (size_t)i * ldy + 4 * k) =
            make_uint2((uint32_t)hh[0] | ((uint32_t)hh[1] << 16), (uint32_t)hh[2] | ((uint32_t)hh[3] << 16));
        *reinterpret_cast<uint2*>(yl + (size_t)i * ldy + 4 * k) =
            make_uint2((uint32_t)ll[0] | ((uint32_t)ll[1] << 16), (uint32_t)ll[2] | ((uint32_t)ll[3] << 16));
      }
    }
    return;
  }
  for (int k = threadIdx.x; k < H; k += 256) { float v = xr[k]; ss += v * v; }
  ss = block_sum256(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  for (int k = threadIdx.x; k < H; k += 256) {
    const float v = ldw(g, k) * (xr[k] * r);
    if (y) y[(size_t)i * ldy + k] = v;
    if (yh) {
      const u16 h = f32_to_bf16(v);
      yh[(size_t)i * ldy + k] = h;
      yl[(size_t)i * ldy + k] = f32_to_bf16(v - bf16_to_f32(h));
    }
  }
}

// ----------------------------------------------------------------------------
// K3 (bf16 models): Y[M,N] = A[M,K] · W[N,K]^T on MFMA 32x32x16 bf16, with the
// float32 activation given as two bf16 planes (hi + lo): Y = W·hi + W·lo.
// Block tile 128x128, K step 64, 4 waves in a 2x2 arrangement (64x64 each),
// register-staged global loads.
// W is described by up to three row segments (e.g. wq | wk | wv).
// Grid: 1-D, rounded up to a multiple of 8; the linear block id is remapped so
// that blocks dispatched to the same XCD share a W tile (same N tile and K
// split, different M tiles) and reuse it from that XCD's L2.
// ----------------------------------------------------------------------------
#define GBM 128
#define GBN 128
#define GBK 64
#define GLD (GBK + 8)   // LDS row stride in bf16 elements (144 B: conflict-free 16 B reads)

// Direct global->LDS loads in the buffer form: a wave-uniform resource (base, 2 GB range),
// a 32-bit byte offset per lane and a uniform byte offset in an SGPR.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ const u16* seg_row(const GemmSegs& s, int n, int K) {
  if (n < s.n_end[0]) return s.w[0] + (size_t)n * K;
  if (n < s.n_end[1]) return s.w[1] + (size_t)(n - s.n_end[0]) * K;
  return s.w[2] + (size_t)(n - s.n_end[1]) * K;
}

// F16: the activation is one float16 plane (Ah; Al unused) against the float16 mirror of
// the weights, one f16 MFMA pass (the products whose few output columns would make the
// 128 x 256 kernel split K many ways).
template <bool F16>
__global__ void __launch_bounds__(256, 2) gemm_bf16s(const u16* __restrict__ Ah, const u16* __restrict__ Al,
                                                     int lda, int M, int K, GemmSegs seg, int N, int m_tiles,
                                                     int n_tiles, int splits, int k_chunk, float* __restrict__ C,
                                                     int ldc, size_t split_stride, int accum) {
  __shared__ __attribute__((aligned(16))) u16 sAh[GBM * GLD];
  __shared__ __attribute__((aligned(16))) u16 sAl[F16 ? 8 : GBM * GLD];
  __shared__ __attribute__((aligned(16))) u16 sW[GBN * GLD];

  const int nb = m_tiles * n_tiles * splits;
  const int per = gridDim.x >> 3;
  const int v = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (v >= nb) return;
  const int mt = v % m_tiles;
  const int rest = v / m_tiles;
  const int ks = rest % splits;
  const int nt = rest / splits;
  const int m0 = mt * GBM, n0 = nt * GBN;
  const int kbeg = ks * k_chunk;
  const int kend = min(K, kbeg + k_chunk);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int ql = lane & 31, hl = lane >> 5;
  const bool wave_active = (m0 + wm * 64) < M;
  // W row of tile row nr
  auto w_row = [&](int nr, bool& ok) -> const u16* {
    ok = n0 + nr < N;
    return seg_row(seg, ok ? n0 + nr : 0, K);
  };

  // global -> register staging; rows past M / N read row 0 and are zeroed at the LDS store
  uint4 rh[4], rl[4], rw[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx >> 3, c8 = idx & 7;
      const int gm = (m0 + row < M) ? m0 + row : 0;
      const size_t off = (size_t)gm * lda + k0 + c8 * 8;
      rh[i] = *reinterpret_cast<const uint4*>(Ah + off);
      if (!F16) rl[i] = *reinterpret_cast<const uint4*>(Al + off);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int nr = idx >> 3, c8 = idx & 7;
      bool ok;
      rw[i] = *reinterpret_cast<const uint4*>(w_row(nr, ok) + k0 + c8 * 8);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx >> 3, c8 = idx & 7;
      bool okw;
      (void)w_row(row, okw);
      const uint32_t ma = (m0 + row < M) ? 0xFFFFFFFFu : 0u;
      const uint32_t mw = okw ? 0xFFFFFFFFu : 0u;
      *reinterpret_cast<uint4*>(&sAh[row * GLD + c8 * 8]) =
          make_uint4(rh[i].x & ma, rh[i].y & ma, rh[i].z & ma, rh[i].w & ma);
      if (!F16)
        *reinterpret_cast<uint4*>(&sAl[row * GLD + c8 * 8]) =
            make_uint4(rl[i].x & ma, rl[i].y & ma, rl[i].z & ma, rl[i].w & ma);
      *reinterpret_cast<uint4*>(&sW[row * GLD + c8 * 8]) =
          make_uint4(rw[i].x & mw, rw[i].y & mw, rw[i].z & mw, rw[i].w & mw);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (kbeg < kend) {
    gload(kbeg);
    sstore();
    __syncthreads();
    for (int k0 = kbeg; k0 < kend; k0 += GBK) {
      const bool more = (k0 + GBK) < kend;
      if (more) gload(k0 + GBK);
      if (wave_active) {
#pragma unroll
        for (int kk = 0; kk < GBK / 16; ++kk) {
          if constexpr (F16) {
            f16x8 ah[2], bw[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const int r = wm * 64 + i * 32 + ql;
              ah[i] = *reinterpret_cast<const f16x8*>(&sAh[r * GLD + kk * 16 + hl * 8]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int c = wn * 64 + j * 32 + ql;
              bw[j] = *reinterpret_cast<const f16x8*>(&sW[c * GLD + kk * 16 + hl * 8]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bw[j], acc[i][j], 0, 0, 0);
          } else {
            bf16x8 ah[2], al[2], bw[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const int r = wm * 64 + i * 32 + ql;
              ah[i] = *reinterpret_cast<const bf16x8*>(&sAh[r * GLD + kk * 16 + hl * 8]);
              al[i] = *reinterpret_cast<const bf16x8*>(&sAl[r * GLD + kk * 16 + hl * 8]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int c = wn * 64 + j * 32 + ql;
              bw[j] = *reinterpret_cast<const bf16x8*>(&sW[c * GLD + kk * 16 + hl * 8]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bw[j], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bw[j], acc[i][j], 0, 0, 0);
              }
          }
        }
      }
      __syncthreads();
      if (more) {
        sstore();
        __syncthreads();
      }
    }
  }

  if (!wave_active) return;
  float* Cb = C + (splits > 1 ? (size_t)ks * split_stride : 0);
  const bool add = (splits == 1) && accum;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + ql;
      const int rbase = m0 + wm * 64 + i * 32 + 4 * hl;
      float old[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rbase + 8 * (r >> 2) + (r & 3);
        old[r] = (add && row < M && col < N) ? Cb[(size_t)row * ldc + col] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rbase + 8 * (r >> 2) + (r & 3);
        if (row < M && col < N) Cb[(size_t)row * ldc + col] = old[r] + acc[i][j][r];
      }
    }
}

// ----------------------------------------------------------------------------
// K3 wide (bf16 models): the same product on a 128 x 256 block tile, 4 waves of
// 64 x 128 (8 MFMA tiles each, half the LDS bytes per MFMA of the 64 x 64 wave
// tile), K stages of 32 staged by direct global->LDS loads into a ring of buffers
// (one float16 plane: three, the next two stages in flight while the current one is
// multiplied; two bf16 planes: two).  LDS rows are
// 64 B with the 16 B chunk c of row r at position c ^ ((r / 4) % 4), which makes
// the operand reads bank-conflict free.  All hi-plane MFMAs of a k-step are
// issued before the lo-plane ones, so no two consecutive MFMAs share an
// accumulator.  Same block remap and split-K layout as the 128 x 128 kernel.
// SWIGLU: the 256 W rows are [gate 32 | up 32] x 2 per column wave.
// F16: the activation is one float16 plane (Ah; Al unused), W is the float16
// mirror of the weights, one f16 MFMA pass.  SWIGLU writes u as bf16 hi/lo planes
// (oh, ol), or as one float16 plane into oh when ol is null.
// ----------------------------------------------------------------------------
#define G2M 128
#define G2N 256
#define G2K 32
template <bool SWIGLU, bool F16, bool LSE = false, bool BUF = false>
__global__ void __launch_bounds__(256, 2) gemm_bf16w(const u16* __restrict__ Ah, const u16* __restrict__ Al, int lda,
                                                int M, int K, GemmSegs seg, int N, int m_tiles, int n_tiles,
                                                int splits, int k_chunk, float* __restrict__ C, int ldc,
                                                size_t split_stride, int accum, u16* __restrict__ oh,
                                                u16* __restrict__ ol, int* __restrict__ flags) {
  // K stages in the LDS ring: three for the float16 SwiGLU (72 KiB of LDS, two blocks per CU;
  // 14% faster than two on the 1024-row prefill shape), two elsewhere (the plain float16
  // product measured 2% slower with three; for two bf16 planes a third would leave one
  // block per CU).  Each buffer is its own array so that the compiler can
  // tell the direct-to-LDS loads of later stages from the reads of the current one.
  constexpr int NS = (F16 && SWIGLU && !LSE) ? 3 : 2;
  __shared__ __attribute__((aligned(16))) u16 sAh0[G2M * G2K];
  __shared__ __attribute__((aligned(16))) u16 sAl0[G2M * G2K];
  __shared__ __attribute__((aligned(16))) u16 sW0[G2N * G2K];
  __shared__ __attribute__((aligned(16))) u16 sAh1[G2M * G2K];
  __shared__ __attribute__((aligned(16))) u16 sAl1[G2M * G2K];
  __shared__ __attribute__((aligned(16))) u16 sW1[G2N * G2K];
  __shared__ __attribute__((aligned(16))) u16 sAh2[NS > 2 ? G2M * G2K : 8];
  __shared__ __attribute__((aligned(16))) u16 sW2[NS > 2 ? G2N * G2K : 8];

  const int nb = m_tiles * n_tiles * splits;
  const int per = gridDim.x >> 3;
  const int v = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (v >= nb) return;
  const int mt = v % m_tiles;
  const int rest = v / m_tiles;
  const int ks = rest % splits;
  const int ntile = rest / splits;
  const int m0 = mt * G2M, n0 = ntile * (SWIGLU ? G2N / 2 : G2N);
  const int kbeg = ks * k_chunk;
  const int kend = min(K, kbeg + k_chunk);
  const int nst = (kend - kbeg) / G2K;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int ql = lane & 31, hl = lane >> 5;

  // W tile row nr -> weight row (rows past N read row 0; their outputs are not stored).
  // K is a multiple of 32 and k_chunk a multiple of G2K.
  auto w_row = [&](int nr) -> const u16* {
    if (SWIGLU) {
      const int gi = nr >> 5;
      const int n = n0 + (gi >> 2) * 64 + ((gi & 3) >> 1) * 32 + (nr & 31);
      return ((gi & 1) ? seg.w[1] : seg.w[0]) + (size_t)(n < N ? n : 0) * K;
    }
    const int n = n0 + nr;
    if (n >= N) return seg.w[0];
    if (n < seg.n_end[0]) return seg.w[0] + (size_t)n * K;
    if (n < seg.n_end[1]) return seg.w[1] + (size_t)(n - seg.n_end[0]) * K;
    return seg.w[2] + (size_t)(n - seg.n_end[1]) * K;
  };
  // per-thread source rows of its 8 loads (slot = i*256 + tid; row = slot/4; 16 B chunk c = (slot%4) ^ ((row/4)%4))
  const u16* srcA[2];
  const u16* srcL[2];
  const u16* srcW[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int slot = i * 256 + tid, row = slot >> 2, c = (slot & 3) ^ ((row >> 2) & 3);
    const size_t off = (size_t)(m0 + row < M ? m0 + row : 0) * lda + c * 8;
    srcA[i] = Ah + off;
    srcL[i] = Al + off;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = i * 256 + tid, row = slot >> 2, c = (slot & 3) ^ ((row >> 2) & 3);
    srcW[i] = w_row(row) + c * 8;
  }
  // BUF (the SwiGLU products, when every byte offset fits 31 bits): the same loads in the
  // buffer form, a 32-bit offset per lane and the K position in a scalar register (measured
  // 1.5% faster on the float16 SwiGLU of 1024 rows; the plain products, on their two-stage
  // ring, measured 0-2% slower and keep the global form).  A W load instruction of a wave
  // covers 16 consecutive tile rows: all gate rows (waves 0, 1) or all up rows (waves 2, 3),
  // so its resource is uniform.
  static_assert(!BUF || (SWIGLU && !LSE), "buffer-form loads: the SwiGLU products only");
  int offA[2], offW[4];
  __amdgpu_buffer_rsrc_t rA, rL, rW;
  if constexpr (BUF) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    rA = buf_rsrc(Ah);
    rL = buf_rsrc(F16 ? Ah : Al);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int slot = i * 256 + tid, row = slot >> 2, c = (slot & 3) ^ ((row >> 2) & 3);
      offA[i] = ((m0 + row < M ? m0 + row : 0) * lda + c * 8) * 2;
    }
    rW = buf_rsrc((wv >> 1) ? seg.w[1] : seg.w[0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = i * 256 + tid, nr = slot >> 2, c = (slot & 3) ^ ((nr >> 2) & 3);
      const int gi = nr >> 5;
      const int n = n0 + (gi >> 2) * 64 + ((gi & 3) >> 1) * 32 + (nr & 31);
      offW[i] = ((n < N ? n : 0) * K + c * 8) * 2;
    }
  }
  auto load_stage = [&](int k0, u16* dA, u16* dL, u16* dW) {
    if constexpr (BUF) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void_t*)(dA + (i * 256 + wave * 64) * 8), 16, offA[i],
                                                 k0 * 2, 0, 0);
        if (!F16)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rL, (lds_void_t*)(dL + (i * 256 + wave * 64) * 8), 16, offA[i],
                                                   k0 * 2, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_void_t*)(dW + (i * 256 + wave * 64) * 8), 16, offW[i],
                                                 k0 * 2, 0, 0);
      return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_global_load_lds(srcA[i] + k0, dA + (i * 256 + wave * 64) * 8, 16, 0, 0);
      if (!F16) __builtin_amdgcn_global_load_lds(srcL[i] + k0, dL + (i * 256 + wave * 64) * 8, 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(srcW[i] + k0, dW + (i * 256 + wave * 64) * 8, 16, 0, 0);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // One K stage (two 16-wide k-steps).  Schedule: the 8 operand reads of the first
  // k-step, then its 16 MFMAs with the second k-step's 8 reads issued one per two
  // MFMAs, then the second k-step's 16 MFMAs (measured best of the orders tried).
  auto compute = [&](const u16* sA, const u16* sL, const u16* sW) {
    bf16x8 ah[2][2], al[2][2], bw[2][4];
#pragma unroll
    for (int kk = 0; kk < G2K / 16; ++kk) {
      const int c = kk * 2 + hl;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + ql;
        ah[kk][i] = *reinterpret_cast<const bf16x8*>(sA + r * G2K + ((c ^ ((r >> 2) & 3)) * 8));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 128 + j * 32 + ql;
        bw[kk][j] = *reinterpret_cast<const bf16x8*>(sW + r * G2K + ((c ^ ((r >> 2) & 3)) * 8));
      }
      if (!F16) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = wm * 64 + i * 32 + ql;
          al[kk][i] = *reinterpret_cast<const bf16x8*>(sL + r * G2K + ((c ^ ((r >> 2) & 3)) * 8));
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < G2K / 16; ++kk) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = F16 ? __builtin_amdgcn_mfma_f32_32x32x16_f16((f16x8)ah[kk][i], (f16x8)bw[kk][j], acc[i][j], 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[kk][i], bw[kk][j], acc[i][j], 0, 0, 0);
      if (!F16) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[kk][i], bw[kk][j], acc[i][j], 0, 0, 0);
      }
    }
    if (F16) {
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);   // LDS reads of k-step 0
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // one MFMA of k-step 0
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // one LDS read of k-step 1
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);  // the rest
    } else {
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // LDS reads of k-step 0
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); // two MFMAs of k-step 0
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // one LDS read of k-step 1
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);  // MFMAs of k-step 1
    }
  };
  // Stage s: wait for this thread's loads of stage s (the NS - 2 later stages already issued
  // stay in flight), a barrier (every thread's stage-s bytes are in LDS and every wave is done
  // reading stage s - 1), then the loads of stage s + NS - 1 into the buffer stage s - 1 used,
  // then stage s's MFMAs.
  constexpr int LPS = F16 ? 6 : 8;   // direct-to-LDS loads per thread per stage
  auto step = [&](int s, const u16* cA, const u16* cL, const u16* cW, u16* nA, u16* nL, u16* nW) {
    if (NS > 2 && s + 1 < nst)
      __builtin_amdgcn_s_waitcnt(0x70 | (LPS & 15) | ((LPS >> 4) << 14));   // vmcnt(LPS) lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x70);                                       // vmcnt(0) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    if (s + NS - 1 < nst) load_stage(kbeg + (s + NS - 1) * G2K, nA, nL, nW);
    compute(cA, cL, cW);
    // every MFMA of the stage is issued before the next wait: left alone, the scheduler
    // hoists that wait above most of them, leaving the loads little cover
    __builtin_amdgcn_sched_barrier(0);
  };
  // a stage with a later stage in flight and a stage to load (the three-stage ring only)
  auto full_step = [&](const u16* cA, const u16* cW, u16* nA, u16* nW, int knext) {
    __builtin_amdgcn_s_waitcnt(0x70 | (LPS & 15) | ((LPS >> 4) << 14));   // vmcnt(LPS) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    load_stage(knext, nA, nullptr, nW);
    compute(cA, nullptr, cW);
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (NS == 2) {
    if (nst > 0) load_stage(kbeg, sAh0, sAl0, sW0);
    for (int s = 0; s < nst; s += 2) {
      step(s, sAh0, sAl0, sW0, sAh1, sAl1, sW1);
      if (s + 1 < nst) step(s + 1, sAh1, sAl1, sW1, sAh0, sAl0, sW0);
    }
  } else {
    // the prologue loads are unconditional, which keeps the compiler's count of loads in
    // flight exact where the loop starts; with one stage (a short last split) the second is
    // clamped into the chunk and left unused
    load_stage(kbeg, sAh0, nullptr, sW0);
    load_stage(min(kbeg + G2K, kend - G2K), sAh1, nullptr, sW1);
    // whole groups of three stages whose loads all exist, then the tail with its checks
    int s = 0;
    for (; s + 4 < nst; s += 3) {
      full_step(sAh0, sW0, sAh2, sW2, kbeg + (s + 2) * G2K);
      full_step(sAh1, sW1, sAh0, sW0, kbeg + (s + 3) * G2K);
      full_step(sAh2, sW2, sAh1, sW1, kbeg + (s + 4) * G2K);
    }
    for (; s < nst; s += 3) {
      step(s, sAh0, sAl0, sW0, sAh2, nullptr, sW2);
      if (s + 1 < nst) step(s + 1, sAh1, sAl1, sW1, sAh0, sAl0, sW0);
      if (s + 2 < nst) step(s + 2, sAh2, nullptr, sW2, sAh1, sAl1, sW1);
    }
  }

  if (m0 + wm * 64 >= M) return;
  if (LSE) {
    // Full-vocabulary readout: the logits stay in registers.  Per row of the wave's 64, the
    // max and the sum of exp over its 128 columns (those past N excluded), reduced across
    // the 32 lanes that hold the row's columns: one (max, sum) pair per row and 128-column
    // slice, in C viewed as float2 [M][ldc].
    float2* part = reinterpret_cast<float2*>(C);
    const int slice = ntile * 2 + wn;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        float mx = NEG_INF;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n0 + wn * 128 + j * 32 + ql < N) mx = fmaxf(mx, acc[i][j][r]);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        float se = 0.f;
        if (mx != NEG_INF) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (n0 + wn * 128 + j * 32 + ql < N) se += expf(acc[i][j][r] - mx);
        }
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) se += __shfl_xor(se, o, 64);
        if (ql == 0 && row < M) part[(size_t)row * ldc + slice] = make_float2(mx, se);
      }
    return;
  }
  if (SWIGLU) {
    bool bad = false;
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const int col = n0 + wn * 64 + jp * 32 + ql;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (row < M && col < N) {
            const float g = acc[i][2 * jp][r], u = acc[i][2 * jp + 1][r];
            const float val = g / (1.0f + expf(-g)) * u;
            if (ol == nullptr) {   // one float16 plane
              bad |= f16_out_of_range(val);
              reinterpret_cast<f16*>(oh)[(size_t)row * ldc + col] = (f16)val;
            } else {
              const u16 h = f32_to_bf16(val);
              oh[(size_t)row * ldc + col] = h;
              ol[(size_t)row * ldc + col] = f32_to_bf16(val - bf16_to_f32(h));
            }
          }
        }
    }
    flag_f16_range(flags, bad);
    return;
  }
  float* Cb = C + (splits > 1 ? (size_t)ks * split_stride : 0);
  const bool add = (splits == 1) && accum;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + ql;
      const int rbase = m0 + wm * 64 + i * 32 + 4 * hl;
      float old[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rbase + 8 * (r >> 2) + (r & 3);
        old[r] = (add && row < M && col < N) ? Cb[(size_t)row * ldc + col] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rbase + 8 * (r >> 2) + (r & 3);
        if (row < M && col < N) Cb[(size_t)row * ldc + col] = old[r] + acc[i][j][r];
      }
    }
}

// ----------------------------------------------------------------------------
// K3 for few rows (M <= 64): a weight-streaming product.  Block = 4 waves and 128 output
// columns (32 per wave) over one K chunk, walked in stages of 64 of K.  A stage's weight
// tile (128 rows x 128 B) and its activation tile (32 rows x 128 B per plane; rows past M
// repeat row M - 1, their outputs dropped) are staged in LDS by direct global->LDS loads
// in which a wave's instruction covers 8 whole 128 B row segments (fully used cache
// lines).  Loading the MFMA operand layout straight into registers touches 32 rows per
// instruction and issued every wave's own copy of the activations: 30-40% slower.  The
// 16 B chunk c of row r sits at position c ^ ((r / 2) % 8), so the operand reads are
// bank-conflict free.  A ring of three stages keeps two stages of loads in flight.  F16:
// one f16 activation plane x the f16 weight mirror; else two bf16 planes x bf16 weights
// (W·hi + W·lo).  The chunk's sum goes to C (splits == 1) or to partials [split][M][N].
// ----------------------------------------------------------------------------
#define SKS 64   // K per stage of the few-row product
template <bool F16>
__global__ void __launch_bounds__(256, 2) gemm_skinny(const u16* __restrict__ Ah, const u16* __restrict__ Al,
                                                     int lda, int M, int K, GemmSegs seg, int N, int n_tiles,
                                                     int splits, int k_chunk, float* __restrict__ C, int ldc,
                                                     size_t split_stride, int accum, int row_groups) {
  constexpr int NB = F16 ? 1 : 2;   // activation planes
  constexpr int AS = 32 * SKS;      // one activation plane of a stage
  __shared__ __attribute__((aligned(16))) u16 sW0[128 * SKS];
  __shared__ __attribute__((aligned(16))) u16 sW1[128 * SKS];
  __shared__ __attribute__((aligned(16))) u16 sW2[128 * SKS];
  __shared__ __attribute__((aligned(16))) u16 sA0[NB * AS];
  __shared__ __attribute__((aligned(16))) u16 sA1[NB * AS];
  __shared__ __attribute__((aligned(16))) u16 sA2[NB * AS];
  // Rows past 32 (at most 64): two row groups per work item, blocks 8 apart in the grid so
  // that both run on the same XCD (blocks go round-robin over the 8) and the second reads
  // the weight tile from that XCD's L2.
  const int rg = row_groups == 2 ? (blockIdx.x >> 3) & 1 : 0;
  const int v = row_groups == 2 ? ((blockIdx.x >> 4) << 3) + (blockIdx.x & 7) : blockIdx.x;
  if (v >= n_tiles * splits) return;
  const int m0 = rg * 32;
  const int ntile = v % n_tiles, ks = v / n_tiles;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hl = lane >> 5;
  const int kb = ks * k_chunk, ke = min(K, kb + k_chunk);
  const int nst = (ke - kb) / SKS;   // >= 1
  // the thread's loads per stage: 4 weight slots q * 256 + tid (row slot / 8, chunk slot % 8)
  // and, per plane, activation slot tid (row tid / 8)
  const u16* srcW[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int slot = q * 256 + tid, row = slot >> 3, c = (slot & 7) ^ ((row >> 1) & 7);
    const int n = ntile * 128 + row;
    srcW[q] = seg_row(seg, n < N ? n : 0, K) + c * 8;
  }
  const u16* srcA[2];   // fixed size: a template-sized array of these loads drops the host stub
  {
    const int row = tid >> 3, c = (tid & 7) ^ ((row >> 1) & 7);
    const size_t off = (size_t)(m0 + row < M ? m0 + row : M - 1) * lda + c * 8;
    srcA[0] = Ah + off;
    srcA[1] = F16 ? srcA[0] : Al + off;
  }
  auto load = [&](int k0, u16* dw, u16* da) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds(srcW[q] + k0, dw + (q * 256 + wave * 64) * 8, 16, 0, 0);
#pragma unroll
    for (int p = 0; p < NB; ++p)
      __builtin_amdgcn_global_load_lds(srcA[p] + k0, da + p * AS + wave * 64 * 8, 16, 0, 0);
  };
  typedef u16 u16x8 __attribute__((ext_vector_type(8)));
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int wr = wave * 32 + ql;   // the lane's weight row (output column) in the tile
  auto compute = [&](const u16* sw, const u16* sa) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = 2 * j + hl;
      const u16x8 b = *reinterpret_cast<const u16x8*>(sw + wr * SKS + ((g ^ ((wr >> 1) & 7)) * 8));
#pragma unroll
      for (int p = 0; p < NB; ++p) {
        const u16x8 a = *reinterpret_cast<const u16x8*>(sa + p * AS + ql * SKS + ((g ^ ((ql >> 1) & 7)) * 8));
        if (F16)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      acc, 0, 0, 0);
        else
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
      }
    }
  };
  // Stage s waits until only stage s + 1's loads may be in flight (4 + NB per thread), then a
  // barrier (every thread's stage s is in LDS, every wave is done reading stage s - 1's
  // buffers), then the loads of stage s + 2 into those buffers, then stage s's MFMAs.  Both
  // prologue loads are unconditional (the second clamped into the chunk, unused when
  // nst == 1), which keeps the compiler's count of loads in flight exact at the loop head.
  auto wait_stage = [&]() {
    if constexpr (F16) __builtin_amdgcn_s_waitcnt(0x75);   // vmcnt(5) lgkmcnt(0)
    else __builtin_amdgcn_s_waitcnt(0x76);                 // vmcnt(6) lgkmcnt(0)
  };
  load(kb, sW0, sA0);
  load(min(kb + SKS, ke - SKS), sW1, sA1);
  auto full = [&](int s, const u16* cw, const u16* ca, u16* nw, u16* na) {
    wait_stage();
    asm volatile("s_barrier" ::: "memory");
    load(kb + (s + 2) * SKS, nw, na);
    __builtin_amdgcn_sched_barrier(0);
    compute(cw, ca);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto tail = [&](int s, const u16* cw, const u16* ca, u16* nw, u16* na) {
    if (s + 1 < nst) wait_stage();
    else __builtin_amdgcn_s_waitcnt(0x70);   // vmcnt(0) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    if (s + 2 < nst) load(kb + (s + 2) * SKS, nw, na);
    __builtin_amdgcn_sched_barrier(0);
    compute(cw, ca);
    __builtin_amdgcn_sched_barrier(0);
  };
  int s = 0;
  for (; s + 4 < nst; s += 3) {
    full(s, sW0, sA0, sW2, sA2);
    full(s + 1, sW1, sA1, sW0, sA0);
    full(s + 2, sW2, sA2, sW1, sA1);
  }
  for (; s < nst; s += 3) {
    tail(s, sW0, sA0, sW2, sA2);
    if (s + 1 < nst) tail(s + 1, sW1, sA1, sW0, sA0);
    if (s + 2 < nst) tail(s + 2, sW2, sA2, sW1, sA1);
  }
  const int n = ntile * 128 + wr;
  if (n >= N) return;
  // acc[r]: row m0 + 8 (r / 4) + 4 hl + r % 4, column n
  float* Cb = C + (splits > 1 ? (size_t)ks * split_stride : 0);
  const bool add = (splits == 1) && accum;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + 8 * (r >> 2) + 4 * hl + (r & 3);
    if (row < M) {
      float* o = Cb + (size_t)row * ldc + n;
      *o = add ? *o + acc[r] : acc[r];
    }
  }
}

// Deterministic split-K reduction: out = (accum ? out : 0) + sum_s part[s] (fixed order).
__global__ void __launch_bounds__(256) splitk_reduce(const float* __restrict__ part, size_t split_stride,
                                                     int splits, int M, int N, int ldp,
                                                     float* __restrict__ out, int ldo, int accum) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)M * N) return;
  const int m = (int)(i / N), n = (int)(i % N);
  float s = 0.f;
  for (int k = 0; k < splits; ++k) s += part[k * split_stride + (size_t)m * ldp + n];
  float* o = out + (size_t)m * ldo + n;
  *o = accum ? (*o + s) : s;
}

// ----------------------------------------------------------------------------
// SwiGLU from split-K partials of the gate|up product (few output tiles): part[s] is
// [M][2I] with the gate columns first; u = silu(sum_s gate) * (sum_s up), splits summed in
// order, written as bf16 hi/lo planes or (ul == nullptr) one float16 plane [M][ldu].
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) splitk_swiglu(const float* __restrict__ part, size_t split_stride,
                                                     int splits, int M, int I, u16* __restrict__ uh,
                                                     u16* __restrict__ ul, int ldu, int* __restrict__ flags) {
  const int I4 = I >> 2;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)M * I4) return;
  const int row = (int)(i / I4), c = (int)(i % I4) * 4;
  const float* p = part + (size_t)row * 2 * I + c;
  float4 g = *reinterpret_cast<const float4*>(p), u = *reinterpret_cast<const float4*>(p + I);
  for (int k0 = 1; k0 < splits; k0 += 4) {   // split order; four splits' loads per round
    float4 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (k0 + j < splits) {
        a[j] = *reinterpret_cast<const float4*>(p + (k0 + j) * split_stride);
        b[j] = *reinterpret_cast<const float4*>(p + (k0 + j) * split_stride + I);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (k0 + j < splits) {
        g.x += a[j].x; g.y += a[j].y; g.z += a[j].z; g.w += a[j].w;
        u.x += b[j].x; u.y += b[j].y; u.z += b[j].z; u.w += b[j].w;
      }
  }
  const float gv[4] = {g.x, g.y, g.z, g.w}, uv[4] = {u.x, u.y, u.z, u.w};
  const size_t o = (size_t)row * ldu + c;
  if (ul == nullptr) {
    f16x4 v4;
    bool bad = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = gv[j] / (1.0f + expf(-gv[j])) * uv[j];
      bad |= f16_out_of_range(v);
      v4[j] = (f16)v;
    }
    *reinterpret_cast<f16x4*>(uh + o) = v4;
    flag_f16_range(flags, bad);
    return;
  }
  u16 h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float v = gv[j] / (1.0f + expf(-gv[j])) * uv[j];
    h[j] = f32_to_bf16(v);
    l[j] = f32_to_bf16(v - bf16_to_f32(h[j]));
  }
  *reinterpret_cast<uint2*>(uh + o) =
      make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
  *reinterpret_cast<uint2*>(ul + o) =
      make_uint2((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16));
}

// ----------------------------------------------------------------------------
// K3 (float32 models): tiled VALU GEMM, 64x64 tile, 4x4 outputs per thread.
// ----------------------------------------------------------------------------
__device__ __forceinline__ const float* seg_row_f(const GemmSegsF& s, int n, int K) {
  if (n < s.n_end[0]) return s.w[0] + (size_t)n * K;
  if (n < s.n_end[1]) return s.w[1] + (size_t)(n - s.n_end[0]) * K;
  return s.w[2] + (size_t)(n - s.n_end[1]) * K;
}

__global__ void __launch_bounds__(256) gemm_f32(const float* __restrict__ A, int lda, int M, int K,
                                                GemmSegsF seg, int N, float* __restrict__ C, int ldc,
                                                int accum) {
  __shared__ float sA[16][64 + 1];
  __shared__ float sB[16][64 + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;     // 0..1023: row = idx/16, k = idx%16
      const int r = idx >> 4, kk = idx & 15;
      const int gm = m0 + r, gk = k0 + kk, gn = n0 + r;
      sA[kk][r] = (gm < M && gk < K) ? A[(size_t)gm * lda + gk] : 0.f;
      sB[kk][r] = (gn < N && gk < K) ? seg_row_f(seg, gn, K)[gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sA[kk][ty * 4 + i]; b[i] = sB[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      float* p = C + (size_t)row * ldc + col;
      *p = accum ? (*p + acc[i][j]) : acc[i][j];
    }
  }
}

// ----------------------------------------------------------------------------
// RoPE + layout: q/k from the fused projection output [T][(Hq+2Hkv)*D] are
// rotated at their row's position (rotate-half: pair t with t + D/2, angle
// pos * theta^(-2t/D), angle and sin/cos in float64) and written as
//   Q  [T][Hq][D]         (query rows, token-major)
//   K  [Hkv][ldk][D]      at row `row0 + t`
// V is written transposed by v_transpose below.
// ----------------------------------------------------------------------------
template <typename OT> __device__ __forceinline__ OT cvt_out(float v);
template <> __device__ __forceinline__ f16 cvt_out<f16>(float v) { return (f16)v; }
template <> __device__ __forceinline__ float cvt_out<float>(float v) { return v; }

template <typename OT>
__global__ void __launch_bounds__(256) rope_qk(const float* __restrict__ qkv, int T, int Hq, int Hkv, int D,
                                               const int* __restrict__ pos, double log2_theta,
                                               OT* __restrict__ q_out, OT* __restrict__ q_lo, OT* __restrict__ k_out,
                                               int ldk, int row0) {
  const int t = blockIdx.x;
  if (t >= T) return;
  const int half = D >> 1;
  const int nh = Hq + Hkv;
  const double p = (double)pos[t];
  const float* src = qkv + (size_t)t * (size_t)(Hq + 2 * Hkv) * D;
  for (int idx = threadIdx.x; idx < nh * half; idx += 256) {
    const int h = idx / half, i = idx % half;
    const double inv_freq = exp2(-(2.0 * i / (double)D) * log2_theta);
    double sd, cd;
    sincos(p * inv_freq, &sd, &cd);
    const float c = (float)cd, s = (float)sd;
    const float a = src[h * D + i], b = src[h * D + i + half];
    const float ra = a * c - b * s;
    const float rb = b * c + a * s;
    if (h < Hq) {
      const size_t o = ((size_t)t * Hq + h) * D;
      const OT qa = cvt_out<OT>(ra), qb = cvt_out<OT>(rb);
      q_out[o + i] = qa;
      q_out[o + i + half] = qb;
      if (q_lo) {
        q_lo[o + i] = cvt_out<OT>(ra - (float)qa);
        q_lo[o + i + half] = cvt_out<OT>(rb - (float)qb);
      }
    } else {
      OT* d = k_out + ((size_t)(h - Hq) * ldk + row0 + t) * D;
      d[i] = cvt_out<OT>(ra);
      d[i + half] = cvt_out<OT>(rb);
    }
  }
}

// V [T][Hkv*D] (a column slice of the projection output) -> Vt [Hkv][D][ldv] at column col0 + t.
// 64x64 tile transpose through LDS so both the read and the write are coalesced.
template <typename OT>
__global__ void __launch_bounds__(256) v_transpose(const float* __restrict__ src, int lds, int T, int HD,
                                                   OT* __restrict__ vt, int ldv, int col0) {
  __shared__ float tile[64][65];
  const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int t = t0 + r, c = c0 + tx;
    tile[r][tx] = (t < T && c < HD) ? src[(size_t)t * lds + c] : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int c = c0 + r, t = t0 + tx;     // c = hk*D + d
    if (c < HD && t < T) vt[(size_t)c * ldv + col0 + t] = cvt_out<OT>(tile[tx][r]);
  }
}

// ----------------------------------------------------------------------------
// K4/K5: attention of query rows over (a) the shared prefix keys and (b) the
// rows' own keys, float16 MFMA 32x32x16, float32 online softmax (base 2).
//
// Per KV head hk the query rows are r = t*G + g (token-major, G = Hq/Hkv), so
// one block of 128 rows covers ~128/G tokens and all G heads that share hk;
// every K/V tile staged in LDS is used by all 128 rows.
// Scores are formed transposed, S^T = K · Q^T: the MFMA "A" operand is a
// 32-key slice of K and the "B" operand is the wave's 32 queries, so each
// lane's accumulators belong to ONE query row (lane % 32) and the softmax
// rescale is a per-lane scalar.  O^T = V^T · P^T likewise keeps a lane on its
// query; P^T is fed straight from the score registers.  The K rows of each
// 32-key slice are read in the order that swaps key-index bits 2 and 3, which
// makes score register i of half hs hold key 32*hs + 16*(i/8) + 8*(lane/32) + i%8:
// the 8 keys one lane feeds to a P·V step are then consecutive in V^T.
//
// Key tiles of 64: a row tile sees the prefix tiles [0, ceil(P/64)) followed by
// the tiles of its own keys (from the first row's sequence start, causal within
// the row's sequence, or the row's 64-bit ancestor mask over its group).
// Split z takes the contiguous share [z*n/S, (z+1)*n/S) of those n tiles; or, in the
// balanced schedule (sk_chunk > 0), every block takes sk_chunk consecutive tiles of all
// (KV head, row tile) sequences laid end to end, so blocks hold equal work whatever the
// number of row tiles, and a row tile's partials sit in slots 0.. of its first block on.  Tiles
// arrive by direct global->LDS loads (16 B per lane) into a double buffer, the
// next tile's loads in flight while the current one is computed.  LDS rows are
// XOR-swizzled by 16 B chunk so the operand reads are bank-conflict free.  With
// S == 1 the block writes o as bf16 hi/lo planes (or one f16 plane); otherwise a
// normalised partial o and its log2-sum-exp for attn_merge.
//
// Arithmetic: q arrives multiplied by log2(e)/sqrt(D) (qkv_post), so a score is in
// log2 units; the score accumulators start at -m (the row's reference max), so the
// MFMAs leave score - m and a weight is exp2 of it with no further arithmetic.
// QT = 1 takes q rounded once to f16; QT = 2 adds the second term q - f16(q)
// (twice the score MFMAs), for rows that see long prefixes.  The weights are
// rounded to f16 in pairs (v_cvt_pk) and the row sum adds exactly those rounded
// values (v_dot2 against 1, 1).
// ----------------------------------------------------------------------------
#define AT_BR 128
#define AT_BK 64

// Key-index bit swap 2 <-> 3 inside a 32-key slice (the A-operand row order of S^T).
__device__ __forceinline__ int attn_key_perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Reductions across the two 32-lane halves of the wave (lanes l and l^32 hold the same query).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 B per lane from base + byte_off into LDS at dst + lane * 16.  The buffer form of the
// direct load is counted by vmcnt alone, so the waits the compiler places for LDS reads
// stay exact (the global form is also tracked as an LDS access, forcing full drains).
__device__ __forceinline__ void dma16(const void* base, int byte_off, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(buf_rsrc(base), (lds_void_t*)dst, 16, byte_off, 0, 0, 0);
}

struct AttnTile {
  const f16* K;   // [ld][128]
  const f16* V;   // V^T [128][ld]
  int ld, k0, ke; // tile keys [k0, k0+64); keys >= ke are not visible (and not read)
  bool own;
};

template <int QT, bool BAL>
__global__ void __launch_bounds__(256, 2) attn_fwd_f16(AttnArgs a) {
  constexpr int RB = AT_BR;         // query rows per block, 32 per wave
  __shared__ __attribute__((aligned(16))) f16 smem[2 * 2 * AT_BK * 128];
  // buffer b: K tile at smem + 2 b tiles, V^T tile right after it
  auto sk = [&](int b) { return smem + (size_t)(b * 2) * (AT_BK * 128); };
  auto sv = [&](int b) { return smem + (size_t)(b * 2 + 1) * (AT_BK * 128); };

  // row tiles in reverse order: with long causal sequences the later tiles see the most keys
  // and are dispatched first
  const int G = a.G, T = a.T, Hq = a.Hq, ns = a.n_split;
  const int R = G * T;
  const int n_rt = (R + RB - 1) / RB;
  // Block order.  With prefix keys (scoring calls) each XCD (blocks are dispatched to the 8
  // XCDs round-robin) takes a contiguous run of (KV head, row tile, split) items, so the row
  // tiles of a KV head share its prefix K/V through one L2.  Without them (prefills: causal
  // rows whose work grows with the row) consecutive items go to different XCDs, which keeps
  // the heavy and the light row tiles spread over all of them.
  const int per = gridDim.x >> 3;
  const int vv = a.P > 0 ? (blockIdx.x & 7) * per + (blockIdx.x >> 3) : blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hl = lane >> 5;
  const bool parts = BAL || ns > 1;   // partials for attn_merge

  // One work item: KV head hk, row tile x, the key tiles [vb, ve_u) of the row tile's nominal
  // tile sequence (last: the item's final share, which also takes any tiles past the nominal
  // bound), its partial written to slot z.  vb < 0: share z of ns equal splits.
  auto run = [&](const int hk, const int x, const int z, int vb, int ve_u, bool last) {
    const int r0 = x * RB;
    const int r = r0 + wave * 32 + ql;
    const bool rvalid = r < R;
    const int rc = rvalid ? r : R - 1;          // clamped row: loads stay in bounds
    const int t = rc / G;
    const int hq = hk * G + rc % G;

    // Prefix key tiles of this row tile: [ptb, ptb + ntp), every one of them visible in full to
    // all of its rows when inside [vis_lo, vis_hi).  One shared prefix: all ceil(P/64) tiles,
    // visible below P.  Segmented prefixes: the hull of the rows' segments (host table).
    // (the host's table is per 128-row tile; a smaller row tile takes its tile's entry)
    const int4 pt = a.ptile ? a.ptile[r0 / AT_BR] : make_int4(0, (a.P + AT_BK - 1) / AT_BK, 0, a.P);
    const int ptb = pt.x, ntp = pt.y - pt.x, vis_lo = pt.z, vis_hi = pt.w;
    // The splits divide ntp + own_tiles key tiles (own_tiles: the host's bound on any row
    // tile's own-key tiles), so a block whose range starts on a prefix tile issues that
    // tile's loads before the sequence starts it depends on for the rest have arrived.
    if (vb < 0) {
      const int nt_u = ntp + a.own_tiles;
      vb = (int)(((long)z * nt_u) / ns);
      ve_u = (int)(((long)(z + 1) * nt_u) / ns);
      last = z == ns - 1;
    }
    const f16* Kp = a.kp + (size_t)hk * a.ldp * 128;
    const f16* Vp = a.vtp + (size_t)hk * 128 * a.ldp;
    // K tile: 64 rows of 256 B, chunk c (16 B) of key row k at chunk position c ^ (k & 15).
    // V^T tile: 128 dim rows of 128 B, key chunk c of dim d at position c ^ ((d >> 1) & 7).
    // Rows / chunks at or past ke load row / column 0 instead (finite, never weighted);
    // a V chunk straddling ke holds later rows of this call or zeroed padding.
    auto load_kv = [&](const f16* K, const f16* V, int ld, int k0, int ke, f16* dk, f16* dv) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = i * 256 + tid;
        const int row = slot >> 4, c = (slot & 15) ^ (row & 15);
        const int key = k0 + row;
        dma16(K, ((key < ke ? key : 0) * 128 + c * 8) * 2, dk + (i * 256 + wave * 64) * 8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = i * 256 + tid;
        const int d = slot >> 3, c = (slot & 7) ^ ((d >> 1) & 7);
        const int key = k0 + c * 8;
        dma16(V, (d * ld + (key < ke ? key : 0)) * 2, dv + (i * 256 + wave * 64) * 8);
      }
    };
    // the first prefix tile goes out before the sequence metadata it does not need
    const bool early = vb < ntp && vb < ve_u;
    if (early) load_kv(Kp, Vp, a.ldp, (ptb + vb) * AT_BK, a.P, sk(0), sv(0));

    const int t_first = r0 / G, t_last = min(R - 1, r0 + RB - 1) / G;
    const int s_first = a.seq_start[t_first];
    const int max_start = a.seq_start[t_last];
    const int my_start = a.seq_start[t];
    const bool use_mask = a.mask != nullptr;
    const uint64_t my_mask = use_mask ? a.mask[t] : 0ull;
    const int2 my_pk = a.pseg ? a.pseg[t] : make_int2(0, a.P);   // the row's prefix keys

    // q = q_hi + q_lo (two f16 terms): scores are K·q_hi + K·q_lo, so the rounding
    // of q, which would shift every score of the row coherently, stays out.
    f16x8 qreg[8], qlo[QT == 2 ? 8 : 1];
    {
      // operand-ordered q: slice c of the wave's 32 rows is one contiguous 1 KB run
      const size_t qo = ((size_t)hk * attn_q_rows(T, G) + (rc & ~31)) * 128 + (size_t)(hl * 32 + (rc & 31)) * 8;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        qreg[c] = *reinterpret_cast<const f16x8*>(a.q + qo + c * 512);
        if (QT == 2) qlo[c] = *reinterpret_cast<const f16x8*>(a.q_lo + qo + c * 512);
      }
    }

    // this block's share of the tile sequence: [vb, ve) of the row tile's real tiles (the last
    // split also takes any tiles past the bound, should the host's bound be short)
    const int own_end = t_last + 1;
    const int own0 = s_first & ~7;   // 16 B aligned start of the block's own keys
    const int nt_all = ntp + (own_end - own0 + AT_BK - 1) / AT_BK;
    const int ve = last ? nt_all : min(ve_u, nt_all);
    const int nt = max(0, ve - vb);

    auto tile = [&](int v) {
      AttnTile s;
      if (v < ntp) {
        s.K = Kp; s.V = Vp; s.ld = a.ldp;
        s.k0 = (ptb + v) * AT_BK; s.ke = a.P; s.own = false;
      } else {
        s.K = a.ks + (size_t)hk * a.lds * 128; s.V = a.vts + (size_t)hk * 128 * a.lds; s.ld = a.lds;
        s.k0 = own0 + (v - ntp) * AT_BK; s.ke = own_end; s.own = true;
      }
      return s;
    };
    auto load_tile = [&](const AttnTile& s, f16* dk, f16* dv) { load_kv(s.K, s.V, s.ld, s.k0, s.ke, dk, dv); };

    const int prow = attn_key_perm(ql);
    float m_ref = NEG_INF, l_run = 0.f;   // m_ref: reference max of the row, in scaled log2 units
    f32x16 acc[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[d][i] = 0.f;

    auto step = [&](int i, int b) {
      if (i + 1 < nt) load_tile(tile(vb + i + 1), sk(b ^ 1), sv(b ^ 1));   // in flight during this tile
      const f16* skb = sk(b);
      const f16* svb = sv(b);
      // scores start at -m_use (q carries the log2(e)/sqrt(D) scale): the MFMAs leave
      // score - m_use, in log2 units, and a weight is exp2 of it
      f32x16 s[2];
      const float m_init = (m_ref == NEG_INF) ? 0.f : -m_ref;
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[hs][e] = m_init;
      // the K operands of half the tile's dims are read ahead of their MFMAs (one LDS round
      // trip per half instead of one per 16-dim step)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        f16x8 k0op[4], k1op[4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const int ch = (2 * (4 * h2 + c4) + hl) ^ (prow & 15);
          k0op[c4] = *reinterpret_cast<const f16x8*>(skb + prow * 128 + ch * 8);
          k1op[c4] = *reinterpret_cast<const f16x8*>(skb + (32 + prow) * 128 + ch * 8);
        }
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const int c = 4 * h2 + c4;
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0op[c4], qreg[c], s[0], 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1op[c4], qreg[c], s[1], 0, 0, 0);
          if (QT == 2) {
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0op[c4], qlo[c], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1op[c4], qlo[c], s[1], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);            // the 8 LDS reads first
        __builtin_amdgcn_sched_group_barrier(0x008, QT == 2 ? 16 : 8, 0);   // then their MFMAs
      }
      // Masks only where some row of the block does not see the whole tile (uniform test):
      // a prefix tile reaching outside [vis_lo, vis_hi) (the partial last tile, segment
      // edges), and own-key tiles not fully visible to every row.
      const AttnTile ts = tile(vb + i);
      const bool need = ts.own ? (use_mask || ts.k0 < max_start || ts.k0 + AT_BK > t_first + 1)
                               : (ts.k0 < vis_lo || ts.k0 + AT_BK > vis_hi);
      if (need) {
        const int lo = ts.own ? my_start : my_pk.x;
        const int hi = ts.own ? t + 1 : my_pk.y;
        const uint64_t mm = (ts.own && use_mask) ? my_mask : ~0ull;
        const int base = ts.k0 + 8 * hl;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = base + hs * 32 + 16 * (e >> 3) + (e & 7);
            const bool in = ((unsigned)(key - lo) < (unsigned)(hi - lo)) && ((mm >> ((key - lo) & 63)) & 1ull);
            s[hs][e] = in ? s[hs][e] : NEG_INF;
          }
      }
      float mx = NEG_INF;
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[hs][e]);
      mx = halves_max(mx);
      // The reference max moves only when a score exceeds it by more than 8 (log2 units):
      // the weights p = 2^(score - m_ref) stay below 2^8 (exact to f16's relative
      // precision), and the accumulators are rescaled on few tiles.
      const bool first = m_ref == NEG_INF;
      const bool grow = first ? (mx != NEG_INF) : (mx > 8.f);
      if (__ballot(grow)) {
        const float d = grow ? mx : 0.f;
        const float alpha = grow ? (first ? 0.f : __builtin_amdgcn_exp2f(-mx)) : 1.f;
        if (grow) m_ref = (first ? 0.f : m_ref) + mx;
        l_run *= alpha;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[dd][e] *= alpha;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs)
#pragma unroll
          for (int e = 0; e < 16; ++e) s[hs][e] -= d;
      }
      // p is rounded to nearest f16 in pairs; the row sum adds exactly the rounded weights
      float rs = 0.f;
      f16x8 pops[2][2];
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x2 e2 = {__builtin_amdgcn_exp2f(s[hs][8 * p + 2 * j]),
                              __builtin_amdgcn_exp2f(s[hs][8 * p + 2 * j + 1])};
            const f16x2 h2 = __builtin_convertvector(e2, f16x2);
            rs = __builtin_amdgcn_fdot2(h2, f16x2{(f16)1.0f, (f16)1.0f}, rs, false);
            pops[hs][p][2 * j] = h2[0];
            pops[hs][p][2 * j + 1] = h2[1];
          }
      l_run += halves_sum(rs);
      // O^T += V^T · P^T, four 16-key steps
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int c = 4 * hs + 2 * p + hl;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const int d = dt * 32 + ql;
            const f16x8 vop = *reinterpret_cast<const f16x8*>(svb + d * AT_BK + ((c ^ ((d >> 1) & 7)) * 8));
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, pops[hs][p], acc[dt], 0, 0, 0);
          }
        }
      // The next tile's loads have landed and every wave is done with this tile's buffers.
      // (The wait is a builtin so the compiler knows the loads are complete; the barrier is
      // asm with a memory clobber so no LDS access moves across it.)
      __builtin_amdgcn_s_waitcnt(0x70);   // vmcnt(0) lgkmcnt(0)
      asm volatile("s_barrier" ::: "memory");
    };
    if (nt > 0 && !early) load_tile(tile(vb), sk(0), sv(0));
    // the first tile has landed (or, with no tile to process, the early load is done before
    // the block's LDS is released)
    __builtin_amdgcn_s_waitcnt(0x70);
    if (nt > 0) asm volatile("s_barrier" ::: "memory");
    for (int i = 0; i < nt; i += 2) {   // two steps per trip: the buffers are named statically
      step(i, 0);
      if (i + 1 < nt) step(i + 1, 1);
    }
    // this block's normalised partial o (acc / l) and its log2-sum-exp
    const float inv = (l_run > 0.f) ? 1.0f / l_run : 0.f;
    float lse = (l_run > 0.f) ? m_ref + log2f(l_run) : NEG_INF;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[dt][e] *= inv;
    if (parts) {
      float* op = a.o_part + (((size_t)z * T + t) * Hq + hq) * 128;
      if (rvalid) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int d = dt * 32 + 8 * ii + 4 * hl;
            *reinterpret_cast<float4*>(op + d) =
                make_float4(acc[dt][4 * ii], acc[dt][4 * ii + 1], acc[dt][4 * ii + 2], acc[dt][4 * ii + 3]);
          }
        if (hl == 0) a.lse_part[((size_t)z * T + t) * Hq + hq] = lse;
      }
      return;   // attn_merge combines the splits
    }
    if (!rvalid) return;
    // o [T][Hq][D]: the first D of the 128 dims (a 64-dim head runs zero-padded)
    const int Do = a.D;
    const size_t ob = ((size_t)t * Hq + hq) * Do;
    if (a.o_f16) {   // one float16 plane
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int d = dt * 32 + 8 * ii + 4 * hl;
          if (d >= Do) continue;
          f16x4 v4;
#pragma unroll
          for (int j = 0; j < 4; ++j) v4[j] = (f16)acc[dt][4 * ii + j];
          *reinterpret_cast<f16x4*>(a.oh + ob + d) = v4;
        }
      return;
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int d = dt * 32 + 8 * ii + 4 * hl;
        if (d >= Do) continue;
        u16 h[4], l[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = acc[dt][4 * ii + j];
          h[j] = f32_to_bf16(v);
          l[j] = f32_to_bf16(v - bf16_to_f32(h[j]));
        }
        *reinterpret_cast<uint2*>(a.oh + ob + d) =
            make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
        *reinterpret_cast<uint2*>(a.ol + ob + d) =
            make_uint2((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16));
      }
  };

  if constexpr (BAL) {
    // Balanced: the items' nominal tile sequences laid end to end (item u = KV head u / n_rt,
    // row tile n_rt - 1 - u % n_rt), block vv taking the run [vv*c, (vv+1)*c) of them, which
    // may cover the end of one item and the start of the next.  An item's partial slot is the
    // block's offset from the first block on that item.
    // (the host keeps n_rt * Hkv * nt_u within int)
    attn_balanced_items(vv, a.sk_chunk, (a.P + AT_BK - 1) / AT_BK + a.own_tiles, n_rt * a.Hkv,
                        [&](int u, int z, int vb, int ve, bool last) {
                          run(u / n_rt, n_rt - 1 - u % n_rt, z, vb, ve, last);
                        });
  } else {
    if (vv >= n_rt * a.Hkv * ns) return;
    run(vv / (ns * n_rt), n_rt - 1 - (vv / ns) % n_rt, vv % ns, -1, 0, false);
  }
}

// ----------------------------------------------------------------------------
// Fused split-K reduce + residual + RMSNorm (bf16 models), one block per row:
//   x[row] += sum_s part[s][row]      (fixed order; nothing to add if splits == 0)
//   y = g * x / sqrt(mean(x^2) + eps) written as bf16 hi/lo planes, or as one float16
//   plane into yh when f16out (skipped if yh == nullptr)
// H % 4 == 0 and H <= 8192.  NT threads per block: 256, or 1024 for few rows, where a
// thread's (at most two) float4 columns take each group of eight split partials in one
// round of loads, sixteen when every column fits the first pass of the threads, and narrow
// rows with many partials share the splits out over thread groups (below).
// ----------------------------------------------------------------------------
template <typename WT, int NT>
__global__ void __launch_bounds__(NT) residual_norm(const float* __restrict__ part, size_t split_stride, int splits,
                                                    float* __restrict__ x, int H, const WT* __restrict__ g,
                                                    float eps, u16* __restrict__ yh, u16* __restrict__ yl,
                                                    int ldy, int f16out, int* __restrict__ flags) {
  constexpr int J = 2048 / NT;   // float4 columns per thread
  __shared__ float red[NT / 64];
  const int row = blockIdx.x;
  const int H4 = H >> 2;
  float4* xr = reinterpret_cast<float4*>(x + (size_t)row * H);
  const float4* pr = splits > 0 ? reinterpret_cast<const float4*>(part + (size_t)row * H) : nullptr;
  float4 v[J];
  float ss = 0.f;
  if constexpr (J <= 2) {
    bool ok[J];
    // More than one round of partials and at most half as many columns as threads (whole
    // waves of them): G groups of H/4 threads each sum a contiguous share of the splits (in
    // split order), and the shares are added to x in group order, so each thread waits on
    // fewer rounds of loads.  A group is whole waves, so its share is wave-uniform.
    const int G = (splits > 8 && H4 % 64 == 0) ? (H4 <= NT / 4 ? 4 : (H4 <= NT / 2 ? 2 : 1)) : 1;
    if (G > 1) {
      __shared__ float4 gsum[3 * (NT / 4)];   // shares of groups 1 .. G-1: (G - 1) * H4 <= 3 NT / 4
      const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / H4), k = threadIdx.x - grp * H4;
      const bool act = grp < G;
      const int sb = (int)(((long)grp * splits) / G), se = (int)(((long)(grp + 1) * splits) / G);
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s0 = sb; act && s0 < se; s0 += 8) {
        float4 b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < se) b[u] = pr[(s0 + u) * (split_stride >> 2) + k];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < se) { a.x += b[u].x; a.y += b[u].y; a.z += b[u].z; a.w += b[u].w; }
      }
      if (act && grp > 0) gsum[(grp - 1) * H4 + k] = a;
      __syncthreads();
      ok[0] = grp == 0;   // then k == threadIdx.x < H4
      v[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok[0]) {
        const float4 xv = xr[k];
        v[0] = make_float4(xv.x + a.x, xv.y + a.y, xv.z + a.z, xv.w + a.w);
        for (int gi = 1; gi < G; ++gi) {
          const float4 c = gsum[(gi - 1) * H4 + k];
          v[0].x += c.x; v[0].y += c.y; v[0].z += c.z; v[0].w += c.w;
        }
      }
#pragma unroll
      for (int j = 1; j < J; ++j) {
        ok[j] = false;
        v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    } else if (H4 <= NT) {
      // every column in the thread's first slot: rounds of sixteen partials.  Whole waves past
      // the columns skip the loads; inside a wave the loads are unconditional (lanes past the
      // columns read the last one and drop it), so a round goes out without lane branches.
      ok[0] = threadIdx.x < H4;
      const int kc = ok[0] ? threadIdx.x : H4 - 1;
      v[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      if ((threadIdx.x & ~63) < H4) {
        v[0] = xr[kc];
        for (int s0 = 0; s0 < splits; s0 += 16) {   // partials summed in split order
          float4 b[16];
#pragma unroll
          for (int u = 0; u < 16; ++u)
            if (s0 + u < splits) b[u] = pr[(s0 + u) * (split_stride >> 2) + kc];
#pragma unroll
          for (int u = 0; u < 16; ++u)
            if (s0 + u < splits) { v[0].x += b[u].x; v[0].y += b[u].y; v[0].z += b[u].z; v[0].w += b[u].w; }
        }
        if (!ok[0]) v[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 1; j < J; ++j) {
        ok[j] = false;
        v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    } else {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int k = threadIdx.x + NT * j;
      ok[j] = k < H4;
      v[j] = ok[j] ? xr[k] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int s0 = 0; s0 < splits; s0 += 8) {   // partials summed in split order
      float4 b[J][8];
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (ok[j] && s0 + u < splits) b[j][u] = pr[(s0 + u) * (split_stride >> 2) + threadIdx.x + NT * j];
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (ok[j] && s0 + u < splits) {
            v[j].x += b[j][u].x; v[j].y += b[j][u].y; v[j].z += b[j][u].z; v[j].w += b[j][u].w;
          }
    }
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (ok[j]) {
        if (splits > 0) xr[threadIdx.x + NT * j] = v[j];
        ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
      }
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int k = threadIdx.x + NT * j;
      if (k < H4) {
        float4 a = xr[k];
        // partials summed in split order; loaded eight at a time so their loads overlap
        for (int s0 = 0; s0 < splits; s0 += 8) {
          float4 b[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (s0 + u < splits) b[u] = pr[(s0 + u) * (split_stride >> 2) + k];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (s0 + u < splits) { a.x += b[u].x; a.y += b[u].y; a.z += b[u].z; a.w += b[u].w; }
        }
        if (splits > 0) xr[k] = a;
        v[j] = a;
        ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
      }
    }
  }
  if (yh == nullptr) return;
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  ss = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) ss += red[w];
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int k = threadIdx.x + NT * j;
    if (k < H4) {
      const float in[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      const size_t o = (size_t)row * ldy + 4 * k;
      if (f16out) {   // one float16 plane
        f16x4 y4;
        bool bad = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y = ldw(g, 4 * k + e) * (in[e] * r);
          bad |= f16_out_of_range(y);
          y4[e] = (f16)y;
        }
        *reinterpret_cast<f16x4*>(yh + o) = y4;
        flag_f16_range(flags, bad);
        continue;
      }
      u16 h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y = ldw(g, 4 * k + e) * (in[e] * r);
        h[e] = f32_to_bf16(y);
        l[e] = f32_to_bf16(y - bf16_to_f32(h[e]));
      }
      *reinterpret_cast<uint2*>(yh + o) =
          make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
      *reinterpret_cast<uint2*>(yl + o) =
          make_uint2((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16));
    }
  }
}

// ----------------------------------------------------------------------------
// RoPE table for the rows of one forward: cs[t][i] = (cos, sin)(pos[t] * theta^(-2i/D)) for
// the D/2 pairs of a head (i < D/2 of 64 slots), angle and sin/cos in float64; shared by
// every layer of the forward.
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) rope_table(const int* __restrict__ pos, int T, int D, double log2_theta,
                                                  float2* __restrict__ cs) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * 64) return;
  const int t = idx >> 6, i = idx & 63;
  if (2 * i >= D) return;
  double sd, cd;
  sincos((double)pos[t] * exp2(-(2.0 * i / D) * log2_theta), &sd, &cd);
  cs[idx] = make_float2((float)cd, (float)sd);
}

// ----------------------------------------------------------------------------
// Fused split-K reduce + RoPE + KV layout for the q|k|v projection.
// src: projection output [T][(Hq+2Hkv)*D] (splits == 1) or its split partials, D = 64 or
// 128.  The attention's heads are 128 wide: a 64-dim head is written zero-padded (q and K
// dims [D, 128), V^T rows [D, 128)).
// Grid (ceil(T/16), Hq + 2 Hkv): y < Hq + Hkv rotates head y over 16 rows (q as
// f16 hi + lo, k as f16 into K[hk][ldk][128]); the last Hkv values of y
// transpose one kv head's V over 16 rows into Vt[hk][128][ldv] via LDS.
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) qkv_post(const float* __restrict__ src, int lds, size_t split_stride,
                                                int splits, int T, int Hq, int Hkv,
                                                const float2* __restrict__ cs,
                                                f16* __restrict__ q_hi, f16* __restrict__ q_lo,
                                                f16* __restrict__ kdst, int ldk, f16* __restrict__ vtdst,
                                                int ldv, int D, float qscale, int* __restrict__ flags) {
  __shared__ float vt[16][129];
  bool bad = false;
  const int t0 = blockIdx.x * 16;
  const int nqk = Hq + Hkv;
  const int h = blockIdx.y;
  // The thread's N float4 groups (offsets off[n] into a partial, valid ok[n]) summed over the
  // split partials in split order; every group's loads of a set of four partials go out in
  // one round.  The loads are unconditional (invalid groups read offset 0, splits past the
  // last re-read the last), so none waits on a branch; only the sums are selected.
  auto ld_all = [&](auto& val, const auto& off, const auto& ok) {
    constexpr int N = sizeof(val) / sizeof(float4);
    auto at4 = [&](size_t o) { return *reinterpret_cast<const float4*>(src + o); };
    size_t o[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      o[n] = ok[n] ? off[n] : 0;
      const float4 a = at4(o[n]);
      val[n] = ok[n] ? a : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int s0 = 1; s0 < splits; s0 += 4) {
      float4 b[N][4];
#pragma unroll
      for (int n = 0; n < N; ++n)
#pragma unroll
        for (int u = 0; u < 4; ++u) b[n][u] = at4(min(s0 + u, splits - 1) * split_stride + o[n]);
#pragma unroll
      for (int n = 0; n < N; ++n)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (ok[n] && s0 + u < splits) {
            val[n].x += b[n][u].x; val[n].y += b[n][u].y; val[n].z += b[n][u].z; val[n].w += b[n][u].w;
          }
    }
  };
  if (h < nqk) {
    const int half = D >> 1;
    // row t0 + rr, rotation slots i0 .. i0 + 3 (the pairs (i, i + D/2)); slots at or past D/2
    // (64-dim heads) write the zero padding of dims [D, 128)
    const int rr = threadIdx.x >> 4, i0 = 4 * (threadIdx.x & 15);
    const int t = t0 + rr;
    float4 val[2];
    size_t off[2];
    bool ok[2];
    ok[0] = ok[1] = t < T && i0 < half;
    off[0] = (size_t)t * lds + h * D + i0;
    off[1] = off[0] + half;
    ld_all(val, off, ok);
    if (t < T) {
      const float av[4] = {val[0].x, val[0].y, val[0].z, val[0].w};
      const float bv[4] = {val[1].x, val[1].y, val[1].z, val[1].w};
      float ra[4] = {0.f, 0.f, 0.f, 0.f}, rb[4] = {0.f, 0.f, 0.f, 0.f};
      int da = D + (i0 - half), db = D + half + (i0 - half);
      if (i0 < half) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 c = cs[t * 64 + i0 + e];
          ra[e] = av[e] * c.x - bv[e] * c.y;
          rb[e] = bv[e] * c.x + av[e] * c.y;
        }
        da = i0;
        db = i0 + half;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) bad |= f16_out_of_range(ra[e]) || f16_out_of_range(rb[e]);
      if (h < Hq) {
        // operand-ordered layout (see AttnArgs): row r = t*G + g of KV head h / G; dims d..d+3
        // (d % 4 == 0) are 4 consecutive elements
        const int G = Hq / Hkv, r = t * G + h % G;
        const size_t base = ((size_t)(h / G) * attn_q_rows(T, G) + (r & ~31)) * 128 + (size_t)(r & 31) * 8;
        auto at = [&](int d) { return base + (size_t)(((d >> 4) * 2 + ((d >> 3) & 1)) * 256) + (d & 7); };
        // q carries the softmax scale log2(e)/sqrt(D): scores come out in log2 units
        f16x4 qa, qb, la, lb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sa = ra[e] * qscale, sb = rb[e] * qscale;
          qa[e] = (f16)sa;
          qb[e] = (f16)sb;
          la[e] = (f16)(sa - (float)qa[e]);
          lb[e] = (f16)(sb - (float)qb[e]);
        }
        *reinterpret_cast<f16x4*>(q_hi + at(da)) = qa;
        *reinterpret_cast<f16x4*>(q_hi + at(db)) = qb;
        if (q_lo) {
          *reinterpret_cast<f16x4*>(q_lo + at(da)) = la;
          *reinterpret_cast<f16x4*>(q_lo + at(db)) = lb;
        }
      } else {
        f16* kd = kdst + ((size_t)(h - Hq) * ldk + t) * 128;
        f16x4 ka, kb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ka[e] = (f16)ra[e];
          kb[e] = (f16)rb[e];
        }
        *reinterpret_cast<f16x4*>(kd + da) = ka;
        *reinterpret_cast<f16x4*>(kd + db) = kb;
      }
    }
  } else {
    const int hk = h - nqk;
    const int c0 = nqk * D + hk * D;
    // rows t0 + rr and t0 + rr + 8, dims d4 .. d4 + 3
    const int rr = threadIdx.x >> 5, d4 = 4 * (threadIdx.x & 31);
    float4 val[2];
    size_t off[2];
    bool ok[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = t0 + rr + 8 * j;
      ok[j] = t < T && d4 < D;
      off[j] = (size_t)t * lds + c0 + d4;
    }
    ld_all(val, off, ok);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float v4[4] = {val[j].x, val[j].y, val[j].z, val[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt[rr + 8 * j][d4 + e] = v4[e];
        bad |= f16_out_of_range(v4[e]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = threadIdx.x + 256 * j;
      const int d = idx >> 4, rr = idx & 15;
      const int t = t0 + rr;
      // columns up to the next multiple of 8 are written (zeros past T): attention reads V^T in 8-key chunks
      if (t < ((T + 7) & ~7)) vtdst[((size_t)hk * 128 + d) * ldv + t] = (f16)vt[rr][d];
    }
  }
  flag_f16_range(flags, bad);
}

// Combine split partials: o = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M), written as
// bf16 hi/lo planes or (f16out) one float16 plane.  chunk > 0 (balanced schedule): the row's
// row tile holds the slots [0, number of blocks on its tile sequence), found from the same
// layout the attention used (nt_u nominal tiles per row tile, chunk tiles per block).
template <int MAXS>
__global__ void __launch_bounds__(256) attn_merge(const float* __restrict__ o_part,
                                                  const float* __restrict__ lse_part, int S, int T, int Hq,
                                                  int D, int Dp, u16* __restrict__ oh, u16* __restrict__ ol,
                                                  int f16out, int G, int nt_u, int chunk) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;   // one float4 of one (t, hq)
  const int d4 = D >> 2;
  if (i >= (size_t)T * Hq * d4) return;
  const size_t th = i / d4;
  const int c = (int)(i % d4);
  if (chunk > 0) {
    const int t = (int)(th / Hq), hq = (int)(th % Hq);
    const int n_rt = (G * T + AT_BR - 1) / AT_BR;
    S = attn_balanced_item_slots((hq / G) * n_rt + (n_rt - 1 - (t * G + hq % G) / AT_BR), chunk, nt_u);
  }
  // every split's lse and partial are loaded up front (S <= MAXS), so the loads are in
  // flight together instead of one round trip per split
  float lse[MAXS];
  float4 part[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (s < S) {
      lse[s] = lse_part[(size_t)s * T * Hq + th];
      part[s] = reinterpret_cast<const float4*>(o_part + ((size_t)s * T * Hq + th) * Dp)[c];
    }
  }
  float M = NEG_INF;
#pragma unroll
  for (int s = 0; s < MAXS; ++s)
    if (s < S) M = fmaxf(M, lse[s]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  if (M != NEG_INF) {
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      if (s < S && lse[s] != NEG_INF) {
        const float w = __builtin_amdgcn_exp2f(lse[s] - M);
        acc.x += w * part[s].x; acc.y += w * part[s].y; acc.z += w * part[s].z; acc.w += w * part[s].w;
        wsum += w;
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const float v[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  const size_t at4 = th * D + 4 * c;
  if (f16out) {   // one float16 plane
    f16x4 v4;
#pragma unroll
    for (int j = 0; j < 4; ++j) v4[j] = (f16)v[j];
    *reinterpret_cast<f16x4*>(oh + at4) = v4;
    return;
  }
  u16 h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = f32_to_bf16(v[j]);
    l[j] = f32_to_bf16(v[j] - bf16_to_f32(h[j]));
  }
  *reinterpret_cast<uint2*>(oh + at4) =
      make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
  *reinterpret_cast<uint2*>(ol + at4) =
      make_uint2((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16));
}

// ----------------------------------------------------------------------------
// float32 attention (float32 models): one thread per (row t, q head), online
// softmax over the prefix keys then the row's own visible keys; writes o directly.
// ----------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(64) attn_fwd_f32(AttnArgsF a) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= a.T * a.Hq) return;
  const int t = i / a.Hq, hq = i % a.Hq;
  const int hk = hq / a.G;
  float q[D], acc[D];
  const float* qp = a.q + ((size_t)t * a.Hq + hq) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) { q[d] = qp[d] * a.scale; acc[d] = 0.f; }
  float m = NEG_INF, l = 0.f;
  auto visit = [&](const float* krow, const float* vcol, int ldv) {
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(q[d], krow[d], s);
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn);
    const float p = expf(s - mn);
    l = l * al + p;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = acc[d] * al + p * vcol[(size_t)d * ldv];
    m = mn;
  };
  const float* Kp = a.kp + (size_t)hk * a.ldp * D;
  const float* Vp = a.vtp + (size_t)hk * D * a.ldp;
  const int pb = a.pseg ? a.pseg[t].x : 0, pe = a.pseg ? a.pseg[t].y : a.P;
  for (int j = pb; j < pe; ++j) visit(Kp + (size_t)j * D, Vp + j, a.ldp);
  const float* Ks = a.ks + (size_t)hk * a.lds * D;
  const float* Vs = a.vts + (size_t)hk * D * a.lds;
  const int st = a.seq_start[t];
  const uint64_t mk = a.mask ? a.mask[t] : 0ull;
  for (int j = st; j <= t; ++j) {
    if (a.mask && !((mk >> ((j - st) & 63)) & 1ull)) continue;
    visit(Ks + (size_t)j * D, Vs + j, a.lds);
  }
  float* op = a.o + (size_t)t * a.Hq * D + (size_t)hq * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
}

// ----------------------------------------------------------------------------
// SwiGLU: u[t][i] = silu(gu[t][i]) * gu[t][I + i]
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) silu_mul(const float* __restrict__ gu, int T, int I,
                                                float* __restrict__ u, u16* __restrict__ uh,
                                                u16* __restrict__ ul) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)T * I) return;
  const size_t t = i / I, c = i % I;
  const float g = gu[t * 2 * I + c], up = gu[t * 2 * I + I + c];
  const float v = g / (1.0f + expf(-g)) * up;
  if (u) u[i] = v;
  if (uh) {
    const u16 h = f32_to_bf16(v);
    uh[i] = h;
    ul[i] = f32_to_bf16(v - bf16_to_f32(h));
  }
}

// ----------------------------------------------------------------------------
// K7: candidate logits z[p] = h[ridx[p]] · W_lm[tok[p]] (float32 accumulate),
// one wave per target; tok < 0 marks an unused slot (z = -inf).  bf16 rows (vec): 16 B
// loads, eight elements per lane and step.
// ----------------------------------------------------------------------------
template <typename WT>
__global__ void __launch_bounds__(256) target_logits(const float* __restrict__ h, int H,
                                                     const WT* __restrict__ W, const int* __restrict__ ridx,
                                                     const int* __restrict__ tok, int NT,
                                                     float* __restrict__ z, int vec) {
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (p >= NT) return;
  const int w = tok[p];
  if (w < 0) {
    if (lane == 0) z[p] = NEG_INF;
    return;
  }
  const float* hr = h + (size_t)ridx[p] * H;
  const WT* wr = W + (size_t)w * H;
  float s = 0.f;
  if constexpr (sizeof(WT) == 2) {
    if (vec) {   // H % 8 == 0, h and W 16 B aligned
      // bf16 rows: 8 consecutive elements per lane and step (16 B of W, 32 B of h), the
      // loads of up to four steps issued together
      for (int k0 = lane * 8; k0 < H; k0 += 64 * 8 * 4) {
        u16x8_t wv[4];
        float4 ha[4], hb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = min(k0 + q * 512, H - 8);
          wv[q] = *reinterpret_cast<const u16x8_t*>(wr + k);
          ha[q] = *reinterpret_cast<const float4*>(hr + k);
          hb[q] = *reinterpret_cast<const float4*>(hr + k + 4);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (k0 + q * 512 < H) {
            const float hv[8] = {ha[q].x, ha[q].y, ha[q].z, ha[q].w, hb[q].x, hb[q].y, hb[q].z, hb[q].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) s = fmaf(hv[e], bf16_to_f32(wv[q][e]), s);
          }
      }
      s = wave_sum(s);
      if (lane == 0) z[p] = s;
      return;
    }
  }
  for (int k = lane; k < H; k += 64) s = fmaf(hr[k], ldw(wr, k), s);
  s = wave_sum(s);
  if (lane == 0) z[p] = s;
}

// out[b][c] = z[b*C + c] - logsumexp_{c < n_b} z[b*C + c]; slots c >= n_b are -inf.
__global__ void cand_logsoftmax(const float* __restrict__ z, const int* __restrict__ n_cands, int B, int C,
                                float* __restrict__ out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int n = n_cands[b];
  const float* zb = z + (size_t)b * C;
  float m = NEG_INF;
  for (int c = 0; c < n; ++c) m = fmaxf(m, zb[c]);
  float s = 0.f;
  for (int c = 0; c < n; ++c) s += expf(zb[c] - m);
  const float lse = m + logf(s);
  for (int c = 0; c < C; ++c) out[(size_t)b * C + c] = (c < n) ? zb[c] - lse : NEG_INF;
}

// Row-wise log-sum-exp (natural log) from 128-column slice partials (max, sum of exp):
// lse = M + log(sum_p s_p * exp(m_p - M)), M the largest slice max; one block per row,
// slices combined in a fixed order.
__global__ void __launch_bounds__(256) lse_merge(const float2* __restrict__ part, int nparts, int R,
                                                 float* __restrict__ lse) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  if (r >= R) return;
  const float2* p = part + (size_t)r * nparts;
  float m = NEG_INF;
  for (int k = threadIdx.x; k < nparts; k += 256) m = fmaxf(m, p[k].x);
  m = wave_max(m);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) red[w] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = 0.f;
  if (m != NEG_INF)
    for (int k = threadIdx.x; k < nparts; k += 256) {
      const float2 v = p[k];
      if (v.x != NEG_INF) s += v.y * expf(v.x - m);
    }
  s = block_sum256(s, red);
  if (threadIdx.x == 0) lse[r] = m + logf(s);
}

// float32 models: the same slice partials straight from h and the float32 LM head, one
// block of 128 threads per (slice, row), one column per thread.
__global__ void __launch_bounds__(128) lmhead_lse_f32(const float* __restrict__ h, int H,
                                                      const float* __restrict__ W, int V, int nparts,
                                                      float2* __restrict__ part) {
  __shared__ float red[2];
  const int slice = blockIdx.x, r = blockIdx.y;
  const int col = slice * 128 + threadIdx.x;
  const float* hr = h + (size_t)r * H;
  float z = NEG_INF;
  if (col < V) {
    const float* wr = W + (size_t)col * H;
    float acc = 0.f;
    for (int k = 0; k < H; ++k) acc = fmaf(hr[k], wr[k], acc);
    z = acc;
  }
  float m = wave_max(z);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) red[w] = m;
  __syncthreads();
  m = fmaxf(red[0], red[1]);
  __syncthreads();
  float e = (col < V && m != NEG_INF) ? expf(z - m) : 0.f;
  e = wave_sum(e);
  if (l == 0) red[w] = e;
  __syncthreads();
  if (threadIdx.x == 0) part[(size_t)r * nparts + slice] = make_float2(m, red[0] + red[1]);
}

// Tree readout: score[q][c] = sum_k (z[t] - lse[ridx[t]]) over targets t = (q*C + c)*K + k
// with tok >= 0; norm = score - logsumexp over the question's candidates.  One block per question.
__global__ void tree_finalize(const float* __restrict__ z, const float* __restrict__ lse_rows,
                              const int* __restrict__ ridx, const int* __restrict__ tok,
                              const int* __restrict__ n_cands, int Q, int C, int K,
                              float* __restrict__ score, float* __restrict__ norm) {
  __shared__ float sc[64];
  const int q = blockIdx.x;
  const int c = threadIdx.x;
  if (q >= Q) return;
  const int n = n_cands[q];
  float s = NEG_INF;
  if (c < n) {
    double acc = 0.0;
    for (int k = 0; k < K; ++k) {
      const int tt = (q * C + c) * K + k;
      if (tok[tt] < 0) break;
      acc += (double)z[tt] - (double)lse_rows[ridx[tt]];
    }
    s = (float)acc;
  }
  if (c < 64) sc[c] = s;
  __syncthreads();
  if (c < C) {
    score[(size_t)q * C + c] = s;
    if (norm) {
      float m = NEG_INF;
      for (int j = 0; j < n; ++j) m = fmaxf(m, sc[j]);
      float e = 0.f;
      for (int j = 0; j < n; ++j) e += expf(sc[j] - m);
      norm[(size_t)q * C + c] = (c < n) ? s - (m + logf(e)) : NEG_INF;
    }
  }
}

}  // namespace jevk

// ============================================================================
// launch wrappers (host)
// ============================================================================
using namespace jevk;

static inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

hipError_t launch_embed(bool bf16, const void* E, const int* tok, int T, int H, const void* vis, float* x,
                        int* flags, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  auto al16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  const int vec = H % 8 == 0 && al16(E) && (vis == nullptr || al16(vis)) && al16(x);
  if (bf16)
    embed_rows<u16><<<T, 256, 0, s>>>((const u16*)E, tok, T, H, (const u16*)vis, x, flags, vec);
  else
    embed_rows<float><<<T, 256, 0, s>>>((const float*)E, tok, T, H, (const float*)vis, x, flags, 0);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(bool bf16, const float* x, int ldx, const int* rows, int n_rows, int H, const void* g,
                          float eps, float* y, uint16_t* yh, uint16_t* yl, int ldy, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  auto al16 = [](const void* p) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  const int vec = H % 4 == 0 && ldx % 4 == 0 && ldy % 4 == 0 && al16(x) && al16(y) && al16(yh) && al16(yl);
  if (bf16)
    rmsnorm_rows<u16><<<n_rows, 256, 0, s>>>(x, ldx, rows, n_rows, H, (const u16*)g, eps, y, yh, yl, ldy, vec);
  else
    rmsnorm_rows<float><<<n_rows, 256, 0, s>>>(x, ldx, rows, n_rows, H, (const float*)g, eps, y, yh, yl, ldy, vec);
  return hipGetLastError();
}

// Kernel and split-K choice.  The 128 x 256 kernel is used when its tiles with at
// most 4 K splits give about 1.5 blocks per CU (384 blocks) and each split keeps
// >= 512 of K; otherwise the 128 x 128 kernel with as many splits as fill one
// round of 512 resident blocks (2 per CU), at most 8, each >= 256 of K.  Split
// partials never exceed part_cap floats.  Chosen by measurement on the 2B/7B
// projection shapes.
GemmPlan gemm_bf16_plan(int M, int N, int K, size_t part_cap) {
  GemmPlan p{};
  const long t2 = (long)cdiv(M, G2M) * cdiv(N, G2N);
  int s2 = (int)((384 + t2 - 1) / t2);
  if (s2 <= 4 && K / s2 >= 512) {
    p.wide = true;
    p.splits = s2;
  } else {
    const long t1 = (long)cdiv(M, GBM) * cdiv(N, GBN);
    int s1 = (int)(512 / t1);
    s1 = std::min(s1, K / 256);
    p.wide = false;
    p.splits = std::max(1, std::min(s1, 8));
  }
  while (p.splits > 1 && (size_t)p.splits * M * N > part_cap) --p.splits;
  return p;
}

// Few-row plan (measured on the 7B and 2B projection shapes): about 1024 blocks of 128
// columns at first, each chunk at least 3 stages, at most 32 splits; then, while the grid
// exceeds 512 blocks and chunks are shorter than 1024 of K, fewer splits (long chunks keep
// the split partials, written here and read by the consumer, small); partials within
// part_cap floats.
static int skinny_splits(int M, int N, int K, size_t part_cap) {
  const long nt = cdiv(N, 128);
  long sp = std::max(1L, 1024 / nt);
  sp = std::min<long>(sp, std::max(1, K / (3 * SKS)));
  sp = std::min<long>(sp, 32);
  while (sp > 1 && sp * nt > 512 && K / sp < 1024) --sp;
  while (sp > 1 && (size_t)sp * M * N > part_cap) --sp;
  return (int)sp;
}

static hipError_t launch_skinny(bool f16, const uint16_t* Ah, const uint16_t* Al, int lda, int M, int K,
                                const GemmSegs& seg, int N, float* C, int ldc, int accum, size_t part_cap,
                                float* part, hipStream_t s, int* eff_splits) {
  const int sp = skinny_splits(M, N, K, part_cap);
  const int k_chunk = cdiv(cdiv(K, sp), SKS) * SKS;
  const int splits = cdiv(K, k_chunk);
  *eff_splits = splits;
  const int nt = cdiv(N, 128);
  float* out = splits == 1 ? C : part;
  const int ldo = splits == 1 ? ldc : N;
  const int acc = splits == 1 ? accum : 0;
  // two row groups: work item w runs as blocks 16 (w / 8) + w % 8 and that + 8
  const int rgs = M > 32 ? 2 : 1;
  const int items = nt * splits;
  const int grid = rgs == 2 ? cdiv(items, 8) * 16 : items;
  if (f16)
    gemm_skinny<true><<<grid, 256, 0, s>>>(Ah, nullptr, lda, M, K, seg, N, nt, splits, k_chunk, out, ldo,
                                           (size_t)M * N, acc, rgs);
  else
    gemm_skinny<false><<<grid, 256, 0, s>>>(Ah, Al, lda, M, K, seg, N, nt, splits, k_chunk, out, ldo, (size_t)M * N,
                                            acc, rgs);
  return hipGetLastError();
}

// the weight-streaming kernel takes products of at most 64 rows (two row groups past 32)
// with K a multiple of its stage
static bool use_skinny(int M, int K) { return M <= 64 && K % SKS == 0; }

hipError_t launch_gemm_bf16(const uint16_t* Ah, const uint16_t* Al, int lda, int M, int K, const GemmSegs& seg, int N,
                            float* C, int ldc, int accum, size_t part_cap, float* part, hipStream_t s,
                            int* eff_splits) {
  *eff_splits = 1;
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % G2K) return hipErrorInvalidValue;
  if (use_skinny(M, K)) return launch_skinny(false, Ah, Al, lda, M, K, seg, N, C, ldc, accum, part_cap, part, s, eff_splits);
  const GemmPlan pl = gemm_bf16_plan(M, N, K, part_cap);
  const int bk = pl.wide ? G2K : GBK;
  const int mt = cdiv(M, GBM), nt = cdiv(N, pl.wide ? G2N : GBN);
  const int k_chunk = cdiv(cdiv(K, pl.splits), bk) * bk;
  const int splits = cdiv(K, k_chunk);
  *eff_splits = splits;
  const int grid = cdiv(mt * nt * splits, 8) * 8;
  float* out = splits == 1 ? C : part;
  const int ldo = splits == 1 ? ldc : N;
  const int acc = splits == 1 ? accum : 0;
  if (pl.wide)
    gemm_bf16w<false, false><<<grid, 256, 0, s>>>(Ah, Al, lda, M, K, seg, N, mt, nt, splits, k_chunk, out, ldo,
                                           (size_t)M * N, acc, nullptr, nullptr, nullptr);
  else
    gemm_bf16s<false><<<grid, 256, 0, s>>>(Ah, Al, lda, M, K, seg, N, mt, nt, splits, k_chunk, out, ldo,
                                           (size_t)M * N, acc);
  return hipGetLastError();
}

hipError_t launch_gemm_swiglu(const uint16_t* Ah, const uint16_t* Al, int lda, int M, int K, const uint16_t* w_gate,
                              const uint16_t* w_up, int I, uint16_t* uh, uint16_t* ul, int ldu, int* flags,
                              hipStream_t s) {
  if (M <= 0 || I <= 0) return hipSuccess;
  if (K % G2K) return hipErrorInvalidValue;
  const int mt = cdiv(M, G2M), nt = cdiv(I, G2N / 2);
  const int grid = cdiv(mt * nt, 8) * 8;
  GemmSegs seg{{w_gate, w_up, nullptr}, {I, 2 * I, 2 * I}};
  // buffer-form loads while every byte offset they form fits the 31-bit range
  if ((size_t)M * lda * 2 < (1ull << 31) && (size_t)I * K * 2 < (1ull << 31))
    gemm_bf16w<true, false, false, true><<<grid, 256, 0, s>>>(Ah, Al, lda, M, K, seg, I, mt, nt, 1, K, nullptr, ldu,
                                                              0, 0, uh, ul, flags);
  else
    gemm_bf16w<true, false><<<grid, 256, 0, s>>>(Ah, Al, lda, M, K, seg, I, mt, nt, 1, K, nullptr, ldu, 0, 0, uh, ul,
                                                  flags);
  return hipGetLastError();
}

// Single-pass float16 GEMMs: the activation as one float16 plane, W the float16 mirror.
// The 128 x 256 kernel as a rule; K splits bring the grid to about 448 blocks (1.75 per
// CU), at most 16, each >= 256 of K (measured on the 7B / 2B projection shapes, split-K
// consumer included).
GemmPlan gemm_f16_plan(int M, int N, int K, size_t part_cap) {
  GemmPlan p{};
  p.wide = true;
  const long t = (long)cdiv(M, G2M) * cdiv(N, G2N);
  long sp = (448 + t / 2) / t;
  // one row tile (few rows: streaming the weights bounds it) may split K up to 32 ways
  sp = std::min<long>(sp, std::min(M <= G2M ? 32 : 16, std::max(1, K / 256)));
  p.splits = (int)std::max<long>(1, sp);
  // The 128 x 128 kernel instead (gemm_bf16s<true>) when the wide tiles leave the chip
  // under-filled even with their splits (fewer than 256 blocks: the 2B scoring call's down
  // projection of 129 rows, 192 -> 456 blocks), or split a short K (<= 4608) four or more
  // ways, where writing and summing the partials costs more than the wider tile saves (the
  // 1024-row o projection: 54.4 -> 46.9 us).  Three splits stay wide (the 1024-row q|k|v ran
  // 13% slower on unsplit narrow tiles), as do long K (the 1024-row down projection).
  if (M > G2M && K % GBK == 0 && (t * p.splits < 256 || (p.splits >= 4 && K <= 4608))) {
    const long tn = (long)cdiv(M, GBM) * cdiv(N, GBN);
    long sn = (448 + tn / 2) / tn;
    sn = std::min<long>(sn, std::max(1L, 512 / tn));
    sn = std::min<long>(sn, std::max(1, K / 256));
    p.wide = false;
    p.splits = (int)std::max<long>(1, sn);
  }
  while (p.splits > 1 && (size_t)p.splits * M * N > part_cap) --p.splits;
  return p;
}

hipError_t launch_gemm_f16(const uint16_t* A, int lda, int M, int K, const GemmSegs& seg, int N, float* C, int ldc,
                           int accum, size_t part_cap, float* part, hipStream_t s, int* eff_splits) {
  *eff_splits = 1;
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % G2K) return hipErrorInvalidValue;
  if (use_skinny(M, K)) return launch_skinny(true, A, nullptr, lda, M, K, seg, N, C, ldc, accum, part_cap, part, s, eff_splits);
  const GemmPlan pl = gemm_f16_plan(M, N, K, part_cap);
  const int bk = pl.wide ? G2K : GBK;
  const int mt = cdiv(M, pl.wide ? G2M : GBM), nt = cdiv(N, pl.wide ? G2N : GBN);
  const int k_chunk = cdiv(cdiv(K, pl.splits), bk) * bk;
  const int splits = cdiv(K, k_chunk);
  *eff_splits = splits;
  const int grid = cdiv(mt * nt * splits, 8) * 8;
  float* out = splits == 1 ? C : part;
  const int ldo = splits == 1 ? ldc : N;
  const int acc = splits == 1 ? accum : 0;
  if (pl.wide)
    gemm_bf16w<false, true><<<grid, 256, 0, s>>>(A, nullptr, lda, M, K, seg, N, mt, nt, splits, k_chunk, out, ldo,
                                                 (size_t)M * N, acc, nullptr, nullptr, nullptr);
  else
    gemm_bf16s<true><<<grid, 256, 0, s>>>(A, nullptr, lda, M, K, seg, N, mt, nt, splits, k_chunk, out, ldo,
                                          (size_t)M * N, acc);
  return hipGetLastError();
}

hipError_t launch_gemm_swiglu_f16(const uint16_t* A, int lda, int M, int K, const uint16_t* w_gate,
                                  const uint16_t* w_up, int I, uint16_t* uh, uint16_t* ul, int ldu, int* flags,
                                  hipStream_t s) {
  if (M <= 0 || I <= 0) return hipSuccess;
  if (K % G2K) return hipErrorInvalidValue;
  const int mt = cdiv(M, G2M), nt = cdiv(I, G2N / 2);
  const int grid = cdiv(mt * nt, 8) * 8;
  GemmSegs seg{{w_gate, w_up, nullptr}, {I, 2 * I, 2 * I}};
  // buffer-form loads while every byte offset they form fits the 31-bit range
  if ((size_t)M * lda * 2 < (1ull << 31) && (size_t)I * K * 2 < (1ull << 31))
    gemm_bf16w<true, true, false, true><<<grid, 256, 0, s>>>(A, nullptr, lda, M, K, seg, I, mt, nt, 1, K, nullptr, ldu,
                                                             0, 0, uh, ul, flags);
  else
    gemm_bf16w<true, true><<<grid, 256, 0, s>>>(A, nullptr, lda, M, K, seg, I, mt, nt, 1, K, nullptr, ldu, 0, 0, uh,
                                                ul, flags);
  return hipGetLastError();
}

// bfloat16 -> float16 copy of a weight matrix (n % 8 == 0); *bad = 1 if a finite value
// falls outside the float16 range.
__global__ void __launch_bounds__(256) bf16_to_f16(const u16* __restrict__ src, size_t n8, u16* __restrict__ dst,
                                                   int* __restrict__ bad) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
    const uint4 v = reinterpret_cast<const uint4*>(src)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
    bool out_of_range = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_to_f32((u16)(w[j] & 0xFFFF)), b = bf16_to_f32((u16)(w[j] >> 16));
      out_of_range |= (fabsf(a) > 65504.f && isfinite(a)) || (fabsf(b) > 65504.f && isfinite(b));
      const f16 ha = (f16)a, hb = (f16)b;
      o[j] = (uint32_t)__builtin_bit_cast(u16, ha) | ((uint32_t)__builtin_bit_cast(u16, hb) << 16);
    }
    reinterpret_cast<uint4*>(dst)[i] = make_uint4(o[0], o[1], o[2], o[3]);
    if (out_of_range) *bad = 1;
  }
}

bool swiglu_use_split(int M, int I, size_t part_cap) {
  const long fused_blocks = (long)cdiv(M, G2M) * cdiv(I, G2N / 2);
  return fused_blocks < 256 && (size_t)M * 2 * I <= part_cap && I % 4 == 0;
}

hipError_t launch_splitk_swiglu(const float* part, int splits, int M, int I, uint16_t* uh, uint16_t* ul, int ldu,
                                int* flags, hipStream_t s) {
  if (M <= 0 || I <= 0) return hipSuccess;
  if (I % 4 || ldu % 4 || splits < 1) return hipErrorInvalidValue;
  splitk_swiglu<<<cdiv((long)M * (I / 4), 256), 256, 0, s>>>(part, (size_t)M * 2 * I, splits, M, I, uh, ul, ldu, flags);
  return hipGetLastError();
}

hipError_t launch_bf16_to_f16(const uint16_t* src, size_t n, uint16_t* dst, int* bad, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  const size_t n8 = n / 8;
  const int grid = (int)std::min<size_t>(4096, (n8 + 255) / 256);
  bf16_to_f16<<<grid, 256, 0, s>>>(src, n8, dst, bad);
  return hipGetLastError();
}

hipError_t launch_residual_norm(bool bf16, const float* part, size_t split_stride, int splits, float* x, int M,
                                int H, const void* g, float eps, uint16_t* yh, uint16_t* yl, int ldy, bool f16out,
                                int* flags, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (H % 4 || H > 8192 || split_stride % 4) return hipErrorInvalidValue;
  // few rows: 1024 threads per row, so each thread's partial loads go out in one round
  const bool wide = M <= 64;
  if (bf16) {
    if (wide)
      residual_norm<u16, 1024><<<M, 1024, 0, s>>>(part, split_stride, splits, x, H, (const u16*)g, eps, yh, yl, ldy,
                                                  f16out, flags);
    else
      residual_norm<u16, 256><<<M, 256, 0, s>>>(part, split_stride, splits, x, H, (const u16*)g, eps, yh, yl, ldy,
                                                f16out, flags);
  } else {
    if (wide)
      residual_norm<float, 1024><<<M, 1024, 0, s>>>(part, split_stride, splits, x, H, (const float*)g, eps, yh, yl,
                                                    ldy, f16out, flags);
    else
      residual_norm<float, 256><<<M, 256, 0, s>>>(part, split_stride, splits, x, H, (const float*)g, eps, yh, yl,
                                                  ldy, f16out, flags);
  }
  return hipGetLastError();
}

hipError_t launch_rope_table(const int* pos, int T, int D, double log2_theta, float2* cs, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (D != 64 && D != 128) return hipErrorInvalidValue;
  rope_table<<<cdiv((long)T * 64, 256), 256, 0, s>>>(pos, T, D, log2_theta, cs);
  return hipGetLastError();
}

hipError_t launch_qkv_post(const float* src, int lds, size_t split_stride, int splits, int T, int Hq, int Hkv,
                           const float2* cs, void* q_hi, void* q_lo, void* kdst, int ldk, void* vtdst, int ldv,
                           int D, float qscale, int* flags, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if ((D != 64 && D != 128) || lds % 4 || split_stride % 4) return hipErrorInvalidValue;
  dim3 grid(cdiv(T, 16), Hq + 2 * Hkv);
  qkv_post<<<grid, 256, 0, s>>>(src, lds, split_stride, splits, T, Hq, Hkv, cs, (f16*)q_hi, (f16*)q_lo, (f16*)kdst,
                                ldk, (f16*)vtdst, ldv, D, qscale, flags);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* part, int splits, int M, int N, float* C, int ldc, int accum,
                                hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  splitk_reduce<<<cdiv((long)M * N, 256), 256, 0, s>>>(part, (size_t)M * N, splits, M, N, N, C, ldc, accum);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const float* A, int lda, int M, int K, const GemmSegsF& seg, int N, float* C, int ldc,
                           int accum, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  dim3 grid(cdiv(N, 64), cdiv(M, 64));
  gemm_f32<<<grid, 256, 0, s>>>(A, lda, M, K, seg, N, C, ldc, accum);
  return hipGetLastError();
}

hipError_t launch_rope_qk(bool f16out, const float* qkv, int T, int Hq, int Hkv, int D, const int* pos,
                          double log2_theta, void* q_out, void* q_lo, void* k_out, int ldk, int row0, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (f16out)
    rope_qk<f16><<<T, 256, 0, s>>>(qkv, T, Hq, Hkv, D, pos, log2_theta, (f16*)q_out, (f16*)q_lo, (f16*)k_out, ldk,
                                   row0);
  else
    rope_qk<float><<<T, 256, 0, s>>>(qkv, T, Hq, Hkv, D, pos, log2_theta, (float*)q_out, (float*)q_lo,
                                     (float*)k_out, ldk, row0);
  return hipGetLastError();
}

hipError_t launch_v_transpose(bool f16out, const float* src, int lds, int T, int HD, void* vt, int ldv, int col0,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dim3 grid(cdiv(T, 64), cdiv(HD, 64));
  if (f16out)
    v_transpose<f16><<<grid, 256, 0, s>>>(src, lds, T, HD, (f16*)vt, ldv, col0);
  else
    v_transpose<float><<<grid, 256, 0, s>>>(src, lds, T, HD, (float*)vt, ldv, col0);
  return hipGetLastError();
}

int attn_own_tiles(const int* seq_start, int T, int G) {
  const int R = G * T;
  int mx = 0;
  for (int r0 = 0; r0 < R; r0 += AT_BR) {
    const int t_first = r0 / G, t_last = std::min(R - 1, r0 + AT_BR - 1) / G;
    mx = std::max(mx, cdiv(t_last + 1 - (seq_start[t_first] & ~7), AT_BK));
  }
  return mx;
}

int attn_seg_tiles(const int* pseg, int T, int G, int* ptile) {
  const int R = G * T;
  int mx = 0, x = 0;
  for (int r0 = 0; r0 < R; r0 += AT_BR, ++x) {
    const int t_first = r0 / G, t_last = std::min(R - 1, r0 + AT_BR - 1) / G;
    int lo = INT_MAX, hi = INT_MIN, vlo = INT_MIN, vhi = INT_MAX;
    for (int t = t_first; t <= t_last; ++t) {
      const int b = pseg[2 * t], e = pseg[2 * t + 1];
      if (e > b) {
        lo = std::min(lo, b);
        hi = std::max(hi, e);
      }
      vlo = std::max(vlo, b);
      vhi = std::min(vhi, e);
    }
    const int tb = (hi > lo) ? lo / AT_BK : 0, te = (hi > lo) ? cdiv(hi, AT_BK) : 0;
    ptile[4 * x] = tb;
    ptile[4 * x + 1] = te;
    ptile[4 * x + 2] = vlo;
    ptile[4 * x + 3] = vhi;
    mx = std::max(mx, te - tb);
  }
  return mx;
}

constexpr long kAttnResidentBlocks = 512;   // 256 CUs x 2 blocks of 4 waves

int attn_splits(int T, int G, int Hkv, int P, int own_tiles) {
  const long base = (long)cdiv((long)G * T, AT_BR) * Hkv;
  const int tiles = cdiv(P, AT_BK) + own_tiles;
  // About one block per compute unit; two (a full 8 waves per CU) once every split
  // keeps enough tiles to amortise the larger merge (measured: P = 1024 favours one,
  // P = 8192 two).
  const long target = tiles >= 64 ? 512 : 256;
  long ns = (target + base / 2) / base;
  // never past the blocks the chip holds at once (two per CU): a few blocks over it run
  // as a second round of their own (532 blocks took 21% longer than 504)
  ns = std::min<long>(ns, std::max(1L, kAttnResidentBlocks / base));
  ns = std::min<long>(ns, std::max(1, tiles / 2));     // at least two tiles per split
  return (int)std::max<long>(1, std::min<long>(ns, kAttnMaxSplits));
}


// Largest partial slot count of any row tile under the balanced schedule: a run of nt_u
// tiles starting anywhere meets at most floor((nt_u - 1) / chunk) + 2 blocks of chunk tiles.
static long attn_balanced_slots(long nt_u, long chunk) { return (nt_u - 1) / chunk + 2; }

AttnSchedule attn_schedule(int T, int G, int Hkv, int P, int own_tiles, bool segmented) {
  const int ns = attn_splits(T, G, Hkv, P, own_tiles);
  const AttnSchedule equal{ns, 0};
  if (segmented || P <= 0) return equal;
  const long base = (long)cdiv((long)G * T, AT_BR) * Hkv;
  const long nt_u = cdiv(P, AT_BK) + own_tiles;
  // the block count the equal splits aim at (as attn_splits); they fall short of it or load
  // the compute units unevenly when the row tiles do not divide it (376 blocks = 120 CUs
  // with two blocks, 136 with one: the launch takes as long as the two-block CUs)
  const long target = nt_u >= 64 ? kAttnResidentBlocks : kAttnResidentBlocks / 2;
  if (base * ns >= target * 7 / 8) return equal;
  const long chunk = cdiv(base * nt_u, target);
  // long runs only: a block pays a prologue per row tile it touches, and every row tile
  // more partials to merge
  if (chunk < 16 || chunk >= nt_u) return equal;
  const long slots = attn_balanced_slots(nt_u, chunk);
  if (slots > kAttnMaxSplits) return equal;
  return AttnSchedule{(int)slots, (int)chunk};
}

hipError_t launch_attn_f16(const AttnArgs& a, int q_terms, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.n_split < 1 || a.n_split > kAttnMaxSplits || (q_terms != 1 && q_terms != 2)) return hipErrorInvalidValue;
  long nb = (long)cdiv((long)a.G * a.T, AT_BR) * a.Hkv * a.n_split;
  if (a.sk_chunk > 0) {
    // one shared prefix only, and the slots a row tile may need within n_split
    const long nt_u = cdiv(a.P, AT_BK) + a.own_tiles;
    const long W = (long)cdiv((long)a.G * a.T, AT_BR) * a.Hkv * nt_u;
    if (a.ptile || a.P <= 0 || attn_balanced_slots(nt_u, a.sk_chunk) > a.n_split || W > INT_MAX / 2)
      return hipErrorInvalidValue;
    nb = cdiv(W, a.sk_chunk);
  }
  const int grid = (int)(cdiv(nb, 8) * 8);
  const bool bal = a.sk_chunk > 0;
  if (q_terms == 1) {
    if (bal) attn_fwd_f16<1, true><<<grid, 256, 0, s>>>(a);
    else attn_fwd_f16<1, false><<<grid, 256, 0, s>>>(a);
  } else {
    if (bal) attn_fwd_f16<2, true><<<grid, 256, 0, s>>>(a);
    else attn_fwd_f16<2, false><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_merge(const float* o_part, const float* lse_part, int S, int T, int Hq, int D, uint16_t* oh,
                             uint16_t* ol, bool f16out, int G, int P, int own_tiles, int chunk, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (S < 1 || S > kAttnMaxSplits || G < 1 || Hq % G) return hipErrorInvalidValue;
  const int nt_u = chunk > 0 ? cdiv(P, AT_BK) + own_tiles : 0;
  if (chunk > 0 && attn_balanced_slots(nt_u, chunk) > S) return hipErrorInvalidValue;
  const int grid = cdiv((long)T * Hq * (D / 4), 256);
  if (S <= 8)
    attn_merge<8><<<grid, 256, 0, s>>>(o_part, lse_part, S, T, Hq, D, 128, oh, ol, f16out, G, nt_u, chunk);
  else
    attn_merge<kAttnMaxSplits><<<grid, 256, 0, s>>>(o_part, lse_part, S, T, Hq, D, 128, oh, ol, f16out, G, nt_u,
                                                    chunk);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgsF& a, int D, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int n = a.T * a.Hq;
  if (D == 64)
    attn_fwd_f32<64><<<cdiv(n, 64), 64, 0, s>>>(a);
  else
    attn_fwd_f32<128><<<cdiv(n, 64), 64, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const float* gu, int T, int I, float* u, uint16_t* uh, uint16_t* ul, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  silu_mul<<<cdiv((long)T * I, 256), 256, 0, s>>>(gu, T, I, u, uh, ul);
  return hipGetLastError();
}

hipError_t launch_target_logits(bool bf16, const float* h, int H, const void* W, const int* ridx, const int* tok,
                                int NT, float* z, hipStream_t s) {
  if (NT <= 0) return hipSuccess;
  const int vec = H % 8 == 0 && reinterpret_cast<uintptr_t>(h) % 16 == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0;
  if (bf16)
    target_logits<u16><<<cdiv(NT, 4), 256, 0, s>>>(h, H, (const u16*)W, ridx, tok, NT, z, vec);
  else
    target_logits<float><<<cdiv(NT, 4), 256, 0, s>>>(h, H, (const float*)W, ridx, tok, NT, z, 0);
  return hipGetLastError();
}

hipError_t launch_cand_logsoftmax(const float* z, const int* n_cands, int B, int C, float* out, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  cand_logsoftmax<<<cdiv(B, 64), 64, 0, s>>>(z, n_cands, B, C, out);
  return hipGetLastError();
}

// Full-vocabulary LSE of R rows without storing their logits: slice partials [R][nparts]
// (nparts = ceil(V / 128)); launch_lse_merge combines them in a fixed order into lse[R].
hipError_t launch_lmhead_lse(bool bf16, const float* h, const uint16_t* h_hi, const uint16_t* h_lo, int H, int R,
                             const void* W, int V, float2* part, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  const int nparts = cdiv(V, 128);
  if (bf16) {
    if (H % G2K) return hipErrorInvalidValue;
    const int mt = cdiv(R, G2M), nt = cdiv(V, G2N);
    const int grid = cdiv((long)mt * nt, 8) * 8;
    GemmSegs seg{{static_cast<const uint16_t*>(W), nullptr, nullptr}, {V, V, V}};
    gemm_bf16w<false, false, true><<<grid, 256, 0, s>>>(h_hi, h_lo, H, R, H, seg, V, mt, nt, 1, H,
                                                         reinterpret_cast<float*>(part), nparts, 0, 0, nullptr,
                                                         nullptr, nullptr);
  } else {
    lmhead_lse_f32<<<dim3(nparts, R), 128, 0, s>>>(h, H, static_cast<const float*>(W), V, nparts, part);
  }
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float2* part, int R, int V, float* lse, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  lse_merge<<<R, 256, 0, s>>>(part, cdiv(V, 128), R, lse);
  return hipGetLastError();
}

hipError_t launch_tree_finalize(const float* z, const float* lse_rows, const int* ridx, const int* tok,
                                const int* n_cands, int Q, int C, int K, float* score, float* norm,
                                hipStream_t s) {
  if (Q <= 0) return hipSuccess;
  tree_finalize<<<Q, 64, 0, s>>>(z, lse_rows, ridx, tok, n_cands, Q, C, K, score, norm);
  return hipGetLastError();
}
