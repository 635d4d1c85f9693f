// Host-side declarations of the device kernels' launchers (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Up to three weight row segments forming one GEMM's N axis (e.g. wq | wk | wv).
// Segment s covers output columns [n_end[s-1], n_end[s]) (n_end[-1] = 0).
struct GemmSegs {
  const uint16_t* w[3];
  int n_end[3];
};
struct GemmSegsF {
  const float* w[3];
  int n_end[3];
};

// float16 attention (head_dim 128) of T query rows: prefix keys then the rows' own keys.
//
// q is stored in the order the attention kernel feeds it to the matrix cores: per KV
// head hk, query row r = t*G + g (head hq = hk*G + g) of R = G*T rows, padded to a
// multiple of 32 rows (attn_q_rows); in each group of 32 rows, element d of row
// 32w + l sits at ((d/16)*2 + (d/8)%2)*32*8 + l*8 + d%8 after the group's base, so
// each 16-dim slice of a group is one contiguous 1 KB run.
#if defined(__HIPCC__)
#define JEV_HD __host__ __device__
#else
#define JEV_HD
#endif
inline JEV_HD int attn_q_rows(int T, int G) { return (G * T + 31) / 32 * 32; }
inline size_t attn_q_plane_elems(int T, int Hq, int Hkv) {
  return (size_t)Hkv * attn_q_rows(T, Hq / Hkv) * 128;
}
struct AttnArgs {
  const _Float16* q;       // q * log2(e)/sqrt(128) rounded to f16 (hi), layout above
  const _Float16* q_lo;    // the rounding remainder as f16, same layout (two-term q only)
  int T, Hq, Hkv, G;
  const _Float16* kp;      // prefix K  [Hkv][ldp][128]
  const _Float16* vtp;     // prefix Vt [Hkv][128][ldp], columns [P, round8(P)) zero
  int P, ldp;
  const _Float16* ks;      // own K  [Hkv][lds][128]
  const _Float16* vts;     // own Vt [Hkv][128][lds], columns [T, round8(T)) zero
  int lds;
  const int* seq_start;    // [T] first row of the row's sequence / group
  const uint64_t* mask;    // [T] visibility over the group (nullptr: causal)
  // segmented prefixes (nullptr: every row sees prefix keys [0, P)): the row's prefix keys
  // [x, y), and per 128-row tile (attn_seg_tiles) its prefix key tiles [x, y) and the keys
  // [z, w) every row of the tile sees
  const int2* pseg;        // [T]
  const int4* ptile;       // [ceil(G*T / 128)]
  int n_split;             // splits of each row tile's key tiles, 1..kAttnMaxSplits (balanced
                           // schedule: the partial slots a row tile may need)
  int sk_chunk;            // > 0: balanced schedule, sk_chunk key tiles per block (attn_schedule)
  int own_tiles;           // bound on any row tile's own-key tiles (attn_own_tiles); the splits
                           // divide ceil(P/64) + own_tiles tiles
  float* o_part;           // [n_split][T][Hq][128]  (n_split > 1 or balanced; always 128 dims)
  float* lse_part;         // [n_split][T][Hq]       (log2 units; n_split > 1 or balanced)
  uint16_t* oh;            // [T][Hq*128] bf16 hi/lo planes of o (n_split == 1, not balanced) ...
  uint16_t* ol;
  int o_f16;               // ... or (non-zero) one float16 plane of o in oh
  int D;                   // the model's head dim (64 or 128): o is [T][Hq][D], the first D of
                           // the 128 computed dims (a 64-dim head runs zero-padded to 128)
};

// Balanced schedule (AttnArgs::sk_chunk = c > 0): the n_items (KV head, row tile) items'
// nominal tile sequences of nt_u tiles each laid end to end, block vv taking tiles
// [vv*c, (vv+1)*c) of them.  f(u, z, vb, ve, last) is called for each item u the block
// touches, in order: its tiles [vb, ve), z the block's partial slot for that item (its
// offset from the item's first block) and last whether the block ends the item.  The
// attention kernel and the host checks run this same enumeration.
template <typename F>
inline JEV_HD void attn_balanced_items(int vv, int c, int nt_u, int n_items, F&& f) {
  const int W = n_items * nt_u;
  const int w0 = vv * c, w1 = (W < w0 + c) ? W : w0 + c;
  for (int u = w0 / nt_u; u * nt_u < w1; ++u) {
    const int b0 = u * nt_u;
    f(u, vv - b0 / c, (w0 > b0 ? w0 : b0) - b0, (w1 < b0 + nt_u ? w1 : b0 + nt_u) - b0, b0 + nt_u <= w1);
  }
}
// The partial slots item u holds under the balanced schedule: the blocks its tiles meet.
inline JEV_HD int attn_balanced_item_slots(int u, int c, int nt_u) {
  return ((u + 1) * nt_u - 1) / c - (u * nt_u) / c + 1;
}

// float32 attention (head_dim 64 or 128).
struct AttnArgsF {
  const float* q;          // [T][Hq][D]
  int T, Hq, G;
  const float* kp;
  const float* vtp;
  int P, ldp;
  const float* ks;
  const float* vts;
  int lds;
  const int* seq_start;
  const uint64_t* mask;
  const int2* pseg;        // [T] the row's prefix keys [x, y) (nullptr: [0, P))
  float scale;             // 1 / sqrt(D)
  float* o;                // [T][Hq*D]
};

// Range flag of a forward (nullable everywhere): bit 0 is set by any kernel that writes a
// float16 activation plane (q/k/v, a norm's float16 output, the SwiGLU output) and meets a
// value outside the float16 range or not finite.
constexpr int kFlagF16Range = 1;
// Row t: E[tok[t]] for tok[t] >= 0, vis[-1 - tok[t]] otherwise.  Clears *flags.
hipError_t launch_embed(bool bf16, const void* E, const int* tok, int T, int H, const void* vis, float* x,
                        int* flags, hipStream_t s);
// y (float32) and/or yh/yl (bfloat16 hi/lo planes) may be null.
hipError_t launch_rmsnorm(bool bf16, const float* x, int ldx, const int* rows, int n_rows, int H, const void* g,
                          float eps, float* y, uint16_t* yh, uint16_t* yl, int ldy, hipStream_t s);
struct GemmPlan {
  bool wide;    // 128 x 256 kernel (else 128 x 128)
  int splits;   // K splits (partials [splits][M][N] when > 1)
};
GemmPlan gemm_bf16_plan(int M, int N, int K, size_t part_cap);
// A is given as two bfloat16 planes (hi, lo) with row stride lda; the product is W·hi + W·lo.
// K % 32 == 0.  With *eff_splits > 1 it wrote split partials [splits][M][N] (at most part_cap
// floats) into `part` and a split-K reduction must follow.
hipError_t launch_gemm_bf16(const uint16_t* Ah, const uint16_t* Al, int lda, int M, int K, const GemmSegs& seg, int N,
                            float* C, int ldc, int accum, size_t part_cap, float* part, hipStream_t s,
                            int* eff_splits);
// gate|up GEMM with the SwiGLU epilogue: u = silu(A·W_gateᵀ) * (A·W_upᵀ) as bf16 hi/lo planes [M][ldu],
// or as one float16 plane into uh when ul is null.
hipError_t launch_gemm_swiglu(const uint16_t* Ah, const uint16_t* Al, int lda, int M, int K, const uint16_t* w_gate,
                              const uint16_t* w_up, int I, uint16_t* uh, uint16_t* ul, int ldu, int* flags,
                              hipStream_t s);
// Single-pass float16 GEMM: A is one float16 plane, seg holds float16 weights; otherwise as
// launch_gemm_bf16 (split partials when *eff_splits > 1).
GemmPlan gemm_f16_plan(int M, int N, int K, size_t part_cap);
hipError_t launch_gemm_f16(const uint16_t* A, int lda, int M, int K, const GemmSegs& seg, int N, float* C, int ldc,
                           int accum, size_t part_cap, float* part, hipStream_t s, int* eff_splits);
// gate|up GEMM with the SwiGLU epilogue on a float16 activation plane and float16 weights; u as in
// launch_gemm_swiglu (hi/lo planes, or one float16 plane when ul is null).
hipError_t launch_gemm_swiglu_f16(const uint16_t* A, int lda, int M, int K, const uint16_t* w_gate,
                                  const uint16_t* w_up, int I, uint16_t* uh, uint16_t* ul, int ldu, int* flags,
                                  hipStream_t s);
// gate|up with few output tiles (the fused kernel would fill under one block per compute
// unit): run it as a plain split-K GEMM over [W_gate | W_up] into [splits][M][2I] partials (or
// [M][2I] when one split), then launch_splitk_swiglu writes u as launch_gemm_swiglu would.
bool swiglu_use_split(int M, int I, size_t part_cap);
hipError_t launch_splitk_swiglu(const float* part, int splits, int M, int I, uint16_t* uh, uint16_t* ul, int ldu,
                                int* flags, hipStream_t s);
// float16 copy of n bfloat16 values (n % 8 == 0); sets *bad = 1 if a finite value exceeds the
// float16 range (*bad is not cleared).
hipError_t launch_bf16_to_f16(const uint16_t* src, size_t n, uint16_t* dst, int* bad, hipStream_t s);
// x[row] += sum of `splits` partials [M][H] (splits may be 0), then RMSNorm of x into bf16 hi/lo
// planes, or one float16 plane into yh when f16out (skipped when yh is null).  H % 4 == 0, H <= 8192.
hipError_t launch_residual_norm(bool bf16, const float* part, size_t split_stride, int splits, float* x, int M,
                                int H, const void* g, float eps, uint16_t* yh, uint16_t* yl, int ldy, bool f16out,
                                int* flags, hipStream_t s);
// Sum of `splits` projection partials (row stride lds) -> RoPE (table cs) -> q * qscale as f16 hi (and
// lo = the rounding remainder, when q_lo is not null) in the attention's operand order,
// K [Hkv][ldk][128] f16 at rows 0..T-1, Vt [Hkv][128][ldv] f16 at columns 0..T-1 and zeros in
// columns T..round8(T)-1 (ldv >= round8(T)).
// cs[t][i] = (cos, sin) of pos[t] * theta^(-2i/D), i < D/2 of 64 slots per row (D = 64 or 128).
hipError_t launch_rope_table(const int* pos, int T, int D, double log2_theta, float2* cs, hipStream_t s);
hipError_t launch_qkv_post(const float* src, int lds, size_t split_stride, int splits, int T, int Hq, int Hkv,
                           const float2* cs, void* q_hi, void* q_lo, void* kdst, int ldk, void* vtdst, int ldv,
                           int D, float qscale, int* flags, hipStream_t s);
hipError_t launch_splitk_reduce(const float* part, int splits, int M, int N, float* C, int ldc, int accum,
                                hipStream_t s);
hipError_t launch_gemm_f32(const float* A, int lda, int M, int K, const GemmSegsF& seg, int N, float* C, int ldc,
                           int accum, hipStream_t s);
// q_lo (nullable): second f16 term of q (q - f16(q)); only for f16 output.
hipError_t launch_rope_qk(bool f16out, const float* qkv, int T, int Hq, int Hkv, int D, const int* pos,
                          double log2_theta, void* q_out, void* q_lo, void* k_out, int ldk, int row0, hipStream_t s);
hipError_t launch_v_transpose(bool f16out, const float* src, int lds, int T, int HD, void* vt, int ldv, int col0,
                              hipStream_t s);
constexpr int kAttnMaxSplits = 32;
// Splits for the bf16 attention of T rows (G q heads per KV head) over P prefix keys plus
// own_tiles tiles of own keys: about one block per compute unit (two from 64 key tiles on),
// at least two tiles each.
int attn_splits(int T, int G, int Hkv, int P, int own_tiles);
// The attention's work split: n_split equal key splits per row tile (chunk 0), or the
// balanced schedule (chunk > 0: chunk key tiles per block over the row tiles' sequences laid
// end to end; n_split = the partial slots any row tile needs), chosen for one shared prefix
// (not segmented) when equal splits would leave the compute units unevenly loaded.
struct AttnSchedule {
  int n_split;
  int chunk;
};
AttnSchedule attn_schedule(int T, int G, int Hkv, int P, int own_tiles, bool segmented);
// Own-key tiles (64 keys) of the 128-row tile that needs the most, from the host copy of
// the rows' sequence starts.
int attn_own_tiles(const int* seq_start, int T, int G);
// Segmented prefixes: from the rows' prefix key ranges pseg (host, [T] pairs), per 128-row
// tile of the G*T query rows its prefix key tiles [x, y) (the hull of its rows' ranges) and
// the keys [z, w) every one of its rows sees (z >= w when there are none); returns the largest
// tile count y - x.
int attn_seg_tiles(const int* pseg, int T, int G, int* ptile);
// q_terms 1: q as one float16 term (q_lo unused); 2: q = q_hi + q_lo.  q is pre-scaled by
// log2(e)/sqrt(128) (qkv_post's qscale), so the kernel's scores are in log2 units.
hipError_t launch_attn_f16(const AttnArgs& a, int q_terms, hipStream_t s);
// S: the partial slots (n_split); under the balanced schedule (chunk > 0, with the launch's
// G, P and own_tiles) each row merges the slots its row tile has.
hipError_t launch_attn_merge(const float* o_part, const float* lse_part, int S, int T, int Hq, int D, uint16_t* oh,
                             uint16_t* ol, bool f16out, int G, int P, int own_tiles, int chunk, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgsF& a, int D, hipStream_t s);
hipError_t launch_silu_mul(const float* gu, int T, int I, float* u, uint16_t* uh, uint16_t* ul, hipStream_t s);
hipError_t launch_target_logits(bool bf16, const float* h, int H, const void* W, const int* ridx, const int* tok,
                                int NT, float* z, hipStream_t s);
hipError_t launch_cand_logsoftmax(const float* z, const int* n_cands, int B, int C, float* out, hipStream_t s);
// Full-vocabulary log-sum-exp of R rows without storing the [R][V] logits: the LM-head GEMM
// (bf16 models: h as bf16 hi/lo planes, two matrix-core passes; float32 models: h in float32)
// leaves per-row (max, sum of exp) pairs of each 128-column slice in part [R][ceil(V/128)];
// launch_lse_merge combines them in a fixed order into lse[R].
hipError_t launch_lmhead_lse(bool bf16, const float* h, const uint16_t* h_hi, const uint16_t* h_lo, int H, int R,
                             const void* W, int V, float2* part, hipStream_t s);
hipError_t launch_lse_merge(const float2* part, int R, int V, float* lse, hipStream_t s);
hipError_t launch_tree_finalize(const float* z, const float* lse_rows, const int* ridx, const int* tok,
                                const int* n_cands, int Q, int C, int K, float* score, float* norm,
                                hipStream_t s);
