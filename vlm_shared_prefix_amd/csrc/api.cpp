// C-ABI of the shared-prefix candidate scorer (see include/jev.h).
//
// One forward = embed -> L x [RMSNorm -> q|k|v GEMM -> RoPE/layout ->
// attention over prefix + own rows -> merge -> o GEMM (+residual) -> RMSNorm
// -> gate|up GEMM -> SwiGLU -> down GEMM (+residual)] -> readout, all
// enqueued on the caller's stream.  The only host->device traffic is one copy
// of the packed request metadata into the workspace.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/jev.h"
#include "kernels.h"
#include "plan.h"

using jevp::Plan;
using jevp::Status;

// Per-kernel event timing (diagnostics; one stream at a time while enabled).
struct ProfRec {
  int kind;
  hipEvent_t a, b;
  double flops, bytes;
};
struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<ProfRec> recs;
  hipEvent_t take() {
    if (used == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
  ~Profiler() {
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
  }
};

// Pinned host staging of each call's metadata.  hipMemcpyAsync from pageable memory may be
// carried out by the runtime after the call has returned (the source is read when the stream
// reaches the copy), so the packed metadata is first written into one of kSlots pinned slots
// and copied from there.  A slot is rewritten only after the copy that last read it has
// completed (its event), so no pending copy ever sees its bytes change.  Metadata larger
// than a slot goes through the slots in slot-sized pieces.
struct StageRing {
  static constexpr int kSlots = 8;
  static constexpr size_t kSlotBytes = 1u << 20;
  bool ready = false;
  char* host[kSlots] = {};
  hipEvent_t done[kSlots] = {};
  bool pending[kSlots] = {};
  int next = 0;
  hipError_t init() {
    if (ready) return hipSuccess;
    for (int i = 0; i < kSlots; ++i) {
      hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&host[i]), kSlotBytes, hipHostMallocDefault);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&done[i], hipEventDisableTiming);
      if (e != hipSuccess) {
        release();
        return e;
      }
    }
    ready = true;
    return hipSuccess;
  }
  // enqueue the host->device copy of bytes [0, n) of src into dst on stream s
  hipError_t copy(void* dst, const char* src, size_t n, hipStream_t s) {
    for (size_t off = 0; off < n; off += kSlotBytes) {
      const size_t len = std::min(kSlotBytes, n - off);
      const int k = next;
      next = (next + 1) % kSlots;
      if (pending[k]) {
        hipError_t e = hipEventSynchronize(done[k]);
        if (e != hipSuccess) return e;
        pending[k] = false;
      }
      std::memcpy(host[k], src + off, len);
      hipError_t e = hipMemcpyAsync(static_cast<char*>(dst) + off, host[k], len, hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = hipEventRecord(done[k], s);
      if (e != hipSuccess) return e;
      pending[k] = true;
    }
    return hipSuccess;
  }
  void release() {
    for (int i = 0; i < kSlots; ++i) {
      if (done[i]) {
        if (pending[i]) (void)hipEventSynchronize(done[i]);
        (void)hipEventDestroy(done[i]);
        done[i] = nullptr;
      }
      if (host[i]) {
        (void)hipHostFree(host[i]);
        host[i] = nullptr;
      }
      pending[i] = false;
    }
    ready = false;
  }
};

struct jev_model {
  jev_config cfg;
  jev_weights w;
  std::vector<jev_layer> layers;
  // float16 mirror of some decoder matrices (caller-owned buffer): the GEMMs of the mirrored
  // groups run as single float16 passes on float16 activations
  std::vector<jev_layer> layers16;
  bool f16_gu = false;     // w_gate, w_up mirrored
  // groups mirrored for prefills only (scoring calls keep their two bfloat16 terms)
  bool f16_gu_prefill = false, f16_qkv_prefill = false, f16_o_prefill = false;
  bool f16_gu_score = false;   // gate|up on the f16 pass in prefills and suffix-scoring calls
  bool f16_down = false;   // w_down mirrored
  bool f16_qkv = false;    // wq, wk, wv mirrored
  bool f16_o = false;      // wo mirrored
  // blocks the candidate rows bypass in scoring calls (empty: none); prefills run every block
  std::vector<uint8_t> skip;
  // float16 terms of q in the attention: 0 = by prefix length, 1 or 2 (jev_model_set_attn_q_terms)
  int q_terms = 0;
  std::atomic<uint64_t> prefills{0}, forwards{0}, rows{0}, launches{0};
  Profiler prof;
  // digest of the metadata last staged into each workspace address (launch-only calls check it)
  std::mutex staged_mu;
  std::unordered_map<const void*, uint64_t> staged;
  // pinned host slots the calls' metadata is copied from (created by the first staging call;
  // guarded by staged_mu)
  StageRing ring;
  ~jev_model() { ring.release(); }
};

struct jev_prefix {
  jev_model* m;
  int P;        // rows of the store: the sum of the segments
  int Pc;
  void* kv;
  size_t kv_bytes;
  // independent prefixes stored back to back (one per image); a plain prefix is one segment
  std::vector<int> seg_off, seg_len;
};

static thread_local std::string g_err;

static jev_status fail(jev_status code, const std::string& msg) {
  g_err = msg;
  return code;
}

extern "C" const char* jev_last_error(void) { return g_err.c_str(); }

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline int round64(int x) { return (x + 63) & ~63; }

static bool is_bf16(const jev_model* m) { return m->cfg.dtype == JEV_BF16; }
static size_t kv_elem(const jev_model* m) { return is_bf16(m) ? 2 : 4; }
static int nqkv(const jev_config& c) { return (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim; }
// Head width of the KV store and of the attention's operands: bf16 models run their float16
// attention on 128-dim heads (a 64-dim head zero-padded); float32 models use head_dim itself.
static int kv_dim(const jev_model* m) { return is_bf16(m) ? 128 : m->cfg.head_dim; }

// ---------------------------------------------------------------------------
// model / prefix
// ---------------------------------------------------------------------------
extern "C" jev_status jev_model_create(const jev_config* cfg, const jev_weights* w, jev_model** out) {
  if (!cfg || !w || !out) return fail(JEV_E_INVALID, "null argument");
  const jev_config& c = *cfg;
  if (c.n_layers < 0 || c.hidden <= 0 || c.n_q_heads <= 0 || c.n_kv_heads <= 0 || c.head_dim <= 0 || c.mlp <= 0 ||
      c.vocab <= 0)
    return fail(JEV_E_INVALID, "non-positive model dimension");
  if (!(c.rope_theta > 0.f) || !(c.rms_eps >= 0.f)) return fail(JEV_E_INVALID, "bad rope_theta or rms_eps");
  if (c.dtype != JEV_F32 && c.dtype != JEV_BF16) return fail(JEV_E_INVALID, "unknown dtype");
  if (c.n_q_heads % c.n_kv_heads) return fail(JEV_E_UNSUPPORTED, "n_q_heads not a multiple of n_kv_heads");
  if (c.dtype == JEV_BF16 && (c.hidden % 64 || c.mlp % 64))
    return fail(JEV_E_UNSUPPORTED, "bf16 models need hidden and mlp multiples of 64");
  if (c.dtype == JEV_BF16 && c.hidden > 8192) return fail(JEV_E_UNSUPPORTED, "bf16 models need hidden <= 8192");
  if (c.head_dim != 64 && c.head_dim != 128) return fail(JEV_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!w->embed || !w->final_norm || !w->lm_head || (c.n_layers > 0 && !w->layers))
    return fail(JEV_E_INVALID, "null weight pointer");
  for (int l = 0; l < c.n_layers; ++l) {
    const jev_layer& L = w->layers[l];
    if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.mlp_norm || !L.w_gate || !L.w_up || !L.w_down)
      return fail(JEV_E_INVALID, "null pointer in layer " + std::to_string(l));
  }
  jev_model* m = new jev_model();
  m->cfg = c;
  m->w = *w;
  m->layers.assign(w->layers, w->layers + c.n_layers);
  m->w.layers = m->layers.data();
  *out = m;
  return JEV_OK;
}

extern "C" void jev_model_destroy(jev_model* m) { delete m; }

namespace {
// element counts of the seven decoder matrices of one layer, in mirror order
void layer_matrix_elems(const jev_config& c, size_t n[7]) {
  const size_t H = c.hidden, HqD = (size_t)c.n_q_heads * c.head_dim, HkD = (size_t)c.n_kv_heads * c.head_dim,
               I = c.mlp;
  n[0] = HqD * H; n[1] = HkD * H; n[2] = HkD * H; n[3] = H * HqD; n[4] = I * H; n[5] = I * H; n[6] = H * I;
}
size_t mirror_align(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

constexpr int32_t kAllGroups = JEV_F16_GATE_UP | JEV_F16_QKV | JEV_F16_DOWN | JEV_F16_O | JEV_F16_GATE_UP_PREFILL |
                                JEV_F16_QKV_PREFILL | JEV_F16_O_PREFILL | JEV_F16_GATE_UP_SCORE;
// group of matrix i of a layer (wq, wk, wv, wo, w_gate, w_up, w_down)
static bool mirrored(int i, int32_t groups) {
  constexpr int32_t gu = JEV_F16_GATE_UP | JEV_F16_GATE_UP_PREFILL | JEV_F16_GATE_UP_SCORE,
                    qkv = JEV_F16_QKV | JEV_F16_QKV_PREFILL,
                    o = JEV_F16_O | JEV_F16_O_PREFILL;
  static const int32_t group_of[7] = {qkv, qkv, qkv, o, gu, gu, JEV_F16_DOWN};
  return (groups & group_of[i]) != 0;
}

extern "C" size_t jev_model_f16_bytes(const jev_model* m, int32_t groups) {
  if (!m || m->cfg.dtype != JEV_BF16 || (groups & ~kAllGroups)) return 0;
  size_t n[7], total = 0;
  layer_matrix_elems(m->cfg, n);
  for (int l = 0; l < m->cfg.n_layers; ++l)
    for (int i = 0; i < 7; ++i)
      if (mirrored(i, groups)) total += mirror_align(2 * n[i]);
  return total + 256;   // + the range flag
}

// Back to the two-term bfloat16 path for every GEMM.
static void detach_f16(jev_model* m) {
  m->f16_gu = m->f16_down = m->f16_qkv = m->f16_o = false;
  m->f16_gu_prefill = m->f16_qkv_prefill = m->f16_o_prefill = m->f16_gu_score = false;
  m->layers16.clear();
}

extern "C" jev_status jev_model_attach_f16(jev_model* m, int32_t groups, void* buf, size_t bytes, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!m) return fail(JEV_E_INVALID, "null model");
  if (groups & ~kAllGroups) return fail(JEV_E_INVALID, "unknown matrix group bits");
  if (!buf || groups == 0) {   // detach: back to the two-term bf16 path
    detach_f16(m);
    return JEV_OK;
  }
  if (m->cfg.dtype != JEV_BF16) return fail(JEV_E_UNSUPPORTED, "a float16 mirror applies to bf16 models only");
  const size_t need = jev_model_f16_bytes(m, groups);
  if (bytes < need) return fail(JEV_E_WORKSPACE, "mirror buffer smaller than jev_model_f16_bytes");
  // From here on the buffer is being rewritten: a failure leaves the model detached (a mirror
  // attached earlier may live in this same buffer and no longer holds its matrices).
  detach_f16(m);
  size_t n[7];
  layer_matrix_elems(m->cfg, n);
  char* at = static_cast<char*>(buf);
  int* bad = reinterpret_cast<int*>(at + need - 256);
  std::vector<jev_layer> l16(m->layers);
  if (hipMemsetAsync(bad, 0, sizeof(int), s) != hipSuccess) return fail(JEV_E_HIP, "hipMemsetAsync failed");
  for (int l = 0; l < m->cfg.n_layers; ++l) {
    const jev_layer& W = m->layers[l];
    const void* src[7] = {W.wq, W.wk, W.wv, W.wo, W.w_gate, W.w_up, W.w_down};
    const void** dst[7] = {&l16[l].wq, &l16[l].wk, &l16[l].wv, &l16[l].wo, &l16[l].w_gate, &l16[l].w_up,
                           &l16[l].w_down};
    for (int i = 0; i < 7; ++i) {
      if (!mirrored(i, groups)) continue;
      if (launch_bf16_to_f16(static_cast<const uint16_t*>(src[i]), n[i], reinterpret_cast<uint16_t*>(at), bad, s) !=
          hipSuccess)
        return fail(JEV_E_HIP, "conversion launch failed");
      *dst[i] = at;
      at += mirror_align(2 * n[i]);
    }
  }
  int h_bad = 0;
  if (hipMemcpyAsync(&h_bad, bad, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(JEV_E_HIP, "mirror conversion failed");
  if (h_bad) return fail(JEV_E_UNSUPPORTED, "a weight exceeds the float16 range");
  // every flag follows from `groups` alone; a group mirrored for every call needs no
  // prefill-only bit
  m->layers16 = std::move(l16);
  m->f16_gu = (groups & JEV_F16_GATE_UP) != 0;
  m->f16_qkv = (groups & JEV_F16_QKV) != 0;
  m->f16_o = (groups & JEV_F16_O) != 0;
  m->f16_down = (groups & JEV_F16_DOWN) != 0;
  m->f16_gu_score = !m->f16_gu && (groups & JEV_F16_GATE_UP_SCORE) != 0;
  m->f16_gu_prefill = !m->f16_gu && !m->f16_gu_score && (groups & JEV_F16_GATE_UP_PREFILL) != 0;
  m->f16_qkv_prefill = !m->f16_qkv && (groups & JEV_F16_QKV_PREFILL) != 0;
  m->f16_o_prefill = !m->f16_o && (groups & JEV_F16_O_PREFILL) != 0;
  return JEV_OK;
}

extern "C" int32_t jev_model_f16_groups(const jev_model* m) {
  if (!m) return 0;
  return (m->f16_gu ? JEV_F16_GATE_UP : 0) | (m->f16_qkv ? JEV_F16_QKV : 0) | (m->f16_down ? JEV_F16_DOWN : 0) |
         (m->f16_o ? JEV_F16_O : 0) | (m->f16_gu_prefill ? JEV_F16_GATE_UP_PREFILL : 0) |
         (m->f16_gu_score ? JEV_F16_GATE_UP_SCORE : 0) |
         (m->f16_qkv_prefill ? JEV_F16_QKV_PREFILL : 0) | (m->f16_o_prefill ? JEV_F16_O_PREFILL : 0);
}

extern "C" jev_status jev_get_stats(const jev_model* m, jev_stats* out) {
  if (!m || !out) return fail(JEV_E_INVALID, "null argument");
  out->prefills = m->prefills.load();
  out->forwards = m->forwards.load();
  out->rows = m->rows.load();
  out->launches = m->launches.load();
  return JEV_OK;
}

extern "C" jev_status jev_model_set_skip(jev_model* m, const uint8_t* skip, int32_t n) {
  if (!m) return fail(JEV_E_INVALID, "null model");
  if (!skip || n == 0) {
    m->skip.clear();
    return JEV_OK;
  }
  if (n != m->cfg.n_layers) return fail(JEV_E_INVALID, "skip mask length differs from n_layers");
  std::vector<uint8_t> v(skip, skip + n);
  bool any = false;
  for (uint8_t b : v) any |= b != 0;
  if (any) m->skip = std::move(v); else m->skip.clear();
  return JEV_OK;
}

extern "C" jev_status jev_model_set_attn_q_terms(jev_model* m, int32_t terms) {
  if (!m) return fail(JEV_E_INVALID, "null model");
  if (terms < 0 || terms > 2) return fail(JEV_E_INVALID, "terms must be 0, 1 or 2");
  m->q_terms = terms;
  return JEV_OK;
}

extern "C" jev_status jev_workspace_flags(const void* ws, int32_t* flags, void* stream) {
  if (!ws || !flags) return fail(JEV_E_INVALID, "null argument");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  // the flag word sits at the start of every call's workspace layout
  if (hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
    return fail(JEV_E_HIP, "reading the workspace flags failed");
  *flags = v;
  return JEV_OK;
}

extern "C" size_t jev_prefix_bytes(const jev_model* m, int32_t prefix_len) {
  if (!m || prefix_len < 0) return 0;
  const jev_config& c = m->cfg;
  const size_t Pc = (size_t)round64(prefix_len);
  return (size_t)c.n_layers * 2 * c.n_kv_heads * Pc * kv_dim(m) * kv_elem(m);
}

extern "C" jev_status jev_prefix_create(jev_model* m, int32_t prefix_len, void* kv_buf, size_t kv_bytes,
                                        jev_prefix** out) {
  if (!m || !out) return fail(JEV_E_INVALID, "null argument");
  if (prefix_len < 0) return fail(JEV_E_INVALID, "prefix_len < 0");
  if (prefix_len > jevp::kMaxPrefix) return fail(JEV_E_UNSUPPORTED, "prefix_len > 32768");
  const size_t need = jev_prefix_bytes(m, prefix_len);
  if (need > 0 && !kv_buf) return fail(JEV_E_INVALID, "null kv_buf");
  if (kv_bytes < need) return fail(JEV_E_WORKSPACE, "kv buffer smaller than jev_prefix_bytes");
  jev_prefix* p = new jev_prefix();
  p->m = m;
  p->P = prefix_len;
  p->Pc = round64(prefix_len);
  p->kv = kv_buf;
  p->kv_bytes = kv_bytes;
  p->seg_off = {0};
  p->seg_len = {prefix_len};
  *out = p;
  return JEV_OK;
}

extern "C" jev_status jev_prefix_create_segments(jev_model* m, const int32_t* seg_lens, int32_t n_seg, void* kv_buf,
                                                 size_t kv_bytes, jev_prefix** out) {
  if (!m || !out || !seg_lens) return fail(JEV_E_INVALID, "null argument");
  if (n_seg < 1) return fail(JEV_E_INVALID, "n_seg must be >= 1");
  if (n_seg > jevp::kMaxSegments) return fail(JEV_E_UNSUPPORTED, "more than 64 segments");
  long total = 0;
  for (int i = 0; i < n_seg; ++i) {
    if (seg_lens[i] < 0) return fail(JEV_E_INVALID, "seg_lens[" + std::to_string(i) + "] < 0");
    total += seg_lens[i];
  }
  if (total > jevp::kMaxPrefix) return fail(JEV_E_UNSUPPORTED, "segments hold more than 32768 rows");
  jev_prefix* p = nullptr;
  if (jev_status st = jev_prefix_create(m, (int32_t)total, kv_buf, kv_bytes, &p)) return st;
  p->seg_off.assign(n_seg, 0);
  p->seg_len.assign(seg_lens, seg_lens + n_seg);
  for (int i = 1; i < n_seg; ++i) p->seg_off[i] = p->seg_off[i - 1] + seg_lens[i - 1];
  *out = p;
  return JEV_OK;
}

extern "C" void jev_prefix_destroy(jev_prefix* p) { delete p; }

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kGemmPartFloats = 16ull << 20;        // bound of split-K partials (gemm_bf16_plan)

struct Layout {
  // range flag word, then metadata (staged from the host in one copy)
  size_t flags, tok, pos, seq_start, read_rows, tgt_ridx, tgt_tok, out_n, mask, pseg, ptile, meta_end;
  // float buffers
  size_t x, act, big, q, ks, vts, o_part, lse_part, gpart, h, hsplit, z, lse_rows, lse_slices, rope;
  size_t total;
  size_t prow;   // rows of attention partials (o_part / lse_part) the layout holds
  int Tc;
};

// Rows of attention partials a call of T rows may need: max over T' <= T of splits(T') * T'
// when splits(T') > 1 (the split count falls as rows grow).
constexpr int AT_KEYS = 64;   // attention key tile

size_t attn_part_rows(const jev_config& c, int T, int P) {
  const int G = c.n_q_heads / c.n_kv_heads;
  size_t best = 0;
  for (int t = 1; t <= T; ++t) {
    // the split count grows with the tiles; a row tile's own keys span at most t + 7 rows,
    // and prefills (no prefix keys) count as well
    const int own = (t + 7 + AT_KEYS - 1) / AT_KEYS;
    const int ns = std::max({attn_splits(t, G, c.n_kv_heads, P, own), attn_splits(t, G, c.n_kv_heads, 0, own),
                             attn_schedule(t, G, c.n_kv_heads, P, own, false).n_split});
    if (ns > 1) best = std::max(best, (size_t)ns * t);
  }
  return best;
}

Layout make_layout(const jev_model* m, int T, int R, int NT, int NG, bool has_mask, bool need_logits, int P) {
  const jev_config& c = m->cfg;
  const bool bf = is_bf16(m);
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.flags = take(4);
  L.tok = take(4ull * T);
  L.pos = take(4ull * T);
  L.seq_start = take(4ull * T);
  L.read_rows = take(4ull * R);
  L.tgt_ridx = take(4ull * NT);
  L.tgt_tok = take(4ull * NT);
  L.out_n = take(4ull * NG);
  L.mask = take(has_mask ? 8ull * T : 0);
  L.pseg = take(8ull * T);
  L.ptile = take(16ull * ((c.n_q_heads / c.n_kv_heads * (size_t)T + 127) / 128));
  L.meta_end = o;
  const int HqD = c.n_q_heads * c.head_dim;
  const int wide = std::max(std::max(c.hidden, HqD), c.mlp);
  const int bigw = std::max(nqkv(c), 2 * c.mlp);
  L.Tc = round64(std::max(T, 1));
  const size_t e = kv_elem(m);
  L.x = take(4ull * T * c.hidden);
  L.act = take(4ull * T * wide);
  L.big = take(4ull * T * bigw);
  L.q = take(bf ? 2 * 2 * attn_q_plane_elems(T, c.n_q_heads, c.n_kv_heads)   // bf16 models: q hi and lo planes
                : e * T * HqD);
  L.ks = take(e * c.n_kv_heads * (size_t)L.Tc * kv_dim(m));
  L.vts = take(e * c.n_kv_heads * (size_t)L.Tc * kv_dim(m));
  const size_t prow = bf ? attn_part_rows(c, T, P) : 0;
  L.prow = prow;
  L.o_part = take(4ull * prow * c.n_q_heads * kv_dim(m));
  L.lse_part = take(4ull * prow * c.n_q_heads);
  L.gpart = take(bf ? 4ull * kGemmPartFloats : 0);
  L.h = take(4ull * R * c.hidden);
  L.hsplit = take(bf && need_logits ? 4ull * R * c.hidden : 0);
  L.z = take(4ull * NT);
  L.lse_rows = take(4ull * R);
  // full-vocabulary readout: per row one (max, sum of exp) pair per 128 logits, never the logits
  L.lse_slices = take(need_logits ? 8ull * R * ((c.vocab + 127) / 128) : 0);
  L.rope = take(bf ? 8ull * T * 64 : 0);
  L.total = o;
  return L;
}
}  // namespace

extern "C" size_t jev_workspace_bytes(const jev_model* m, int32_t prefix_len, int32_t max_rows, int32_t max_seqs,
                                      int32_t max_targets) {
  if (!m || prefix_len < 0 || max_rows < 0 || max_seqs < 0 || max_targets < 0) return 0;
  const int R = std::min(max_rows, max_targets);
  return make_layout(m, max_rows, R, max_targets, max_seqs, true, max_targets > 0, prefix_len).total;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
namespace {
enum class Mode { Prefill, Score, Tree };

// Terms of q in the attention's QK^T products: with one term q is rounded once to float16;
// the second term (q - f16(q)) removes that rounding, which shifts every score of a row
// coherently and grows in weight with the number of keys a row sees.
constexpr int kAttnQ2Keys = 2048;   // the automatic choice takes two terms above this many prefix keys
constexpr int kF16QkvPrefillKeys = 2048;   // longest prefix segment whose prefill runs q|k|v on float16
// keys: the most prefix keys (the longest segment) a row of the call sees.
int attn_q_terms(const jev_model* m, int keys) {
  if (m->q_terms == 1 || m->q_terms == 2) return m->q_terms;
  return keys > kAttnQ2Keys ? 2 : 1;
}

// Layers a forward runs: all of them for a prefill; in scoring calls the candidate rows bypass
// the blocks of the model's skip mask ("FastJEV", §2.3 and §3.4: the shared context keeps every
// block, candidate evaluation skips the selected complete blocks).
std::vector<int> run_layers(const jev_model* m, Mode mode) {
  std::vector<int> out;
  for (int l = 0; l < m->cfg.n_layers; ++l)
    if (mode == Mode::Prefill || m->skip.empty() || !m->skip[l]) out.push_back(l);
  return out;
}

#define HIP_OK(expr)                                                                  \
  do {                                                                                \
    hipError_t e_ = (expr);                                                           \
    if (e_ != hipSuccess) return fail(JEV_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Profiled launch kinds, named after the kernels they launch; the decoder's projections are
// told apart by role (two bf16 passes, or one float16 pass: _f16).
enum Kind {
  K_EMBED, K_RMSNORM, K_RESNORM, K_ROPETAB, K_QKVPOST, K_GEMM, K_SWIGLU, K_SPLITK, K_ROPE, K_VT, K_ATTN, K_MERGE,
  K_SILU, K_TARGET, K_CANDSM, K_LMHEAD, K_ROWLSE, K_TREEFIN, K_GEMM16, K_SWIGLU16, K_SPLITSWIGLU,
  K_QKV, K_QKV16, K_O, K_O16, K_GU, K_GU16, K_DOWN, K_DOWN16, K_NKINDS
};
const char* const kKindName[K_NKINDS] = {
    "embed_rows", "rmsnorm_rows", "residual_norm", "rope_table", "qkv_post", "gemm", "gemm_swiglu",
    "splitk_reduce", "rope_qk", "v_transpose", "attn_fwd", "attn_merge", "silu_mul", "target_logits",
    "cand_logsoftmax", "lm_head_lse", "lse_merge", "tree_finalize", "gemm_f16", "gemm_swiglu_f16", "splitk_swiglu",
    "gemm_qkv", "gemm_qkv_f16", "gemm_o", "gemm_o_f16", "gemm_gate_up", "gemm_gate_up_f16", "gemm_down",
    "gemm_down_f16"};

struct Forward {
  const jev_prefix* pf;
  jev_model* m;
  const jev_config& c;
  const Plan& plan;
  const Layout& L;
  void* ws;
  hipStream_t s;
  Mode mode;
  Profiler* prof;
  int launches = 0;
  double own_pairs = 0;      // (row, own visible key) pairs of the attention
  double prefix_pairs = 0;   // (row, prefix key) pairs

  Forward(const jev_prefix* p, const Plan& pl, const Layout& lay, void* w, hipStream_t st, Mode md)
      : pf(p), m(p->m), c(p->m->cfg), plan(pl), L(lay), ws(w), s(st), mode(md),
        prof(p->m->prof.on ? &p->m->prof : nullptr) {
    for (int t = 0; t < plan.T; ++t)
      own_pairs += plan.mask.empty() ? (double)(t - plan.seq_start[t] + 1)
                                     : (double)__builtin_popcountll(plan.mask[t]);
    if (mode != Mode::Prefill) {
      if (plan.pseg.empty())
        prefix_pairs = (double)plan.T * pf->P;
      else
        for (int t = 0; t < plan.T; ++t) prefix_pairs += plan.pseg[2 * t + 1] - plan.pseg[2 * t];
    }
  }

  // Launch one kernel through `fn`, timing it with events when profiling is on.
  template <class Fn>
  jev_status run_k(int kind, double flops, double bytes, Fn&& fn) {
    hipEvent_t a = nullptr;
    if (prof) {
      a = prof->take();
      if (a) (void)hipEventRecord(a, s);
    }
    const hipError_t e = fn();
    ++launches;
    if (e != hipSuccess) return fail(JEV_E_HIP, std::string(kKindName[kind]) + ": " + hipGetErrorString(e));
    if (prof && a) {
      hipEvent_t b = prof->take();
      if (b) {
        (void)hipEventRecord(b, s);
        prof->recs.push_back({kind, a, b, flops, bytes});
      }
    }
    return JEV_OK;
  }

  // layer l's K / Vt in the prefix store
  char* store_k(int l) const {
    const size_t per = (size_t)c.n_kv_heads * pf->Pc * kv_dim(m) * kv_elem(m);
    return static_cast<char*>(pf->kv) + (size_t)l * 2 * per;
  }
  char* store_vt(int l) const { return store_k(l) + (size_t)c.n_kv_heads * pf->Pc * kv_dim(m) * kv_elem(m); }


  // A operand: float32 rows (float32 models), bfloat16 hi/lo planes, or one float16 plane
  // in hi (bf16 models with a float16 mirror: f16 set)
  struct AOp {
    const float* f;
    const uint16_t* hi;
    const uint16_t* lo;
    bool f16 = false;
  };
  jev_status gemm(AOp A, int lda, int M, int K, const void* w0, int n0, const void* w1, int n1,
                  const void* w2, int n2, float* C, int ldc, int accum, int kind = K_GEMM) {
    const int N = n0 + n1 + n2;
    const double flops = 2.0 * M * N * K;
    const double wbytes = (double)N * K * (is_bf16(m) ? 2 : 4);
    const double bytes = wbytes + 4.0 * M * K + 4.0 * M * N * (accum ? 2 : 1);
    if (is_bf16(m)) {
      GemmSegs sg{{(const uint16_t*)w0, (const uint16_t*)w1, (const uint16_t*)w2}, {n0, n0 + n1, N}};
      int eff = 1;
      float* part = at<float>(ws, L.gpart);
      if (jev_status st = run_k(kind, flops, bytes, [&] {
            return launch_gemm_bf16(A.hi, A.lo, lda, M, K, sg, N, C, ldc, accum, kGemmPartFloats, part, s, &eff);
          }))
        return st;
      if (eff > 1)
        return run_k(K_SPLITK, 0.0, 4.0 * M * N * (eff + (accum ? 2 : 1)),
                 [&] { return launch_splitk_reduce(part, eff, M, N, C, ldc, accum, s); });
      return JEV_OK;
    }
    GemmSegsF sg{{(const float*)w0, (const float*)w1, (const float*)w2}, {n0, n0 + n1, N}};
    return run_k(kind, flops, bytes, [&] { return launch_gemm_f32(A.f, lda, M, K, sg, N, C, ldc, accum, s); });
  }

  // bf16 GEMM whose split-K partials (if any) are left for a fused consumer:
  // on return *splits_out is 1 (C written / accumulated) or > 1 (partials in gpart, stride M*N).
  // kind: the role's two-pass kind; its float16 kind is the next one
  jev_status gemm_deferred(int kind, AOp A, int lda, int M, int K, const void* w0, int n0, const void* w1, int n1,
                           const void* w2, int n2, float* C, int ldc, int accum, int* splits_out) {
    const int N = n0 + n1 + n2;
    const double flops = 2.0 * M * N * K;
    const double bytes = 2.0 * N * K + (A.f16 ? 2.0 : 4.0) * M * K + 4.0 * M * N * (accum ? 2 : 1);
    GemmSegs sg{{(const uint16_t*)w0, (const uint16_t*)w1, (const uint16_t*)w2}, {n0, n0 + n1, N}};
    float* part = at<float>(ws, L.gpart);
    return run_k(A.f16 ? kind + 1 : kind, flops, bytes, [&] {
      return A.f16 ? launch_gemm_f16(A.hi, lda, M, K, sg, N, C, ldc, accum, kGemmPartFloats, part, s, splits_out)
                   : launch_gemm_bf16(A.hi, A.lo, lda, M, K, sg, N, C, ldc, accum, kGemmPartFloats, part, s,
                                      splits_out);
    });
  }

  // Forward of a bf16 model: every GEMM consumer fused with the split-K reduction.
  jev_status run_bf16(const void* vis) {
    const int T = plan.T;
    const int H = c.hidden, Hq = c.n_q_heads, Hkv = c.n_kv_heads, D = c.head_dim, I = c.mlp;
    const int HqD = Hq * D, NQKV = nqkv(c);
    const int wide = std::max(std::max(H, HqD), I);
    float* x = at<float>(ws, L.x);
    int* flags = at<int>(ws, L.flags);
    // GEMMs of a mirrored group take one float16 plane (in the hi slot), and the kernels that
    // produce their inputs write that plane: the input norm and attention output for the
    // q|k|v and o projections, the post-attention norm for gate|up, the SwiGLU output for down
    const bool pre = mode == Mode::Prefill;
    // the longest key segment a row of this call sees (the prefix's longest segment)
    const int seg_max = *std::max_element(pf->seg_len.begin(), pf->seg_len.end());
    // q|k|v of prefills on the float16 pass only up to kF16QkvPrefillKeys rows: K and V reach
    // every query's scores, and their rounding error grows with the keys a query sees
    const bool fq = m->f16_qkv || (m->f16_qkv_prefill && pre && seg_max <= kF16QkvPrefillKeys);
    const bool fo = m->f16_o || (m->f16_o_prefill && pre);
    const bool fd = m->f16_down,
               fg = m->f16_gu || (m->f16_gu_prefill && pre) || (m->f16_gu_score && mode != Mode::Tree);
    uint16_t* a_hi = at<uint16_t>(ws, L.act);                 // normalised activations / attention output
    uint16_t* a_lo = a_hi + (size_t)T * wide;
    const AOp A_qkv{nullptr, a_hi, a_lo, fq};
    const AOp A_o{nullptr, a_hi, a_lo, fo};
    float* big = at<float>(ws, L.big);                        // projection output (fp32) ...
    uint16_t* u_hi = reinterpret_cast<uint16_t*>(big);        // ... or the SwiGLU planes [T][I]
    uint16_t* u_lo = u_hi + (size_t)T * I;
    const AOp A_u{nullptr, u_hi, u_lo, fd};
    float* part = at<float>(ws, L.gpart);
    const int* tok = at<int>(ws, L.tok);
    const int* pos = at<int>(ws, L.pos);
    const int* seq_start = at<int>(ws, L.seq_start);
    const uint64_t* mask = plan.mask.empty() ? nullptr : at<uint64_t>(ws, L.mask);
    const double log2_theta = std::log2((double)c.rope_theta);
    const int P = (mode == Mode::Prefill) ? 0 : pf->P;
    const double rowbytes = 4.0 * T * H;

    if (jev_status st = run_k(K_EMBED, 0.0, rowbytes * 1.5,
                              [&] { return launch_embed(true, m->w.embed, tok, T, H, vis, x, flags, s); }))
      return st;
    const std::vector<int> layers = run_layers(m, mode);
    if (layers.empty()) return JEV_OK;
    float2* rope = at<float2>(ws, L.rope);
    if (jev_status st = run_k(K_ROPETAB, 0.0, 8.0 * T * 64,
                              [&] { return launch_rope_table(pos, T, D, log2_theta, rope, s); }))
      return st;
    if (jev_status st = run_k(K_RESNORM, 0.0, 2 * rowbytes, [&] {
          return launch_residual_norm(true, nullptr, 0, 0, x, T, H, m->layers[layers[0]].attn_norm, c.rms_eps, a_hi,
                                      a_lo, wide, fq, flags, s);
        }))
      return st;

    // q as one float16 term, or two (q_hi + q_lo) when rows see long prefixes (jev_model_set_attn_q_terms)
    const int q_terms = attn_q_terms(m, seg_max);
    const float qscale = (float)(1.4426950408889634 / std::sqrt((double)D));
    // attention splits: about one block per compute unit (partials merged when > 1), or the
    // balanced schedule where equal splits would load the compute units unevenly (it falls
    // back to equal splits should its partials not fit the layout's)
    const int own_tiles = attn_own_tiles(plan.seq_start.data(), T, Hq / Hkv);
    const int split_keys = plan.seg_keys >= 0 ? plan.seg_keys : P;
    AttnSchedule sched = attn_schedule(T, Hq / Hkv, Hkv, split_keys, own_tiles, !plan.pseg.empty());
    if (sched.chunk > 0 && (size_t)sched.n_split * T > L.prow)
      sched = AttnSchedule{attn_splits(T, Hq / Hkv, Hkv, split_keys, own_tiles), 0};
    const int n_split = sched.n_split;
    const bool attn_parts = n_split > 1 || sched.chunk > 0;
    const int2* pseg = plan.pseg.empty() ? nullptr : at<int2>(ws, L.pseg);
    const int4* ptile = plan.pseg.empty() ? nullptr : at<int4>(ws, L.ptile);
    const double attn_flops = 4.0 * D * Hq * (prefix_pairs + own_pairs);
    const double attn_bytes = 2.0 * (2.0 * Hkv * P * D + 2.0 * Hkv * T * D + 2.0 * T * HqD) + 4.0 * T * HqD;

    for (size_t li = 0; li < layers.size(); ++li) {
      const int l = layers[li];
      const jev_layer& W = m->layers[l];
      const jev_layer& WQ = fq ? m->layers16[l] : W;   // the matrices the GEMMs read
      const jev_layer& WO = fo ? m->layers16[l] : W;
      const jev_layer& WG = fg ? m->layers16[l] : W;
      const jev_layer& WD = fd ? m->layers16[l] : W;
      const bool last_prefill = (mode == Mode::Prefill) && (l == c.n_layers - 1);
      int sp = 1;
      if (jev_status st = gemm_deferred(K_QKV, A_qkv, wide, T, H, WQ.wq, HqD, WQ.wk, Hkv * D, WQ.wv, Hkv * D, big, NQKV, 0, &sp))
        return st;
      void *kdst, *vdst;
      int kld;
      if (mode == Mode::Prefill) {
        kdst = store_k(l);
        vdst = store_vt(l);
        kld = pf->Pc;
      } else {
        kdst = at<char>(ws, L.ks);
        vdst = at<char>(ws, L.vts);
        kld = L.Tc;
      }
      _Float16* q_hi = at<_Float16>(ws, L.q);
      _Float16* q_lo = q_terms == 2 ? q_hi + attn_q_plane_elems(T, Hq, Hkv) : nullptr;
      if (jev_status st = run_k(K_QKVPOST, 0.0, (double)T * NQKV * 4 * sp + (double)T * (q_terms * HqD + 2 * Hkv * D) * 2, [&] {
            return launch_qkv_post(sp > 1 ? part : big, NQKV, (size_t)T * NQKV, sp, T, Hq, Hkv, rope, q_hi, q_lo,
                                   kdst, kld, vdst, kld, D, qscale, flags, s);
          }))
        return st;
      if (last_prefill) break;   // the prefix store is complete; later rows of this layer are unused

      AttnArgs a{};
      a.q = q_hi;
      a.q_lo = q_lo;
      a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
      if (P > 0) {
        a.kp = reinterpret_cast<const _Float16*>(store_k(l));
        a.vtp = reinterpret_cast<const _Float16*>(store_vt(l));
      }
      a.P = P; a.ldp = pf->Pc;
      a.ks = static_cast<const _Float16*>(kdst);
      a.vts = static_cast<const _Float16*>(vdst);
      a.lds = kld;
      a.seq_start = seq_start; a.mask = mask;
      a.pseg = pseg; a.ptile = ptile;
      a.n_split = n_split;
      a.sk_chunk = sched.chunk;
      a.own_tiles = own_tiles;
      a.o_part = at<float>(ws, L.o_part);
      a.lse_part = at<float>(ws, L.lse_part);
      a.oh = a_hi; a.ol = a_lo;
      a.o_f16 = fo ? 1 : 0;
      a.D = D;
      if (jev_status st = run_k(K_ATTN, attn_flops, attn_bytes, [&] { return launch_attn_f16(a, q_terms, s); }))
        return st;
      if (attn_parts) {
        if (jev_status st = run_k(K_MERGE, 0.0, 4.0 * (n_split + 1) * T * HqD, [&] {
              return launch_attn_merge(a.o_part, a.lse_part, n_split, T, Hq, D, a_hi, a_lo, fo, Hq / Hkv, P,
                                       own_tiles, sched.chunk, s);
            }))
          return st;
      }
      // o-proj: x += o·W_oᵀ, then m = RMSNorm(x; g2) into the activation planes
      if (jev_status st = gemm_deferred(K_O, A_o, HqD, T, HqD, WO.wo, H, nullptr, 0, nullptr, 0, x, H, 1, &sp)) return st;
      if (jev_status st = run_k(K_RESNORM, 0.0, rowbytes * (2 + (sp > 1 ? sp + 1 : 0)), [&] {
            return launch_residual_norm(true, part, (size_t)T * H, sp > 1 ? sp : 0, x, T, H, W.mlp_norm, c.rms_eps,
                                        a_hi, a_lo, wide, fg, flags, s);
          }))
        return st;
      // activation bytes per element: two bf16 planes, or one float16 plane
      const double in_b = fg ? 2.0 : 4.0, out_b = fd ? 2.0 : 4.0;
      if (swiglu_use_split(T, I, kGemmPartFloats)) {
        // few rows: a split-K GEMM over [W_gate | W_up] streams the weights with more blocks,
        // then the SwiGLU is applied while the partials are summed
        int sg = 1;
        const AOp A_g{nullptr, a_hi, a_lo, fg};
        if (jev_status st = gemm_deferred(K_GU, A_g, wide, T, H, WG.w_gate, I, WG.w_up, I, nullptr, 0, part, 2 * I, 0, &sg))
          return st;
        if (jev_status st = run_k(K_SPLITSWIGLU, 0.0, 4.0 * sg * T * 2 * I + out_b * T * I, [&] {
              return launch_splitk_swiglu(part, sg, T, I, u_hi, fd ? nullptr : u_lo, I, flags, s);
            }))
          return st;
      } else if (jev_status st = run_k(fg ? K_SWIGLU16 : K_SWIGLU, 2.0 * T * 2 * I * H,
                                2.0 * 2 * I * H + in_b * T * H + out_b * T * I, [&] {
            uint16_t* ul = fd ? nullptr : u_lo;   // u as one float16 plane for a float16 down GEMM
            return fg ? launch_gemm_swiglu_f16(a_hi, wide, T, H, static_cast<const uint16_t*>(WG.w_gate),
                                               static_cast<const uint16_t*>(WG.w_up), I, u_hi, ul, I, flags, s)
                      : launch_gemm_swiglu(a_hi, a_lo, wide, T, H, static_cast<const uint16_t*>(W.w_gate),
                                           static_cast<const uint16_t*>(W.w_up), I, u_hi, ul, I, flags, s);
          }))
        return st;
      // down: x += u·W_dᵀ, then the next layer's input norm
      if (jev_status st = gemm_deferred(K_DOWN, A_u, I, T, I, WD.w_down, H, nullptr, 0, nullptr, 0, x, H, 1, &sp)) return st;
      const void* next_g = (li + 1 < layers.size()) ? m->layers[layers[li + 1]].attn_norm : nullptr;
      if (jev_status st = run_k(K_RESNORM, 0.0, rowbytes * (2 + (sp > 1 ? sp + 1 : 0)), [&] {
            return launch_residual_norm(true, part, (size_t)T * H, sp > 1 ? sp : 0, x, T, H,
                                        next_g ? next_g : W.mlp_norm, c.rms_eps, next_g ? a_hi : nullptr,
                                        next_g ? a_lo : nullptr, wide, fq, flags, s);
          }))
        return st;
    }
    return JEV_OK;
  }

  jev_status run(const void* vis) { return is_bf16(m) ? run_bf16(vis) : run_f32(vis); }

  // float32 models: every step in float32 (VALU GEMMs, one-thread-per-row attention).
  jev_status run_f32(const void* vis) {
    const int T = plan.T;
    const int H = c.hidden, Hq = c.n_q_heads, Hkv = c.n_kv_heads, D = c.head_dim, I = c.mlp;
    const int HqD = Hq * D, NQKV = nqkv(c);
    const int wide = std::max(std::max(H, HqD), I);
    float* x = at<float>(ws, L.x);
    int* flags = at<int>(ws, L.flags);
    float* act = at<float>(ws, L.act);
    const AOp A_act{act, nullptr, nullptr};
    float* big = at<float>(ws, L.big);
    const int* tok = at<int>(ws, L.tok);
    const int* pos = at<int>(ws, L.pos);
    const int* seq_start = at<int>(ws, L.seq_start);
    const uint64_t* mask = plan.mask.empty() ? nullptr : at<uint64_t>(ws, L.mask);
    const double log2_theta = std::log2((double)c.rope_theta);
    const int P = (mode == Mode::Prefill) ? 0 : pf->P;
    const double rowbytes = 4.0 * T * H;

    if (jev_status st = run_k(K_EMBED, 0.0, rowbytes * 2.0,
                              [&] { return launch_embed(false, m->w.embed, tok, T, H, vis, x, flags, s); }))
      return st;
    const int2* pseg = plan.pseg.empty() ? nullptr : at<int2>(ws, L.pseg);
    const double attn_flops = 4.0 * D * Hq * (prefix_pairs + own_pairs);
    const double attn_bytes = 4.0 * (2.0 * Hkv * P * D + 2.0 * Hkv * T * D + (double)T * HqD) + 4.0 * T * HqD;

    for (int l : run_layers(m, mode)) {
      const jev_layer& W = m->layers[l];
      const bool last_prefill = (mode == Mode::Prefill) && (l == c.n_layers - 1);
      if (jev_status st = run_k(K_RMSNORM, 0.0, 2 * rowbytes, [&] {
            return launch_rmsnorm(false, x, H, nullptr, T, H, W.attn_norm, c.rms_eps, act, nullptr, nullptr, wide,
                                  s);
          }))
        return st;
      if (jev_status st = gemm(A_act, wide, T, H, W.wq, HqD, W.wk, Hkv * D, W.wv, Hkv * D, big, NQKV, 0)) return st;
      // K / V destination: the prefix store (prefill) or the workspace (scoring)
      void *kdst, *vdst;
      int kld;
      if (mode == Mode::Prefill) {
        kdst = store_k(l);
        vdst = store_vt(l);
        kld = pf->Pc;
      } else {
        kdst = at<char>(ws, L.ks);
        vdst = at<char>(ws, L.vts);
        kld = L.Tc;
      }
      if (jev_status st = run_k(K_ROPE, 0.0, (double)T * (Hq + Hkv) * D * 8, [&] {
            return launch_rope_qk(false, big, T, Hq, Hkv, D, pos, log2_theta, at<char>(ws, L.q), nullptr, kdst, kld,
                                  0, s);
          }))
        return st;
      if (jev_status st = run_k(K_VT, 0.0, (double)T * Hkv * D * 8, [&] {
            return launch_v_transpose(false, big + (size_t)(Hq + Hkv) * D, NQKV, T, Hkv * D, vdst, kld, 0, s);
          }))
        return st;
      if (last_prefill) break;   // the prefix store is complete; later rows of this layer are unused

      AttnArgsF a{};
      a.q = at<float>(ws, L.q);
      a.T = T; a.Hq = Hq; a.G = Hq / Hkv;
      if (P > 0) {
        a.kp = reinterpret_cast<const float*>(store_k(l));
        a.vtp = reinterpret_cast<const float*>(store_vt(l));
      }
      a.P = P; a.ldp = pf->Pc;
      a.ks = static_cast<const float*>(kdst);
      a.vts = static_cast<const float*>(vdst);
      a.lds = kld;
      a.seq_start = seq_start; a.mask = mask;
      a.pseg = pseg;
      a.scale = (float)(1.0 / std::sqrt((double)D));
      a.o = act;
      if (jev_status st = run_k(K_ATTN, attn_flops, attn_bytes, [&] { return launch_attn_f32(a, D, s); })) return st;
      // act now holds o [T][HqD] with row stride HqD
      if (jev_status st = gemm(A_act, HqD, T, HqD, W.wo, H, nullptr, 0, nullptr, 0, x, H, 1)) return st;
      if (jev_status st = run_k(K_RMSNORM, 0.0, 2 * rowbytes, [&] {
            return launch_rmsnorm(false, x, H, nullptr, T, H, W.mlp_norm, c.rms_eps, act, nullptr, nullptr, wide, s);
          }))
        return st;
      if (jev_status st = gemm(A_act, wide, T, H, W.w_gate, I, W.w_up, I, nullptr, 0, big, 2 * I, 0)) return st;
      if (jev_status st = run_k(K_SILU, 0.0, 12.0 * T * I,
                                [&] { return launch_silu_mul(big, T, I, act, nullptr, nullptr, s); }))
        return st;   // gate|up [T][2I] -> u [T][I]
      if (jev_status st = gemm(A_act, I, T, I, W.w_down, H, nullptr, 0, nullptr, 0, x, H, 1)) return st;
    }
    return JEV_OK;
  }

  jev_status readout(float* out_a, float* out_b) {
    const int H = c.hidden;
    const bool bf = is_bf16(m);
    const int R = (int)plan.read_rows.size();
    const int NT = (int)plan.tgt_tok.size();
    const double we = bf ? 2.0 : 4.0;
    float* h = at<float>(ws, L.h);
    float* z = at<float>(ws, L.z);
    const bool split_h = bf && mode == Mode::Tree;
    uint16_t* h_hi = split_h ? at<uint16_t>(ws, L.hsplit) : nullptr;
    uint16_t* h_lo = split_h ? h_hi + (size_t)R * H : nullptr;
    if (jev_status st = run_k(K_RMSNORM, 0.0, 8.0 * R * H, [&] {
          return launch_rmsnorm(bf, at<float>(ws, L.x), H, at<int>(ws, L.read_rows), R, H, m->w.final_norm,
                                c.rms_eps, h, h_hi, h_lo, H, s);
        }))
      return st;
    if (jev_status st = run_k(K_TARGET, 2.0 * NT * H, NT * H * we, [&] {
          return launch_target_logits(bf, h, H, m->w.lm_head, at<int>(ws, L.tgt_ridx), at<int>(ws, L.tgt_tok), NT,
                                      z, s);
        }))
      return st;
    if (mode == Mode::Score) {
      const int B = (int)plan.out_n.size();
      return run_k(K_CANDSM, 0.0, 8.0 * NT,
               [&] { return launch_cand_logsoftmax(z, at<int>(ws, L.out_n), B, NT / std::max(B, 1), out_a, s); });
    }
    // LSE over all V logits of every readout row, the logits never leaving the GEMM's registers
    float2* slices = at<float2>(ws, L.lse_slices);
    const double slice_bytes = 8.0 * R * ((c.vocab + 127) / 128);
    if (jev_status st = run_k(K_LMHEAD, 2.0 * R * c.vocab * H, (double)c.vocab * H * we + slice_bytes, [&] {
          return launch_lmhead_lse(bf, h, h_hi, h_lo, H, R, m->w.lm_head, c.vocab, slices, s);
        }))
      return st;
    if (jev_status st = run_k(K_ROWLSE, 0.0, slice_bytes + 4.0 * R, [&] {
          return launch_lse_merge(slices, R, c.vocab, at<float>(ws, L.lse_rows), s);
        }))
      return st;
    const int Q = (int)plan.out_n.size();
    return run_k(K_TREEFIN, 0.0, 8.0 * NT, [&] {
      return launch_tree_finalize(z, at<float>(ws, L.lse_rows), at<int>(ws, L.tgt_ridx), at<int>(ws, L.tgt_tok),
                                  at<int>(ws, L.out_n), Q, tree_C, tree_K, out_a, out_b, s);
    });
  }
  int tree_C = 0, tree_K = 0;
};

constexpr size_t kMaxStagedWorkspaces = 1024;   // digests remembered per model

// 64-bit FNV-1a of the staged metadata bytes.
uint64_t meta_digest(const std::vector<char>& b) {
  uint64_t h = 1469598103934665603ull;
  for (char c : b) h = (h ^ (uint8_t)c) * 1099511628211ull;
  return h ^ (uint64_t)b.size();
}

// Copy the plan's metadata into the workspace with one host->device copy and record its
// digest for the workspace address; with stage == false copy nothing and check instead that
// the workspace holds this plan's metadata (launch-only calls).
jev_status stage_meta(jev_model* m, const Plan& p, const Layout& L, void* ws, hipStream_t s, bool stage,
                      bool may_alloc = true) {
  std::vector<char> buf(L.meta_end, 0);
  auto put = [&](size_t off, const void* src, size_t bytes) {
    if (bytes) std::memcpy(buf.data() + off, src, bytes);
  };
  put(L.tok, p.tok.data(), 4 * p.tok.size());
  put(L.pos, p.pos.data(), 4 * p.pos.size());
  put(L.seq_start, p.seq_start.data(), 4 * p.seq_start.size());
  put(L.read_rows, p.read_rows.data(), 4 * p.read_rows.size());
  put(L.tgt_ridx, p.tgt_ridx.data(), 4 * p.tgt_ridx.size());
  put(L.tgt_tok, p.tgt_tok.data(), 4 * p.tgt_tok.size());
  put(L.out_n, p.out_n.data(), 4 * p.out_n.size());
  put(L.mask, p.mask.data(), 8 * p.mask.size());
  put(L.pseg, p.pseg.data(), 4 * p.pseg.size());
  put(L.ptile, p.ptile.data(), 4 * p.ptile.size());
  const uint64_t h = meta_digest(buf);
  std::lock_guard<std::mutex> lock(m->staged_mu);
  if (!stage) {
    auto it = m->staged.find(ws);
    if (it == m->staged.end() || it->second != h)
      return fail(JEV_E_INVALID, "workspace does not hold this call's metadata: stage it with the copying call first");
    return JEV_OK;
  }
  if (may_alloc) HIP_OK(m->ring.init());
  if (m->ring.ready) {
    HIP_OK(m->ring.copy(ws, buf.data(), L.meta_end, s));
  } else {
    // no pinned ring and none may be made: copy and wait, so the host buffer outlives the copy
    HIP_OK(hipMemcpyAsync(ws, buf.data(), L.meta_end, hipMemcpyHostToDevice, s));
    HIP_OK(hipStreamSynchronize(s));
  }
  // bounded: a caller cycling through many workspaces forgets the oldest digests (a
  // launch-only call on such a workspace then asks for a fresh staging call)
  if (m->staged.size() >= kMaxStagedWorkspaces && !m->staged.count(ws)) m->staged.clear();
  m->staged[ws] = h;
  return JEV_OK;
}
}  // namespace

// ---------------------------------------------------------------------------
// entry points
// ---------------------------------------------------------------------------
// The causal forward over every row of the store: segment i's rows sit at positions 0..P_i-1
// and see only the rows of their own segment (sequence start = the segment's first row).
// Row sources: tok >= 0 an embedding row, tok = -1 - j row j of vis.
static jev_status prefill_rows(jev_prefix* p, const void* vis, std::vector<int32_t> tok, void* ws, size_t ws_bytes,
                               void* stream) {
  const jev_model* m = p->m;
  if (p->P == 0 || m->cfg.n_layers == 0) return JEV_OK;
  Plan plan;
  plan.T = p->P;
  plan.n_groups = (int)p->seg_len.size();
  plan.tok = std::move(tok);
  plan.pos.resize(p->P);
  plan.seq_start.resize(p->P);
  for (size_t i = 0; i < p->seg_len.size(); ++i)
    for (int j = 0; j < p->seg_len[i]; ++j) {
      plan.pos[p->seg_off[i] + j] = j;
      plan.seq_start[p->seg_off[i] + j] = p->seg_off[i];
    }
  const Layout L = make_layout(m, plan.T, 0, 0, 1, false, false, 0);
  if (!ws) return fail(JEV_E_INVALID, "null workspace");
  if (ws_bytes < L.total)
    return fail(JEV_E_WORKSPACE, "workspace too small: need " + std::to_string(L.total) + " bytes");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (jev_status st = stage_meta(p->m, plan, L, ws, s, true)) return st;
  Forward f(p, plan, L, ws, s, Mode::Prefill);
  jev_status st = f.run(vis);
  p->m->launches += f.launches;
  if (st) return st;
  p->m->prefills++;
  return JEV_OK;
}

extern "C" jev_status jev_prefill_prefix(jev_prefix* p, const void* vis_embeds, int32_t n_vis,
                                         const int32_t* text_ids, int32_t n_text, void* ws, size_t ws_bytes,
                                         void* stream) {
  if (!p) return fail(JEV_E_INVALID, "null prefix");
  const jev_model* m = p->m;
  if (p->seg_len.size() != 1) return fail(JEV_E_INVALID, "segmented prefix: use jev_prefill_segments");
  if (n_vis < 0 || n_text < 0) return fail(JEV_E_INVALID, "negative counts");
  if (n_vis + n_text != p->P) return fail(JEV_E_INVALID, "n_vis + n_text must equal prefix_len");
  if (n_vis > 0 && !vis_embeds) return fail(JEV_E_INVALID, "null vis_embeds");
  if (n_text > 0 && !text_ids) return fail(JEV_E_INVALID, "null text_ids");
  for (int i = 0; i < n_text; ++i)
    if (text_ids[i] < 0 || text_ids[i] >= m->cfg.vocab) return fail(JEV_E_INVALID, "text id out of range");
  std::vector<int32_t> tok(p->P);
  for (int i = 0; i < n_vis; ++i) tok[i] = -1 - i;
  for (int i = 0; i < n_text; ++i) tok[n_vis + i] = text_ids[i];
  return prefill_rows(p, vis_embeds, std::move(tok), ws, ws_bytes, stream);
}

extern "C" jev_status jev_prefill_segments(jev_prefix* p, const void* vis_embeds, const int32_t* n_vis,
                                           const int32_t* text_ids, const int32_t* n_text, void* ws,
                                           size_t ws_bytes, void* stream) {
  if (!p) return fail(JEV_E_INVALID, "null prefix");
  const jev_model* m = p->m;
  const int n = (int)p->seg_len.size();
  if (!n_vis || !n_text) return fail(JEV_E_INVALID, "null n_vis / n_text");
  long nv = 0, nt = 0;
  for (int i = 0; i < n; ++i) {
    if (n_vis[i] < 0 || n_text[i] < 0) return fail(JEV_E_INVALID, "negative counts");
    if (n_vis[i] + n_text[i] != p->seg_len[i])
      return fail(JEV_E_INVALID, "n_vis[" + std::to_string(i) + "] + n_text[" + std::to_string(i) +
                                     "] must equal the segment's length");
    nv += n_vis[i];
    nt += n_text[i];
  }
  if (nv > 0 && !vis_embeds) return fail(JEV_E_INVALID, "null vis_embeds");
  if (nt > 0 && !text_ids) return fail(JEV_E_INVALID, "null text_ids");
  for (long i = 0; i < nt; ++i)
    if (text_ids[i] < 0 || text_ids[i] >= m->cfg.vocab) return fail(JEV_E_INVALID, "text id out of range");
  std::vector<int32_t> tok(p->P);
  long vi = 0, ti = 0;
  for (int i = 0; i < n; ++i) {
    int r = p->seg_off[i];
    for (int j = 0; j < n_vis[i]; ++j) tok[r++] = (int32_t)(-1 - vi++);
    for (int j = 0; j < n_text[i]; ++j) tok[r++] = text_ids[ti++];
  }
  return prefill_rows(p, vis_embeds, std::move(tok), ws, ws_bytes, stream);
}

// segmented == false: every suffix over the one prefix.  Otherwise suffix b continues
// segment seg[b] of a segmented store: positions P_seg + j, prefix keys the segment's rows only.
static void* static_scratch(jev_status* st);
static constexpr size_t kStaticScratchBytes = 256ull << 20;

// ws == nullptr with use_static: the library's static device scratch (no allocation anywhere)
static jev_status score_suffixes(const jev_prefix* p, bool segmented, const int32_t* seg, const int32_t* ids,
                                 const int32_t* lens, int32_t B, int32_t S_max, const int32_t* cand_ids,
                                 const int32_t* n_cands, int32_t C_max, float* out_logp, void* ws, size_t ws_bytes,
                                 void* stream, bool stage, bool use_static = false) {
  if (!p) return fail(JEV_E_INVALID, "null prefix");
  jev_model* m = p->m;
  if (!segmented && p->seg_len.size() != 1) return fail(JEV_E_INVALID, "segmented prefix: use jev_score_segments");
  Plan plan;
  Status st = jevp::plan_suffixes(segmented ? 0 : p->P, m->cfg.vocab, ids, lens, B, S_max, cand_ids, n_cands, C_max,
                                  &plan);
  if (!st.ok()) return fail(st.code, st.msg);
  if (B == 0) return JEV_OK;
  if (!out_logp) return fail(JEV_E_INVALID, "null out_logp");
  if (segmented) {
    if (!seg) return fail(JEV_E_INVALID, "null seg");
    const int n = (int)p->seg_len.size();
    for (int b = 0; b < B; ++b)
      if (seg[b] < 0 || seg[b] >= n) return fail(JEV_E_INVALID, "seg[" + std::to_string(b) + "] out of range");
    plan.pseg.resize(2 * (size_t)plan.T);
    for (int b = 0, row = 0; b < B; ++b)
      for (int j = 0; j < lens[b]; ++j, ++row) {
        const int off = p->seg_off[seg[b]], len = p->seg_len[seg[b]];
        plan.pos[row] = len + j;
        plan.pseg[2 * row] = off;
        plan.pseg[2 * row + 1] = off + len;
      }
    const int G = m->cfg.n_q_heads / m->cfg.n_kv_heads;
    plan.ptile.resize(4 * (((size_t)G * plan.T + 127) / 128));
    plan.seg_keys = 64 * attn_seg_tiles(plan.pseg.data(), plan.T, G, plan.ptile.data());
  }
  const Layout L = make_layout(m, plan.T, (int)plan.read_rows.size(), (int)plan.tgt_tok.size(),
                               (int)plan.out_n.size(), false, false, p->P);
  if (use_static) {
    if (L.total > kStaticScratchBytes)
      return fail(JEV_E_WORKSPACE, "request needs " + std::to_string(L.total) + " bytes of scratch; the static "
                                   "scratch holds " + std::to_string(kStaticScratchBytes));
    jev_status st2 = JEV_OK;
    ws = static_scratch(&st2);
    if (st2) return st2;
    ws_bytes = kStaticScratchBytes;
  }
  if (!ws) return fail(JEV_E_INVALID, "null workspace");
  if (ws_bytes < L.total)
    return fail(JEV_E_WORKSPACE, "workspace too small: need " + std::to_string(L.total) + " bytes");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (jev_status e = stage_meta(m, plan, L, ws, s, stage, !use_static)) return e;
  Forward f(p, plan, L, ws, s, Mode::Score);
  jev_status e = f.run(nullptr);
  if (!e) e = f.readout(out_logp, nullptr);
  m->launches += f.launches;
  if (e) return e;
  m->forwards++;
  m->rows += (uint64_t)plan.T;
  return JEV_OK;
}

extern "C" jev_status jev_score_suffixes(const jev_prefix* p, const int32_t* ids, const int32_t* lens, int32_t B,
                                         int32_t S_max, const int32_t* cand_ids, const int32_t* n_cands,
                                         int32_t C_max, float* out_logp, void* ws, size_t ws_bytes, void* stream) {
  return score_suffixes(p, false, nullptr, ids, lens, B, S_max, cand_ids, n_cands, C_max, out_logp, ws, ws_bytes,
                        stream, true);
}

// ---------------------------------------------------------------------------
// scoring without allocation: the workspace is a file-scope device array
// ---------------------------------------------------------------------------
// Each device that runs the library holds its own copy of `scratch` until the process ends.
// In host code its name is only a stand-in: the device address comes from hipGetSymbolAddress,
// once per device, and only that address is ever handed to kernels or copies.
static __device__ __align__(256) char scratch[kStaticScratchBytes];
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64] = {};

static void* static_scratch(jev_status* st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    *st = fail(JEV_E_HIP, "no current HIP device for the static scratch");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *st = fail(JEV_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

extern "C" size_t jev_static_scratch_bytes(void) { return kStaticScratchBytes; }

extern "C" jev_status jev_score_suffixes_noalloc(const jev_prefix* p, const int32_t* ids, const int32_t* lens,
                                                 int32_t B, int32_t S_max, const int32_t* cand_ids,
                                                 const int32_t* n_cands, int32_t C_max, float* out_logp,
                                                 void* stream) {
  return score_suffixes(p, false, nullptr, ids, lens, B, S_max, cand_ids, n_cands, C_max, out_logp, nullptr, 0,
                        stream, true, true);
}

extern "C" jev_status jev_score_segments(const jev_prefix* p, const int32_t* seg, const int32_t* ids,
                                         const int32_t* lens, int32_t B, int32_t S_max, const int32_t* cand_ids,
                                         const int32_t* n_cands, int32_t C_max, float* out_logp, void* ws,
                                         size_t ws_bytes, void* stream) {
  return score_suffixes(p, true, seg, ids, lens, B, S_max, cand_ids, n_cands, C_max, out_logp, ws, ws_bytes, stream,
                        true);
}

extern "C" jev_status jev_score_suffixes_launch(const jev_prefix* p, const int32_t* ids, const int32_t* lens,
                                                int32_t B, int32_t S_max, const int32_t* cand_ids,
                                                const int32_t* n_cands, int32_t C_max, float* out_logp, void* ws,
                                                size_t ws_bytes, void* stream) {
  return score_suffixes(p, false, nullptr, ids, lens, B, S_max, cand_ids, n_cands, C_max, out_logp, ws, ws_bytes,
                        stream, false);
}

static jev_status score_tree(const jev_prefix* p, const int32_t* stem_ids, const int32_t* stem_lens, int32_t Q,
                             int32_t S_max, const int32_t* cand_tok, const int32_t* cand_lens, const int32_t* n_cands,
                             int32_t C_max, int32_t K_max, int32_t mode, float* out_score, float* out_norm, void* ws,
                             size_t ws_bytes, void* stream, bool stage) {
  if (!p) return fail(JEV_E_INVALID, "null prefix");
  jev_model* m = p->m;
  if (p->seg_len.size() != 1) return fail(JEV_E_INVALID, "segmented prefix: jev_score_tree takes one prefix");
  Plan plan;
  Status st = jevp::plan_tree(p->P, m->cfg.vocab, stem_ids, stem_lens, Q, S_max, cand_tok, cand_lens, n_cands,
                              C_max, K_max, mode, &plan);
  if (!st.ok()) return fail(st.code, st.msg);
  if (Q == 0) return JEV_OK;
  if (!out_score) return fail(JEV_E_INVALID, "null out_score");
  const int R = (int)plan.read_rows.size();
  const int NT = (int)plan.tgt_tok.size();
  const Layout L = make_layout(m, plan.T, R, NT, (int)plan.out_n.size(), true, true, p->P);
  if (!ws) return fail(JEV_E_INVALID, "null workspace");
  if (ws_bytes < L.total)
    return fail(JEV_E_WORKSPACE, "workspace too small: need " + std::to_string(L.total) + " bytes");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (jev_status e = stage_meta(m, plan, L, ws, s, stage)) return e;
  Forward f(p, plan, L, ws, s, Mode::Tree);
  f.tree_C = C_max;
  f.tree_K = K_max;
  jev_status e = f.run(nullptr);
  if (!e) e = f.readout(out_score, out_norm);
  m->launches += f.launches;
  if (e) return e;
  m->forwards++;
  m->rows += (uint64_t)plan.T;
  return JEV_OK;
}

extern "C" jev_status jev_score_tree(const jev_prefix* p, const int32_t* stem_ids, const int32_t* stem_lens,
                                     int32_t Q, int32_t S_max, const int32_t* cand_tok, const int32_t* cand_lens,
                                     const int32_t* n_cands, int32_t C_max, int32_t K_max, int32_t mode,
                                     float* out_score, float* out_norm, void* ws, size_t ws_bytes, void* stream) {
  return score_tree(p, stem_ids, stem_lens, Q, S_max, cand_tok, cand_lens, n_cands, C_max, K_max, mode, out_score,
                    out_norm, ws, ws_bytes, stream, true);
}

extern "C" jev_status jev_score_tree_launch(const jev_prefix* p, const int32_t* stem_ids, const int32_t* stem_lens,
                                            int32_t Q, int32_t S_max, const int32_t* cand_tok,
                                            const int32_t* cand_lens, const int32_t* n_cands, int32_t C_max,
                                            int32_t K_max, int32_t mode, float* out_score, float* out_norm, void* ws,
                                            size_t ws_bytes, void* stream) {
  return score_tree(p, stem_ids, stem_lens, Q, S_max, cand_tok, cand_lens, n_cands, C_max, K_max, mode, out_score,
                    out_norm, ws, ws_bytes, stream, false);
}

extern "C" jev_status jev_tree_plan_size(const int32_t* stem_ids, const int32_t* stem_lens, int32_t Q,
                                         int32_t S_max, const int32_t* cand_tok, const int32_t* cand_lens,
                                         const int32_t* n_cands, int32_t C_max, int32_t K_max, int32_t mode,
                                         int32_t* rows, int32_t* seqs, int32_t* targets) {
  if (!rows || !seqs || !targets) return fail(JEV_E_INVALID, "null output");
  Plan plan;
  Status st = jevp::plan_tree(0, -1, stem_ids, stem_lens, Q, S_max, cand_tok, cand_lens, n_cands, C_max, K_max,
                              mode, &plan);
  if (!st.ok()) return fail(st.code, st.msg);
  *rows = plan.T;
  *seqs = plan.n_groups;
  *targets = (int32_t)plan.tgt_tok.size();
  return JEV_OK;
}

extern "C" jev_status jev_tree_plan_rows(const int32_t* stem_ids, const int32_t* stem_lens, int32_t Q,
                                         int32_t S_max, const int32_t* cand_tok, const int32_t* cand_lens,
                                         const int32_t* n_cands, int32_t C_max, int32_t K_max, int32_t mode,
                                         int32_t* row_tok, int32_t* row_depth, int32_t* row_group,
                                         uint64_t* row_mask, int32_t* target_row) {
  if (!row_tok || !row_depth || !row_group || !row_mask || !target_row) return fail(JEV_E_INVALID, "null output");
  Plan plan;
  Status st = jevp::plan_tree(0, -1, stem_ids, stem_lens, Q, S_max, cand_tok, cand_lens, n_cands, C_max, K_max,
                              mode, &plan);
  if (!st.ok()) return fail(st.code, st.msg);
  for (int r = 0; r < plan.T; ++r) {
    row_tok[r] = plan.tok[r];
    row_depth[r] = plan.depth[r];
    row_group[r] = plan.group[r];
    row_mask[r] = plan.mask[r];
  }
  for (size_t i = 0; i < plan.tgt_tok.size(); ++i)
    target_row[i] = plan.tgt_tok[i] >= 0 ? plan.read_rows[plan.tgt_ridx[i]] : -1;
  return JEV_OK;
}

extern "C" jev_status jev_segment_plan_tiles(const int32_t* pseg, int32_t T, int32_t G, int32_t* ptile,
                                             int32_t* max_tiles) {
  if (T < 0 || G < 1) return fail(JEV_E_INVALID, "T must be >= 0 and G >= 1");
  if (T > 0 && (!pseg || !ptile)) return fail(JEV_E_INVALID, "null array");
  for (int t = 0; t < T; ++t)
    if (pseg[2 * t] < 0 || pseg[2 * t + 1] < pseg[2 * t]) return fail(JEV_E_INVALID, "bad key range");
  const int mx = T > 0 ? attn_seg_tiles(pseg, T, G, ptile) : 0;
  if (max_tiles) *max_tiles = mx;
  return JEV_OK;
}

extern "C" jev_status jev_attn_schedule(int32_t T, int32_t G, int32_t Hkv, int32_t P, int32_t own_tiles,
                                        int32_t segmented, int32_t* n_split, int32_t* chunk, int32_t* blocks,
                                        int32_t* spans, int32_t cap, int32_t* n_spans) {
  if (T < 1 || G < 1 || Hkv < 1 || P < 0 || own_tiles < 0 || (long)G * T > (1L << 24))
    return fail(JEV_E_INVALID, "sizes out of range");
  if (!n_split || !chunk || !blocks) return fail(JEV_E_INVALID, "null output");
  const AttnSchedule sc = attn_schedule(T, G, Hkv, P, own_tiles, segmented != 0);
  const int n_rt = (G * T + 127) / 128, nt_u = (P + AT_KEYS - 1) / AT_KEYS + own_tiles;
  *n_split = sc.n_split;
  *chunk = sc.chunk;
  *blocks = sc.chunk > 0 ? (int)(((long)n_rt * Hkv * nt_u + sc.chunk - 1) / sc.chunk) : n_rt * Hkv * sc.n_split;
  if (!spans || sc.chunk <= 0) {
    if (n_spans) *n_spans = 0;
    return JEV_OK;
  }
  int n = 0;
  bool over = false;
  for (int b = 0; b < *blocks; ++b)
    attn_balanced_items(b, sc.chunk, nt_u, n_rt * Hkv, [&](int u, int z, int vb, int ve, bool last) {
      if (n >= cap) {
        over = true;
        return;
      }
      const int32_t row[7] = {b, u, z, vb, ve, last ? 1 : 0, attn_balanced_item_slots(u, sc.chunk, nt_u)};
      std::memcpy(spans + 7 * n++, row, sizeof(row));
    });
  if (n_spans) *n_spans = n;
  return over ? fail(JEV_E_INVALID, "spans capacity too small") : JEV_OK;
}

extern "C" jev_status jev_profile_start(jev_model* m) {
  if (!m) return fail(JEV_E_INVALID, "null model");
  m->prof.recs.clear();
  m->prof.used = 0;
  m->prof.on = true;
  return JEV_OK;
}

extern "C" jev_status jev_profile_stop(jev_model* m, jev_kernel_stat* out, int32_t max_out, int32_t* n_out) {
  if (!m || !n_out || (max_out > 0 && !out)) return fail(JEV_E_INVALID, "null argument");
  Profiler& P = m->prof;
  P.on = false;
  std::vector<jev_kernel_stat> acc(K_NKINDS);
  for (int k = 0; k < K_NKINDS; ++k) {
    std::memset(&acc[k], 0, sizeof(jev_kernel_stat));
    std::strncpy(acc[k].name, kKindName[k], sizeof(acc[k].name) - 1);
  }
  if (!P.recs.empty()) {
    hipError_t e = hipEventSynchronize(P.recs.back().b);
    if (e != hipSuccess) return fail(JEV_E_HIP, std::string("hipEventSynchronize: ") + hipGetErrorString(e));
  }
  for (const ProfRec& r : P.recs) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) continue;
    jev_kernel_stat& a = acc[r.kind];
    a.launches++;
    a.ms += ms;
    a.flops += r.flops;
    a.bytes += r.bytes;
  }
  P.recs.clear();
  P.used = 0;
  int n = 0;
  for (int k = 0; k < K_NKINDS; ++k)
    if (acc[k].launches) {
      if (n < max_out) out[n] = acc[k];
      ++n;
    }
  *n_out = n;
  return JEV_OK;
}
