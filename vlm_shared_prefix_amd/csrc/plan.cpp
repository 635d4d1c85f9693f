// Request planning (host).  See plan.h.
//
// Suffix batches ("How to Deploy Visual Jev ...", Step 3; Ochevid "Run"):
// right-padded [B, S_max] ids become T = sum(lens) packed rows; suffix b's
// token j sits at position P + j and sees the prefix plus its own rows
// 0..j.  Padding is dropped here, so pad ids are never read on the device.
//
// Candidate trees ("FastJEV", §3.3): per question a group of rows holds the
// stem as a chain and the candidates' fed tokens (all but the last).  In the
// trie layout a token is merged with an existing node only if that node has
// the same parent and the same token, so equal tokens after different
// histories stay separate; the stem-only layout never merges candidate
// tokens; the flat layout gives every candidate its own group.  A node at
// depth d below the prefix sits at position P + d and sees its ancestors and
// itself (a 64-bit mask over its group).  The row that predicts candidate
// token k is the node right before it: the last stem node for k = 0.
#include "plan.h"

#include <map>
#include <utility>

namespace jevp {

static Status err(jev_status c, std::string m) {
  Status s;
  s.code = c;
  s.msg = std::move(m);
  return s;
}

Status plan_suffixes(int P, int vocab, const int32_t* ids, const int32_t* lens, int B, int S_max,
                     const int32_t* cand_ids, const int32_t* n_cands, int C_max, Plan* out) {
  if (B < 0) return err(JEV_E_INVALID, "B must be >= 0");
  if (B == 0) {
    *out = Plan();
    return Status();
  }
  if (!ids || !lens || !cand_ids || !n_cands) return err(JEV_E_INVALID, "null host array");
  if (S_max < 1) return err(JEV_E_INVALID, "S_max must be >= 1");
  if (S_max > kMaxSuffixLen) return err(JEV_E_UNSUPPORTED, "S_max > 256");
  if (C_max < 1) return err(JEV_E_INVALID, "C_max must be >= 1");
  if (C_max > kMaxCands) return err(JEV_E_UNSUPPORTED, "C_max > 64");
  long T = 0;
  for (int b = 0; b < B; ++b) {
    if (lens[b] < 1 || lens[b] > S_max)
      return err(JEV_E_INVALID, "lens[" + std::to_string(b) + "] = " + std::to_string(lens[b]) +
                                    " outside [1, S_max]");
    if (n_cands[b] < 1 || n_cands[b] > C_max)
      return err(JEV_E_INVALID, "n_cands[" + std::to_string(b) + "] outside [1, C_max]");
    for (int j = 0; j < lens[b]; ++j) {
      const int v = ids[(size_t)b * S_max + j];
      if (v < 0 || v >= vocab)
        return err(JEV_E_INVALID, "ids[" + std::to_string(b) + "," + std::to_string(j) + "] out of range");
    }
    for (int c = 0; c < n_cands[b]; ++c) {
      const int v = cand_ids[(size_t)b * C_max + c];
      if (v < 0 || v >= vocab)
        return err(JEV_E_INVALID, "cand_ids[" + std::to_string(b) + "," + std::to_string(c) + "] out of range");
    }
    T += lens[b];
  }
  if (T > kMaxRows) return err(JEV_E_UNSUPPORTED, "more than 65536 suffix rows");
  Plan p;
  p.T = (int)T;
  p.n_groups = B;
  p.tok.reserve(T);
  p.pos.reserve(T);
  p.seq_start.reserve(T);
  p.group.reserve(T);
  int row = 0;
  for (int b = 0; b < B; ++b) {
    const int start = row;
    for (int j = 0; j < lens[b]; ++j, ++row) {
      p.tok.push_back(ids[(size_t)b * S_max + j]);
      p.pos.push_back(P + j);
      p.seq_start.push_back(start);
      p.group.push_back(b);
    }
    p.read_rows.push_back(row - 1);
    p.out_n.push_back(n_cands[b]);
    for (int c = 0; c < C_max; ++c) {
      p.tgt_ridx.push_back(b);
      p.tgt_tok.push_back(c < n_cands[b] ? cand_ids[(size_t)b * C_max + c] : -1);
    }
  }
  *out = std::move(p);
  return Status();
}

namespace {
struct TreeBuilder {
  Plan& p;
  int P;
  int group_start = 0;
  explicit TreeBuilder(Plan& plan, int prefix) : p(plan), P(prefix) {}
  void new_group() {
    group_start = p.T;
    ++p.n_groups;
  }
  // returns the new row, or -1 if the group overflows 64 rows
  int add(int tok, int depth, int parent) {
    const int local = p.T - group_start;
    if (local >= kMaxGroupRows) return -1;
    const uint64_t pm = parent >= 0 ? p.mask[parent] : 0ull;
    p.tok.push_back(tok);
    p.pos.push_back(P + depth);
    p.depth.push_back(depth);
    p.seq_start.push_back(group_start);
    p.group.push_back(p.n_groups - 1);
    p.mask.push_back(pm | (1ull << local));
    return p.T++;
  }
};
}  // namespace

Status plan_tree(int P, int vocab, const int32_t* stem_ids, const int32_t* stem_lens, int Q, int S_max,
                 const int32_t* cand_tok, const int32_t* cand_lens, const int32_t* n_cands, int C_max,
                 int K_max, int mode, Plan* out) {
  if (Q < 0) return err(JEV_E_INVALID, "Q must be >= 0");
  if (mode < JEV_TREE_TRIE || mode > JEV_TREE_FLAT) return err(JEV_E_INVALID, "unknown tree mode");
  if (Q == 0) {
    *out = Plan();
    return Status();
  }
  if (!stem_ids || !stem_lens || !cand_tok || !cand_lens || !n_cands) return err(JEV_E_INVALID, "null host array");
  if (S_max < 1 || C_max < 1 || K_max < 1) return err(JEV_E_INVALID, "S_max, C_max, K_max must be >= 1");
  if (S_max > kMaxGroupRows || K_max > kMaxGroupRows) return err(JEV_E_UNSUPPORTED, "S_max or K_max > 64");
  if (C_max > kMaxCands) return err(JEV_E_UNSUPPORTED, "C_max > 64");
  for (int q = 0; q < Q; ++q) {
    if (stem_lens[q] < 1 || stem_lens[q] > S_max) return err(JEV_E_INVALID, "stem_lens out of [1, S_max]");
    if (n_cands[q] < 1 || n_cands[q] > C_max) return err(JEV_E_INVALID, "n_cands out of [1, C_max]");
    if (vocab >= 0)
      for (int j = 0; j < stem_lens[q]; ++j) {
        const int v = stem_ids[(size_t)q * S_max + j];
        if (v < 0 || v >= vocab) return err(JEV_E_INVALID, "stem id out of range");
      }
    for (int c = 0; c < n_cands[q]; ++c) {
      const int K = cand_lens[(size_t)q * C_max + c];
      if (K < 1 || K > K_max) return err(JEV_E_INVALID, "cand_lens out of [1, K_max]");
      if (vocab >= 0)
        for (int k = 0; k < K; ++k) {
          const int v = cand_tok[((size_t)q * C_max + c) * K_max + k];
          if (v < 0 || v >= vocab) return err(JEV_E_INVALID, "candidate token out of range");
        }
    }
  }

  Plan p;
  TreeBuilder tb(p, P);
  const size_t NT = (size_t)Q * C_max * K_max;
  std::vector<int32_t> pred_row(NT, -1);
  p.tgt_tok.assign(NT, -1);
  auto overflow = [&]() { return err(JEV_E_UNSUPPORTED, "a question's group needs more than 64 rows"); };

  for (int q = 0; q < Q; ++q) {
    const int s = stem_lens[q];
    const int32_t* stem = stem_ids + (size_t)q * S_max;
    auto add_stem = [&]() -> int {
      int prev = -1;
      for (int j = 0; j < s; ++j) {
        prev = tb.add(stem[j], j, prev);
        if (prev < 0) return -1;
      }
      return prev;
    };
    int last_stem = -1;
    std::map<std::pair<int, int>, int> children;   // (parent row, token) -> row
    if (mode != JEV_TREE_FLAT) {
      tb.new_group();
      last_stem = add_stem();
      if (last_stem < 0) return overflow();
    }
    for (int c = 0; c < n_cands[q]; ++c) {
      const int K = cand_lens[(size_t)q * C_max + c];
      const int32_t* w = cand_tok + ((size_t)q * C_max + c) * K_max;
      if (mode == JEV_TREE_FLAT) {
        tb.new_group();
        last_stem = add_stem();
        if (last_stem < 0) return overflow();
      }
      int parent = last_stem;
      for (int k = 0; k < K; ++k) {
        const size_t ti = ((size_t)q * C_max + c) * K_max + k;
        pred_row[ti] = parent;
        p.tgt_tok[ti] = w[k];
        if (k == K - 1) break;          // the last token is predicted, never fed
        int child = -1;
        if (mode == JEV_TREE_TRIE) {
          auto it = children.find({parent, w[k]});
          if (it != children.end()) child = it->second;
        }
        if (child < 0) {
          child = tb.add(w[k], s + k, parent);
          if (child < 0) return overflow();
          if (mode == JEV_TREE_TRIE) children[{parent, w[k]}] = child;
        }
        parent = child;
      }
    }
    p.out_n.push_back(n_cands[q]);
  }
  if (p.T > kMaxRows) return err(JEV_E_UNSUPPORTED, "more than 65536 tree rows");

  // scored rows: unique predictor rows, in row order
  std::vector<int32_t> ridx_of(p.T, -1);
  for (size_t i = 0; i < NT; ++i)
    if (pred_row[i] >= 0) ridx_of[pred_row[i]] = 1;
  for (int r = 0; r < p.T; ++r)
    if (ridx_of[r] > 0) {
      ridx_of[r] = (int)p.read_rows.size();
      p.read_rows.push_back(r);
    }
  p.tgt_ridx.assign(NT, 0);
  for (size_t i = 0; i < NT; ++i)
    if (pred_row[i] >= 0) p.tgt_ridx[i] = ridx_of[pred_row[i]];
  *out = std::move(p);
  return Status();
}

}  // namespace jevp
