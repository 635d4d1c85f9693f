// Host-side request planning: validation, packing of suffix rows and the
// candidate prefix tree.  Plain C++17, no HIP dependency.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/jev.h"

namespace jevp {

// Rows of one batched forward plus what the readout needs.
struct Plan {
  int T = 0;                          // decoder rows
  std::vector<int32_t> tok;           // [T] token id of the row
  std::vector<int32_t> pos;           // [T] RoPE position
  std::vector<int32_t> seq_start;     // [T] first row of the row's sequence / group
  std::vector<uint64_t> mask;         // [T] tree visibility over the group; empty = causal
  std::vector<int32_t> depth;         // [T] depth below the prefix (tree plans)
  std::vector<int32_t> group;         // [T] group index
  int n_groups = 0;
  // readout
  std::vector<int32_t> read_rows;     // [R] rows that need the final norm
  std::vector<int32_t> tgt_ridx;      // [NT] target -> index into read_rows
  std::vector<int32_t> tgt_tok;       // [NT] target token (-1: unused slot)
  std::vector<int32_t> out_n;         // [B or Q] valid candidates per output row
  // segmented prefixes (empty otherwise): per row its prefix keys [2t, 2t+1]; per 128-row
  // attention tile its prefix key tiles and fully visible keys (4 ints); seg_keys: 64 x the
  // largest tile count (the attention split rule's prefix length)
  std::vector<int32_t> pseg;
  std::vector<int32_t> ptile;
  int seg_keys = -1;
};

// Validation result.
struct Status {
  jev_status code = JEV_OK;
  std::string msg;
  bool ok() const { return code == JEV_OK; }
};

Status plan_suffixes(int P, int vocab, const int32_t* ids, const int32_t* lens, int B, int S_max,
                     const int32_t* cand_ids, const int32_t* n_cands, int C_max, Plan* out);

// vocab < 0 skips the id range checks (planning-only helpers).
Status plan_tree(int P, int vocab, const int32_t* stem_ids, const int32_t* stem_lens, int Q, int S_max,
                 const int32_t* cand_tok, const int32_t* cand_lens, const int32_t* n_cands, int C_max,
                 int K_max, int mode, Plan* out);

constexpr int kMaxSuffixLen = 256;
constexpr int kMaxCands = 64;
constexpr int kMaxRows = 65536;
constexpr int kMaxGroupRows = 64;
constexpr int kMaxPrefix = 32768;
constexpr int kMaxSegments = 64;   // independent prefixes in one segmented store

}  // namespace jevp
