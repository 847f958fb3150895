// Host-side plan object (opaque mk_plan_t of include/mk.h).
#pragma once
#include <string>
#include <vector>

#include "mk.h"
#include "mk_internal.hpp"

struct mk_plan {
  uint64_t uid = 0;  // unique per plan built in this process (never reused)
  mk_model_desc m;
  mk_plan_opts opts = {};  // as built (n_cu resolved), for mk_plan_update
  int32_t B = 0, max_pages = 0, bound = 0, n_cu = 0;
  bool batch = false;                 // B > 1: MFMA batch tasks
  std::vector<int32_t> seq_lens, page_table;
  std::vector<int32_t> seq_bound;     // per sequence context bound

  // derived shape
  int32_t HG = 0, QKV_ROWS = 0, F = 0, n_pairs_g = 0;

  std::vector<std::vector<mk::Task>> lists;  // per compute unit, in execution order
  std::vector<int32_t> stage_of_task;        // parallel to the flattened lists
  std::vector<uint32_t> targets;             // per counter: producers per epoch
  std::vector<std::string> ctr_name;

  // counter ids
  std::vector<int32_t> c_qkv, c_attn;  // [L][Hkv]
  std::vector<int32_t> c_comb, c_o, c_router, c_expert;  // [L]
  std::vector<int32_t> c_queue;  // [L] attention split queue (queue mode)
  std::vector<int32_t> c_topk, c_bcomb;  // [L] batch: top-k per sequence, expert combine
  int o_kb = 1;                          // batch: reduction blocks of the O projection
  int q_kb = 1;                          // batch: reduction blocks of the QKV projection
  int q_rb = 0;                          // batch: QKV row blocks (tasks per reduction block)
  int32_t c_lm = -1;
  bool attn_queue = false;
  bool router_fold = false;         // batch-1 MoE: router tasks beside O (TF_FOLD)
  bool expert_share = false;        // batch MoE: expert rows shared by live routing (TF_SHARE)

  int32_t S_max = 0;                // attention splits per (b, g), max over b
  int32_t comb_dim_tasks = 1;       // combine tasks per (b, query head)
  int32_t kernel_class = -1;        // compiled kernel variant for this shape
  std::vector<int32_t> n_split;     // per b
  std::vector<mk::Task> split_table;  // queue plans: the splits queue tasks pull (every layer)
  int32_t n_lm = 0, n_stages = 0;

  // workspace layout: base offset (bytes) and per-layer stride (bytes) per MK_BUF_*
  static constexpr int N_BUF = 14;
  size_t ws_off[N_BUF] = {}, ws_stride[N_BUF] = {}, ws_layer_bytes[N_BUF] = {};
  int32_t n_exp_parts = 1;          // batch: expert tasks per expert
  size_t ws_total = 0;

  std::vector<uint8_t> image;  // device image
  size_t n_tasks = 0;
};

inline int mk_buf_lmpart() { return MK_BUF_LMPART; }

namespace mkh {
void set_error(const std::string& s);
mk_status fail(mk_status st, const std::string& s);
}  // namespace mkh
