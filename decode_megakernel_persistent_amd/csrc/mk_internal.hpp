// Internal formats shared by the host planner and the device megakernel:
// the 32-byte task record, the plan image in device memory and the kernel
// argument block. Not part of the public ABI (include/mk.h), except that the
// task record layout is documented for mk_plan_export consumers.
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define MK_HD __host__ __device__
#else
#define MK_HD
#endif

namespace mk {

// Task kinds. One task = one tile of one operation (megakernel page,
// "What is a Megakernel?": the unit of scheduling is one tile of one op).
enum Op : uint8_t {
  OP_NONE = 0,
  OP_QKV = 1,     // a0 = kv group g, a1 = first rotary pair, a2 = pairs
  OP_ATTN = 2,    // a0 = b, a1 = g, a2 = first page, a3 = pages; aux = split index
  OP_COMB = 3,    // a0 = b, a1 = q head, a2 = heads (1), a3 = splits of (b, g)
  OP_O = 4,       // a1 = first row, a2 = rows
  OP_ROUTER = 5,  // a1 = first expert row, a2 = rows
  OP_GATEUP = 6,  // a0 = b (MoE) or -1 (dense, all rows), aux = slot j, a1 = first row, a2 = rows
  OP_DOWN = 7,    // a1 = first row, a2 = rows
  OP_LM = 8,      // a1 = first row, a2 = rows, a3 = index of this LM tile
  OP_FINAL = 9,   // a0 = LM tiles
  OP_COUNT = 10
};

// flags: bit 0 TF_WRITE_TOPK; bits 4-7 log2 of the GEMV threads per row (TC).
enum TaskFlags : uint8_t { TF_WRITE_TOPK = 1 };

constexpr uint16_t NO_CTR = 0xFFFF;

struct Task {
  uint8_t op, flags;
  uint16_t layer;
  uint16_t wait_a, wait_b;  // counter indices (NO_CTR: none); wait_a gates address
                            // computation (routing), wait_b gates the data
  uint16_t cnt_a, cnt_b;    // per-epoch producer counts of wait_a / wait_b
  uint16_t signal;          // counter incremented on completion (NO_CTR: none)
  uint16_t aux;
  int32_t a0, a1, a2, a3;
};
static_assert(sizeof(Task) == 32, "task record is 32 bytes");

// Plan image: u32 header[PLAN_HDR_WORDS], u32 cu_off[n_cu + 1] (task index
// ranges per list), padding to 32 B, Task tasks[n_tasks] (lists back to back).
constexpr uint32_t PLAN_MAGIC = 0x31504B4Du;  // "MKP1"
constexpr int PLAN_HDR_WORDS = 16;
enum PlanHdr { H_MAGIC = 0, H_NCU = 1, H_NTASKS = 2, H_NCTR = 3, H_TASK_OFF_BYTES = 4,
               H_STAGES = 5 };

constexpr int CTR_STRIDE = 16;  // u32 words between counters (one 64-byte line each)
constexpr int NT = 512;         // threads per workgroup (8 wave64)
constexpr int NWAVE = NT / 64;

// Per-task trace record (u64 words, constant 100 MHz clock): task start,
// routing wait begin/end, data wait begin/end (0 where the task has no such
// wait), body end, signal end, and (cu << 32 | op << 16 | layer).
constexpr int TRACE_WORDS = 8;

// Status words written by the device on failure.
enum DevStatus : uint32_t { DS_OK = 0, DS_TIMEOUT = 1, DS_BOUNDS = 2 };

// Thread mapping of a block GEMV over rows of K bf16 elements: each row is
// read as K/8 16-byte chunks by TC threads (a power of two in [32, NT]),
// CPL chunks per thread. Returns false when K has no such mapping.
MK_HD inline bool gemv_map(int K, int* tc, int* cpl) {
  if (K <= 0 || K % 8) return false;
  int chunks = K / 8;
  for (int c = 1; c <= 4; ++c) {
    if (chunks % c) continue;
    int t = chunks / c;
    if (t >= 32 && t <= NT && (t & (t - 1)) == 0) { *tc = t; *cpl = c; return true; }
  }
  return false;
}

// Rows of W_qkv are taken by kv group and rotary pair: group g owns the q
// rows of its HG query heads, then its k head, then its v head; pair p of the
// group covers dims i and i + D/2 of one head (rotation partners). Returns
// the section (0 q, 1 k, 2 v), the head (q: query head; k, v: kv head), the
// dim i < D/2 and the logical row of dim i (the partner row is +D/2).
MK_HD inline int qkv_pair(int p, int g, int HG, int D, int Hq, int Hkv, int* head, int* i, int* row) {
  const int h2 = D / 2;
  if (p < HG * h2) {
    *head = g * HG + p / h2; *i = p % h2; *row = *head * D + *i; return 0;
  }
  p -= HG * h2;
  if (p < h2) { *head = g; *i = p; *row = Hq * D + g * D + p; return 1; }
  p -= h2;
  *head = g; *i = p; *row = (Hq + Hkv) * D + g * D + p; return 2;
}

// Floats of LDS available to one task's per-row partial sums.
constexpr int GEMV_LDS_FLOATS = 8192;

struct KArgs {
  // shape
  int32_t L, H, Hq, Hkv, D, HG, F, E, K, V, B, max_pages, dense, norm_topk;
  float eps, attn_scale;
  // weights (bf16)
  const uint16_t *embed, *attn_norm, *wqkv, *wo, *ffn_norm, *router, *gate, *up, *down,
      *final_norm, *lm;
  // KV cache
  uint16_t* pool;
  int64_t page_stride, layer_stride;  // bf16 elements
  int64_t n_pages;
  const int32_t* page_table;
  int32_t* seq_lens;
  const float *rope_cos, *rope_sin;
  int32_t n_rope, bound;
  // io
  const int32_t* tok_in;
  int32_t* tok_out;
  int32_t* topk_ids;
  float* topk_w;
  float* logits;
  // workspace (fp32 unless noted) and per-layer strides in elements
  float *xa, *xf, *q, *part, *o, *rlog, *act;
  uint32_t* lmpart;  // [n_lm][B][2] (value bits, index)
  int64_t s_x, s_q, s_part, s_o, s_rlog, s_act;
  int32_t S_max, n_lm;
  // plan and sync
  const uint32_t* plan;
  uint32_t* ctr;
  uint32_t* status;
  uint32_t epoch;
  uint64_t timeout_ticks;  // of the 100 MHz constant clock
  uint64_t* trace;         // NULL, or TRACE_WORDS per task (see mk_step_buffers.trace)
};

}  // namespace mk
