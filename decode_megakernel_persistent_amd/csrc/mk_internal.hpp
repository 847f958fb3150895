// Internal formats shared by the host planner and the device megakernel:
// the 32-byte task record, the plan image in device memory, the tagged
// activation word and the kernel argument block. Not part of the public ABI
// (include/mk.h), except that the task record layout is documented for
// mk_plan_export consumers.
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
  OP_ATTN = 2,    // a0 = b, a1 = g, a2 = first page, a3 = pages; aux = split index;
                  // with TF_QUEUE: splits pulled from a shared queue: a0 = queue
                  // counter, a1 = first record of the splits in the plan's split
                  // table, a2 = splits, a3 = queue tasks of the layer
  OP_COMB = 3,    // a0 = b, a1 = query head, a2 = first dim, a3 = dims; aux = splits of (b, g)
  OP_O = 4,       // a1 = first row, a2 = rows
  OP_ROUTER = 5,  // a1 = first expert row, a2 = rows
  OP_EXPERT = 6,  // gate/up part: a0 = b, aux = expert slot j, a1 = first FFN row, a2 = FFN
                  // rows (may be 0); down part: a3 = first hidden row << 16 | hidden rows
                  // (may be 0), over every slot of sequence 0
                  // (7 is unused)
  OP_LM = 8,      // a1 = first row, a2 = rows, a3 = index of this LM tile
  OP_FINAL = 9,   // a0 = LM tiles, a2 = rows per tile
  // batch (B > 1) tasks: the dense projections cover all sequences at once
  // as MFMA tiles of 16-row blocks
  OP_BQKV = 10,   // a0 = kv group g, a1 = first rotary pair, a2 = pairs
  OP_BO = 11,     // a0 = reduction block, a1 = first row, a2 = rows, a3 = reduction blocks
                  // (TF_REDUCE: the rows' sum over the blocks)
                  // (12 is unused)
  OP_TOPK = 13,   // a0 = b: router rows, softmax and top-k of one sequence
  OP_BEXP = 14,   // a0 = expert, a1 = first FFN row, a2 = FFN rows,
                  // a3 = first hidden row << 16 | hidden rows (down part)
  OP_BCOMB = 15,  // a0 = b, a1 = first row, a2 = rows: weighted expert sum + residual
  OP_BLM = 16,    // a1 = first row, a2 = rows, a3 = index of this LM tile
  OP_BFINAL = 17, // a0 = LM tiles, a1 = b, a2 = rows per tile
  OP_COUNT = 18
};

// TF_LOGITS (batch top-k): the router rows of the sequence were computed by
// router tasks; the task reads the logits instead of computing them.
// TF_STAGE_KV: before its body the task requests the first pages of this
// unit's next attention split (the first attention task at most STAGE_SCAN
// tasks further on in the same list) into LDS.
// TF_PREFILL (chunked-prefill plans): a QKV task makes its pool writes visible
// before its tagged words; an attention task of chunk row b first waits for
// rows 0 .. b-1's K and V words and then reads the pool.
// TF_FOLD (batch-1 MoE): router tasks form the logits before the RMSNorm
// scale from x and o (W_r (g x) + (W_r diag(g) W_o) o); expert tasks apply it.
// TF_SHARE (batch MoE): the expert task is share aux of a1 of the layer's
// expert work over the experts the routing chose (rows assigned on device).
// TF_REDUCE (batch O projection split over a3 > 1 reduction blocks): the
// task adds the a3 blocks' partial sums of rows a1 .. a1 + a2 and the
// residual; without it, a task of block a0 publishes the partial sums of
// rows a1 .. a1 + a2 (its tile).
enum TaskFlags : uint8_t { TF_WRITE_TOPK = 1, TF_QUEUE = 2, TF_STAGE_KV = 4, TF_LOGITS = 8, TF_PREFILL = 16,
                           TF_FOLD = 32, TF_SHARE = 64, TF_REDUCE = 128 };

// Batch QKV tasks: rotary pairs per row block (the rows of a block are 2
// BQKV_PAIRS), and the words per (reduction block, row block, sequence) of
// a partial QKV projection: the rows, the sum of squares, a pad word.
constexpr int BQKV_PAIRS = 32;
constexpr int QPART_STRIDE = 2 * BQKV_PAIRS + 2;

// Words (floats) a batch combine task may gather: the whole shared area.
constexpr int COMB_BATCH_WORDS = 24576;

// Attention pages staged ahead of their split: the split's first twelve
// pages (wave w takes pages w and w + 8), 96 KB at a head dim of 128.
constexpr int STAGE_PAGES = 12;
constexpr int STAGE_SCAN = 8;
constexpr int MAX_SHARE_EXPERTS = 256;  // experts a shared expert task can list

// Pages per attention split when long contexts use the shared split queue.
constexpr int QUEUE_PAGES = 64;

constexpr uint16_t NO_CTR = 0xFFFF;

// wait_a / wait_b name the producer classes (completion counters) a task
// depends on (wait_a: the routing decision, wait_b: the data); the device
// waits on the tagged data itself (see tag_word), so these name the
// dependency for the validator and the simulator. signal is the completion
// counter the task adds `units` to when it finishes: the number of outputs it
// produced (rows, pages, elements or sequences of its operation), so that a
// counter grows by its class's whole work per step whatever the tiling.
// Tasks that produce only partial sums of another task's outputs signal no
// counter. rsv is zero.
struct Task {
  uint8_t op, flags;
  uint16_t layer;
  uint16_t wait_a, wait_b;
  uint16_t units, rsv;
  uint16_t signal;
  uint16_t aux;
  int32_t a0, a1, a2, a3;
};
static_assert(sizeof(Task) == 32, "task record is 32 bytes");

// Plan image: u32 header[PLAN_HDR_WORDS], u32 cu_off[n_cu + 1] (task index
// ranges per list), padding to 32 B, Task tasks[n_tasks] (lists back to back).
// After the tasks: int32 seq_bound[B], each sequence's context bound.
// Then (queue plans) Task splits[H_NSPLITS]: the attention splits that queue
// tasks pull (op OP_ATTN, a0 = b, a1 = g, a2 = first page, a3 = pages, aux
// = split index; the layer is the queue task's), longest first.
constexpr uint32_t PLAN_MAGIC = 0x35504B4Du;  // "MKP5"
constexpr int PLAN_HDR_WORDS = 16;
enum PlanHdr { H_MAGIC = 0, H_NCU = 1, H_NTASKS = 2, H_NCTR = 3, H_TASK_OFF_BYTES = 4,
               H_STAGES = 5, H_BOUND_OFF_BYTES = 6, H_BATCH = 7, H_SPLIT_OFF_BYTES = 8, H_NSPLITS = 9 };

// Batch projections: MFMA 16x16x32 bf16 tiles of 16 weight rows x 16 or 32
// sequences. The sequences' inputs stream through LDS in panels of MT_KP
// elements (bf16 hi and lo parts of every element), and a task holds at most
// MT_MAX_BLOCKS row blocks. The reduction width must be a multiple of MT_KP.
constexpr int MAX_BATCH = 32;
constexpr int MT_KP = 256;
constexpr int MT_MAX_BLOCKS = 8;
// Expert tasks of a batch take the sequences routed to them in groups of
// EXP_GROUP (their inputs are held in LDS together).
constexpr int EXP_GROUP = 8;
// Floats of the LDS gather vector of the megakernel.
MK_HD constexpr int dev_lds_vec() { return 8192; }

// Completion counters: counter c is CTR_LINES sub-counters, one 64-byte line
// each; a task on compute unit cu increments sub-counter cu % CTR_LINES.
constexpr int CTR_LINES = 8;
constexpr int CTR_STRIDE = 16;  // u32 words per line
constexpr int NT = 512;         // threads per workgroup (8 wave64)
constexpr int NWAVE = NT / 64;

// Per-task trace record (u64 words, constant 100 MHz clock): task start,
// routing wait begin/end, data wait begin/end (0 where the task has no such
// wait), body end, task end, (cu << 32 | op << 16 | layer), then 8 marks a
// task body may set at points of its own (0 = unset).
constexpr int TRACE_WORDS = 16;
constexpr int TRACE_MARKS = 8;

// Status words written by the device on failure.
enum DevStatus : uint32_t { DS_OK = 0, DS_TIMEOUT = 1, DS_BOUNDS = 2 };

// Tagged word: every activation passed between tasks is a 64-bit word
// (epoch << 32 | fp32 bits) written with one device-coherent store. A
// consumer spins on the word until its tag equals the current step's epoch:
// the tag is the word's own completion counter, so the value and its
// readiness arrive in the same access. Buffers start zeroed and epochs start
// at 1, so a stale word never carries the current tag.
MK_HD inline uint64_t tag_word(float v, uint32_t epoch) {
  union { float f; uint32_t u; } c;
  c.f = v;
  return ((uint64_t)epoch << 32) | c.u;
}

// GEMV mapping of a reduction width K (bf16 elements): a lane group of TC
// lanes (64 or 32) covers a row as K/8 16-byte chunks, CPL chunks per lane.
MK_HD inline bool gemv_map(int K, int* tc, int* cpl) {
  if (K <= 0 || K % 8) return false;
  const int chunks = K / 8;
  int t = 0;
  if (chunks % 64 == 0) t = 64;
  else if (chunks % 32 == 0) t = 32;
  else return false;
  const int c = chunks / t;
  if (!(c == 1 || c == 2 || c == 3 || c == 4 || c == 6 || c == 8)) return false;
  *tc = t;
  *cpl = c;
  return true;
}
// Lane groups of a workgroup for lane-group width tc.
MK_HD inline int gemv_groups(int tc) { return NWAVE * (64 / tc); }
// Most 16-byte chunks a lane may hold for a prefetched GEMV tile.
constexpr int GEMV_REG_CHUNKS = 28;
constexpr int GEMV_RPW_MAX = 8;   // rows per lane group of a prefetched tile

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

// Element offsets of K[s][dim] and V[s][dim] of one token slot s within a
// page block of one (page, layer, kv head) (2 x 16 x D bf16): the order in
// which the attention MFMA operands are loaded, so that every 64-lane load
// is one contiguous kilobyte. K chunk i of lane (s, kq) holds dims
// 32 i + 8 kq .. + 7 of slot s; V chunk m of lane (r, kq) holds slots
// 4 kq .. + 3 of dims 32 m + r and 32 m + 16 + r.
MK_HD inline int kv_k_offset(int s, int dim) {
  return (((dim >> 5) * 4 + ((dim & 31) >> 3)) * 16 + s) * 8 + (dim & 7);
}
MK_HD inline int kv_v_offset(int s, int dim, int D) {
  return 16 * D + (((dim >> 5) * 4 + (s >> 2)) * 16 + (dim & 15)) * 8 + ((dim & 31) >> 4) * 4 + (s & 3);
}

// Kernel variants: the megakernel is compiled once per shape class, given by
// the GEMV mappings (lane-group width, 16-byte chunks per lane) of the
// hidden size, the attention output (query heads x head dim) and the FFN
// width, and the head dim. Returns the class index, or -1 when no variant is
// compiled for the shape.
MK_HD inline int kernel_class(int hidden, int attn_out, int ffn, int head_dim) {
  int th, ch, to, co, tf, cf;
  if (!gemv_map(hidden, &th, &ch) || !gemv_map(attn_out, &to, &co) || !gemv_map(ffn, &tf, &cf))
    return -1;
  if (th == 32 && ch == 1 && to == 32 && co == 1 && tf == 64 && cf == 1 && head_dim == 64) return 0;
  if (th == 64 && ch == 2 && to == 64 && co == 2 && tf == 64 && cf == 1 && head_dim == 64) return 1;
  if (th == 64 && ch == 4 && to == 64 && co == 8 && tf == 32 && cf == 3 && head_dim == 128) return 2;
  return -1;
}

// LM-head tiles stream their rows in batches of LM_BATCH rows per lane group.
constexpr int LM_BATCH = 2;
// Batches of an LM-head tile in flight together (a ring of registers).
constexpr int LM_RING = 3;

struct KArgs {
  // shape
  int32_t L, H, Hq, Hkv, D, HG, F, E, K, V, B, max_pages, dense, norm_topk;
  float eps, attn_scale;
  // weights (bf16)
  const uint16_t *embed, *attn_norm, *wqkv, *wo, *ffn_norm, *router, *gate, *up, *down,
      *final_norm, *lm;
  const float* rfold;  // [L][E][Hq D] W_r diag(g) W_o (folded router), or NULL
  const uint16_t* etile;  // batch expert weights in MFMA tile order (mk_expert_tile), or NULL
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
  // tagged activation buffers and their per-layer strides (words):
  //  x [L][B][H] layer outputs, xa [L][B][H] after attention, q [L][B][Hq][D],
  //  kvn [L][B][Hkv][2][D] new K and V (bf16 bits), part [L][B][Hkv][S_max][HG][D+2]
  //  split partials (o, m, l), o [L][B][Hq][D], rlog [L][B][E], act [L][B][K][F],
  //  lmpart [n_lm][B][2] (value, index)
  //  batch only: route [L][B][K][2] (expert id bits, weight) per selected slot,
  //  y [L][B][K][H] expert outputs
  uint64_t *x, *xa, *q, *kvn, *part, *o, *rlog, *act, *lmpart, *route, *y, *opart, *qpart;
  uint64_t* lw;  // logit words [B][V] (written by sampling steps only)
  // sampling (device [B] arrays; smp_u == NULL: greedy for every sequence)
  const float *smp_t, *smp_p, *smp_minp, *smp_u;
  const int32_t* smp_k;
  const uint64_t* ws;  // the workspace holding all of them (256-byte aligned)
  uint32_t ws_bytes;   // its size (under 4 GiB)
  int64_t s_x, s_q, s_kvn, s_part, s_o, s_rlog, s_act, s_route, s_y, s_opart, s_qpart;
  const int32_t* seq_bound;  // [B] context bound per sequence (in the plan image)
  int32_t S_max, n_lm;
  // plan and sync
  const uint32_t* plan;
  uint32_t* ctr;
  uint32_t* status;
  uint32_t epoch;
  uint64_t timeout_ticks;  // of the 100 MHz constant clock
  uint64_t* trace;         // NULL, or TRACE_WORDS per task
};

}  // namespace mk
