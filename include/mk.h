/* mk.h -- C ABI of a persistent decode megakernel for MI355X (gfx950).
 *
 * One decode step of a decoder-only LLM over a paged KV cache runs as ONE
 * persistent kernel: one workgroup per compute unit, each walking its own
 * host-built task list in device memory, each task one tile of one
 * operation; dependencies are counters in device memory that a task
 * increments when it finishes and that its consumers spin on before they
 * read (megakernel page, "Inside the megakernel serving engine for North
 * Mini Code", section "What is a Megakernel?" and the caption of Image 2).
 *
 * Conventions
 *  - Ownership: the library never allocates device memory. The caller owns
 *    every device buffer (sizes come from mk_plan_*_bytes). Plans and pools
 *    are host objects owned by the library and freed with *_free.
 *  - Errors: every call returns an mk_status; on failure mk_last_error()
 *    gives a message for the calling thread (Kinetic book, "Python, C and
 *    Rust": NULL or -1 on failure plus a per-thread last-error string).
 *    Calls validate before they launch; a batch, context or page outside a
 *    plan's declared bounds is MK_EBOUNDS (kern page, "The manifest": a call
 *    outside declared bounds is rejected before it launches).
 *  - Asynchrony: mk_decode_step only enqueues work on the caller's HIP
 *    stream. Device-side failures (a dependency wait that exceeded its
 *    deadline, a context past the plan's bound) are written to the status
 *    words, which the caller reads after its next synchronisation and
 *    decodes with mk_step_status.
 *  - Threads: a plan is immutable except through mk_plan_update and may be
 *    used from several threads; a pool is single-threaded.
 *  - Determinism: the same inputs give the same plan bytes and the same
 *    output bits (kern page, "The harness": running twice and diffing is a
 *    test).
 *
 * Data formats (all device pointers unless stated otherwise)
 *  - Weights: bf16, logical row-major [out][in] matrices, stacked over
 *    layers (and experts) as documented in mk_weights.
 *  - Activations between tasks: fp32, in the caller's workspace.
 *  - KV pool: bf16 pages of page_tokens (= 16) tokens holding every layer.
 *    For physical page p, layer l, kv head g, the block of 2*16*d elements
 *    starting at element p*page_stride + l*layer_stride + g*(2*16*d) holds
 *    K (16*d elements) then V (16*d elements), where layer_stride =
 *    Hkv*2*16*d and page_stride = L*layer_stride. Token t of sequence b is
 *    in page page_table[b][t/16], slot s = t%16. Within the block, in the
 *    order the attention MFMA operands are read (each 64 consecutive
 *    16-byte chunks are one 64-lane load):
 *      K[s][dim]: element ((dim/32*4 + dim%32/8)*16 + s)*8 + dim%8
 *      V[s][dim]: element 16*d + ((dim/32*4 + s/4)*16 + dim%16)*8
 *                 + (dim%32/16)*4 + s%4
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_ABI_VERSION 2

typedef enum mk_status {
  MK_OK = 0,
  MK_EINVAL = -1,       /* bad argument, NULL pointer, inconsistent sizes */
  MK_ENOMEM = -2,       /* pool exhausted; pool state unchanged */
  MK_EBOUNDS = -3,      /* batch / context / page outside the plan's bounds */
  MK_EDEVICE = -4,      /* a HIP runtime call failed */
  MK_ETIMEOUT = -5,     /* a device dependency wait passed its deadline */
  MK_ESTATE = -6,       /* object in the wrong state (e.g. sequence not leased) */
  MK_EUNSUPPORTED = -7  /* shape outside what the kernels implement */
} mk_status;

/* Model shape. Dense FFN if n_experts == 0 (uses ffn_dim), MoE otherwise. */
typedef struct mk_model_desc {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim;
  int32_t ffn_dim;                       /* dense SwiGLU width; 0 for MoE */
  int32_t n_experts, top_k, expert_ffn;  /* MoE; 0 for dense */
  int32_t norm_topk;                     /* 1: renormalise the top-k softmax weights */
  int32_t vocab, page_tokens;            /* page_tokens must be 16 */
  float rms_eps, rope_theta;
} mk_model_desc;

/* One step's batch. Host pointers; copied by mk_plan. */
typedef struct mk_batch_desc {
  int32_t batch;
  int32_t max_pages;           /* columns of the page table */
  const int32_t* seq_lens;     /* [batch] tokens already cached (= position of the new token) */
  const int32_t* page_table;   /* [batch][max_pages] physical page ids, -1 = none */
  int32_t max_ctx_bound;       /* the plan stays valid while every seq_len + 1 <= bound;
                                  every sequence must have ceil(bound/16) pages mapped */
  const int32_t* ctx_bounds;   /* [batch] per-sequence bounds (<= max_ctx_bound; sequence b
                                  needs ceil(ctx_bounds[b]/16) pages mapped), or NULL: every
                                  sequence uses max_ctx_bound. Attention work is split by
                                  these bounds, so ragged batches plan only live pages. */
} mk_batch_desc;

typedef struct mk_plan_opts {
  int32_t n_cu;                /* workgroups = task lists (0: the current device's CU count) */
  int32_t attn_split_pages;    /* pages per attention task (0: automatic) */
  int32_t flags;               /* MK_PLAN_* bits, 0 = defaults */
} mk_plan_opts;
/* Attention splits from a shared queue that every compute unit pulls from
 * (megakernel page, caption of Image 2: attention work whose amount depends
 * on live sequence lengths sits in queues any processor can take from),
 * instead of one static split per task: one queue task per unit and layer
 * pulls splits, longest first, from a table in the plan image (batch 1:
 * splits of 64 pages; a batch: the splits the static plan would deal).
 * Decode plans only (not MK_PLAN_PREFILL). Off unless asked for. */
#define MK_PLAN_ATTN_QUEUE 1     /* use the queue */
#define MK_PLAN_NO_ATTN_QUEUE 2  /* never use it */
/* Chunked prefill: the batch rows are 2 .. 32 consecutive prompt tokens of
 * ONE sequence (every page-table row the same, seq_lens[i] = seq_lens[0] + i,
 * tokens_in the chunk's tokens in order), run as one step of the batch path:
 * MFMA tiles over the chunk's rows write their K and V into the shared pages
 * (row i at position seq_lens[0] + i) and row i attends to the tokens before
 * it, the chunk's earlier rows included -- each row's result is the decode
 * step of its token, so the chunk equals its tokens decoded one by one. The
 * last row's next token continues the sequence; afterwards its length is
 * seq_lens[0] + chunk (each row's own seq_lens entry grows by one). */
#define MK_PLAN_PREFILL 4
/* Batch-1 MoE plans compute the router logits beside the O projection:
 * since the router reads RMSNorm(x + W_o o), its logits before the norm's
 * 1/rms scale are [W_r diag(g) | W_r diag(g) W_o] [x | o], which needs only
 * the layer input x and the attention output o; the expert tasks apply the
 * scale, which they compute anyway. The folded matrix is made once by
 * mk_router_fold. This flag keeps the router as its own stage after O. */
#define MK_PLAN_NO_ROUTER_FOLD 8
/* Batch MoE plans share the layer's expert work by live routing: every
 * expert task reads the routing (which it needs anyway), lists the experts
 * at least one sequence was routed to, and takes an equal share of their
 * gate/up rows and of their down rows (the megakernel page, caption of Image
 * 2: MoE work whose amount depends on the routing goes where processors are
 * free), so no unit idles on an expert nobody chose. This flag keeps one
 * fixed (expert, part) per task. */
#define MK_PLAN_NO_EXPERT_SHARE 16

typedef struct mk_plan mk_plan_t;   /* opaque host object */
typedef struct mk_pool mk_pool_t;   /* opaque host object */

/* Device pointers to bf16 weights (logical row-major layouts). */
typedef struct mk_weights {
  const void* embed;       /* [vocab][hidden] */
  const void* attn_norm;   /* [L][hidden] */
  const void* w_qkv;       /* [L][(Hq + 2 Hkv) d][hidden]: rows q (head-major), k, v */
  const void* w_o;         /* [L][hidden][Hq d] */
  const void* ffn_norm;    /* [L][hidden] */
  const void* router;      /* [L][E][hidden] (MoE) or NULL */
  const void* gate;        /* [L][E][F][hidden] (MoE) or [L][ffn][hidden] */
  const void* up;          /* same shape as gate */
  const void* down;        /* [L][E][hidden][F] (MoE) or [L][hidden][ffn] */
  const void* final_norm;  /* [hidden] */
  const void* lm_head;     /* [vocab][hidden] (untied) */
  const float* router_fold; /* fp32 [L][E][hidden + Hq d]: per layer and expert the row
                               [W_r diag(ffn_norm) | W_r diag(ffn_norm) W_o], made by
                               mk_router_fold from the weights above; read by batch-1 MoE plans
                               (unless MK_PLAN_NO_ROUTER_FOLD), NULL otherwise */
  const void* expert_tiles; /* bf16 [L][E][3 F hidden] (dense FFN: E = 1, F = ffn): the gate, up
                               and down rows in MFMA tile order, made by mk_expert_tile; read by
                               batch plans' expert tasks when not NULL (else they read gate, up
                               and down), 16-byte aligned */
} mk_weights;

/* KV cache and positions. */
typedef struct mk_kv {
  void* pool;                /* bf16 KV pool, format above */
  int64_t n_pages;           /* pages in the pool */
  const int32_t* page_table; /* device [batch][max_pages] (same shape as the plan's) */
  int32_t* seq_lens;         /* device [batch]; incremented by one when the step completes */
  const float* rope_cos;     /* device [n_rope_pos][head_dim/2] (see mk_rope_table) */
  const float* rope_sin;     /* device [n_rope_pos][head_dim/2] */
  int32_t n_rope_pos;        /* positions covered by the tables (>= max_ctx_bound) */
} mk_kv;

/* Sampling of the next token beyond greedy, per sequence, in the step's last
 * stage (the Kinetic book, "Pick the sampling" and the sampler flags: the
 * llama.cpp samplers and their default order -- top-k, top-p, min-p, then
 * temperature -- and temperature 0 always takes the likeliest token). Every
 * array is device [batch], read when the step's last stage runs:
 *   temperature  <= 0: greedy (as with no sampling); else the logits of the
 *                kept candidates are divided by it before the draw;
 *   top_k        candidates: the top_k largest logits (ties to the lower
 *                id); values <= 0 ("all") or above MK_SAMPLE_TOP_K_MAX are
 *                served as MK_SAMPLE_TOP_K_MAX (the device keeps at most that
 *                many candidates);
 *   top_p        keep the shortest run of candidates, most likely first,
 *                whose probabilities (softmax over the candidates at
 *                temperature 1) add up to at least top_p; >= 1: off;
 *   min_p        keep candidates at least min_p times as likely as the best;
 *                <= 0: off;
 *   uniform      one draw u in [0, 1) per sequence and step, supplied by the
 *                caller (so that a seeded run repeats): the token is the
 *                first kept candidate, most likely first, at which the
 *                running sum of exp((z - z_max) / temperature) exceeds u
 *                times its total. */
#define MK_SAMPLE_TOP_K_MAX 64
typedef struct mk_sampling {
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  const float* min_p;
  const float* uniform;
} mk_sampling;

/* Per-step inputs and outputs. */
typedef struct mk_io {
  const int32_t* tokens_in;  /* device [batch] */
  int32_t* tokens_out;       /* device [batch] next tokens (greedy, or sampled); may alias nothing else */
  int32_t* topk_ids;         /* device [L][batch][top_k] or NULL */
  float* topk_w;             /* device [L][batch][top_k] or NULL */
  float* logits;             /* device [batch][vocab] or NULL */
  const mk_sampling* sampling; /* host struct of device arrays, or NULL: greedy for every sequence */
} mk_io;

/* Caller-owned device buffers of a plan. */
typedef struct mk_step_buffers {
  const void* plan; size_t plan_bytes;      /* image uploaded by mk_plan_upload */
  void* workspace; size_t workspace_bytes;  /* tagged activations: zero-filled before the
                                               first step; thereafter every step on this
                                               workspace uses a larger epoch */
  uint32_t* counters; size_t counter_bytes; /* completion counters, 8 sub-counters of one
                                               64-byte line each per counter, zero-filled
                                               before the first step; every finished task adds
                                               the number of outputs it produced, so each step
                                               adds the counter's target to the sum of its
                                               lines (modulo 2^32) */
  uint32_t* status;                         /* 4 words, zeroed once */
  uint64_t* trace; size_t trace_bytes;      /* NULL (no tracing), or 16 u64 per task
                                               (128 * mk_plan_n_tasks bytes), indexed by
                                               the task's position in the plan image:
                                               start, routing-wait begin/end, data-wait
                                               begin/end (0 = no such wait), body end,
                                               task end (ticks of the 100 MHz constant
                                               clock), cu << 32 | op << 16 | layer, then
                                               8 marks set inside the task body */
} mk_step_buffers;

/* ---- library ---- */
int32_t mk_abi_version(void);
const char* mk_last_error(void);
/* Compute units of the current HIP device. */
mk_status mk_device_cu_count(int32_t* n_cu);
/* Device-to-device copy of `bytes` (a multiple of 16; both pointers 16-byte
 * aligned) with 16-byte non-temporal loads and stores, enqueued on `stream`.
 * A bandwidth probe and the known-size kernel that calibrates hardware byte
 * counters; dst and src must not overlap. MK_EINVAL on a bad size/alignment. */
mk_status mk_stream_copy(void* dst, const void* src, size_t bytes, void* stream);

/* ---- model-level helpers (host only) ---- */
/* Rotary tables: angle(p, i) = p * theta^(-2i/d) for p < n_pos, i < d/2, computed
 * in fp64 and rounded to fp32. Host outputs of n_pos*d/2 floats each. */
mk_status mk_rope_table(float theta, int32_t head_dim, int32_t n_pos, float* cos_out,
                        float* sin_out);
/* The folded router (fp32 [L][E][hidden + Hq d], device): row (l, e) is
 * out[h] = W_r[l][e][h] * ffn_norm[l][h] for h < hidden, then
 * out[hidden + j] = sum_h W_r[l][e][h] * ffn_norm[l][h] * W_o[l][h][j], from
 * w->router, w->ffn_norm and w->w_o; enqueued on hip_stream. Needed once per
 * set of weights by batch-1 MoE plans (see MK_PLAN_NO_ROUTER_FOLD): each term
 * is a product of bf16 values, exact in fp32, summed in fp32. MK_EINVAL for a
 * dense model or a missing pointer; MK_EUNSUPPORTED if hidden + Hq d is not a
 * multiple of 4 or exceeds 8192. */
mk_status mk_router_fold(const mk_model_desc* m, const mk_weights* w, float* out, void* hip_stream);

/* Expert weights in MFMA tile order, for the batch path's expert GEMMs (the
 * article's point that a decode step is bound by streaming the weights from
 * HBM, "Inside the megakernel serving engine for North Mini Code",
 * introduction: the batch GEMMs read their A operand 16 rows x 32 columns at
 * a time, and row-major rows give each wave load 16 runs of 64 bytes; the
 * tile order gives it one contiguous kilobyte). Fills out (device, 16-byte
 * aligned, L x E x 3 F x hidden bf16, E = 1 and F = ffn for a dense FFN)
 * from w->gate, w->up and w->down, enqueued on hip_stream: per layer and
 * expert the gate/up rows interleaved (row 2f = gate row f, 2f + 1 = up row
 * f) in 2F/16 blocks of 16 rows, then the down rows in hidden/16 blocks;
 * block rb's k-step s (columns 32 s .. 32 s + 31) is 64 x 16 bytes, entry t
 * holding row 16 rb + t % 16, columns 32 s + 8 (t / 16) .. + 7. The caller
 * owns out and passes it as mk_weights.expert_tiles. Errors: MK_EINVAL (NULL
 * or misaligned pointers, bad shape), MK_EUNSUPPORTED (hidden or FFN width
 * not a multiple of 32), MK_EDEVICE (launch failure). */
mk_status mk_expert_tile(const mk_model_desc* m, const mk_weights* w, void* out, void* hip_stream);
/* Elements (bf16) of a KV pool of n_pages pages. */
int64_t mk_kv_pool_elems(const mk_model_desc* m, int64_t n_pages);
/* Algorithmic bytes of one step: weights read once (selected experts only:
 * distinct_experts[l] per layer, or NULL for min(E, batch*top_k)), one embedding
 * row per sequence, KV read (every cached token incl. the new one) and written. */
mk_status mk_step_bytes(const mk_model_desc* m, int32_t batch, const int32_t* seq_lens,
                        const int32_t* distinct_experts, double* weight_bytes,
                        double* kv_read_bytes, double* kv_write_bytes);

/* ---- plan (host; no device is touched except by mk_plan_upload) ---- */
/* Build the task lists, counters and workspace layout for one batch shape
 * (megakernel page, caption of Image 2: the host decomposes the step into
 * tasks of one tile of one operation each and deals them round-robin over
 * the compute units). Batch 1 runs GEMV tiles; a batch of 2 .. 32 sequences
 * (continuous batching with ragged contexts, megakernel page, "Inside the
 * megakernel serving engine": continuous batching over a paged cache) runs
 * every projection as MFMA tiles over all sequences, a top-k task per
 * sequence and expert tasks that pick up the sequences routed to them. */
mk_status mk_plan(const mk_model_desc* m, const mk_batch_desc* b, const mk_plan_opts* o,
                  mk_plan_t** out);
/* Refresh a plan for the next steps of the same batch (same size, page-table
 * width, model and options): new sequence lengths and page table (host; e.g.
 * after the pool mapped a sequence's next page at a 16-token boundary, or a
 * sequence was replaced in its batch slot) and new context bounds, with the
 * same meaning as in mk_batch_desc. The plan is rebuilt in place and is then
 * byte-identical to mk_plan of the same arguments. *changed (may be NULL)
 * receives MK_PLAN_CHANGED_* bits: IMAGE -- the device image changed:
 * upload it again before the next step; WORKSPACE -- the workspace layout
 * changed; COUNTERS -- the counters or their targets changed. After either
 * of the last two, start again as after mk_plan: a zero-filled workspace of
 * mk_plan_workspace_bytes, zeroed counters, epochs from 1
 * (mk_decode_step_static does this by itself). The device page table and
 * sequence lengths are the caller's buffers: copy the new values there.
 * On failure (e.g. MK_EBOUNDS for a length past its bound) the plan is left
 * as it was. A plan may not be updated while a step that uses it runs. */
#define MK_PLAN_CHANGED_IMAGE 1
#define MK_PLAN_CHANGED_WORKSPACE 2
#define MK_PLAN_CHANGED_COUNTERS 4
mk_status mk_plan_update(mk_plan_t* p, const int32_t* seq_lens, const int32_t* page_table,
                         int32_t max_ctx_bound, const int32_t* ctx_bounds, int32_t* changed);
/* Coverage (every output row / KV page exactly once), counter targets equal
 * the outputs of the tasks that signal them, per-list stage order, waits on
 * earlier stages only. MK_OK or MK_EINVAL with a message. */
mk_status mk_plan_validate(const mk_plan_t* p);
/* Execute the lists on n_cu virtual compute units under seeded random
 * interleavings, n_runs times, each unit in list order and each task
 * starting only once every producer of the data it reads has finished (the
 * waits the device performs, taken per producer class); fails (MK_ESTATE) on
 * a deadlock (message names the blocked tasks) or a counter that does not
 * end at epoch x target. */
mk_status mk_plan_simulate(const mk_plan_t* p, uint64_t seed, int32_t n_runs);
size_t mk_plan_device_bytes(const mk_plan_t* p);
size_t mk_plan_workspace_bytes(const mk_plan_t* p);
size_t mk_plan_counter_bytes(const mk_plan_t* p);
int32_t mk_plan_n_tasks(const mk_plan_t* p);
int32_t mk_plan_n_counters(const mk_plan_t* p);
int32_t mk_plan_n_cu(const mk_plan_t* p);
/* The device image (the bytes mk_plan_upload copies) into a host buffer. */
mk_status mk_plan_export(const mk_plan_t* p, void* host_buf, size_t bytes);
mk_status mk_plan_upload(const mk_plan_t* p, void* d_plan, size_t bytes, void* hip_stream);
/* Workspace sub-buffer `which` (MK_BUF_*) of layer `layer` (ignored for
 * MK_BUF_LMPART and MK_BUF_LOGIT): byte offset and size. Every workspace
 * buffer holds tagged words: u64 = (epoch << 32) | fp32 bits of the value,
 * written by the step of that epoch (KVN holds bf16 bits in the low 16 bits
 * of the value; LMPART holds (value, index) pairs per LM-head tile; LOGIT
 * [B][vocab] the logits, written only by steps that sample). Per layer:
 *   XATTN [B][H] hidden after the attention residual, XFFN [B][H] layer output,
 *   Q [B][Hq][d] rotated queries, KVN [B][Hkv][2][d] the new token's K and V,
 *   PART [B][Hkv][splits][Hq/Hkv][d+2] attention split partials (o, max, sum),
 *   O [B][Hq][d] combined attention, RLOG [B][E] router logits (batch-1 MoE
 *   plans that fold the router: before the RMSNorm's 1/rms scale),
 *   ACT [B][top_k][F] SwiGLU activations;
 * batch plans only (0 bytes at batch 1):
 *   ROUTE [B][top_k][2] selected expert id (int bits) and weight per slot,
 *   Y [B][top_k][H] each selected expert's down-projection output,
 *   OPART [kb][B][H] partial O projections over reduction blocks 0 .. kb-1
 *   (the O projection is split over kb > 1 blocks of the attention output;
 *   0 bytes when kb = 1),
 *   QPART [qkb - 1][row blocks][B][rows + 2] partial QKV projections over
 *   reduction blocks 1 .. qkb-1 of the hidden state, per row block of the
 *   QKV tasks: the block's rows, then the block's sum of squares of the
 *   hidden state (for the RMSNorm), then a zero pad word. */
enum { MK_BUF_XATTN = 0, MK_BUF_XFFN = 1, MK_BUF_Q = 2, MK_BUF_PART = 3, MK_BUF_O = 4,
       MK_BUF_RLOG = 5, MK_BUF_ACT = 6, MK_BUF_LMPART = 7, MK_BUF_KVN = 8,
       MK_BUF_ROUTE = 9, MK_BUF_Y = 10, MK_BUF_OPART = 11, MK_BUF_QPART = 12,
       MK_BUF_LOGIT = 13 };
mk_status mk_plan_buffer(const mk_plan_t* p, int32_t which, int32_t layer, size_t* offset,
                         size_t* bytes);
/* The plan's per-step counter targets, [n_counters] (host): for each
 * completion counter, the outputs its class produces in one step -- QKV rows
 * of a kv group, (sequence, page) pairs of a kv head's attention, combined
 * attention elements, O rows, router rows, selected sequences (batch top-k),
 * expert gate/up outputs plus down rows, expert-combine rows (batch), LM-head
 * rows. An attention queue's head counter (batch 1 with MK_PLAN_ATTN_QUEUE)
 * instead gains one per split taken plus one per queue task. */
mk_status mk_plan_counter_targets(const mk_plan_t* p, uint32_t* out, int32_t n);
/* Name of counter i: "<class>[<layer>]" or "<class>[<layer>][<kv head>]"
 * (classes qkv, attn, comb, o, router, topk, expert, ffn, queue) or "lm";
 * the string lives as long as the plan. NULL (and mk_last_error) if i is out
 * of range. */
const char* mk_plan_counter_name(const mk_plan_t* p, int32_t i);
void mk_plan_free(mk_plan_t* p);

/* ---- one decode step (asynchronous on hip_stream) ----
 * epoch: the tag of this step's activations; >= 1 and larger than every epoch
 * used before on the same workspace since it was zero-filled (steps on one
 * workspace run in stream order; a step never reads a word of another epoch).
 * tokens_in -> tokens_out: greedy argmax of the LM head (ties to the lower id).
 * On completion every seq_lens[b] has grown by one: the new token's K and V
 * sit at position seq_lens[b] (old value) of its sequence. timeout_ms bounds
 * every dependency wait (0: 2000 ms); on expiry the kernel records
 * MK_ETIMEOUT in the status words and every workgroup exits. After a failed
 * step the outputs, the new token's K/V slots and the counters are
 * undefined and a sequence's length may or may not have advanced: zero the
 * status words and the counters, restore seq_lens and run the step again
 * with a larger epoch (a plan with the attention queue: start again as after
 * mk_plan, from a zero-filled workspace and epoch 1). */
mk_status mk_decode_step(const mk_plan_t* p, const mk_weights* w, const mk_kv* kv,
                         const mk_io* io, const mk_step_buffers* bufs, uint32_t epoch,
                         uint32_t timeout_ms, void* hip_stream);
/* ---- one decode step that allocates nothing (asynchronous on hip_stream) ----
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as mk_decode_step, with the plan's workspace and completion counters
 * held in a static scratch array of the library (MK_STATIC_SCRATCH_BYTES per
 * device, taken when the library's kernels are first loaded on the device and
 * held until the process ends) instead of caller buffers. No allocation and
 * no allocating library call is made. The caller passes the inputs and
 * outputs: the plan image uploaded with mk_plan_upload (d_plan, plan_bytes),
 * the weights, the KV cache and io as for mk_decode_step, and 4 status words
 * (device, zeroed once; read and decoded as for mk_decode_step). The library
 * keeps the epochs: a plan other than the last one used on this device starts
 * from a zero-filled scratch (a fill kernel on hip_stream) and epoch 1, and
 * every further step of it uses the next epoch. Every call on one device
 * shares that device's scratch: calls that overlap on one device (other
 * streams, other threads) race and must be serialised by the caller; the
 * counters and tagged activations are not readable through this entry point.
 * After a failed step, zero the status words, restore seq_lens and call again
 * (the next epoch); a plan with the attention queue must be built again.
 * MK_EBOUNDS if the plan's workspace and counters exceed the scratch (large
 * batch plans: use mk_decode_step). */
#define MK_STATIC_SCRATCH_BYTES (128u << 20)
mk_status mk_decode_step_static(const mk_plan_t* p, const mk_weights* w, const mk_kv* kv,
                                const mk_io* io, const void* d_plan, size_t plan_bytes,
                                uint32_t* d_status, uint32_t timeout_ms, void* hip_stream);
/* Decode a host copy of the 4 status words: MK_OK, MK_ETIMEOUT (word 1: the
 * index of the task that waited, in the plan's task order; words 2 and 3:
 * what it waited for -- word 3 = 0xFFFFFFFD: a gather of tagged word pairs,
 * word 2 the first stale pair of the thread that gave up; 0xFFFFFFFE: a
 * batch activation panel, word 2 the sequence; otherwise word 2 is the
 * offset of the awaited word in its buffer and word 3 the tag it held) or
 * MK_EBOUNDS (word 1: the task; a token, position or page outside the plan
 * or pool). Sets mk_last_error. */
mk_status mk_step_status(const uint32_t* h_status);

/* ---- page/slot pool with prefix sharing (pure host; kern page, "The runtime") ----
 * n_pages pages of page_tokens tokens, n_slots sequence slots. The free list
 * starts in initial_order (a permutation of [0, n_pages); NULL = ascending).
 * A lease takes ceil(tokens/page_tokens) pages from the front of the free list
 * and the lowest free slot, all or nothing (MK_ENOMEM: nothing changed); a
 * release returns every page no one else holds to the back of the free list,
 * in the sequence's page order.
 * Prefix sharing: mk_pool_finish freezes a finished sequence's pages in place
 * as a checkpoint, keyed by the tokens whose K/V they hold, in a token radix
 * tree with one page per node (a run the tree already holds keeps its node;
 * the duplicate page is freed). mk_pool_lease_prefix finds the longest
 * checkpointed prefix of a prompt, at most n_prompt - 1 tokens (the last
 * prompt token always runs, giving the next token's logits): the sequence's
 * list starts with the checkpoint's whole pages inside the match, shared and
 * never written by anyone; if the match ends inside a page, the first fresh
 * page is that page's private copy -- the caller copies page *copy_src to
 * page *copy_dst in the device pool (whole pages are contiguous, see the KV
 * layout) before the sequence's next step writes it -- so every page has at
 * most one writer. Positions >= *matched must then be filled (prefilled or
 * decoded) by the caller. At each page the longest common run wins, ties to
 * the earlier checkpoint. Under pressure (a lease or extension that the free
 * list cannot serve) checkpoint pages that no sequence holds are evicted,
 * least recently used leaf first (ties: earlier inserted), all or nothing; an
 * evicted checkpoint is dropped (it is not parked in host memory). */
mk_status mk_pool_create(int32_t n_pages, int32_t page_tokens, int32_t n_slots,
                         const int32_t* initial_order, mk_pool_t** out);
mk_status mk_pool_lease(mk_pool_t* p, int64_t seq_id, int32_t worst_case_tokens,
                        int32_t* slot_out);
/* prompt: host [n_prompt] token ids; worst_case_tokens >= n_prompt (else
 * MK_EINVAL). Outputs (each may be NULL): slot, tokens reused (*matched),
 * and the page copy to make (-1, -1: none). */
mk_status mk_pool_lease_prefix(mk_pool_t* p, int64_t seq_id, const int32_t* prompt, int32_t n_prompt,
                               int32_t worst_case_tokens, int32_t* slot_out, int32_t* matched,
                               int32_t* copy_src, int32_t* copy_dst);
mk_status mk_pool_extend(mk_pool_t* p, int64_t seq_id, int32_t worst_case_tokens);
mk_status mk_pool_release(mk_pool_t* p, int64_t seq_id);
/* Freeze the pages holding the first n_tokens tokens of seq_id (tokens: host
 * [n_tokens], the ids whose K/V those pages hold, from position 0) as a
 * checkpoint, then release the sequence. MK_EBOUNDS if its pages hold fewer
 * tokens; MK_EINVAL if the tokens disagree with a checkpoint page the
 * sequence shares (nothing changed then). */
mk_status mk_pool_finish(mk_pool_t* p, int64_t seq_id, const int32_t* tokens, int32_t n_tokens);
/* out[i][j] = page j of seq_ids[i], -1 past its pages (host [n][max_pages]). */
mk_status mk_pool_page_table(const mk_pool_t* p, const int64_t* seq_ids, int32_t n,
                             int32_t max_pages, int32_t* out);
int32_t mk_pool_free_pages(const mk_pool_t* p);
/* Pages held by checkpoints. */
int32_t mk_pool_cached_pages(const mk_pool_t* p);
int32_t mk_pool_seq_pages(const mk_pool_t* p, int64_t seq_id);
void mk_pool_free(mk_pool_t* p);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
