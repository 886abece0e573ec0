/*
 * mk.h -- C ABI of the persistent decode megakernel library (libmk.so).
 *
 * One Llama-style decoder forward pass per generated token, run on an
 * MI355X (gfx950) as ONE persistent launch: one workgroup per compute unit,
 * each walking a host-built list of instructions and waiting on dependency
 * counters in global memory instead of kernel boundaries.  The megakernel
 * page ("2 . Definition et genealogie") defines the object in section 2.1
 * (single launch, persistence, fine dependencies in global memory, internal
 * dispatch of heterogeneous ops), states in section 2.5 that the host builds
 * the instruction lists the GPU consumes, and lists in section 2.6 the five
 * mechanisms this library implements: a grid sized for full residency,
 * opcode dispatch, dependency counters, a paged shared-memory allocator and
 * static scheduling.
 *
 * Conventions for every call:
 *   - Plain C types only.  `stream` arguments are hipStream_t values passed as
 *     void* (NULL = the legacy default stream).  "d_" pointers are device
 *     memory, everything else is host memory.
 *   - The library never allocates device memory.  All device buffers
 *     (weights, KV cache, workspace, logits, tokens, positions) belong to the
 *     caller and must outlive every call that was enqueued with them.
 *   - Device-touching calls enqueue work on `stream` and return without
 *     synchronising, except mk_get_device_error which synchronises `stream`.
 *   - Return value: MK_OK (0) or a negative MK_ERR_* code; mk_strerror turns
 *     it into text.  A failing call leaves its outputs untouched.
 *   - A plan or a context is used by one host thread at a time.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ error codes */
#define MK_OK 0
#define MK_ERR_INVALID_ARG (-1)   /* NULL pointer, out-of-range option */
#define MK_ERR_SHAPE (-2)         /* model shape the kernels do not support */
#define MK_ERR_ALIGN (-3)         /* a device pointer is not 16-byte aligned */
#define MK_ERR_NOT_RESIDENT (-4)  /* grid larger than the co-resident limit */
#define MK_ERR_CTX_OVERFLOW (-5)  /* batch > max_batch or workspace too small */
#define MK_ERR_HIP (-6)           /* a HIP runtime call failed */
#define MK_ERR_TIMEOUT (-7)       /* device watchdog: a dependency wait expired */
#define MK_ERR_INPUT (-8)         /* device saw a token or position out of range */
#define MK_ERR_PLAN (-9)          /* plan validation failed */
#define MK_ERR_STATE (-10)        /* context poisoned by a device error; reset it */
#define MK_ERR_UNSUPPORTED (-11)  /* option combination not built */
#define MK_ERR_SCRATCH (-12)      /* workspace larger than the static scratch */

/* ------------------------------------------------------------ model shape */
/* Standard Llama decoder, nn.Linear weight convention W[out][in], bf16.
 * Rotate-half RoPE pairs element i with i + head_dim/2; q head h reads kv head
 * h * n_kv_heads / n_q_heads.  Requirements: head_dim in {64, 128};
 * n_q_heads % n_kv_heads == 0; hidden, ffn and n_q_heads*head_dim multiples
 * of 256. */
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  double rms_eps;      /* RMSNorm epsilon, added inside the square root */
  double rope_theta;   /* RoPE base: angle(p, i) = p * theta^(-2i/head_dim) */
  int32_t tie_embeddings; /* 1: the LM head is the embedding matrix */
} mk_model_shape;

/* ------------------------------------------------------------ plan options */
enum { MK_SYNC_COUNTER = 0, /* one monotonic counter per event, atomic add */
       MK_SYNC_FLAG = 1,    /* one epoch flag per producer, plain stores */
       MK_SYNC_SENTINEL = 2 /* the data is the signal: activation words start as a
                               NaN sentinel pattern each step and consumers poll
                               the data itself (MK_EXEC_MEGA; MK_EXEC_FLAT with
                               max_batch 1) */ };
enum { MK_EXEC_MEGA = 0,    /* one persistent launch per decode step, loader /
                               sync-storer / compute wavefronts, LDS page ring */
       MK_EXEC_MULTI = 1,   /* the same role-specialised ops, one launch per
                               dependency level (kernel boundaries) */
       MK_EXEC_FLAT = 2,    /* one persistent launch with homogeneous waves: all
                               waves load, wait and compute each instruction */
       MK_EXEC_STREAM = 3,  /* one persistent launch, one sequence per step:
                               streamer waves keep projection weights in flight
                               across instructions, one wave synchronises
                               (MK_SYNC_COUNTER or MK_SYNC_FLAG, max_batch 1) */
       MK_EXEC_FLAT_MULTI = 4, /* MK_EXEC_FLAT's plan and ops, one launch per
                               dependency level with no waits: the multi-kernel
                               baseline of the homogeneous engine (also
                               capturable as a hipGraph, mk_graph_create) */
       MK_EXEC_QUEUE = 5    /* one persistent launch, homogeneous ops, no per-CU
                               lists: every workgroup takes the next instruction
                               of the plan's breadth-first queue from a global
                               atomic ticket (dynamic scheduling, megakernel page
                               sections 2.4 and 2.6 item 5; MK_SYNC_COUNTER or
                               MK_SYNC_FLAG) */ };

typedef struct {
  int32_t max_batch;   /* sequences per step: 1..16 (MK_EXEC_FLAT), 1 (MK_EXEC_STREAM),
                          1..4 otherwise */
  int32_t max_ctx;     /* KV slots per sequence */
  int32_t kv_splits;   /* attention splits per (sequence, kv head); 0 = auto */
  int32_t sync_mode;   /* MK_SYNC_* */
  int32_t exec_mode;   /* MK_EXEC_* */
  int32_t num_cus;     /* 0 = query the current device; >0 = plan for that many
                          (host-only planning, tests) */
  int32_t flags;       /* reserved, 0 */
} mk_plan_opts;

typedef struct mk_plan_s mk_plan_t; /* opaque, host memory, owned by the library */
typedef struct mk_ctx mk_ctx;   /* opaque, host memory, owned by the library */

/* Read-only description of a plan (for tests and tools). */
typedef struct {
  int32_t num_cus, n_instructions, n_levels, n_counters, kv_splits;
  int32_t max_instr_per_cu, block_threads, lds_bytes;
  int32_t sync_mode, exec_mode, max_batch, max_ctx;
  double weight_bytes;   /* bf16 parameter bytes one pass streams */
} mk_plan_info;

/* One instruction as the planner emitted it (for tests and tools). */
typedef struct {
  int32_t cu, slot;          /* executing workgroup and position in its list */
  int32_t op, layer, level;
  int32_t r0, r1;            /* GEMV: output rows [r0, r1); ATTN: seq, kv head */
  int32_t split, n_splits;   /* ATTN: key range split index / count */
  int32_t wait_event, wait_count; /* event it waits for (-1 none), triggers per step */
  int32_t signal_event;      /* event it triggers when done (-1 none) */
} mk_instr_desc;

enum { MK_OP_QKV = 1, MK_OP_ATTN = 2, MK_OP_OPROJ = 3, MK_OP_GATEUP = 4, MK_OP_DOWN = 5,
       MK_OP_LMHEAD = 6 };

/* Build a plan on the host: split every layer into per-CU instructions
 * (QKV row slices with the RMSNorm prologue; RoPE + KV append + split-KV
 * decode attention per (sequence, kv head, split); O-projection + residual;
 * gate/up + SiLU; down-projection + residual; LM-head row slices with
 * argmax), give each instruction the event it waits for and the event it
 * triggers, order each CU's list by dependency level (deadlock-free under
 * co-residency), and validate the result.  Host only; no device work unless
 * opts->num_cus == 0, which queries the current device's CU count.
 * (Megakernel page, section 2.5: the CPU builds the per-unit instruction
 * lists; section 2.6 item 5: static per-unit lists.) */
int mk_plan(const mk_model_shape *shape, const mk_plan_opts *opts, mk_plan_t **out);
/* The same call under its longer name (kept for existing callers). */
int mk_plan_create(const mk_model_shape *shape, const mk_plan_opts *opts, mk_plan_t **out);

/* Re-check a plan: every RAW dependency is covered by a waited event whose
 * triggers all precede it by level, no event is waited for more often than it
 * is triggered, lists are level-sorted, and the counters' targets are
 * reachable.  MK_OK or MK_ERR_PLAN. */
int mk_plan_validate(const mk_plan_t *plan);

/* Bytes the caller must allocate: workspace (device, 256-byte aligned), KV
 * cache (bf16 [n_layers][2][max_batch][n_kv_heads][max_ctx][head_dim]; plane
 * 0 keys, plane 1 values), logits (fp32 [max_batch][vocab]). */
int mk_plan_sizes(const mk_plan_t *plan, size_t *workspace_bytes, size_t *kv_cache_bytes,
                  size_t *logits_bytes, size_t *n_instructions);
int mk_plan_get_info(const mk_plan_t *plan, mk_plan_info *out);
/* Copy up to `cap` instruction descriptors into `out` (host array); *n_out
 * receives the total count. */
int mk_plan_export(const mk_plan_t *plan, mk_instr_desc *out, size_t cap, size_t *n_out);
/* Run the host-side schedule simulator: execute the plan's lists under
 * `n_trials` random interleavings (seeded) with no arithmetic, checking that
 * every wait is eventually satisfied and every read follows its producers.
 * MK_OK or MK_ERR_PLAN. */
int mk_plan_simulate(const mk_plan_t *plan, int32_t n_trials, uint64_t seed);

/* Event normalisation of a task graph, the scheme the megakernel page's Q&A
 * attributes to MPK ("En quoi le mécanisme de MPK diffère-t-il de simples
 * compteurs ?"): every task waits for at most one event and triggers at most
 * one; tasks with the same predecessors share one event and events that
 * share a predecessor are fused; events and tasks are then numbered
 * breadth-first, so the tasks one event releases are contiguous in `order`.
 * mk_plan_create derives its plans' events this way from the slices each
 * instruction reads and writes (the splits of an attention unit are one task).
 * Input: n_tasks; raw predecessors of task t are pred_list[pred_begin[t] ..
 * pred_begin[t+1]) (CSR, duplicates and transitively implied edges allowed:
 * the latter are removed); rank (optional, int64[n_tasks]) breaks ties in the
 * breadth-first order (smaller first; NULL: task index); flags bit 0 skips
 * the transitive reduction (tests).  Output arrays of n_tasks entries:
 * wait_event / trigger_event (-1: none), trigger_slot (the task's index among
 * its event's triggers), event_count[e] (triggers of event e; entries below
 * *n_events are written), order (tasks in breadth-first order).  Errors:
 * MK_ERR_INVALID_ARG (NULL array, bad offsets or task id), MK_ERR_PLAN (a
 * cycle among the edges, or a fused event that one of its own waiters would
 * have to precede).  Host only; no allocation is kept. */
#define MK_NORM_NO_REDUCTION 1u
int mk_events_normalize(int32_t n_tasks, const int32_t *pred_begin, const int32_t *pred_list, const int64_t *rank,
                        uint32_t flags, int32_t *wait_event, int32_t *trigger_event, int32_t *trigger_slot,
                        int32_t *event_count, int32_t *order, int32_t *n_events);
/* The plan's breadth-first instruction order (indices as mk_plan_export
 * numbers them): the order a global work queue hands instructions out in.
 * Writes min(cap, count) entries; *n_out receives the count. */
int mk_plan_get_queue(const mk_plan_t *plan, int32_t *out, size_t cap, size_t *n_out);
void mk_plan_destroy(mk_plan_t *plan);

/* Bind a plan to caller-owned device workspace (d_workspace, at least the
 * size mk_plan_sizes reports, 256-byte aligned).  Enqueues the upload of the
 * instruction lists and RoPE table and the zeroing of the counters on
 * `stream`.  The plan may be destroyed afterwards. */
int mk_ctx_create(const mk_plan_t *plan, void *d_workspace, size_t workspace_bytes, void *stream,
                  mk_ctx **out);

/* For callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * as mk_ctx_create, with the workspace taken from the library's static
 * device scratch array (32 MiB, MK_SCRATCH_BYTES in the library; each
 * device the library runs on holds it until the process ends) instead of a
 * caller buffer.  Calls no device allocator.  The caller still owns the
 * weights, KV cache, logits, tokens and positions.  Errors: MK_ERR_SCRATCH
 * when the plan's workspace (mk_plan_sizes) exceeds 32 MiB, plus those of
 * mk_ctx_create.  Every scratch context on a device shares the one array:
 * creating one re-initialises it (counters and flags cleared with a fill
 * kernel) and ends the previous scratch context on that device, whose later
 * mk_decode_step calls return MK_ERR_STATE; calls on two scratch contexts
 * that overlap on one device would race. */
int mk_ctx_create_scratch(const mk_plan_t *plan, void *stream, mk_ctx **out);

/* Weight tensors, all bf16 device pointers, 16-byte aligned, row-major
 * W[out][in].  Per-layer tensors come as host arrays of n_layers device
 * pointers.  lm_head is ignored (may be NULL) when the shape ties
 * embeddings.  The library borrows the pointers; they must outlive ctx. */
typedef struct {
  const void *embed;       /* [vocab][hidden] */
  const void *lm_head;     /* [vocab][hidden] */
  const void *final_norm;  /* [hidden] */
  const void *const *attn_norm; /* [hidden] */
  const void *const *wq;   /* [n_q_heads*head_dim][hidden] */
  const void *const *wk;   /* [n_kv_heads*head_dim][hidden] */
  const void *const *wv;   /* [n_kv_heads*head_dim][hidden] */
  const void *const *wo;   /* [hidden][n_q_heads*head_dim] */
  const void *const *mlp_norm;  /* [hidden] */
  const void *const *wg;   /* [ffn][hidden] */
  const void *const *wu;   /* [ffn][hidden] */
  const void *const *wd;   /* [hidden][ffn] */
} mk_weights;

/* Check and record the weight pointers and enqueue their upload into the
 * workspace's pointer table on `stream`; synchronises `stream` before
 * returning.  The host binds what the GPU consumes, once: the megakernel
 * page puts the host on the preparing side (section 2.5: the CPU builds the
 * instruction lists and hands them over) and the persistent kernel on the
 * consuming side (section 2.1).  Errors: MK_ERR_INVALID_ARG for a NULL
 * context, table or tensor pointer (lm_head only when untied);
 * MK_ERR_ALIGN when a tensor is not 16-byte aligned; MK_ERR_HIP when the
 * upload fails.  On error the context keeps its previous binding. */
int mk_load_weights(mk_ctx *ctx, const mk_weights *w, void *stream);

#define MK_ADVANCE 1u  /* after the step: tokens[b] = next token, positions[b] += 1 */

/* The hot path: one decoder forward pass for `batch` sequences, as the
 * megakernel page defines the object (section 2.1: one persistent launch
 * whose workgroups stay resident and resolve dependencies in global memory;
 * section 2.5: the GPU consumes the lists the host prepared).
 * d_tokens[b] (int32) is read at position d_positions[b] (int32); the step
 * writes keys/values of that position into d_kv_cache for every layer,
 * attends over slots [0, positions[b]], writes fp32 logits d_logits[b][vocab]
 * and, when d_next_tokens is not NULL, the greedy next token (smallest index
 * among equal maxima).  With MK_ADVANCE the step also stores the next token
 * into d_tokens and increments d_positions on the device, so steps can be
 * enqueued back to back without the host.  Enqueued on `stream`; device-side
 * input errors (token or position out of range) and watchdog expiries are
 * reported by mk_get_device_error.  MK_EXEC_MEGA, MK_EXEC_FLAT and
 * MK_EXEC_STREAM: exactly one kernel launch; MK_EXEC_MULTI and
 * MK_EXEC_FLAT_MULTI: one launch per dependency level.
 * Layouts: d_tokens, d_positions int32[batch] (sequence b uses sequence
 * slot b of the cache); d_kv_cache as mk_plan_sizes describes; d_logits
 * fp32 [batch][vocab]; d_next_tokens int32[batch].  Sequence slots
 * batch..max_batch-1 of the cache are neither read nor written.
 * Host-side errors (nothing is enqueued): MK_ERR_INVALID_ARG (NULL context
 * or buffer, unknown flag, weights not bound), MK_ERR_CTX_OVERFLOW (batch
 * outside 1..max_batch), MK_ERR_ALIGN (d_kv_cache not 16-byte aligned or an
 * int32/fp32 buffer not 4-byte aligned), MK_ERR_STATE (context poisoned),
 * MK_ERR_HIP (launch failed); MK_ERR_STATE also for a scratch context
 * that a newer one on the same device replaced. */
int mk_decode_step(mk_ctx *ctx, int32_t *d_tokens, int32_t *d_positions, int32_t batch, void *d_kv_cache,
                   float *d_logits, int32_t *d_next_tokens, uint32_t flags, void *stream);

/* Multi-token persistent decode: n_steps greedy steps in ONE launch of the
 * homogeneous engine (MK_EXEC_FLAT, any sync mode).  The executive-summary
 * page names what a kernel boundary costs per token (launch latency and the
 * memory bubble while the next kernel's first loads travel, "Le problème");
 * here the argmax of step t feeds step t + 1's embedding on the device and
 * step t + 1 starts as soon as that token is published, inside the same
 * persistent launch (megakernel page, section 2.1).  Step t reads
 * d_tokens/d_positions as step t - 1 left them (the device advances both,
 * as MK_ADVANCE does), appends cache slot positions[b] and writes its
 * logits at d_logits + t * batch * vocab and, when d_next_tokens is not
 * NULL, its tokens at d_next_tokens + t * batch.  Buffers: d_logits fp32
 * [n_steps][batch][vocab]; d_next_tokens int32 [n_steps][batch]; others as
 * for mk_decode_step.  Results are bit-identical to n_steps calls of
 * mk_decode_step with MK_ADVANCE.  The context's epoch advances by n_steps.
 * Host-side errors: those of mk_decode_step, MK_ERR_UNSUPPORTED (exec mode
 * not MK_EXEC_FLAT), MK_ERR_INVALID_ARG (n_steps outside 1..MK_MAX_STEPS),
 * MK_ERR_ALIGN (d_kv_cache not 128-byte aligned: an appended row must not
 * share a cache line with rows an earlier step of the launch has read).
 * Device-side errors as for mk_decode_step (a position reaching max_ctx
 * stops the launch with MK_ERR_INPUT). */
#define MK_MAX_STEPS 65536
int mk_decode_steps(mk_ctx *ctx, int32_t *d_tokens, int32_t *d_positions, int32_t batch, void *d_kv_cache,
                    float *d_logits, int32_t *d_next_tokens, int32_t n_steps, void *stream);

/* The per-level build (MK_EXEC_FLAT_MULTI) of one decode step captured into
 * a hipGraph: the baseline that separates the host's launch cost from the
 * kernel-boundary bubble.  The megakernel page (section 2.2) sets the
 * persistent kernel apart from a captured graph, which still ends and starts
 * a kernel at every node; the executive-summary page ("Le problème") names
 * the costs a boundary keeps even when the graph removes the host's launch
 * latency (the drain of the finishing kernel, the next kernel's cold start).
 * mk_graph_create captures one step on these buffers and flags (MK_ADVANCE
 * or 0) as n_levels kernel nodes plus one node that advances the step's
 * epoch on the device; mk_graph_launch replays it on `stream` (one step,
 * results identical to mk_decode_step with the same arguments); steps
 * enqueued by other calls in between are accounted for before the replay.
 * The graph owns a small device record of the step (allocated at creation);
 * destroy graphs before their context.  Errors: those of mk_decode_step's
 * host checks, MK_ERR_UNSUPPORTED (exec mode not MK_EXEC_FLAT_MULTI),
 * MK_ERR_HIP (allocation, capture or instantiation failed). */
typedef struct mk_graph_s mk_graph; /* opaque, host memory, owned by the library */
int mk_graph_create(mk_ctx *ctx, int32_t *d_tokens, int32_t *d_positions, int32_t batch, void *d_kv_cache,
                    float *d_logits, int32_t *d_next_tokens, uint32_t flags, void *stream, mk_graph **out);
int mk_graph_launch(mk_graph *graph, void *stream);
void mk_graph_destroy(mk_graph *graph);

/* Synchronise `stream`, read the device error word: MK_OK, MK_ERR_TIMEOUT or
 * MK_ERR_INPUT.  *detail (optional) receives the instruction/ CU code.  A
 * non-OK result poisons ctx (mk_decode_step returns MK_ERR_STATE) until
 * mk_ctx_reset. */
int mk_get_device_error(mk_ctx *ctx, void *stream, int32_t *detail);
/* Zero the counters, flags and error word and restart the epoch. */
int mk_ctx_reset(mk_ctx *ctx, void *stream);
/* Number of decode steps enqueued since creation or the last reset. */
int64_t mk_ctx_epoch(const mk_ctx *ctx);
void mk_ctx_destroy(mk_ctx *ctx);

const char *mk_strerror(int code);

/* ------------------------------------------------------------ device facts */
typedef struct {
  int32_t num_cus, lds_per_block, lds_per_cu, warp_size, clock_khz, mem_clock_khz, mem_bus_bits;
  int32_t max_threads_per_block, mega_blocks_per_cu; /* occupancy of the megakernel */
  char arch[64];
} mk_device_info;
int mk_device_query(int32_t device, mk_device_info *out);

/* ------------------------------------------------------------ measurement */
/* Grid-wide barrier microbenchmark (megakernel page, section 2.6 item 3 and
 * the executive-summary page's comparison of atomic versus sentinel grid
 * synchronisation).  Launches n_blocks persistent workgroups that perform
 * n_barriers grid barriers with the chosen variant:
 *   0 cooperative-groups grid sync (cooperative launch),
 *   1 monotonic counter, agent-scope release add + acquire poll,
 *   2 monotonic counter, write-through data + relaxed atomics, no cache
 *     maintenance,
 *   3 per-block epoch flags (plain stores, one vector poll of all flags),
 *   4 data sentinel: each block's payload word starts as a NaN pattern no
 *     arithmetic produces and the barrier waits until every payload changed,
 *   5 two-level epoch flags (n_blocks >= 8): blocks b % 8 == g form group g
 *     (one XCD under round-robin dispatch, up to a rotation); block g polls
 *     every flag and publishes a group flag that the group's other blocks
 *     poll.
 * d_scratch: device memory of at least mk_gridsync_scratch_bytes(n_blocks)
 * bytes; d_result: device int32[4]: [0] = number of data-visibility errors
 * seen, [1] = watchdog expiries, [2] = (variant 5) blocks whose XCD differs
 * from b % 8 (information only: every access is device scope).  Enqueued on `stream`; MK_ERR_INVALID_ARG for an unknown
 * variant or variant 5 with fewer than 8 blocks. */
size_t mk_gridsync_scratch_bytes(int32_t n_blocks);
int mk_gridsync_bench(int32_t variant, int32_t n_barriers, int32_t n_blocks, void *d_scratch,
                      int32_t *d_result, void *stream);

/* Streaming-read probe: read `bytes` (multiple of 16) of d_buf with 16-byte
 * non-temporal loads from n_blocks workgroups and write one checksum word per
 * block to d_out (uint32[n_blocks]).  Gives the achievable HBM read rate. */
int mk_stream_read(const void *d_buf, size_t bytes, uint32_t *d_out, int32_t n_blocks, void *stream);

/* Streaming-read probe through LDS: n_waves (1..8) waves per workgroup stream
 * `bytes` (multiple of 1024) of d_buf into a 64 KiB LDS ring with direct
 * global->LDS loads, as the megakernel's loader waves do.  d_out: uint32
 * [n_blocks]. */
int mk_lds_stream_read(const void *d_buf, size_t bytes, uint32_t *d_out, int32_t n_blocks, int32_t n_waves,
                       void *stream);

/* ------------------------------------------------------------ test hooks */
/* Replace a plan's instruction list with `n` descriptors (fields as
 * mk_plan_export writes them; slots, tickets and partial indices are
 * re-derived).  Used by tests that corrupt a plan on purpose; the plan is
 * then accepted only if mk_plan_validate passes.  Host only. */
int mk_plan_set_instructions(mk_plan_t *plan, const mk_instr_desc *descs, size_t n);
/* Byte offsets of the activation buffers inside the workspace, for tests
 * and debugging: out[0..7] = qkv, attn, xmid, hbuf, xout, end of the
 * activation block, attention partials, parity stride (bytes; 0 unless
 * sentinel mode).  Each activation buffer is fp32 [n_layers][max_batch][n]
 * with n = (n_q + 2 n_kv) head_dim, n_q head_dim, hidden, ffn, hidden. */
int mk_plan_get_layout(const mk_plan_t *plan, uint64_t out[8]);
/* Shorten the device watchdog of a context (microseconds) so tests can turn a
 * wait that cannot be met into MK_ERR_TIMEOUT quickly.  Synchronises stream. */
int mk_ctx_set_watchdog_us(mk_ctx *ctx, uint32_t us, void *stream);
/* Instruction trace of the persistent kernels: when d_trace is not NULL
 * every instruction i of later steps stores 8 uint64 at d_trace[8*i]: the
 * 100 MHz real-time counter when its wait began, when its inputs were
 * staged (work began) and when it finished; (cu << 32 | step epoch); for the
 * role-specialised kernel the CU's cumulative ticks of loader waves blocked
 * on a free page and of compute waves waiting for a landed page, the
 * instruction's page count and when its compute waves finished (before the
 * sync wave's epilogue); for a projection of the stream engine, when its
 * input event was seen and when every streamer had finished its rows (words
 * 4 and 5); else 0.  n_records must cover the plan's
 * instruction count.  NULL switches tracing off.  Synchronises stream. */
int mk_ctx_set_trace(mk_ctx *ctx, void *d_trace, size_t n_records, void *stream);
/* Overwrite the host-side step counter of a context.  Setting it ahead of the
 * device counters makes the next step's dependency waits unsatisfiable, which
 * (with a short watchdog) exercises the MK_ERR_TIMEOUT path without a hang. */
int mk_ctx_set_epoch(mk_ctx *ctx, int64_t epoch);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
