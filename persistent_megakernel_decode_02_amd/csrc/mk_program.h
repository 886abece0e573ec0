// Device-visible program layout shared by the host planner and the kernels.
//
// A plan is a set of per-CU instruction lists (megakernel page, section 2.5:
// the host builds the lists, each compute unit runs its own; section 2.6
// items 2, 3 and 5: opcode dispatch, dependency counters, static lists).
// Everything the kernels need lives in one MkProgram record inside the
// caller's workspace; per-step values travel in MkStep by value.
#pragma once
#include <stdint.h>

// Counter mode keeps one row of event counters per XCD: a producer bumps its
// own XCD's row and a waiter sums the rows, so the atomic adds of one event
// land on MK_CTR_ROWS addresses (4 KiB apart) instead of queueing on one.
#define MK_CTR_ROWS 8
static inline int mk_ctr_stride(int n_events) { return ((n_events > 1 ? n_events : 1) + 1023) & ~1023; }

#define MK_MAX_BATCH 16
#define MK_MAX_GROUP 4     // q heads per kv head
#define MK_BLOCK 512       // threads per workgroup (8 wave64)
#define MK_NWAVES (MK_BLOCK / 64)

// role engine
#define MK_PAGE 4096                      // bytes per LDS page
#define MK_MAXNP 64                       // most pages in the ring
#define MK_NLW 2                          // loader waves
#define MK_NCW (MK_NWAVES - MK_NLW - 1)   // compute waves (one more wave syncs and stores)
#define MK_RB_MAXB 4                      // sequences the role engine stages per instruction
#define MK_CTL_BYTES 1024                 // LDS control block
#define MK_LDS_TOTAL (160 * 1024)         // LDS of one gfx950 workgroup

// batched projections of the homogeneous engine (bf16 MFMA, up to 16 sequences)
// data-sentinel synchronisation: activation words hold this quiet-NaN
// payload (which no arithmetic produces) until their producer writes them
#define MK_SENTINEL 0x7FBADBADu

// stream engine: streamer waves per workgroup (the last wave synchronises)
#define MK_STREAMERS (MK_NWAVES - 1)

#define MK_MAX_VOCAB 131070                // token rows fit 17 bits (0x1ffff: no row)
#define MK_MFMA_MIN_BATCH 2                   // sequences from which projections run on MFMA
#define MK_BKC 2048                           // input columns staged in LDS per chunk
#define MK_BROW (MK_BKC * 2 + 16)             // bytes per sequence row of one bf16 plane (+16: bank skew)
#define MK_BPLANE (MK_MAX_BATCH * MK_BROW)    // one bf16 plane (high or low parts) of the staged inputs
#define MK_BRED (2 * MK_BPLANE)               // per-wave fp32 partial tiles [MK_NWAVES][256]
#define MK_BARG (MK_BRED + MK_NWAVES * 1024)  // per-wave argmax (value, index) per sequence
#define MK_BLDS (MK_BARG + MK_NWAVES * MK_MAX_BATCH * 8)
#define MK_BGAIN MK_BLDS                      // [MK_BKC / 4] RMSNorm gain of a one-chunk row, 4 bf16 each
#define MK_BLDS_END (MK_BGAIN + MK_BKC * 2)

// attention instruction of the homogeneous engine (byte offsets into dynamic LDS)
#define MK_FA_Q 0                                                // [G][d] fp32 scaled, rotated queries
#define MK_FA_KN (MK_FA_Q + MK_MAX_GROUP * 128 * 4)              // [d] bf16 key of this step
#define MK_FA_VN (MK_FA_KN + 256)                                // [d] bf16 value of this step
#define MK_FA_VB (MK_FA_VN + 256)                                // [MK_NWAVES][32][2 d + 16 bytes] bf16 value blocks
#define MK_FA_WP (MK_FA_VB + MK_NWAVES * 32 * (2 * 128 + 16))    // [MK_NWAVES][G][d + 2] wave partials
#define MK_FA_LDS (MK_FA_WP + MK_NWAVES * MK_MAX_GROUP * 130 * 4)

enum MkSync : int32_t { MKSYNC_COUNTER = 0, MKSYNC_FLAG = 1, MKSYNC_SENTINEL = 2 };
enum MkExec : int32_t {
  MKEXEC_MEGA = 0,
  MKEXEC_MULTI = 1,
  MKEXEC_FLAT = 2,
  MKEXEC_STREAM = 3,
  MKEXEC_FLAT_MULTI = 4,
  MKEXEC_QUEUE = 5
};

enum MkOp : int32_t {
  MKOP_QKV = 1,
  MKOP_ATTN = 2,
  MKOP_OPROJ = 3,
  MKOP_GATEUP = 4,
  MKOP_DOWN = 5,
  MKOP_LMHEAD = 6,
};

// One instruction: 48 bytes, read with scalar loads (uniform per workgroup).
struct MkInstr {
  int32_t op, layer;
  int32_t r0, r1;        // GEMV: output rows [r0, r1).  ATTN: r0 = sequence, r1 = kv head
  int32_t split, nsplit; // ATTN: key-range split s of S
  int32_t wait_ev;       // event waited for before starting (-1: none)
  int32_t sig_ev;        // event triggered when done (-1: none)
  int32_t sig_slot;      // flag slot inside sig_ev (flag mode)
  int32_t ticket;        // ATTN: merge ticket index; LMHEAD: argmax ticket index; else -1
  int32_t part;          // LMHEAD: slot of this instruction's argmax partial
  int32_t level;
};

// Stream engine: where a projection instruction's rows are, built on the
// host once the weights are bound.  Virtual row v of the instruction starts
// at (v odd ? b1 : b0) + (v / 2) * stride2 bytes and is rb bytes long
// (gate/up: b0 = first gate row, b1 = first up row, stride2 = rb; other
// projections: b1 = b0 + rb, stride2 = 2 rb).  off: the row rotation of the
// instruction in its CU's list (virtual row v belongs to streamer
// (v + off) mod the streamer count).  Attention instructions have n = 0.
struct MkRowTab {
  uint64_t b0, b1;
  int32_t n, rb, stride2, off;
};

struct MkLayerW {
  const uint16_t *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *wg, *wu, *wd;
};

struct MkProgram {
  // model shape
  int32_t L, H, nq, nkv, d, I, V, G;  // G = nq / nkv
  int32_t B_max, max_ctx, S;          // S = attention splits per (sequence, kv head)
  float eps;
  int32_t tied;
  int32_t sync_mode;                  // 0 counters, 1 flags, 2 data sentinels
  int32_t n_cu, n_instr, n_levels, n_events, n_lm_parts;
  int32_t ctr_stride;                 // words between the per-XCD rows of ctr
  uint32_t watchdog_ticks;            // s_memrealtime ticks (100 MHz) before a wait gives up
  // role-engine LDS layout (byte offsets into dynamic LDS) and ring size
  int32_t lds_x, lds_resid, lds_out, lds_ring, n_pages, lds_total;
  int32_t out_stride;                 // floats per sequence in the per-row result area
  // stream engine LDS layout (byte offsets into dynamic LDS; the staged
  // input vector starts at 0): row results, residual rows, control block
  int32_t st_out, st_resid, st_ctl;
  // activations occupy one contiguous block starting at qkv; in sentinel
  // mode a second copy (the other step parity) follows at +par_stride floats
  int64_t par_stride;
  // homogeneous engine, sentinel mode: this record is the one for steps of
  // one parity; `act_other` is the other parity's activation block, which a
  // step resets to the sentinel for the step after it
  float *act_other;
  // epoch+1 of the last step whose greedy tokens are merged (multi-step
  // launches: a step starts once the previous one has produced its token)
  uint32_t *lm_done;

  // lists (device pointers into the workspace)
  const MkInstr *instr;        // CU-major
  const int32_t *cu_begin;     // [n_cu + 1]
  const int32_t *level_begin;  // [n_levels + 1] into level_list (multi-launch)
  const int32_t *level_list;   // instruction indices grouped by level
  const int32_t *queue;        // [n_instr] breadth-first instruction order (work-queue engine)
  uint32_t *queue_ctr;         // tickets handed out so far (n_instr + n_cu per step)
  const int32_t *ev_count;     // [n_events] triggers per step
  const int32_t *ev_flag_base; // [n_events] first flag slot

  // tables and weights
  const float *rope;           // [max_ctx][d/2][2] (cos, sin), fp32
  MkLayerW *layers;            // [L]
  const MkRowTab *rowtab;      // [n_instr] (stream engine)
  const uint16_t *embed, *lm_head, *final_norm;
  // batched plans: the LM-head matrix repacked as 1 KiB operand-order tiles
  // (16 rows x 32 columns, rows padded to a multiple of 16 with zeros), or null
  const uint16_t *lm_tiled;
  // batched plans: each layer's gate and up matrices as 1 KiB tiles of 8
  // hidden units (rows 0-7 gate, 8-15 up), layer l at l * 2 I H, or null
  const uint16_t *gu_tiled;

  // activations (fp32), one buffer per layer so no slot is rewritten in a step
  float *qkv;    // [L][B][(nq + 2 nkv) d]
  float *attn;   // [L][B][nq d]
  float *xmid;   // [L][B][H]
  float *hbuf;   // [L][B][I]
  float *xout;   // [L][B][H]
  float *part;   // [L][B][nkv][S][G][d + 2]   (m, l, o[d]) per split and q head
  float *dpart;  // batched down projection split by input columns: [L][Sd][B][H] partial sums per part
  uint64_t *lm_pk; // [n_lm_parts][B] tagged (value, row) of the homogeneous engine's LM-head parts
  float *lm_val; // [n_lm_parts][B]
  int32_t *lm_idx;

  // synchronisation
  uint32_t *ctr;     // [MK_CTR_ROWS][ctr_stride] monotonic counters, one row per XCD
  uint32_t *flags;   // [sum ev_count] epoch flags
  uint32_t *tickets; // [n_tickets] monotonic last-arriver tickets
  int32_t *err;      // [4]: code, detail, abort flag, spare
  uint64_t *trace;   // optional: [n_instr][4] wait-begin, start, end (100 MHz ticks), cu
};

struct MkStep {
  int32_t *tokens;
  int32_t *positions;
  uint16_t *kv;    // [L][2][B_max][nkv][max_ctx][d] bf16
  float *logits;   // [B][V]
  int32_t *next;   // [B] or null
  int32_t batch;
  uint32_t epoch;  // steps completed on this context before this one
  uint32_t flags;  // MK_ADVANCE
  int32_t multi;   // 1: launched per level (no waits/signals)
  int32_t level;   // multi-launch: level this launch runs
  int32_t n_steps; // homogeneous engine: greedy steps run by this launch (>= 1)
};

// Device code of the role engine reads the program and step records through
// the constant address space (scalar loads that stay valid across the
// engine's LDS-flag assembly); on the host these are the plain types.
#if defined(__HIP_DEVICE_COMPILE__)
#define MK_CONST __attribute__((address_space(4)))
#else
#define MK_CONST
#endif
typedef const MK_CONST MkProgram MkProgC;
typedef const MK_CONST MkStep MkStepC;

