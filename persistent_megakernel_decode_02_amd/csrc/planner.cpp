// Host planner, plan validator and schedule simulator.
//
// The megakernel page ("2 . Definition et genealogie") has the host build
// the instruction lists (section 2.5), gives every instruction an input
// counter, a target value and an output counter (section 2.6 item 3) and
// runs static per-unit lists (section 2.6 item 5).  Its Q&A explains why the
// grid must be fully resident: a block waiting on a counter that a
// not-yet-resident block must bump never finishes.  The planner therefore
// orders every CU's list by dependency level; under co-residency this is
// deadlock-free by induction on the level, and mk_plan_check verifies it
// together with read-after-write coverage of every activation slice.
#include "planner.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <map>
#include <random>

namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

enum { LV_QKV = 0, LV_ATTN = 1, LV_O = 2, LV_GU = 3, LV_DOWN = 4, LV_PER_LAYER = 5 };

struct Pending {
  MkInstr in;
  double bytes;
};

}  // namespace

static int check_shape(const mk_model_shape *s, const mk_plan_opts *o) {
  if (!s || !o) return MK_ERR_INVALID_ARG;
  if (s->n_layers < 1 || s->hidden < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->ffn < 1 ||
      s->vocab < 1)
    return MK_ERR_SHAPE;
  if (s->head_dim != 64 && s->head_dim != 128) return MK_ERR_SHAPE;
  if (s->n_q_heads % s->n_kv_heads) return MK_ERR_SHAPE;
  if (s->n_q_heads / s->n_kv_heads > MK_MAX_GROUP) return MK_ERR_SHAPE;
  if (s->hidden % 256 || s->ffn % 256 || (s->n_q_heads * s->head_dim) % 256) return MK_ERR_SHAPE;
  if (!(s->rms_eps > 0) || !(s->rope_theta > 1)) return MK_ERR_SHAPE;
  if (o->max_batch < 1 || o->max_batch > MK_MAX_BATCH) return MK_ERR_INVALID_ARG;
  if (s->vocab > MK_MAX_VOCAB) return MK_ERR_SHAPE;  // a token index fits the tagged argmax record
  if (o->max_ctx < 1 || o->max_ctx > (1 << 20)) return MK_ERR_INVALID_ARG;
  if (o->kv_splits < 0 || o->kv_splits > o->max_ctx) return MK_ERR_INVALID_ARG;
  if (o->sync_mode < MK_SYNC_COUNTER || o->sync_mode > MK_SYNC_SENTINEL) return MK_ERR_INVALID_ARG;
  if (o->exec_mode < MK_EXEC_MEGA || o->exec_mode > MK_EXEC_QUEUE) return MK_ERR_INVALID_ARG;
  // data sentinels replace the events only inside one persistent launch; the
  // homogeneous engine polls them in its one-sequence ops only
  if (o->sync_mode == MK_SYNC_SENTINEL && o->exec_mode != MK_EXEC_MEGA &&
      !(o->exec_mode == MK_EXEC_FLAT && o->max_batch < MK_MFMA_MIN_BATCH))
    return MK_ERR_UNSUPPORTED;
  // the stream engine runs one sequence per step; its sync wave holds a
  // normalised vector of at most 4096 floats in registers
  if (o->exec_mode == MK_EXEC_STREAM && (o->max_batch != 1 || s->hidden > 4096)) return MK_ERR_UNSUPPORTED;
  return MK_OK;
}

// Role-engine LDS: control block | per-compute-wave scratch | residual rows |
// staged input vectors | page ring (the rest of the workgroup's 160 KiB).
static int role_lds_layout(mk_plan_t *p) {
  const mk_model_shape &s = p->shape;
  const int B = p->B, d = s.head_dim, G = p->G;
  if (B > MK_RB_MAXB) return MK_ERR_UNSUPPORTED;
  int max_rows = 1, max_out = 1;
  for (const MkInstr &in : p->instr) {
    if (in.op == MKOP_OPROJ || in.op == MKOP_DOWN) max_rows = std::max(max_rows, in.r1 - in.r0);
    if (in.op != MKOP_ATTN) max_out = std::max(max_out, in.r1 - in.r0);
  }
  int64_t kmax = std::max<int64_t>({(int64_t)s.hidden, (int64_t)s.n_q_heads * d, (int64_t)s.ffn});
  int64_t x_floats = std::max<int64_t>((int64_t)B * kmax, (int64_t)(G + 2) * d + (int64_t)MK_NCW * G * (d + 2));
  int64_t o = MK_CTL_BYTES;
  // per-row results of the compute waves: [B][out_stride]
  p->out_stride = (max_out + 3) / 4 * 4;
  p->lds_out = (int)o;
  o += (int64_t)B * p->out_stride * 4;
  p->lds_resid = (int)o;
  o += ((int64_t)B * max_rows * 4 + 15) / 16 * 16;
  p->lds_x = (int)o;
  o += (x_floats * 4 + 255) / 256 * 256;
  p->lds_ring = (int)o;
  int64_t pages = (MK_LDS_TOTAL - o) / MK_PAGE;
  if (pages > MK_MAXNP) pages = MK_MAXNP;
  if (pages < 4) return MK_ERR_UNSUPPORTED;
  p->n_pages = (int)pages;
  p->lds_bytes = MK_LDS_TOTAL;
  return MK_OK;
}

static int lds_requirement(const mk_plan_t *p) {
  const mk_model_shape &s = p->shape;
  const int B = p->B, d = s.head_dim;
  int64_t kmax = std::max<int64_t>({(int64_t)s.hidden, (int64_t)s.n_q_heads * d, (int64_t)s.ffn});
  // vector GEMV ops stage one sequence's input vector at a time; with two or
  // more sequences the projections stage bf16 high/low planes of every
  // sequence's inputs (MK_BKC columns at a time) for the matrix cores
  // (the staged vector, 64 floats of norm/argmax scratch, per-wave partial
  // sums of 4 rows for instructions that split the columns, then the
  // residual inputs of an instruction's output rows, at most H)
  // (plus the instruction's output rows, gathered before they are stored)
  int64_t rows = 0;
  for (const MkInstr &in : p->instr)
    if (in.op != MKOP_ATTN) rows = std::max<int64_t>(rows, in.r1 - in.r0);
  int64_t gemv = kmax * 4 + 256 + (int64_t)MK_NWAVES * 4 * 4 + (int64_t)s.hidden * 4 + (rows + 4) * 4;
  if (B >= MK_MFMA_MIN_BATCH) gemv = std::max<int64_t>(gemv, MK_BLDS_END);
  // attention: queries, this step's key/value, per-wave value blocks and partials
  return (int)std::max<int64_t>(gemv, MK_FA_LDS);
}

// Stream engine LDS: the staged input vector at 0 (the widest projection
// input), the row results of one instruction, the residual rows of an O or
// down slice, then (past the attention instruction's own layout, which
// overlays the first two while all waves run attention) the control block.
static void stream_lds_layout(mk_plan_t *p) {
  const mk_model_shape &s = p->shape;
  // row results: one partial sum per 4 KiB unit of every row
  auto nsub = [](int64_t K) { return (int)((2 * K + 4095) / 4096); };
  int max_out = 1, max_res = 1;
  for (const MkInstr &in : p->instr) {
    const int n = in.r1 - in.r0;
    switch (in.op) {
      case MKOP_QKV:
      case MKOP_LMHEAD: max_out = std::max(max_out, n * nsub(s.hidden)); break;
      case MKOP_GATEUP: max_out = std::max(max_out, 2 * n * nsub(s.hidden)); break;
      case MKOP_OPROJ: max_out = std::max(max_out, n * nsub((int64_t)s.n_q_heads * s.head_dim)); break;
      case MKOP_DOWN: max_out = std::max(max_out, n * nsub(s.ffn)); break;
      default: break;
    }
    if (in.op == MKOP_OPROJ || in.op == MKOP_DOWN) max_res = std::max(max_res, n);
  }
  const int64_t kmax = std::max<int64_t>({(int64_t)s.hidden, (int64_t)s.n_q_heads * s.head_dim, (int64_t)s.ffn});
  // the input vector is staged in whole 2048-column units (zero tail)
  int64_t o = align_up((size_t)(kmax + 2047) / 2048 * 2048 * 4, 256);
  p->st_out = (int)o;
  o = align_up((size_t)(o + (int64_t)max_out * 4), 256);
  p->st_resid = (int)o;
  o = align_up((size_t)(o + (int64_t)max_res * 4), 256);
  o = std::max<int64_t>(o, align_up(MK_FA_LDS, 256));
  p->st_ctl = (int)o;
  p->lds_bytes = (int)(o + 256);
}

// Batched plans of the homogeneous engine multiply the LM head and gate/up
// on the matrix cores from copies of their matrices in operand-order tiles
// (built by mk_load_weights); the hidden size must be a multiple of the tile
// width and the FFN size of the 8-unit gate/up tile.
bool mk_plan_tiles(const mk_plan_t *p) {
  const int m = p->opts.exec_mode;
  return p->B >= MK_MFMA_MIN_BATCH && p->shape.hidden % 32 == 0 && p->shape.ffn % 8 == 0 &&
         (m == MK_EXEC_FLAT || m == MK_EXEC_FLAT_MULTI || m == MK_EXEC_QUEUE);
}

void mk_plan_finalize_lists(mk_plan_t *p) {
  // stable sort instructions by (cu, slot order as given), recompute cu_begin and level lists
  const int n = (int)p->instr.size();
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return p->instr_cu[a] < p->instr_cu[b]; });
  std::vector<MkInstr> in2(n);
  std::vector<int32_t> cu2(n);
  for (int i = 0; i < n; ++i) {
    in2[i] = p->instr[order[i]];
    cu2[i] = p->instr_cu[order[i]];
  }
  p->instr.swap(in2);
  p->instr_cu.swap(cu2);
  p->cu_begin.assign(p->n_cu + 1, 0);
  for (int i = 0; i < n; ++i) p->cu_begin[p->instr_cu[i] + 1]++;
  for (int c = 0; c < p->n_cu; ++c) p->cu_begin[c + 1] += p->cu_begin[c];
  p->level_begin.assign(p->n_levels + 1, 0);
  for (int i = 0; i < n; ++i) {
    int lv = p->instr[i].level;
    if (lv >= 0 && lv < p->n_levels) p->level_begin[lv + 1]++;
  }
  for (int l = 0; l < p->n_levels; ++l) p->level_begin[l + 1] += p->level_begin[l];
  p->level_list.assign(n, 0);
  std::vector<int32_t> fill(p->level_begin.begin(), p->level_begin.end() - 1);
  for (int i = 0; i < n; ++i) {
    int lv = p->instr[i].level;
    if (lv >= 0 && lv < p->n_levels) p->level_list[fill[lv]++] = i;
  }
}

void mk_plan_compute_layout(mk_plan_t *p) {
  const mk_model_shape &s = p->shape;
  const size_t L = s.n_layers, B = p->B, H = s.hidden, d = s.head_dim, nq = s.n_q_heads,
               nkv = s.n_kv_heads, I = s.ffn, R = (nq + 2 * nkv) * d;
  MkLayout &y = p->lay;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  y.prog = take(sizeof(MkProgram));
  y.prog_odd = take(sizeof(MkProgram));
  y.instr = take(sizeof(MkInstr) * std::max<size_t>(p->instr.size(), 1));
  y.cu_begin = take(4 * (p->n_cu + 1));
  y.level_begin = take(4 * (p->n_levels + 1));
  y.level_list = take(4 * std::max<size_t>(p->instr.size(), 1));
  y.queue = take(4 * std::max<size_t>(p->instr.size(), 1));
  y.ev_count = take(4 * std::max(p->n_events, 1));
  y.ev_flag_base = take(4 * std::max(p->n_events, 1));
  y.rope = take(4 * (size_t)p->max_ctx * d);
  y.layers = take(sizeof(MkLayerW) * L);
  y.rowtab = take(sizeof(MkRowTab) * std::max<size_t>(p->instr.size(), 1));
  y.lm_tiled_bytes = mk_plan_tiles(p) ? (size_t)ceil_div(s.vocab, 16) * 16 * s.hidden * 2 : 0;
  y.lm_tiled = y.lm_tiled_bytes ? take(y.lm_tiled_bytes) : 0;
  y.gu_tiled_bytes = mk_plan_tiles(p) ? L * 2 * I * H * 2 : 0;  // every layer's gate and up rows
  y.gu_tiled = y.gu_tiled_bytes ? take(y.gu_tiled_bytes) : 0;
  y.qkv = take(4 * L * B * R);
  y.attn = take(4 * L * B * nq * d);
  y.xmid = take(4 * L * B * H);
  y.hbuf = take(4 * L * B * I);
  y.xout = take(4 * L * B * H);
  y.act_end = o;
  if (p->opts.sync_mode == MK_SYNC_SENTINEL) o += y.act_end - y.qkv;  // second parity
  y.part = take(4 * L * B * nkv * p->S * p->G * (d + 2));
  y.dpart = take(p->Sd > 1 ? 4 * L * (size_t)p->Sd * B * H : 0);
  y.lm_val = take(4 * (size_t)std::max(p->n_lm_parts, 1) * B);
  y.lm_idx = take(4 * (size_t)std::max(p->n_lm_parts, 1) * B);
  y.sync_begin = o;
  y.ctr = take(4 * (size_t)MK_CTR_ROWS * mk_ctr_stride(p->n_events));
  y.flags = take(4 * std::max(p->n_flags, 1));
  y.tickets = take(4 * std::max(p->n_tickets, 1));
  y.lm_pk = take(8 * (size_t)std::max(p->n_lm_parts, 1) * B);
  y.lm_done = take(4);
  y.queue_ctr = take(4);
  y.err = take(16);
  y.sync_end = o;
  y.total = o;
}

int mk_plan_build(const mk_model_shape *shape, const mk_plan_opts *opts, int n_cu, mk_plan_t **out) {
  if (!out) return MK_ERR_INVALID_ARG;
  *out = nullptr;
  int rc = check_shape(shape, opts);
  if (rc) return rc;
  if (n_cu < 1 || n_cu > 4096) return MK_ERR_INVALID_ARG;

  mk_plan_t *p = new (std::nothrow) mk_plan_t();
  if (!p) return MK_ERR_INVALID_ARG;
  p->shape = *shape;
  p->opts = *opts;
  p->n_cu = n_cu;
  p->B = opts->max_batch;
  p->max_ctx = opts->max_ctx;
  const mk_model_shape &s = *shape;
  const int L = s.n_layers, H = s.hidden, d = s.head_dim, nq = s.n_q_heads, nkv = s.n_kv_heads,
            I = s.ffn, V = s.vocab, B = p->B;
  p->G = nq / nkv;
  const int R = (nq + 2 * nkv) * d;

  // attention splits: when contexts are long, spread the key stream over the
  // CUs (about one split per 384 positions, at most one unit per CU).  The
  // CUs that run attention are kept off O and gate/up, whose rows then
  // crowd the others, so the units may take at most 3/8 of the CUs (at
  // least two splits per sequence where one unit per CU allows it): at
  // Llama-1B 8192 the uncapped 22 splits took 0.849 ms per pass, 12 take
  // 0.76.
  int S = opts->kv_splits;
  if (S == 0) {
    const int64_t s1 = ceil_div(p->max_ctx, 384);
    const int64_t per_cu = std::max<int64_t>(1, n_cu / (B * nkv));
    const int64_t cap = std::min<int64_t>(per_cu, std::max<int64_t>(2, 3 * (int64_t)n_cu / (8 * B * nkv)));
    S = (int)std::max<int64_t>(1, std::min(s1, cap));
  }
  p->S = S;

  p->n_levels = LV_PER_LAYER * L + 1;

  // rows per instruction
  int rq = d;
  while (rq > 8 && (R / (rq / 2)) <= n_cu) rq /= 2;
  // O and gate/up slices: on the homogeneous engine at batch 1 the CUs that
  // run a layer's attention get none (the least-loaded CUs take the slices,
  // and attention CUs carry the most bytes).  They finish attention when O's
  // input is about ready; weights they request only then queue behind the
  // gate/up stream the other CUs started during attention, and would hold
  // up the O and gate/up events
  int og_cus = n_cu;
  if ((opts->exec_mode == MK_EXEC_FLAT || opts->exec_mode == MK_EXEC_FLAT_MULTI || opts->exec_mode == MK_EXEC_STREAM ||
       opts->exec_mode == MK_EXEC_QUEUE) &&
      B == 1 &&
      (int64_t)B * nkv * S < n_cu / 2)
    og_cus = n_cu - B * nkv * S;
  // gate/up slices: multiples of 4 hidden units (8 when a batched plan
  // reads the tiled copy, whose tiles hold 8 units' gate and up rows)
  const int ru = mk_plan_tiles(p) ? 8 : 4;
  const int rg = (int)((ceil_div(I, og_cus) + ru - 1) / ru * ru), ro = (int)ceil_div(H, og_cus);
  // LM-head slices; a batched plan of the homogeneous engine reads the
  // tiled copy of the matrix, so its slices start on 16-row tile boundaries
  int rl = (int)ceil_div(V, n_cu);
  if (mk_plan_tiles(p)) rl = (rl + 15) / 16 * 16;
  int rd = (int)ceil_div(H, n_cu);
  // Batched plans of the homogeneous engine split each down-projection slice
  // by its input columns into Sd parts of one staged chunk each (instead of
  // one instruction staging all I columns chunk by chunk): every part stores
  // a partial tile, and the last of them to finish adds the parts in order,
  // plus the residual, and triggers (the attention splits' ticket protocol).
  // Slices are whole 16-row tiles.
  int Sd = 1;
  if ((opts->exec_mode == MK_EXEC_FLAT || opts->exec_mode == MK_EXEC_FLAT_MULTI || opts->exec_mode == MK_EXEC_QUEUE) &&
      B >= MK_MFMA_MIN_BATCH && I % MK_BKC == 0 && I >= 2 * MK_BKC && H % 16 == 0) {
    Sd = I / MK_BKC;
    rd = (int)(ceil_div(ceil_div((int64_t)H * Sd, n_cu), 16) * 16);
  }
  p->Sd = Sd;
  const int n_dslices = (int)ceil_div(H, rd);
  const int dticket0 = S > 1 ? L * B * nkv : 0;
  p->n_lm_parts = (int)ceil_div(V, rl);
  p->n_tickets = dticket0 + (Sd > 1 ? L * n_dslices : 0) + 1;
  const int lm_ticket = p->n_tickets - 1;

  auto blank = [](int op, int layer, int level) {
    MkInstr in;
    std::memset(&in, 0, sizeof in);
    in.op = op;
    in.layer = layer;
    in.level = level;
    in.wait_ev = -1;
    in.sig_ev = -1;
    in.sig_slot = 0;
    in.ticket = -1;
    in.part = -1;
    in.nsplit = 1;
    return in;
  };

  std::vector<double> load(n_cu, 0.0);
  std::vector<char> busy(n_cu, 0);  // CUs left out of a level (this layer's attention CUs)
  auto assign = [&](std::vector<Pending> &lvl, bool skip_busy = false) {
    // spread a level evenly (each CU gets floor or ceil of n / n_cu slices);
    // the CUs with the least bytes so far take the first and largest slices
    std::stable_sort(lvl.begin(), lvl.end(), [](const Pending &a, const Pending &b) { return a.bytes > b.bytes; });
    std::vector<int> order;
    for (int c = 0; c < n_cu; ++c)
      if (!skip_busy || !busy[c]) order.push_back(c);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return load[a] < load[b]; });
    const size_t nc = order.size();
    for (size_t k = 0; k < lvl.size(); ++k) {
      const int c = order[k % nc];
      p->instr.push_back(lvl[k].in);
      p->instr_cu.push_back(c);
      load[c] += lvl[k].bytes;
    }
    lvl.clear();
  };

  double wbytes = 0;
  std::vector<Pending> lvl;
  for (int l = 0; l < L; ++l) {
    const int base = l * LV_PER_LAYER;
    // QKV row slices (each inside one head, hence one kv group)
    {
      for (int r0 = 0; r0 < R; r0 += rq) {
        MkInstr in = blank(MKOP_QKV, l, base + LV_QKV);
        in.r0 = r0;
        in.r1 = std::min(R, r0 + rq);
        lvl.push_back({in, 2.0 * (in.r1 - in.r0) * H});
        wbytes += 2.0 * (in.r1 - in.r0) * H;
      }
      assign(lvl);
    }
    // attention splits
    {
      for (int b = 0; b < B; ++b)
        for (int g = 0; g < nkv; ++g)
          for (int sp = 0; sp < S; ++sp) {
            MkInstr in = blank(MKOP_ATTN, l, base + LV_ATTN);
            in.r0 = b;
            in.r1 = g;
            in.split = sp;
            in.nsplit = S;
            in.ticket = S > 1 ? (l * B + b) * nkv + g : -1;
            lvl.push_back({in, 4.0 * d * (double)ceil_div(p->max_ctx, S)});
          }
      const size_t first = p->instr_cu.size();
      assign(lvl);
      std::fill(busy.begin(), busy.end(), 0);
      for (size_t k = first; k < p->instr_cu.size(); ++k) busy[p->instr_cu[k]] = 1;
    }
    // O projection + residual
    {
      for (int r0 = 0; r0 < H; r0 += ro) {
        MkInstr in = blank(MKOP_OPROJ, l, base + LV_O);
        in.r0 = r0;
        in.r1 = std::min(H, r0 + ro);
        lvl.push_back({in, 2.0 * (in.r1 - in.r0) * nq * d});
        wbytes += 2.0 * (in.r1 - in.r0) * nq * d;
      }
      assign(lvl, og_cus < n_cu);
    }
    // gate/up + SiLU (RMSNorm prologue)
    {
      for (int r0 = 0; r0 < I; r0 += rg) {
        MkInstr in = blank(MKOP_GATEUP, l, base + LV_GU);
        in.r0 = r0;
        in.r1 = std::min(I, r0 + rg);
        lvl.push_back({in, 4.0 * (in.r1 - in.r0) * H});
        wbytes += 4.0 * (in.r1 - in.r0) * H;
      }
      assign(lvl, og_cus < n_cu);
    }
    // down projection + residual
    {
      int k = 0;
      for (int r0 = 0; r0 < H; r0 += rd, ++k)
        for (int sp = 0; sp < Sd; ++sp) {
          MkInstr in = blank(MKOP_DOWN, l, base + LV_DOWN);
          in.r0 = r0;
          in.r1 = std::min(H, r0 + rd);
          in.split = sp;
          in.nsplit = Sd;
          in.ticket = Sd > 1 ? dticket0 + l * n_dslices + k : -1;
          lvl.push_back({in, 2.0 * (in.r1 - in.r0) * I / Sd});
          wbytes += 2.0 * (in.r1 - in.r0) * I / Sd;
        }
      assign(lvl);
    }
    wbytes += 4.0 * H;  // two norm gains
  }
  // LM head + argmax
  {
    int k = 0;
    for (int r0 = 0; r0 < V; r0 += rl, ++k) {
      MkInstr in = blank(MKOP_LMHEAD, L, LV_PER_LAYER * L);
      in.r0 = r0;
      in.r1 = std::min(V, r0 + rl);
      in.ticket = lm_ticket;
      in.part = k;
      lvl.push_back({in, 2.0 * (in.r1 - in.r0) * H});
      wbytes += 2.0 * (in.r1 - in.r0) * H;
    }
    assign(lvl);
    wbytes += 2.0 * H;  // final norm gain
  }
  p->weight_bytes = wbytes;

  // per-CU lists in level order (stable)
  {
    const int n = (int)p->instr.size();
    std::vector<int> order(n);
    for (int i = 0; i < n; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
      if (p->instr_cu[a] != p->instr_cu[b]) return p->instr_cu[a] < p->instr_cu[b];
      return p->instr[a].level < p->instr[b].level;
    });
    std::vector<MkInstr> in2(n);
    std::vector<int32_t> cu2(n);
    for (int i = 0; i < n; ++i) {
      in2[i] = p->instr[order[i]];
      cu2[i] = p->instr_cu[order[i]];
    }
    p->instr.swap(in2);
    p->instr_cu.swap(cu2);
  }
  mk_plan_finalize_lists(p);
  // the events the instructions wait for and trigger, derived from their data
  rc = mk_plan_normalize_events(p);
  if (rc) {
    delete p;
    return rc;
  }
  if (opts->exec_mode == MK_EXEC_STREAM) {
    stream_lds_layout(p);
    if (p->lds_bytes > MK_LDS_TOTAL) {
      delete p;
      return MK_ERR_UNSUPPORTED;
    }
  } else if (opts->exec_mode == MK_EXEC_FLAT || opts->exec_mode == MK_EXEC_FLAT_MULTI ||
             opts->exec_mode == MK_EXEC_QUEUE) {
    p->lds_bytes = lds_requirement(p);
    // the one-sequence ops stage a normalised vector of at most 16 floats per thread
    if (p->lds_bytes > MK_LDS_TOTAL || shape->hidden > 16 * MK_BLOCK) {
      delete p;
      return MK_ERR_UNSUPPORTED;
    }
  } else {
    rc = role_lds_layout(p);
    if (rc) {
      delete p;
      return rc;
    }
  }
  mk_plan_compute_layout(p);
  rc = mk_plan_check(p, false, 0, 0);
  if (rc) {
    delete p;
    return rc;
  }
  p->validated = true;
  *out = p;
  return MK_OK;
}

// ------------------------------------------------------------------ checks

namespace {

enum BufKind { BK_XOUT = 0, BK_QKV = 1, BK_ATTN = 2, BK_XMID = 3, BK_H = 4, BK_N = 5 };

struct Access {
  int buf;  // kind * L + layer
  int64_t lo, hi;
};

struct Checker {
  const mk_plan_t *p;
  int L, H, d, nq, nkv, I, V, R, B, G, S;
  explicit Checker(const mk_plan_t *pp) : p(pp) {
    const mk_model_shape &s = p->shape;
    L = s.n_layers;
    H = s.hidden;
    d = s.head_dim;
    nq = s.n_q_heads;
    nkv = s.n_kv_heads;
    I = s.ffn;
    V = s.vocab;
    R = (nq + 2 * nkv) * d;
    B = p->B;
    G = p->G;
    S = p->S;
  }
  int buf(int kind, int layer) const { return kind * L + layer; }

  void accesses(const MkInstr &in, std::vector<Access> &rd, std::vector<Access> &wr) const {
    rd.clear();
    wr.clear();
    const int l = in.layer;
    switch (in.op) {
      case MKOP_QKV:
        if (l > 0) rd.push_back({buf(BK_XOUT, l - 1), 0, (int64_t)B * H});
        for (int b = 0; b < B; ++b) wr.push_back({buf(BK_QKV, l), (int64_t)b * R + in.r0, (int64_t)b * R + in.r1});
        break;
      case MKOP_ATTN: {
        const int b = in.r0, g = in.r1;
        const int64_t o = (int64_t)b * R;
        rd.push_back({buf(BK_QKV, l), o + (int64_t)g * G * d, o + (int64_t)(g + 1) * G * d});
        rd.push_back({buf(BK_QKV, l), o + (int64_t)nq * d + g * d, o + (int64_t)nq * d + (g + 1) * d});
        rd.push_back({buf(BK_QKV, l), o + (int64_t)(nq + nkv) * d + g * d, o + (int64_t)(nq + nkv) * d + (g + 1) * d});
        const int64_t a = (int64_t)b * nq * d + (int64_t)g * G * d;
        wr.push_back({buf(BK_ATTN, l), a, a + (int64_t)G * d});
        break;
      }
      case MKOP_OPROJ:
        rd.push_back({buf(BK_ATTN, l), 0, (int64_t)B * nq * d});
        for (int b = 0; b < B; ++b) {
          if (l > 0) rd.push_back({buf(BK_XOUT, l - 1), (int64_t)b * H + in.r0, (int64_t)b * H + in.r1});
          wr.push_back({buf(BK_XMID, l), (int64_t)b * H + in.r0, (int64_t)b * H + in.r1});
        }
        break;
      case MKOP_GATEUP:
        rd.push_back({buf(BK_XMID, l), 0, (int64_t)B * H});
        for (int b = 0; b < B; ++b) wr.push_back({buf(BK_H, l), (int64_t)b * I + in.r0, (int64_t)b * I + in.r1});
        break;
      case MKOP_DOWN:
        rd.push_back({buf(BK_H, l), 0, (int64_t)B * I});
        for (int b = 0; b < B; ++b) {
          rd.push_back({buf(BK_XMID, l), (int64_t)b * H + in.r0, (int64_t)b * H + in.r1});
          wr.push_back({buf(BK_XOUT, l), (int64_t)b * H + in.r0, (int64_t)b * H + in.r1});
        }
        break;
      case MKOP_LMHEAD:
        rd.push_back({buf(BK_XOUT, L - 1), 0, (int64_t)B * H});
        break;
      default:
        break;
    }
  }
};

struct Writer {
  int64_t lo, hi;
  int instr;
};

}  // namespace

int mk_plan_check(const mk_plan_t *p, bool simulate, int trials, uint64_t seed) {
  if (!p) return MK_ERR_INVALID_ARG;
  Checker ck(p);
  const int n = (int)p->instr.size();
  const int L = ck.L;
  if ((int)p->instr_cu.size() != n) return MK_ERR_PLAN;
  if ((int)p->cu_begin.size() != p->n_cu + 1 || p->cu_begin[p->n_cu] != n) return MK_ERR_PLAN;
  if ((int)p->ev_count.size() != p->n_events || (int)p->ev_flag_base.size() != p->n_events) return MK_ERR_PLAN;
  // the queue order (when present): a permutation in which every
  // instruction follows all triggers of the event it waits for
  if (!p->queue.empty()) {
    if ((int)p->queue.size() != n) return MK_ERR_PLAN;
    std::vector<int> pos(n, -1), last_trig(std::max(p->n_events, 1), -1);
    for (int k = 0; k < n; ++k) {
      const int i = p->queue[k];
      if (i < 0 || i >= n || pos[i] >= 0) return MK_ERR_PLAN;
      pos[i] = k;
    }
    for (int i = 0; i < n; ++i)
      if (p->instr[i].sig_ev >= 0 && p->instr[i].sig_ev < p->n_events)
        last_trig[p->instr[i].sig_ev] = std::max(last_trig[p->instr[i].sig_ev], pos[i]);
    for (int i = 0; i < n; ++i) {
      const int e = p->instr[i].wait_ev;
      if (e >= 0 && e < p->n_events && last_trig[e] >= pos[i]) return MK_ERR_PLAN;
    }
  }

  // 1. structure: fields in range, lists level-sorted, one token merger
  int n_merge = 0;
  for (int i = 0; i < n; ++i) {
    const MkInstr &in = p->instr[i];
    if (p->instr_cu[i] < 0 || p->instr_cu[i] >= p->n_cu) return MK_ERR_PLAN;
    if (in.level < 0 || in.level >= p->n_levels) return MK_ERR_PLAN;
    if (in.wait_ev < -1 || in.wait_ev >= p->n_events) return MK_ERR_PLAN;
    if (in.sig_ev < -1 || in.sig_ev >= p->n_events) return MK_ERR_PLAN;
    if (in.sig_ev >= 0 && (in.sig_slot < 0 || in.sig_slot >= p->ev_count[in.sig_ev])) return MK_ERR_PLAN;
    if (in.ticket < -1 || in.ticket >= p->n_tickets) return MK_ERR_PLAN;
    const int l = in.layer;
    switch (in.op) {
      case MKOP_QKV: {
        if (l < 0 || l >= L || in.r0 < 0 || in.r1 > ck.R || in.r0 >= in.r1) return MK_ERR_PLAN;
        // a slice lies inside one of the q, k and v weight matrices
        const int qd = ck.nq * ck.d, kd = ck.nkv * ck.d;
        auto part_of = [&](int r) { return r < qd ? 0 : r < qd + kd ? 1 : 2; };
        if (part_of(in.r0) != part_of(in.r1 - 1)) return MK_ERR_PLAN;
        break;
      }
      case MKOP_ATTN:
        if (l < 0 || l >= L || in.r0 < 0 || in.r0 >= ck.B || in.r1 < 0 || in.r1 >= ck.nkv) return MK_ERR_PLAN;
        if (in.nsplit != p->S || in.split < 0 || in.split >= in.nsplit) return MK_ERR_PLAN;
        if ((p->S > 1) != (in.ticket >= 0)) return MK_ERR_PLAN;
        break;
      case MKOP_OPROJ:
        if (l < 0 || l >= L || in.r0 < 0 || in.r1 > ck.H || in.r0 >= in.r1) return MK_ERR_PLAN;
        break;
      case MKOP_DOWN:
        if (l < 0 || l >= L || in.r0 < 0 || in.r1 > ck.H || in.r0 >= in.r1) return MK_ERR_PLAN;
        if (in.nsplit != p->Sd || in.split < 0 || in.split >= in.nsplit) return MK_ERR_PLAN;
        if ((p->Sd > 1) != (in.ticket >= 0)) return MK_ERR_PLAN;
        if (p->Sd > 1 && (in.r0 % 16 || ck.I % (p->Sd * MK_BKC) != 0 || ck.I / p->Sd != MK_BKC)) return MK_ERR_PLAN;
        break;
      case MKOP_GATEUP:
        if (l < 0 || l >= L || in.r0 < 0 || in.r1 > ck.I || in.r0 >= in.r1) return MK_ERR_PLAN;
        break;
      case MKOP_LMHEAD:
        if (in.r0 < 0 || in.r1 > ck.V || in.r0 >= in.r1 || in.ticket < 0) return MK_ERR_PLAN;
        if (in.part < 0 || in.part >= p->n_lm_parts) return MK_ERR_PLAN;
        if (in.split != 0 && in.split != 1) return MK_ERR_PLAN;
        n_merge += in.split;
        break;
      default:
        return MK_ERR_PLAN;
    }
  }
  if (n_merge != 1) return MK_ERR_PLAN;
  for (int c = 0; c < p->n_cu; ++c)
    for (int i = p->cu_begin[c] + 1; i < p->cu_begin[c + 1]; ++i)
      if (p->instr[i].level < p->instr[i - 1].level) return MK_ERR_PLAN;

  // 2. events: trigger counts match, flag slots distinct, triggers strictly
  //    below every waiter's level (otherwise a wait could never be met)
  std::vector<int> trig(p->n_events, 0), min_wait(p->n_events, 1 << 30), max_trig(p->n_events, -1);
  std::vector<std::vector<char>> slot_used(p->n_events);
  for (int e = 0; e < p->n_events; ++e) slot_used[e].assign(std::max(p->ev_count[e], 1), 0);
  std::vector<int> attn_units(p->n_events, 0);
  for (int i = 0; i < n; ++i) {
    const MkInstr &in = p->instr[i];
    if (in.wait_ev >= 0) min_wait[in.wait_ev] = std::min(min_wait[in.wait_ev], in.level);
    if (in.sig_ev >= 0) {
      max_trig[in.sig_ev] = std::max(max_trig[in.sig_ev], in.level);
      if (in.op == MKOP_ATTN || (in.op == MKOP_DOWN && p->Sd > 1)) {
        if (in.split == 0) attn_units[in.sig_ev]++;  // one trigger per attention unit / down slice
      } else {
        if (slot_used[in.sig_ev][in.sig_slot]) return MK_ERR_PLAN;
        slot_used[in.sig_ev][in.sig_slot] = 1;
        trig[in.sig_ev]++;
      }
    }
  }
  for (int e = 0; e < p->n_events; ++e) {
    int t = trig[e] + attn_units[e];
    if (t != p->ev_count[e]) return MK_ERR_PLAN;
    if (min_wait[e] < (1 << 30) && max_trig[e] >= min_wait[e]) return MK_ERR_PLAN;
    if (min_wait[e] < (1 << 30) && t == 0) return MK_ERR_PLAN;
  }
  // every attention unit has all S splits
  {
    std::vector<int> cnt((size_t)L * ck.B * ck.nkv, 0);
    for (int i = 0; i < n; ++i) {
      const MkInstr &in = p->instr[i];
      if (in.op == MKOP_ATTN) cnt[((size_t)in.layer * ck.B + in.r0) * ck.nkv + in.r1] |= (1 << std::min(in.split, 30));
    }
    int full = p->S >= 31 ? -1 : (1 << p->S) - 1;
    if (p->S < 31)
      for (int v : cnt)
        if (v != full) return MK_ERR_PLAN;
  }

  // every down slice has all Sd parts
  if (p->Sd > 1) {
    std::map<std::pair<int, int>, int> parts;
    for (int i = 0; i < n; ++i) {
      const MkInstr &in = p->instr[i];
      if (in.op == MKOP_DOWN) parts[{in.layer, in.r0}] |= 1 << std::min(in.split, 30);
    }
    const int full = p->Sd >= 31 ? -1 : (1 << p->Sd) - 1;
    for (auto &kv : parts)
      if (kv.second != full) return MK_ERR_PLAN;
  }

  // 3. writes: every output slice written exactly once per step
  std::vector<std::vector<Writer>> writers(BK_N * L);
  std::vector<Access> rd, wr;
  for (int i = 0; i < n; ++i) {
    ck.accesses(p->instr[i], rd, wr);
    for (auto &a : wr) writers[a.buf].push_back({a.lo, a.hi, i});
  }
  for (int k = 0; k < BK_N; ++k)
    for (int l = 0; l < L; ++l) {
      auto &w = writers[k * L + l];
      std::sort(w.begin(), w.end(), [](const Writer &a, const Writer &b) {
        return a.lo != b.lo ? a.lo < b.lo : a.instr < b.instr;
      });
      int64_t size = 0;
      switch (k) {
        case BK_XOUT: size = (int64_t)ck.B * ck.H; break;
        case BK_QKV: size = (int64_t)ck.B * ck.R; break;
        case BK_ATTN: size = (int64_t)ck.B * ck.nq * ck.d; break;
        case BK_XMID: size = (int64_t)ck.B * ck.H; break;
        case BK_H: size = (int64_t)ck.B * ck.I; break;
      }
      int64_t covered = 0;
      for (size_t j = 0; j < w.size(); ++j) {
        if (k == BK_ATTN || (k == BK_XOUT && p->Sd > 1)) {  // all splits / parts of one unit share its slice
          if (w[j].lo < covered && !(j > 0 && w[j].lo == w[j - 1].lo && w[j].hi == w[j - 1].hi)) return MK_ERR_PLAN;
          covered = std::max(covered, w[j].hi);
          continue;
        }
        if (w[j].lo != covered) return MK_ERR_PLAN;  // gap or overlap
        covered = w[j].hi;
      }
      if (covered != size) return MK_ERR_PLAN;
    }
  // LM rows covered exactly once
  {
    std::vector<std::pair<int, int>> lm;
    for (int i = 0; i < n; ++i)
      if (p->instr[i].op == MKOP_LMHEAD) lm.push_back({p->instr[i].r0, p->instr[i].r1});
    std::sort(lm.begin(), lm.end());
    int c = 0;
    for (auto &r : lm) {
      if (r.first != c) return MK_ERR_PLAN;
      c = r.second;
    }
    if (c != ck.V) return MK_ERR_PLAN;
  }

  // 4. read-after-write: every writer of a slice an instruction reads
  //    happens-before it (program order on a CU + event edges)
  std::vector<int> topo(n);
  for (int i = 0; i < n; ++i) topo[i] = i;
  std::stable_sort(topo.begin(), topo.end(), [&](int a, int b) {
    if (p->instr[a].level != p->instr[b].level) return p->instr[a].level < p->instr[b].level;
    return a < b;
  });
  const size_t words = ((size_t)n + 63) / 64;
  std::vector<uint64_t> anc((size_t)n * words, 0), evanc((size_t)p->n_events * words, 0);
  std::vector<int> prev_on_cu(n, -1);
  for (int c = 0; c < p->n_cu; ++c)
    for (int i = p->cu_begin[c] + 1; i < p->cu_begin[c + 1]; ++i) prev_on_cu[i] = i - 1;
  // process level by level: event ancestor sets of a level are complete before
  // any waiter (strictly higher level) reads them
  size_t t = 0;
  while (t < topo.size()) {
    const int lv = p->instr[topo[t]].level;
    size_t t1 = t;
    while (t1 < topo.size() && p->instr[topo[t1]].level == lv) ++t1;
    // within a level, program order predecessors may be in the same level:
    // visit in CU-list order (index order) which topo preserves
    for (size_t k = t; k < t1; ++k) {
      int i = topo[k];
      uint64_t *a = &anc[(size_t)i * words];
      int pr = prev_on_cu[i];
      if (pr >= 0) {
        const uint64_t *b = &anc[(size_t)pr * words];
        for (size_t w = 0; w < words; ++w) a[w] |= b[w];
        a[pr / 64] |= 1ull << (pr % 64);
      }
      int e = p->instr[i].wait_ev;
      if (e >= 0) {
        const uint64_t *b = &evanc[(size_t)e * words];
        for (size_t w = 0; w < words; ++w) a[w] |= b[w];
      }
    }
    for (size_t k = t; k < t1; ++k) {
      int i = topo[k];
      int e = p->instr[i].sig_ev;
      if (e >= 0) {
        uint64_t *b = &evanc[(size_t)e * words];
        const uint64_t *a = &anc[(size_t)i * words];
        for (size_t w = 0; w < words; ++w) b[w] |= a[w];
        b[i / 64] |= 1ull << (i % 64);
      }
    }
    t = t1;
  }
  std::vector<std::vector<int>> producers(simulate ? n : 0);
  for (int i = 0; i < n; ++i) {
    ck.accesses(p->instr[i], rd, wr);
    const uint64_t *a = &anc[(size_t)i * words];
    for (auto &r : rd) {
      auto &w = writers[r.buf];
      // writers sorted by lo; scan those overlapping [r.lo, r.hi)
      auto it = std::lower_bound(w.begin(), w.end(), r.lo, [](const Writer &x, int64_t v) { return x.hi <= v; });
      // lower_bound on hi requires hi sorted, which holds for disjoint slices and
      // for the shared attention slices (equal ranges are adjacent)
      for (; it != w.end() && it->lo < r.hi; ++it) {
        if (it->hi <= r.lo) continue;
        int wi = it->instr;
        if (!((a[wi / 64] >> (wi % 64)) & 1)) return MK_ERR_PLAN;
        if (simulate) producers[i].push_back(wi);
      }
    }
  }

  // 5. optional: random interleavings of the lists with counters, tickets and
  //    producer checks, no arithmetic
  if (simulate) {
    std::mt19937_64 rng(seed);
    for (int tr = 0; tr < trials; ++tr) {
      std::vector<int> pc(p->n_cu), ctr(p->n_events, 0), tick(std::max(p->n_tickets, 1), 0);
      std::vector<char> done(n, 0);
      std::vector<std::vector<int>> waiting(p->n_events);
      std::vector<int> ready;
      for (int c = 0; c < p->n_cu; ++c) pc[c] = p->cu_begin[c];
      auto park_or_ready = [&](int c) {
        if (pc[c] >= p->cu_begin[c + 1]) return;
        const MkInstr &in = p->instr[pc[c]];
        if (in.wait_ev < 0 || ctr[in.wait_ev] >= p->ev_count[in.wait_ev])
          ready.push_back(c);
        else
          waiting[in.wait_ev].push_back(c);
      };
      for (int c = 0; c < p->n_cu; ++c) park_or_ready(c);
      int executed = 0;
      while (!ready.empty()) {
        size_t k = rng() % ready.size();
        int c = ready[k];
        ready[k] = ready.back();
        ready.pop_back();
        int i = pc[c];
        for (int pi : producers[i])
          if (!done[pi]) return MK_ERR_PLAN;
        done[i] = 1;
        ++executed;
        const MkInstr &in = p->instr[i];
        int fire = -1;
        if ((in.op == MKOP_ATTN || in.op == MKOP_DOWN) && in.ticket >= 0) {
          if (++tick[in.ticket] == in.nsplit) fire = in.sig_ev;
        } else {
          fire = in.sig_ev;
        }
        if (fire >= 0) {
          if (++ctr[fire] == p->ev_count[fire]) {
            for (int wc : waiting[fire]) ready.push_back(wc);
            waiting[fire].clear();
          }
        }
        pc[c]++;
        park_or_ready(c);
      }
      if (executed != n) return MK_ERR_PLAN;  // some CU never got past a wait: deadlock
    }
  }
  return MK_OK;
}

// ------------------------------------------------------- event normalisation
//
// The megakernel page's Q&A on MPK describes how a task graph's events are
// normalised: each task waits for at most one event and triggers at most
// one, events are fused by their predecessor and successor sets, and the
// graph is linearised breadth-first so that the tasks one event releases
// have contiguous indices.  mk_events_normalize does this for any DAG given
// as raw predecessor lists:
//   1. topological order (Kahn); a cycle among the raw edges is an error;
//   2. transitive reduction: an edge q -> t is dropped when q is already an
//      ancestor of another predecessor of t (ancestor bitsets filled in
//      topological order; the union over a predecessor list is cached, since
//      whole levels of tasks share one);
//   3. fusion by predecessor set: tasks with the same reduced predecessors
//      wait for one event;
//   4. fusion by successor set: two events that share a predecessor are
//      merged (union-find), so every task triggers at most one; a merged
//      event one of whose waiters precedes one of its producers would never
//      fire, and is reported;
//   5. breadth-first linearisation from the source tasks (ties by rank): an
//      event fires once its last predecessor has been visited and appends
//      its waiters together; events are numbered in firing order, trigger
//      slots in visiting order.

namespace {
struct UnionFind {
  std::vector<int> p;
  explicit UnionFind(int n) : p(n) {
    for (int i = 0; i < n; ++i) p[i] = i;
  }
  int find(int x) {
    while (p[x] != x) x = p[x] = p[p[x]];
    return x;
  }
  void join(int a, int b) {
    a = find(a);
    b = find(b);
    if (a != b) p[std::max(a, b)] = std::min(a, b);
  }
};
}  // namespace

extern "C" int mk_events_normalize(int32_t nt, const int32_t *pred_begin, const int32_t *pred_list, const int64_t *rank,
                                   uint32_t flags, int32_t *wait_event, int32_t *trigger_event, int32_t *trigger_slot,
                                   int32_t *event_count, int32_t *order_out, int32_t *n_events_out) {
  if (nt < 0 || (nt > 0 && (!pred_begin || !wait_event || !trigger_event || !trigger_slot || !event_count ||
                            !order_out)) || !n_events_out)
    return MK_ERR_INVALID_ARG;
  if (nt == 0) {
    *n_events_out = 0;
    return MK_OK;
  }
  if (pred_begin[0] != 0) return MK_ERR_INVALID_ARG;
  // raw predecessor lists, sorted and without duplicates
  std::vector<std::vector<int>> raw(nt);
  for (int t = 0; t < nt; ++t) {
    if (pred_begin[t + 1] < pred_begin[t]) return MK_ERR_INVALID_ARG;
    for (int k = pred_begin[t]; k < pred_begin[t + 1]; ++k) {
      const int q = pred_list[k];
      if (q < 0 || q >= nt) return MK_ERR_INVALID_ARG;
      if (q == t) return MK_ERR_PLAN;
      raw[t].push_back(q);
    }
    std::sort(raw[t].begin(), raw[t].end());
    raw[t].erase(std::unique(raw[t].begin(), raw[t].end()), raw[t].end());
  }
  // 1. topological order
  std::vector<std::vector<int>> succ(nt);
  std::vector<int> indeg(nt, 0), topo;
  for (int t = 0; t < nt; ++t) {
    for (int q : raw[t]) succ[q].push_back(t);
    indeg[t] = (int)raw[t].size();
  }
  topo.reserve(nt);
  for (int t = 0; t < nt; ++t)
    if (!indeg[t]) topo.push_back(t);
  for (size_t k = 0; k < topo.size(); ++k)
    for (int s : succ[topo[k]])
      if (--indeg[s] == 0) topo.push_back(s);
  if ((int)topo.size() != nt) return MK_ERR_PLAN;

  // 2. ancestors and transitive reduction
  const size_t words = ((size_t)nt + 63) / 64;
  std::vector<uint64_t> anc((size_t)nt * words, 0);
  std::map<std::vector<int>, std::vector<uint64_t>> through_of;  // predecessor list -> union of their ancestors
  std::vector<std::vector<int>> preds(nt);
  const bool reduce = !(flags & 1u);
  for (int t : topo) {
    if (raw[t].empty()) continue;
    auto it = through_of.find(raw[t]);
    if (it == through_of.end()) {
      std::vector<uint64_t> u(words, 0);
      for (int q : raw[t]) {
        const uint64_t *a = &anc[(size_t)q * words];
        for (size_t w = 0; w < words; ++w) u[w] |= a[w];
      }
      it = through_of.emplace(raw[t], std::move(u)).first;
    }
    const std::vector<uint64_t> &through = it->second;
    uint64_t *a = &anc[(size_t)t * words];
    for (size_t w = 0; w < words; ++w) a[w] = through[w];
    for (int q : raw[t]) {
      a[q / 64] |= 1ull << (q % 64);
      if (!reduce || !((through[q / 64] >> (q % 64)) & 1)) preds[t].push_back(q);
    }
  }
  auto is_anc = [&](int x, int of) { return (anc[(size_t)of * words + x / 64] >> (x % 64)) & 1; };

  // 3. fusion by predecessor set
  std::map<std::vector<int>, int> ev_of_set;
  std::vector<std::vector<int>> ev_preds, ev_waiters;
  std::vector<int> wait_of(nt, -1);
  for (int t = 0; t < nt; ++t) {
    if (preds[t].empty()) continue;
    auto it = ev_of_set.find(preds[t]);
    int e;
    if (it == ev_of_set.end()) {
      e = (int)ev_preds.size();
      ev_of_set[preds[t]] = e;
      ev_preds.push_back(preds[t]);
      ev_waiters.emplace_back();
    } else {
      e = it->second;
    }
    wait_of[t] = e;
    ev_waiters[e].push_back(t);
  }
  // 4. fusion by successor set
  const int ne0 = (int)ev_preds.size();
  UnionFind uf(std::max(ne0, 1));
  std::vector<int> trig_first(nt, -1);
  for (int e = 0; e < ne0; ++e)
    for (int q : ev_preds[e]) {
      if (trig_first[q] < 0) trig_first[q] = e;
      else uf.join(trig_first[q], e);
    }
  std::vector<int> root_id(std::max(ne0, 1), -1);
  std::vector<std::vector<int>> mpreds, mwaiters;
  for (int e = 0; e < ne0; ++e) {
    const int r = uf.find(e);
    if (root_id[r] < 0) {
      root_id[r] = (int)mpreds.size();
      mpreds.emplace_back();
      mwaiters.emplace_back();
    }
    const int m = root_id[r];
    mpreds[m].insert(mpreds[m].end(), ev_preds[e].begin(), ev_preds[e].end());
    mwaiters[m].insert(mwaiters[m].end(), ev_waiters[e].begin(), ev_waiters[e].end());
  }
  const int ne = (int)mpreds.size();
  std::vector<int> trig_of(nt, -1);
  for (int m = 0; m < ne; ++m) {
    auto &pr = mpreds[m];
    std::sort(pr.begin(), pr.end());
    pr.erase(std::unique(pr.begin(), pr.end()), pr.end());
    for (int q : pr) trig_of[q] = m;
    for (int w : mwaiters[m])
      for (int q : pr)
        if (q == w || is_anc(w, q)) return MK_ERR_PLAN;
  }
  for (int t = 0; t < nt; ++t)
    if (wait_of[t] >= 0) wait_of[t] = root_id[uf.find(wait_of[t])];

  // 5. breadth-first linearisation
  std::vector<int> remaining(ne);
  for (int m = 0; m < ne; ++m) remaining[m] = (int)mpreds[m].size();
  auto before = [&](int x, int y) {
    const int64_t rx = rank ? rank[x] : x, ry = rank ? rank[y] : y;
    return rx != ry ? rx < ry : x < y;
  };
  std::vector<int> order;
  order.reserve(nt);
  for (int t = 0; t < nt; ++t)
    if (wait_of[t] < 0) order.push_back(t);
  std::sort(order.begin(), order.end(), before);
  std::vector<int> ev_num(ne, -1), slot(nt, 0), ev_n(ne, 0);
  int fired = 0;
  for (size_t k = 0; k < order.size(); ++k) {
    const int t = order[k];
    const int m = trig_of[t];
    if (m < 0) continue;
    slot[t] = ev_n[m]++;
    if (--remaining[m] == 0) {
      ev_num[m] = fired++;
      std::vector<int> ws = mwaiters[m];
      std::sort(ws.begin(), ws.end(), before);
      order.insert(order.end(), ws.begin(), ws.end());
    }
  }
  if ((int)order.size() != nt || fired != ne) return MK_ERR_PLAN;
  for (int t = 0; t < nt; ++t) {
    wait_event[t] = wait_of[t] >= 0 ? ev_num[wait_of[t]] : -1;
    trigger_event[t] = trig_of[t] >= 0 ? ev_num[trig_of[t]] : -1;
    trigger_slot[t] = slot[t];
    order_out[t] = order[t];
  }
  for (int m = 0; m < ne; ++m) event_count[ev_num[m]] = (int)mpreds[m].size();
  *n_events_out = ne;
  return MK_OK;
}

// The plan's tasks are its instructions, except that the splits of one
// attention unit, and the parts of one down slice, are one task (only the
// last arriver triggers); the
// raw edges run from the writers of every slice an instruction reads.
int mk_plan_normalize_events(mk_plan_t *p) {
  if (!p) return MK_ERR_INVALID_ARG;
  Checker ck(p);
  const int n = (int)p->instr.size();
  std::vector<int> task_of(n, -1), first_instr;
  std::map<std::tuple<int, int, int, int>, int> attn_task;
  for (int i = 0; i < n; ++i) {
    const MkInstr &in = p->instr[i];
    if (in.op == MKOP_ATTN || (in.op == MKOP_DOWN && in.nsplit > 1)) {
      auto key = std::make_tuple(in.op, in.layer, in.r0, in.r1);
      auto it = attn_task.find(key);
      if (it != attn_task.end()) {
        task_of[i] = it->second;
        continue;
      }
      attn_task[key] = (int)first_instr.size();
    }
    task_of[i] = (int)first_instr.size();
    first_instr.push_back(i);
  }
  const int nt = (int)first_instr.size();
  std::vector<std::vector<Writer>> writers(BK_N * ck.L);
  std::vector<Access> rd, wr;
  for (int t = 0; t < nt; ++t) {
    ck.accesses(p->instr[first_instr[t]], rd, wr);
    for (auto &a : wr) writers[a.buf].push_back({a.lo, a.hi, t});
  }
  for (auto &w : writers)
    std::sort(w.begin(), w.end(), [](const Writer &a, const Writer &b) { return a.lo != b.lo ? a.lo < b.lo : a.instr < b.instr; });
  std::vector<int32_t> begin(nt + 1, 0), list;
  std::vector<int64_t> rank(nt);
  std::vector<int> seen(nt, -1);  // a task writes one slice per sequence: list it once per reader
  for (int t = 0; t < nt; ++t) {
    ck.accesses(p->instr[first_instr[t]], rd, wr);
    for (auto &r : rd) {
      const auto &ws = writers[r.buf];  // disjoint slices sorted by lo
      auto it = std::lower_bound(ws.begin(), ws.end(), r.lo, [](const Writer &w, int64_t v) { return w.lo < v; });
      if (it != ws.begin() && std::prev(it)->hi > r.lo) --it;
      int64_t covered = r.lo;
      for (; it != ws.end() && it->lo < r.hi; ++it) {
        if (it->hi <= r.lo) continue;
        if (seen[it->instr] != t) {
          seen[it->instr] = t;
          list.push_back(it->instr);
        }
        if (it->lo <= covered) covered = std::max(covered, it->hi);
      }
      if (covered < r.hi) return MK_ERR_PLAN;  // part of the slice has no writer
    }
    begin[t + 1] = (int32_t)list.size();
    rank[t] = (int64_t)p->instr[first_instr[t]].level * n + first_instr[t];  // level, then list order
  }
  std::vector<int32_t> wait(nt), trig(nt), slot(nt), count(nt), order(nt);
  int32_t ne = 0;
  const int rc = mk_events_normalize(nt, begin.data(), list.data(), rank.data(), 0, wait.data(), trig.data(),
                                     slot.data(), count.data(), order.data(), &ne);
  if (rc != MK_OK) return rc;
  p->n_events = ne;
  p->ev_count.assign(count.begin(), count.begin() + ne);
  p->ev_flag_base.assign(ne, 0);
  int acc = 0;
  for (int e = 0; e < ne; ++e) {
    p->ev_flag_base[e] = acc;
    acc += p->ev_count[e];
  }
  p->n_flags = acc;
  std::vector<std::vector<int>> members(nt);
  for (int i = 0; i < n; ++i) members[task_of[i]].push_back(i);
  p->queue.clear();
  for (int k = 0; k < nt; ++k) {
    const int t = order[k];
    for (int i : members[t]) {
      MkInstr &in = p->instr[i];
      in.wait_ev = wait[t];
      in.sig_ev = trig[t];
      in.sig_slot = trig[t] >= 0 ? slot[t] : 0;
      p->queue.push_back(i);
    }
  }
  // the LM-head instruction that merges the greedy tokens: the last one
  // handed out, so a work-queue workgroup that runs it holds nothing else
  for (MkInstr &in : p->instr)
    if (in.op == MKOP_LMHEAD) in.split = 0;
  if (p->queue.empty() || p->instr[p->queue.back()].op != MKOP_LMHEAD) return MK_ERR_PLAN;
  p->instr[p->queue.back()].split = 1;
  return MK_OK;
}
