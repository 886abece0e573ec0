// C ABI of libmk.so: plans, contexts, weight binding, the decode step and
// the measurement entry points.  See include/mk.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "mk.h"
#include "mk_launch.h"
#include "planner.h"

struct mk_ctx {
  mk_plan_t plan;              // private copy
  char *ws = nullptr;        // device workspace base
  size_t ws_bytes = 0;
  MkProgram prog{};          // host image of the device MkProgram
  MkProgram prog_odd{};      // sentinel mode: the odd-step record of the homogeneous engine
  std::vector<MkLayerW> layers;
  std::vector<MkRowTab> rowtab;  // stream engine row table (host staging)
  std::vector<float> rope;   // host staging kept alive for async uploads
  bool weights = false;
  bool poisoned = false;
  int64_t epoch = 0;
  int device = 0;
  uint64_t scratch_gen = 0;  // non-zero: the workspace is the library's static scratch
};

static inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The megakernel asks for more than half of a CU's 160 KiB LDS so that the
// dispatcher can place only one of its workgroups on each CU.
static inline int mega_lds(const mk_plan_t *p) { return std::max(p->lds_bytes, 80 * 1024 + 256); }
// dynamic LDS a plan's kernel is launched with
static inline int launch_lds(const mk_plan_t *p) {
  const int m = p->opts.exec_mode;
  return m == MK_EXEC_FLAT || m == MK_EXEC_FLAT_MULTI || m == MK_EXEC_STREAM || m == MK_EXEC_QUEUE ? mega_lds(p)
                                                                                                    : p->lds_bytes;
}

extern "C" {

const char *mk_strerror(int code) {
  switch (code) {
    case MK_OK: return "ok";
    case MK_ERR_INVALID_ARG: return "invalid argument";
    case MK_ERR_SHAPE: return "unsupported model shape";
    case MK_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MK_ERR_NOT_RESIDENT: return "grid exceeds the co-resident workgroup limit";
    case MK_ERR_CTX_OVERFLOW: return "batch or workspace exceeds the plan";
    case MK_ERR_HIP: return "HIP runtime error";
    case MK_ERR_TIMEOUT: return "device watchdog expired while waiting on a dependency";
    case MK_ERR_INPUT: return "token id or position out of range";
    case MK_ERR_PLAN: return "plan validation failed";
    case MK_ERR_STATE: return "context poisoned by an earlier device error; reset it";
    case MK_ERR_UNSUPPORTED: return "option combination not supported";
    case MK_ERR_SCRATCH: return "plan workspace exceeds the library's static scratch (32 MiB)";
    default: return "unknown error";
  }
}

int mk_plan_create(const mk_model_shape *shape, const mk_plan_opts *opts, mk_plan_t **out) {
  if (!shape || !opts || !out) return MK_ERR_INVALID_ARG;
  int n_cu = opts->num_cus;
  if (n_cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MK_ERR_HIP;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MK_ERR_HIP;
  }
  return mk_plan_build(shape, opts, n_cu, out);
}

int mk_plan(const mk_model_shape *shape, const mk_plan_opts *opts, mk_plan_t **out) {
  return mk_plan_create(shape, opts, out);
}

int mk_plan_validate(const mk_plan_t *p) { return p ? mk_plan_check(p, false, 0, 0) : MK_ERR_INVALID_ARG; }

int mk_plan_simulate(const mk_plan_t *p, int32_t n_trials, uint64_t seed) {
  if (!p || n_trials < 0) return MK_ERR_INVALID_ARG;
  return mk_plan_check(p, true, n_trials, seed);
}

int mk_plan_sizes(const mk_plan_t *p, size_t *ws, size_t *kv, size_t *logits, size_t *n_instr) {
  if (!p) return MK_ERR_INVALID_ARG;
  const mk_model_shape &s = p->shape;
  if (ws) *ws = p->lay.total;
  if (kv) *kv = (size_t)s.n_layers * 2 * p->B * s.n_kv_heads * (size_t)p->max_ctx * s.head_dim * 2;
  if (logits) *logits = (size_t)p->B * s.vocab * 4;
  if (n_instr) *n_instr = p->instr.size();
  return MK_OK;
}

int mk_plan_get_info(const mk_plan_t *p, mk_plan_info *o) {
  if (!p || !o) return MK_ERR_INVALID_ARG;
  std::memset(o, 0, sizeof *o);
  o->num_cus = p->n_cu;
  o->n_instructions = (int32_t)p->instr.size();
  o->n_levels = p->n_levels;
  o->n_counters = p->n_events;
  o->kv_splits = p->S;
  int mx = 0;
  for (int c = 0; c < p->n_cu; ++c) mx = std::max(mx, p->cu_begin[c + 1] - p->cu_begin[c]);
  o->max_instr_per_cu = mx;
  o->block_threads = MK_BLOCK;
  o->lds_bytes = p->lds_bytes;
  o->sync_mode = p->opts.sync_mode;
  o->exec_mode = p->opts.exec_mode;
  o->max_batch = p->B;
  o->max_ctx = p->max_ctx;
  o->weight_bytes = p->weight_bytes;
  return MK_OK;
}

int mk_plan_export(const mk_plan_t *p, mk_instr_desc *out, size_t cap, size_t *n_out) {
  if (!p) return MK_ERR_INVALID_ARG;
  if (n_out) *n_out = p->instr.size();
  if (!out) return MK_OK;
  for (int c = 0; c < p->n_cu; ++c)
    for (int i = p->cu_begin[c]; i < p->cu_begin[c + 1]; ++i) {
      if ((size_t)i >= cap) return MK_OK;
      const MkInstr &in = p->instr[i];
      mk_instr_desc &d = out[i];
      d.cu = c;
      d.slot = i - p->cu_begin[c];
      d.op = in.op;
      d.layer = in.layer;
      d.level = in.level;
      d.r0 = in.r0;
      d.r1 = in.r1;
      d.split = in.split;
      d.n_splits = in.nsplit;
      d.wait_event = in.wait_ev;
      d.wait_count = in.wait_ev >= 0 ? p->ev_count[in.wait_ev] : 0;
      d.signal_event = in.sig_ev;
    }
  return MK_OK;
}

int mk_plan_get_queue(const mk_plan_t *p, int32_t *out, size_t cap, size_t *n_out) {
  if (!p) return MK_ERR_INVALID_ARG;
  if (n_out) *n_out = p->queue.size();
  for (size_t i = 0; out && i < cap && i < p->queue.size(); ++i) out[i] = p->queue[i];
  return MK_OK;
}

void mk_plan_destroy(mk_plan_t *p) { delete p; }

// Host-side test hook: replace the instruction list of a plan with `n`
// descriptors (cu/slot/op/layer/level/rows/split/wait/signal as exported).
// Slots, tickets and partial indices are re-derived; the plan is then only
// as valid as mk_plan_validate says.
int mk_plan_set_instructions(mk_plan_t *p, const mk_instr_desc *d, size_t n) {
  if (!p || (!d && n)) return MK_ERR_INVALID_ARG;
  std::vector<std::pair<std::pair<int, int>, size_t>> order;
  for (size_t i = 0; i < n; ++i) order.push_back({{d[i].cu, d[i].slot}, i});
  std::sort(order.begin(), order.end());
  std::vector<MkInstr> ins;
  std::vector<int32_t> cus;
  std::vector<int> slots(p->n_events, 0);
  int lm = 0;
  const mk_model_shape &s = p->shape;
  for (auto &o : order) {
    const mk_instr_desc &x = d[o.second];
    if (x.cu < 0 || x.cu >= p->n_cu) return MK_ERR_PLAN;
    MkInstr in;
    std::memset(&in, 0, sizeof in);
    in.op = x.op;
    in.layer = x.layer;
    in.level = x.level;
    in.r0 = x.r0;
    in.r1 = x.r1;
    in.split = x.split;
    in.nsplit = x.n_splits;
    in.wait_ev = x.wait_event;
    in.sig_ev = x.signal_event;
    in.ticket = -1;
    in.part = -1;
    if (in.op == MKOP_ATTN) {
      in.sig_slot = x.r0 * s.n_kv_heads + x.r1;
      in.ticket = p->S > 1 ? (x.layer * p->B + x.r0) * s.n_kv_heads + x.r1 : -1;
    } else if (in.op == MKOP_LMHEAD) {
      in.ticket = p->n_tickets - 1;
      in.part = lm++;
    } else if (in.sig_ev >= 0 && in.sig_ev < p->n_events) {
      in.sig_slot = slots[in.sig_ev]++;
    }
    ins.push_back(in);
    cus.push_back(x.cu);
  }
  p->instr.swap(ins);
  p->instr_cu.swap(cus);
  p->queue.clear();  // indices of the previous instruction array
  mk_plan_finalize_lists(p);
  mk_plan_compute_layout(p);
  p->validated = mk_plan_check(p, false, 0, 0) == MK_OK;
  return MK_OK;
}

// ------------------------------------------------------------------ ctx

static void build_rope(const mk_plan_t &p, std::vector<float> &rope) {
  // angle(pos, i) = pos * theta^(-2i/d), evaluated in double, stored as fp32 (cos, sin)
  const int d = p.shape.head_dim, half = d / 2;
  rope.resize((size_t)p.max_ctx * d);
  std::vector<double> inv(half);
  for (int i = 0; i < half; ++i) inv[i] = std::pow(p.shape.rope_theta, -2.0 * i / d);
  for (int t = 0; t < p.max_ctx; ++t)
    for (int i = 0; i < half; ++i) {
      double a = (double)t * inv[i];
      rope[(size_t)t * d + 2 * i] = (float)std::cos(a);
      rope[(size_t)t * d + 2 * i + 1] = (float)std::sin(a);
    }
}

// Upload the program record(s).  In sentinel mode the activations have two
// copies (one per step parity); the role engine offsets into them itself,
// while the homogeneous engine gets a second record whose activation
// pointers name the odd copy.  Each record's act_other is the copy its steps
// reset for the step after.
static int upload_prog(mk_ctx *c, hipStream_t st) {
  MkProgram &P = c->prog;
  const int64_t ps = P.par_stride;
  if (c->plan.opts.sync_mode == MK_SYNC_SENTINEL) P.act_other = P.qkv + ps;
  if (hipMemcpyAsync(c->ws + c->plan.lay.prog, &P, sizeof(MkProgram), hipMemcpyHostToDevice, st) != hipSuccess)
    return MK_ERR_HIP;
  if (c->plan.opts.sync_mode == MK_SYNC_SENTINEL) {
    MkProgram &Q = c->prog_odd;
    Q = P;
    Q.qkv += ps;
    Q.attn += ps;
    Q.xmid += ps;
    Q.hbuf += ps;
    Q.xout += ps;
    Q.act_other = P.qkv;
    if (hipMemcpyAsync(c->ws + c->plan.lay.prog_odd, &Q, sizeof(MkProgram), hipMemcpyHostToDevice, st) != hipSuccess)
      return MK_ERR_HIP;
  }
  if (!c->layers.empty() &&
      hipMemcpyAsync(c->ws + c->plan.lay.layers, c->layers.data(), sizeof(MkLayerW) * c->layers.size(),
                     hipMemcpyHostToDevice, st) != hipSuccess)
    return MK_ERR_HIP;
  if (!c->rowtab.empty() &&
      hipMemcpyAsync(c->ws + c->plan.lay.rowtab, c->rowtab.data(), sizeof(MkRowTab) * c->rowtab.size(),
                     hipMemcpyHostToDevice, st) != hipSuccess)
    return MK_ERR_HIP;
  return MK_OK;
}

// Row table of the stream engine: for every projection instruction, where its
// virtual rows start in memory, their length, and the row rotation that
// deals them to the streamer waves (carried along each CU's list, so every
// streamer's share of the list stays within one row of the others').
static void build_rowtab(mk_ctx *c) {
  const mk_plan_t &p = c->plan;
  const mk_model_shape &s = p.shape;
  const int64_t H = s.hidden, qd = (int64_t)s.n_q_heads * s.head_dim, kd = (int64_t)s.n_kv_heads * s.head_dim,
                I = s.ffn;
  c->rowtab.assign(p.instr.size(), MkRowTab{});
  for (int cu = 0; cu < p.n_cu; ++cu) {
    int off = 0;
    for (int i = p.cu_begin[cu]; i < p.cu_begin[cu + 1]; ++i) {
      const MkInstr &in = p.instr[i];
      MkRowTab &t = c->rowtab[i];
      t.off = off;
      if (in.op == MKOP_ATTN) continue;
      const MkLayerW *W = in.op == MKOP_LMHEAD ? nullptr : &c->layers[in.layer];
      const int64_t r0 = in.r0;
      int64_t K = H;
      const uint16_t *b0 = nullptr, *b1 = nullptr;
      int n = in.r1 - in.r0;
      switch (in.op) {
        case MKOP_QKV:
          b0 = r0 < qd ? W->wq + r0 * H : r0 < qd + kd ? W->wk + (r0 - qd) * H : W->wv + (r0 - qd - kd) * H;
          break;
        case MKOP_OPROJ:
          K = qd;
          b0 = W->wo + r0 * K;
          break;
        case MKOP_GATEUP:
          b0 = W->wg + r0 * H;
          b1 = W->wu + r0 * H;
          n *= 2;
          break;
        case MKOP_DOWN:
          K = I;
          b0 = W->wd + r0 * I;
          break;
        default:  // MKOP_LMHEAD
          b0 = c->prog.lm_head + r0 * H;
          break;
      }
      t.b0 = (uint64_t)(uintptr_t)b0;
      t.rb = (int32_t)(2 * K);
      if (b1) {
        t.b1 = (uint64_t)(uintptr_t)b1;
        t.stride2 = t.rb;
      } else {
        t.b1 = t.b0 + (uint64_t)t.rb;
        t.stride2 = 2 * t.rb;
      }
      t.n = n;
      off = (off + n) % MK_STREAMERS;
    }
  }
}

static int zero_sync(mk_ctx *c, hipStream_t st) {
  const MkLayout &y = c->plan.lay;
  size_t words = (y.sync_end - y.sync_begin) / 4;
  if (mk_launch_fill(c->ws + y.sync_begin, 0u, words, st)) return MK_ERR_HIP;
  if (c->plan.opts.sync_mode == MK_SYNC_SENTINEL) {
    // both step parities of the activations start as "not produced yet"
    const size_t act_words = 2 * (y.act_end - y.qkv) / 4;
    if (mk_launch_fill(c->ws + y.qkv, 0x7FBADBADu, act_words, st)) return MK_ERR_HIP;
  }
  return MK_OK;
}

// Bind a plan to workspace ws on device dev (the shared body of both
// context constructors).
static int ctx_create_on(const mk_plan_t *plan, void *d_workspace, size_t ws_bytes, int dev, hipStream_t st,
                         uint64_t scratch_gen, mk_ctx **out);

int mk_ctx_create(const mk_plan_t *plan, void *d_workspace, size_t ws_bytes, void *stream, mk_ctx **out) {
  if (!plan || !d_workspace || !out) return MK_ERR_INVALID_ARG;
  *out = nullptr;
  if (((uintptr_t)d_workspace & 255u) != 0) return MK_ERR_ALIGN;
  if (ws_bytes < plan->lay.total) return MK_ERR_CTX_OVERFLOW;
  if (mk_plan_check(plan, false, 0, 0) != MK_OK) return MK_ERR_PLAN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MK_ERR_HIP;
  return ctx_create_on(plan, d_workspace, ws_bytes, dev, (hipStream_t)stream, 0, out);
}

int mk_ctx_create_scratch(const mk_plan_t *plan, void *stream, mk_ctx **out) {
  if (!plan || !out) return MK_ERR_INVALID_ARG;
  *out = nullptr;
  if (plan->lay.total > MK_SCRATCH_BYTES) return MK_ERR_SCRATCH;
  if (mk_plan_check(plan, false, 0, 0) != MK_OK) return MK_ERR_PLAN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MK_ERR_HIP;
  void *ws = nullptr;
  uint64_t gen = 0;
  if (mk_scratch_acquire(dev, &ws, &gen)) return MK_ERR_HIP;
  return ctx_create_on(plan, ws, MK_SCRATCH_BYTES, dev, (hipStream_t)stream, gen, out);
}

static int ctx_create_on(const mk_plan_t *plan, void *d_workspace, size_t ws_bytes, int dev, hipStream_t st,
                         uint64_t scratch_gen, mk_ctx **out) {
  if (plan->opts.exec_mode != MK_EXEC_MULTI && plan->opts.exec_mode != MK_EXEC_FLAT_MULTI) {
    int n_dev_cu = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&n_dev_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MK_ERR_HIP;
    const int occ = mk_occupancy(plan->opts.exec_mode, plan->opts.sync_mode, launch_lds(plan), &per_cu);
    if (occ) return MK_ERR_HIP;
    // persistence: every workgroup of the grid must be resident at once
    if (per_cu < 1 || (int64_t)plan->n_cu > (int64_t)per_cu * n_dev_cu) return MK_ERR_NOT_RESIDENT;
  }
  if (mk_prepare_launch(plan->opts.exec_mode, plan->opts.sync_mode, launch_lds(plan))) return MK_ERR_HIP;
  mk_ctx *c = new (std::nothrow) mk_ctx();
  if (!c) return MK_ERR_INVALID_ARG;
  c->plan = *plan;
  c->ws = (char *)d_workspace;
  c->ws_bytes = ws_bytes;
  c->device = dev;
  c->scratch_gen = scratch_gen;
  const mk_plan_t &p = c->plan;
  const MkLayout &y = p.lay;
  const mk_model_shape &s = p.shape;
  MkProgram &P = c->prog;
  std::memset(&P, 0, sizeof P);
  P.L = s.n_layers;
  P.H = s.hidden;
  P.nq = s.n_q_heads;
  P.nkv = s.n_kv_heads;
  P.d = s.head_dim;
  P.I = s.ffn;
  P.V = s.vocab;
  P.G = p.G;
  P.B_max = p.B;
  P.max_ctx = p.max_ctx;
  P.S = p.S;
  P.eps = (float)s.rms_eps;
  P.tied = s.tie_embeddings ? 1 : 0;
  P.sync_mode = p.opts.sync_mode;
  P.n_cu = p.n_cu;
  P.n_instr = (int32_t)p.instr.size();
  P.n_levels = p.n_levels;
  P.n_events = p.n_events;
  P.ctr_stride = mk_ctr_stride(p.n_events);
  P.n_lm_parts = p.n_lm_parts;
  P.watchdog_ticks = 200000000u;  // 2 s
  P.lds_x = p.lds_x;
  P.lds_resid = p.lds_resid;
  P.lds_out = p.lds_out;
  P.out_stride = p.out_stride;
  P.lds_ring = p.lds_ring;
  P.n_pages = p.n_pages;
  P.lds_total = p.lds_bytes;
  P.par_stride = (int64_t)((y.act_end - y.qkv) / 4);
  P.st_out = p.st_out;
  P.st_resid = p.st_resid;
  P.st_ctl = p.st_ctl;
  char *w = c->ws;
  P.instr = (const MkInstr *)(w + y.instr);
  P.cu_begin = (const int32_t *)(w + y.cu_begin);
  P.level_begin = (const int32_t *)(w + y.level_begin);
  P.level_list = (const int32_t *)(w + y.level_list);
  P.queue = (const int32_t *)(w + y.queue);
  P.queue_ctr = (uint32_t *)(w + y.queue_ctr);
  P.ev_count = (const int32_t *)(w + y.ev_count);
  P.ev_flag_base = (const int32_t *)(w + y.ev_flag_base);
  P.rope = (const float *)(w + y.rope);
  P.layers = (MkLayerW *)(w + y.layers);
  P.rowtab = (const MkRowTab *)(w + y.rowtab);
  P.qkv = (float *)(w + y.qkv);
  P.attn = (float *)(w + y.attn);
  P.xmid = (float *)(w + y.xmid);
  P.hbuf = (float *)(w + y.hbuf);
  P.xout = (float *)(w + y.xout);
  P.part = (float *)(w + y.part);
  P.dpart = (float *)(w + y.dpart);
  P.lm_pk = (uint64_t *)(w + y.lm_pk);
  P.lm_val = (float *)(w + y.lm_val);
  P.lm_idx = (int32_t *)(w + y.lm_idx);
  P.ctr = (uint32_t *)(w + y.ctr);
  P.flags = (uint32_t *)(w + y.flags);
  P.tickets = (uint32_t *)(w + y.tickets);
  P.lm_done = (uint32_t *)(w + y.lm_done);
  P.err = (int32_t *)(w + y.err);
  build_rope(p, c->rope);
  int rc = MK_OK;
  auto up = [&](size_t off, const void *src, size_t bytes) {
    if (rc == MK_OK && bytes && hipMemcpyAsync(w + off, src, bytes, hipMemcpyHostToDevice, st) != hipSuccess)
      rc = MK_ERR_HIP;
  };
  up(y.instr, p.instr.data(), sizeof(MkInstr) * p.instr.size());
  up(y.cu_begin, p.cu_begin.data(), 4 * p.cu_begin.size());
  up(y.level_begin, p.level_begin.data(), 4 * p.level_begin.size());
  up(y.level_list, p.level_list.data(), 4 * p.level_list.size());
  up(y.queue, p.queue.data(), 4 * p.queue.size());
  up(y.ev_count, p.ev_count.data(), 4 * p.ev_count.size());
  up(y.ev_flag_base, p.ev_flag_base.data(), 4 * p.ev_flag_base.size());
  up(y.rope, c->rope.data(), 4 * c->rope.size());
  if (rc == MK_OK) rc = upload_prog(c, st);
  if (rc == MK_OK) rc = zero_sync(c, st);
  // the uploads read host memory owned by c; finish them before returning so
  // a caller that destroys the plan or ctx early cannot race them
  if (rc == MK_OK && hipStreamSynchronize(st) != hipSuccess) rc = MK_ERR_HIP;
  if (rc != MK_OK) {
    delete c;
    return rc;
  }
  *out = c;
  return MK_OK;
}

int mk_load_weights(mk_ctx *c, const mk_weights *wt, void *stream) {
  if (!c || !wt) return MK_ERR_INVALID_ARG;
  const mk_model_shape &s = c->plan.shape;
  const int L = s.n_layers;
  if (!wt->embed || !wt->final_norm) return MK_ERR_INVALID_ARG;
  if (!s.tie_embeddings && !wt->lm_head) return MK_ERR_INVALID_ARG;
  if (!aligned16(wt->embed) || !aligned16(wt->final_norm) || (!s.tie_embeddings && !aligned16(wt->lm_head)))
    return MK_ERR_ALIGN;
  const void *const *arrs[9] = {wt->attn_norm, wt->wq, wt->wk, wt->wv, wt->wo, wt->mlp_norm, wt->wg, wt->wu, wt->wd};
  for (auto a : arrs)
    if (!a) return MK_ERR_INVALID_ARG;
  std::vector<MkLayerW> layers(L);
  for (int l = 0; l < L; ++l) {
    for (auto a : arrs) {
      if (!a[l]) return MK_ERR_INVALID_ARG;
      if (!aligned16(a[l])) return MK_ERR_ALIGN;
    }
    layers[l].attn_norm = (const uint16_t *)wt->attn_norm[l];
    layers[l].wq = (const uint16_t *)wt->wq[l];
    layers[l].wk = (const uint16_t *)wt->wk[l];
    layers[l].wv = (const uint16_t *)wt->wv[l];
    layers[l].wo = (const uint16_t *)wt->wo[l];
    layers[l].mlp_norm = (const uint16_t *)wt->mlp_norm[l];
    layers[l].wg = (const uint16_t *)wt->wg[l];
    layers[l].wu = (const uint16_t *)wt->wu[l];
    layers[l].wd = (const uint16_t *)wt->wd[l];
  }
  c->layers.swap(layers);
  c->prog.embed = (const uint16_t *)wt->embed;
  c->prog.lm_head = (const uint16_t *)(s.tie_embeddings ? wt->embed : wt->lm_head);
  c->prog.final_norm = (const uint16_t *)wt->final_norm;
  build_rowtab(c);
  hipStream_t st = (hipStream_t)stream;
  // batched plans: the LM-head matrix as operand-order tiles in the workspace
  c->prog.lm_tiled = nullptr;
  const MkLayout &y = c->plan.lay;
  if (y.lm_tiled_bytes) {
    uint16_t *dst = (uint16_t *)(c->ws + y.lm_tiled);
    if (mk_launch_tile_rows(c->prog.lm_head, s.vocab, s.hidden, dst, st)) return MK_ERR_HIP;
    c->prog.lm_tiled = dst;
  }
  c->prog.gu_tiled = nullptr;
  if (y.gu_tiled_bytes) {
    uint16_t *dst = (uint16_t *)(c->ws + y.gu_tiled);
    for (int l = 0; l < L; ++l)
      if (mk_launch_tile_pairs(c->layers[l].wg, c->layers[l].wu, s.ffn, s.hidden, dst + (size_t)l * 2 * s.ffn * s.hidden,
                               st))
        return MK_ERR_HIP;
    c->prog.gu_tiled = dst;
  }
  int rc = upload_prog(c, st);
  if (rc == MK_OK && hipStreamSynchronize(st) != hipSuccess) rc = MK_ERR_HIP;
  if (rc == MK_OK) c->weights = true;
  return rc;
}

// Shared checks and step record of mk_decode_step / mk_decode_steps.
static int step_record(mk_ctx *c, int32_t *d_tokens, int32_t *d_positions, int32_t batch, void *d_kv, float *d_logits,
                       int32_t *d_next, uint32_t flags, MkStep &S) {
  if (!c || !d_tokens || !d_positions || !d_kv || !d_logits) return MK_ERR_INVALID_ARG;
  if (c->poisoned) return MK_ERR_STATE;
  if (!c->weights) return MK_ERR_INVALID_ARG;
  // a newer scratch context on this device has re-initialised the array
  if (c->scratch_gen && !mk_scratch_current(c->device, c->scratch_gen)) return MK_ERR_STATE;
  if (batch < 1 || batch > c->plan.B) return MK_ERR_CTX_OVERFLOW;
  if (flags & ~MK_ADVANCE) return MK_ERR_INVALID_ARG;
  if (!aligned16(d_kv) || ((uintptr_t)d_logits & 3u) || ((uintptr_t)d_tokens & 3u) || ((uintptr_t)d_positions & 3u) ||
      ((uintptr_t)d_next & 3u))
    return MK_ERR_ALIGN;
  std::memset(&S, 0, sizeof S);
  S.tokens = d_tokens;
  S.positions = d_positions;
  S.kv = (uint16_t *)d_kv;
  S.logits = d_logits;
  S.next = d_next;
  S.batch = batch;
  S.epoch = (uint32_t)c->epoch;
  S.flags = flags;
  S.n_steps = 1;
  return MK_OK;
}

// Homogeneous engine: the program record of the step with this epoch, and
// the other parity's (sentinel mode keeps one record per activation copy).
static void flat_records(const mk_ctx *c, uint64_t epoch, const MkProgram **first, const MkProgram **other) {
  const MkProgram *even = (const MkProgram *)(c->ws + c->plan.lay.prog);
  const MkProgram *odd = (const MkProgram *)(c->ws + c->plan.lay.prog_odd);
  const bool sent = c->plan.opts.sync_mode == MK_SYNC_SENTINEL;
  *first = sent && (epoch & 1) ? odd : even;
  *other = sent && !(epoch & 1) ? odd : even;
}

int mk_decode_step(mk_ctx *c, int32_t *d_tokens, int32_t *d_positions, int32_t batch, void *d_kv, float *d_logits,
                   int32_t *d_next, uint32_t flags, void *stream) {
  MkStep S;
  const int rc = step_record(c, d_tokens, d_positions, batch, d_kv, d_logits, d_next, flags, S);
  if (rc != MK_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const MkProgram *dp = (const MkProgram *)(c->ws + c->plan.lay.prog);
  const int mode = c->plan.opts.exec_mode;
  if (mode == MK_EXEC_MEGA) {
    if (mk_launch_role_mega(dp, S, c->plan.n_cu, c->plan.lds_bytes, st)) return MK_ERR_HIP;
  } else if (mode == MK_EXEC_FLAT) {
    const MkProgram *other = nullptr;
    flat_records(c, c->epoch, &dp, &other);
    if (mk_launch_mega(dp, other, S, c->plan.n_cu, mega_lds(&c->plan), c->plan.opts.sync_mode == MK_SYNC_SENTINEL, st))
      return MK_ERR_HIP;
  } else if (mode == MK_EXEC_STREAM) {
    if (mk_launch_stream(dp, S, c->plan.n_cu, mega_lds(&c->plan), st)) return MK_ERR_HIP;
  } else if (mode == MK_EXEC_QUEUE) {
    if (c->plan.queue.size() != c->plan.instr.size()) return MK_ERR_PLAN;  // a plan whose list was replaced
    if (mk_launch_queue(dp, S, c->plan.n_cu, mega_lds(&c->plan), st)) return MK_ERR_HIP;
  } else if (mode == MK_EXEC_FLAT_MULTI) {
    S.multi = 1;
    for (int lv = 0; lv < c->plan.n_levels; ++lv) {
      S.level = lv;
      const int nb = c->plan.level_begin[lv + 1] - c->plan.level_begin[lv];
      if (mk_launch_flat_level(dp, nullptr, S, nb, mega_lds(&c->plan), st)) return MK_ERR_HIP;
    }
  } else {
    S.multi = 1;
    for (int lv = 0; lv < c->plan.n_levels; ++lv) {
      S.level = lv;
      int nb = c->plan.level_begin[lv + 1] - c->plan.level_begin[lv];
      if (mk_launch_role_level(dp, S, nb, c->plan.lds_bytes, st)) return MK_ERR_HIP;
    }
  }
  c->epoch++;
  return MK_OK;
}

int mk_decode_steps(mk_ctx *c, int32_t *d_tokens, int32_t *d_positions, int32_t batch, void *d_kv, float *d_logits,
                    int32_t *d_next, int32_t n_steps, void *stream) {
  MkStep S;
  const int rc = step_record(c, d_tokens, d_positions, batch, d_kv, d_logits, d_next, MK_ADVANCE, S);
  if (rc != MK_OK) return rc;
  if (c->plan.opts.exec_mode != MK_EXEC_FLAT) return MK_ERR_UNSUPPORTED;
  if (n_steps < 1 || n_steps > MK_MAX_STEPS) return MK_ERR_INVALID_ARG;
  // cache rows start on 128-byte lines, so no line holds both a row that a
  // step appends and one that an earlier step of the launch has read
  if ((uintptr_t)d_kv & 127u) return MK_ERR_ALIGN;
  S.n_steps = n_steps;
  const MkProgram *dp = nullptr, *other = nullptr;
  flat_records(c, c->epoch, &dp, &other);
  if (mk_launch_mega(dp, other, S, c->plan.n_cu, mega_lds(&c->plan), c->plan.opts.sync_mode == MK_SYNC_SENTINEL,
                     (hipStream_t)stream))
    return MK_ERR_HIP;
  c->epoch += (uint64_t)n_steps;
  return MK_OK;
}

// A step of the per-level build captured into a hipGraph.  The captured
// launches read the step record from device memory (d_step): a replay cannot
// change kernel arguments, and the epoch moves on the device (the graph's
// last node increments it).
struct mk_graph_s {
  mk_ctx *ctx = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  MkStep *d_step = nullptr;
  uint64_t dev_epoch = 0;  // the epoch d_step holds once the last replay has run
  ~mk_graph_s() {
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
    if (d_step) (void)hipFree(d_step);
  }
};

int mk_graph_create(mk_ctx *c, int32_t *d_tokens, int32_t *d_positions, int32_t batch, void *d_kv, float *d_logits,
                    int32_t *d_next, uint32_t flags, void *stream, mk_graph **out) {
  if (!out) return MK_ERR_INVALID_ARG;
  *out = nullptr;
  MkStep S;
  int rc = step_record(c, d_tokens, d_positions, batch, d_kv, d_logits, d_next, flags, S);
  if (rc != MK_OK) return rc;
  if (c->plan.opts.exec_mode != MK_EXEC_FLAT_MULTI) return MK_ERR_UNSUPPORTED;
  mk_graph *g = new (std::nothrow) mk_graph_s();
  if (!g) return MK_ERR_INVALID_ARG;
  g->ctx = c;
  hipStream_t st = (hipStream_t)stream, cs = nullptr;
  S.multi = 1;
  rc = hipMalloc((void **)&g->d_step, sizeof(MkStep)) == hipSuccess ? MK_OK : MK_ERR_HIP;
  if (rc == MK_OK && (hipMemcpyAsync(g->d_step, &S, sizeof S, hipMemcpyHostToDevice, st) != hipSuccess ||
                      hipStreamSynchronize(st) != hipSuccess))
    rc = MK_ERR_HIP;
  g->dev_epoch = c->epoch;
  if (rc == MK_OK && hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) rc = MK_ERR_HIP;
  if (rc == MK_OK && hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) rc = MK_ERR_HIP;
  if (rc == MK_OK) {
    const MkProgram *dp = (const MkProgram *)(c->ws + c->plan.lay.prog);
    for (int lv = 0; lv < c->plan.n_levels && rc == MK_OK; ++lv) {
      S.level = lv;
      const int nb = c->plan.level_begin[lv + 1] - c->plan.level_begin[lv];
      if (mk_launch_flat_level(dp, g->d_step, S, nb, mega_lds(&c->plan), cs)) rc = MK_ERR_HIP;
    }
    if (rc == MK_OK && mk_launch_step_end(g->d_step, cs)) rc = MK_ERR_HIP;
    hipGraph_t graph = nullptr;
    if (hipStreamEndCapture(cs, &graph) != hipSuccess) rc = MK_ERR_HIP;
    g->graph = graph;
  }
  if (rc == MK_OK && hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0) != hipSuccess) rc = MK_ERR_HIP;
  if (cs) (void)hipStreamDestroy(cs);
  if (rc != MK_OK) {
    delete g;
    return rc;
  }
  *out = g;
  return MK_OK;
}

int mk_graph_launch(mk_graph *g, void *stream) {
  if (!g) return MK_ERR_INVALID_ARG;
  mk_ctx *c = g->ctx;
  if (c->poisoned) return MK_ERR_STATE;
  if (c->scratch_gen && !mk_scratch_current(c->device, c->scratch_gen)) return MK_ERR_STATE;
  hipStream_t st = (hipStream_t)stream;
  // other steps ran on the context since this graph's last replay: bring the
  // device record's epoch up to date first (a fill kernel, outside the graph)
  if (g->dev_epoch != (uint64_t)c->epoch &&
      mk_launch_fill(&g->d_step->epoch, (uint32_t)c->epoch, 1, st))
    return MK_ERR_HIP;
  if (hipGraphLaunch(g->exec, st) != hipSuccess) return MK_ERR_HIP;
  c->epoch++;
  g->dev_epoch = c->epoch;
  return MK_OK;
}

void mk_graph_destroy(mk_graph *g) { delete g; }

int mk_get_device_error(mk_ctx *c, void *stream, int32_t *detail) {
  if (!c) return MK_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return MK_ERR_HIP;
  int32_t e[4] = {0, 0, 0, 0};
  if (hipMemcpy(e, c->ws + c->plan.lay.err, sizeof e, hipMemcpyDeviceToHost) != hipSuccess) return MK_ERR_HIP;
  if (detail) *detail = e[1];
  if (e[0] != 0 || e[2] != 0) {
    c->poisoned = true;
    return e[0] != 0 ? e[0] : MK_ERR_TIMEOUT;
  }
  return MK_OK;
}

int mk_ctx_reset(mk_ctx *c, void *stream) {
  if (!c) return MK_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  int rc = zero_sync(c, st);
  if (rc == MK_OK && hipStreamSynchronize(st) != hipSuccess) rc = MK_ERR_HIP;
  if (rc == MK_OK) {
    c->epoch = 0;
    c->poisoned = false;
  }
  return rc;
}

int64_t mk_ctx_epoch(const mk_ctx *c) { return c ? c->epoch : -1; }

void mk_ctx_destroy(mk_ctx *c) { delete c; }

// Test hook: shorten the device watchdog (microseconds) of a context.
int mk_ctx_set_watchdog_us(mk_ctx *c, uint32_t us, void *stream) {
  if (!c || us == 0) return MK_ERR_INVALID_ARG;
  uint64_t ticks = (uint64_t)us * 100u;  // 100 MHz real-time counter
  c->prog.watchdog_ticks = ticks > 0xffffffffu ? 0xffffffffu : (uint32_t)ticks;
  hipStream_t st = (hipStream_t)stream;
  int rc = upload_prog(c, st);
  if (rc == MK_OK && hipStreamSynchronize(st) != hipSuccess) rc = MK_ERR_HIP;
  return rc;
}

int mk_plan_get_layout(const mk_plan_t *p, uint64_t out[8]) {
  if (!p || !out) return MK_ERR_INVALID_ARG;
  const MkLayout &y = p->lay;
  out[0] = y.qkv;
  out[1] = y.attn;
  out[2] = y.xmid;
  out[3] = y.hbuf;
  out[4] = y.xout;
  out[5] = y.act_end;
  out[6] = y.part;
  out[7] = p->opts.sync_mode == MK_SYNC_SENTINEL ? (y.act_end - y.qkv) : 0;
  return MK_OK;
}

int mk_ctx_set_trace(mk_ctx *c, void *d_trace, size_t n_records, void *stream) {
  if (!c) return MK_ERR_INVALID_ARG;
  if (d_trace && n_records < c->plan.instr.size()) return MK_ERR_CTX_OVERFLOW;
  if (d_trace && !aligned16(d_trace)) return MK_ERR_ALIGN;
  c->prog.trace = (uint64_t *)d_trace;
  hipStream_t st = (hipStream_t)stream;
  int rc = upload_prog(c, st);
  if (rc == MK_OK && hipStreamSynchronize(st) != hipSuccess) rc = MK_ERR_HIP;
  return rc;
}

int mk_ctx_set_epoch(mk_ctx *c, int64_t epoch) {
  if (!c || epoch < 0) return MK_ERR_INVALID_ARG;
  c->epoch = epoch;
  return MK_OK;
}

int mk_device_query(int32_t device, mk_device_info *o) {
  if (!o) return MK_ERR_INVALID_ARG;
  std::memset(o, 0, sizeof *o);
  hipDeviceProp_t pr;
  if (hipGetDeviceProperties(&pr, device) != hipSuccess) return MK_ERR_HIP;
  o->num_cus = pr.multiProcessorCount;
  o->lds_per_block = (int32_t)pr.sharedMemPerBlock;
  o->lds_per_cu = (int32_t)pr.maxSharedMemoryPerMultiProcessor;
  o->warp_size = pr.warpSize;
  o->clock_khz = pr.clockRate;
  o->mem_clock_khz = pr.memoryClockRate;
  o->mem_bus_bits = pr.memoryBusWidth;
  o->max_threads_per_block = pr.maxThreadsPerBlock;
  std::strncpy(o->arch, pr.gcnArchName, sizeof(o->arch) - 1);
  int per = 0;
  if (hipSetDevice(device) == hipSuccess && mk_occupancy_mega(64 * 1024, &per) == 0) o->mega_blocks_per_cu = per;
  return MK_OK;
}

size_t mk_gridsync_scratch_bytes(int32_t n_blocks) { return n_blocks > 0 ? mk_gridsync_scratch(n_blocks) : 0; }

int mk_gridsync_bench(int32_t variant, int32_t n_barriers, int32_t n_blocks, void *d_scratch, int32_t *d_result,
                      void *stream) {
  if (variant < 0 || variant > 5 || n_barriers < 1 || n_blocks < 1 || !d_scratch || !d_result || (variant == 5 && n_blocks < 8))
    return MK_ERR_INVALID_ARG;
  if (((uintptr_t)d_scratch & 255u) != 0) return MK_ERR_ALIGN;
  int rc = mk_launch_gridsync(variant, n_barriers, n_blocks, d_scratch, d_result, (hipStream_t)stream);
  if (rc == -2) return MK_ERR_INVALID_ARG;
  return rc ? MK_ERR_HIP : MK_OK;
}

int mk_stream_read(const void *d_buf, size_t bytes, uint32_t *d_out, int32_t n_blocks, void *stream) {
  if (!d_buf || !d_out || n_blocks < 1 || (bytes & 15u)) return MK_ERR_INVALID_ARG;
  if (!aligned16(d_buf)) return MK_ERR_ALIGN;
  return mk_launch_stream_read(d_buf, bytes, d_out, n_blocks, (hipStream_t)stream) ? MK_ERR_HIP : MK_OK;
}

int mk_lds_stream_read(const void *d_buf, size_t bytes, uint32_t *d_out, int32_t n_blocks, int32_t n_waves,
                       void *stream) {
  if (!d_buf || !d_out || n_blocks < 1 || n_waves < 1 || n_waves > 8 || (bytes & 1023u)) return MK_ERR_INVALID_ARG;
  if (!aligned16(d_buf)) return MK_ERR_ALIGN;
  return mk_launch_lds_stream(d_buf, bytes, d_out, n_blocks, n_waves, (hipStream_t)stream) ? MK_ERR_HIP : MK_OK;
}

}  // extern "C"
