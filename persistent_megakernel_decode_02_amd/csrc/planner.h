// Host planner: model shape -> per-CU instruction lists, events, workspace
// layout.  Pure host C++; no HIP calls.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "mk.h"
#include "mk_program.h"

// byte offsets inside the caller's workspace; prog_odd: the homogeneous
// engine's program record for odd steps in sentinel mode
struct MkLayout {
  size_t prog, prog_odd, instr, cu_begin, level_begin, level_list, queue, ev_count, ev_flag_base, rope, layers, rowtab;
  size_t qkv, attn, xmid, hbuf, xout, act_end, part, dpart, lm_val, lm_idx, ctr, flags, tickets, lm_pk, lm_done, queue_ctr, err;
  size_t lm_tiled, lm_tiled_bytes;  // batched plans: tiled copy of the LM-head matrix (0 bytes: none)
  size_t gu_tiled, gu_tiled_bytes;  // batched plans: tiled gate/up rows of every layer (0 bytes: none)
  size_t sync_begin, sync_end;  // [ctr .. err] zeroed on create/reset
  size_t total;
};

struct mk_plan_s {
  mk_model_shape shape;
  mk_plan_opts opts;
  int n_cu = 0, S = 1, B = 1, max_ctx = 0, G = 1;
  int Sd = 1;  // input-column parts of each down-projection slice (batched plans)
  int n_levels = 0, n_events = 0, n_flags = 0, n_tickets = 0, n_lm_parts = 0;
  int lds_bytes = 0;
  int lds_x = 0, lds_resid = 0, lds_out = 0, lds_ring = 0, n_pages = 0, out_stride = 0;  // role engine
  int st_out = 0, st_resid = 0, st_ctl = 0;  // stream engine
  std::vector<MkInstr> instr;  // CU-major
  std::vector<int32_t> instr_cu;
  std::vector<int32_t> cu_begin, level_begin, level_list, ev_count, ev_flag_base;
  // BFS linearisation of the instructions (indices into instr): the order a
  // global work queue hands them out in; the instructions one event releases
  // are contiguous, and every instruction comes after all its producers
  std::vector<int32_t> queue;
  MkLayout lay{};
  bool validated = false;
  double weight_bytes = 0;
};

int mk_plan_build(const mk_model_shape *shape, const mk_plan_opts *opts, int n_cu, mk_plan_t **out);
int mk_plan_check(const mk_plan_t *p, bool simulate, int trials, uint64_t seed);
bool mk_plan_tiles(const mk_plan_t *p);
// Derive the plan's events from the instructions' data accesses (MPK-style
// normalisation): at most one wait and one trigger event per instruction,
// events fused by predecessor set and by successor set, numbered and
// linearised breadth-first (fills ev_count, ev_flag_base, n_flags, the
// instructions' wait/trigger fields and `queue`).  MK_ERR_PLAN when the
// fusion would create a cycle or an instruction reads a slice nobody writes.
int mk_plan_normalize_events(mk_plan_t *p);
void mk_plan_finalize_lists(mk_plan_t *p);  // recompute cu_begin / level lists from instr + instr_cu
void mk_plan_compute_layout(mk_plan_t *p);
