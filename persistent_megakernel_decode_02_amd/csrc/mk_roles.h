// Role-specialised execution of the instruction lists: loader, sync/storer
// and compute wavefronts inside each workgroup, talking through a paged LDS
// ring and LDS counters.
//
// The warp-specialisation page ("5 . La specialisation des warps") splits a
// kernel's warps into a producer that only moves data and consumers that
// only compute (section 5.2), names the loader / compute / storer /
// scheduler roles of megakernels (section 5.4), maps the circular staging
// buffer of a GEMM onto shared-memory pages in a megakernel (section 5.5),
// and notes that fast AMD kernels stream weights continuously into LDS with
// non-temporal hints (its Q&A on porting to MI300X).  The megakernel page's
// section 2.6 item 4 makes shared memory a paged heap that successive
// instructions share.  Here:
//
//   * loader waves stream every instruction's weight rows (or key/value
//     blocks) into 4 KiB LDS pages with direct global->LDS loads, in list
//     order, as far ahead as free pages allow -- including past the
//     dependency wait of the instruction the data belongs to, since weights
//     never depend on activations;
//   * the sync/storer wave waits for the instruction's input (counter, flag,
//     or the data itself in sentinel mode), stages it in LDS (RMSNorm,
//     RoPE, residual rows), publishes it, and after the compute waves finish
//     stores their results (residual adds, argmax, merges, tickets) and
//     triggers the event;
//   * compute waves take whole output rows (or key blocks) round-robin, read
//     their pages, free them and leave one value per row in LDS.
//
// On CDNA a wave issues at most one instruction every four cycles, so the
// per-page work of every role is kept to a few dozen instructions: page
// addresses and ring slots advance incrementally (no division per page),
// full pages are loaded and read without bounds checks, and compute waves
// keep their row results in a register (one lane per row) instead of
// storing each one.
//
// Every wait is a bounded spin (watchdog + abort flag), so a protocol error
// ends the kernel with MK_ERR_TIMEOUT instead of hanging.
#pragma once
#include "mk_device.h"

#define MK_SYNCW MK_NLW                   // the sync/storer wave
#define MK_QMAX 12                        // pages a loader keeps in flight (4 loads each, vmcnt <= 63)


// LDS control block (start of dynamic LDS)
struct MkCtl {
  uint32_t pg_ready[MK_MAXNP];  // seq + 1 of the page in the slot once it has landed
  uint32_t pg_done[MK_MAXNP];   // seq + 1 of the page in the slot once consumed
  uint32_t x_ready;             // instructions whose inputs are staged
  uint32_t cw_done;             // compute-wave instruction completions
  uint32_t abort;               // a role gave up: everyone leaves
  uint32_t pad0;
  int32_t pos[MK_RB_MAXB];      // positions of this step, read once at kernel start
  uint32_t st_load_block;       // trace only: 100 MHz ticks the loaders spent waiting for a free page
  uint32_t st_page_wait;        // trace only: ticks compute waves spent waiting for a landed page
  uint32_t st_pages;            // trace only: pages issued
};
typedef __attribute__((address_space(3))) MkCtl MkCtl3;

struct MkRole {
  MkProgC &P;
  MkStepC &S;
  MkCtl3 *ctl;       // control block (LDS address space: flags are ds instructions)
  lds_float *X;       // staged input vector(s) [B][K] (ATTN: q | k | v | wave partials)
  lds_float *resid;   // residual rows [B][rows]
  lds_float *out;     // per-row results of the compute waves [B][out_stride]
  lds_char *ring;     // NP pages
  int np;
  int par;            // activation parity (sentinel mode)
};

static_assert(sizeof(MkCtl) <= MK_CTL_BYTES, "LDS control block");

// ------------------------------------------------------------- LDS sync



// Spin (one wave, uniform) until *p >= v.  false: the kernel is aborting.
// Long waits (`nap`) sleep 4 x 64 clocks per poll so the spinning wave
// leaves issue slots to the waves doing work.
MKD bool role_wait(const MkRole &R, lds_u32 *p, uint32_t v, bool nap = false) {
  if ((int32_t)(lds_ld(p) - v) >= 0) return true;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  uint32_t n = 0;
  while ((int32_t)(lds_ld(p) - v) < 0) {
    if (nap) __builtin_amdgcn_s_sleep(4);
    else __builtin_amdgcn_s_sleep(1);
    if ((++n & 63u) == 0) {
      if (lds_ld(&R.ctl->abort)) return false;
      if (mk_aborted(R.P)) {
        lds_st(&R.ctl->abort, 1u);
        return false;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)R.P.watchdog_ticks) {
        if ((threadIdx.x & 63) == 0) mk_raise(R.P, MK_E_TIMEOUT, 0x10000 + (int)(p - (lds_u32 *)R.ctl));
        lds_st(&R.ctl->abort, 1u);
        return false;
      }
    }
  }
  return true;
}

MKD void role_abort(const MkRole &R) { lds_st(&R.ctl->abort, 1u); }

// ---------------------------------------------------- instruction geometry
//
// Every role derives the same page stream from an instruction: units (one
// output row of a projection, or one block of key positions) in order, each
// made of nh halves (gate and up rows; key and value blocks) of ppr pages.
// Page k of half h of unit u starts at src[h] + u * ustride + k * 4 KiB.

struct MkGeo {
  int n_units, ppr, nh, ppu;
  int K;              // input length of a projection row
  int rb;             // bytes per weight row (ATTN: bytes per full key block)
  int full;           // every page of the instruction is a whole 4 KiB page
  const char *src0, *src1;
  size_t ustride;
  // attention
  int d, p, t0, t1, bp;  // head_dim, current position, key range [t0, t1), positions per page
};

MKD bool mk_geo(MkProgC &P, MkStepC &S, const MkCtl3 *ctl, const MkInstr &in, MkGeo &g) {
  g.d = P.d;
  g.p = g.t0 = g.t1 = g.bp = 0;
  g.nh = 1;
  g.src1 = nullptr;
  MkLayerW LW;
  if (in.op != MKOP_LMHEAD) LW = cld(&P.layers[in.layer]);
  const uint16_t *w0 = nullptr;
  switch (in.op) {
    case MKOP_QKV: {
      g.K = P.H;
      const int qd = P.nq * P.d, kd = P.nkv * P.d;
      const int r = in.r0;
      if (r < qd) w0 = LW.wq + (size_t)r * P.H;
      else if (r < qd + kd) w0 = LW.wk + (size_t)(r - qd) * P.H;
      else w0 = LW.wv + (size_t)(r - qd - kd) * P.H;
      break;
    }
    case MKOP_OPROJ:
      g.K = P.nq * P.d;
      w0 = LW.wo + (size_t)in.r0 * g.K;
      break;
    case MKOP_GATEUP:
      g.K = P.H;
      w0 = LW.wg + (size_t)in.r0 * P.H;
      g.src1 = (const char *)(LW.wu + (size_t)in.r0 * P.H);
      g.nh = 2;
      break;
    case MKOP_DOWN:
      g.K = P.I;
      w0 = LW.wd + (size_t)in.r0 * P.I;
      break;
    case MKOP_LMHEAD:
      g.K = P.H;
      w0 = (P.tied ? P.embed : P.lm_head) + (size_t)in.r0 * P.H;
      break;
    case MKOP_ATTN: {
      const int b = in.r0, gg = in.r1, NS = in.nsplit;
      g.bp = MK_PAGE / (2 * P.d);
      g.nh = 2;
      g.ppr = 1;
      g.ppu = 2;
      g.K = 0;
      g.rb = MK_PAGE;
      g.ustride = MK_PAGE;
      if (b >= S.batch) {  // a sequence slot beyond this step's batch: no keys, no cache access
        g.p = -1;
        g.n_units = 0;
        g.full = 1;
        g.src0 = g.src1 = nullptr;
        return true;
      }
      const int p = __builtin_amdgcn_readfirstlane(ctl->pos[b]);
      if (p < 0 || p >= P.max_ctx) return false;
      const int n = p + 1;
      // splits start on page boundaries so pages never straddle two splits
      const int chunk = ((n + NS - 1) / NS + g.bp - 1) / g.bp * g.bp;
      g.p = p;
      g.t0 = min(n, in.split * chunk);
      g.t1 = min(n, g.t0 + chunk);
      g.src0 = (const char *)(S.kv + kv_off(P, in.layer, 0, b, gg) + (size_t)g.t0 * P.d);
      g.src1 = (const char *)(S.kv + kv_off(P, in.layer, 1, b, gg) + (size_t)g.t0 * P.d);
      g.n_units = (g.t1 - g.t0 + g.bp - 1) / g.bp;
      g.full = ((g.t1 - g.t0) % g.bp) == 0;
      return true;
    }
    default:
      return false;
  }
  g.src0 = (const char *)w0;
  g.n_units = in.r1 - in.r0;
  g.rb = g.K * 2;
  g.ppr = (g.rb + MK_PAGE - 1) / MK_PAGE;
  g.ppu = g.ppr * g.nh;
  g.ustride = (size_t)g.rb;
  g.full = (g.rb % MK_PAGE) == 0;
  return true;
}

// valid bytes of page k of a row / key block of unit u
MKD int mk_page_valid(const MkGeo &g, int u, int k) {
  if (g.bp) return min(g.bp, g.t1 - (g.t0 + u * g.bp)) * 2 * g.d;
  return min(MK_PAGE, g.rb - k * MK_PAGE);
}

// ------------------------------------------------------------- loader role

MKD void vm_wait_le(int n) {  // until at most n (0..60, multiple of 4) vector loads are in flight
  switch (n >> 2) {
    case 15: asm volatile("s_waitcnt vmcnt(60)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(56)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(52)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(44)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(40)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(36)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

struct LoaderState {
  uint32_t s;     // next page sequence number this loader issues
  int slot;       // its ring slot (s % np)
  uint32_t pub;   // sequence number of the oldest issued, unpublished page
  int pub_slot;
  int inflight;   // issued, unpublished pages
};

// publish the oldest in-flight page once it has landed
MKD void loader_publish_one(const MkRole &R, LoaderState &L) {
  vm_wait_le(4 * (L.inflight - 1));
  lds_st(&R.ctl->pg_ready[L.pub_slot], L.pub + 1u);
  L.pub += MK_NLW;
  L.pub_slot += MK_NLW;
  if (L.pub_slot >= R.np) L.pub_slot -= R.np;
  --L.inflight;
}

// Issue one page into the loader's next slot.  Waits (publishing landed
// pages meanwhile) until the slot's previous page was consumed.  false on abort.
// SWZ (key/value pages, rows of rb bytes): LDS chunk p of row t receives
// source chunk p ^ (t & 7) (a permutation of each row's 16-byte chunks)
template <bool FULL, bool SWZ>
MKD bool loader_page(const MkRole &R, LoaderState &L, const char *src, int valid, int rb) {
  if (L.s >= (uint32_t)R.np) {
    const uint32_t need = L.s - (uint32_t)R.np + 1u;
    if ((int32_t)(lds_ld(&R.ctl->pg_done[L.slot]) - need) < 0) {
      const uint64_t t0 = R.P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
      // never sit on landed pages while blocked: publish them one by one
      while (L.inflight > 0) {
        loader_publish_one(R, L);
        if ((int32_t)(lds_ld(&R.ctl->pg_done[L.slot]) - need) >= 0) break;
      }
      if (!role_wait(R, &R.ctl->pg_done[L.slot], need)) return false;
      if (R.P.trace && (threadIdx.x & 63) == 0)
        lds_add(&R.ctl->st_load_block, (uint32_t)(__builtin_amdgcn_s_memrealtime() - t0));
    }
  }
  const int lane = threadIdx.x & 63;
  lds_char *dst = R.ring + (size_t)L.slot * MK_PAGE;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int off = q * 1024 + lane * 16;
    if (SWZ) {
      const int t = off / rb, in_row = off - t * rb;
      off = t * rb + ((((in_row >> 4) ^ (t & 7)) << 4) | (in_row & 15));
    }
    if (!FULL && off > valid - 16) off = valid - 16;  // stay inside the source; the tail is never read
    __builtin_amdgcn_global_load_lds((const void *)(src + off), (lds_void *)(dst + q * 1024), 16, 0, 0);
  }
  if (L.inflight == 0) {
    L.pub = L.s;
    L.pub_slot = L.slot;
  }
  ++L.inflight;
  L.s += MK_NLW;
  L.slot += MK_NLW;
  if (L.slot >= R.np) L.slot -= R.np;
  if (L.inflight > MK_QMAX) loader_publish_one(R, L);
  return true;
}

// ------------------------------------------------------- compute helpers

MKD void page_wait_slow(const MkRole &R, int slot, uint32_t want, bool *ok) {
  const uint64_t t0 = R.P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
  *ok = role_wait(R, &R.ctl->pg_ready[slot], want);
  if (R.P.trace && (threadIdx.x & 63) == 0)
    lds_add(&R.ctl->st_page_wait, (uint32_t)(__builtin_amdgcn_s_memrealtime() - t0));
}
// wait until page seq s is in ring slot `slot`; false on abort
MKD bool page_wait(const MkRole &R, int slot, uint32_t s) {
  if ((int32_t)(lds_ld(&R.ctl->pg_ready[slot]) - (s + 1u)) >= 0) return true;
  bool ok;
  page_wait_slow(R, slot, s + 1u, &ok);
  return ok;
}
MKD void page_free(const MkRole &R, int slot, uint32_t s) { lds_st(&R.ctl->pg_done[slot], s + 1u); }

MKD int ring_add(int slot, int k, int np) {
  slot += k;
  while (slot >= np) slot -= np;
  return slot;
}

MKD float dot8(const mk_u32x4 w, const mk_f32x4 xa, const mk_f32x4 xb, float a) {
  a = fmaf(bf_lo(w.x), xa.x, a);
  a = fmaf(bf_hi(w.x), xa.y, a);
  a = fmaf(bf_lo(w.y), xa.z, a);
  a = fmaf(bf_hi(w.y), xa.w, a);
  a = fmaf(bf_lo(w.z), xb.x, a);
  a = fmaf(bf_hi(w.z), xb.y, a);
  a = fmaf(bf_lo(w.w), xb.z, a);
  a = fmaf(bf_hi(w.w), xb.w, a);
  return a;
}

// Lane slice of a staged input for one page of a row: chunk q of page kk
// covers input elements kk*2048 + q*512 + lane*8 .. +8.
struct XSlice {
  mk_f32x4 v[4][2];
};
MKD void load_xslice(const lds_float *x, int kk, XSlice &xs) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const lds_f32x4 *x4 = reinterpret_cast<const lds_f32x4 *>(x + kk * 2048 + q * 512 + lane * 8);
    xs.v[q][0] = x4[0];
    xs.v[q][1] = x4[1];
  }
}
MKD float page_dot(const lds_char *pg, const XSlice &xs, float a) {
  const int lane = threadIdx.x & 63;
  mk_u32x4 w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) w[q] = *reinterpret_cast<const lds_u32x4 *>(pg + q * 1024 + lane * 16);
#pragma unroll
  for (int q = 0; q < 4; ++q) a = dot8(w[q], xs.v[q][0], xs.v[q][1], a);
  return a;
}
