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
//     performs the epilogue: merges, tickets and the event trigger;
//   * compute waves take whole output rows (or key blocks) round-robin, read
//     their pages, write results with device-coherent stores and free the
//     pages.
//
// Every wait is a bounded spin (watchdog + abort flag), so a protocol error
// ends the kernel with MK_ERR_TIMEOUT instead of hanging.
#pragma once
#include "mk_device.h"

#define MK_SYNCW MK_NLW                   // the sync/storer wave
#define MK_QMAX 15                        // pages a loader keeps in flight (4 loads each, vmcnt <= 63)
#define MK_SENTINEL 0x7FBADBADu           // quiet NaN payload the arithmetic never produces

typedef __attribute__((address_space(3))) void lds_void;

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
  float lm_v[MK_NCW * MK_RB_MAXB];
  int32_t lm_i[MK_NCW * MK_RB_MAXB];
};

struct MkRole {
  const MkProgram &P;
  const MkStep &S;
  MkCtl *ctl;
  float *X;           // staged input vector(s) [B][K] (ATTN: q | k | v | wave partials)
  float *resid;       // residual rows [B][rows]
  float *wsc;         // per-compute-wave scratch [NCW][MK_WSC]
  char *ring;         // NP pages
  int np;
  int par;            // activation parity (sentinel mode)
};

static_assert(sizeof(MkCtl) <= MK_CTL_BYTES, "LDS control block");

// ------------------------------------------------------------- LDS sync

// LDS flags: explicit address space 3 (ds_* instructions, counted by
// lgkmcnt only, so they never wait for a loader's in-flight global->LDS
// loads) with workgroup fences restricted to LDS.
typedef __attribute__((address_space(3))) uint32_t mk_lds_u32;
MKD uint32_t lds_ld(uint32_t *p) {
  const uint32_t v = __hip_atomic_load((mk_lds_u32 *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return v;
}
MKD void lds_st(uint32_t *p, uint32_t v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __hip_atomic_store((mk_lds_u32 *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// The loader's own flag accesses are written as ds instructions in inline
// assembly.  Compiled LDS accesses would make the compiler wait for every
// global->LDS load still in flight (those write LDS and are counted by
// vmcnt, and it cannot prove the flag and the pages do not overlap); the
// loader has already waited for exactly the pages it publishes.
MKD uint32_t lds_off(const void *p) { return (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)p; }
MKD void lds_publish(uint32_t *p, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_off(p)), "v"(v) : "memory");
}
MKD uint32_t lds_peek(uint32_t *p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(p)) : "memory");
  return v;
}
MKD void lds_add(uint32_t *p, uint32_t v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __hip_atomic_fetch_add((mk_lds_u32 *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// read-only program data (instruction lists, pointer tables) through the
// constant address space: scalar loads, counted by lgkmcnt, never by vmcnt
template <class T>
MKD T cld(const T *p) {
#if defined(__HIP_DEVICE_COMPILE__)
  T v;
  const __attribute__((address_space(4))) uint32_t *src = (const __attribute__((address_space(4))) uint32_t *)p;
  uint32_t *dst = reinterpret_cast<uint32_t *>(&v);
  static_assert(sizeof(T) % 4 == 0, "word-sized records");
#pragma unroll
  for (unsigned i = 0; i < sizeof(T) / 4; ++i) dst[i] = src[i];
  return v;
#else
  return *p;
#endif
}

// Spin (one wave, uniform) until *p >= v.  false: the kernel is aborting.
MKD bool role_wait(const MkRole &R, uint32_t *p, uint32_t v) {
  if ((int32_t)(lds_ld(p) - v) >= 0) return true;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  uint32_t n = 0;
  while ((int32_t)(lds_ld(p) - v) < 0) {
    if (lds_ld(&R.ctl->abort)) return false;
    __builtin_amdgcn_s_sleep(1);
    if ((++n & 127u) == 0) {
      if (mk_aborted(R.P)) {
        lds_st(&R.ctl->abort, 1u);
        return false;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)R.P.watchdog_ticks) {
        if ((threadIdx.x & 63) == 0) mk_raise(R.P, MK_E_TIMEOUT, 0x10000 + (int)(p - (uint32_t *)R.ctl));
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
// made of ppu pages.

struct MkGeo {
  int n_units, ppu;
  int d;              // head_dim
  int K;              // input length of a projection row
  int rb;             // bytes per weight row
  int ppr;            // pages per weight row
  const uint16_t *w0, *w1;  // matrices (gate/up use both)
  // attention
  int p, t0, t1, bp;  // current position, key range [t0, t1), positions per page
  const uint16_t *kc, *vc;
};

MKD int role_batch(const MkStep &S) { return S.batch; }

MKD bool mk_geo(const MkProgram &P, const MkStep &S, const MkCtl *ctl, const MkInstr &in, MkGeo &g) {
  g.w1 = nullptr;
  g.d = P.d;
  g.kc = g.vc = nullptr;
  g.p = g.t0 = g.t1 = g.bp = 0;
  MkLayerW LWv;
  if (in.op != MKOP_LMHEAD) LWv = cld(&P.layers[in.layer]);
  const MkLayerW *LW = &LWv;
  switch (in.op) {
    case MKOP_QKV: {
      g.K = P.H;
      const int qd = P.nq * P.d, kd = P.nkv * P.d;
      const int r = in.r0;
      if (r < qd) g.w0 = LW->wq + (size_t)r * P.H;
      else if (r < qd + kd) g.w0 = LW->wk + (size_t)(r - qd) * P.H;
      else g.w0 = LW->wv + (size_t)(r - qd - kd) * P.H;
      g.n_units = in.r1 - in.r0;
      break;
    }
    case MKOP_OPROJ:
      g.K = P.nq * P.d;
      g.w0 = LW->wo + (size_t)in.r0 * g.K;
      g.n_units = in.r1 - in.r0;
      break;
    case MKOP_GATEUP:
      g.K = P.H;
      g.w0 = LW->wg + (size_t)in.r0 * P.H;
      g.w1 = LW->wu + (size_t)in.r0 * P.H;
      g.n_units = in.r1 - in.r0;
      break;
    case MKOP_DOWN:
      g.K = P.I;
      g.w0 = LW->wd + (size_t)in.r0 * P.I;
      g.n_units = in.r1 - in.r0;
      break;
    case MKOP_LMHEAD:
      g.K = P.H;
      g.w0 = (P.tied ? P.embed : P.lm_head) + (size_t)in.r0 * P.H;
      g.n_units = in.r1 - in.r0;
      break;
    case MKOP_ATTN: {
      const int b = in.r0, gg = in.r1, NS = in.nsplit;
      const int p = ctl->pos[b];
      if (p < 0 || p >= P.max_ctx) return false;
      const int n = p + 1;
      g.bp = MK_PAGE / (2 * P.d);
      // splits start on page boundaries so pages never straddle two splits
      const int chunk = ((n + NS - 1) / NS + g.bp - 1) / g.bp * g.bp;
      g.p = p;
      g.t0 = min(n, in.split * chunk);
      g.t1 = min(n, g.t0 + chunk);
      g.kc = S.kv + kv_off(P, in.layer, 0, b, gg);
      g.vc = S.kv + kv_off(P, in.layer, 1, b, gg);
      g.n_units = (g.t1 - g.t0 + g.bp - 1) / g.bp;
      g.ppu = 2;
      g.K = 0;
      g.rb = 0;
      g.ppr = 0;
      return true;
    }
    default:
      return false;
  }
  g.rb = g.K * 2;
  g.ppr = (g.rb + MK_PAGE - 1) / MK_PAGE;
  g.ppu = g.ppr * (g.w1 ? 2 : 1);
  return true;
}

// global source of page k (0 <= k < ppu) of unit u, and its valid bytes
MKD const char *mk_page_src(const MkGeo &g, int op, int u, int k, int *valid) {
  if (op == MKOP_ATTN) {
    const int t = g.t0 + u * g.bp;
    const int npos = min(g.bp, g.t1 - t);
    *valid = npos * 2 * g.d;  // npos rows of d bf16
    const uint16_t *base = (k == 0) ? g.kc : g.vc;
    return (const char *)(base + (size_t)t * g.d);
  }
  const int m = k / g.ppr, kk = k - m * g.ppr;
  const uint16_t *w = m ? g.w1 : g.w0;
  *valid = min(MK_PAGE, g.rb - kk * MK_PAGE);
  return (const char *)(w + (size_t)u * g.K) + (size_t)kk * MK_PAGE;
}

// ------------------------------------------------------------- loader role

struct LoaderState {
  uint32_t iss, pub;  // pages of this loader issued / published
};

MKD void loader_publish_all(const MkRole &R, LoaderState &L, int lid) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  while (L.pub < L.iss) {
    const uint32_t s = (uint32_t)lid + MK_NLW * L.pub;
    lds_publish(&R.ctl->pg_ready[s % R.np], s + 1u);
    ++L.pub;
  }
}

MKD void loader_issue(const MkRole &R, const char *src, int valid, int slot) {
  const int lane = threadIdx.x & 63;
  char *dst = R.ring + (size_t)slot * MK_PAGE;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int off = q * 1024 + lane * 16;
    if (off > valid - 16) off = valid - 16;  // stay inside the source; the tail is never read
    __builtin_amdgcn_global_load_lds((const void *)(src + off), (lds_void *)(dst + q * 1024), 16, 0, 0);
  }
}

// returns false on abort
MKD bool loader_page(const MkRole &R, LoaderState &L, int lid, uint32_t s, const char *src, int valid) {
  const int slot = (int)(s % (uint32_t)R.np);
  if (s >= (uint32_t)R.np) {
    const uint32_t need = s - (uint32_t)R.np + 1u;
    if ((int32_t)(lds_peek(&R.ctl->pg_done[slot]) - need) < 0) {
      loader_publish_all(R, L, lid);  // never block while holding landed pages
      const uint64_t t0 = R.P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
      if (!role_wait(R, &R.ctl->pg_done[slot], need)) return false;
      if (R.P.trace && (threadIdx.x & 63) == 0)
        lds_add(&R.ctl->st_load_block, (uint32_t)(__builtin_amdgcn_s_memrealtime() - t0));
    }
  }
  loader_issue(R, src, valid, slot);
  ++L.iss;
  if (L.iss - L.pub > MK_QMAX) {
    asm volatile("s_waitcnt vmcnt(60)" ::: "memory");  // all but the last 15 pages (60 loads) landed
    const uint32_t s0 = (uint32_t)lid + MK_NLW * L.pub;
    lds_publish(&R.ctl->pg_ready[s0 % R.np], s0 + 1u);
    ++L.pub;
  }
  return true;
}

// --------------------------------------------------------- compute helpers

MKD const char *page_wait(const MkRole &R, uint32_t s, bool *ok) {
  const int slot = (int)(s % (uint32_t)R.np);
  if (R.P.trace && (int32_t)(lds_ld(&R.ctl->pg_ready[slot]) - (s + 1u)) < 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    *ok = role_wait(R, &R.ctl->pg_ready[slot], s + 1u);
    if ((threadIdx.x & 63) == 0) lds_add(&R.ctl->st_page_wait, (uint32_t)(__builtin_amdgcn_s_memrealtime() - t0));
  } else {
    *ok = role_wait(R, &R.ctl->pg_ready[slot], s + 1u);
  }
  return R.ring + (size_t)slot * MK_PAGE;
}
MKD void page_free(const MkRole &R, uint32_t s) {
  lds_st(&R.ctl->pg_done[s % (uint32_t)R.np], s + 1u);
}

MKD float dot8(const mk_u32x4 w, const float4 xa, const float4 xb, float a) {
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

// Lane slice of the staged input for one page of a row: chunk q of page kk
// covers input elements kk*2048 + q*512 + lane*8 .. +8.  For one sequence
// and rows of one page (K <= 2048) the slice is the same for every row, so
// compute waves keep it in registers for the whole instruction.
template <int NB>
struct XSlice {
  float4 v[NB][4][2];
};

template <int NB>
MKD void load_xslice(const MkRole &R, const MkGeo &g, int B, int kk, XSlice<NB> &xs) {
  const int lane = threadIdx.x & 63;
  const int valid = min(MK_PAGE, g.rb - kk * MK_PAGE);
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool on = b < B && q * 1024 + lane * 16 < valid;
      const float4 *x4 = reinterpret_cast<const float4 *>(R.X + (size_t)b * g.K + kk * 2048 + q * 512 + lane * 8);
      xs.v[b][q][0] = on ? x4[0] : make_float4(0.f, 0.f, 0.f, 0.f);
      xs.v[b][q][1] = on ? x4[1] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// Dot products of one weight row (ppr pages starting at page seq s) with the
// staged vectors X[b][K], b < B <= NB.  acc[b] ends with the full sum
// (uniform).  CACHED: the input slice is `xc` (single-page rows); otherwise
// each page's slice is read from LDS together with the page.
template <int NB, bool CACHED>
MKD bool row_dot(const MkRole &R, const MkGeo &g, uint32_t s, int B, const XSlice<NB> &xc, float *acc) {
  const int lane = threadIdx.x & 63;
  float a[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) a[b] = 0.f;
  for (int kk = 0; kk < g.ppr; ++kk) {
    bool ok;
    const char *pg = page_wait(R, s + kk, &ok);
    if (!ok) return false;
    const int valid = min(MK_PAGE, g.rb - kk * MK_PAGE);
    mk_u32x4 w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int off = q * 1024 + lane * 16;
      w[q] = off < valid ? *(const mk_u32x4 *)(pg + off) : mk_u32x4{0, 0, 0, 0};
    }
    if (CACHED) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int b = 0; b < NB; ++b) a[b] = dot8(w[q], xc.v[b][q][0], xc.v[b][q][1], a[b]);
    } else {
      XSlice<NB> xl;
      load_xslice<NB>(R, g, B, kk, xl);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int b = 0; b < NB; ++b) a[b] = dot8(w[q], xl.v[b][q][0], xl.v[b][q][1], a[b]);
    }
    page_free(R, s + kk);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = wave_total(a[b]);
  return true;
}
