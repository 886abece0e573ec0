// Stream engine: one-sequence decode with the weight stream decoupled from
// the dependency waits.
//
// The megakernel page (section 2.5) lets a block stream the next
// instruction's operands while it computes the current one, and the
// warp-specialisation page (sections 5.2 and 5.4) splits a block's warps
// into producers of data, consumers that compute and a role that
// synchronises and stores.  On gfx950 the producer role does not go through
// LDS pages here: a wave's vector loads complete in issue order, so a wave
// that polls for an input while its own weight loads are in flight sees the
// input only once those weights have landed, and a wave that waits for its
// stores to complete (before it signals) also waits for its loads.  The
// roles are therefore split by what a wave keeps in flight:
//
//  * 7 streamer waves each own a ring of MK_RING 16-byte loads per lane in
//    registers.  A wave's share of the CU's projection rows (whole rows,
//    dealt round robin with a rotation that carries across instructions) is
//    one continuous stream of 1 KiB pieces; the ring keeps MK_RING pieces
//    requested ahead of the piece being multiplied, across instruction
//    boundaries, so the next instructions' weights travel while the current
//    one waits for its input.  Streamers never touch global memory except
//    through the ring: dot products go to LDS, and the wave reports how far
//    it got in an LDS word.
//  * 1 sync wave has nothing in flight but its own few accesses: it polls
//    the instruction's input event, stages the input vector into LDS
//    (RMSNorm fused), publishes it with an LDS word, waits until every
//    streamer has reported the instruction, applies the epilogue (residual
//    add, SiLU * up, logits and argmax), stores the outputs, waits for their
//    completion and triggers the output event.
//
// Attention instructions are joint: the streamers' rings stop short of them
// and drain, and all eight waves run the attention instruction together
// (mk_ops_batched.h), then the rings restart behind it.  A CU that runs a
// layer's attention holds no O or gate/up slice of that layer (planner), so
// its stream pauses only there.
#pragma once
#include "mk_ops_batched.h"

#define MK_NSW 7  // streamer waves; wave MK_NSW synchronises
#ifndef MK_RING
#define MK_RING 8  // 4 KiB units each streamer keeps in flight (4 loads of 16 B per lane each)
#endif

static_assert(MK_NSW == MK_STREAMERS, "the host deals rows to the same number of streamers");

// LDS control block (byte offset P.st_ctl)
struct StCtl {
  uint32_t x_ready;       // 1 + index of the last instruction whose input is staged
  uint32_t abort;         // set by the sync wave when the launch is ending early
  uint32_t prog[MK_NSW];  // per streamer: every instruction below this index is done
  uint32_t t_in[MK_NSW];  // tracing: when the streamer saw its instruction's input
  uint32_t t_out[MK_NSW]; // tracing: when it finished its rows of the instruction
  uint32_t t_u[4];        // tracing: when streamer 0 finished its first units of the instruction
};
#define ST_CTL_WORDS (2 + 3 * MK_NSW + 4)

MKD lds_char *st_lds() { return (lds_char *)mk_flat_lds; }
static_assert(sizeof(StCtl) == 4 * ST_CTL_WORDS, "control block words: x_ready, abort, prog[], t_in[], t_out[]");

// per-lane LDS word (the wave reads several words at once)
MKD uint32_t lds_ld_lane(lds_u32 *p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(p)) : "memory");
  return v;
}

// ------------------------------------------------------------ cursors

// The streaming unit is 4 KiB of one weight row: 2048 bf16 columns, four
// 16-byte loads per lane.  A row of K columns is ceil(K / 2048) units
// ("sub-rows"); each unit's dot product with its 2048 input columns goes to
// the result array at out[v * nsub + sub], and the sync wave adds a row's
// nsub partial sums.
#define MK_UNIT 4096
#define MK_UCOLS (MK_UNIT / 2)

// The cursor is wave-uniform; every update goes through readfirstlane so the
// compiler keeps it (and the descriptors built from it) in scalar registers
// instead of proving uniformity through the engine's control flow.
MKD int su(int v) { return __builtin_amdgcn_readfirstlane(v); }
MKD uint64_t su64(uint64_t v) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
}

// A streamer's position in its own unit stream over instructions [i, end):
// instruction i, virtual row v of it, unit sub of that row.  The row table
// (MkRowTab, built by the host) says where each instruction's rows are and
// how they are dealt: virtual row v belongs to streamer (v + off) mod
// MK_NSW.  When i == end the stream is exhausted.
struct StCur {
  int i, end, v, sub, nsub, n, rb, stride2;
  uint64_t b0, b1;
};

// Move to the first instruction at or after c.i (below c.end) holding a row
// of streamer w.
MKD void st_enter(const MkProgram &P, StCur &c, int w) {
  while (c.i < c.end) {
    const MkRowTab t = cld(&P.rowtab[c.i]);
    int v0 = w - su(t.off);
    if (v0 < 0) v0 += MK_NSW;
    if (v0 < su(t.n)) {
      c.v = v0;
      c.sub = 0;
      c.n = su(t.n);
      c.rb = su(t.rb);
      c.stride2 = su(t.stride2);
      c.nsub = su((c.rb + MK_UNIT - 1) / MK_UNIT);
      c.b0 = su64(t.b0);
      c.b1 = su64(t.b1);
      return;
    }
    c.i = su(c.i + 1);
  }
}

MKD void st_start(const MkProgram &P, StCur &c, int i0, int i1, int w) {
  c.i = i0;
  c.end = i1;
  c.v = c.sub = c.n = c.rb = c.stride2 = 0;
  c.nsub = 1;
  c.b0 = c.b1 = 0;
  st_enter(P, c, w);
}

// advance by one unit; true when the instruction was finished
MKD bool st_next(const MkProgram &P, StCur &c, int w) {
  c.sub = su(c.sub + 1);
  if (c.sub < c.nsub) return false;
  c.sub = 0;
  c.v = su(c.v + MK_NSW);
  if (c.v < c.n) return false;
  c.i = su(c.i + 1);
  st_enter(P, c, w);
  return true;
}

MKD uint64_t st_unitptr(const StCur &c) {
  return ((c.v & 1) ? c.b1 : c.b0) + (uint64_t)(c.v >> 1) * (uint64_t)c.stride2 + (uint64_t)c.sub * MK_UNIT;
}

// ------------------------------------------------------------ streamers

// One streamer over the projection instructions [i0, i1) of its CU (no
// attention among them).  R units (R x 4 KiB) in flight.  false: the launch
// is aborting.
template <int R>
MKD bool st_streamer(const MkProgram &P, int i0, int i1, int w) {
  lds_char *L = st_lds();
  const int lane = mk_tid() & 63;
  lds_u32 *ctl = (lds_u32 *)(L + P.st_ctl);
  lds_u32 *x_ready = ctl, *abort_f = ctl + 1, *prog = ctl + 2 + w;
  const lds_float *xs = (const lds_float *)L;
  lds_float *out = (lds_float *)(L + P.st_out);

  const bool traced = su(P.trace != nullptr);
  StCur lc, cc;  // load cursor (R units ahead) and compute cursor
  st_start(P, lc, i0, i1, w);
  st_start(P, cc, i0, i1, w);
  if (lane == 0) lds_st(prog, (uint32_t)cc.i);

  // Every slot refill issues exactly four loads, so the compiler's vmcnt
  // waits stay exact; past the segment's last unit a refill loads through an
  // empty descriptor (no memory access, zeros).
  uint32_t real = 0;  // bit s: slot s holds a unit of the stream
  auto issue = [&](mk_u32x4 (&u)[4], int slot) {
    const bool live = lc.i < lc.end;
    const int room = su(live ? min(MK_UNIT, lc.rb - lc.sub * MK_UNIT) : 0);
    const __amdgpu_buffer_rsrc_t r = mk_rsrc((const void *)su64(st_unitptr(lc)), (uint32_t)room);
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] = __builtin_amdgcn_raw_buffer_load_b128(r, q * 1024 + lane * 16, 0, 2);
    if (live) st_next(P, lc, w);
    real = su(live ? (real | (1u << slot)) : (real & ~(1u << slot)));
  };

  mk_u32x4 ring[R][4];
#pragma unroll
  for (int s = 0; s < R; ++s) issue(ring[s], s);

  int ready = -1;  // instruction whose input is known to be staged
  int nu = 0;       // tracing: units done in the current instruction
  bool ok = true, go = cc.i < cc.end;
  while (go) {
#pragma unroll
    for (int s = 0; s < R; ++s) {
      if (real & (1u << s)) {
        if (cc.i != ready) {
          // first unit of this wave in instruction cc.i: its input must be staged
          const uint32_t want = (uint32_t)cc.i + 1u;
          if ((int32_t)(lds_ld(x_ready) - want) < 0) {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            uint32_t n = 0;
            while ((int32_t)(lds_ld(x_ready) - want) < 0) {
              __builtin_amdgcn_s_sleep(1);
              if ((++n & 63u) == 0) {
                if (lds_ld(abort_f) || __builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)P.watchdog_ticks) {
                  ok = false;
                  break;
                }
              }
            }
            if (!ok) {
              go = false;
              break;
            }
          }
          ready = cc.i;
          nu = 0;
          if (traced && lane == 0) lds_st(ctl + 2 + MK_NSW + w, (uint32_t)__builtin_amdgcn_s_memrealtime());
        }
        float acc = 0.f;
        {
          // the input in its LDS layout (st_xoff): this lane's 8 columns of
          // piece q are two 16-byte words 1 KiB apart, and a wave's 64 reads
          // of either are 1 KiB contiguous (no bank conflicts)
          const lds_float *xu = xs + cc.sub * MK_UCOLS + lane * 4;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const mk_f32x4 xa = *(const lds_f32x4 *)(xu + q * 512), xb = *(const lds_f32x4 *)(xu + q * 512 + 256);
            const mk_u32x4 wv = ring[s][q];
            acc = fmaf(bf_lo(wv.x), xa.x, acc);
            acc = fmaf(bf_hi(wv.x), xa.y, acc);
            acc = fmaf(bf_lo(wv.y), xa.z, acc);
            acc = fmaf(bf_hi(wv.y), xa.w, acc);
            acc = fmaf(bf_lo(wv.z), xb.x, acc);
            acc = fmaf(bf_hi(wv.z), xb.y, acc);
            acc = fmaf(bf_lo(wv.w), xb.z, acc);
            acc = fmaf(bf_hi(wv.w), xb.w, acc);
          }
        }
        const float t = wave_total(acc);
        if (lane == 0) out[cc.v * cc.nsub + cc.sub] = t;
        if (traced && w == 0 && lane == 0 && nu < 4) lds_st(ctl + 2 + 3 * MK_NSW + nu, (uint32_t)__builtin_amdgcn_s_memrealtime());
        ++nu;
        if (st_next(P, cc, w) && lane == 0) {
          if (traced) lds_st(ctl + 2 + 2 * MK_NSW + w, (uint32_t)__builtin_amdgcn_s_memrealtime());
          lds_st(prog, (uint32_t)cc.i);
        }
      }
      issue(ring[s], s);
      if (cc.i >= cc.end) {
        go = false;
        break;
      }
    }
  }
  wait_vm();  // the rest of the ring: loads through the empty descriptor
  if (!ok) return false;
  if (lane == 0) lds_st(prog, (uint32_t)i1);
  return true;
}

// ------------------------------------------------------------ sync wave

// Wait for event `ev` of this step, one wave polling (nothing else of this
// wave is in flight).  false: the launch is aborting (error raised).
MKD bool st_wait_event(const MkProgram &P, const MkStep &S, int ev) {
  const int lane = mk_tid() & 63;
  uint64_t t0 = 0;
  uint32_t spins = 0;
  if (P.sync_mode == MKSYNC_COUNTER) {
    const uint32_t need = (S.epoch + 1u) * (uint32_t)P.ev_count[ev];
    while (true) {
      const uint32_t c = __builtin_amdgcn_readfirstlane(ctr_total(P, ev));
      if ((int32_t)(c - need) >= 0) return true;
      if (spins == 0) t0 = __builtin_amdgcn_s_memrealtime();
      __builtin_amdgcn_s_sleep(1);
      if ((++spins & 31u) == 0) {
        if (mk_aborted(P)) return false;
        if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)P.watchdog_ticks) {
          if (lane == 0) mk_raise(P, MK_E_TIMEOUT, ev);
          return false;
        }
      }
    }
  }
  const uint32_t want = S.epoch + 1u;
  const int n = P.ev_count[ev];
  const uint32_t *f = P.flags + P.ev_flag_base[ev];
  while (true) {
    bool mine = true;
    for (int k = lane; k < n; k += 64) mine = mine && ((int32_t)(ldcu(f + k) - want) >= 0);
    if (__all(mine)) return true;
    if (spins == 0) t0 = __builtin_amdgcn_s_memrealtime();
    __builtin_amdgcn_s_sleep(1);
    if ((++spins & 31u) == 0) {
      if (mk_aborted(P)) return false;
      if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)P.watchdog_ticks) {
        if (lane == 0) mk_raise(P, MK_E_TIMEOUT, ev);
        return false;
      }
    }
  }
}

MKD void st_signal(const MkProgram &P, const MkStep &S, int ev, int slot) {
  wait_vm();  // this wave's output stores have completed
  if ((mk_tid() & 63) == 0) {
    if (P.sync_mode == MKSYNC_COUNTER)
      ctr_bump(P, ev);
    else
      stcu(P.flags + P.ev_flag_base[ev] + slot, S.epoch + 1u);
  }
}

#define ST_NC 16  // float4 chunks per lane the sync wave holds at once (hidden <= 4096)

// LDS layout of a staged input vector: in each block of 512 columns, the
// 4-column group 2 i + h (h = 0, 1) sits at float offset 256 h + 4 i, so
// streamer lane i finds its columns 8 i .. 8 i + 7 of the block in two
// 16-byte words that the wave reads as two contiguous 1 KiB runs.  Float
// offset of the 4-column group starting at column e (e % 4 == 0):
MKD int st_xoff(int e) { return (e & ~511) | (((e >> 2) & 1) << 8) | ((e & 511) >> 3 << 2); }

MKD void st_xput(lds_float *xs, int e, float a, float b, float c, float d) {
  *(lds_f32x4 *)(xs + st_xoff(e)) = mk_f32x4{a, b, c, d};
}

// zero the columns [K, round up to a whole unit) of the staged input: a
// unit past a row's end carries zero weights, and must meet finite inputs
MKD void st_xtail(lds_float *xs, int K) {
  const int lane = mk_tid() & 63, end = (K + MK_UCOLS - 1) / MK_UCOLS * MK_UCOLS;
  for (int e = K + 4 * lane; e < end; e += 256) st_xput(xs, e, 0.f, 0.f, 0.f, 0.f);
}

// Stage src[K] (fp32, device-coherent) into LDS xs, K a multiple of 4,
// ST_NC float4 per lane per round.
MKD void st_copy(lds_float *xs, const float *src, int K) {
  const int lane = mk_tid() & 63, nc = K >> 2;
  const __amdgpu_buffer_rsrc_t r = mk_rsrc((const void *)su64((uint64_t)src), (uint32_t)su(K) * 4u);
  for (int c0 = 0; c0 < nc; c0 += 64 * ST_NC) {
    mk_u32x4 v[ST_NC];
#pragma unroll
    for (int k = 0; k < ST_NC; ++k) {
      const int c = c0 + lane + 64 * k;
      v[k] = ldc16(r, c < nc ? c * 16 : MK_OOB);
    }
#pragma unroll
    for (int k = 0; k < ST_NC; ++k) {
      const int c = c0 + lane + 64 * k;
      if (c < nc)
        st_xput(xs, 4 * c, __uint_as_float(v[k].x), __uint_as_float(v[k].y), __uint_as_float(v[k].z),
                __uint_as_float(v[k].w));
    }
  }
}

// Stage x[H] (fp32, or the bf16 embedding row when emb) into xs as
// x * (1 / sqrt(mean(x^2) + eps)) * gain; H <= 256 * ST_NC.
MKD void st_norm(lds_float *xs, const float *src, const uint16_t *emb, int H, const uint32_t (&gw)[ST_NC][2],
                 float eps) {
  const int lane = mk_tid() & 63, nc = H >> 2;
  float4 x[ST_NC];
  if (emb) {
    const __amdgpu_buffer_rsrc_t r = mk_rsrc((const void *)su64((uint64_t)emb), (uint32_t)su(H) * 2u);
#pragma unroll
    for (int k = 0; k < ST_NC; ++k) {
      const int c = lane + 64 * k;
      const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, c < nc ? c * 8 : MK_OOB, 0, 0);
      x[k] = make_float4(bf_lo(u[0]), bf_hi(u[0]), bf_lo(u[1]), bf_hi(u[1]));
    }
  } else {
    const __amdgpu_buffer_rsrc_t r = mk_rsrc((const void *)su64((uint64_t)src), (uint32_t)su(H) * 4u);
#pragma unroll
    for (int k = 0; k < ST_NC; ++k) {
      const int c = lane + 64 * k;
      const mk_u32x4 u = ldc16(r, c < nc ? c * 16 : MK_OOB);
      x[k] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < ST_NC; ++k) {
    ss = fmaf(x[k].x, x[k].x, ss);
    ss = fmaf(x[k].y, x[k].y, ss);
    ss = fmaf(x[k].z, x[k].z, ss);
    ss = fmaf(x[k].w, x[k].w, ss);
  }
  ss = wave_total(ss);
  const float rn = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int k = 0; k < ST_NC; ++k) {
    const int c = lane + 64 * k;
    if (c < nc)
      st_xput(xs, 4 * c, (x[k].x * rn) * bf_lo(gw[k][0]), (x[k].y * rn) * bf_hi(gw[k][0]),
              (x[k].z * rn) * bf_lo(gw[k][1]), (x[k].w * rn) * bf_hi(gw[k][1]));
  }
}

MKD void st_gain(uint32_t (&gw)[ST_NC][2], const uint16_t *gain, int H) {
  const int lane = mk_tid() & 63, nc = H >> 2;
  const __amdgpu_buffer_rsrc_t r = mk_rsrc((const void *)su64((uint64_t)gain), (uint32_t)su(H) * 2u);
#pragma unroll
  for (int k = 0; k < ST_NC; ++k) {
    const int c = lane + 64 * k;
    const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, c < nc ? c * 8 : MK_OOB, 0, 0);
    gw[k][0] = u[0];
    gw[k][1] = u[1];
  }
}

// The sync wave over the projection instructions [i0, i1).  false: aborting.
MKD bool st_sync(const MkProgram &P, const MkStep &S, int i0, int i1) {
  lds_char *L = st_lds();
  const int lane = mk_tid() & 63;
  lds_u32 *ctl = (lds_u32 *)(L + P.st_ctl);
  lds_u32 *x_ready = ctl, *abort_f = ctl + 1, *prog = ctl + 2;
  lds_float *xs = (lds_float *)L;
  const lds_float *out = (const lds_float *)(L + P.st_out);
  lds_float *res = (lds_float *)(L + P.st_resid);
  const int H = P.H, B = P.B_max;
  for (int i = i0; i < i1; ++i) {
    const MkInstr in = cld(&P.instr[i]);
    const uint64_t tw = P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    const int l = in.layer, n = in.r1 - in.r0;
    const int K = in.op == MKOP_OPROJ ? P.nq * P.d : in.op == MKOP_DOWN ? P.I : H;
    const int nsub = (2 * K + MK_UNIT - 1) / MK_UNIT;  // partial sums per row (4 KiB units)
    // row v's dot product: the sum of its units' partials
    auto row = [&](int v) -> float {
      float a = out[v * nsub];
      for (int u = 1; u < nsub; ++u) a += out[v * nsub + u];
      return a;
    };
    const bool normed = in.op == MKOP_QKV || in.op == MKOP_GATEUP || in.op == MKOP_LMHEAD;
    uint32_t gw[ST_NC][2];
    if (normed) {
      const uint16_t *gain = in.op == MKOP_QKV ? cld(&P.layers[l].attn_norm)
                             : in.op == MKOP_GATEUP ? cld(&P.layers[l].mlp_norm)
                                                    : P.final_norm;
      st_gain(gw, gain, H);
    }
    int tok = 0;
    if (l == 0 && (in.op == MKOP_QKV || in.op == MKOP_OPROJ)) {
      tok = __builtin_amdgcn_readfirstlane(gld(S.tokens));
      if (tok < 0 || tok >= P.V) {
        if (lane == 0) mk_raise(P, MK_E_INPUT, 0);
        if (lane == 0) lds_st(abort_f, 1u);
        return false;
      }
    }
    if (in.wait_ev >= 0 && !st_wait_event(P, S, in.wait_ev)) {
      if (lane == 0) lds_st(abort_f, 1u);
      return false;
    }
    const uint64_t tv = P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    // stage the input (and the residual rows of O / down)
    switch (in.op) {
      case MKOP_QKV:
        st_norm(xs, l > 0 ? P.xout + (size_t)(l - 1) * B * H : nullptr,
                l == 0 ? P.embed + (size_t)tok * H : nullptr, H, gw, P.eps);
        break;
      case MKOP_GATEUP: st_norm(xs, P.xmid + (size_t)l * B * H, nullptr, H, gw, P.eps); break;
      case MKOP_LMHEAD: st_norm(xs, P.xout + (size_t)(P.L - 1) * B * H, nullptr, H, gw, P.eps); break;
      case MKOP_OPROJ:
        for (int k = lane; k < n; k += 64)
          res[k] = l == 0 ? bf2f(gld(P.embed + (size_t)tok * H + in.r0 + k))
                          : ldc(P.xout + (size_t)(l - 1) * B * H + in.r0 + k);
        st_copy(xs, P.attn + (size_t)l * B * P.nq * P.d, P.nq * P.d);
        break;
      default:  // MKOP_DOWN
        for (int k = lane; k < n; k += 64) res[k] = ldc(P.xmid + (size_t)l * B * H + in.r0 + k);
        st_copy(xs, P.hbuf + (size_t)l * B * P.I, P.I);
        break;
    }
    st_xtail(xs, K);
    if (lane == 0) lds_st(x_ready, (uint32_t)i + 1u);
    const uint64_t ts = P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    // every streamer has reported instruction i
    {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      uint32_t spins = 0;
      while (true) {
        bool done = true;
        if (lane < MK_NSW) done = (int32_t)(lds_ld_lane(prog + lane) - ((uint32_t)i + 1u)) >= 0;
        if (__all(done)) break;
        __builtin_amdgcn_s_sleep(1);
        if ((++spins & 255u) == 0 && __builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)P.watchdog_ticks) {
          if (lane == 0) {
            mk_raise(P, MK_E_TIMEOUT, 0x20000 + i);
            lds_st(abort_f, 1u);
          }
          return false;
        }
      }
    }
    const uint64_t tc = P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    uint64_t tsi = 0, tu = 0;
    if (P.trace) {
      // streamers with rows in this instruction reported when they saw its
      // input and when they finished (others keep older values)
      uint32_t a = 0xffffffffu, b = 0;
      if (lane < MK_NSW) {
        a = lds_ld_lane(ctl + 2 + MK_NSW + lane);
        b = lds_ld_lane(ctl + 2 + 2 * MK_NSW + lane);
        if ((int32_t)(a - (uint32_t)tv) < 0) a = 0xffffffffu;  // stale: before this staging
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        a = min(a, (uint32_t)__shfl_xor((int)a, o, 64));
        b = max(b, (uint32_t)__shfl_xor((int)b, o, 64));
      }
      tsi = ((uint64_t)b << 32) | a;
      const uint32_t a0 = lds_ld(ctl + 2 + MK_NSW);
      for (int k = 0; k < 4; ++k) {
        const uint32_t d = lds_ld(ctl + 2 + 3 * MK_NSW + k) - a0;
        tu |= (uint64_t)(d > 0xffffu ? 0xffffu : d) << (16 * k);
      }
    }
    // epilogue
    switch (in.op) {
      case MKOP_QKV: {
        float *dst = P.qkv + (size_t)l * B * ((P.nq + 2 * P.nkv) * P.d) + in.r0;
        for (int k = lane; k < n; k += 64) stc(dst + k, row(k));
        break;
      }
      case MKOP_OPROJ: {
        float *dst = P.xmid + (size_t)l * B * H + in.r0;
        for (int k = lane; k < n; k += 64) stc(dst + k, res[k] + row(k));
        break;
      }
      case MKOP_GATEUP: {
        float *dst = P.hbuf + (size_t)l * B * P.I + in.r0;
        for (int k = lane; k < n; k += 64) {
          const float a = row(2 * k), u = row(2 * k + 1);
          stc(dst + k, (a / (1.0f + expf(-a))) * u);
        }
        break;
      }
      case MKOP_DOWN: {
        float *dst = P.xout + (size_t)l * B * H + in.r0;
        for (int k = lane; k < n; k += 64) stc(dst + k, res[k] + row(k));
        break;
      }
      default: {  // MKOP_LMHEAD: logits, this slice's greedy partial, last arriver merges
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int k = lane; k < n; k += 64) {
          const float v = row(k);
          const int r = in.r0 + k;
          gst(S.logits + r, v);
          if (better(v, r, bv, bi)) {
            bv = v;
            bi = r;
          }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          const float ov = __shfl_xor(bv, o, 64);
          const int oi = __shfl_xor(bi, o, 64);
          if (better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
          }
        }
        if (lane == 0) {
          stc(P.lm_val + (size_t)in.part * B, bv);
          stci(P.lm_idx + (size_t)in.part * B, bi);
        }
        wait_vm();
        uint32_t old = 0;
        if (lane == 0) old = addcu(P.tickets + in.ticket, 1u);
        old = __builtin_amdgcn_readfirstlane(old);
        if (old + 1u == (S.epoch + 1u) * (uint32_t)P.n_lm_parts) {
          float v = -INFINITY;
          int ix = 0x7fffffff;
          for (int k = lane; k < P.n_lm_parts; k += 64) {
            const float pv = ldc(P.lm_val + (size_t)k * B);
            const int pi = ldci(P.lm_idx + (size_t)k * B);
            if (better(pv, pi, v, ix)) {
              v = pv;
              ix = pi;
            }
          }
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) {
            const float ov = __shfl_xor(v, o, 64);
            const int oi = __shfl_xor(ix, o, 64);
            if (better(ov, oi, v, ix)) {
              v = ov;
              ix = oi;
            }
          }
          if (lane == 0) {
            if (ix == 0x7fffffff) ix = 0;  // every logit NaN: token 0
            if (S.next) S.next[0] = ix;
            if (S.flags & 1u) {
              S.tokens[0] = ix;
              S.positions[0] = S.positions[0] + 1;
            }
          }
        }
        break;
      }
    }
    if (in.op != MKOP_LMHEAD && in.sig_ev >= 0) st_signal(P, S, in.sig_ev, in.sig_slot);
    if (P.trace && lane == 0) {
      uint64_t *r = P.trace + (size_t)i * 8;
      r[0] = tw;
      r[1] = ts;
      r[2] = __builtin_amdgcn_s_memrealtime();
      r[3] = ((uint64_t)blockIdx.x << 32) | S.epoch;
      r[4] = tv;  // input event seen (staging starts)
      r[5] = tc;  // every streamer done (epilogue starts)
      r[6] = tsi;  // low 32 bits: first streamer past the input; high: last streamer done
      r[7] = tu;   // streamer 0: 16-bit tick offsets of its first four units' ends from word 6's low half
    }
  }
  return true;
}
