// Per-op staging (sync wave), compute (compute waves) and epilogue (sync
// wave) of the role-specialised engine, and the three role loops.
#pragma once
#include "mk_roles.h"

#define MK_SYNC_SENTINEL MKSYNC_SENTINEL
#define MK_XCH 16  // 16-byte chunks per lane the sync wave stages in one round (4096 floats)

// activation buffers of this step (two parities in sentinel mode)
struct MkAct {
  float *qkv, *attn, *xmid, *hbuf, *xout;
};
MKD MkAct mk_act(MkProgC &P, int par) {
  const size_t o = (size_t)par * P.par_stride;
  MkAct a;
  a.qkv = P.qkv + o;
  a.attn = P.attn + o;
  a.xmid = P.xmid + o;
  a.hbuf = P.hbuf + o;
  a.xout = P.xout + o;
  return a;
}

MKD bool has_sentinel(mk_u32x4 v) {
  return v.x == MK_SENTINEL || v.y == MK_SENTINEL || v.z == MK_SENTINEL || v.w == MK_SENTINEL;
}

// abort / watchdog check inside a sync-wave poll; false: give up
MKD bool poll_check(const MkRole &R, uint64_t t0, int code) {
  if (lds_ld(&R.ctl->abort) || mk_aborted(R.P)) {
    role_abort(R);
    return false;
  }
  if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)R.P.watchdog_ticks) {
    if ((threadIdx.x & 63) == 0) mk_raise(R.P, MK_E_TIMEOUT, code);
    role_abort(R);
    return false;
  }
  return true;
}

// Load up to MK_XCH 16-byte chunks per lane of the fp32 vector src[0, n)
// (chunk j of a lane covers elements (j * 64 + lane) * 4 .. + 4) with
// device-coherent loads, all in flight at once.  With `sentinel`, chunks
// still holding the sentinel are re-read until every word has been produced.
MKD bool load_vec(const MkRole &R, const float *src, int n, bool sentinel, mk_u32x4 (&v)[MK_XCH]) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rs = mk_rsrc(src, (uint32_t)n * 4u);
  const int nch = (n + 255) / 256;
#pragma unroll
  for (int j = 0; j < MK_XCH; ++j)
    if (j < nch) v[j] = ldc16(rs, (j * 64 + lane) * 16);  // out-of-range offsets read 0 (buffer bounds)
  if (!sentinel) return true;
  uint64_t t0 = 0;
  uint32_t spins = 0;
  while (true) {
    bool miss = false;
#pragma unroll
    for (int j = 0; j < MK_XCH; ++j)
      if (j < nch) miss = miss || ((j * 64 + lane) * 4 < n && has_sentinel(v[j]));
    if (!__any(miss)) return true;
    if (spins == 0) t0 = __builtin_amdgcn_s_memrealtime();
    __builtin_amdgcn_s_sleep(1);
    if ((++spins & 63u) == 0 && !poll_check(R, t0, 0x20000)) return false;
#pragma unroll
    for (int j = 0; j < MK_XCH; ++j)
      if (j < nch && (j * 64 + lane) * 4 < n && has_sentinel(v[j])) v[j] = ldc16(rs, (j * 64 + lane) * 16);
  }
}

MKD void store_vec(lds_float *dst, int n, const mk_u32x4 (&v)[MK_XCH]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < MK_XCH; ++j) {
    const int e = (j * 64 + lane) * 4;
    if (e < n)
      *reinterpret_cast<lds_f32x4 *>(dst + e) = mk_f32x4{__uint_as_float(v[j].x), __uint_as_float(v[j].y),
                                                         __uint_as_float(v[j].z), __uint_as_float(v[j].w)};
  }
}

// Copy n floats (n % 4 == 0) from global to LDS, MK_XCH chunks per lane per round.
MKD bool stage_vec(const MkRole &R, lds_float *dst, const float *src, int n, bool sentinel) {
  for (int base = 0; base < n; base += 256 * MK_XCH) {
    mk_u32x4 v[MK_XCH];
    const int m = min(n - base, 256 * MK_XCH);
    if (!load_vec(R, src + base, m, sentinel, v)) return false;
    store_vec(dst + base, m, v);
  }
  return true;
}

// n scalar floats (any alignment), device-coherent, sentinel-checked
MKD bool stage_scalars(const MkRole &R, lds_float *dst, const float *src, int n, bool sentinel) {
  const int lane = threadIdx.x & 63;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    float v = i < n ? ldc(src + i) : 0.f;
    if (sentinel) {
      uint64_t t0 = 0;
      uint32_t spins = 0;
      while (true) {
        const bool miss = i < n && __float_as_uint(v) == MK_SENTINEL;
        if (!__any(miss)) break;
        if (spins == 0) t0 = __builtin_amdgcn_s_memrealtime();
        __builtin_amdgcn_s_sleep(1);
        if ((++spins & 63u) == 0 && !poll_check(R, t0, 0x20001)) return false;
        if (miss) v = ldc(src + i);
      }
    }
    if (i < n) dst[i] = v;
  }
  return true;
}

// One round of a vector stage together with up to 64 scalars (any
// alignment; lane i loads scalar i): all loads in flight at once, polled
// together, so the residual rows cost no extra memory round trip.
MKD bool load_vec_and_scalars(const MkRole &R, const float *src, int n, const float *ssrc, int sn, bool sentinel,
                              mk_u32x4 (&v)[MK_XCH], float &sv) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rs = mk_rsrc(src, (uint32_t)n * 4u);
  const int nch = (n + 255) / 256;
  const bool has_s = lane < sn;
#pragma unroll
  for (int j = 0; j < MK_XCH; ++j)
    if (j < nch) v[j] = ldc16(rs, (j * 64 + lane) * 16);
  sv = has_s ? ldc(ssrc + lane) : 0.f;
  if (!sentinel) return true;
  uint64_t t0 = 0;
  uint32_t spins = 0;
  while (true) {
    bool miss = has_s && __float_as_uint(sv) == MK_SENTINEL;
#pragma unroll
    for (int j = 0; j < MK_XCH; ++j)
      if (j < nch) miss = miss || ((j * 64 + lane) * 4 < n && has_sentinel(v[j]));
    if (!__any(miss)) return true;
    if (spins == 0) t0 = __builtin_amdgcn_s_memrealtime();
    __builtin_amdgcn_s_sleep(1);
    if ((++spins & 63u) == 0 && !poll_check(R, t0, 0x20002)) return false;
#pragma unroll
    for (int j = 0; j < MK_XCH; ++j)
      if (j < nch && (j * 64 + lane) * 4 < n && has_sentinel(v[j])) v[j] = ldc16(rs, (j * 64 + lane) * 16);
    if (has_s && __float_as_uint(sv) == MK_SENTINEL) sv = ldc(ssrc + lane);
  }
}

// The attention instruction's query group, key and value (each a multiple
// of 64 floats, at most 512 / 128 / 128): one round, polled together.
MKD bool stage_qkv(const MkRole &R, const float *qs, int nqf, const float *ks, const float *vs, int d, lds_float *dq,
                   lds_float *dk, lds_float *dv, bool sentinel) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rq = mk_rsrc(qs, (uint32_t)nqf * 4u), rk = mk_rsrc(ks, (uint32_t)d * 4u),
                               rv = mk_rsrc(vs, (uint32_t)d * 4u);
  mk_u32x4 a0 = ldc16(rq, lane * 16), a1 = ldc16(rq, (64 + lane) * 16);
  mk_u32x4 bk = ldc16(rk, lane * 16), bv = ldc16(rv, lane * 16);
  const bool on0 = lane * 4 < nqf, on1 = (64 + lane) * 4 < nqf, onk = lane * 4 < d;
  if (sentinel) {
    uint64_t t0 = 0;
    uint32_t spins = 0;
    while (true) {
      const bool m0 = on0 && has_sentinel(a0), m1 = on1 && has_sentinel(a1), mk = onk && has_sentinel(bk),
                 mv = onk && has_sentinel(bv);
      if (!__any(m0 || m1 || mk || mv)) break;
      if (spins == 0) t0 = __builtin_amdgcn_s_memrealtime();
      __builtin_amdgcn_s_sleep(1);
      if ((++spins & 63u) == 0 && !poll_check(R, t0, 0x20003)) return false;
      if (m0) a0 = ldc16(rq, lane * 16);
      if (m1) a1 = ldc16(rq, (64 + lane) * 16);
      if (mk) bk = ldc16(rk, lane * 16);
      if (mv) bv = ldc16(rv, lane * 16);
    }
  }
  const auto put = [](lds_float *dst, mk_u32x4 w) {
    *reinterpret_cast<lds_f32x4 *>(dst) =
        mk_f32x4{__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w)};
  };
  if (on0) put(dq + lane * 4, a0);
  if (on1) put(dq + (64 + lane) * 4, a1);
  if (onk) {
    put(dk + lane * 4, bk);
    put(dv + lane * 4, bv);
  }
  return true;
}

// bf16 values of a length-n vector in the lane layout of load_vec (4 per chunk)
MKD void load_bf16_chunks(const uint16_t *p, int n, uint32_t (&g)[MK_XCH][2]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < MK_XCH; ++j) {
    const int e = (j * 64 + lane) * 4;
    if (e < n) {
      const uint64_t w = gld(reinterpret_cast<const uint64_t *>(p + e));
      g[j][0] = (uint32_t)w;
      g[j][1] = (uint32_t)(w >> 32);
    } else {
      g[j][0] = g[j][1] = 0u;
    }
  }
}

// RMSNorm of a vector held in registers (load_vec layout, n <= 256 * MK_XCH),
// gains g; result written to LDS dst
MKD void norm_store(lds_float *dst, int n, mk_u32x4 (&v)[MK_XCH], const uint32_t (&g)[MK_XCH][2], float eps) {
  const int lane = threadIdx.x & 63;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MK_XCH; ++j) {
    const int e = (j * 64 + lane) * 4;
    if (e < n) {
      const float a = __uint_as_float(v[j].x), b = __uint_as_float(v[j].y), c = __uint_as_float(v[j].z),
                  d = __uint_as_float(v[j].w);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
      ss = fmaf(c, c, ss);
      ss = fmaf(d, d, ss);
    }
  }
  ss = wave_total(ss);
  const float r = 1.0f / sqrtf(ss / (float)n + eps);
#pragma unroll
  for (int j = 0; j < MK_XCH; ++j) {
    const int e = (j * 64 + lane) * 4;
    if (e < n)
      *reinterpret_cast<lds_f32x4 *>(dst + e) = mk_f32x4{
          (__uint_as_float(v[j].x) * r) * bf_lo(g[j][0]), (__uint_as_float(v[j].y) * r) * bf_hi(g[j][0]),
          (__uint_as_float(v[j].z) * r) * bf_lo(g[j][1]), (__uint_as_float(v[j].w) * r) * bf_hi(g[j][1])};
  }
}

// ------------------------------------------------------- sync-wave staging

MKD bool normed_op(int op) { return op == MKOP_QKV || op == MKOP_GATEUP || op == MKOP_LMHEAD; }

MKD const uint16_t *norm_gain(MkProgC &P, const MkInstr &in) {
  return in.op == MKOP_QKV ? P.layers[in.layer].attn_norm
                           : in.op == MKOP_GATEUP ? P.layers[in.layer].mlp_norm : P.final_norm;
}

// returns false on abort (error already raised).  `gain` holds the norm
// gains of a normed op, loaded before the dependency wait.
// values a stage needs that do not depend on the instruction's input, loaded
// before the dependency wait: norm gains, RoPE cos/sin of this position
struct StagePre {
  uint32_t gain[MK_XCH][2];
  float rc, rs;
};

MKD bool sync_stage(const MkRole &R, const MkInstr &in, const MkGeo &g, const MkAct &A, bool sent,
                    const StagePre &pre) {
  MkProgC &P = R.P;
  MkStepC &S = R.S;
  const int lane = threadIdx.x & 63;
  const int B = S.batch, H = P.H, l = in.layer;
  switch (in.op) {
    case MKOP_QKV:
    case MKOP_GATEUP:
    case MKOP_LMHEAD: {
      for (int b = 0; b < B; ++b) {
        mk_u32x4 v[MK_XCH];
        if (in.op == MKOP_QKV && l == 0) {
          const int tok = gld(S.tokens + b);
          if (tok < 0 || tok >= P.V) {
            if (lane == 0) mk_raise(P, MK_E_INPUT, b);
            role_abort(R);
            return false;
          }
          uint32_t e2[MK_XCH][2];
          load_bf16_chunks(P.embed + (size_t)tok * H, H, e2);
#pragma unroll
          for (int j = 0; j < MK_XCH; ++j) v[j] = mk_u32x4{e2[j][0] << 16, e2[j][0] & 0xffff0000u, e2[j][1] << 16,
                                                           e2[j][1] & 0xffff0000u};
        } else {
          const float *src = in.op == MKOP_QKV ? A.xout + ((size_t)(l - 1) * P.B_max + b) * H
                             : in.op == MKOP_GATEUP ? A.xmid + ((size_t)l * P.B_max + b) * H
                                                    : A.xout + ((size_t)(P.L - 1) * P.B_max + b) * H;
          if (!load_vec(R, src, H, sent, v)) return false;
        }
        norm_store(R.X + (size_t)b * H, H, v, pre.gain, P.eps);
      }
      return true;
    }
    case MKOP_OPROJ:
    case MKOP_DOWN: {
      const int K = g.K, nr = in.r1 - in.r0;
      for (int b = 0; b < B; ++b) {
        lds_float *rd = R.resid + (size_t)b * nr;
        const float *src = in.op == MKOP_OPROJ ? A.attn + ((size_t)l * P.B_max + b) * K
                                               : A.hbuf + ((size_t)l * P.B_max + b) * K;
        const float *rs = in.op == MKOP_OPROJ ? A.xout + ((size_t)(l - 1) * P.B_max + b) * H + in.r0
                                              : A.xmid + ((size_t)l * P.B_max + b) * H + in.r0;
        int sn = nr <= 64 ? nr : 0;  // residual rows ride along with the first round
        if (in.op == MKOP_OPROJ && l == 0) {
          const int tok = gld(S.tokens + b);
          if (tok < 0 || tok >= P.V) {
            if (lane == 0) mk_raise(P, MK_E_INPUT, b);
            role_abort(R);
            return false;
          }
          for (int i = lane; i < nr; i += 64) rd[i] = bf2f(gld(P.embed + (size_t)tok * H + in.r0 + i));
          sn = 0;
        } else if (nr > 64) {
          if (!stage_scalars(R, rd, rs, nr, sent)) return false;
        }
        lds_float *x = R.X + (size_t)b * K;
        for (int base = 0; base < K; base += 256 * MK_XCH) {
          mk_u32x4 v[MK_XCH];
          float sv;
          const int m = min(K - base, 256 * MK_XCH);
          if (!load_vec_and_scalars(R, src + base, m, rs, base == 0 ? sn : 0, sent, v, sv)) return false;
          store_vec(x + base, m, v);
          if (base == 0 && lane < sn) rd[lane] = sv;
        }
      }
      return true;
    }
    case MKOP_ATTN: {
      if (g.p < 0) return true;  // sequence slot beyond this step's batch: nothing to stage
      const int b = in.r0, gg = in.r1, d = P.d, G = P.G, half = d / 2;
      const int R0 = (P.nq + 2 * P.nkv) * d;
      const float *qkv = A.qkv + ((size_t)l * P.B_max + b) * R0;
      lds_float *q = R.X, *kc = R.X + G * d, *vc = kc + d;
      if (!stage_qkv(R, qkv + (size_t)gg * G * d, G * d, qkv + (size_t)P.nq * d + (size_t)gg * d,
                     qkv + (size_t)(P.nq + P.nkv) * d + (size_t)gg * d, d, q, kc, vc, sent))
        return false;
      // queries are pre-scaled by log2(e) / sqrt(d): scores come out in base 2.
      // pre.rc / pre.rs: cos and sin of pair i = lane % half at this position
      // (every element a lane handles below has that pair index)
      const float qs = 1.4426950408889634f / sqrtf((float)d);
      for (int e = lane; e < (G + 1) * half; e += 64) {
        const int j = e / half, i = e - j * half;  // j == G is the key
        lds_float *u = j < G ? q + j * d : kc;
        const float a = u[i], c = u[i + half], co = pre.rc, si = pre.rs;
        float r0 = a * co - c * si, r1 = c * co + a * si;
        if (j == G) {
          r0 = bf2f(f2bf(r0));
          r1 = bf2f(f2bf(r1));
        } else {
          r0 *= qs;
          r1 *= qs;
        }
        u[i] = r0;
        u[i + half] = r1;
      }
      for (int i = lane; i < d; i += 64) vc[i] = bf2f(f2bf(vc[i]));
      if (g.t0 <= g.p && g.p < g.t1) {
        uint16_t *K = S.kv + kv_off(P, l, 0, b, gg) + (size_t)g.p * d;
        uint16_t *V = S.kv + kv_off(P, l, 1, b, gg) + (size_t)g.p * d;
        for (int i = lane; i < d; i += 64) {
          gst(K + i, f2bf(kc[i]));
          gst(V + i, f2bf(vc[i]));
        }
      }
      return true;
    }
    default:
      return false;
  }
}

// --------------------------------------------------------- compute waves

// results of one wave, one lane per row: lane t holds the wave's t-th row
// of the current 64-row chunk; written to R.out[b][unit] when full
struct RowRes {
  float v[MK_RB_MAXB];
  int t, ubase;
};
MKD void rowres_init(RowRes &rr, int cw) {
#pragma unroll
  for (int b = 0; b < MK_RB_MAXB; ++b) rr.v[b] = 0.f;
  rr.t = 0;
  rr.ubase = cw;
}
template <int NB>
MKD void rowres_put(const MkRole &R, RowRes &rr, const float *r, int B) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int b = 0; b < NB; ++b) rr.v[b] = lane == rr.t ? r[b] : rr.v[b];
  if (++rr.t == 64) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (b < B) R.out[(size_t)b * R.P.out_stride + rr.ubase + MK_NCW * lane] = rr.v[b];
    rr.t = 0;
    rr.ubase += 64 * MK_NCW;
  }
}
template <int NB>
MKD void rowres_flush(const MkRole &R, RowRes &rr, int B) {
  const int lane = threadIdx.x & 63;
  if (lane < rr.t) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (b < B) R.out[(size_t)b * R.P.out_stride + rr.ubase + MK_NCW * lane] = rr.v[b];
  }
}

MKD float silu_mul(float g, float u) { return (g / (1.0f + expf(-g))) * u; }

// One sequence, whole pages.  ONE: rows are one page, the input slice stays
// in registers; TWO: gate and up rows, SiLU(gate) * up per unit.
template <bool ONE, bool TWO>
MKD bool gemv_fast(const MkRole &R, const MkGeo &g, uint32_t seq0, int slot0, int cw) {
  const int ppr = ONE ? 1 : g.ppr, ppu = ONE ? (TWO ? 2 : 1) : g.ppu;
  XSlice xc;
  if (ONE && cw < g.n_units) load_xslice(R.X, 0, xc);
  RowRes rr;
  rowres_init(rr, cw);
  uint32_t s = seq0 + (uint32_t)(cw * ppu);
  int slot = ring_add(slot0, cw * ppu, R.np);
  const int ustep = (MK_NCW - 1) * ppu;  // pages of the other waves' units between two of ours
  for (int u = cw; u < g.n_units; u += MK_NCW) {
    float tot[2];
#pragma unroll
    for (int h = 0; h < (TWO ? 2 : 1); ++h) {
      float a = 0.f;
      for (int kk = 0; kk < ppr; ++kk) {
        if (!page_wait(R, slot, s)) return false;
        const lds_char *pg = R.ring + (size_t)slot * MK_PAGE;
        if (ONE) {
          a = page_dot(pg, xc, a);
        } else {
          XSlice xs;
          load_xslice(R.X, kk, xs);
          a = page_dot(pg, xs, a);
        }
        page_free(R, slot, s);
        ++s;
        if (++slot == R.np) slot = 0;
      }
      tot[h] = wave_total(a);
    }
    float r = tot[0];
    if (TWO) r = silu_mul(tot[0], tot[1]);
    rowres_put<1>(R, rr, &r, 1);
    s += (uint32_t)ustep;
    slot = ring_add(slot, ustep, R.np);
  }
  rowres_flush<1>(R, rr, 1);
  return true;
}

// Any batch (<= MK_RB_MAXB) and partial pages (rows shorter than a page,
// or not a whole number of pages): bounds-checked reads.
template <bool TWO>
MKD bool gemv_general(const MkRole &R, const MkGeo &g, uint32_t seq0, int slot0, int cw, int B) {
  const int lane = threadIdx.x & 63;
  RowRes rr;
  rowres_init(rr, cw);
  uint32_t s = seq0 + (uint32_t)(cw * g.ppu);
  int slot = ring_add(slot0, cw * g.ppu, R.np);
  const int ustep = (MK_NCW - 1) * g.ppu;
  for (int u = cw; u < g.n_units; u += MK_NCW) {
    float tot[2][MK_RB_MAXB];
#pragma unroll
    for (int h = 0; h < (TWO ? 2 : 1); ++h) {
      float a[MK_RB_MAXB];
#pragma unroll
      for (int b = 0; b < MK_RB_MAXB; ++b) a[b] = 0.f;
      for (int kk = 0; kk < g.ppr; ++kk) {
        if (!page_wait(R, slot, s)) return false;
        const lds_char *pg = R.ring + (size_t)slot * MK_PAGE;
        const int valid = g.full ? MK_PAGE : mk_page_valid(g, u, kk);
        mk_u32x4 w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int off = q * 1024 + lane * 16;
          w[q] = off < valid ? *reinterpret_cast<const lds_u32x4 *>(pg + off) : mk_u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int b = 0; b < MK_RB_MAXB; ++b) {
          if (b >= B) continue;
          const lds_float *x = R.X + (size_t)b * g.K + kk * 2048;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int off = q * 1024 + lane * 16;
            const bool on = off < valid;
            const lds_f32x4 *x4 = reinterpret_cast<const lds_f32x4 *>(x + q * 512 + lane * 8);
            const mk_f32x4 z = {0.f, 0.f, 0.f, 0.f};
            a[b] = dot8(w[q], on ? x4[0] : z, on ? x4[1] : z, a[b]);
          }
        }
        page_free(R, slot, s);
        ++s;
        if (++slot == R.np) slot = 0;
      }
#pragma unroll
      for (int b = 0; b < MK_RB_MAXB; ++b) tot[h][b] = b < B ? wave_total(a[b]) : 0.f;
    }
    float r[MK_RB_MAXB];
#pragma unroll
    for (int b = 0; b < MK_RB_MAXB; ++b) r[b] = TWO ? silu_mul(tot[0][b], tot[1][b]) : tot[0][b];
    rowres_put<MK_RB_MAXB>(R, rr, r, B);
    s += (uint32_t)ustep;
    slot = ring_add(slot, ustep, R.np);
  }
  rowres_flush<MK_RB_MAXB>(R, rr, B);
  return true;
}

// wave partials of attention live after q | k | v in X: [NCW][G][d + 2]
MKD lds_float *attn_wpart(const MkRole &R, int cw) {
  const int d = R.P.d, G = R.P.G;
  return R.X + (size_t)(G + 2) * d + (size_t)cw * G * (d + 2);
}


// ---------------------------------------------------- attention on MFMA
//
// Decode attention over this instruction's key blocks (the flash-decoding
// split of the megakernel page, section 2.6's attention instruction).  A
// key block is one 4 KiB page: 32 positions for d = 64, 16 for d = 128.
// Scores and the probability-weighted values are bf16 matrix-core products
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//   scores  S[t][h] = sum_k K[t][k] q[h][k]   (M = 16 positions, N = heads)
//   output  O[h][n] = sum_t P[h][t] V[t][n]   (M = heads, N = 16 dims, K = 32 positions)
// Keys and values are bf16 already; the fp32 queries and probabilities are
// split into bf16 high and low parts (two products each), so the products
// keep about 16 significant bits, like the fp32 dot products they replace.
// Heads beyond the group size are zero padding.  Operand layout (one lane
// i of 64): A[m = i % 16][k = 8 (i / 16) + j], B[k = 8 (i / 16) + j][n = i % 16],
// D[m = 4 (i / 16) + j][n = i % 16].  The contraction index k may be mapped
// to dims or positions in any order both operands share: scores use
// dim = (d/4)(i/16) + 8 s + j for k-step s, so a lane reads one contiguous
// run of its key row; the value product maps k to position
// t = j < 4 ? 4 (i/16) + j : 16 + 4 (i/16) + (j - 4), which is exactly where
// the score product left each probability, so no lanes exchange data.



template <int D>
MKD bool attn_instr_d(const MkRole &R, const MkGeo &g, uint32_t seq0, int slot0, int cw) {
  constexpr int KS = D / 32, NT = D / 16, BP = MK_PAGE / (2 * D), NTILE = BP / 16, DQ = D / 4;
  const int lane = threadIdx.x & 63;
  const int G = R.P.G;
  const int col = lane & 15, qd = lane >> 4;
  // queries (pre-scaled by log2(e)/sqrt(d)) as the B operand, high and low parts
  mk_u32x4 qhi[KS], qlo[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = col < G ? R.X[col * D + DQ * qd + 8 * s + e] : 0.f;
    split_hi_lo(x, qhi[s], qlo[s]);
  }
  const lds_float *kn = R.X + G * D, *vn = kn + D;  // this step's key and value (bf16-exact)
  float m = -INFINITY, l = 0.f;                     // running max / partial sum of head `col`
  mk_f32x4v o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = mk_f32x4v{0.f, 0.f, 0.f, 0.f};
  uint32_t s = seq0 + (uint32_t)(cw * 2);
  int slot = ring_add(slot0, cw * 2, R.np);
  for (int u = cw; u < g.n_units; u += MK_NCW) {
    const int ta = g.t0 + u * BP;
    const int npos = min(BP, g.t1 - ta);
    const int vslot = slot + 1 == R.np ? 0 : slot + 1;
    if (!page_wait(R, slot, s) || !page_wait(R, vslot, s + 1)) return false;
    lds_char *kp = R.ring + (size_t)slot * MK_PAGE, *vp = R.ring + (size_t)vslot * MK_PAGE;
    if (ta <= g.p && g.p < ta + npos) {
      // the page holds the slot's previous contents: write this step's key and value
      const int row = g.p - ta;
      for (int e = lane; e < D; e += 64) {
        const int off = row * 2 * D + kv_swz(row, 2 * e);
        *reinterpret_cast<lds_u16 *>(kp + off) = f2bf(kn[e]);
        *reinterpret_cast<lds_u16 *>(vp + off) = f2bf(vn[e]);
      }
    }
    // scores, one 16-position tile at a time
    float sc[2][4];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      if (T < NTILE) {
        mk_f32x4v acc = {0.f, 0.f, 0.f, 0.f};
        const int t = 16 * T + col;
        const lds_char *kr = kp + t * 2 * D;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
          const mk_bf16x8 a = as_bf16x8(*reinterpret_cast<const lds_u32x4 *>(kr + kv_swz(t, 2 * DQ * qd + 16 * s2)));
          acc = mfma16x16x32(a, as_bf16x8(qhi[s2]), acc);
          acc = mfma16x16x32(a, as_bf16x8(qlo[s2]), acc);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[T][j] = 16 * T + 4 * qd + j < npos ? acc[j] : -INFINITY;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[T][j] = -INFINITY;
      }
    }
    page_free(R, slot, s);
    // online softmax for head `col` (its four lane rows share the max)
    float mb = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mb = max_x16(mb);
    mb = max_x32(mb);
    const float mn = fmaxf(m, mb);
    const float c = m == mn ? 1.f : exp2_fast(m - mn);
    float pr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = sc[j >> 2][j & 3];
      pr[j] = v == -INFINITY ? 0.f : exp2_fast(v - mn);
    }
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ls += pr[j];
    l = fmaf(l, c, ls);
    m = mn;
    // rescale the output rows: row h of the output sits in register h % 4 of
    // lanes 16 (h / 4) ..; the real heads (h < 4) are in the first 16 lanes
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float cj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), j));
#pragma unroll
      for (int n = 0; n < NT; ++n) o[n][j] *= cj;
    }
    // probabilities as the A operand (rows: heads, k: positions t(qd, j))
    mk_u32x4 phi, plo;
    split_hi_lo(pr, phi, plo);
    // values as the B operand: column = dim, k = position t(qd, j)
    int vrow[8];
    bool von[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = j < 4 ? 4 * qd + j : 16 + 4 * qd + (j - 4);
      von[j] = t < npos;
      vrow[j] = min(t, BP - 1);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int dim = 16 * n + col;
      uint32_t vv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t raw = *reinterpret_cast<const lds_u16 *>(vp + vrow[j] * 2 * D + kv_swz(vrow[j], 2 * dim));
        vv[j] = von[j] ? raw : 0u;
      }
      const mk_u32x4 vw = {vv[0] | (vv[1] << 16), vv[2] | (vv[3] << 16), vv[4] | (vv[5] << 16), vv[6] | (vv[7] << 16)};
      o[n] = mfma16x16x32(as_bf16x8(phi), as_bf16x8(vw), o[n]);
      o[n] = mfma16x16x32(as_bf16x8(plo), as_bf16x8(vw), o[n]);
    }
    page_free(R, vslot, s + 1);
    s += (uint32_t)(MK_NCW * 2);
    slot = ring_add(slot, MK_NCW * 2, R.np);
  }
  // this wave's partial per head: max, sum, unnormalised output (base-2 scores)
  l = sum_x16(l);
  l = sum_x32(l);
  lds_float *wp = attn_wpart(R, cw);
  if (lane < G) {
    wp[lane * (D + 2)] = m;
    wp[lane * (D + 2) + 1] = l;
  }
  if (qd == 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < G) wp[j * (D + 2) + 2 + 16 * n + col] = o[n][j];
  }
  return true;
}

MKD bool attn_instr(const MkRole &R, const MkGeo &g, uint32_t seq0, int slot0, int cw) {
  return g.d == 64 ? attn_instr_d<64>(R, g, seq0, slot0, cw) : attn_instr_d<128>(R, g, seq0, slot0, cw);
}

// ------------------------------------------------------- sync epilogues

MKD void argmax_merge(float &v, int &i, float ov, int oi) {
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// returns 1: trigger the event, 0: do not, -1: abort
MKD int sync_epilogue(const MkRole &R, const MkInstr &in, const MkGeo &g, const MkAct &A) {
  MkProgC &P = R.P;
  MkStepC &S = R.S;
  const int lane = threadIdx.x & 63;
  const int B = S.batch, l = in.layer;
  if (in.op == MKOP_ATTN && g.p < 0) {
    // sequence slot beyond this step's batch: only the event and ticket protocol
    if (in.nsplit == 1) return 1;
    uint32_t old = 0;
    if (lane == 0) old = addcu(P.tickets + in.ticket, 1u);
    old = __builtin_amdgcn_readfirstlane(old);
    return old + 1u == (S.epoch + 1u) * (uint32_t)in.nsplit ? 1 : 0;
  }
  if (in.op == MKOP_ATTN) {
    const int b = in.r0, gg = in.r1, d = P.d, G = P.G, NS = in.nsplit;
    float *out = A.attn + ((size_t)l * P.B_max + b) * P.nq * d + (size_t)gg * G * d;
    float *part = P.part + ((((size_t)l * P.B_max + b) * P.nkv + gg) * NS) * G * (d + 2);
    // merge the compute waves' partials (base-2 scores)
    for (int e = lane; e < G * d; e += 64) {
      const int j = e / d, i = e - j * d;
      float mx = -INFINITY;
      for (int w = 0; w < MK_NCW; ++w) mx = fmaxf(mx, attn_wpart(R, w)[j * (d + 2)]);
      float z = 0.f, o = 0.f;
      for (int w = 0; w < MK_NCW; ++w) {
        const lds_float *wp = attn_wpart(R, w) + j * (d + 2);
        const float c = wp[0] == -INFINITY ? 0.f : exp2_fast(wp[0] - mx);
        z = fmaf(wp[1], c, z);
        o = fmaf(wp[2 + i], c, o);
      }
      if (NS == 1) {
        stc(out + e, o / z);
      } else {
        float *pp = part + ((size_t)in.split * G + j) * (d + 2);
        stc(pp + 2 + i, o);
        if (i == 0) {
          stc(pp, mx);
          stc(pp + 1, z);
        }
      }
    }
    if (NS == 1) return 1;
    wait_vm();
    uint32_t old = 0;
    if (lane == 0) old = addcu(P.tickets + in.ticket, 1u);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old + 1u != (S.epoch + 1u) * (uint32_t)NS) return 0;
    for (int e = lane; e < G * d; e += 64) {
      const int j = e / d, i = e - j * d;
      stc(out + e, merge_splits(part, NS, G, d, j, i));
    }
    return 1;
  }
  // projections: coalesced stores of the compute waves' row results
  const int n = g.n_units;
  float lmv[MK_RB_MAXB];
  int lmi[MK_RB_MAXB];
  for (int b = 0; b < B; ++b) {
    const lds_float *ob = R.out + (size_t)b * P.out_stride;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int u = lane; u < n; u += 64) {
      const float v = ob[u];
      const int r = in.r0 + u;
      switch (in.op) {
        case MKOP_QKV:
          stc(A.qkv + ((size_t)l * P.B_max + b) * ((P.nq + 2 * P.nkv) * P.d) + r, v);
          break;
        case MKOP_OPROJ:
          stc(A.xmid + ((size_t)l * P.B_max + b) * P.H + r, R.resid[(size_t)b * n + u] + v);
          break;
        case MKOP_GATEUP:
          stc(A.hbuf + ((size_t)l * P.B_max + b) * P.I + r, v);
          break;
        case MKOP_DOWN:
          stc(A.xout + ((size_t)l * P.B_max + b) * P.H + r, R.resid[(size_t)b * n + u] + v);
          break;
        case MKOP_LMHEAD:
          gst(S.logits + (size_t)b * P.V + r, v);
          argmax_merge(bv, bi, v, r);
          break;
      }
    }
    if (in.op == MKOP_LMHEAD) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) argmax_merge(bv, bi, __shfl_xor(bv, o, 64), __shfl_xor(bi, o, 64));
      if (b < MK_RB_MAXB) {
        lmv[b] = bv;
        lmi[b] = bi;
      }
    }
  }
  if (in.op != MKOP_LMHEAD) return 1;
  if (lane == 0) {
    for (int b = 0; b < B && b < MK_RB_MAXB; ++b) {
      stc(P.lm_val + (size_t)in.part * P.B_max + b, lmv[b]);
      stci(P.lm_idx + (size_t)in.part * P.B_max + b, lmi[b]);
    }
  }
  wait_vm();
  uint32_t old = 0;
  if (lane == 0) old = addcu(P.tickets + in.ticket, 1u);
  old = __builtin_amdgcn_readfirstlane(old);
  if (old + 1u != (S.epoch + 1u) * (uint32_t)P.n_lm_parts) return 0;
  // last arriver: merge every instruction's (max, index) pair, lanes in parallel
  for (int b = 0; b < B; ++b) {
    float v = -INFINITY;
    int ix = 0x7fffffff;
    for (int k = lane; k < P.n_lm_parts; k += 64)
      argmax_merge(v, ix, ldc(P.lm_val + (size_t)k * P.B_max + b), ldci(P.lm_idx + (size_t)k * P.B_max + b));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) argmax_merge(v, ix, __shfl_xor(v, o, 64), __shfl_xor(ix, o, 64));
    if (lane == 0) {
      if (ix == 0x7fffffff) ix = 0;
      if (S.next) gst(S.next + b, ix);
      if (S.flags & 1u) {
        gst(S.tokens + b, ix);
        gst(S.positions + b, R.ctl->pos[b] + 1);
      }
    }
  }
  return 0;
}

// ------------------------------------------------------- role loops

// wave-level dependency wait (counter or flag mode)
MKD bool wave_wait_event(const MkRole &R, int ev) {
  MkProgC &P = R.P;
  MkStepC &S = R.S;
  const int lane = threadIdx.x & 63;
  uint64_t t0 = 0;
  uint32_t spins = 0;
  while (true) {
    bool ready;
    if (P.sync_mode == 0) {
      const uint32_t need = (S.epoch + 1u) * (uint32_t)P.ev_count[ev];
      ready = (int32_t)(__builtin_amdgcn_readfirstlane(ctr_total(P, ev)) - need) >= 0;
    } else {
      const uint32_t want = S.epoch + 1u;
      const int n = P.ev_count[ev];
      const uint32_t *f = P.flags + P.ev_flag_base[ev];
      bool mine = true;
      for (int k = lane; k < n; k += 64) mine = mine && ((int32_t)(ldcu(f + k) - want) >= 0);
      ready = __all(mine);
    }
    if (ready) return true;
    if (spins == 0) t0 = __builtin_amdgcn_s_memrealtime();
    __builtin_amdgcn_s_sleep(1);
    if ((++spins & 31u) == 0 && !poll_check(R, t0, ev)) return false;
  }
}

MKD void wave_signal_event(const MkRole &R, int ev, int slot) {
  MkProgC &P = R.P;
  if ((threadIdx.x & 63) != 0) return;
  if (P.sync_mode == 0)
    ctr_bump(P, ev);
  else
    stcu(P.flags + P.ev_flag_base[ev] + slot, R.S.epoch + 1u);
}

template <bool FULL, bool SWZ>
MKD bool loader_instr(const MkRole &R, LoaderState &L, const MkGeo &g, uint32_t seq) {
  const uint32_t npg = (uint32_t)(g.n_units * g.ppu);
  uint32_t j = L.s - seq;  // first page of this instruction with the loader's parity
  if (j >= npg) return true;
  int u = (int)(j / (uint32_t)g.ppu);
  const int rem = (int)(j - (uint32_t)u * (uint32_t)g.ppu);
  int h = rem / g.ppr, kk = rem - h * g.ppr;
  const char *row0 = g.src0 + (size_t)u * g.ustride;
  const char *row1 = g.nh > 1 ? g.src1 + (size_t)u * g.ustride : row0;
  for (; j < npg; j += MK_NLW) {
    const char *src = (h ? row1 : row0) + (size_t)kk * MK_PAGE;
    const int valid = FULL ? MK_PAGE : mk_page_valid(g, u, kk);
    if (!loader_page<FULL, SWZ>(R, L, src, valid, 2 * g.d)) return false;
#pragma unroll
    for (int i = 0; i < MK_NLW; ++i) {
      if (++kk == g.ppr) {
        kk = 0;
        if (++h == g.nh) {
          h = 0;
          ++u;
          row0 += g.ustride;
          row1 += g.ustride;
        }
      }
    }
  }
  return true;
}

// ------------------------------------------------------- role entries
//
// Each role is a separate function (not inlined into the kernel) so that the
// register allocator sees one role's loop at a time; inlining all three
// into one body made it spill hundreds of scalar registers into vector
// lanes, which the hot loops then paid for.  Arguments of a called
// function arrive in vector registers, so they are made wave-uniform
// (readfirstlane) again, and the program and step records are read through
// the constant address space (scalar loads).

extern __shared__ __attribute__((aligned(16))) char mk_role_lds[];

// A role's wave ends inside its function: the functions never return, so
// they need not save the registers a returning call must preserve.
[[noreturn]] MKD void mk_end() {
  __builtin_amdgcn_endpgm();
}

MKD int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
MKD const void *uni_ptr(const void *p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void *)(((uint64_t)hi << 32) | lo);
}

// lb: LDS address of the dynamic allocation, taken in the kernel and passed
// down (inside a called function the address would come from a per-kernel
// table, which the compiler reloads instead of keeping in a register)
MKD MkRole make_role(MkProgC &P, MkStepC &S, uint32_t lb) {
  const int par = (P.sync_mode == MK_SYNC_SENTINEL && !S.multi) ? (int)(S.epoch & 1u) : 0;
  return MkRole{P,
                S,
                (MkCtl3 *)(size_t)lb,
                (lds_float *)(size_t)(lb + P.lds_x),
                (lds_float *)(size_t)(lb + P.lds_resid),
                (lds_float *)(size_t)(lb + P.lds_out),
                (lds_char *)(size_t)(lb + P.lds_ring),
                P.n_pages,
                par};
}

[[noreturn]] __device__ __noinline__ void role_loader_entry(const MkProgram *Pg, const MkStep *Sg, uint32_t lb, int first, int n,
                                                int lid) {
  MkProgC &P = *(MkProgC *)uni_ptr(Pg);
  MkStepC &S = *(MkStepC *)uni_ptr(Sg);
  first = uni(first);
  n = uni(n);
  lid = uni(lid);
  const MkRole R = make_role(P, S, (uint32_t)uni((int)lb));
  LoaderState L{(uint32_t)lid, lid, 0u, 0, 0};
  uint32_t seq = 0;
  for (int k = 0; k < n; ++k) {
    const MkInstr in = cld(&P.instr[first + k]);
    MkGeo g;
    if (!mk_geo(P, S, R.ctl, in, g)) {
      role_abort(R);
      break;
    }
    const bool ok = in.op == MKOP_ATTN ? loader_instr<false, true>(R, L, g, seq)
                    : g.full          ? loader_instr<true, false>(R, L, g, seq)
                                      : loader_instr<false, false>(R, L, g, seq);
    if (!ok) mk_end();
    seq += (uint32_t)(g.n_units * g.ppu);
  }
  while (L.inflight > 0) loader_publish_one(R, L);
  mk_end();
}

[[noreturn]] __device__ __noinline__ void role_compute_entry(const MkProgram *Pg, const MkStep *Sg, uint32_t lb, int first, int n,
                                                 int cw) {
  MkProgC &P = *(MkProgC *)uni_ptr(Pg);
  MkStepC &S = *(MkStepC *)uni_ptr(Sg);
  first = uni(first);
  n = uni(n);
  cw = uni(cw);
  const MkRole R = make_role(P, S, (uint32_t)uni((int)lb));
  uint32_t seq = 0;
  int slot0 = 0;
  const int B = S.batch;
  for (int k = 0; k < n; ++k) {
    const MkInstr in = cld(&P.instr[first + k]);
    MkGeo g;
    if (!mk_geo(P, S, R.ctl, in, g)) {
      role_abort(R);
      mk_end();
    }
    if (!role_wait(R, &R.ctl->x_ready, (uint32_t)k + 1u, true)) mk_end();
    bool ok;
    const bool two = in.op == MKOP_GATEUP;
    if (in.op == MKOP_ATTN) ok = attn_instr(R, g, seq, slot0, cw);
    else if (B == 1 && g.full && g.ppr == 1) ok = two ? gemv_fast<true, true>(R, g, seq, slot0, cw)
                                                      : gemv_fast<true, false>(R, g, seq, slot0, cw);
    else if (B == 1 && g.full) ok = two ? gemv_fast<false, true>(R, g, seq, slot0, cw)
                                        : gemv_fast<false, false>(R, g, seq, slot0, cw);
    else ok = two ? gemv_general<true>(R, g, seq, slot0, cw, B) : gemv_general<false>(R, g, seq, slot0, cw, B);
    if (!ok) mk_end();
    if ((threadIdx.x & 63) == 0) lds_add(&R.ctl->cw_done, 1u);  // one increment per wave
    const uint32_t npg = (uint32_t)(g.n_units * g.ppu);
    seq += npg;
    slot0 = (int)(((uint32_t)slot0 + npg) % (uint32_t)R.np);
  }
  mk_end();
}

[[noreturn]] __device__ __noinline__ void role_sync_entry(const MkProgram *Pg, const MkStep *Sg, uint32_t lb, int first, int n) {
  MkProgC &P = *(MkProgC *)uni_ptr(Pg);
  MkStepC &S = *(MkStepC *)uni_ptr(Sg);
  first = uni(first);
  n = uni(n);
  const MkRole R = make_role(P, S, (uint32_t)uni((int)lb));
  const MkAct A = mk_act(P, R.par);
  const bool sent = P.sync_mode == MK_SYNC_SENTINEL && !S.multi;
  if (sent) {
    // reset this CU's share of the other parity's activations to the sentinel
    float *other = P.qkv + (size_t)(R.par ^ 1) * P.par_stride;
    const size_t per = (P.par_stride + P.n_cu - 1) / P.n_cu;
    const size_t lo = (size_t)blockIdx.x * per, hi = min(lo + per, (size_t)P.par_stride);
    for (size_t i = lo + (threadIdx.x & 63); i < hi; i += 64) stcu(reinterpret_cast<uint32_t *>(other) + i, MK_SENTINEL);
  }
  for (int k = 0; k < n; ++k) {
    const MkInstr in = cld(&P.instr[first + k]);
    MkGeo g;
    if (!mk_geo(P, S, R.ctl, in, g)) {
      if ((threadIdx.x & 63) == 0) mk_raise(P, MK_E_INPUT, 1000 + in.r0);
      role_abort(R);
      mk_end();
    }
    const uint64_t tw = P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    StagePre pre;  // ahead of the wait
    if (normed_op(in.op)) load_bf16_chunks(norm_gain(P, in), P.H, pre.gain);
    if (in.op == MKOP_ATTN && g.p >= 0) {
      const int half = P.d / 2, i = (threadIdx.x & 63) % half;
      pre.rc = gld(P.rope + (size_t)g.p * P.d + 2 * i);
      pre.rs = gld(P.rope + (size_t)g.p * P.d + 2 * i + 1);
    }
    if (!S.multi && !sent && in.wait_ev >= 0 && !wave_wait_event(R, in.wait_ev)) mk_end();
    if (!role_wait(R, &R.ctl->cw_done, (uint32_t)k * MK_NCW)) mk_end();  // X is free again
    if (!sync_stage(R, in, g, A, sent, pre)) mk_end();
    lds_st(&R.ctl->x_ready, (uint32_t)k + 1u);
    const uint64_t ts = P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    if (!role_wait(R, &R.ctl->cw_done, (uint32_t)(k + 1) * MK_NCW, true)) mk_end();
    const uint64_t tc = P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    const int sig = sync_epilogue(R, in, g, A);
    if (sig < 0) {
      role_abort(R);
      mk_end();
    }
    if (sig && !S.multi && !sent && in.sig_ev >= 0) {
      wait_vm();
      wave_signal_event(R, in.sig_ev, in.sig_slot);
    }
    if (P.trace && (threadIdx.x & 63) == 0) {
      uint64_t *r = P.trace + (size_t)(first + k) * 8;
      r[0] = tw;
      r[1] = ts;
      r[2] = __builtin_amdgcn_s_memrealtime();
      r[3] = ((uint64_t)blockIdx.x << 32) | S.epoch;
      // stall counters so far in this launch (cumulative over the CU's list)
      r[4] = lds_ld(&R.ctl->st_load_block);
      r[5] = lds_ld(&R.ctl->st_page_wait);
      r[6] = (uint64_t)(g.n_units * g.ppu);
      r[7] = tc;  // compute waves done; the epilogue follows
    }
  }
  mk_end();
}

// Entry used by both kernels: run instructions [first, first + n) of the
// program with roles.  Sg points at the kernel's step argument in the
// kernarg segment (valid for the whole launch).
MKD void role_run(const MkProgram *Pg, const MkStep *Sg, int first, int n) {
  MkCtl *ctl = reinterpret_cast<MkCtl *>(mk_role_lds);
  for (int i = threadIdx.x; i < (int)(sizeof(MkCtl) / 4); i += MK_BLOCK) reinterpret_cast<uint32_t *>(ctl)[i] = 0;
  __syncthreads();
  if ((int)threadIdx.x < Sg->batch) ctl->pos[threadIdx.x] = gld(Sg->positions + threadIdx.x);
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  uint32_t lb = (uint32_t)(size_t)(lds_char *)mk_role_lds;
  asm volatile("" : "+s"(lb));  // an opaque value, so it is not propagated back into the callees as a constant
  if (wave < MK_NLW) role_loader_entry(Pg, Sg, lb, first, n, wave);
  else if (wave == MK_SYNCW) role_sync_entry(Pg, Sg, lb, first, n);
  else role_compute_entry(Pg, Sg, lb, first, n, wave - MK_NLW - 1);
}
