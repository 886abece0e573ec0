// Per-op staging (sync wave), compute (compute waves) and epilogue (sync
// wave) of the role-specialised engine, and the three role loops.
#pragma once
#include "mk_roles.h"

#define MK_SYNC_SENTINEL MKSYNC_SENTINEL
#define MK_XCH 16  // 16-byte chunks per lane the sync wave stages in one round (4096 floats)

// ----------------------------------------------- device-coherent vector loads

MKD __amdgpu_buffer_rsrc_t mk_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}
// 16-byte load with device scope (sc1): coherent across XCDs
MKD mk_u32x4 ldc16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16);
}

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
MKD bool sync_stage(const MkRole &R, const MkInstr &in, const MkGeo &g, const MkAct &A, bool sent,
                    const uint32_t (&gain)[MK_XCH][2]) {
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
        norm_store(R.X + (size_t)b * H, H, v, gain, P.eps);
      }
      return true;
    }
    case MKOP_OPROJ:
    case MKOP_DOWN: {
      const int K = g.K, nr = in.r1 - in.r0;
      for (int b = 0; b < B; ++b) {
        lds_float *rd = R.resid + (size_t)b * nr;
        if (in.op == MKOP_OPROJ && l == 0) {
          const int tok = gld(S.tokens + b);
          if (tok < 0 || tok >= P.V) {
            if (lane == 0) mk_raise(P, MK_E_INPUT, b);
            role_abort(R);
            return false;
          }
          for (int i = lane; i < nr; i += 64) rd[i] = bf2f(gld(P.embed + (size_t)tok * H + in.r0 + i));
        } else {
          // residual rows first: they were complete before this instruction's input
          const float *rs = in.op == MKOP_OPROJ ? A.xout + ((size_t)(l - 1) * P.B_max + b) * H + in.r0
                                                : A.xmid + ((size_t)l * P.B_max + b) * H + in.r0;
          if (!stage_scalars(R, rd, rs, nr, sent)) return false;
        }
        const float *src = in.op == MKOP_OPROJ ? A.attn + ((size_t)l * P.B_max + b) * K
                                               : A.hbuf + ((size_t)l * P.B_max + b) * K;
        if (!stage_vec(R, R.X + (size_t)b * K, src, K, sent)) return false;
      }
      return true;
    }
    case MKOP_ATTN: {
      const int b = in.r0, gg = in.r1, d = P.d, G = P.G, half = d / 2;
      const int R0 = (P.nq + 2 * P.nkv) * d;
      const float *qkv = A.qkv + ((size_t)l * P.B_max + b) * R0;
      lds_float *q = R.X, *kc = R.X + G * d, *vc = kc + d;
      if (!stage_vec(R, q, qkv + (size_t)gg * G * d, G * d, sent)) return false;
      if (!stage_vec(R, kc, qkv + (size_t)P.nq * d + (size_t)gg * d, d, sent)) return false;
      if (!stage_vec(R, vc, qkv + (size_t)(P.nq + P.nkv) * d + (size_t)gg * d, d, sent)) return false;
      const float *cs = P.rope + (size_t)g.p * d;  // read below through gld
      // queries are pre-scaled by log2(e) / sqrt(d): scores come out in base 2
      const float qs = 1.4426950408889634f / sqrtf((float)d);
      for (int e = lane; e < (G + 1) * half; e += 64) {
        const int j = e / half, i = e - j * half;  // j == G is the key
        lds_float *u = j < G ? q + j * d : kc;
        const float a = u[i], c = u[i + half], co = gld(cs + 2 * i), si = gld(cs + 2 * i + 1);
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

// sum over the lpp (8 or 16) consecutive lanes that hold one key position
MKD float group_sum(float v, int lpp) {
  v += dpp_term<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_term<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_term<0x141, 0xF>(v);  // row_half_mirror: the other quad of the half row
  if (lpp == 16) v += dpp_term<0x140, 0xF>(v);  // row_mirror: the other half row
  return v;
}

MKD float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Decode attention over this instruction's key blocks (flash-decoding split
// of the megakernel page, section 2.6's attention instruction).  Lanes come
// in groups of lpp = d/8, one group per key position, 8 dims per lane; each
// group keeps its own running max / sum / output for the positions it saw
// (scores in base 2: the staged queries carry log2(e)/sqrt(d)), and the
// groups of the wave are merged at the end into one partial per q head.
MKD bool attn_instr(const MkRole &R, const MkGeo &g, uint32_t seq0, int slot0, int cw) {
  const int lane = threadIdx.x & 63;
  const int d = g.d, G = R.P.G;
  const int lpp = d / 8, ppi = 64 / lpp;
  const int c8 = (lane % lpp) * 8, pin = lane / lpp;
  float qv[MK_MAX_GROUP][8];
#pragma unroll
  for (int j = 0; j < MK_MAX_GROUP; ++j) {
    const lds_f32x4 *q4 = reinterpret_cast<const lds_f32x4 *>(R.X + j * d + c8);
    const mk_f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const mk_f32x4 a = j < G ? q4[0] : z;
    const mk_f32x4 b = j < G ? q4[1] : z;
    qv[j][0] = a.x, qv[j][1] = a.y, qv[j][2] = a.z, qv[j][3] = a.w;
    qv[j][4] = b.x, qv[j][5] = b.y, qv[j][6] = b.z, qv[j][7] = b.w;
  }
  float m[MK_MAX_GROUP], l[MK_MAX_GROUP], o[MK_MAX_GROUP][8];
#pragma unroll
  for (int j = 0; j < MK_MAX_GROUP; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
  }
  const lds_float *kn = R.X + G * d, *vn = kn + d;  // this step's key and value (bf16-rounded)
  uint32_t s = seq0 + (uint32_t)(cw * 2);
  int slot = ring_add(slot0, cw * 2, R.np);
  for (int u = cw; u < g.n_units; u += MK_NCW) {
    const int ta = g.t0 + u * g.bp;
    const int npos = min(g.bp, g.t1 - ta);
    const bool here = ta <= g.p && g.p < ta + npos;  // the block holds this step's position
    const int vslot = slot + 1 == R.np ? 0 : slot + 1;
    if (!page_wait(R, slot, s) || !page_wait(R, vslot, s + 1)) return false;
    const lds_char *kp = R.ring + (size_t)slot * MK_PAGE, *vp = R.ring + (size_t)vslot * MK_PAGE;
    float sc[4][MK_MAX_GROUP];
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int row = pass * ppi + pin;
      const mk_u32x4 kw = row < npos ? *reinterpret_cast<const lds_u32x4 *>(kp + (size_t)row * 2 * d + c8 * 2)
                                     : mk_u32x4{0, 0, 0, 0};
      float k8[8] = {bf_lo(kw.x), bf_hi(kw.x), bf_lo(kw.y), bf_hi(kw.y),
                     bf_lo(kw.z), bf_hi(kw.z), bf_lo(kw.w), bf_hi(kw.w)};
      if (here && ta + row == g.p) {  // the page holds the slot's previous contents
#pragma unroll
        for (int e = 0; e < 8; ++e) k8[e] = kn[c8 + e];
      }
#pragma unroll
      for (int j = 0; j < MK_MAX_GROUP; ++j) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(qv[j][e], k8[e], a);
        a = group_sum(a, lpp);
        sc[pass][j] = row < npos ? a : -INFINITY;
      }
    }
    page_free(R, slot, s);
    float pr[4][MK_MAX_GROUP];
#pragma unroll
    for (int j = 0; j < MK_MAX_GROUP; ++j) {
      const float mb = fmaxf(fmaxf(sc[0][j], sc[1][j]), fmaxf(sc[2][j], sc[3][j]));
      const float mn = fmaxf(m[j], mb);
      const float c = m[j] == mn ? 1.f : exp2_fast(m[j] - mn);
      float ls = 0.f;
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        pr[pass][j] = sc[pass][j] == -INFINITY ? 0.f : exp2_fast(sc[pass][j] - mn);
        ls += pr[pass][j];
      }
      l[j] = fmaf(l[j], c, ls);
      m[j] = mn;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] *= c;
    }
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int row = pass * ppi + pin;
      const mk_u32x4 vw = row < npos ? *reinterpret_cast<const lds_u32x4 *>(vp + (size_t)row * 2 * d + c8 * 2)
                                     : mk_u32x4{0, 0, 0, 0};
      float v8[8] = {bf_lo(vw.x), bf_hi(vw.x), bf_lo(vw.y), bf_hi(vw.y),
                     bf_lo(vw.z), bf_hi(vw.z), bf_lo(vw.w), bf_hi(vw.w)};
      if (here && ta + row == g.p) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] = vn[c8 + e];
      }
#pragma unroll
      for (int j = 0; j < MK_MAX_GROUP; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = fmaf(pr[pass][j], v8[e], o[j][e]);
    }
    page_free(R, vslot, s + 1);
    s += (uint32_t)(MK_NCW * 2);
    slot = ring_add(slot, MK_NCW * 2, R.np);
  }
  // merge the lane groups: rescale to the wave max, then sum groups lane-wise
  lds_float *wp = attn_wpart(R, cw);
#pragma unroll
  for (int j = 0; j < MK_MAX_GROUP; ++j) {
    if (j >= G) continue;
    const float M = wave_max_all(m[j]);
    const float f = m[j] == -INFINITY ? 0.f : exp2_fast(m[j] - M);
    const float L = wave_total(l[j] * f) * (1.0f / (float)lpp);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = o[j][e] * f;
      if (lpp == 8) v += dpp_term<0x128, 0xF>(v);  // row_ror:8: the other 8-lane group of the row
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      o[j][e] = v;
    }
    if (lane < lpp) {
#pragma unroll
      for (int e = 0; e < 8; ++e) wp[j * (d + 2) + 2 + c8 + e] = o[j][e];
    }
    if (lane == 0) {
      wp[j * (d + 2)] = M;
      wp[j * (d + 2) + 1] = L;
    }
  }
  return true;
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
      float mx = -INFINITY;
      for (int s2 = 0; s2 < NS; ++s2) mx = fmaxf(mx, ldc(part + ((size_t)s2 * G + j) * (d + 2)));
      float z = 0.f, o = 0.f;
      for (int s2 = 0; s2 < NS; ++s2) {
        const float *pp = part + ((size_t)s2 * G + j) * (d + 2);
        const float ms = ldc(pp);
        const float c = ms == -INFINITY ? 0.f : exp2_fast(ms - mx);
        z = fmaf(ldc(pp + 1), c, z);
        o = fmaf(ldc(pp + 2 + i), c, o);
      }
      stc(out + e, o / z);
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
  if (lane < B) {
    const int b = lane;
    float v = -INFINITY;
    int ix = 0x7fffffff;
    for (int k = 0; k < P.n_lm_parts; ++k)
      argmax_merge(v, ix, ldc(P.lm_val + (size_t)k * P.B_max + b), ldci(P.lm_idx + (size_t)k * P.B_max + b));
    if (ix == 0x7fffffff) ix = 0;
    if (S.next) gst(S.next + b, ix);
    if (S.flags & 1u) {
      gst(S.tokens + b, ix);
      gst(S.positions + b, R.ctl->pos[b] + 1);
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
      ready = (int32_t)(__builtin_amdgcn_readfirstlane(ldcu(P.ctr + ev)) - need) >= 0;
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
    addcu(P.ctr + ev, 1u);
  else
    stcu(P.flags + P.ev_flag_base[ev] + slot, R.S.epoch + 1u);
}

template <bool FULL>
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
    if (!loader_page<FULL>(R, L, src, valid)) return false;
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

__device__ __noinline__ void role_loader_entry(const MkProgram *Pg, const MkStep *Sg, uint32_t lb, int first, int n,
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
    const bool ok = g.full ? loader_instr<true>(R, L, g, seq) : loader_instr<false>(R, L, g, seq);
    if (!ok) return;
    seq += (uint32_t)(g.n_units * g.ppu);
  }
  while (L.inflight > 0) loader_publish_one(R, L);
}

__device__ __noinline__ void role_compute_entry(const MkProgram *Pg, const MkStep *Sg, uint32_t lb, int first, int n,
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
      return;
    }
    if (!role_wait(R, &R.ctl->x_ready, (uint32_t)k + 1u, true)) return;
    bool ok;
    const bool two = in.op == MKOP_GATEUP;
    if (in.op == MKOP_ATTN) ok = attn_instr(R, g, seq, slot0, cw);
    else if (B == 1 && g.full && g.ppr == 1) ok = two ? gemv_fast<true, true>(R, g, seq, slot0, cw)
                                                      : gemv_fast<true, false>(R, g, seq, slot0, cw);
    else if (B == 1 && g.full) ok = two ? gemv_fast<false, true>(R, g, seq, slot0, cw)
                                        : gemv_fast<false, false>(R, g, seq, slot0, cw);
    else ok = two ? gemv_general<true>(R, g, seq, slot0, cw, B) : gemv_general<false>(R, g, seq, slot0, cw, B);
    if (!ok) return;
    if ((threadIdx.x & 63) == 0) lds_add(&R.ctl->cw_done, 1u);  // one increment per wave
    const uint32_t npg = (uint32_t)(g.n_units * g.ppu);
    seq += npg;
    slot0 = (int)(((uint32_t)slot0 + npg) % (uint32_t)R.np);
  }
}

__device__ __noinline__ void role_sync_entry(const MkProgram *Pg, const MkStep *Sg, uint32_t lb, int first, int n) {
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
      return;
    }
    const uint64_t tw = P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    uint32_t gain[MK_XCH][2];
    if (normed_op(in.op)) load_bf16_chunks(norm_gain(P, in), P.H, gain);  // ahead of the wait
    if (!S.multi && !sent && in.wait_ev >= 0 && !wave_wait_event(R, in.wait_ev)) return;
    if (!role_wait(R, &R.ctl->cw_done, (uint32_t)k * MK_NCW)) return;  // X is free again
    if (!sync_stage(R, in, g, A, sent, gain)) return;
    lds_st(&R.ctl->x_ready, (uint32_t)k + 1u);
    const uint64_t ts = P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    if (!role_wait(R, &R.ctl->cw_done, (uint32_t)(k + 1) * MK_NCW, true)) return;
    const int sig = sync_epilogue(R, in, g, A);
    if (sig < 0) {
      role_abort(R);
      return;
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
      r[7] = 0;
    }
  }
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
