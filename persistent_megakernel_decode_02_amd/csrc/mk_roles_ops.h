// Per-op staging (sync wave), compute (compute waves) and epilogue (sync
// wave) of the role-specialised engine, and the three role loops.
#pragma once
#include "mk_roles.h"

#define MK_SYNC_SENTINEL MKSYNC_SENTINEL

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
MKD MkAct mk_act(const MkProgram &P, int par) {
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

// One wave copies n floats (n % 4 == 0, src 16-byte aligned) from global to
// LDS with device-coherent 16-byte loads.  With `sentinel`, words still
// holding the sentinel are re-read until every word has been produced.
MKD bool stage_vec(const MkRole &R, float *dst, const float *src, int n, bool sentinel) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rs = mk_rsrc(src, (uint32_t)n * 4u);
  constexpr int NB = 4;
  for (int base = 0; base < n; base += 64 * 4 * NB) {
    mk_u32x4 v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int e = base + (j * 64 + lane) * 4;
      v[j] = ldc16(rs, e * 4);  // out-of-range offsets read 0 (buffer bounds)
    }
    if (sentinel) {
      uint64_t t0 = 0;
      uint32_t spins = 0;
      while (true) {
        bool miss = false;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int e = base + (j * 64 + lane) * 4;
          miss = miss || (e < n && has_sentinel(v[j]));
        }
        if (!__any(miss)) break;
        if (spins == 0) t0 = __builtin_amdgcn_s_memrealtime();
        __builtin_amdgcn_s_sleep(1);
        if ((++spins & 63u) == 0) {
          if (lds_ld(&R.ctl->abort) || mk_aborted(R.P)) {
            role_abort(R);
            return false;
          }
          if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)R.P.watchdog_ticks) {
            if (lane == 0) mk_raise(R.P, MK_E_TIMEOUT, 0x20000);
            role_abort(R);
            return false;
          }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int e = base + (j * 64 + lane) * 4;
          if (e < n && has_sentinel(v[j])) v[j] = ldc16(rs, e * 4);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int e = base + (j * 64 + lane) * 4;
      if (e < n) {
        float4 f = make_float4(__uint_as_float(v[j].x), __uint_as_float(v[j].y), __uint_as_float(v[j].z),
                               __uint_as_float(v[j].w));
        *reinterpret_cast<float4 *>(dst + e) = f;
      }
    }
  }
  return true;
}

// n scalar floats (any alignment), device-coherent, sentinel-checked
MKD bool stage_scalars(const MkRole &R, float *dst, const float *src, int n, bool sentinel) {
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
        if ((++spins & 63u) == 0) {
          if (lds_ld(&R.ctl->abort) || mk_aborted(R.P)) {
            role_abort(R);
            return false;
          }
          if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)R.P.watchdog_ticks) {
            if (lane == 0) mk_raise(R.P, MK_E_TIMEOUT, 0x20001);
            role_abort(R);
            return false;
          }
        }
        if (miss) v = ldc(src + i);
      }
    }
    if (i < n) dst[i] = v;
  }
  return true;
}

// In-place RMSNorm of one staged vector by one wave
MKD void wave_rmsnorm(float *x, int K, const uint16_t *gain, float eps) {
  const int lane = threadIdx.x & 63;
  float ss = 0.f;
  for (int i = lane; i < K; i += 64) ss = fmaf(x[i], x[i], ss);
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)K + eps);
  for (int i = lane; i < K; i += 64) x[i] = (x[i] * r) * bf2f(gld(gain + i));
}

// ------------------------------------------------------------ wave barrier
// (sync wave waiting on its own earlier LDS writes before publishing: the
// release store in lds_st orders them)

// ------------------------------------------------------- sync-wave staging

// returns false on abort (error already raised)
MKD bool sync_stage(const MkRole &R, const MkInstr &in, const MkGeo &g, const MkAct &A, bool sent) {
  const MkProgram &P = R.P;
  const MkStep &S = R.S;
  const int lane = threadIdx.x & 63;
  const int B = S.batch, H = P.H, l = in.layer;
  switch (in.op) {
    case MKOP_QKV:
    case MKOP_GATEUP:
    case MKOP_LMHEAD: {
      const uint16_t *gain = in.op == MKOP_QKV ? P.layers[l].attn_norm
                             : in.op == MKOP_GATEUP ? P.layers[l].mlp_norm : P.final_norm;
      for (int b = 0; b < B; ++b) {
        float *x = R.X + (size_t)b * H;
        if (in.op == MKOP_QKV && l == 0) {
          const int tok = gld(S.tokens + b);
          if (tok < 0 || tok >= P.V) {
            if (lane == 0) mk_raise(P, MK_E_INPUT, b);
            role_abort(R);
            return false;
          }
          const uint16_t *e = P.embed + (size_t)tok * H;
          for (int i = lane; i < H; i += 64) x[i] = bf2f(gld(e + i));
        } else {
          const float *src = in.op == MKOP_QKV ? A.xout + ((size_t)(l - 1) * P.B_max + b) * H
                             : in.op == MKOP_GATEUP ? A.xmid + ((size_t)l * P.B_max + b) * H
                                                    : A.xout + ((size_t)(P.L - 1) * P.B_max + b) * H;
          if (!stage_vec(R, x, src, H, sent)) return false;
        }
        wave_rmsnorm(x, H, gain, P.eps);
      }
      return true;
    }
    case MKOP_OPROJ:
    case MKOP_DOWN: {
      const int K = g.K, nr = in.r1 - in.r0;
      for (int b = 0; b < B; ++b) {
        const float *src = in.op == MKOP_OPROJ ? A.attn + ((size_t)l * P.B_max + b) * K
                                               : A.hbuf + ((size_t)l * P.B_max + b) * K;
        if (!stage_vec(R, R.X + (size_t)b * K, src, K, sent)) return false;
        float *rd = R.resid + (size_t)b * nr;
        if (in.op == MKOP_OPROJ && l == 0) {
          const int tok = gld(S.tokens + b);
          if (tok < 0 || tok >= P.V) {
            if (lane == 0) mk_raise(P, MK_E_INPUT, b);
            role_abort(R);
            return false;
          }
          for (int i = lane; i < nr; i += 64) rd[i] = bf2f(gld(P.embed + (size_t)tok * H + in.r0 + i));
        } else {
          const float *rs = in.op == MKOP_OPROJ ? A.xout + ((size_t)(l - 1) * P.B_max + b) * H + in.r0
                                                : A.xmid + ((size_t)l * P.B_max + b) * H + in.r0;
          if (!stage_scalars(R, rd, rs, nr, sent)) return false;
        }
      }
      return true;
    }
    case MKOP_ATTN: {
      const int b = in.r0, gg = in.r1, d = P.d, G = P.G, half = d / 2;
      const int R0 = (P.nq + 2 * P.nkv) * d;
      const float *qkv = A.qkv + ((size_t)l * P.B_max + b) * R0;
      float *q = R.X, *kc = R.X + G * d, *vc = kc + d;
      if (!stage_vec(R, q, qkv + (size_t)gg * G * d, G * d, sent)) return false;
      if (!stage_vec(R, kc, qkv + (size_t)P.nq * d + (size_t)gg * d, d, sent)) return false;
      if (!stage_vec(R, vc, qkv + (size_t)(P.nq + P.nkv) * d + (size_t)gg * d, d, sent)) return false;
      const float *cs = P.rope + (size_t)g.p * d;  // read below through gld
      for (int e = lane; e < (G + 1) * half; e += 64) {
        const int j = e / half, i = e - j * half;  // j == G is the key
        float *u = j < G ? q + j * d : kc;
        const float a = u[i], c = u[i + half], co = gld(cs + 2 * i), si = gld(cs + 2 * i + 1);
        float r0 = a * co - c * si, r1 = c * co + a * si;
        if (j == G) {
          r0 = bf2f(f2bf(r0));
          r1 = bf2f(f2bf(r1));
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

// ------------------------------------------------------- compute waves

struct AttnAcc {
  float m[MK_MAX_GROUP], l[MK_MAX_GROUP];
  float o[MK_MAX_GROUP][2];  // dims lane and lane + 64
};

// One block of bp key positions: scores, online softmax update, values.
MKD bool attn_unit(const MkRole &R, const MkGeo &g, int u, uint32_t s, const float (*qv)[8], AttnAcc &acc, float *wsc) {
  const int lane = threadIdx.x & 63;
  const int d = g.d, G = R.P.G, bp = g.bp;
  const int lpp = d / 8, ppi = 64 / lpp;  // lanes per position, positions per pass
  const int ta = g.t0 + u * bp;
  const int npos = min(bp, g.t1 - ta);
  bool ok;
  char *kp = const_cast<char *>(page_wait(R, s, &ok));
  if (!ok) return false;
  char *vp = const_cast<char *>(page_wait(R, s + 1, &ok));
  if (!ok) return false;
  // the page holds the cache's old slot for the current position: use the new key/value
  if (ta <= g.p && g.p < ta + npos) {
    const int row = g.p - ta;
    const float *kc = R.X + G * d, *vc = kc + d;
    uint16_t *kr = reinterpret_cast<uint16_t *>(kp + (size_t)row * 2 * d);
    uint16_t *vr = reinterpret_cast<uint16_t *>(vp + (size_t)row * 2 * d);
    for (int i = lane; i < d; i += 64) {
      kr[i] = f2bf(kc[i]);
      vr[i] = f2bf(vc[i]);
    }
  }
  const float scale = 1.0f / sqrtf((float)d);
  // scores: lpp lanes per position, 8 dims per lane
  const int c8 = (lane % lpp) * 8, pin = lane / lpp;
  for (int pass = 0; pass < bp / ppi; ++pass) {
    const int row = pass * ppi + pin;
    float sc[MK_MAX_GROUP];
    const mk_u32x4 w = row < npos ? *reinterpret_cast<const mk_u32x4 *>(kp + (size_t)row * 2 * d + c8 * 2)
                                  : mk_u32x4{0, 0, 0, 0};
    const float k8[8] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y), bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
#pragma unroll
    for (int j = 0; j < MK_MAX_GROUP; ++j) {
      float a = 0.f;
      if (j < G) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(qv[j][e], k8[e], a);
      }
      sc[j] = a;
    }
#pragma unroll
    for (int j = 0; j < MK_MAX_GROUP; ++j) {
      if (j < G) {
        for (int o = 1; o < lpp; o <<= 1) sc[j] += __shfl_xor(sc[j], o, 64);
      }
    }
    if ((lane % lpp) == 0) {
#pragma unroll
      for (int j = 0; j < MK_MAX_GROUP; ++j)
        if (j < G) wsc[j * 32 + row] = row < npos ? sc[j] * scale : -INFINITY;
    }
  }
  page_free(R, s);
  // online softmax update; lane i < npos owns position i
#pragma unroll
  for (int j = 0; j < MK_MAX_GROUP; ++j) {
    if (j >= G) continue;
    const float sv = lane < npos ? wsc[j * 32 + lane] : -INFINITY;
    const float mb = wave_max(sv);
    const float mn = fmaxf(acc.m[j], mb);
    const float corr = acc.m[j] == -INFINITY ? 0.f : expf(acc.m[j] - mn);
    const float pv = lane < npos ? expf(sv - mn) : 0.f;
    acc.l[j] = acc.l[j] * corr + wave_sum(pv);
    acc.o[j][0] *= corr;
    acc.o[j][1] *= corr;
    acc.m[j] = mn;
    if (lane < bp) wsc[j * 32 + lane] = pv;
  }
  // weighted values: lane owns dims lane (and lane + 64 when d = 128)
  const uint16_t *vr = reinterpret_cast<const uint16_t *>(vp);
  for (int i = 0; i < npos; ++i) {
    const float v0 = bf2f(vr[(size_t)i * d + lane]);
    const float v1 = d > 64 ? bf2f(vr[(size_t)i * d + lane + 64]) : 0.f;
#pragma unroll
    for (int j = 0; j < MK_MAX_GROUP; ++j)
      if (j < G) {
        const float pj = wsc[j * 32 + i];
        acc.o[j][0] = fmaf(pj, v0, acc.o[j][0]);
        acc.o[j][1] = fmaf(pj, v1, acc.o[j][1]);
      }
  }
  page_free(R, s + 1);
  return true;
}

// wave partials of attention live after q | k | v in X: [NCW][G][d + 2]
MKD float *attn_wpart(const MkRole &R, int cw) {
  const int d = R.P.d, G = R.P.G;
  return R.X + (size_t)(G + 2) * d + (size_t)cw * G * (d + 2);
}

// projection rows (QKV, O, gate/up, down, LM head) of one instruction for up
// to NB sequences
template <int NB>
MKD bool gemv_instr(const MkRole &R, const MkInstr &in, const MkGeo &g, const MkAct &A, uint32_t seq0, int cw) {
  const MkProgram &P = R.P;
  const MkStep &S = R.S;
  const int lane = threadIdx.x & 63;
  const int B = S.batch, l = in.layer;
  float best_v[NB];
  int best_i[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    best_v[b] = -INFINITY;
    best_i[b] = 0x7fffffff;
  }
  const int nr = in.r1 - in.r0;
  // one sequence, rows of one page: the input slice stays in registers
  XSlice<NB> xc;
  const bool cached = NB == 1 && g.ppr == 1;
  if (cached && cw < g.n_units) load_xslice<NB>(R, g, B, 0, xc);
  for (int u = cw; u < g.n_units; u += MK_NCW) {
    const uint32_t s = seq0 + (uint32_t)u * (uint32_t)g.ppu;
    float acc[NB], acc2[NB];
    if (cached) {
      if (!row_dot<NB, true>(R, g, s, B, xc, acc)) return false;
      if (in.op == MKOP_GATEUP && !row_dot<NB, true>(R, g, s + g.ppr, B, xc, acc2)) return false;
    } else {
      if (!row_dot<NB, false>(R, g, s, B, xc, acc)) return false;
      if (in.op == MKOP_GATEUP && !row_dot<NB, false>(R, g, s + g.ppr, B, xc, acc2)) return false;
    }
    const int r = in.r0 + u;
    if (lane == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b >= B) continue;
        switch (in.op) {
          case MKOP_QKV:
            stc(A.qkv + ((size_t)l * P.B_max + b) * ((P.nq + 2 * P.nkv) * P.d) + r, acc[b]);
            break;
          case MKOP_OPROJ:
            stc(A.xmid + ((size_t)l * P.B_max + b) * P.H + r, R.resid[(size_t)b * nr + u] + acc[b]);
            break;
          case MKOP_GATEUP: {
            const float a = acc[b];
            stc(A.hbuf + ((size_t)l * P.B_max + b) * P.I + r, (a / (1.0f + expf(-a))) * acc2[b]);
            break;
          }
          case MKOP_DOWN:
            stc(A.xout + ((size_t)l * P.B_max + b) * P.H + r, R.resid[(size_t)b * nr + u] + acc[b]);
            break;
          case MKOP_LMHEAD:
            gst(S.logits + (size_t)b * P.V + r, acc[b]);
            break;
        }
      }
    }
    if (in.op == MKOP_LMHEAD) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (b < B && better(acc[b], r, best_v[b], best_i[b])) {
          best_v[b] = acc[b];
          best_i[b] = r;
        }
    }
  }
  if (in.op == MKOP_LMHEAD && lane == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b >= B) continue;
      R.ctl->lm_v[cw * MK_RB_MAXB + b] = best_v[b];
      R.ctl->lm_i[cw * MK_RB_MAXB + b] = best_i[b];
    }
  }
  return true;
}

MKD bool compute_instr(const MkRole &R, const MkInstr &in, const MkGeo &g, const MkAct &A, uint32_t seq0, int cw) {
  const MkProgram &P = R.P;
  const MkStep &S = R.S;
  const int lane = threadIdx.x & 63;
  const int B = S.batch, l = in.layer;
  float *wsc = R.wsc + (size_t)cw * MK_WSC;
  if (in.op == MKOP_ATTN) {
    const int d = P.d, G = P.G, lpp = d / 8;
    float qv[MK_MAX_GROUP][8];
#pragma unroll
    for (int j = 0; j < MK_MAX_GROUP; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[j][e] = j < G ? R.X[j * d + (lane % lpp) * 8 + e] : 0.f;
    AttnAcc acc;
#pragma unroll
    for (int j = 0; j < MK_MAX_GROUP; ++j) {
      acc.m[j] = -INFINITY;
      acc.l[j] = 0.f;
      acc.o[j][0] = acc.o[j][1] = 0.f;
    }
    for (int u = cw; u < g.n_units; u += MK_NCW)
      if (!attn_unit(R, g, u, seq0 + (uint32_t)u * 2u, qv, acc, wsc)) return false;
    float *wp = attn_wpart(R, cw);
#pragma unroll
    for (int j = 0; j < MK_MAX_GROUP; ++j) {
      if (j >= G) continue;
      wp[j * (d + 2) + 2 + lane] = acc.o[j][0];
      if (d > 64) wp[j * (d + 2) + 2 + lane + 64] = acc.o[j][1];
      if (lane == 0) {
        wp[j * (d + 2)] = acc.m[j];
        wp[j * (d + 2) + 1] = acc.l[j];
      }
    }
    return true;
  }
  return B == 1 ? gemv_instr<1>(R, in, g, A, seq0, cw) : gemv_instr<MK_RB_MAXB>(R, in, g, A, seq0, cw);
}

// ------------------------------------------------------- sync epilogues

// returns 1: trigger the event, 0: do not, -1: abort
MKD int sync_epilogue(const MkRole &R, const MkInstr &in, const MkGeo &g, const MkAct &A) {
  const MkProgram &P = R.P;
  const MkStep &S = R.S;
  const int lane = threadIdx.x & 63;
  if (in.op == MKOP_ATTN) {
    const int b = in.r0, gg = in.r1, d = P.d, G = P.G, NS = in.nsplit, l = in.layer;
    float *out = A.attn + ((size_t)l * P.B_max + b) * P.nq * d + (size_t)gg * G * d;
    float *part = P.part + ((((size_t)l * P.B_max + b) * P.nkv + gg) * NS) * G * (d + 2);
    // merge the compute waves' partials
    for (int e = lane; e < G * d; e += 64) {
      const int j = e / d, i = e - j * d;
      float mx = -INFINITY;
      for (int w = 0; w < MK_NCW; ++w) mx = fmaxf(mx, attn_wpart(R, w)[j * (d + 2)]);
      float z = 0.f, o = 0.f;
      for (int w = 0; w < MK_NCW; ++w) {
        const float *wp = attn_wpart(R, w) + j * (d + 2);
        const float c = wp[0] == -INFINITY ? 0.f : expf(wp[0] - mx);
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
    old = __shfl(old, 0, 64);
    if (old + 1u != (S.epoch + 1u) * (uint32_t)NS) return 0;
    for (int e = lane; e < G * d; e += 64) {
      const int j = e / d, i = e - j * d;
      float mx = -INFINITY;
      for (int s2 = 0; s2 < NS; ++s2) mx = fmaxf(mx, ldc(part + ((size_t)s2 * G + j) * (d + 2)));
      float z = 0.f, o = 0.f;
      for (int s2 = 0; s2 < NS; ++s2) {
        const float *pp = part + ((size_t)s2 * G + j) * (d + 2);
        const float ms = ldc(pp);
        const float c = ms == -INFINITY ? 0.f : expf(ms - mx);
        z = fmaf(ldc(pp + 1), c, z);
        o = fmaf(ldc(pp + 2 + i), c, o);
      }
      stc(out + e, o / z);
    }
    return 1;
  }
  if (in.op == MKOP_LMHEAD) {
    for (int b = 0; b < S.batch; ++b) {
      float v = -INFINITY;
      int ix = 0x7fffffff;
      for (int w = 0; w < MK_NCW; ++w)
        if (better(R.ctl->lm_v[w * MK_RB_MAXB + b], R.ctl->lm_i[w * MK_RB_MAXB + b], v, ix)) {
          v = R.ctl->lm_v[w * MK_RB_MAXB + b];
          ix = R.ctl->lm_i[w * MK_RB_MAXB + b];
        }
      if (lane == 0) {
        stc(P.lm_val + (size_t)in.part * P.B_max + b, v);
        stci(P.lm_idx + (size_t)in.part * P.B_max + b, ix);
      }
    }
    wait_vm();
    uint32_t old = 0;
    if (lane == 0) old = addcu(P.tickets + in.ticket, 1u);
    old = __shfl(old, 0, 64);
    if (old + 1u != (S.epoch + 1u) * (uint32_t)P.n_lm_parts) return 0;
    if (lane < S.batch) {
      const int b = lane;
      float v = -INFINITY;
      int ix = 0x7fffffff;
      for (int k = 0; k < P.n_lm_parts; ++k) {
        const float pv = ldc(P.lm_val + (size_t)k * P.B_max + b);
        const int pi = ldci(P.lm_idx + (size_t)k * P.B_max + b);
        if (better(pv, pi, v, ix)) {
          v = pv;
          ix = pi;
        }
      }
      if (ix == 0x7fffffff) ix = 0;
      if (S.next) gst(S.next + b, ix);
      if (S.flags & 1u) {
        gst(S.tokens + b, ix);
        gst(S.positions + b, R.ctl->pos[b] + 1);
      }
    }
    return 0;
  }
  return 1;
}

// ------------------------------------------------------- role loops

// wave-level dependency wait (counter or flag mode)
MKD bool wave_wait_event(const MkRole &R, int ev) {
  const MkProgram &P = R.P;
  const MkStep &S = R.S;
  const int lane = threadIdx.x & 63;
  uint64_t t0 = 0;
  uint32_t spins = 0;
  while (true) {
    bool ready;
    if (P.sync_mode == 0) {
      const uint32_t need = (S.epoch + 1u) * (uint32_t)P.ev_count[ev];
      ready = (int32_t)(ldcu(P.ctr + ev) - need) >= 0;
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
    if ((++spins & 31u) == 0) {
      if (lds_ld(&R.ctl->abort) || mk_aborted(P)) {
        role_abort(R);
        return false;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)P.watchdog_ticks) {
        if (lane == 0) mk_raise(P, MK_E_TIMEOUT, ev);
        role_abort(R);
        return false;
      }
    }
  }
}

MKD void wave_signal_event(const MkRole &R, int ev, int slot) {
  const MkProgram &P = R.P;
  if ((threadIdx.x & 63) != 0) return;
  if (P.sync_mode == 0)
    addcu(P.ctr + ev, 1u);
  else
    stcu(P.flags + P.ev_flag_base[ev] + slot, R.S.epoch + 1u);
}

MKD void role_loader(const MkRole &R, const int32_t *list, int first, int n, int lid) {
  LoaderState L{0u, 0u};
  uint32_t seq = 0;
  for (int k = 0; k < n; ++k) {
    const MkInstr in = cld(&R.P.instr[list ? list[k] : first + k]);
    MkGeo g;
    if (!mk_geo(R.P, R.S, R.ctl, in, g)) {
      role_abort(R);
      break;
    }
    const uint32_t npg = (uint32_t)(g.n_units * g.ppu);
    for (uint32_t j = (uint32_t)((lid - (int)(seq % MK_NLW) + MK_NLW) % MK_NLW); j < npg; j += MK_NLW) {
      const int u = (int)(j / (uint32_t)g.ppu), kk = (int)(j % (uint32_t)g.ppu);
      int valid;
      const char *src = mk_page_src(g, in.op, u, kk, &valid);
      if (!loader_page(R, L, lid, seq + j, src, valid)) return;
    }
    seq += npg;
  }
  loader_publish_all(R, L, lid);
}

MKD void role_compute(const MkRole &R, const int32_t *list, int first, int n, int cw, const MkAct &A) {
  uint32_t seq = 0;
  const bool sent = R.P.sync_mode == MK_SYNC_SENTINEL && !R.S.multi;
  for (int k = 0; k < n; ++k) {
    const MkInstr in = cld(&R.P.instr[list ? list[k] : first + k]);
    MkGeo g;
    if (!mk_geo(R.P, R.S, R.ctl, in, g)) {
      role_abort(R);
      return;
    }
    if (!role_wait(R, &R.ctl->x_ready, (uint32_t)k + 1u)) return;
    if (!compute_instr(R, in, g, A, seq, cw)) return;
    if (!sent) wait_vm();  // outputs complete before the storer may trigger the event
    if ((threadIdx.x & 63) == 0) lds_add(&R.ctl->cw_done, 1u);  // one increment per wave
    seq += (uint32_t)(g.n_units * g.ppu);
  }
}

MKD void role_sync(const MkRole &R, const int32_t *list, int first, int n, const MkAct &A) {
  const MkProgram &P = R.P;
  const MkStep &S = R.S;
  const bool sent = P.sync_mode == MK_SYNC_SENTINEL && !S.multi;
  for (int k = 0; k < n; ++k) {
    const MkInstr in = cld(&P.instr[list ? list[k] : first + k]);
    MkGeo g;
    if (!mk_geo(P, S, R.ctl, in, g)) {
      if ((threadIdx.x & 63) == 0) mk_raise(P, MK_E_INPUT, 1000 + in.r0);
      role_abort(R);
      return;
    }
    const uint64_t tw = P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    if (!S.multi && !sent && in.wait_ev >= 0 && !wave_wait_event(R, in.wait_ev)) return;
    if (!role_wait(R, &R.ctl->cw_done, (uint32_t)k * MK_NCW)) return;  // X is free again
    if (!sync_stage(R, in, g, A, sent)) return;
    lds_st(&R.ctl->x_ready, (uint32_t)k + 1u);
    const uint64_t ts = P.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    if (!role_wait(R, &R.ctl->cw_done, (uint32_t)(k + 1) * MK_NCW)) return;
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
      uint64_t *r = P.trace + (size_t)(list ? list[k] : first + k) * 8;
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

// Entry used by both kernels: run `n` instructions of `list` with roles.
MKD void role_run(const MkProgram &P, const MkStep &S, const int32_t *list, int first, int n, char *lds) {
  MkCtl *ctl = reinterpret_cast<MkCtl *>(lds);
  for (int i = threadIdx.x; i < (int)(sizeof(MkCtl) / 4); i += MK_BLOCK) reinterpret_cast<uint32_t *>(ctl)[i] = 0;
  __syncthreads();
  if (threadIdx.x < S.batch) ctl->pos[threadIdx.x] = gld(S.positions + threadIdx.x);
  __syncthreads();
  const int par = (P.sync_mode == MK_SYNC_SENTINEL && !S.multi) ? (int)(S.epoch & 1u) : 0;
  MkRole R{P, S, ctl, reinterpret_cast<float *>(lds + P.lds_x), reinterpret_cast<float *>(lds + P.lds_resid),
           reinterpret_cast<float *>(lds + P.lds_wsc), lds + P.lds_ring, P.n_pages, par};
  const MkAct A = mk_act(P, par);
  const int wave = threadIdx.x >> 6;
  if (wave < MK_NLW) {
    role_loader(R, list, first, n, wave);
  } else if (wave == MK_SYNCW) {
    if (P.sync_mode == MK_SYNC_SENTINEL && !S.multi) {
      // reset this CU's share of the other parity's activations to the sentinel
      float *other = P.qkv + (size_t)(par ^ 1) * P.par_stride;
      const size_t per = (P.par_stride + P.n_cu - 1) / P.n_cu;
      const size_t lo = (size_t)blockIdx.x * per, hi = min(lo + per, (size_t)P.par_stride);
      for (size_t i = lo + (threadIdx.x & 63); i < hi; i += 64) stcu(reinterpret_cast<uint32_t *>(other) + i, MK_SENTINEL);
    }
    role_sync(R, list, first, n, A);
  } else {
    role_compute(R, list, first, n, wave - MK_NLW - 1, A);
  }
}
