// Per-op device functions shared by the persistent megakernel and the
// multi-launch build.  Each runs one planned instruction with the whole
// workgroup (MK_BLOCK threads) and writes its outputs with device-coherent
// stores.  The op kinds are the fused instructions of a decoder pass that the
// megakernel page names in section 2.6 (an RMSNorm+QKV+RoPE instruction,
// attention, the output projection, ...), completed with the MLP and LM-head
// instructions of a Llama decoder.
#pragma once
#include "mk_device.h"

// -------------------------------------------------------------- GEMV core
//
// Dot products of `nrows` weight rows (bf16, K columns, rowptr(r) gives row
// r) with one fp32 vector xs[K] held in LDS.  Waves take NR consecutive
// rows at a time; lanes stride over 8-element (16-byte) chunks so a wave's
// loads of one row are contiguous 1 KiB pieces.  Weights are read once per
// pass, so they use non-temporal loads.  fin(first_row, acc) runs on every
// lane with the NR full sums.
template <int NR, class RowPtr, class Fin>
MKD void gemv_rows(int K, int nrows, const float *xs, RowPtr rowptr, Fin fin) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = K >> 3;
  const float4 *x4 = reinterpret_cast<const float4 *>(xs);
  for (int g0 = wave * NR; g0 < nrows; g0 += MK_NWAVES * NR) {
    const mk_u32x4 *rp[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) rp[j] = reinterpret_cast<const mk_u32x4 *>(rowptr(min(g0 + j, nrows - 1)));
    float acc[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[j] = 0.f;
#pragma unroll 2
    for (int c = lane; c < nch; c += 64) {
      mk_u32x4 w[NR];
#pragma unroll
      for (int j = 0; j < NR; ++j) w[j] = __builtin_nontemporal_load(rp[j] + c);
      const float4 xa = x4[2 * c], xb = x4[2 * c + 1];
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        float a = acc[j];
        a = fmaf(bf_lo(w[j].x), xa.x, a);
        a = fmaf(bf_hi(w[j].x), xa.y, a);
        a = fmaf(bf_lo(w[j].y), xa.z, a);
        a = fmaf(bf_hi(w[j].y), xa.w, a);
        a = fmaf(bf_lo(w[j].z), xb.x, a);
        a = fmaf(bf_hi(w[j].z), xb.y, a);
        a = fmaf(bf_lo(w[j].w), xb.z, a);
        a = fmaf(bf_hi(w[j].w), xb.w, a);
        acc[j] = a;
      }
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[j] = wave_sum(acc[j]);
    fin(g0, acc);
  }
}

// In-place RMSNorm of xs[K] (LDS): x * (1 / sqrt(mean(x^2) + eps)) * gain.
MKD void rmsnorm_lds(float *xs, int K, const uint16_t *gain, float eps, float *red) {
  float ss = 0.f;
  for (int i = threadIdx.x; i < K; i += MK_BLOCK) ss = fmaf(xs[i], xs[i], ss);
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)K + eps);
  for (int i = threadIdx.x; i < K; i += MK_BLOCK) xs[i] = (xs[i] * r) * bf2f(gain[i]);
  __syncthreads();
}


// Residual-stream input of layer l for sequence b, element i: the embedding
// row of the token for layer 0, else the previous layer's output.
MKD float resid_in(const MkProgram &P, const MkStep &S, int l, int b, int i, int tok) {
  if (l == 0) return bf2f(P.embed[(size_t)tok * P.H + i]);
  return ldc(P.xout + ((size_t)(l - 1) * P.B_max + b) * P.H + i);
}

MKD bool token_ok(const MkProgram &P, const MkStep &S, int b, int *tok) {
  int t = S.tokens[b];
  *tok = t;
  return t >= 0 && t < P.V;
}

// status: 1 = done, trigger the event; 0 = done, do not trigger; -1 = abort
enum { MK_ST_ABORT = -1, MK_ST_QUIET = 0, MK_ST_SIGNAL = 1 };

// ---------------------------------------------------------------- QKV
MKD int op_qkv(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem) {
  const int H = P.H, l = in.layer;
  const int R = (P.nq + 2 * P.nkv) * P.d;
  float *xs = smem, *red = smem + H;
  const MkLayerW &W = P.layers[l];
  for (int b = 0; b < S.batch; ++b) {
    int tok = 0;
    if (l == 0 && !token_ok(P, S, b, &tok)) {
      if (threadIdx.x == 0) mk_raise(P, MK_E_INPUT, b);
      return MK_ST_ABORT;
    }
    for (int i = threadIdx.x; i < H; i += MK_BLOCK) xs[i] = resid_in(P, S, l, b, i, tok);
    __syncthreads();
    rmsnorm_lds(xs, H, W.attn_norm, P.eps, red);
    float *out = P.qkv + ((size_t)l * P.B_max + b) * R + in.r0;
    const int qd = P.nq * P.d, kd = P.nkv * P.d, r0 = in.r0;
    auto rowptr = [&](int r) -> const uint16_t * {
      const int row = r0 + r;
      if (row < qd) return W.wq + (size_t)row * H;
      if (row < qd + kd) return W.wk + (size_t)(row - qd) * H;
      return W.wv + (size_t)(row - qd - kd) * H;
    };
    const int n = in.r1 - in.r0;
    gemv_rows<4>(H, n, xs, rowptr, [&](int g0, const float *acc) {
      if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (g0 + j < n) stc(out + g0 + j, acc[j]);
    });
    __syncthreads();
  }
  return MK_ST_SIGNAL;
}

// ------------------------------------------------- RoPE + append + attention
//
// One (sequence b, kv head g, key split s) unit: rotate the group's q heads
// and the new key at position p, store the new key/value (bf16, RNE) into
// cache slot p when this split holds it, then softmax-weighted sums over the
// split's key range for every q head of the group.  With S > 1 splits each
// writes (max, sum, unnormalised output) and the last one to finish merges
// them with the usual log-sum-exp rescaling.
MKD int op_attn(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem, int *s_flag) {
  const int b = in.r0, g = in.r1, sp = in.split, NS = in.nsplit, l = in.layer;
  const int d = P.d, G = P.G, half = d / 2, nq = P.nq, nkv = P.nkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = S.positions[b];
  if (p < 0 || p >= P.max_ctx) {
    if (tid == 0) mk_raise(P, MK_E_INPUT, 1000 + b);
    return MK_ST_ABORT;
  }
  const int n = p + 1;
  const int chunk = (n + NS - 1) / NS;
  const int chunk_max = (P.max_ctx + NS - 1) / NS;
  const int t0 = min(n, sp * chunk), t1 = min(n, t0 + chunk);
  const int R = (nq + 2 * nkv) * d;
  const float *qkv = P.qkv + ((size_t)l * P.B_max + b) * R;

  float *q = smem;              // [G][d]
  float *kc = q + G * d;        // [d] new key, rotated, bf16-rounded
  float *vc = kc + d;           // [d] new value, bf16-rounded
  float *sc = vc + d;           // [G][chunk_max] scores, then weights
  float *tmp = sc + G * chunk_max;  // [MK_BLOCK]
  float *st = tmp + MK_BLOCK;   // [2G]: max, sum per head

  const float *cs = P.rope + (size_t)p * d;  // (cos, sin) pairs
  for (int e = tid; e < G * half; e += MK_BLOCK) {
    const int j = e / half, i = e - j * half;
    const float *qh = qkv + (size_t)(g * G + j) * d;
    const float a = ldc(qh + i), c = ldc(qh + i + half);
    const float co = cs[2 * i], si = cs[2 * i + 1];
    q[j * d + i] = a * co - c * si;
    q[j * d + i + half] = c * co + a * si;
  }
  for (int i = tid; i < half; i += MK_BLOCK) {
    const float *kh = qkv + (size_t)nq * d + (size_t)g * d;
    const float a = ldc(kh + i), c = ldc(kh + i + half);
    const float co = cs[2 * i], si = cs[2 * i + 1];
    kc[i] = bf2f(f2bf(a * co - c * si));
    kc[i + half] = bf2f(f2bf(c * co + a * si));
  }
  for (int i = tid; i < d; i += MK_BLOCK) vc[i] = bf2f(f2bf(ldc(qkv + (size_t)(nq + nkv) * d + (size_t)g * d + i)));
  __syncthreads();

  uint16_t *Kc = S.kv + kv_off(P, l, 0, b, g);
  uint16_t *Vc = S.kv + kv_off(P, l, 1, b, g);
  if (t0 <= p && p < t1)
    for (int i = tid; i < d; i += MK_BLOCK) {
      Kc[(size_t)p * d + i] = f2bf(kc[i]);
      Vc[(size_t)p * d + i] = f2bf(vc[i]);
    }

  // scores
  const float scale = 1.0f / sqrtf((float)d);
  for (int t = t0 + tid; t < t1; t += MK_BLOCK) {
    float acc[MK_MAX_GROUP];
#pragma unroll
    for (int j = 0; j < MK_MAX_GROUP; ++j) acc[j] = 0.f;
    if (t == p) {
      for (int i = 0; i < d; ++i) {
        const float kv = kc[i];
#pragma unroll
        for (int j = 0; j < MK_MAX_GROUP; ++j)
          if (j < G) acc[j] = fmaf(q[j * d + i], kv, acc[j]);
      }
    } else {
      const mk_u32x4 *kr = reinterpret_cast<const mk_u32x4 *>(Kc + (size_t)t * d);
      for (int c = 0; c < d / 8; ++c) {
        const mk_u32x4 w = kr[c];
        float kv[8] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y), bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int j = 0; j < MK_MAX_GROUP; ++j)
            if (j < G) acc[j] = fmaf(q[j * d + c * 8 + e], kv[e], acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < MK_MAX_GROUP; ++j)
      if (j < G) sc[j * chunk_max + (t - t0)] = acc[j] * scale;
  }
  __syncthreads();

  // per-head max and exponentials (wave j owns head j; G <= MK_NWAVES)
  if (wave < G) {
    float m = -INFINITY;
    for (int t = lane; t < t1 - t0; t += 64) m = fmaxf(m, sc[wave * chunk_max + t]);
    m = wave_max(m);
    float z = 0.f;
    for (int t = lane; t < t1 - t0; t += 64) {
      const float e = expf(sc[wave * chunk_max + t] - m);
      sc[wave * chunk_max + t] = e;
      z += e;
    }
    z = wave_sum(z);
    if (lane == 0) {
      st[wave] = m;
      st[G + wave] = z;
    }
  }
  __syncthreads();

  // weighted value sums: thread (j, i) over a strided subset of positions
  const int GD = G * d, ntg = MK_BLOCK / GD;
  if (tid < ntg * GD) {
    const int tg = tid / GD, e = tid - tg * GD, j = e / d, i = e - j * d;
    float acc = 0.f;
    for (int t = t0 + tg; t < t1; t += ntg) {
      const float v = (t == p) ? vc[i] : bf2f(Vc[(size_t)t * d + i]);
      acc = fmaf(sc[j * chunk_max + (t - t0)], v, acc);
    }
    tmp[tid] = acc;
  }
  __syncthreads();
  float *attn_out = P.attn + ((size_t)l * P.B_max + b) * nq * d + (size_t)g * G * d;
  if (NS == 1) {
    if (tid < GD) {
      float o = 0.f;
      for (int k = 0; k < ntg; ++k) o += tmp[k * GD + tid];
      stc(attn_out + tid, o / st[G + tid / d]);
    }
    return MK_ST_SIGNAL;
  }
  float *part = P.part + ((((size_t)l * P.B_max + b) * nkv + g) * NS) * G * (d + 2);
  if (tid < GD) {
    float o = 0.f;
    for (int k = 0; k < ntg; ++k) o += tmp[k * GD + tid];
    const int j = tid / d, i = tid - j * d;
    float *pp = part + ((size_t)sp * G + j) * (d + 2);
    stc(pp + 2 + i, o);
    if (i == 0) {
      stc(pp, st[j]);
      stc(pp + 1, st[G + j]);
    }
  }
  // last arriver merges the splits
  wait_vm();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = addcu(P.tickets + in.ticket, 1u);
    *s_flag = (old + 1u == (S.epoch + 1u) * (uint32_t)NS) ? 1 : 0;
  }
  __syncthreads();
  const int last = *s_flag;
  __syncthreads();
  if (!last) return MK_ST_QUIET;
  if (tid < GD) {
    const int j = tid / d, i = tid - j * d;
    float mx = -INFINITY;
    for (int s2 = 0; s2 < NS; ++s2) mx = fmaxf(mx, ldc(part + ((size_t)s2 * G + j) * (d + 2)));
    float z = 0.f, o = 0.f;
    for (int s2 = 0; s2 < NS; ++s2) {
      const float *pp = part + ((size_t)s2 * G + j) * (d + 2);
      const float ms = ldc(pp);
      const float w = (ms == -INFINITY) ? 0.f : expf(ms - mx);
      z = fmaf(ldc(pp + 1), w, z);
      o = fmaf(ldc(pp + 2 + i), w, o);
    }
    stc(attn_out + tid, o / z);
  }
  return MK_ST_SIGNAL;
}

// ------------------------------------------------------ O projection + add
MKD int op_oproj(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem) {
  const int H = P.H, l = in.layer, K = P.nq * P.d;
  float *xs = smem;
  const MkLayerW &W = P.layers[l];
  for (int b = 0; b < S.batch; ++b) {
    int tok = 0;
    if (l == 0 && !token_ok(P, S, b, &tok)) {
      if (threadIdx.x == 0) mk_raise(P, MK_E_INPUT, b);
      return MK_ST_ABORT;
    }
    const float *a = P.attn + ((size_t)l * P.B_max + b) * K;
    for (int i = threadIdx.x; i < K; i += MK_BLOCK) xs[i] = ldc(a + i);
    __syncthreads();
    float *out = P.xmid + ((size_t)l * P.B_max + b) * H;
    const int r0 = in.r0, n = in.r1 - in.r0;
    gemv_rows<4>(K, n, xs, [&](int r) { return W.wo + (size_t)(r0 + r) * K; }, [&](int g0, const float *acc) {
      if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (g0 + j < n) {
            const int row = r0 + g0 + j;
            stc(out + row, resid_in(P, S, l, b, row, tok) + acc[j]);
          }
    });
    __syncthreads();
  }
  return MK_ST_SIGNAL;
}

// ------------------------------------------- gate/up + SiLU (norm prologue)
MKD int op_gateup(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem) {
  const int H = P.H, l = in.layer;
  float *xs = smem, *red = smem + H;
  const MkLayerW &W = P.layers[l];
  for (int b = 0; b < S.batch; ++b) {
    const float *x = P.xmid + ((size_t)l * P.B_max + b) * H;
    for (int i = threadIdx.x; i < H; i += MK_BLOCK) xs[i] = ldc(x + i);
    __syncthreads();
    rmsnorm_lds(xs, H, W.mlp_norm, P.eps, red);
    float *out = P.hbuf + ((size_t)l * P.B_max + b) * P.I;
    const int r0 = in.r0, n = 2 * (in.r1 - in.r0);
    // virtual rows: 2j = gate row r0+j, 2j+1 = up row r0+j
    gemv_rows<4>(H, n, xs, [&](int v) { return ((v & 1) ? W.wu : W.wg) + (size_t)(r0 + (v >> 1)) * H; },
                 [&](int g0, const float *acc) {
                   if ((threadIdx.x & 63) == 0)
#pragma unroll
                     for (int j = 0; j < 4; j += 2)
                       if (g0 + j < n) {
                         const float a = acc[j], u = acc[j + 1];
                         stc(out + r0 + ((g0 + j) >> 1), (a / (1.0f + expf(-a))) * u);
                       }
                 });
    __syncthreads();
  }
  return MK_ST_SIGNAL;
}

// ------------------------------------------------ down projection + add
MKD int op_down(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem) {
  const int H = P.H, l = in.layer, K = P.I;
  float *xs = smem;
  const MkLayerW &W = P.layers[l];
  for (int b = 0; b < S.batch; ++b) {
    const float *h = P.hbuf + ((size_t)l * P.B_max + b) * K;
    for (int i = threadIdx.x; i < K; i += MK_BLOCK) xs[i] = ldc(h + i);
    __syncthreads();
    const float *xm = P.xmid + ((size_t)l * P.B_max + b) * H;
    float *out = P.xout + ((size_t)l * P.B_max + b) * H;
    const int r0 = in.r0, n = in.r1 - in.r0;
    gemv_rows<4>(K, n, xs, [&](int r) { return W.wd + (size_t)(r0 + r) * K; }, [&](int g0, const float *acc) {
      if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (g0 + j < n) stc(out + r0 + g0 + j, ldc(xm + r0 + g0 + j) + acc[j]);
    });
    __syncthreads();
  }
  return MK_ST_SIGNAL;
}

// ------------------------------------------ LM head + greedy argmax

MKD int op_lmhead(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem, int *s_flag) {
  const int H = P.H, L = P.L, V = P.V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float *xs = smem, *red = smem + H;
  float *wv = red + MK_NWAVES;            // [MK_NWAVES] best value per wave
  int *wi = reinterpret_cast<int *>(wv + MK_NWAVES);  // [MK_NWAVES] best index per wave
  const uint16_t *Wlm = P.tied ? P.embed : P.lm_head;
  for (int b = 0; b < S.batch; ++b) {
    const float *x = P.xout + ((size_t)(L - 1) * P.B_max + b) * H;
    for (int i = tid; i < H; i += MK_BLOCK) xs[i] = ldc(x + i);
    __syncthreads();
    rmsnorm_lds(xs, H, P.final_norm, P.eps, red);
    float *lg = S.logits + (size_t)b * V;
    const int r0 = in.r0, n = in.r1 - in.r0;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    gemv_rows<4>(H, n, xs, [&](int r) { return Wlm + (size_t)(r0 + r) * H; }, [&](int g0, const float *acc) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (g0 + j < n) {
          const int row = r0 + g0 + j;
          if (lane == 0) lg[row] = acc[j];
          if (better(acc[j], row, bv, bi)) {
            bv = acc[j];
            bi = row;
          }
        }
    });
    if (lane == 0) {
      wv[wave] = bv;
      wi[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      float v = wv[0];
      int ix = wi[0];
      for (int w = 1; w < MK_NWAVES; ++w)
        if (better(wv[w], wi[w], v, ix)) {
          v = wv[w];
          ix = wi[w];
        }
      stc(P.lm_val + (size_t)in.part * P.B_max + b, v);
      stci(P.lm_idx + (size_t)in.part * P.B_max + b, ix);
    }
    __syncthreads();
  }
  wait_vm();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = addcu(P.tickets + in.ticket, 1u);
    *s_flag = (old + 1u == (S.epoch + 1u) * (uint32_t)P.n_lm_parts) ? 1 : 0;
  }
  __syncthreads();
  const int last = *s_flag;
  __syncthreads();
  // last arriver: one wave per sequence merges every instruction's (max, index) pair
  for (int b = tid >> 6; last && b < S.batch; b += MK_NWAVES) {
    float v = -INFINITY;
    int ix = 0x7fffffff;
    for (int k = lane; k < P.n_lm_parts; k += 64) {
      const float pv = ldc(P.lm_val + (size_t)k * P.B_max + b);
      const int pi = ldci(P.lm_idx + (size_t)k * P.B_max + b);
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
      if (ix == 0x7fffffff) ix = 0;  // every logit NaN: fall back to token 0
      if (S.next) S.next[b] = ix;
      if (S.flags & 1u) {
        S.tokens[b] = ix;
        S.positions[b] = S.positions[b] + 1;
      }
    }
  }
  return MK_ST_QUIET;
}

MKD int run_instr(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem, int *s_flag) {
  switch (in.op) {
    case MKOP_QKV: return op_qkv(P, S, in, smem);
    case MKOP_ATTN: return op_attn(P, S, in, smem, s_flag);
    case MKOP_OPROJ: return op_oproj(P, S, in, smem);
    case MKOP_GATEUP: return op_gateup(P, S, in, smem);
    case MKOP_DOWN: return op_down(P, S, in, smem);
    case MKOP_LMHEAD: return op_lmhead(P, S, in, smem, s_flag);
    default: return MK_ST_ABORT;
  }
}
