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
  const int lane = mk_tid() & 63, wave = mk_tid() >> 6;
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
  for (int i = mk_tid(); i < K; i += MK_BLOCK) ss = fmaf(xs[i], xs[i], ss);
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)K + eps);
  for (int i = mk_tid(); i < K; i += MK_BLOCK) xs[i] = (xs[i] * r) * bf2f(gain[i]);
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
  const MkLayerW W = cld(&P.layers[l]);
  for (int b = 0; b < S.batch; ++b) {
    int tok = 0;
    if (l == 0 && !token_ok(P, S, b, &tok)) {
      if (mk_tid() == 0) mk_raise(P, MK_E_INPUT, b);
      return MK_ST_ABORT;
    }
    for (int i = mk_tid(); i < H; i += MK_BLOCK) xs[i] = resid_in(P, S, l, b, i, tok);
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
      if ((mk_tid() & 63) == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (g0 + j < n) stc(out + g0 + j, acc[j]);
    });
    __syncthreads();
  }
  return MK_ST_SIGNAL;
}

// ------------------------------------------------------ O projection + add
MKD int op_oproj(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem) {
  const int H = P.H, l = in.layer, K = P.nq * P.d;
  float *xs = smem;
  const MkLayerW W = cld(&P.layers[l]);
  for (int b = 0; b < S.batch; ++b) {
    int tok = 0;
    if (l == 0 && !token_ok(P, S, b, &tok)) {
      if (mk_tid() == 0) mk_raise(P, MK_E_INPUT, b);
      return MK_ST_ABORT;
    }
    const float *a = P.attn + ((size_t)l * P.B_max + b) * K;
    for (int i = mk_tid(); i < K; i += MK_BLOCK) xs[i] = ldc(a + i);
    __syncthreads();
    float *out = P.xmid + ((size_t)l * P.B_max + b) * H;
    const int r0 = in.r0, n = in.r1 - in.r0;
    gemv_rows<4>(K, n, xs, [&](int r) { return W.wo + (size_t)(r0 + r) * K; }, [&](int g0, const float *acc) {
      if ((mk_tid() & 63) == 0)
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
  const MkLayerW W = cld(&P.layers[l]);
  for (int b = 0; b < S.batch; ++b) {
    const float *x = P.xmid + ((size_t)l * P.B_max + b) * H;
    for (int i = mk_tid(); i < H; i += MK_BLOCK) xs[i] = ldc(x + i);
    __syncthreads();
    rmsnorm_lds(xs, H, W.mlp_norm, P.eps, red);
    float *out = P.hbuf + ((size_t)l * P.B_max + b) * P.I;
    const int r0 = in.r0, n = 2 * (in.r1 - in.r0);
    // virtual rows: 2j = gate row r0+j, 2j+1 = up row r0+j
    gemv_rows<4>(H, n, xs, [&](int v) { return ((v & 1) ? W.wu : W.wg) + (size_t)(r0 + (v >> 1)) * H; },
                 [&](int g0, const float *acc) {
                   if ((mk_tid() & 63) == 0)
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
  const MkLayerW W = cld(&P.layers[l]);
  for (int b = 0; b < S.batch; ++b) {
    const float *h = P.hbuf + ((size_t)l * P.B_max + b) * K;
    for (int i = mk_tid(); i < K; i += MK_BLOCK) xs[i] = ldc(h + i);
    __syncthreads();
    const float *xm = P.xmid + ((size_t)l * P.B_max + b) * H;
    float *out = P.xout + ((size_t)l * P.B_max + b) * H;
    const int r0 = in.r0, n = in.r1 - in.r0;
    gemv_rows<4>(K, n, xs, [&](int r) { return W.wd + (size_t)(r0 + r) * K; }, [&](int g0, const float *acc) {
      if ((mk_tid() & 63) == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (g0 + j < n) stc(out + r0 + g0 + j, ldc(xm + r0 + g0 + j) + acc[j]);
    });
    __syncthreads();
  }
  return MK_ST_SIGNAL;
}

// ------------------------------------------ LM head + greedy argmax

// Every LM-head instruction has stored its (max, index) partial per sequence:
// take a ticket; the last arriver merges all partials into the greedy token
// (and, with MK_ADVANCE, feeds it back as the next input).
MKD int lm_finish(const MkProgram &P, const MkStep &S, const MkInstr &in, int *s_flag) {
  const int tid = mk_tid(), lane = tid & 63;
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

MKD int op_lmhead(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem, int *s_flag) {
  const int H = P.H, L = P.L, V = P.V;
  const int tid = mk_tid(), lane = tid & 63, wave = tid >> 6;
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
  return lm_finish(P, S, in, s_flag);
}
