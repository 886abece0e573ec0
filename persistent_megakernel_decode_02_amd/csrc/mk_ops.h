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
// r) with one fp32 vector x[K] held in LDS in two halves (xs_put): elements
// 8c .. 8c+3 at xs[4c ..], elements 8c+4 .. 8c+7 at xs[K/2 + 4c ..], so the
// lanes of a wave read consecutive 16-byte pieces (one 16-byte piece per
// lane at a 32-byte stride hit every LDS bank twice).
//
// Work split.  Rows form groups of NR; a wave owns whole groups.  With fewer
// groups than waves the waves also split the columns of each group into kp
// parts (as long as each part keeps U iterations of 64 chunks) and add their
// partial sums through LDS (`part`: MK_NWAVES * NR floats; callers put it 64
// floats past the staged vector, after the norm and argmax scratch).
//
// Streaming.  A batch is NR rows x U iterations; lanes stride over 8-element
// (16-byte) chunks, so one row's loads are contiguous 1 KiB pieces.  The
// loads are buffer loads on a per-row descriptor: a chunk past the part's
// end, a row past nrows, or a whole batch past the wave's last one falls
// outside the descriptor's range and reads zero without touching memory, so
// every load is issued unconditionally.  Two batches are in flight: the
// next is issued before the current one is reduced, and the compiler's
// wait counts stay exact because no load sits under a branch.  Weights are
// read once per pass, so the loads are non-temporal.  pro() runs on every
// thread once the first two batches are in flight (it may wait, stage xs
// and synchronise the block; false aborts and is returned).  fin(first_row,
// acc) runs on every lane of one wave with the NR full sums.
template <int NR, int U, class RowPtr, class Pro, class Fin>
MKD bool gemv_rows(int K, int nrows, const float *xs, float *part, RowPtr rowptr, Pro pro, Fin fin) {
  const int lane = mk_tid() & 63;
  const int wave = __builtin_amdgcn_readfirstlane(mk_tid() >> 6);  // wave-uniform, scalar
  const int nch = K >> 3;
  const int ng = (nrows + NR - 1) / NR;
  if (ng <= 0) return pro();
  const int nit = (nch + 63) >> 6;
  const int kp = max(1, min(ng >= MK_NWAVES ? 1 : MK_NWAVES / ng, nit / U));  // column parts
  const int nw = min(ng, MK_NWAVES);                                          // waves per part
  const int kpart = wave / nw, gw = wave - kpart * nw;
  const int pit = (nit + kp - 1) / kp;  // iterations per part
  const int c0 = kpart * pit * 64, c1 = min(nch, c0 + pit * 64);
  const int nb = (pit + U - 1) / U;  // batches per group
  const int T = kpart < kp ? (ng - gw + nw - 1) / nw * nb : 0;
  const float4 *x4 = reinterpret_cast<const float4 *>(xs), *x4b = x4 + (K >> 3);
  float acc[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = 0.f;

  auto load = [&](int k, bool on, mk_u32x4 (&w)[NR][U]) {
    const int gi = k / nb, ib = k - gi * nb;
    const int g0 = (gw + gi * nw) * NR;
    const int cb = c0 + ib * (U * 64) + lane;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const bool row_on = on && g0 + j < nrows;
      const __amdgpu_buffer_rsrc_t r = mk_rsrc(rowptr(min(g0 + j, nrows - 1)), row_on ? (uint32_t)K * 2u : 0u);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = cb + 64 * u;
        w[j][u] = __builtin_amdgcn_raw_buffer_load_b128(r, c < c1 ? c * 16 : 0x40000000, 0, 2);
      }
    }
  };
  auto comp = [&](int k, const mk_u32x4 (&w)[NR][U]) {
    const int gi = k / nb, ib = k - gi * nb;
    const int cb = c0 + ib * (U * 64) + lane;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(cb + 64 * u, nch - 1);  // out-of-range chunks carry zero weights
      const float4 xa = x4[c], xb = x4b[c];
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        float a = acc[j];
        a = fmaf(bf_lo(w[j][u].x), xa.x, a);
        a = fmaf(bf_hi(w[j][u].x), xa.y, a);
        a = fmaf(bf_lo(w[j][u].y), xa.z, a);
        a = fmaf(bf_hi(w[j][u].y), xa.w, a);
        a = fmaf(bf_lo(w[j][u].z), xb.x, a);
        a = fmaf(bf_hi(w[j][u].z), xb.y, a);
        a = fmaf(bf_lo(w[j][u].w), xb.z, a);
        a = fmaf(bf_hi(w[j][u].w), xb.w, a);
        acc[j] = a;
      }
    }
    if (kp == 1 && ib == nb - 1) {  // group complete
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] = wave_sum(acc[j]);
      fin((gw + gi * nw) * NR, acc);
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] = 0.f;
    }
  };

  // the first two batches go out before the prologue (the dependency wait
  // and the staging of xs), so they load while the wave waits
  mk_u32x4 wa[NR][U], wb[NR][U];
  load(0, T > 0, wa);
  load(min(1, max(T - 1, 0)), T > 1, wb);
  if (!pro()) return false;
  for (int k = 0; k < T; k += 2) {
    comp(k, wa);
    if (k + 1 >= T) break;
    load(min(k + 2, T - 1), k + 2 < T, wa);
    comp(k + 1, wb);
    load(min(k + 3, T - 1), k + 3 < T, wb);
  }
  if (kp > 1) {  // one group per wave of each part: add the parts
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[j] = wave_sum(acc[j]);
    if (lane == 0)
#pragma unroll
      for (int j = 0; j < NR; ++j) part[wave * NR + j] = acc[j];
    __syncthreads();
    if (kpart == 0)
      for (int k2 = 1; k2 < kp; ++k2)
#pragma unroll
        for (int j = 0; j < NR; ++j) acc[j] += part[(wave + k2 * nw) * NR + j];
    __syncthreads();
    if (kpart == 0) fin(gw * NR, acc);
  }
  return true;
}

// ------------------------------------------------------- input staging
//
// xs_put: elements 4k .. 4k+3 of an n-element GEMV input into the two-half
// layout gemv_rows reads.
MKD float *xs_put(float *xs, int n, int k) { return xs + (k & 1) * (n >> 1) + 4 * (k >> 1); }
//
// Inputs are staged with 16-byte device-coherent loads, all issued back to
// back: a chunk past the end reads zero through the descriptor's range, so
// no load sits under a branch.  n is a multiple of 4.
#define MK_OOB 0x40000000  // byte offset past every descriptor's range

// sent: poll each chunk until its producer has written it (data-sentinel
// mode); ok turns false on a timeout or abort.
MKD void stage_vec(const MkProgram &P, float *xs, const float *src, int n, bool sent, bool &ok) {
  const int tid = mk_tid(), nc = n >> 2;
  const __amdgpu_buffer_rsrc_t r = mk_rsrc(src, (uint32_t)n * 4u);
  for (int c0 = 0; c0 < nc; c0 += 4 * MK_BLOCK) {
    mk_u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + tid + k * MK_BLOCK;
      v[k] = ldc16(r, c < nc ? c * 16 : MK_OOB);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + tid + k * MK_BLOCK;
      if (sent) v[k] = poll16(P, r, c < nc ? c * 16 : MK_OOB, v[k], ok);
      if (c < nc) *reinterpret_cast<mk_u32x4 *>(xs_put(xs, n, c)) = v[k];
    }
  }
}

// RMSNorm gain chunks of this thread (4 bf16 per chunk, up to four chunks:
// n <= 16 * MK_BLOCK), loaded ahead of the dependency wait.
struct NormGain {
  uint32_t w[4][2];
};
MKD void load_gain(NormGain &g, const uint16_t *gain, int n) {
  const int tid = mk_tid(), nc = n >> 2;
  const __amdgpu_buffer_rsrc_t r = mk_rsrc(gain, (uint32_t)n * 2u);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = tid + k * MK_BLOCK;
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, c < nc ? c * 8 : MK_OOB, 0, 0);
    g.w[k][0] = v[0];
    g.w[k][1] = v[1];
  }
}

// Stage x[n] (fp32 from coherent memory, or the bf16 embedding row when
// `emb` is set) into xs as x * (1 / sqrt(mean(x^2) + eps)) * gain.  The sum
// of squares comes from the registers the loads filled; ends with a barrier.
MKD void stage_norm(const MkProgram &P, float *xs, const float *src, const uint16_t *emb, int n, const NormGain &g,
                    float eps, float *red, bool sent, bool &ok) {
  const int tid = mk_tid(), nc = n >> 2;
  float4 x[4];
  if (emb) {
    const __amdgpu_buffer_rsrc_t r = mk_rsrc(emb, (uint32_t)n * 2u);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = tid + k * MK_BLOCK;
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, c < nc ? c * 8 : MK_OOB, 0, 0);
      x[k] = make_float4(bf_lo(v[0]), bf_hi(v[0]), bf_lo(v[1]), bf_hi(v[1]));
    }
  } else {
    const __amdgpu_buffer_rsrc_t r = mk_rsrc(src, (uint32_t)n * 4u);
    mk_u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = tid + k * MK_BLOCK;
      v[k] = ldc16(r, c < nc ? c * 16 : MK_OOB);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = tid + k * MK_BLOCK;
      if (sent) v[k] = poll16(P, r, c < nc ? c * 16 : MK_OOB, v[k], ok);
      x[k] = make_float4(__uint_as_float(v[k].x), __uint_as_float(v[k].y), __uint_as_float(v[k].z),
                         __uint_as_float(v[k].w));
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ss = fmaf(x[k].x, x[k].x, ss);
    ss = fmaf(x[k].y, x[k].y, ss);
    ss = fmaf(x[k].z, x[k].z, ss);
    ss = fmaf(x[k].w, x[k].w, ss);
  }
  ss = block_sum(ss, red);
  const float rn = 1.0f / sqrtf(ss / (float)n + eps);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = tid + k * MK_BLOCK;
    if (c < nc)
      *reinterpret_cast<float4 *>(xs_put(xs, n, c)) =
          make_float4((x[k].x * rn) * bf_lo(g.w[k][0]), (x[k].y * rn) * bf_hi(g.w[k][0]),
                      (x[k].z * rn) * bf_lo(g.w[k][1]), (x[k].w * rn) * bf_hi(g.w[k][1]));
  }
  __syncthreads();
}

// Residual-stream input of layer l for sequence b, element i: the embedding
// row of the token for layer 0, else the previous layer's output.
MKD float resid_in(const MkProgram &P, const MkStep &S, int l, int b, int i, int tok, bool sent, bool &ok) {
  if (l == 0) return bf2f(P.embed[(size_t)tok * P.H + i]);
  return ldcp(P, P.xout + ((size_t)(l - 1) * P.B_max + b) * P.H + i, sent, ok);
}

// Output rows are gathered in LDS (`ob`) by the row groups' finishers and
// stored by the whole block once the instruction's last weight batch has been
// consumed: a wave's vector-memory counter retires loads and stores in issue
// order, so a device-scope store issued between two load batches would hold
// the second batch back until the store is acknowledged.
MKD void flush_rows(float *dst, const float *ob, int n) {
  lds_barrier();
  for (int i = mk_tid(); i < n; i += MK_BLOCK) stc(dst + i, ob[i]);
}

// After staging: true (block-uniform) when some thread's poll failed (data
// sentinels); with events, only the barrier the caller asks for (bar).
template <bool SENT>
MKD bool block_failed(bool ok, bool bar) {
  if constexpr (SENT) return __syncthreads_or(!ok) != 0;
  if (bar) __syncthreads();
  return false;
}

// Tokens and positions are read and written device-coherently: within a
// multi-step launch the previous step's last arriver (on any CU) wrote them.
MKD bool token_ok(const MkProgram &P, const MkStep &S, int b, int *tok) {
  int t = ldci(S.tokens + b);
  *tok = t;
  return t >= 0 && t < P.V;
}

// status: 1 = done, trigger the event; 0 = done, do not trigger; -1 = abort
enum { MK_ST_ABORT = -1, MK_ST_QUIET = 0, MK_ST_SIGNAL = 1 };

// ---------------------------------------------------------------- QKV
// Every op issues its first weight batches, then runs `wait` (the
// instruction's dependency, for the first sequence only) and stages its
// input vector; the weights load meanwhile.
// SENT: inputs are polled for data sentinels (no events between levels).
template <bool SENT = false, class Wait>
MKD int op_qkv(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem, Wait &wait) {
  const int H = P.H, l = in.layer;
  const int R = (P.nq + 2 * P.nkv) * P.d;
  float *xs = smem, *red = smem + H, *ob = smem + H + 96;
  const MkLayerW W = cld(&P.layers[l]);
  const int qd = P.nq * P.d, kd = P.nkv * P.d, r0 = in.r0, n = in.r1 - in.r0;
  // the planner keeps a slice inside one head, so inside one of q, k, v: its
  // first row decides the tensor
  const uint16_t *base = r0 < qd ? W.wq + (size_t)r0 * H
                         : r0 < qd + kd ? W.wk + (size_t)(r0 - qd) * H
                                        : W.wv + (size_t)(r0 - qd - kd) * H;
  auto rowptr = [&](int r) -> const uint16_t * { return base + (size_t)r * H; };
  for (int b = 0; b < S.batch; ++b) {
    int tok = 0;
    if (l == 0 && !token_ok(P, S, b, &tok)) {
      if (mk_tid() == 0) mk_raise(P, MK_E_INPUT, b);
      return MK_ST_ABORT;
    }
    float *out = P.qkv + ((size_t)l * P.B_max + b) * R + in.r0;
    const bool ok = gemv_rows<4, 4>(H, n, xs, xs + H + 64, rowptr, [&]() -> bool {
      NormGain g;
      load_gain(g, W.attn_norm, H);
      if (b == 0 && !wait()) return false;
      bool ok = true;
      stage_norm(P, xs, l > 0 ? P.xout + ((size_t)(l - 1) * P.B_max + b) * H : nullptr,
                 l == 0 ? P.embed + (size_t)tok * H : nullptr, H, g, P.eps, red, SENT, ok);
      return !block_failed<SENT>(ok, false);
    }, [&](int g0, const float *acc) {
      if ((mk_tid() & 63) == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (g0 + j < n) ob[g0 + j] = acc[j];
    });
    if (!ok) return MK_ST_ABORT;
    flush_rows(out, ob, n);
    __syncthreads();
  }
  return MK_ST_SIGNAL;
}

// ------------------------------------------------------ O projection + add
// U: 16-byte pieces per row and lane in one load batch (1 when the op runs
// inside the gate/up instruction's prologue and must leave registers free)
template <bool SENT = false, int U = 4, class Wait>
MKD int op_oproj(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem, Wait &wait) {
  const int H = P.H, l = in.layer, K = P.nq * P.d;
  float *xs = smem, *res = smem + K + 96;  // res: residual inputs of the rows [r0, r1)
  const MkLayerW W = cld(&P.layers[l]);
  const int r0 = in.r0, n = in.r1 - in.r0;
  float *ob = res + ((n + 3) & ~3);
  for (int b = 0; b < S.batch; ++b) {
    int tok = 0;
    if (l == 0 && !token_ok(P, S, b, &tok)) {
      if (mk_tid() == 0) mk_raise(P, MK_E_INPUT, b);
      return MK_ST_ABORT;
    }
    const float *a = P.attn + ((size_t)l * P.B_max + b) * K;
    float *out = P.xmid + ((size_t)l * P.B_max + b) * H;
    const bool ok = gemv_rows<4, U>(K, n, xs, xs + K + 64, [&](int r) { return W.wo + (size_t)(r0 + r) * K; },
                                    [&]() -> bool {
                                      if (b == 0 && !wait()) return false;
                                      bool ok2 = true;
                                      stage_vec(P, xs, a, K, SENT, ok2);
                                      // the residual rows are written before the attention output
                                      // they are added to exists, but are polled all the same
                                      for (int i = mk_tid(); i < n; i += MK_BLOCK)
                                        res[i] = resid_in(P, S, l, b, r0 + i, tok, SENT, ok2);
                                      return !block_failed<SENT>(ok2, true);
                                    },
                                    [&](int g0, const float *acc) {
                                      if ((mk_tid() & 63) == 0)
#pragma unroll
                                        for (int j = 0; j < 4; ++j)
                                          if (g0 + j < n) ob[g0 + j] = res[g0 + j] + acc[j];
                                    });
    if (!ok) return MK_ST_ABORT;
    flush_rows(out + r0, ob, n);
    __syncthreads();
  }
  return MK_ST_SIGNAL;
}

// ------------------------------------------- gate/up + SiLU (norm prologue)
// before(): runs once the first weight batches are in flight and before the
// wait (false aborts); the paired O projection runs there.
template <bool SENT = false, class Wait, class Before>
MKD int op_gateup(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem, Wait &wait, Before &before) {
  const int H = P.H, l = in.layer;
  float *xs = smem, *red = smem + H, *ob = smem + H + 96;
  const MkLayerW W = cld(&P.layers[l]);
  const int r0 = in.r0, n = 2 * (in.r1 - in.r0);
  for (int b = 0; b < S.batch; ++b) {
    const float *x = P.xmid + ((size_t)l * P.B_max + b) * H;
    float *out = P.hbuf + ((size_t)l * P.B_max + b) * P.I;
    // virtual rows: 2j = gate row r0+j, 2j+1 = up row r0+j
    const bool ok = gemv_rows<4, 4>(
        H, n, xs, xs + H + 64, [&](int v) { return ((v & 1) ? W.wu : W.wg) + (size_t)(r0 + (v >> 1)) * H; },
        [&]() -> bool {
          NormGain g;
          load_gain(g, W.mlp_norm, H);
          if (b == 0 && !before()) return false;
          if (b == 0 && !wait()) return false;
          bool ok2 = true;
          stage_norm(P, xs, x, nullptr, H, g, P.eps, red, SENT, ok2);
          return !block_failed<SENT>(ok2, false);
        },
        [&](int g0, const float *acc) {
          if ((mk_tid() & 63) == 0)
#pragma unroll
            for (int j = 0; j < 4; j += 2)
              if (g0 + j < n) {
                const float a = acc[j], u = acc[j + 1];
                ob[(g0 + j) >> 1] = (a / (1.0f + expf(-a))) * u;
              }
        });
    if (!ok) return MK_ST_ABORT;
    flush_rows(out + r0, ob, n >> 1);
    __syncthreads();
  }
  return MK_ST_SIGNAL;
}

// ------------------------------------------------ down projection + add
template <bool SENT = false, class Wait>
MKD int op_down(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem, Wait &wait) {
  const int H = P.H, l = in.layer, K = P.I;
  float *xs = smem, *res = smem + K + 96;  // res: residual inputs of the rows [r0, r1)
  const MkLayerW W = cld(&P.layers[l]);
  const int r0 = in.r0, n = in.r1 - in.r0;
  float *ob = res + ((n + 3) & ~3);
  for (int b = 0; b < S.batch; ++b) {
    const float *h = P.hbuf + ((size_t)l * P.B_max + b) * K;
    const float *xm = P.xmid + ((size_t)l * P.B_max + b) * H;
    float *out = P.xout + ((size_t)l * P.B_max + b) * H;
    const bool ok = gemv_rows<4, 4>(K, n, xs, xs + K + 64, [&](int r) { return W.wd + (size_t)(r0 + r) * K; },
                                    [&]() -> bool {
                                      if (b == 0 && !wait()) return false;
                                      bool ok2 = true;
                                      stage_vec(P, xs, h, K, SENT, ok2);
                                      for (int i = mk_tid(); i < n; i += MK_BLOCK) res[i] = ldcp(P, xm + r0 + i, SENT, ok2);
                                      return !block_failed<SENT>(ok2, true);
                                    },
                                    [&](int g0, const float *acc) {
                                      if ((mk_tid() & 63) == 0)
#pragma unroll
                                        for (int j = 0; j < 4; ++j)
                                          if (g0 + j < n) ob[g0 + j] = res[g0 + j] + acc[j];
                                    });
    if (!ok) return MK_ST_ABORT;
    flush_rows(out + r0, ob, n);
    __syncthreads();
  }
  return MK_ST_SIGNAL;
}

// ------------------------------------------ LM head + greedy argmax

// Greedy-token merge.  Every LM-head instruction publishes, per sequence, its
// best (value, row) tagged with the step in one 64-bit device-scope store:
// value bits << 32 | row << 15 | (epoch + 1) mod 2^15 (row 0x1ffff: every
// logit was NaN).  The one instruction the planner marks (split = 1, the last
// of the breadth-first queue, so in the work-queue engine no instruction is
// held behind it) polls every part until all carry this step's tag, merges
// them (largest value, lowest row among equal values) and publishes the
// token; the others just store.  No ticket: all parts arriving on one counter
// serialised at the memory side.
MKD uint64_t lm_pack(float v, int ix, uint32_t epoch) {
  const uint32_t row = ix < 0 || ix > MK_MAX_VOCAB ? 0x1ffffu : (uint32_t)ix;
  return (uint64_t)__float_as_uint(v) << 32 | (uint64_t)row << 15 | ((epoch + 1u) & 0x7fffu);
}

MKD int lm_merge(const MkProgram &P, const MkStep &S, const MkInstr &in) {
  if (in.split != 1) return MK_ST_QUIET;
  const int tid = mk_tid(), lane = tid & 63;
  const uint32_t tag = (S.epoch + 1u) & 0x7fffu;
  bool ok = true;
  // one wave per sequence merges every part's record
  for (int b = tid >> 6; b < S.batch; b += MK_NWAVES) {
    float v = -INFINITY;
    int ix = 0x7fffffff;
    for (int k = lane; k < P.n_lm_parts; k += 64) {
      const uint64_t *src = P.lm_pk + (size_t)k * P.B_max + b;
      uint64_t e = ldc64(src);
      uint32_t spins = 0;
      uint64_t t0 = 0;
      while (ok && (uint32_t)(e & 0x7fffu) != tag) {
        if (poll_fail(P, spins, t0, 0x30002)) {
          ok = false;
          break;
        }
        e = ldc64(src);
      }
      const uint32_t row = (uint32_t)(e >> 15) & 0x1ffffu;
      const float pv = __uint_as_float((uint32_t)(e >> 32));
      const int pi = row == 0x1ffffu ? 0x7fffffff : (int)row;
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
    if (lane == 0 && ok) {
      if (ix == 0x7fffffff) ix = 0;  // every logit NaN: fall back to token 0
      if (S.next) stci(S.next + b, ix);
      if (S.flags & 1u) {
        stci(S.tokens + b, ix);
        stci(S.positions + b, ldci(S.positions + b) + 1);
      }
    }
  }
  if (__syncthreads_or(!ok)) return MK_ST_ABORT;
  // the step's tokens are out: publish its epoch
  wait_vm();
  __syncthreads();
  if (tid == 0) stcu(P.lm_done, S.epoch + 1u);
  return MK_ST_QUIET;
}

template <bool SENT = false, class Wait>
MKD int op_lmhead(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem, int *s_flag, Wait &wait) {
  const int H = P.H, L = P.L, V = P.V;
  const int tid = mk_tid(), lane = tid & 63, wave = tid >> 6;
  float *xs = smem, *red = smem + H, *ob = smem + H + 96;  // ob: this instruction's logits
  float *wv = red + MK_NWAVES;            // [MK_NWAVES] best value per wave
  int *wi = reinterpret_cast<int *>(wv + MK_NWAVES);  // [MK_NWAVES] best index per wave
  const uint16_t *Wlm = P.tied ? P.embed : P.lm_head;
  for (int b = 0; b < S.batch; ++b) {
    const float *x = P.xout + ((size_t)(L - 1) * P.B_max + b) * H;
    float *lg = S.logits + (size_t)b * V;
    const int r0 = in.r0, n = in.r1 - in.r0;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    auto pro = [&]() -> bool {
      NormGain g;
      load_gain(g, P.final_norm, H);
      if (b == 0 && !wait()) return false;
      bool ok2 = true;
      stage_norm(P, xs, x, nullptr, H, g, P.eps, red, SENT, ok2);
      return !block_failed<SENT>(ok2, false);
    };
    const bool ok = gemv_rows<4, 4>(H, n, xs, xs + H + 64, [&](int r) { return Wlm + (size_t)(r0 + r) * H; }, pro,
                                    [&](int g0, const float *acc) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (g0 + j < n) {
          const int row = r0 + g0 + j;
          if (lane == 0) ob[g0 + j] = acc[j];
          if (better(acc[j], row, bv, bi)) {
            bv = acc[j];
            bi = row;
          }
        }
    });
    if (!ok) return MK_ST_ABORT;
    if (lane == 0) {
      wv[wave] = bv;
      wi[wave] = bi;
    }
    lds_barrier();
    for (int i = tid; i < n; i += MK_BLOCK) gst(lg + r0 + i, ob[i]);
    __syncthreads();
    if (tid == 0) {
      float v = wv[0];
      int ix = wi[0];
      for (int w = 1; w < MK_NWAVES; ++w)
        if (better(wv[w], wi[w], v, ix)) {
          v = wv[w];
          ix = wi[w];
        }
      stc64(P.lm_pk + (size_t)in.part * P.B_max + b, lm_pack(v, ix, S.epoch));
    }
    __syncthreads();
  }
  return lm_merge(P, S, in);
}
