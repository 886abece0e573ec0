// The homogeneous engine's matrix-core ops (batched projections as bf16
// MFMA contractions, decode attention) and its instruction dispatch.
//
// With several sequences per step every projection is a matrix product
// Y[b][r] = sum_k X[b][k] W[r][k] over up to 16 sequences.  One instruction
// reads its weight rows once for the whole batch (the vector path of
// mk_ops.h reads them once per sequence) and runs the product on the matrix
// cores with v_mfma_f32_16x16x32_bf16: A = the 16 staged input rows (one per
// sequence), B = 16 weight rows, fp32 accumulation.  The fp32 inputs are
// split into bf16 high and low parts (x = hi + lo to within 2^-17 |x|) and
// both parts are multiplied, so the products keep the accuracy of the fp32
// vector path while the weights stay bf16.
//
// Work split inside a workgroup: the instruction's rows form nt tiles of 16.
// With nt >= 8 each wave owns whole tiles over the full reduction range;
// with fewer tiles the waves also split the reduction range of each tile in
// ks = 2, 4 or 8 parts and add their partial tiles through LDS.  The inputs
// are staged in LDS in chunks of MK_BKC columns, RMSNorm applied while
// staging; weights stream straight from HBM into the MFMA operands with a
// few steps of prefetch per wave.
#pragma once
#include "mk_ops.h"

extern __shared__ __attribute__((aligned(16))) char mk_flat_lds[];

// ------------------------------------------------------------ input sources

// fp32 activation rows [nb][K], device-coherent 16-byte loads; the buffer
// range ends after row nb - 1, so rows beyond the batch read as zero.
struct BActSrc {
  __amdgpu_buffer_rsrc_t rs;
  int K;
  MKD float4 load(int b, int k) const {
    const mk_u32x4 u = ldc16(rs, (b * K + k) * 4);
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
  }
};
MKD BActSrc bact(const float *rows, int nb, int K) {
  return BActSrc{mk_rsrc(rows, (uint32_t)(nb * K) * 4u), K};
}

// bf16 embedding rows of this step's tokens (the layer-0 input).  `row` is
// the calling thread's sequence row, null beyond the batch (reads as zero).
struct BEmbSrc {
  const uint16_t *row;
  MKD float4 load(int, int k) const {
    if (!row) return make_float4(0.f, 0.f, 0.f, 0.f);
    const uint64_t u = gld((const uint64_t *)(row + k));
    const uint32_t a = (uint32_t)u, c = (uint32_t)(u >> 32);
    return make_float4(bf_lo(a), bf_hi(a), bf_lo(c), bf_hi(c));
  }
};

// ------------------------------------------------------------------ staging
//
// Thread mapping: sequence row b = tid / 32; the 32 threads of a row take
// float4 columns 4 (tid % 32 + 32 j).

MKD float row_sum32(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 32);
  return v;
}

// RMSNorm scale 1 / sqrt(mean(x^2) + eps) of this thread's row over all K
// columns (used when a row does not fit in one staged chunk)
template <class Src>
MKD float bnorm_rs(const Src &src, int K, float eps) {
  const int b = mk_tid() >> 5, t32 = mk_tid() & 31;
  float ss = 0.f;
  for (int k = 4 * t32; k < K; k += 128) {
    const float4 v = src.load(b, k);
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
  ss = row_sum32(ss);
  return 1.0f / sqrtf(ss / (float)K + eps);
}

// Stage columns [c0, c0 + kc) of the 16 input rows into the bf16 high and
// low planes.  With a gain the row is RMS-normalised, x * rs * gain[k]; rs is
// computed here when the chunk is the whole row (kc == K), else taken from
// rs_in.  pre: the gain of a one-chunk row is already in LDS at MK_BGAIN.
template <class Src>
MKD void bstage(lds_char *L, const Src &src, int K, int c0, int kc, const uint16_t *gain, float eps, float rs_in,
                bool pre) {
  const int b = mk_tid() >> 5, t32 = mk_tid() & 31;
  const int nj = kc >> 7;
  float4 v[MK_BKC / 128];
#pragma unroll
  for (int j = 0; j < MK_BKC / 128; ++j)
    if (j < nj) v[j] = src.load(b, c0 + 4 * (t32 + 32 * j));
  float rs = rs_in;
  if (gain && kc == K) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < MK_BKC / 128; ++j)
      if (j < nj) {
        ss = fmaf(v[j].x, v[j].x, ss);
        ss = fmaf(v[j].y, v[j].y, ss);
        ss = fmaf(v[j].z, v[j].z, ss);
        ss = fmaf(v[j].w, v[j].w, ss);
      }
    ss = row_sum32(ss);
    rs = 1.0f / sqrtf(ss / (float)K + eps);
  }
  lds_u64 *hi = (lds_u64 *)(L + b * MK_BROW);
  lds_u64 *lo = (lds_u64 *)(L + MK_BPLANE + b * MK_BROW);
#pragma unroll
  for (int j = 0; j < MK_BKC / 128; ++j)
    if (j < nj) {
      const int c4 = t32 + 32 * j;  // float4 column inside the chunk
      float x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      if (gain) {
        const uint64_t g = pre ? ((const lds_u64 *)(L + MK_BGAIN))[c4] : gld((const uint64_t *)(gain + c0 + 4 * c4));
        const uint32_t g0 = (uint32_t)g, g1 = (uint32_t)(g >> 32);
        x[0] = (x[0] * rs) * bf_lo(g0);
        x[1] = (x[1] * rs) * bf_hi(g0);
        x[2] = (x[2] * rs) * bf_lo(g1);
        x[3] = (x[3] * rs) * bf_hi(g1);
      }
      uint32_t h0, h1, l0, l1;
      split2(x[0], x[1], h0, l0);
      split2(x[2], x[3], h1, l1);
      hi[c4] = (uint64_t)h0 | ((uint64_t)h1 << 32);
      lo[c4] = (uint64_t)l0 | ((uint64_t)l1 << 32);
    }
}

// ------------------------------------------------------- MFMA contraction
//
// Reduction step j of a wave covers 32 input columns: lane quarter
// q = lane / 16 takes columns 8 q .. + 7 of both operands.  A wave's steps
// run chunk by chunk (MK_BKC columns staged at a time; in chunk c it takes
// steps kp pc .. (kp + 1) pc - 1 of the chunk's pc = columns / 32 / ks); its
// weights are loaded PF steps ahead of use into registers (up to 16 steps,
// 16 KiB per wave), the first PF before the instruction's dependency wait,
// so the weight stream overlaps the wait, the input staging and the chunk
// barriers.

// One group of ng tiles starting at tile g0: wave (kp, wl), kp = wave / nw,
// wl = wave % nw, runs tiles g0 + wl + nw t (t < TPW) over reduction part kp
// of ks, with PF steps of weights in flight (PF divides a full chunk's steps
// per wave, (MK_BKC / 32) / ks).  Partial tiles (ks > 1) are added through LDS; fin(tile, acc) then
// runs on all 64 lanes of the wave holding the tile's full sums (lane: weight
// row 16 tile + lane % 16, sequences 4 (lane / 16) + j).  `wait` (the
// instruction's dependency wait) runs once the first weights are in flight
// when `first`; false from it aborts.
//
// TILED: the weights are stored as 1 KiB tiles in the operand order (tile
// (T, j): rows 16 T .. + 15, columns 32 j .. + 31, lane L's 16 bytes = row
// 16 T + L % 16, columns 32 j + 8 (L / 16) .. + 7), so every load
// instruction reads 1 KiB contiguous instead of 16 rows x 64 bytes; rowptr
// then gives the lane's address in step 0 of the tile.
template <int TPW, int PF, bool TILED, class Src, class RowPtr, class Fin, class Wait>
MKD bool bgemm_run(const Src &src, int K, int g0, int ng, int ks, bool first, const uint16_t *gain, float eps,
                   RowPtr rowptr, Fin fin, Wait wait) {
  lds_char *L = (lds_char *)mk_flat_lds;
  const int lane = mk_tid() & 63, wave = mk_tid() >> 6, n = lane & 15, q = lane >> 4;
  const int nw = MK_NWAVES / ks, kp = wave / nw, wl = wave - kp * nw;
  const int nch = (K + MK_BKC - 1) / MK_BKC, kcl = K - (nch - 1) * MK_BKC;
  const int per = (MK_BKC / 32) / ks, perl = (kcl / 32) / ks;  // steps per full / last chunk
  const int J = (nch - 1) * per + perl;
  auto col = [&](int j) {  // weight column of step j (this lane's quarter)
    const int c = min(j / per, nch - 1), s = j - c * per;
    return c * MK_BKC + 32 * (kp * (c == nch - 1 ? perl : per) + s) + 8 * q;
  };
  // element offset of step j's 16 bytes from the lane's row / tile pointer
  auto woff = [&](int j) -> size_t { return TILED ? (size_t)(col(j) >> 5) * 512 : (size_t)col(j); };
  const uint16_t *wrow[TPW];
  bool live[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    live[t] = wl + nw * t < ng;
    wrow[t] = rowptr(16 * (g0 + (live[t] ? wl + nw * t : 0)) + n);
  }
  const bool run = live[0];
  // The RMSNorm gain of a one-chunk row goes out first, one 4-bf16 piece per
  // thread, and into LDS once the wait is over: the gain is read once per
  // layer, so it comes from HBM, where a load issued after the wait would
  // queue behind every CU's weight stream.
  const bool pre = gain && nch == 1;
  uint64_t gpc = 0;
  if (pre && mk_tid() < (K >> 2)) gpc = gld((const uint64_t *)gain + mk_tid());
  mk_u32x4 w[PF][TPW];
  if (run)
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (p < J)
#pragma unroll
        for (int t = 0; t < TPW; ++t) w[p][t] = __builtin_nontemporal_load((const MK_G(mk_u32x4) *)(wrow[t] + woff(p)));
  if (first && !wait()) return false;
  if (pre) ((lds_u64 *)(L + MK_BGAIN))[mk_tid()] = gpc;  // read after the chunk loop's first barrier
  const float rs = (gain && nch > 1) ? bnorm_rs(src, K, eps) : 1.f;
  mk_f32x4v acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = mk_f32x4v{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nch; ++c) {
    const int last = c == nch - 1, kc = last ? kcl : MK_BKC, pc = last ? perl : per, j0 = c * per;
    lds_barrier();
    bstage(L, src, K, c * MK_BKC, kc, gain, eps, rs, pre);
    lds_barrier();
    if (run) {
      const lds_char *xc = L + n * MK_BROW + 16 * q + 64 * kp * pc;
      // j0 is a multiple of PF (per is), so step j0 + s + p sits in ring slot p
      for (int s = 0; s < pc; s += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
          if (s + p < pc) {
            const mk_u32x4 xh = *(const lds_u32x4 *)(xc + 64 * (s + p));
            const mk_u32x4 xl = *(const lds_u32x4 *)(xc + MK_BPLANE + 64 * (s + p));
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
              acc[t] = mfma16x16x32(as_bf16x8(xh), as_bf16x8(w[p][t]), acc[t]);
              acc[t] = mfma16x16x32(as_bf16x8(xl), as_bf16x8(w[p][t]), acc[t]);
            }
            const int jn = j0 + s + p + PF;
            if (jn < J)
#pragma unroll
              for (int t = 0; t < TPW; ++t)
                w[p][t] = __builtin_nontemporal_load((const MK_G(mk_u32x4) *)(wrow[t] + woff(jn)));
          }
        }
      }
    }
  }
  if (ks > 1) {
    lds_f32x4 *red = (lds_f32x4 *)(L + MK_BRED);
    if (kp > 0) red[wave * 64 + lane] = acc[0];
    lds_barrier();
    if (kp == 0 && run)
      for (int k2 = 1; k2 < ks; ++k2) acc[0] += red[(wave + k2 * nw) * 64 + lane];
  }
  if (kp == 0)
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      if (live[t]) fin(g0 + wl + nw * t, acc[t]);
  return true;
}

// Y[b][r] for the instruction's nt tiles of 16 rows (rowptr(v): weight row
// of virtual row v in [0, 16 nt), already clamped to a valid row), inputs
// from src (K columns, RMSNorm with `gain` when non-null).
template <bool TILED = false, class Src, class RowPtr, class Fin, class Wait>
MKD bool bgemm(const Src &src, int K, int nt, const uint16_t *gain, float eps, RowPtr rowptr, Fin fin, Wait wait) {
  // up to 16 steps (64 registers) of weights in flight per wave
  if (nt == 1) return bgemm_run<1, 8, TILED>(src, K, 0, nt, 8, true, gain, eps, rowptr, fin, wait);
  if (nt == 2) return bgemm_run<1, 16, TILED>(src, K, 0, nt, 4, true, gain, eps, rowptr, fin, wait);
  if (nt < MK_NWAVES)
    return bgemm_run<1, 16, TILED>(src, K, 0, nt, nt <= 4 ? 2 : 1, true, gain, eps, rowptr, fin, wait);
  for (int g0 = 0; g0 < nt; g0 += 4 * MK_NWAVES) {
    const int ng = min(nt - g0, 4 * MK_NWAVES);
    const bool first = g0 == 0;
    bool ok;
    if (ng > 2 * MK_NWAVES)
      ok = bgemm_run<4, 4, TILED>(src, K, g0, ng, 1, first, gain, eps, rowptr, fin, wait);
    else if (ng > MK_NWAVES)
      ok = bgemm_run<2, 8, TILED>(src, K, g0, ng, 1, first, gain, eps, rowptr, fin, wait);
    else
      ok = bgemm_run<1, 8, TILED>(src, K, g0, ng, 1, first, gain, eps, rowptr, fin, wait);
    if (!ok) return false;
  }
  return true;
}

// ------------------------------------------------------------ batched ops

MKD bool tokens_ok_all(const MkProgram &P, const MkStep &S) {
  const int tid = mk_tid();
  int tok = 0;
  const bool bad = tid < S.batch && !token_ok(P, S, tid, &tok);
  if (bad) mk_raise(P, MK_E_INPUT, tid);
  return __syncthreads_or(bad) == 0;
}

template <class Wait>
MKD int op_qkv_b(const MkProgram &P, const MkStep &S, const MkInstr &in, Wait wait) {
  const int H = P.H, l = in.layer, nb = S.batch, lane = mk_tid() & 63;
  const int R = (P.nq + 2 * P.nkv) * P.d, qd = P.nq * P.d, kd = P.nkv * P.d;
  const int r0 = in.r0, nr = in.r1 - in.r0, nt = (nr + 15) >> 4;
  const MkLayerW W = cld(&P.layers[l]);
  // the slice lies inside one of q, k, v (the planner keeps it inside one
  // head): a per-lane choice of the tensor became a lookup table in scratch
  const uint16_t *base = r0 < qd ? W.wq + (size_t)r0 * H
                         : r0 < qd + kd ? W.wk + (size_t)(r0 - qd) * H
                                        : W.wv + (size_t)(r0 - qd - kd) * H;
  auto rowptr = [&](int v) -> const uint16_t * { return base + (size_t)min(v, nr - 1) * H; };
  float *out = P.qkv + (size_t)l * P.B_max * R + r0;
  auto fin = [&](int tile, mk_f32x4v a) {
    const int v = 16 * tile + (lane & 15), b0 = 4 * (lane >> 4);
    if (v < nr)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (b0 + j < nb) stc(out + (size_t)(b0 + j) * R + v, a[j]);
  };
  if (l == 0) {
    if (!tokens_ok_all(P, S)) return MK_ST_ABORT;
    const int b = mk_tid() >> 5;
    const BEmbSrc src{b < nb ? P.embed + (size_t)ldci(S.tokens + b) * H : nullptr};
    if (!bgemm(src, H, nt, W.attn_norm, P.eps, rowptr, fin, wait)) return MK_ST_ABORT;
  } else {
    if (!bgemm(bact(P.xout + (size_t)(l - 1) * P.B_max * H, nb, H), H, nt, W.attn_norm, P.eps, rowptr, fin, wait))
      return MK_ST_ABORT;
  }
  return MK_ST_SIGNAL;
}

template <class Wait>
MKD int op_oproj_b(const MkProgram &P, const MkStep &S, const MkInstr &in, Wait wait) {
  const int H = P.H, l = in.layer, K = P.nq * P.d, nb = S.batch, lane = mk_tid() & 63;
  const int r0 = in.r0, nr = in.r1 - in.r0, nt = (nr + 15) >> 4;
  if (l == 0 && !tokens_ok_all(P, S)) return MK_ST_ABORT;
  const MkLayerW W = cld(&P.layers[l]);
  float *out = P.xmid + (size_t)l * P.B_max * H;
  auto fin = [&](int tile, mk_f32x4v a) {
    const int v = 16 * tile + (lane & 15), b0 = 4 * (lane >> 4);
    if (v < nr)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = b0 + j;
        if (b < nb) {
          const int row = r0 + v;
          const float res = l == 0 ? bf2f(P.embed[(size_t)ldci(S.tokens + b) * H + row])
                                   : ldc(P.xout + ((size_t)(l - 1) * P.B_max + b) * H + row);
          stc(out + (size_t)b * H + row, res + a[j]);
        }
      }
  };
  if (!bgemm(bact(P.attn + (size_t)l * P.B_max * K, nb, K), K, nt, nullptr, 0.f,
             [&](int v) { return W.wo + (size_t)(r0 + min(v, nr - 1)) * K; }, fin, wait))
    return MK_ST_ABORT;
  return MK_ST_SIGNAL;
}

// gate/up: tile t holds hidden units r0 + 8 t .. + 7 as virtual rows 0..7
// (gate) and 8..15 (up), so lane n and lane n + 8 of a row group hold the
// gate and up sums of one unit.
template <class Wait>
MKD int op_gateup_b(const MkProgram &P, const MkStep &S, const MkInstr &in, Wait wait) {
  const int H = P.H, l = in.layer, nb = S.batch, lane = mk_tid() & 63;
  const int r0 = in.r0, nh = in.r1 - in.r0, nt = (nh + 7) >> 3;
  const MkLayerW W = cld(&P.layers[l]);
  auto rowptr = [&](int v) -> const uint16_t * {
    const int u = r0 + min(8 * (v >> 4) + (v & 7), nh - 1);
    return ((v & 8) ? W.wu : W.wg) + (size_t)u * H;
  };
  float *out = P.hbuf + (size_t)l * P.B_max * P.I + r0;
  auto fin = [&](int tile, mk_f32x4v a) {
    const int n = lane & 15, u = 8 * tile + n, b0 = 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float up = __shfl_xor(a[j], 8, 64);
      const float g = a[j];
      if (n < 8 && u < nh && b0 + j < nb) stc(out + (size_t)(b0 + j) * P.I + u, (g / (1.0f + expf(-g))) * up);
    }
  };
  const BActSrc xsrc = bact(P.xmid + (size_t)l * P.B_max * H, nb, H);
  bool ok;
  if (P.gu_tiled && (r0 & 7) == 0) {
    // tile t of this slice is tile r0 / 8 + t of the layer's tiled gate/up copy
    const uint16_t *tb = P.gu_tiled + (size_t)l * 2 * P.I * H + (size_t)(r0 >> 3) * (H >> 5) * 512 + 8 * lane;
    ok = bgemm<true>(xsrc, H, nt, W.mlp_norm, P.eps, [&](int v) { return tb + (size_t)(v >> 4) * (H >> 5) * 512; }, fin,
                     wait);
  } else {
    ok = bgemm(xsrc, H, nt, W.mlp_norm, P.eps, rowptr, fin, wait);
  }
  if (!ok) return MK_ST_ABORT;
  return MK_ST_SIGNAL;
}

// Every split of an attention unit (every part of a split down slice) takes
// a ticket once its partial is stored; true (uniformly) on the last arriver
// of this step.
MKD bool attn_ticket(const MkProgram &P, const MkStep &S, const MkInstr &in, int *s_flag) {
  wait_vm();
  __syncthreads();
  if (mk_tid() == 0) {
    const uint32_t old = addcu(P.tickets + in.ticket, 1u);
    *s_flag = (old + 1u == (S.epoch + 1u) * (uint32_t)in.nsplit) ? 1 : 0;
  }
  __syncthreads();
  const int last = *s_flag;
  __syncthreads();
  return last != 0;
}

// Down projection.  A slice split by input columns (in.nsplit parts of
// K / nsplit columns, one staged chunk each) stores its partial tile in
// dpart; the last part to finish (ticket) adds the parts in part order and
// the residual, and stores the rows.
template <class Wait>
MKD int op_down_b(const MkProgram &P, const MkStep &S, const MkInstr &in, int *s_flag, Wait wait) {
  const int H = P.H, l = in.layer, K = P.I, nb = S.batch, lane = mk_tid() & 63;
  const int r0 = in.r0, nr = in.r1 - in.r0, nt = (nr + 15) >> 4;
  const int NS = in.nsplit, Kp = K / NS, k0 = in.split * Kp;
  const MkLayerW W = cld(&P.layers[l]);
  const float *xm = P.xmid + (size_t)l * P.B_max * H;
  float *out = P.xout + (size_t)l * P.B_max * H;
  float *dp = P.dpart + (size_t)l * NS * P.B_max * H;  // part s, sequence b, row r: dp[(s B_max + b) H + r]
  auto fin = [&](int tile, mk_f32x4v a) {
    const int v = 16 * tile + (lane & 15), b0 = 4 * (lane >> 4);
    if (v < nr)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (b0 + j < nb) {
          const size_t o = (size_t)(b0 + j) * H + r0 + v;
          if (NS == 1)
            stc(out + o, ldc(xm + o) + a[j]);
          else
            stc(dp + (size_t)in.split * P.B_max * H + o, a[j]);
        }
  };
  // the part's columns: rows of hbuf from column k0 on (row stride K), and
  // the same columns of every weight row
  if (!bgemm(bact(P.hbuf + (size_t)l * P.B_max * K + k0, nb, K), Kp, nt, nullptr, 0.f,
             [&](int v) { return W.wd + (size_t)(r0 + min(v, nr - 1)) * K + k0; }, fin, wait))
    return MK_ST_ABORT;
  if (NS == 1) return MK_ST_SIGNAL;
  if (!attn_ticket(P, S, in, s_flag)) return MK_ST_QUIET;
  for (int i = mk_tid(); i < nb * nr; i += MK_BLOCK) {
    const int b = i / nr, v = i - b * nr;
    const size_t o = (size_t)b * H + r0 + v;
    float acc = ldc(dp + o);
    for (int s2 = 1; s2 < NS; ++s2) acc += ldc(dp + (size_t)s2 * P.B_max * H + o);
    stc(out + o, ldc(xm + o) + acc);
  }
  return MK_ST_SIGNAL;
}

template <class Wait>
MKD int op_lmhead_b(const MkProgram &P, const MkStep &S, const MkInstr &in, int *s_flag, Wait wait) {
  const int H = P.H, V = P.V, nb = S.batch, tid = mk_tid(), lane = tid & 63, wave = tid >> 6;
  const int r0 = in.r0, nr = in.r1 - in.r0, nt = (nr + 15) >> 4;
  const uint16_t *Wlm = P.tied ? P.embed : P.lm_head;
  float bv[4];
  int bi[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bv[j] = -INFINITY;
    bi[j] = 0x7fffffff;
  }
  auto fin = [&](int tile, mk_f32x4v a) {
    const int v = 16 * tile + (lane & 15), b0 = 4 * (lane >> 4);
    if (v < nr)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (b0 + j < nb) {
          const int row = r0 + v;
          S.logits[(size_t)(b0 + j) * V + row] = a[j];
          if (better(a[j], row, bv[j], bi[j])) {
            bv[j] = a[j];
            bi[j] = row;
          }
        }
  };
  const BActSrc xsrc = bact(P.xout + (size_t)(P.L - 1) * P.B_max * H, nb, H);
  bool ok;
  if (P.lm_tiled && (r0 & 15) == 0) {
    // the tiled copy of the LM-head matrix (tiles of global rows 16 T ..)
    const uint16_t *tb = P.lm_tiled + (size_t)(r0 >> 4) * (H >> 5) * 512 + 8 * lane;
    ok = bgemm<true>(xsrc, H, nt, P.final_norm, P.eps,
                     [&](int v) { return tb + (size_t)(v >> 4) * (H >> 5) * 512; }, fin, wait);
  } else {
    ok = bgemm(xsrc, H, nt, P.final_norm, P.eps, [&](int v) { return Wlm + (size_t)(r0 + min(v, nr - 1)) * H; }, fin,
               wait);
  }
  if (!ok) return MK_ST_ABORT;
  // best per sequence: over the 16 rows of a lane group, then over waves
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv[j], o, 16);
      const int oi = __shfl_xor(bi[j], o, 16);
      if (better(ov, oi, bv[j], bi[j])) {
        bv[j] = ov;
        bi[j] = oi;
      }
    }
  lds_char *L = (lds_char *)mk_flat_lds;
  lds_float *av = (lds_float *)(L + MK_BARG);
  lds_u32 *ai = (lds_u32 *)(L + MK_BARG + MK_NWAVES * MK_MAX_BATCH * 4);
  if ((lane & 15) == 0)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      av[wave * MK_MAX_BATCH + 4 * (lane >> 4) + j] = bv[j];
      ai[wave * MK_MAX_BATCH + 4 * (lane >> 4) + j] = (uint32_t)bi[j];
    }
  __syncthreads();
  if (tid < nb) {
    float v = av[tid];
    int ix = (int)ai[tid];
    for (int w = 1; w < MK_NWAVES; ++w) {
      const float wv = av[w * MK_MAX_BATCH + tid];
      const int wi = (int)ai[w * MK_MAX_BATCH + tid];
      if (better(wv, wi, v, ix)) {
        v = wv;
        ix = wi;
      }
    }
    stc64(P.lm_pk + (size_t)in.part * P.B_max + tid, lm_pack(v, ix, S.epoch));
  }
  __syncthreads();
  return lm_merge(P, S, in);
}

// ------------------------------------------- attention on the matrix cores
//
// One (sequence b, kv head g, key split s) unit of the homogeneous engine:
// rotate the group's q heads and the new key at position p, store the new
// key/value (bf16, RNE) into cache slot p when this split holds it, then the
// softmax-weighted value sums over the split's key range for every q head of
// the group.  The waves take 32-position blocks in turn: scores S = K q on
// the matrix cores (A = 16 key rows, B = the group's queries as bf16 high and
// low parts, the queries scaled by log2(e)/sqrt(d) so that the softmax runs
// on exp2), an online max / sum per head, then O += P V (A = probabilities
// as bf16 high and low parts, B = values gathered from the wave's LDS copy of
// the block).  Keys feed the MFMA straight from HBM; each wave loads its
// next block while it computes the current one.  The waves' partials are
// merged in LDS; with several splits each split stores (max, sum, output)
// and the last one to finish merges them (log-sum-exp rescaling, base 2).
//
// k index maps: the score product gives lane quarter qd the dims
// (d/4) qd + 8 s + 0..7 of k-step s (one contiguous run of a key row per
// lane); the value product gives it positions 4 qd + j (j < 4) and
// 16 + 4 qd + j - 4 (j >= 4), exactly where the score product left that
// lane's probabilities.

template <int D>
struct FaBlock {
  static constexpr int KS = D / 32, CPR = D / 8, CPL = D / 16, DQ = D / 4;
  mk_u32x4 k[2][KS];   // key rows ta + 16 T + lane % 16 (A operand)
  mk_u32x4 v[CPL];     // value block, 16-byte chunks lane + 64 r
};

// Global loads of the block at positions ta .. ta + 31 (rows past the split
// end repeat its last row; their scores are masked).  Slot p of the cache is
// being written by this step, so its row is replaced from LDS afterwards.
template <int D>
MKD void fa_load(FaBlock<D> &f, const uint16_t *Kc, const uint16_t *Vc, int ta, int t1) {
  const int lane = mk_tid() & 63, col = lane & 15, qd = lane >> 4;
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const int t = min(ta + 16 * T + col, t1 - 1);
#pragma unroll
    for (int s = 0; s < FaBlock<D>::KS; ++s)
      f.k[T][s] = gld((const mk_u32x4 *)(Kc + (size_t)t * D + FaBlock<D>::DQ * qd + 8 * s));
  }
#pragma unroll
  for (int r = 0; r < FaBlock<D>::CPL; ++r) {
    const int c = lane + 64 * r, row = c / FaBlock<D>::CPR, ch = c - row * FaBlock<D>::CPR;
    f.v[r] = gld((const mk_u32x4 *)(Vc + (size_t)min(ta + row, t1 - 1) * D + 8 * ch));
  }
}

template <int D, bool SENT, class Wait>
MKD int op_attn_d(const MkProgram &P, const MkStep &S, const MkInstr &in, int *s_flag, Wait &wait) {
  constexpr int KS = D / 32, NT = D / 16, DQ = D / 4, HALF = D / 2, CPR = D / 8, CPL = D / 16;
  constexpr int VROW = 2 * D + 16;  // bytes per value row in LDS (+16: the gathers' four rows hit distinct banks)
  const int b = in.r0, g = in.r1, sp = in.split, NS = in.nsplit, l = in.layer;
  const int G = P.G, nq = P.nq, nkv = P.nkv;
  const int tid = mk_tid(), lane = tid & 63, wave = tid >> 6, col = lane & 15, qd = lane >> 4;
  // a sequence slot beyond this step's batch: no position, no queries, no
  // cache access; the unit only keeps the event and ticket protocol
  if (b >= S.batch) return NS == 1 ? MK_ST_SIGNAL : attn_ticket(P, S, in, s_flag) ? MK_ST_SIGNAL : MK_ST_QUIET;
  const int p = ldci(S.positions + b);
  if (p < 0 || p >= P.max_ctx) {
    if (tid == 0) mk_raise(P, MK_E_INPUT, 1000 + b);
    return MK_ST_ABORT;
  }
  const int n = p + 1;
  const int chunk = (n + NS - 1) / NS;
  const int t0 = min(n, sp * chunk), t1 = min(n, t0 + chunk);
  const int R = (nq + 2 * nkv) * D;
  const float *qkv = P.qkv + ((size_t)l * P.B_max + b) * R;
  lds_char *L = (lds_char *)mk_flat_lds;
  lds_float *qs = (lds_float *)(L + MK_FA_Q);
  lds_u16 *kn = (lds_u16 *)(L + MK_FA_KN), *vn = (lds_u16 *)(L + MK_FA_VN);

  uint16_t *Kc = S.kv + kv_off(P, l, 0, b, g);
  uint16_t *Vc = S.kv + kv_off(P, l, 1, b, g);
  // the cached keys and values do not depend on this step: their first blocks
  // load while the wave waits (slot p is read stale and replaced below)
  lds_char *vb = L + MK_FA_VB + wave * (32 * VROW);
  const int nu = (t1 - t0 + 31) >> 5;
  // blocks u = wave + 8 i; DEPTH of them in flight per wave (a register ring;
  // head_dim 128 keeps one: more would spill)
  constexpr int DEPTH = D == 64 ? 3 : 1;
  FaBlock<D> ring[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i)
    if (wave + MK_NWAVES * i < nu) fa_load<D>(ring[i], Kc, Vc, t0 + 32 * (wave + MK_NWAVES * i), t1);
  if (!wait()) return MK_ST_ABORT;

  // RoPE on the group's queries (scaled) and the new key; the new value
  const float *cs = P.rope + (size_t)p * D;  // (cos, sin) pairs
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
  // (sentinel mode: each word is polled until its producer has written it)
  constexpr bool sent = SENT;
  bool ok = true;
  for (int e = tid; e < G * HALF; e += MK_BLOCK) {
    const int j = e / HALF, i = e - j * HALF;
    const float *qh = qkv + (size_t)(g * G + j) * D;
    const float a = ldcp(P, qh + i, sent, ok), c = ldcp(P, qh + i + HALF, sent, ok);
    const float co = cs[2 * i], si = cs[2 * i + 1];
    qs[j * D + i] = (a * co - c * si) * qscale;
    qs[j * D + i + HALF] = (c * co + a * si) * qscale;
  }
  for (int i = tid; i < HALF; i += MK_BLOCK) {
    const float *kh = qkv + (size_t)(nq + g) * D;
    const float a = ldcp(P, kh + i, sent, ok), c = ldcp(P, kh + i + HALF, sent, ok);
    const float co = cs[2 * i], si = cs[2 * i + 1];
    kn[i] = f2bf(a * co - c * si);
    kn[i + HALF] = f2bf(c * co + a * si);
  }
  for (int i = tid; i < D; i += MK_BLOCK) vn[i] = f2bf(ldcp(P, qkv + (size_t)(nq + nkv + g) * D + i, sent, ok));
  if (block_failed<SENT>(ok, true)) return MK_ST_ABORT;

  // the appended row is stored device-coherently (as bf16 pairs): a later
  // step of the same launch may read it from another XCD
  if (t0 <= p && p < t1)
    for (int i = tid; i < HALF; i += MK_BLOCK) {
      stcu(reinterpret_cast<uint32_t *>(Kc + (size_t)p * D) + i, (uint32_t)kn[2 * i] | ((uint32_t)kn[2 * i + 1] << 16));
      stcu(reinterpret_cast<uint32_t *>(Vc + (size_t)p * D) + i, (uint32_t)vn[2 * i] | ((uint32_t)vn[2 * i + 1] << 16));
    }

  // queries as the B operand (column = head), high and low parts
  mk_u32x4 qhi[KS], qlo[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = col < G ? qs[col * D + DQ * qd + 8 * s + e] : 0.f;
    split_hi_lo(x, qhi[s], qlo[s]);
  }
  float m = -INFINITY, lsum = 0.f;  // running max / partial sum of head `col`
  mk_f32x4v o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = mk_f32x4v{0.f, 0.f, 0.f, 0.f};
  auto process = [&](FaBlock<D> &blk, int u) {
    const int ta = t0 + 32 * u, npos = min(32, t1 - ta);
    // the value block into this wave's LDS rows
#pragma unroll
    for (int r = 0; r < CPL; ++r) {
      // rows past the block's last position repeat a cache row (possibly
      // slot p's stale contents); they meet zero probabilities, and are
      // zeroed so a non-finite stale value cannot reach the product
      const int c = lane + 64 * r, row = c / CPR, ch = c - row * CPR;
      *(lds_u32x4 *)(vb + row * VROW + 16 * ch) = row < npos ? blk.v[r] : mk_u32x4{0u, 0u, 0u, 0u};
    }
    if (ta <= p && p < ta + 32 && lane < CPR) {  // this step's value at slot p
      const int row = p - ta;
      *(lds_u32x4 *)(vb + row * VROW + 16 * lane) = *(const lds_u32x4 *)(vn + 8 * lane);
    }
    // scores of the two 16-position tiles
    float sc[2][4];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      mk_f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        mk_u32x4 kk = blk.k[T][s];
        if (ta + 16 * T + col == p) kk = *(const lds_u32x4 *)(kn + DQ * qd + 8 * s);  // this step's key
        acc = mfma16x16x32(as_bf16x8(kk), as_bf16x8(qhi[s]), acc);
        acc = mfma16x16x32(as_bf16x8(kk), as_bf16x8(qlo[s]), acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[T][j] = 16 * T + 4 * qd + j < npos ? acc[j] : -INFINITY;
    }
    if (u + MK_NWAVES * DEPTH < nu) fa_load<D>(blk, Kc, Vc, ta + 32 * MK_NWAVES * DEPTH, t1);
    // online softmax of head `col` (lanes col, col + 16, col + 32, col + 48 share it)
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
    lsum = fmaf(lsum, c, ls);
    m = mn;
    // output row h (head h) sits in register h % 4 of lanes 16 (h / 4) ..: rescale
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float cj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), j));
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t][j] *= cj;
    }
    mk_u32x4 phi, plo;
    split_hi_lo(pr, phi, plo);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's value rows are in LDS
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int dim = 16 * t + col;
      uint32_t vv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = j < 4 ? 4 * qd + j : 16 + 4 * qd + (j - 4);
        vv[j] = *(const lds_u16 *)(vb + row * VROW + 2 * dim);
      }
      const mk_u32x4 vw = {vv[0] | (vv[1] << 16), vv[2] | (vv[3] << 16), vv[4] | (vv[5] << 16), vv[6] | (vv[7] << 16)};
      o[t] = mfma16x16x32(as_bf16x8(phi), as_bf16x8(vw), o[t]);
      o[t] = mfma16x16x32(as_bf16x8(plo), as_bf16x8(vw), o[t]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // gathers done before the rows are rewritten
  };
  for (int u0 = wave; u0 < nu; u0 += MK_NWAVES * DEPTH) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i)
      if (u0 + MK_NWAVES * i < nu) process(ring[i], u0 + MK_NWAVES * i);
  }
  // wave partials per head: max, sum, unnormalised output (base-2 scores)
  lsum = sum_x16(lsum);
  lsum = sum_x32(lsum);
  lds_float *wpa = (lds_float *)(L + MK_FA_WP);
  lds_float *wp = wpa + wave * MK_MAX_GROUP * (D + 2);
  if (lane < G) {
    wp[lane * (D + 2)] = m;
    wp[lane * (D + 2) + 1] = lsum;
  }
  if (qd == 0)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < G) wp[j * (D + 2) + 2 + 16 * t + col] = o[t][j];
  __syncthreads();

  float *attn_out = P.attn + ((size_t)l * P.B_max + b) * nq * D + (size_t)g * G * D;
  float *part = P.part + ((((size_t)l * P.B_max + b) * nkv + g) * NS) * G * (D + 2);
  if (tid < G * D) {
    const int j = tid / D, i = tid - j * D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < MK_NWAVES; ++w) mx = fmaxf(mx, wpa[(w * MK_MAX_GROUP + j) * (D + 2)]);
    float z = 0.f, ov = 0.f;
#pragma unroll
    for (int w = 0; w < MK_NWAVES; ++w) {
      const lds_float *e = wpa + (w * MK_MAX_GROUP + j) * (D + 2);
      const float cw = e[0] == -INFINITY ? 0.f : exp2_fast(e[0] - mx);
      z = fmaf(e[1], cw, z);
      ov = fmaf(e[2 + i], cw, ov);
    }
    if (NS == 1) {
      stc(attn_out + tid, ov / z);
    } else {
      float *pp = part + ((size_t)sp * G + j) * (D + 2);
      stc(pp + 2 + i, ov);
      if (i == 0) {
        stc(pp, mx);
        stc(pp + 1, z);
      }
    }
  }
  if (NS == 1) return MK_ST_SIGNAL;
  // last arriver merges the splits
  if (!attn_ticket(P, S, in, s_flag)) return MK_ST_QUIET;
  if (tid < G * D) {
    const int j = tid / D, i = tid - j * D;
    stc(attn_out + tid, merge_splits(part, NS, G, D, j, i));
  }
  return MK_ST_SIGNAL;
}

template <bool SENT = false, class Wait>
MKD int op_attn_mfma(const MkProgram &P, const MkStep &S, const MkInstr &in, int *s_flag, Wait &wait) {
  return P.d == 64 ? op_attn_d<64, SENT>(P, S, in, s_flag, wait) : op_attn_d<128, SENT>(P, S, in, s_flag, wait);
}

// ----------------------------------------------------------------- dispatch

// Run one instruction.  Every op starts the loads that do not depend on the
// instruction's input event (weights; attention's cached keys and values),
// then waits for the event inside.  `ts`
// receives the time the wait ended when `timed`.  SENT: data-sentinel
// synchronisation (one sequence per step; the ops poll their inputs and no
// event is waited for).
// NOWAIT: launched per dependency level (the kernel boundary orders the
// levels; nothing is waited for).
template <bool SENT, bool NOWAIT = false>
MKD int run_instr(const MkProgram &P, const MkStep &S, const MkInstr &in, float *smem, int *s_flag, bool timed,
                  uint64_t &ts) {
  auto wait = [&]() -> bool {
    const bool ok = SENT || NOWAIT || in.wait_ev < 0 || mk_wait(P, S, in.wait_ev, s_flag);
    if (timed) ts = __builtin_amdgcn_s_memrealtime();
    return ok;
  };
  // (a down slice split by input columns runs as parts whatever the step's
  // batch: its plan counts one trigger per slice, from the merging part)
  if (!SENT && (S.batch >= MK_MFMA_MIN_BATCH || (in.op == MKOP_DOWN && in.nsplit > 1))) {
    switch (in.op) {
      case MKOP_QKV: return op_qkv_b(P, S, in, wait);
      case MKOP_OPROJ: return op_oproj_b(P, S, in, wait);
      case MKOP_GATEUP: return op_gateup_b(P, S, in, wait);
      case MKOP_DOWN: return op_down_b(P, S, in, s_flag, wait);
      case MKOP_LMHEAD: return op_lmhead_b(P, S, in, s_flag, wait);
      default: break;
    }
  }
  switch (in.op) {
    case MKOP_QKV: return op_qkv<SENT>(P, S, in, smem, wait);
    case MKOP_OPROJ: return op_oproj<SENT>(P, S, in, smem, wait);
    case MKOP_GATEUP: {
      auto none = []() -> bool { return true; };
      return op_gateup<SENT>(P, S, in, smem, wait, none);
    }
    case MKOP_DOWN: return op_down<SENT>(P, S, in, smem, wait);
    case MKOP_LMHEAD: return op_lmhead<SENT>(P, S, in, smem, s_flag, wait);
    case MKOP_ATTN: return op_attn_mfma<SENT>(P, S, in, s_flag, wait);
    default: return MK_ST_ABORT;
  }
}

// One sequence: a CU's O projection and the gate/up instruction that follows
// it in its list run as one unit.  Gate/up's weights (the largest level of a
// layer) are requested first, then the O projection waits for attention,
// computes and signals; the weights travel meanwhile, through the attention
// and O levels, which move little data.  Returns gate/up's status; O's
// status is signalled here.  ts_o / te_o / ts_g: end of O's wait, end of O,
// end of gate/up's wait (when `timed`).
template <bool SENT>
MKD int run_o_gateup(const MkProgram &P, const MkStep &S, const MkInstr &io, const MkInstr &ig, float *smem, int *s_flag,
                     bool timed, uint64_t &ts_o, uint64_t &te_o, uint64_t &ts_g) {
  auto wait_o = [&]() -> bool {
    const bool ok = SENT || io.wait_ev < 0 || mk_wait(P, S, io.wait_ev, s_flag);
    if (timed) ts_o = __builtin_amdgcn_s_memrealtime();
    return ok;
  };
  auto wait_g = [&]() -> bool {
    const bool ok = SENT || ig.wait_ev < 0 || mk_wait(P, S, ig.wait_ev, s_flag);
    if (timed) ts_g = __builtin_amdgcn_s_memrealtime();
    return ok;
  };
  auto o_first = [&]() -> bool {
    const int st = op_oproj<SENT, 1>(P, S, io, smem, wait_o);
    if (st == MK_ST_ABORT) return false;
    if (!SENT && st == MK_ST_SIGNAL && io.sig_ev >= 0) mk_signal(P, S, io.sig_ev, io.sig_slot);
    __syncthreads();
    if (timed) te_o = __builtin_amdgcn_s_memrealtime();
    return true;
  };
  return op_gateup<SENT>(P, S, ig, smem, wait_g, o_first);
}
