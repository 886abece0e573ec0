// Device helpers: bf16 unpacking, wave/block reductions, device-coherent
// loads/stores and the dependency wait/trigger protocol.
//
// Cross-CU data on MI355X: each of the 8 XCDs has its own L2, so data one
// workgroup writes for another must not sit in a private L2.  Activations
// and partials are therefore written with device-scope (sc1) stores, which
// write through to the coherent level, and read with device-scope (sc1)
// loads.  A producer waits for its own stores to complete before it
// triggers an event; consumers poll the event and only then read.  This is
// the counter protocol of the megakernel page, section 2.6 item 3 (fence,
// then one representative thread bumps the output counter; one thread spins
// on the input counter with a sleep, then the block synchronises), with the
// fence replaced by completion of write-through stores so that no whole-L2
// writeback or invalidate is needed.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_program.h"

#define MKD __device__ __forceinline__

typedef uint32_t mk_u32x4 __attribute__((ext_vector_type(4)));
// LDS-typed pointers (address space 3): ds_* instructions, no generic-pointer checks
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) mk_u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) float lds_float;
typedef float mk_f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) mk_f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint64_t lds_u64;

#define MK_E_TIMEOUT (-7)
#define MK_E_INPUT (-8)

MKD float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
MKD float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
MKD float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// fp32 -> bf16, round to nearest even (NaN stays NaN)
MKD uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Device-coherent accesses (sc1): visible across XCDs without cache
// maintenance.  The pointers are cast to the global address space so the
// compiler emits global_* instructions; a generic (flat) access would also
// count against the LDS counter and make every later LDS fence wait for the
// memory round trip.
#define MK_G(T) __attribute__((address_space(1))) T
MKD float ldc(const float *p) { return __hip_atomic_load((MK_G(float) *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MKD void stc(float *p, float v) { __hip_atomic_store((MK_G(float) *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MKD int32_t ldci(const int32_t *p) { return __hip_atomic_load((MK_G(int32_t) *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MKD void stci(int32_t *p, int32_t v) { __hip_atomic_store((MK_G(int32_t) *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MKD uint32_t ldcu(const uint32_t *p) { return __hip_atomic_load((MK_G(uint32_t) *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MKD void stcu(uint32_t *p, uint32_t v) { __hip_atomic_store((MK_G(uint32_t) *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MKD uint64_t ldc64(const uint64_t *p) { return __hip_atomic_load((MK_G(uint64_t) *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MKD void stc64(uint64_t *p, uint64_t v) { __hip_atomic_store((MK_G(uint64_t) *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MKD uint32_t addcu(uint32_t *p, uint32_t v) { return __hip_atomic_fetch_add((MK_G(uint32_t) *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// plain global store / load (no coherence requirement)
template <class T> MKD void gst(T *p, T v) { *(MK_G(T) *)p = v; }
template <class T> MKD T gld(const T *p) { return *(const MK_G(T) *)p; }

MKD __amdgpu_buffer_rsrc_t mk_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}
// 16-byte load with device scope (sc1): coherent across XCDs
MKD mk_u32x4 ldc16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16);
}

// Thread index as an opaque per-use value: the engine's instruction loop
// inlines every op, and values derived from a loop-invariant thread index
// would otherwise be hoisted out of that loop and stay live (in registers)
// across all ops.
MKD int mk_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Workgroup barrier that waits for LDS traffic only (a __syncthreads would
// also wait for every global load in flight, draining the weight prefetch).
MKD void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS flags are plain ds instructions in inline assembly, with no fences.
// A wave's LDS operations execute in program order and LDS is shared by the
// whole workgroup, so a flag written after a wave's data writes (or after its
// last reads of a page) is seen only once those have taken effect.  Compiled
// atomics with workgroup fences would instead wait for every global access
// still in flight (global->LDS loads write LDS and are counted by vmcnt; the
// compiler cannot prove they do not overlap the flag), which puts a full
// memory round trip on every page a compute wave frees after storing an
// output.  Ordering against global memory is made explicit where it matters
// (a vmcnt wait before a wave reports results that other CUs will read).
MKD uint32_t lds_off(const lds_u32 *p) { return (uint32_t)(size_t)p; }
MKD uint32_t lds_ld(lds_u32 *p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(p)) : "memory");
  return __builtin_amdgcn_readfirstlane(v);  // one address for the wave: the value is uniform
}
MKD void lds_st(lds_u32 *p, uint32_t v) { asm volatile("ds_write_b32 %0, %1" ::"v"(lds_off(p)), "v"(v) : "memory"); }
MKD void lds_add(lds_u32 *p, uint32_t v) { asm volatile("ds_add_u32 %0, %1" ::"v"(lds_off(p)), "v"(v) : "memory"); }

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

// wait until this wave's outstanding memory operations (stores included) completed
MKD void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

MKD float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Wave-wide sum with DPP lane moves (no LDS traffic): quad swaps, half-row
// and row mirrors give every lane its 16-lane row sum, two row broadcasts
// accumulate the four rows into lane 63, which is then read as a scalar.
template <int CTRL, int ROWMASK>
MKD float dpp_term(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}
MKD float wave_total(float v) {
  v += dpp_term<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_term<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_term<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_term<0x140, 0xF>(v);  // row_mirror
  v += dpp_term<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_term<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Sum over the wave (all 64 lanes active), returned to every lane.  DPP
// moves instead of cross-lane LDS permutes: the GEMV finishes each row group
// with one of these per row, and six dependent LDS round trips per row group
// sat on the dependency chain of every projection.
MKD float wave_sum(float v) { return wave_total(v); }
// Combine each lane's value with the one 16 or 32 lanes away (lane ^ 16,
// lane ^ 32) with the gfx950 lane swaps (v_permlane16_swap_b32: odd 16-lane
// rows against even rows; v_permlane32_swap_b32: upper half against lower
// half) instead of cross-lane LDS permutes.  The swap returns both partners
// in every lane, in the same order for the two lanes of a pair.
MKD float max_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
MKD float max_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
MKD float sum_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
MKD float sum_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// DPP move where lanes without a source (masked rows) keep their own value
template <int CTRL, int ROWMASK>
MKD float dpp_keep(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}
// wave-wide maximum with the same lane moves as wave_total
MKD float wave_max_all(float v) {
  v = fmaxf(v, dpp_keep<0xB1, 0xF>(v));
  v = fmaxf(v, dpp_keep<0x4E, 0xF>(v));
  v = fmaxf(v, dpp_keep<0x141, 0xF>(v));
  v = fmaxf(v, dpp_keep<0x140, 0xF>(v));
  v = fmaxf(v, dpp_keep<0x142, 0xA>(v));
  v = fmaxf(v, dpp_keep<0x143, 0xC>(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// 2^x on the transcendental unit (v_exp_f32)
MKD float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ----------------------------------------------------- bf16 MFMA 16x16x32
// Operand layout of v_mfma_f32_16x16x32_bf16 (64 lanes): lane i holds row
// (A) or column (B) i % 16 and the eight k values 8 (i / 16) .. + 7; the fp32
// result lane i holds column i % 16, rows 4 (i / 16) + j for j = 0..3.
typedef __bf16 mk_bf16x8 __attribute__((ext_vector_type(8)));
typedef float mk_f32x4v __attribute__((ext_vector_type(4)));

MKD mk_f32x4v mfma16x16x32(mk_bf16x8 a, mk_bf16x8 b, mk_f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
MKD mk_bf16x8 as_bf16x8(mk_u32x4 w) { return __builtin_bit_cast(mk_bf16x8, w); }
// Two fp32 values to a packed bf16 pair, round to nearest even
// (v_cvt_pk_bf16_f32); a in the low half.  Same bits as f2bf for every
// non-NaN input.
typedef __bf16 mk_bf16x2 __attribute__((ext_vector_type(2)));
MKD uint32_t pk_bf16(float a, float b) {
  const mk_bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// bf16 high and low parts of two fp32 values: hi = bf16(x), lo = bf16(x - hi)
MKD void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pk_bf16(a, b);
  lo = pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}
// bf16 high / low parts of 8 fp32 values, packed two per word
MKD void split_hi_lo(const float (&x)[8], mk_u32x4 &hi, mk_u32x4 &lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split2(x[2 * e], x[2 * e + 1], h[e], l[e]);
  hi = mk_u32x4{h[0], h[1], h[2], h[3]};
  lo = mk_u32x4{l[0], l[1], l[2], l[3]};
}

// Key/value rows are written to LDS with their 16-byte chunks permuted
// (chunk c of row t lands in chunk c ^ (t & 7) of that row): the score product reads the same
// chunk of 16 consecutive rows, which would otherwise hit the same LDS banks.
MKD int kv_swz(int t, int byte_in_row) { return (((byte_in_row >> 4) ^ (t & 7)) << 4) | (byte_in_row & 15); }

// sum over the workgroup; red: LDS scratch of MK_NWAVES floats
MKD float block_sum(float v, float *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < MK_NWAVES; ++w) t += red[w];
  __syncthreads();
  return t;
}

// element offset of cache row block [l][plane][b][g][0][0] in the
// [L][2][B_max][nkv][max_ctx][d] bf16 KV cache
template <class PT>
MKD size_t kv_off(const PT &P, int l, int plane, int b, int g) {
  return ((((size_t)l * 2 + plane) * P.B_max + b) * P.nkv + g) * (size_t)P.max_ctx * P.d;
}

// Merge the key-range partials of one attention output element: split s2
// stored (max, sum, unnormalised output) of head j at
// part[(s2 G + j)(d + 2)] (scores in base 2); returns output element i of
// head j.  Up to 8 splits' values are loaded at once (one memory round trip
// per 8 splits), the running sums rescaled to each group's new maximum.
MKD float merge_splits(const float *part, int NS, int G, int d, int j, int i) {
  float mx = -INFINITY, z = 0.f, o = 0.f;
  for (int s0 = 0; s0 < NS; s0 += 8) {
    float ms[8], ls[8], os[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (s0 + k < NS) {
        const float *pp = part + ((size_t)(s0 + k) * G + j) * (d + 2);
        ms[k] = ldc(pp);
        ls[k] = ldc(pp + 1);
        os[k] = ldc(pp + 2 + i);
      } else {
        ms[k] = -INFINITY;
        ls[k] = os[k] = 0.f;
      }
    float gm = mx;
#pragma unroll
    for (int k = 0; k < 8; ++k) gm = fmaxf(gm, ms[k]);
    if (gm == -INFINITY) continue;  // every split so far is empty
    const float c0 = mx == -INFINITY ? 0.f : exp2_fast(mx - gm);
    z *= c0;
    o *= c0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float c = ms[k] == -INFINITY ? 0.f : exp2_fast(ms[k] - gm);
      z = fmaf(ls[k], c, z);
      o = fmaf(os[k], c, o);
    }
    mx = gm;
  }
  return o / z;
}

// greedy order: larger value wins, equal values go to the smaller index
MKD bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// record the first device error and raise the abort flag every wait checks
template <class PT>
MKD void mk_raise(const PT &P, int code, int detail) {
  int32_t *err = P.err;
  int32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong((MK_G(int32_t) *)err, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT))
    stci(err + 1, detail);
  stci(err + 2, 1);
}
template <class PT>
MKD bool mk_aborted(const PT &P) { return __builtin_amdgcn_readfirstlane(ldci(P.err + 2)) != 0; }

// ----------------------------------------------- data-sentinel polling
//
// With MKSYNC_SENTINEL the homogeneous engine has no events between levels:
// an activation word starts each step as MK_SENTINEL and is written once by
// its producer, so a consumer's staging load is also its poll.  These
// loads repeat (per lane) until no word holds the sentinel, bounded by the
// watchdog; `ok` turns false on a timeout or abort (the error is raised).
MKD bool has_sent(const mk_u32x4 &v) {
  return v.x == MK_SENTINEL || v.y == MK_SENTINEL || v.z == MK_SENTINEL || v.w == MK_SENTINEL;
}
template <class PT>
MKD bool poll_fail(const PT &P, uint32_t &spins, uint64_t &t0, int detail) {
  if (spins == 0) t0 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_s_sleep(1);
  if ((++spins & 63u) == 0) {
    if (mk_aborted(P)) return true;
    if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)P.watchdog_ticks) {
      mk_raise(P, MK_E_TIMEOUT, detail);
      return true;
    }
  }
  return false;
}
// finish a 16-byte device-coherent load v (issued at byte offset off of r)
template <class PT>
MKD mk_u32x4 poll16(const PT &P, __amdgpu_buffer_rsrc_t r, int off, mk_u32x4 v, bool &ok) {
  uint32_t spins = 0;
  uint64_t t0 = 0;
  while (ok && has_sent(v)) {
    if (poll_fail(P, spins, t0, 0x30000)) {
      ok = false;
      break;
    }
    v = ldc16(r, off);
  }
  return v;
}
template <class PT>
MKD float ldcp(const PT &P, const float *p, bool sent, bool &ok) {
  float v = ldc(p);
  if (!sent) return v;
  uint32_t spins = 0;
  uint64_t t0 = 0;
  while (ok && __float_as_uint(v) == MK_SENTINEL) {
    if (poll_fail(P, spins, t0, 0x30001)) {
      ok = false;
      break;
    }
    v = ldc(p);
  }
  return v;
}

// This wave's XCD (hardware register XCC_ID, bits 3:0), as a counter row.
MKD uint32_t mk_xcc_row() {
  const uint32_t x = __builtin_amdgcn_s_getreg((20) | (3 << 11)) & 15u;
  return x < (uint32_t)MK_CTR_ROWS ? x : (uint32_t)MK_CTR_ROWS - 1u;
}
// Counter mode: count one trigger of event `ev` in this XCD's row.
MKD void ctr_bump(const MkProgram &P, int ev) { addcu(P.ctr + mk_xcc_row() * (uint32_t)P.ctr_stride + ev, 1u); }
// Counter mode: triggers of event `ev` so far, summed over the XCD rows (the
// eight loads are independent, so they share one round trip).
MKD uint32_t ctr_total(const MkProgram &P, int ev) {
  uint32_t v[MK_CTR_ROWS];
#pragma unroll
  for (int r = 0; r < MK_CTR_ROWS; ++r) v[r] = ldcu(P.ctr + r * P.ctr_stride + ev);
  uint32_t t = 0;
#pragma unroll
  for (int r = 0; r < MK_CTR_ROWS; ++r) t += v[r];
  return t;
}

// Wait for event `ev` of this step (global loads issued before the wait stay
// in flight: the workgroup barriers wait for LDS traffic only).  Counter
// mode: one lane polls the monotonic counters (summed over the XCD rows)
// until they reach (epoch+1) * triggers.  Flag mode: one wave polls all
// trigger flags of the event (each holds the epoch+1 of the last step its
// producer finished).  Bounded by the watchdog; returns false
// (uniformly) when the step is being aborted.
MKD bool mk_wait(const MkProgram &P, const MkStep &S, int ev, int *s_flag) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (P.sync_mode == 0) {
    if (threadIdx.x == 0) {
      const uint32_t need = (S.epoch + 1u) * (uint32_t)P.ev_count[ev];
      int ok = 1;
      if ((int32_t)(ctr_total(P, ev) - need) < 0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        uint32_t spins = 0;
        while ((int32_t)(ctr_total(P, ev) - need) < 0) {
          __builtin_amdgcn_s_sleep(1);
          if ((++spins & 31u) == 0) {
            if (mk_aborted(P)) { ok = 0; break; }
            if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)P.watchdog_ticks) {
              mk_raise(P, MK_E_TIMEOUT, ev);
              ok = 0;
              break;
            }
          }
        }
      }
      *s_flag = ok;
    }
  } else if (wave == 0) {
    const uint32_t want = S.epoch + 1u;
    const int n = P.ev_count[ev];
    const uint32_t *f = P.flags + P.ev_flag_base[ev];
    int ok = 1;
    uint64_t t0 = 0;
    uint32_t spins = 0;
    while (true) {
      bool mine = true;
      for (int k = lane; k < n; k += 64) mine = mine && ((int32_t)(ldcu(f + k) - want) >= 0);
      if (__all(mine)) break;
      if (spins == 0) t0 = __builtin_amdgcn_s_memrealtime();
      __builtin_amdgcn_s_sleep(1);
      if ((++spins & 31u) == 0) {
        if (mk_aborted(P)) { ok = 0; break; }
        if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)P.watchdog_ticks) {
          if (lane == 0) mk_raise(P, MK_E_TIMEOUT, ev);
          ok = 0;
          break;
        }
      }
    }
    if (lane == 0) *s_flag = ok;
  }
  lds_barrier();
  const int ok = *s_flag;
  lds_barrier();
  return ok != 0;
}

// Trigger event `ev`: every wave's stores complete, then one lane bumps the
// counter (counter mode) or stores epoch+1 into its own flag slot (flag mode).
MKD void mk_signal(const MkProgram &P, const MkStep &S, int ev, int slot) {
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (P.sync_mode == 0)
      ctr_bump(P, ev);
    else
      stcu(P.flags + P.ev_flag_base[ev] + slot, S.epoch + 1u);
  }
}
