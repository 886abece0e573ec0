// The persistent decode megakernel, the multi-launch build of the same ops,
// and their host-side launchers.
//
// Megakernel (megakernel page, section 2.1: one launch, persistent blocks,
// dependencies in global memory, internal dispatch; section 2.6 items 1-3
// and 5): one workgroup per CU walks its static instruction list; before an
// instruction it waits for the instruction's input event, dispatches on the
// (workgroup-uniform) opcode, and triggers the output event when done.
// The multi-launch build runs the role-specialised ops one kernel per
// dependency level instead, so kernel boundaries replace the events (the
// contrast the executive-summary page draws between a sequence of kernels and
// one persistent launch).
#include <hip/hip_runtime.h>

#include <mutex>

#include "mk_launch.h"
#include "mk_ops_batched.h"
#include "mk_roles_ops.h"
#include "mk_stream.h"

// Role-specialised persistent kernel: one workgroup per CU runs the CU's
// instruction list with loader / sync-storer / compute waves.
// The step record is the kernel's second argument; role functions read it in
// place in the kernarg segment, after the 8-byte program pointer.
static_assert(alignof(MkStep) == 8, "kernarg layout: MkStep follows the program pointer at offset 8");
MKD const MkStep *kernarg_step() {
  return (const MkStep *)((const __attribute__((address_space(4))) char *)__builtin_amdgcn_kernarg_segment_ptr() + 8);
}

extern "C" __global__ void __launch_bounds__(MK_BLOCK) mk_role_mega_kernel(const MkProgram *__restrict__ Pp, MkStep S) {
  const MkProgram &P = *Pp;
  if (mk_aborted(P)) return;
  const int cu = blockIdx.x;
  const int i0 = P.cu_begin[cu], i1 = P.cu_begin[cu + 1];
  (void)S;
  role_run(Pp, kernarg_step(), i0, i1 - i0);
}

// The same role-specialised ops, one launch per dependency level: block i
// runs instruction i of the level.
extern "C" __global__ void __launch_bounds__(MK_BLOCK) mk_role_level_kernel(const MkProgram *__restrict__ Pp, MkStep S) {
  const MkProgram &P = *Pp;
  if (mk_aborted(P)) return;
  const int idx = P.level_list[P.level_begin[S.level] + blockIdx.x];
  role_run(Pp, kernarg_step(), idx, 1);
}

// per-instruction trace record: start, end of the wait, end, cu | epoch
__device__ __forceinline__ void trace_record(uint64_t *trace, int i, uint64_t tw, uint64_t ts, uint64_t te, int cu,
                                             uint32_t epoch) {
  uint64_t *r = trace + (size_t)i * 8;
  r[0] = tw;
  r[1] = ts;
  r[2] = te;
  r[3] = ((uint64_t)cu << 32) | epoch;
  r[4] = r[5] = r[6] = r[7] = 0;
}

// Homogeneous engine, one step: every workgroup walks its CU's instruction
// list.  SENT: data-sentinel synchronisation (the ops poll their inputs; no
// events), a build of its own so the event build keeps its register
// allocation.  STEPS: one of several steps of a launch.  False when the
// step is being aborted.
template <bool SENT, bool STEPS>
MKD bool mega_step(const MkProgram &P, const MkStep &S, float *smem, int *s_flag) {
  if (mk_aborted(P)) return false;
  const int cu = blockIdx.x;
  if constexpr (SENT) {
    // this CU's share of the other parity's activations (read by the next
    // step, written by no one in this one) goes back to the sentinel
    const size_t n = (size_t)P.par_stride, per = (n + P.n_cu - 1) / P.n_cu;
    const size_t lo = (size_t)cu * per, hi = min(lo + per, n);
    uint32_t *o = reinterpret_cast<uint32_t *>(P.act_other);
    for (size_t i = lo + threadIdx.x; i < hi; i += MK_BLOCK) stcu(o + i, MK_SENTINEL);
    // within a launch the next step's producers write this copy once this
    // step's tokens are out: the resets must have landed before any of this
    // CU's outputs can let the step complete
    if constexpr (STEPS) wait_vm();
  }
  const int i0 = cld(&P.cu_begin[cu]), i1 = cld(&P.cu_begin[cu + 1]);  // scalar: the list walk stays uniform
  uint64_t *const trace = P.trace;
  for (int i = i0; i < i1; ++i) {
    const MkInstr in = cld(&P.instr[i]);  // scalar loads: every field stays wave-uniform
    const uint64_t tw = trace ? __builtin_amdgcn_s_memrealtime() : 0;
    uint64_t ts = 0;
    if (S.batch < MK_MFMA_MIN_BATCH && in.op == MKOP_OPROJ && i + 1 < i1) {
      const MkInstr nx = cld(&P.instr[i + 1]);
      if (nx.op == MKOP_GATEUP && nx.layer == in.layer) {  // O and gate/up as one unit
        uint64_t te_o = 0, ts_g = 0;
        const int st = run_o_gateup<SENT>(P, S, in, nx, smem, s_flag, trace != nullptr, ts, te_o, ts_g);
        if (st == MK_ST_ABORT) return false;
        if (!SENT && st == MK_ST_SIGNAL && nx.sig_ev >= 0) mk_signal(P, S, nx.sig_ev, nx.sig_slot);
        __syncthreads();
        if (trace && threadIdx.x == 0) {
          trace_record(trace, i, tw, ts, te_o, cu, S.epoch);
          trace_record(trace, i + 1, te_o, ts_g, __builtin_amdgcn_s_memrealtime(), cu, S.epoch);
        }
        ++i;
        continue;
      }
    }
    const int st = run_instr<SENT>(P, S, in, smem, s_flag, trace != nullptr, ts);
    if (st == MK_ST_ABORT) return false;
    if (!SENT && st == MK_ST_SIGNAL && in.sig_ev >= 0) mk_signal(P, S, in.sig_ev, in.sig_slot);
    __syncthreads();
    if (trace && threadIdx.x == 0) trace_record(trace, i, tw, ts, __builtin_amdgcn_s_memrealtime(), cu, S.epoch);
  }
  return true;
}

// Wait until the step with this epoch may start: the previous step's last
// LM-head arriver has published its tokens (lm_done >= epoch).  Bounded by
// the watchdog; false (uniformly) on a timeout or abort.
MKD bool wait_prev_step(const MkProgram &P, uint32_t epoch, int *s_flag) {
  if (threadIdx.x == 0) {
    int ok = 1;
    uint64_t t0 = 0;
    uint32_t spins = 0;
    while ((int32_t)(ldcu(P.lm_done) - epoch) < 0) {
      if (spins == 0) t0 = __builtin_amdgcn_s_memrealtime();
      __builtin_amdgcn_s_sleep(1);
      if ((++spins & 31u) == 0) {
        if (mk_aborted(P)) { ok = 0; break; }
        if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)P.watchdog_ticks) {
          mk_raise(P, MK_E_TIMEOUT, 0x40000);
          ok = 0;
          break;
        }
      }
    }
    *s_flag = ok;
  }
  __syncthreads();
  const int ok = *s_flag;
  __syncthreads();
  return ok != 0;
}

// One launch runs S.n_steps greedy steps (STEPS) or one.  Step t has epoch
// S.epoch + t, writes its logits at logits + t * batch * V and its tokens at
// next + t * batch, and feeds its token back on the device for step t + 1,
// which starts once that token is published.  In sentinel mode consecutive
// steps alternate between the two activation copies: Pa is the record of the
// first step's parity, Pb the other's.
template <bool SENT, bool STEPS>
MKD void mega_body(const MkProgram *Pa, const MkProgram *Pb, const MkStep &S, float *smem, int *s_flag) {
  if constexpr (!STEPS) {
    mega_step<SENT, false>(*Pa, S, smem, s_flag);
  } else {
    const int n = S.n_steps;
    for (int t = 0; t < n; ++t) {
      const MkProgram &P = (SENT && (t & 1)) ? *Pb : *Pa;
      MkStep St = S;
      St.epoch = S.epoch + (uint32_t)t;
      St.logits = S.logits + (size_t)t * S.batch * P.V;
      St.next = S.next ? S.next + (size_t)t * S.batch : nullptr;
      St.flags = S.flags | 1u;  // MK_ADVANCE
      if (t > 0 && !wait_prev_step(P, St.epoch, s_flag)) return;
      if (!mega_step<SENT, true>(P, St, smem, s_flag)) return;
    }
  }
}

#define MK_MEGA_KERNEL(name, sent, steps)                                                                     \
  extern "C" __global__ void __launch_bounds__(MK_BLOCK)                                                      \
      name(const MkProgram *__restrict__ Pa, const MkProgram *__restrict__ Pb, MkStep S) {                   \
    extern __shared__ __attribute__((aligned(16))) float smem[];                                              \
    __shared__ int s_flag;                                                                                    \
    mega_body<sent, steps>(Pa, Pb, S, smem, &s_flag);                                                         \
  }
MK_MEGA_KERNEL(mk_mega_kernel, false, false)
MK_MEGA_KERNEL(mk_mega_sent_kernel, true, false)
MK_MEGA_KERNEL(mk_mega_steps_kernel, false, true)
MK_MEGA_KERNEL(mk_mega_sent_steps_kernel, true, true)

// The homogeneous engine's ops, one launch per dependency level: block i
// runs instruction i of level S.level, with no waits and no signals (the
// kernel boundaries order the levels).  Sd, when set, is the step record in
// device memory (graph replays, where the record cannot change per launch).
extern "C" __global__ void __launch_bounds__(MK_BLOCK) mk_flat_level_kernel(const MkProgram *__restrict__ Pp,
                                                                           const MkStep *__restrict__ Sd, MkStep S0) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int s_flag;
  const MkProgram &P = *Pp;
  if (mk_aborted(P)) return;
  const MkStep S = Sd ? cld(Sd) : S0;
  const int idx = cld(&P.level_list[cld(&P.level_begin[S0.level]) + blockIdx.x]);
  const MkInstr in = cld(&P.instr[idx]);
  uint64_t ts = 0;
  run_instr<false, true>(P, S, in, smem, &s_flag, false, ts);
}

// end of a captured step: the device copy of the step record moves to the
// next epoch (one thread, a plain vector store)
extern "C" __global__ void mk_step_end_kernel(MkStep *Sd) {
  if (threadIdx.x == 0 && blockIdx.x == 0) Sd->epoch = Sd->epoch + 1u;
}

// Work-queue engine: the homogeneous ops, but no per-CU lists.  Every
// workgroup takes the next ticket of a global counter (an atomic add) and
// runs the instruction at that position of the breadth-first queue, waiting
// for its event as usual.  The queue puts every instruction after the
// triggers of the event it waits for, and each workgroup finishes the
// instruction it holds before taking another, so the lowest unfinished
// ticket can always run: the grid drains.  The next ticket is requested
// while the current instruction runs.  Each workgroup takes exactly one
// ticket past the end, so a step consumes n_instr + n_cu tickets and step e
// starts at e (n_instr + n_cu) (modulo 2^32).
MKD uint32_t queue_take(const MkProgram &P, int *s_flag) {
  if (threadIdx.x == 0) *s_flag = (int)addcu(P.queue_ctr, 1u);
  __syncthreads();
  const uint32_t t = (uint32_t)__builtin_amdgcn_readfirstlane(*s_flag);  // uniform: scalar queue loads
  __syncthreads();
  return t;
}

extern "C" __global__ void __launch_bounds__(MK_BLOCK) mk_queue_kernel(const MkProgram *__restrict__ Pp, MkStep S) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int s_flag, s_next;
  const MkProgram &P = *Pp;
  if (mk_aborted(P)) return;
  const uint32_t n = (uint32_t)P.n_instr, base = S.epoch * (n + (uint32_t)P.n_cu);
  uint64_t *const trace = P.trace;
  uint32_t t = queue_take(P, &s_flag) - base;
  while (t < n) {
    uint32_t next = 0;  // requested now, consumed (and waited for) once the instruction is done
    if (threadIdx.x == 0) next = addcu(P.queue_ctr, 1u);
    const int i = cld(&P.queue[t]);
    const MkInstr in = cld(&P.instr[i]);
    const uint64_t tw = trace ? __builtin_amdgcn_s_memrealtime() : 0;
    uint64_t ts = 0;
    const int st = run_instr<false>(P, S, in, smem, &s_flag, trace != nullptr, ts);
    if (st == MK_ST_ABORT) return;
    if (st == MK_ST_SIGNAL && in.sig_ev >= 0) mk_signal(P, S, in.sig_ev, in.sig_slot);
    __syncthreads();
    if (trace && threadIdx.x == 0) trace_record(trace, i, tw, ts, __builtin_amdgcn_s_memrealtime(), blockIdx.x, S.epoch);
    if (threadIdx.x == 0) s_next = (int)next;
    __syncthreads();
    t = (uint32_t)__builtin_amdgcn_readfirstlane(s_next) - base;
    __syncthreads();
  }
}

// Stream engine (one sequence per step): waves 0..MK_NSW-1 stream projection
// weights through register rings, wave MK_NSW synchronises; the waves meet
// only at attention instructions, which all of them run together.
extern "C" __global__ void __launch_bounds__(MK_BLOCK) mk_stream_kernel(const MkProgram *__restrict__ Pp, MkStep S) {
  __shared__ int s_flag;
  const MkProgram &P = *Pp;
  if (mk_aborted(P)) return;
  const int cu = blockIdx.x;
  const int i0 = cld(&P.cu_begin[cu]), i1 = cld(&P.cu_begin[cu + 1]);
  const int wave = __builtin_amdgcn_readfirstlane(mk_tid() >> 6);
  {
    lds_u32 *ctl = (lds_u32 *)((lds_char *)mk_flat_lds + P.st_ctl);
    if (mk_tid() < ST_CTL_WORDS) ctl[mk_tid()] = 0u;
  }
  __syncthreads();
  uint64_t *const trace = P.trace;
  int i = i0;
  while (i < i1) {
    const MkInstr in = cld(&P.instr[i]);
    if (in.op == MKOP_ATTN) {
      // joint instruction: every wave arrives with nothing of its own in flight
      __syncthreads();
      const uint64_t tw = trace ? __builtin_amdgcn_s_memrealtime() : 0;
      uint64_t ts = 0;
      auto wait = [&]() -> bool {
        const bool ok = in.wait_ev < 0 || mk_wait(P, S, in.wait_ev, &s_flag);
        if (trace) ts = __builtin_amdgcn_s_memrealtime();
        return ok;
      };
      const int st = op_attn_mfma(P, S, in, &s_flag, wait);
      if (st == MK_ST_ABORT) return;
      if (st == MK_ST_SIGNAL && in.sig_ev >= 0) mk_signal(P, S, in.sig_ev, in.sig_slot);
      __syncthreads();
      if (trace && mk_tid() == 0) trace_record(trace, i, tw, ts, __builtin_amdgcn_s_memrealtime(), cu, S.epoch);
      ++i;
      continue;
    }
    int j = i + 1;  // this segment: projections up to the next attention instruction
    while (j < i1 && cld(&P.instr[j].op) != MKOP_ATTN) ++j;
    const bool ok = wave < MK_NSW ? st_streamer<MK_RING>(P, i, j, wave) : st_sync(P, S, i, j);
    if (!ok) return;
    i = j;
  }
}

// ------------------------------------------------------ static scratch
//
// Workspace of contexts created by mk_ctx_create_scratch: a file-scope device
// array, so those contexts allocate no device memory.  In host code the
// array's name is only a stand-in; its device address is looked up once per
// device (with that device current) and kept.  Every scratch context on a
// device shares the one array: creating a context re-initialises it, which
// ends the previous scratch context on that device (its generation is no
// longer current, and mk_decode_step refuses it).
static __device__ __align__(256) char scratch[MK_SCRATCH_BYTES];

#define MK_SCRATCH_DEVICES 64
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[MK_SCRATCH_DEVICES];
static uint64_t g_scratch_gen[MK_SCRATCH_DEVICES];

int mk_scratch_acquire(int dev, void **ptr, uint64_t *gen) {
  if (dev < 0 || dev >= MK_SCRATCH_DEVICES) return -1;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -1;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *gen = ++g_scratch_gen[dev];
  return 0;
}

bool mk_scratch_current(int dev, uint64_t gen) {
  if (dev < 0 || dev >= MK_SCRATCH_DEVICES) return false;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_gen[dev] == gen;
}

extern "C" __global__ void mk_fill_kernel(uint32_t *p, uint32_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// Repack a row-major bf16 matrix [rows][K] (K a multiple of 32) into 1 KiB
// operand-order tiles: tile (T, j) holds rows 16 T .. + 15 and columns
// 32 j .. + 31, its 16-byte piece L being row 16 T + L % 16, columns
// 32 j + 8 (L / 16) .. + 7; rows past the end are zero.  One thread per
// piece.
extern "C" __global__ void mk_tile_rows_kernel(const uint16_t *src, int rows, int K, uint16_t *dst, size_t n_pieces) {
  const int J = K >> 5;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_pieces; i += (size_t)gridDim.x * blockDim.x) {
    const int L = (int)(i & 63);
    const size_t tj = i >> 6, T = tj / J, j = tj - T * J;
    const size_t row = 16 * T + (L & 15), c = 32 * j + 8 * (L >> 4);
    mk_u32x4 v = {0u, 0u, 0u, 0u};
    if (row < (size_t)rows) v = *(const mk_u32x4 *)(src + row * K + c);
    *(mk_u32x4 *)(dst + 8 * i) = v;
  }
}

// Persistent kernels and the dynamic-LDS limit of each, as last set in this
// process.  Launches compare against it and call hipFuncSetAttribute only
// when it differs (a context binds it once; a later occupancy query may have
// changed it).
static const void *const g_kernels[] = {(const void *)mk_mega_kernel,           (const void *)mk_role_mega_kernel,
                                        (const void *)mk_role_level_kernel,     (const void *)mk_stream_kernel,
                                        (const void *)mk_mega_sent_kernel,      (const void *)mk_mega_steps_kernel,
                                        (const void *)mk_mega_sent_steps_kernel, (const void *)mk_flat_level_kernel,
                                        (const void *)mk_queue_kernel};
static constexpr int MK_NKERNELS = (int)(sizeof g_kernels / sizeof g_kernels[0]);
static int g_lds_set[MK_NKERNELS] = {-1, -1, -1, -1, -1, -1, -1, -1, -1};
static int lds_slot(const void *fn) {
  for (int i = 0; i < MK_NKERNELS; ++i)
    if (g_kernels[i] == fn) return i;
  return 0;
}
static hipError_t set_lds(const void *fn, int lds) {
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  g_lds_set[lds_slot(fn)] = e == hipSuccess ? lds : -1;
  return e;
}
static inline bool ensure_lds(const void *fn, int lds) {
  return g_lds_set[lds_slot(fn)] == lds || set_lds(fn, lds) == hipSuccess;
}
static const void *mega_fn(bool sentinel, bool steps) {
  return steps ? (sentinel ? (const void *)mk_mega_sent_steps_kernel : (const void *)mk_mega_steps_kernel)
               : (sentinel ? (const void *)mk_mega_sent_kernel : (const void *)mk_mega_kernel);
}

// The dynamic-LDS limit of a kernel is set once, when a context is bound
// (mk_prepare_launch), not on every step: the step path is only the launch.
static const void *exec_kernel(int exec_mode, int sync_mode) {
  if (exec_mode == MKEXEC_FLAT) return mega_fn(sync_mode == MKSYNC_SENTINEL, false);
  if (exec_mode == MKEXEC_FLAT_MULTI) return (const void *)mk_flat_level_kernel;
  if (exec_mode == MKEXEC_QUEUE) return (const void *)mk_queue_kernel;
  return exec_mode == MKEXEC_MEGA     ? (const void *)mk_role_mega_kernel
         : exec_mode == MKEXEC_STREAM ? (const void *)mk_stream_kernel
                                      : (const void *)mk_role_level_kernel;
}

int mk_prepare_launch(int exec_mode, int sync_mode, int lds) {
  if (set_lds(exec_kernel(exec_mode, sync_mode), lds) != hipSuccess) return -1;
  if (exec_mode == MKEXEC_FLAT && set_lds(mega_fn(sync_mode == MKSYNC_SENTINEL, true), lds) != hipSuccess) return -1;
  return 0;
}

int mk_launch_stream(const MkProgram *d_prog, const MkStep &st, int n_cu, int lds, hipStream_t s) {
  if (!ensure_lds((const void *)mk_stream_kernel, lds)) return -1;
  hipLaunchKernelGGL(mk_stream_kernel, dim3(n_cu), dim3(MK_BLOCK), lds, s, d_prog, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int mk_occupancy(int exec_mode, int sync_mode, int lds, int *blocks_per_cu) {
  const void *fn = exec_kernel(exec_mode, sync_mode);
  if (set_lds(fn, lds) != hipSuccess) return -1;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, MK_BLOCK, lds) != hipSuccess) return -1;
  *blocks_per_cu = nb;
  return 0;
}

int mk_launch_mega(const MkProgram *d_prog, const MkProgram *d_prog_other, const MkStep &st, int n_cu, int lds,
                   bool sentinel, hipStream_t s) {
  const bool steps = st.n_steps > 1;
  const void *fn = mega_fn(sentinel, steps);
  if (!ensure_lds(fn, lds)) return -1;
  void *args[] = {(void *)&d_prog, (void *)&d_prog_other, (void *)&st};
  if (hipLaunchKernel(fn, dim3(n_cu), dim3(MK_BLOCK), args, (size_t)lds, s) != hipSuccess) return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int mk_launch_role_mega(const MkProgram *d_prog, const MkStep &st, int n_cu, int lds, hipStream_t s) {
  if (!ensure_lds((const void *)mk_role_mega_kernel, lds)) return -1;
  hipLaunchKernelGGL(mk_role_mega_kernel, dim3(n_cu), dim3(MK_BLOCK), lds, s, d_prog, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int mk_launch_flat_level(const MkProgram *d_prog, const MkStep *d_step, const MkStep &st, int n_blocks, int lds,
                         hipStream_t s) {
  if (n_blocks <= 0) return 0;
  if (!ensure_lds((const void *)mk_flat_level_kernel, lds)) return -1;
  hipLaunchKernelGGL(mk_flat_level_kernel, dim3(n_blocks), dim3(MK_BLOCK), lds, s, d_prog, d_step, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int mk_launch_queue(const MkProgram *d_prog, const MkStep &st, int n_cu, int lds, hipStream_t s) {
  if (!ensure_lds((const void *)mk_queue_kernel, lds)) return -1;
  hipLaunchKernelGGL(mk_queue_kernel, dim3(n_cu), dim3(MK_BLOCK), lds, s, d_prog, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int mk_launch_step_end(MkStep *d_step, hipStream_t s) {
  hipLaunchKernelGGL(mk_step_end_kernel, dim3(1), dim3(64), 0, s, d_step);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int mk_launch_role_level(const MkProgram *d_prog, const MkStep &st, int n_blocks, int lds, hipStream_t s) {
  if (n_blocks <= 0) return 0;
  if (!ensure_lds((const void *)mk_role_level_kernel, lds)) return -1;
  hipLaunchKernelGGL(mk_role_level_kernel, dim3(n_blocks), dim3(MK_BLOCK), lds, s, d_prog, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int mk_occupancy_role(int lds, int *blocks_per_cu) {
  if (set_lds((const void *)mk_role_mega_kernel, lds) != hipSuccess) return -1;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void *)mk_role_mega_kernel, MK_BLOCK, lds) != hipSuccess)
    return -1;
  *blocks_per_cu = nb;
  return 0;
}

// The same tiles for a pair of matrices [units][K] read together: tile T
// holds units 8 T .. + 7, rows 0-7 from `a`, rows 8-15 from `b` (units a
// multiple of 8).
extern "C" __global__ void mk_tile_pairs_kernel(const uint16_t *a, const uint16_t *b, int K, uint16_t *dst,
                                                size_t n_pieces) {
  const int J = K >> 5;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_pieces; i += (size_t)gridDim.x * blockDim.x) {
    const int L = (int)(i & 63), r = L & 15;
    const size_t tj = i >> 6, T = tj / J, j = tj - T * J;
    const size_t unit = 8 * T + (r & 7), c = 32 * j + 8 * (L >> 4);
    *(mk_u32x4 *)(dst + 8 * i) = *(const mk_u32x4 *)((r < 8 ? a : b) + unit * K + c);
  }
}

int mk_launch_tile_pairs(const uint16_t *a, const uint16_t *b, int units, int K, uint16_t *dst, hipStream_t s) {
  if (units <= 0 || (units & 7) != 0 || K <= 0 || (K & 31) != 0) return -1;
  const size_t n_pieces = (size_t)(units / 8) * (size_t)(K >> 5) * 64;
  size_t blocks = (n_pieces + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(mk_tile_pairs_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, b, K, dst, n_pieces);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int mk_launch_tile_rows(const uint16_t *src, int rows, int K, uint16_t *dst, hipStream_t s) {
  if (rows <= 0 || K <= 0 || (K & 31) != 0) return -1;
  const size_t n_pieces = (size_t)(rows + 15) / 16 * (size_t)(K >> 5) * 64;
  size_t blocks = (n_pieces + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(mk_tile_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, rows, K, dst, n_pieces);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int mk_launch_fill(void *p, uint32_t v, size_t n_words, hipStream_t s) {
  if (n_words == 0) return 0;
  size_t blocks = (n_words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(mk_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t *)p, v, n_words);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int mk_occupancy_mega(int lds, int *blocks_per_cu) {
  if (set_lds((const void *)mk_mega_kernel, lds) != hipSuccess) return -1;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void *)mk_mega_kernel, MK_BLOCK, lds) != hipSuccess)
    return -1;
  *blocks_per_cu = nb;
  return 0;
}
