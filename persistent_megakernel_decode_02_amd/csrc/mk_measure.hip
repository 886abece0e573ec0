// Measurement kernels: grid-barrier microbenchmark and HBM streaming probe.
//
// The executive-summary page contrasts grid synchronisation with atomics
// against a NaN-sentinel scheme on MI300X (section "Trois familles", the
// monokernel row); the megakernel page lists the cooperative-groups grid
// barrier in its genealogy (section 2.3) and the counter protocol in
// section 2.6 item 3.  Each variant below performs n_barriers grid-wide
// barriers among persistent workgroups and checks, after every barrier, that
// data another workgroup wrote before the barrier is visible.
#include <hip/hip_cooperative_groups.h>
#include <hip/hip_runtime.h>

#include "mk_device.h"
#include "mk_launch.h"

namespace cg = cooperative_groups;

#define GS_BLOCK 256
#define GS_SENTINEL 0x7FBADBADu  // a quiet-NaN payload no arithmetic here produces
#define GS_TIMEOUT_TICKS 200000000ull  // 2 s of the 100 MHz real-time counter

struct GsScratch {
  uint32_t *ctr;     // [1]
  uint32_t *flags;   // [n]
  uint32_t *data;    // [n] value written before each barrier
  uint32_t *pay;     // [3][n] sentinel payloads (triple-buffered)
  uint32_t *abort;   // [1]
  uint32_t *xflag;   // [8] per-group flags of the two-level barrier (one 128-byte line each)
};

static __host__ __device__ size_t gs_align(size_t v) { return (v + 255) / 256 * 256; }

static __device__ GsScratch gs_layout(void *base, int n) {
  char *p = (char *)base;
  GsScratch s;
  s.ctr = (uint32_t *)p;
  p += 256;
  s.flags = (uint32_t *)p;
  p += gs_align(4 * (size_t)n);
  s.data = (uint32_t *)p;
  p += gs_align(4 * (size_t)n);
  s.pay = (uint32_t *)p;
  p += gs_align(12 * (size_t)n);
  s.abort = (uint32_t *)p;
  p += 256;
  s.xflag = (uint32_t *)p;
  return s;
}

size_t mk_gridsync_scratch(int n) {
  return 256 + 2 * gs_align(4 * (size_t)n) + gs_align(12 * (size_t)n) + 256 + 8 * 128;
}

// bounded spin bookkeeping: returns true when the barrier must give up
static __device__ __forceinline__ bool gs_expired(uint64_t t0, uint32_t *abort, int32_t *res) {
  if (ldcu(abort)) return true;
  if (__builtin_amdgcn_s_memrealtime() - t0 > GS_TIMEOUT_TICKS) {
    stcu(abort, 1u);
    atomicAdd(res + 1, 1);
    return true;
  }
  return false;
}

extern "C" __global__ void __launch_bounds__(GS_BLOCK) mk_gs_coop(int nb, void *scratch, int32_t *res) {
  GsScratch s = gs_layout(scratch, gridDim.x);
  cg::grid_group grid = cg::this_grid();
  const int blk = blockIdx.x, n = gridDim.x;
  int errs = 0;
  for (int k = 0; k < nb; ++k) {
    if (threadIdx.x == 0) s.data[blk] = (uint32_t)k + 1u;
    grid.sync();
    if (threadIdx.x == 0 && s.data[(blk + 1) % n] < (uint32_t)k + 1u) ++errs;
  }
  if (threadIdx.x == 0 && errs) atomicAdd(res, errs);
}

// variant 1: agent-scope release add / acquire poll (cache writeback + invalidate)
extern "C" __global__ void __launch_bounds__(GS_BLOCK) mk_gs_relacq(int nb, void *scratch, int32_t *res) {
  GsScratch s = gs_layout(scratch, gridDim.x);
  const int blk = blockIdx.x, n = gridDim.x;
  __shared__ int ok;
  int errs = 0;
  for (int k = 0; k < nb; ++k) {
    if (threadIdx.x == 0) {
      s.data[blk] = (uint32_t)k + 1u;
      __hip_atomic_fetch_add(s.ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t need = (uint32_t)(k + 1) * (uint32_t)n;
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int good = 1;
      uint32_t spins = 0;
      while ((int32_t)(__hip_atomic_load(s.ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) - need) < 0) {
        __builtin_amdgcn_s_sleep(1);
        if ((++spins & 15u) == 0 && gs_expired(t0, s.abort, res)) { good = 0; break; }
      }
      if (good && s.data[(blk + 1) % n] < (uint32_t)k + 1u) ++errs;
      ok = good;
    }
    __syncthreads();
    if (!ok) break;
  }
  if (threadIdx.x == 0 && errs) atomicAdd(res, errs);
}

// variant 2: write-through data, relaxed counter, no cache maintenance
extern "C" __global__ void __launch_bounds__(GS_BLOCK) mk_gs_counter(int nb, void *scratch, int32_t *res) {
  GsScratch s = gs_layout(scratch, gridDim.x);
  const int blk = blockIdx.x, n = gridDim.x;
  __shared__ int ok;
  int errs = 0;
  for (int k = 0; k < nb; ++k) {
    if (threadIdx.x == 0) {
      stcu(s.data + blk, (uint32_t)k + 1u);
      wait_vm();
      addcu(s.ctr, 1u);
      const uint32_t need = (uint32_t)(k + 1) * (uint32_t)n;
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int good = 1;
      uint32_t spins = 0;
      while ((int32_t)(ldcu(s.ctr) - need) < 0) {
        __builtin_amdgcn_s_sleep(1);
        if ((++spins & 15u) == 0 && gs_expired(t0, s.abort, res)) { good = 0; break; }
      }
      if (good && ldcu(s.data + (blk + 1) % n) < (uint32_t)k + 1u) ++errs;
      ok = good;
    }
    __syncthreads();
    if (!ok) break;
  }
  if (threadIdx.x == 0 && errs) atomicAdd(res, errs);
}

// variant 3: one epoch flag per block, wave 0 polls all flags with vector loads
extern "C" __global__ void __launch_bounds__(GS_BLOCK) mk_gs_flags(int nb, void *scratch, int32_t *res) {
  GsScratch s = gs_layout(scratch, gridDim.x);
  const int blk = blockIdx.x, n = gridDim.x, lane = threadIdx.x & 63;
  __shared__ int ok;
  int errs = 0;
  for (int k = 0; k < nb; ++k) {
    const uint32_t want = (uint32_t)k + 1u;
    if (threadIdx.x < 64) {
      if (lane == 0) {
        stcu(s.data + blk, want);
        wait_vm();
        stcu(s.flags + blk, want);
      }
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int good = 1;
      uint32_t spins = 0;
      while (true) {
        bool mine = true;
        for (int j = lane; j < n; j += 64) mine = mine && ((int32_t)(ldcu(s.flags + j) - want) >= 0);
        if (__all(mine)) break;
        __builtin_amdgcn_s_sleep(1);
        if ((++spins & 15u) == 0 && gs_expired(t0, s.abort, res)) { good = 0; break; }
      }
      if (lane == 0) {
        if (good && ldcu(s.data + (blk + 1) % n) < want) ++errs;
        ok = good;
      }
    }
    __syncthreads();
    if (!ok) break;
  }
  if (threadIdx.x == 0 && errs) atomicAdd(res, errs);
}

// variant 4: the payload is the signal.  Round k uses payload buffer k % 3;
// a block polls until no word of the round's buffer holds the sentinel, then
// resets its own word of the buffer round k + 2 will use (everyone has left
// the round that last used it).  The barrier checks the payload values too.
extern "C" __global__ void __launch_bounds__(GS_BLOCK) mk_gs_sentinel(int nb, void *scratch, int32_t *res) {
  GsScratch s = gs_layout(scratch, gridDim.x);
  const int blk = blockIdx.x, n = gridDim.x, lane = threadIdx.x & 63;
  __shared__ int ok;
  int errs = 0;
  for (int k = 0; k < nb; ++k) {
    uint32_t *buf = s.pay + (size_t)(k % 3) * n;
    const uint32_t val = __float_as_uint((float)(k + 1));
    if (threadIdx.x < 64) {
      if (lane == 0) stcu(buf + blk, val);
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int good = 1;
      uint32_t spins = 0;
      int bad = 0;
      while (true) {
        bool mine = true;
        for (int j = lane; j < n; j += 64) mine = mine && (ldcu(buf + j) != GS_SENTINEL);
        if (__all(mine)) break;
        __builtin_amdgcn_s_sleep(1);
        if ((++spins & 15u) == 0 && gs_expired(t0, s.abort, res)) { good = 0; break; }
      }
      if (good)
        for (int j = lane; j < n; j += 64) bad += (ldcu(buf + j) != val);
      for (int o = 32; o >= 1; o >>= 1) bad += __shfl_xor(bad, o, 64);
      if (lane == 0) {
        errs += bad;
        stcu(s.pay + (size_t)((k + 2) % 3) * n + blk, GS_SENTINEL);
        wait_vm();  // the reset lands before this block's next payload write
        ok = good;
      }
    }
    __syncthreads();
    if (!ok) break;
  }
  if (threadIdx.x == 0 && errs) atomicAdd(res, errs);
}

// variant 5: two levels.  Workgroups are dispatched to the 8 XCDs in turn,
// so group g = {blocks b : b % 8 == g} shares one XCD (up to a rotation of
// the XCDs that depends on earlier launches).  Every block stores
// its epoch flag; the group's leader (block g) polls all n flags, then
// stores the group flag (its own 128-byte line), which the other members
// poll.  Only eight blocks read the all-producer lines, and each group line
// has n / 8 readers, so the memory side serves far fewer requests per line
// than when every block polls every flag (variant 3).  Every access is
// device scope: a group flag stored without write-through was not seen by
// the members' L1-bypassing loads, so correctness does not depend on the
// grouping.  Blocks whose XCD (hardware register XCC_ID) differs from b % 8
// are counted in res[2] (information only).
MKD uint32_t gs_xcc_id() { return __builtin_amdgcn_s_getreg((20) | (3 << 11)) & 15u; }

extern "C" __global__ void __launch_bounds__(GS_BLOCK) mk_gs_xcd(int nb, void *scratch, int32_t *res) {
  GsScratch s = gs_layout(scratch, gridDim.x);
  const int blk = blockIdx.x, n = gridDim.x, lane = threadIdx.x & 63;
  const int grp = blk & 7;
  const bool leader = blk < 8;
  __shared__ int ok;
  int errs = 0;
  if (threadIdx.x == 0 && (int)gs_xcc_id() != grp) atomicAdd(res + 2, 1);
  for (int k = 0; k < nb; ++k) {
    const uint32_t want = (uint32_t)k + 1u;
    if (threadIdx.x < 64) {
      if (lane == 0) {
        stcu(s.data + blk, want);
        wait_vm();
        stcu(s.flags + blk, want);
      }
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int good = 1;
      uint32_t spins = 0;
      if (leader) {
        while (true) {
          bool mine = true;
          for (int j = lane; j < n; j += 64) mine = mine && ((int32_t)(ldcu(s.flags + j) - want) >= 0);
          if (__all(mine)) break;
          __builtin_amdgcn_s_sleep(1);
          if ((++spins & 15u) == 0 && gs_expired(t0, s.abort, res)) { good = 0; break; }
        }
        if (lane == 0) stcu(s.xflag + grp * 32, want);
      } else {
        while (true) {
          if ((int32_t)(ldcu(s.xflag + grp * 32) - want) >= 0) break;
          __builtin_amdgcn_s_sleep(1);
          if ((++spins & 15u) == 0 && gs_expired(t0, s.abort, res)) { good = 0; break; }
        }
      }
      if (lane == 0) {
        if (good && ldcu(s.data + (blk + 1) % n) < want) ++errs;
        ok = good;
      }
    }
    __syncthreads();
    if (!ok) break;
  }
  if (threadIdx.x == 0 && errs) atomicAdd(res, errs);
}

extern "C" __global__ void mk_gs_init(void *scratch, int n) {
  GsScratch s = gs_layout(scratch, n);
  const int m = 3 * n > 8 * 32 ? 3 * n : 8 * 32;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < m; i += gridDim.x * blockDim.x) {
    if (i < 3 * n) s.pay[i] = GS_SENTINEL;
    if (i < n) {
      s.flags[i] = 0;
      s.data[i] = 0;
    }
    if (i == 0) {
      *s.ctr = 0;
      *s.abort = 0;
    }
    if (i < 8 * 32) s.xflag[i] = 0;
  }
}

int mk_launch_gridsync(int variant, int n_barriers, int n_blocks, void *d_scratch, int32_t *d_result, hipStream_t st) {
  hipLaunchKernelGGL(mk_gs_init, dim3(16), dim3(256), 0, st, d_scratch, n_blocks);
  if (hipGetLastError() != hipSuccess) return -1;
  switch (variant) {
    case 0: {
      void *args[] = {&n_barriers, &d_scratch, &d_result};
      if (hipLaunchCooperativeKernel((const void *)mk_gs_coop, dim3(n_blocks), dim3(GS_BLOCK), args, 0, st) != hipSuccess)
        return -1;
      break;
    }
    case 1: hipLaunchKernelGGL(mk_gs_relacq, dim3(n_blocks), dim3(GS_BLOCK), 0, st, n_barriers, d_scratch, d_result); break;
    case 2: hipLaunchKernelGGL(mk_gs_counter, dim3(n_blocks), dim3(GS_BLOCK), 0, st, n_barriers, d_scratch, d_result); break;
    case 3: hipLaunchKernelGGL(mk_gs_flags, dim3(n_blocks), dim3(GS_BLOCK), 0, st, n_barriers, d_scratch, d_result); break;
    case 4: hipLaunchKernelGGL(mk_gs_sentinel, dim3(n_blocks), dim3(GS_BLOCK), 0, st, n_barriers, d_scratch, d_result); break;
    case 5:
      if (n_blocks < 8) return -2;
      hipLaunchKernelGGL(mk_gs_xcd, dim3(n_blocks), dim3(GS_BLOCK), 0, st, n_barriers, d_scratch, d_result);
      break;
    default: return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------ HBM probe
#define SR_BLOCK 512
#define SR_UNROLL 8
extern "C" __global__ void __launch_bounds__(SR_BLOCK) mk_stream_read_kernel(const mk_u32x4 *buf, size_t n16, uint32_t *out) {
  // each block reads a contiguous span; within it, a block-wide stride so one
  // load instruction of a wave covers 1 KiB contiguous
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + (SR_UNROLL - 1) * SR_BLOCK < hi; i += SR_UNROLL * SR_BLOCK) {
    mk_u32x4 v[SR_UNROLL];
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) v[u] = __builtin_nontemporal_load(buf + i + (size_t)u * SR_BLOCK);
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += SR_BLOCK) {
    mk_u32x4 v = __builtin_nontemporal_load(buf + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  __shared__ uint32_t red[SR_BLOCK / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < SR_BLOCK / 64; ++w) t ^= red[w];
    out[blockIdx.x] = t;
  }
}

// Streaming through LDS with direct global->LDS loads: `nw` waves of each
// block issue 16-byte-per-lane loads into a 64 KiB LDS ring (1 KiB per
// instruction), keeping up to 60 loads in flight per wave, the way the
// megakernel's loader waves feed their page ring.
typedef __attribute__((address_space(3))) void mk_lds_v;
extern "C" __global__ void __launch_bounds__(SR_BLOCK) mk_lds_stream_kernel(const char *buf, size_t nbytes, uint32_t *out, int nw) {
  extern __shared__ __attribute__((aligned(16))) char ring[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t n1k = nbytes / 1024;
  const size_t per = (n1k + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n1k ? lo + per : n1k;
  if (wave < nw) {
    uint32_t issued = 0;
    for (size_t i = lo + wave; i < hi; i += nw) {
      __builtin_amdgcn_global_load_lds((const void *)(buf + i * 1024 + lane * 16),
                                       (mk_lds_v *)(ring + ((i * 1024) & 65535)), 16, 0, 0);
      if ((++issued & 3u) == 0) asm volatile("s_waitcnt vmcnt(60)" ::: "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = *(const uint32_t *)(ring + (blockIdx.x * 64) % 65536);
}

int mk_launch_lds_stream(const void *d_buf, size_t bytes, uint32_t *d_out, int n_blocks, int nw, hipStream_t st) {
  if (hipFuncSetAttribute((const void *)mk_lds_stream_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 65536) !=
      hipSuccess)
    return -1;
  hipLaunchKernelGGL(mk_lds_stream_kernel, dim3(n_blocks), dim3(SR_BLOCK), 65536, st, (const char *)d_buf, bytes, d_out, nw);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int mk_launch_stream_read(const void *d_buf, size_t bytes, uint32_t *d_out, int n_blocks, hipStream_t st) {
  hipLaunchKernelGGL(mk_stream_read_kernel, dim3(n_blocks), dim3(SR_BLOCK), 0, st, (const mk_u32x4 *)d_buf, bytes / 16, d_out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
