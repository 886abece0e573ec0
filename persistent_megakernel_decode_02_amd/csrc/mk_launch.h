// Host launchers of the device code (internal to libmk.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mk_program.h"

// static scratch (allocation-free contexts): the array's device address on
// device `dev` and a new generation number; whether `gen` is still current
#define MK_SCRATCH_BYTES (32u << 20)
int mk_scratch_acquire(int dev, void **ptr, uint64_t *gen);
bool mk_scratch_current(int dev, uint64_t gen);

int mk_prepare_launch(int exec_mode, int sync_mode, int lds);  // once per context: dynamic LDS limit
int mk_launch_stream(const MkProgram *d_prog, const MkStep &st, int n_cu, int lds, hipStream_t s);
int mk_occupancy(int exec_mode, int sync_mode, int lds, int *blocks_per_cu);  // persistent kernels of the exec modes
// homogeneous engine: d_prog is the first step's record, d_prog_other the
// other parity's (sentinel mode); st.n_steps > 1 selects the multi-step build
int mk_launch_mega(const MkProgram *d_prog, const MkProgram *d_prog_other, const MkStep &st, int n_cu, int lds,
                   bool sentinel, hipStream_t s);
int mk_launch_role_mega(const MkProgram *d_prog, const MkStep &st, int n_cu, int lds, hipStream_t s);
// homogeneous ops of one dependency level (S.level), one block per instruction;
// d_step: device step record or null (then st is used)
int mk_launch_flat_level(const MkProgram *d_prog, const MkStep *d_step, const MkStep &st, int n_blocks, int lds,
                         hipStream_t s);
int mk_launch_step_end(MkStep *d_step, hipStream_t s);
// work-queue engine: n_cu persistent workgroups take instructions from the global queue
int mk_launch_queue(const MkProgram *d_prog, const MkStep &st, int n_cu, int lds, hipStream_t s);  // d_step->epoch += 1 on the device
int mk_launch_role_level(const MkProgram *d_prog, const MkStep &st, int n_blocks, int lds, hipStream_t s);
int mk_occupancy_role(int lds, int *blocks_per_cu);
int mk_launch_fill(void *p, uint32_t v, size_t n_words, hipStream_t s);
// repack a row-major bf16 matrix [rows][K] into operand-order 1 KiB tiles
// (K a multiple of 32; dst holds ceil(rows / 16) * 16 * K elements)
int mk_launch_tile_rows(const uint16_t *src, int rows, int K, uint16_t *dst, hipStream_t s);
// two matrices [units][K] into tiles of 8 units, rows 0-7 from a, 8-15 from b
int mk_launch_tile_pairs(const uint16_t *a, const uint16_t *b, int units, int K, uint16_t *dst, hipStream_t s);
int mk_occupancy_mega(int lds, int *blocks_per_cu);

// measurement kernels (mk_measure.hip)
size_t mk_gridsync_scratch(int n_blocks);
int mk_launch_gridsync(int variant, int n_barriers, int n_blocks, void *d_scratch, int32_t *d_result, hipStream_t s);
int mk_launch_lds_stream(const void *d_buf, size_t bytes, uint32_t *d_out, int n_blocks, int nw, hipStream_t s);
int mk_launch_stream_read(const void *d_buf, size_t bytes, uint32_t *d_out, int n_blocks, hipStream_t s);
