/*
 * far_ceiling.h -- measurement aids for the fused epilogue's benchmark
 * (libfar_ceiling.so; not part of the epilogue's ABI in far.h).
 *
 * The fused "sum of partials + residual add + RMSNorm (+ fp8)" epilogue moves a fixed
 * number of bytes per call: it reads P partial rows and the residual row and writes the
 * new residual plus either the normalised row (same size) or its fp8 codes (half the
 * size, plus four bytes of scale per row). The kernels here move exactly those bytes
 * with no arithmetic (each output pack is the XOR of the input packs, so no load can be
 * dropped), giving the benchmark a ceiling for the fused kernel on this GPU:
 *
 *   far_ceiling_rows   the fused kernel's launch shape (a team of waves per row, packs
 *                      per lane, rows per workgroup, grid-stride over rows), so the
 *                      difference to the fused kernel is the cost of its arithmetic and
 *                      its row reductions;
 *   far_ceiling_flat   the same bytes as flat arrays, any grid (a plain stream);
 *   far_ceiling_empty  an empty kernel: the launch floor;
 *   far_ceiling_sleep  one wave that sleeps a bounded time, so a host can queue timed
 *                      work behind it and the timed launches run back to back;
 *   far_ceiling_stamp  one lane that stores the GPU's constant-rate real-time counter
 *                      (100 MHz) into a device array: placed between the timed launches
 *                      of one captured graph, it marks chunk boundaries inside the graph.
 *
 * Every buffer is device memory owned by the caller; nothing is allocated or kept.
 * Calls are asynchronous on `stream`. Arguments are checked before anything is
 * launched: the functions return 0 on success, 1 for invalid arguments (nothing
 * launched), 2 if the HIP runtime refused the launch.
 */
#ifndef FAR_CEILING_H_
#define FAR_CEILING_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *far_ceiling_stream_t;

#define FAR_CEILING_MAX_INPUTS 9

/*
 * Row-shaped stream. inputs: host array of n_inputs (1..FAR_CEILING_MAX_INPUTS) device
 * pointers, each [rows, row_bytes]. out_full: [rows, row_bytes]. out2: [rows, row_bytes]
 * (out2_half == 0) or [rows, row_bytes / 2] (out2_half != 0), or NULL. out_row: [rows]
 * floats (one per row, written by the row's first lane) or NULL. row_bytes: a multiple
 * of 16, below 2^31. Lane l of a row's team of waves_per_row waves takes the 16-byte
 * packs l, l + 64 * waves_per_row, ... (packs_per_lane of them, n_inputs *
 * packs_per_lane <= 24); rows_per_block teams per workgroup (<= 1024 lanes);
 * grid_blocks workgroups (1..2^20), each looping over rows.
 */
int far_ceiling_rows(const void *const *inputs, int n_inputs, void *out_full, void *out2,
                     int out2_half, float *out_row, int64_t rows, int64_t row_bytes,
                     int waves_per_row, int packs_per_lane, int rows_per_block,
                     int64_t grid_blocks, far_ceiling_stream_t stream);

/*
 * Flat stream of the same traffic: inputs as n_inputs arrays of `bytes` bytes (a
 * multiple of 16, below 2^32); out_full `bytes`; out2 `bytes` or `bytes / 2` (or NULL).
 * Each lane moves `unroll` packs per trip (n_inputs * unroll <= 24), grid-stride over
 * the arrays; block_threads a multiple of 64 up to 1024; grid_blocks 1..2^20.
 */
int far_ceiling_flat(const void *const *inputs, int n_inputs, void *out_full, void *out2,
                     int out2_half, int64_t bytes, int unroll, int block_threads,
                     int64_t grid_blocks, far_ceiling_stream_t stream);

/* Empty kernel over grid_blocks (1..2^20) workgroups of block_threads (64..1024). */
int far_ceiling_empty(int64_t grid_blocks, int block_threads, far_ceiling_stream_t stream);

/* One wave that sleeps `iterations` times (0..100000) for the longest s_sleep interval
 * (about 8,000 clock cycles each), then ends. */
int far_ceiling_sleep(int iterations, far_ceiling_stream_t stream);

/* One lane stores the real-time counter (ticks of 10 ns) into out[index] (a device
 * array of uint64 owned by the caller; index >= 0). */
int far_ceiling_stamp(uint64_t *out, int index, far_ceiling_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FAR_CEILING_H_ */
