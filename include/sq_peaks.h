/*
 * Measured peaks of the GPU the library runs on (libsq_peaks.so): what the
 * matrix cores and HBM deliver to simple kernels on this device, next to
 * which the library's own kernels are judged.  Not part of the quantization
 * API; the benchmark reports these figures beside the published peaks.
 *
 * Every call launches one kernel on `stream` (a hipStream_t, NULL = the
 * default stream) and returns 0, or the HIP error code of the launch.  The
 * caller times the launch (HIP events) and reads the clock samples after the
 * stream has completed.
 *
 * clk (device memory, 4 x uint64, may be NULL): the shader-clock counter
 * and the constant-rate real-time counter, read by the first wave of block 0
 * at its start and its end: {clock_start, clock_end, rt_start, rt_end}.
 * The clock counter advances once per shader-clock cycle, so the ratio of
 * the two spans times the real-time rate (sqp_clock_rates) is the shader
 * clock sustained while that wave ran.
 */
#ifndef SQ_PEAKS_H
#define SQ_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Matrix-core issue rate: `blocks` blocks of 4 waves; each wave runs `iters`
 * iterations of 4 independent accumulator chains of
 *   fp8 == 0: v_mfma_i32_32x32x32_i8          (65536 ops per instruction)
 *   fp8 != 0: v_mfma_scale_f32_32x32x64_f8f6f4 (131072 flops, e4m3 operands)
 * with no memory traffic in the loop, on operands of mixed bit patterns of
 * both signs (finite e4m3 codes).  Ops per launch:
 *   blocks * 4 * iters * 4 * (fp8 ? 131072 : 65536).
 * sink: device int, written only if the accumulators reach an impossible
 * value (keeps the loop from being removed).  iters >= 1, blocks >= 1.
 */
int sqp_mfma_loop(int fp8, int iters, int blocks, int *sink, uint64_t *clk, void *stream);

/*
 * HBM read rate: `blocks` blocks of 256 threads read x[0, bytes) once in
 * 16-byte nontemporal loads (grid-stride) and fold it into one word each;
 * sink (device, `blocks` x uint32) receives the folds.  bytes % 16 == 0.
 */
int sqp_read_stream(const void *x, size_t bytes, int blocks, uint32_t *sink, uint64_t *clk,
                    void *stream);

/*
 * A 2:1 read:write stream, the mix of the quantizers (fp16 in, int8 out):
 * every 16 bytes read from x produce 8 bytes written to y (y holds
 * bytes / 2).  Nontemporal loads; stores nontemporal when nt_store != 0.
 * bytes % 16 == 0.
 */
int sqp_rw_stream(const void *x, size_t bytes, void *y, int blocks, int nt_store, uint64_t *clk,
                  void *stream);

/*
 * Host query of the current device: wall_khz = the real-time counter's
 * constant rate, peak_sclk_khz = the published peak shader clock, both in
 * kHz (hipDeviceAttributeWallClockRate, hipDeviceAttributeClockRate).  The
 * sustained clock of a probe is then
 *   (clock_end - clock_start) / (rt_end - rt_start) * wall_khz.
 * Either pointer may be NULL.  Returns 0 or the HIP error code.
 */
int sqp_clock_rates(int *wall_khz, int *peak_sclk_khz);

#ifdef __cplusplus
}
#endif

#endif
