/*
 * mla_peak.h -- measurement probe exported by libmla.so beside the MLA calls
 * of mla.h. It is not part of the attention path: it measures the dense bf16
 * MFMA rate and the shader clock the chip sustains under an all-MFMA load, so
 * that a kernel's roofline can be stated against that measured peak as well
 * as against the data-sheet peak.
 *
 * mla_peak_mfma_bf16 launches `blocks` workgroups of 8 waves on `stream`
 * (hipStream_t as void*). Each wave runs `iters` rounds of four independent
 * 32x32x16 bf16 MFMAs (4 * 32768 FLOP per round) from registers and writes
 * its elapsed shader cycles and 100 MHz reference ticks to
 * clocks[(block*8 + wave)*2 + {0, 1}] (device memory, blocks*16 entries).
 * sink: device float buffer of blocks*512 entries (results, to keep the work
 * live). The caller times the launch (e.g. with HIP events):
 *   FLOP = 2*32*32*16 * 4 * iters * 8 * blocks,
 *   clock = cycles / (ticks / 100 MHz).
 * Returns 0, -1 on a bad argument (nothing launched), -3 on a launch error.
 */
#ifndef MLA_PEAK_H_
#define MLA_PEAK_H_

#ifdef __cplusplus
extern "C" {
#endif

int mla_peak_mfma_bf16(int blocks, int iters, unsigned long long *clocks, float *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_PEAK_H_ */
