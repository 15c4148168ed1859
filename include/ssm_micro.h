/*
 * ssm_micro.h -- ceiling probes for the selective-scan roofline (gfx950).
 *
 * A separate shared library, libssm_micro.so, next to libssm_scan.so.  It
 * holds no part of the selective scan: it measures what the chip sustains, so
 * that the scan's kernels can be reported as a fraction of it.
 *
 *   ssm_micro_valu    rate of fp32 fused multiply-adds, of the hardware
 *                     exponential (v_exp_f32, the transcendental the scan uses
 *                     once per state and step) and of their mix (one
 *                     exponential per four multiply-adds, the proportion of
 *                     the scan's per-state update), with 1 or 8 independent
 *                     chains per lane;
 *   ssm_micro_stream  HBM streaming bandwidth with 16-byte non-temporal
 *                     accesses: read, write, copy and in-place
 *                     read-modify-write (the access pattern of the decode
 *                     step's state update).
 *
 * Conventions: pointers are DEVICE pointers owned by the caller.  Each call
 * launches one untimed warm-up and then `reps` timed launches on `stream` (a
 * hipStream_t; NULL means the null stream) between two HIP events, waits for
 * the second event and stores the average milliseconds per launch in
 * *ms_out.  Calls are therefore synchronous with respect to the host.
 * Errors are reported only through the return value.
 */
#ifndef SSM_MICRO_H
#define SSM_MICRO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSM_MICRO_OK = 0,
  SSM_MICRO_EINVAL = -1,   /* bad argument: null pointer, size or selector */
  SSM_MICRO_ERUNTIME = -2  /* a HIP launch or event call failed */
} ssm_micro_status;

/*
 * fp32 ALU rate probe.
 *   kind   : 0 = v = v*a + b (FMA); 1 = v = exp2(-v) (v_exp_f32);
 *            2 = one exp2 and four FMAs per element-step
 *   chains : 1 or 8 independent chains per lane
 *   blocks : workgroups of 256 threads (4 waves); blocks = CUs * k puts about
 *            k waves on every SIMD
 *   iters  : loop trips; each runs 16 element-steps per chain
 *   seed   : 10 float32 values: a, b, then 8 chain starts, a and b in
 *            (0, 1) and the starts in [0.5, 1] keep every value in [0.5, 1]
 *   sink   : 256 float32 (written only if the chains reach an impossible
 *            value; it keeps the arithmetic live)
 * Element-steps per launch: blocks * 256 * iters * 16 * chains.
 */
int ssm_micro_valu(int kind, int chains, int blocks, int iters, const float* seed,
                   float* sink, int reps, float* ms_out, void* stream);

/*
 * HBM streaming probe over `bytes` (a multiple of 16; both buffers 16-byte
 * aligned and at least slices * bytes long).  Launch i (the warm-up is launch
 * 0) works on slice i mod `slices` of the buffers, so a working set smaller
 * than the Infinity Cache can still be streamed from HBM (slices * bytes
 * well above 256 MB).
 *   mode   : 0 read src; 1 write dst; 2 copy src -> dst; 3 dst += 1 per
 *            32-bit word, in place (src unused, may be NULL for 1 and 3)
 *   unroll : 1, 2, 4 or 8 vectors in flight per thread
 *   blocks : workgroups of 256 threads, grid-stride over the buffer
 *   sink   : 4 bytes (written only by the read probe on an impossible value)
 * HBM bytes per launch: bytes (read, write) or 2 * bytes (copy, update).
 */
int ssm_micro_stream(int mode, int unroll, int blocks, const void* src, void* dst,
                     int64_t bytes, int slices, void* sink, int reps, float* ms_out,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_MICRO_H */
