/*
 * twomamba_ceilings.h -- measurement aids exported by libtwomamba.so beside the
 * operator's ABI (twomamba.h): two microbenchmark kernels that give the
 * benchmark a measured HBM and MFMA ceiling on the box it runs on.  They are
 * not part of the 2Mamba operator.  Return values are twomamba_status codes;
 * arguments are checked before any HIP call; work is enqueued on `stream`
 * (a hipStream_t as void*, NULL = default stream).
 */
#ifndef TWOMAMBA_CEILINGS_H
#define TWOMAMBA_CEILINGS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming copy of `bytes` bytes from src to dst (device memory, caller-owned,
   16-byte aligned, bytes a multiple of 16, no overlap: TWOMAMBA_ERR_UNSUPPORTED /
   TWOMAMBA_ERR_ALIAS otherwise).  HBM traffic is 2 x bytes. */
int twomamba_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream);

/* `workgroups` workgroups of four waves, each wave issuing iters x 16
   v_mfma_f32_16x16x32_f16 (16384 FLOP each) on register operands, in 16
   independent accumulation chains; one float per
   thread is written to sink[workgroups * 256] (device, caller-owned).  clocks
   (device, [workgroups][2], or NULL) receives per workgroup the shader-clock
   cycles (s_memtime) and the 100 MHz real-time ticks (s_memrealtime) of its
   first wave's loop: their ratio x 100 MHz is the clock the loop ran at. */
int twomamba_ceiling_mfma(int workgroups, int iters, float* sink, unsigned long long* clocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TWOMAMBA_CEILINGS_H */
