/*
 * mla_ceiling.h -- C ABI of libmla_ceiling.so: measurement kernels that give the decode
 * benchmark its on-box ceilings (the roofline fractions are quoted against both the
 * published MI355X peaks and these measured rates).  Not part of the decode path.
 * All pointers are device pointers owned by the caller; launches are asynchronous on
 * `stream` (a hipStream_t, NULL = default); return 0 on success, -1 for an invalid
 * argument (nothing enqueued), -4 if the launch failed.
 */
#ifndef MLA_CEILING_H
#define MLA_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_CEILING_MFMA_BF16 0 /* v_mfma_f32_32x32x16_bf16 */
#define MLA_CEILING_MFMA_FP8 1  /* v_mfma_f32_32x32x64_f8f6f4, E4M3 operands */
#define MLA_CEILING_MFMA_F16 2  /* v_mfma_f32_32x32x16_f16 */

/* Stream read: `blocks` workgroups of 256 threads read the `bytes` of `buf` (16-byte
 * aligned, bytes a multiple of 16) once, in 16-byte coalesced loads, grid-strided;
 * out[blocks * 256] uint32 receives each thread's XOR of the 32-bit words it read (so
 * the XOR over out equals the XOR over buf). */
int mla_ceiling_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, void* stream);

/* MFMA loop: `blocks` workgroups of 4 wavefronts; each wavefront runs `iters` rounds of
 * four independent MFMA chains of the given kind and writes one float to
 * out[blocks * 4].  Flops per launch: blocks * 4 * iters * 4 * mla_ceiling_mfma_flops. */
int mla_ceiling_mfma(int kind, int iters, float* out, int blocks, void* stream);

/* Flops of one MFMA of the given kind (0 for an unknown kind). */
double mla_ceiling_mfma_flops(int kind);

#ifdef __cplusplus
}
#endif

#endif /* MLA_CEILING_H */
