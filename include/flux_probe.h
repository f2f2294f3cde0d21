/*
 * flux_probe.h -- attainable-peak probes of libflux.so (measurement helpers).
 *
 * The roofline figures of the attention kernels are quoted against the
 * published MI355X peaks and, beside them, against what these two probes
 * reach on the same GPU: a dense bf16 MFMA loop and a streaming HBM read.
 * They compute nothing of the attention path.  Same conventions as flux.h:
 * device pointers, asynchronous on `stream`, host validation, 0 = ok,
 * -1 = invalid argument (nothing launched), -4 = HIP launch error.
 */
#ifndef FLUX_PROBE_H
#define FLUX_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* n_workgroups workgroups of 4 waves; each wave issues 4 * iters
 * v_mfma_f32_32x32x16_bf16.  sink [device] float [n_workgroups] receives one
 * value per workgroup.  flux_probe_mfma_flops gives the flops of that launch. */
int32_t flux_probe_mfma(float* sink, int32_t n_workgroups, int32_t iters, void* stream);
double flux_probe_mfma_flops(int32_t n_workgroups, int32_t iters);

/* Reads `bytes` (a multiple of 16) at src [device] once with 16-byte
 * streaming (non-temporal) loads, the form the decode kernel reads its caches
 * with; sink [device] uint32 [n_workgroups] receives one word per workgroup. */
int32_t flux_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t n_workgroups,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLUX_PROBE_H */
