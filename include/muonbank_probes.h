/*
 * muonbank_probes.h -- measurement probes exported by libmuonbank.so.
 *
 * Not part of the Muon step: two kernels that measure, on the device at hand, the rates the step's
 * kernels are judged against (the matrix-core rate for the Newton-Schulz contractions, the HBM rate for
 * the streaming kernels), so that a benchmark can report its fractions of the measured peaks beside
 * the nominal ones.  Both only enqueue on `stream` (a hipStream_t as void*, NULL = the null stream);
 * the caller times them with events.  Status codes are those of muonbank.h.
 */
#ifndef MUONBANK_PROBES_H
#define MUONBANK_PROBES_H

#include <stdint.h>

#include "muonbank.h"

#ifdef __cplusplus
extern "C" {
#endif

/* `workgroups` workgroups of four wavefronts; each wavefront runs `iters` times four independent
 * v_mfma_f32_32x32x16_bf16 (32768 flops each) on register operands and writes one float per lane to
 * sink[workgroups * 256] (device, 16-byte aligned) so the work is kept.  Flops per launch:
 * workgroups * 4 * iters * 4 * 32768.  MB_ERR_NULL, MB_ERR_SHAPE (iters < 1, workgroups outside
 * 1..65535), MB_ERR_ALIGN, MB_ERR_HIP. */
mb_status mb_probe_mfma_bf16(int64_t iters, int32_t workgroups, float *sink, void *stream);

/* dst[0, bytes) = src[0, bytes) with 16-byte non-temporal loads and stores, four per thread, all loads first (device
 * buffers, 16-byte aligned, not overlapping; bytes a positive multiple of 16): 2 * bytes of HBM traffic
 * per launch once the buffers exceed the caches.  MB_ERR_NULL, MB_ERR_SHAPE, MB_ERR_ALIGN, MB_ERR_ALIAS, MB_ERR_HIP. */
mb_status mb_probe_copy(void *dst, const void *src, int64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MUONBANK_PROBES_H */
