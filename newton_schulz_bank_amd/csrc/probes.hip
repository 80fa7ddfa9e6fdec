// Measurement probes for the roofline denominators on gfx950 (not part of the step):
//   * a loop of bf16 MFMAs (v_mfma_f32_32x32x16_bf16) in independent chains, no memory traffic: the
//     matrix cores' sustained rate, beside the nominal 256 CU x 2.4 GHz x 4096 flop/clk;
//   * a streaming device copy in 16-byte vectors: the HBM bandwidth a kernel with this access pattern
//     reaches, beside the nominal 8 TB/s.
// The caller times the launches with events on its stream.

#include "common.hpp"
#include "muonbank.h"
#include "muonbank_probes.h"

namespace mb {

namespace {

constexpr int kProbeChains = 4;     // independent accumulators per wavefront

__global__ void __launch_bounds__(256) mfma_probe_kernel(int64_t iters, float* __restrict__ sink) {
    // operands from the thread index, so that nothing folds at compile time
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)((float)((threadIdx.x + e) & 15) * 0.0625f);
        b[e] = (__bf16)((float)((threadIdx.x * 3 + e) & 15) * 0.0625f);
    }
    f32x16 acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

constexpr int kCopyVecs = 4;        // 16-byte vectors per thread, all loaded before the first store

__global__ void __launch_bounds__(256) copy_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * 256 * kCopyVecs + threadIdx.x;
    u32x4 v[kCopyVecs];
#pragma unroll
    for (int j = 0; j < kCopyVecs; ++j) {
        const int64_t i = base + (int64_t)j * 256;
        if (i < n16) v[j] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int j = 0; j < kCopyVecs; ++j) {
        const int64_t i = base + (int64_t)j * 256;
        if (i < n16) __builtin_nontemporal_store(v[j], dst + i);
    }
}

}  // namespace

}  // namespace mb

extern "C" {

mb_status mb_probe_mfma_bf16(int64_t iters, int32_t workgroups, float* sink, void* stream) {
    if (!sink) return MB_ERR_NULL;
    if (iters < 1 || workgroups < 1 || workgroups > 65535) return MB_ERR_SHAPE;
    if ((uintptr_t)sink & 15u) return MB_ERR_ALIGN;
    mb::mfma_probe_kernel<<<dim3((unsigned)workgroups), 256, 0, (hipStream_t)stream>>>(iters, sink);
    return hipGetLastError() == hipSuccess ? MB_OK : MB_ERR_HIP;
}

mb_status mb_probe_copy(void* dst, const void* src, int64_t bytes, void* stream) {
    if (!dst || !src) return MB_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0) return MB_ERR_SHAPE;
    if (((uintptr_t)dst | (uintptr_t)src) & 15u) return MB_ERR_ALIGN;
    const uintptr_t d = (uintptr_t)dst, s = (uintptr_t)src;
    if (d < s + (uintptr_t)bytes && s < d + (uintptr_t)bytes) return MB_ERR_ALIAS;
    const int64_t n16 = bytes / 16;
    // one workgroup per 256 * kCopyVecs vectors: many short workgroups keep the memory system busy
    const int64_t grid = (n16 + 256 * mb::kCopyVecs - 1) / (256 * mb::kCopyVecs);
    if (grid > 0x7FFFFFFF) return MB_ERR_SHAPE;
    mb::copy_probe_kernel<<<dim3((unsigned)grid), 256, 0, (hipStream_t)stream>>>((const mb::u32x4*)src,
                                                                                  (mb::u32x4*)dst, n16);
    return hipGetLastError() == hipSuccess ? MB_OK : MB_ERR_HIP;
}

}  // extern "C"
