// Bandwidth-bound kernels of the Muon bank step on gfx950:
//   * momentum + Nesterov update, with per-slot partial sums of u^2 for the
//     Frobenius pre-scale;
//   * partial sums of x^2 for a stand-alone Newton-Schulz call;
//   * the per-slot scale s = 1 / (||u||_F + eps) and live flag;
//   * the mixed-precision apply on bf16 weight + uint16 low mantissa.
// Momentum, scale and apply each take up to kMaxStreamBanks banks in one
// launch: the launch's workgroups are numbered bank after bank, and each
// workgroup finds its bank, slot and chunk from that numbering.  Per-slot
// scalars (mu, nu, decay, eta) come from the bank's own values or, if given,
// from one float32 device table with a row per slot of the call (every bank's
// step scalars in one buffer that a graph replay reads, as the "Unified
// zero-copy optimizer and transposed LM head" page, section 4, keeps them).
//
// Momentum follows the two lerps of "Muon Custom Sizing", section 4
// (buf' = mu*buf + (1-mu)*g, then u = (1-mu)*g + mu*buf'); the apply follows
// the Record 7 walkthrough, section 4.1 (recombine, decay, add, split).
//
// Compiled with -ffp-contract=off: every rounding below is the one written.

#include "common.hpp"
#include "kernels.hpp"

namespace mb {

namespace {

// One bank of a multi-bank launch, as the kernels see it (momentum uses grad..partials, the apply
// w_hi..lr_mul_per_slot); its workgroups are [first_block, first_block + batch * nchunks).
struct StreamBank {
    const void* grad;
    void* buf;
    uint16_t* u;
    double* partials;
    uint16_t* w_hi;
    uint16_t* w_lo;
    const uint16_t* v;
    const float* lr_mul_per_slot;
    int64_t slot_numel;
    int64_t first_block;
    int nchunks, batch, slot_base;
    int f32, vec;
    float mu, nu, decay, eta;
};

struct StreamArgs {
    StreamBank bank[kMaxStreamBanks];
    int nbanks;
    const f32x4* slot_scalars;      // NULL, or (mu, nu, decay, eta) per slot of the call
};

struct ScaleArgs {
    ScaleBank bank[kMaxStreamBanks];
    int nbanks;
    double eps;
};

}  // namespace

// ---------------------------------------------------------------------------
// momentum + Nesterov
// ---------------------------------------------------------------------------

// Exact products in binary64 (<=24-bit x <=24-bit significands), then the
// correctly rounded exact sum in the storage format: for float32 through a
// round-to-odd binary64 sum, for bf16 with sum_to_bf16.  buf' and u are the
// correctly rounded exact values.
__device__ __forceinline__ void momentum_elem(float g, float b, float mu, float nu, float& buf_new_f32,
                                              uint16_t& buf_new_bf16, uint16_t& u_bits, bool f32_storage,
                                              float& u_val) {
    double p_buf = (double)mu * (double)b;
    double p_g = (double)nu * (double)g;
    float stored;
    if (f32_storage) {
        buf_new_f32 = odd53_to_f32(sum_round_odd(p_buf, p_g));
        stored = buf_new_f32;
    } else {
        buf_new_bf16 = sum_to_bf16(p_buf, p_g);
        stored = bf16_to_f32(buf_new_bf16);
    }
    u_bits = sum_to_bf16(p_g, (double)mu * (double)stored);
    u_val = bf16_to_f32(u_bits);
}

// Sum of squares of bf16 values in binary64: each square is exact (<= 16 significant bits) and no square
// of a nonzero bf16 value underflows (the smallest is 2^-266) or overflows, so a slot's sum is zero exactly
// when every element is zero.
__device__ __forceinline__ double add_sq(double acc, float v) {
    const double d = (double)v;
    return __fma_rn(d, d, acc);
}

// Fixed-order workgroup sum of 256 threads (wavefront trees, then the four wavefront sums in a fixed
// order); the result is valid in thread 0.
__device__ __forceinline__ double block_sum256(double v, double* red) {
    v = wave_sum_f64(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// 16-byte load / store, non-temporal when NT (streams larger than the last-level cache: nothing to keep).
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}
template <bool NT>
__device__ __forceinline__ void st16(u32x4* p, u32x4 v) {
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// One chunk of one slot: buf' and u of its elements, and their sum of u^2 (returned in every thread).
template <bool F32, bool VEC, bool NT>
__device__ __forceinline__ double momentum_chunk(const void* __restrict__ grad_, void* __restrict__ buf_,
                                                 uint16_t* __restrict__ u, int64_t slot, int64_t chunk,
                                                 int64_t slot_numel, float mu, float nu, double* red) {
    const int64_t base = slot * slot_numel;
    const int64_t lo = chunk * kStreamChunk;
    const int64_t hi = min(lo + kStreamChunk, slot_numel);
    double acc = 0.0;
    if (VEC && !F32 && NT) {
        // a stream larger than the last-level cache: both 8-element groups of this thread (a chunk is
        // kStreamGroups groups of 256 x 8 elements) loaded before the first store, the loads and the store
        // of buf' (which the step does not read again) non-temporal; u, which the Newton-Schulz launch
        // reads next, stored normally.  slot_numel % 8 == 0 and bases are 16-byte aligned.
        u32x4 gv[kStreamGroups], bv[kStreamGroups];
#pragma unroll
        for (int k = 0; k < kStreamGroups; ++k) {
            const int64_t e = lo + (int64_t)threadIdx.x * 8 + (int64_t)k * 256 * 8;
            if (e < hi) {
                gv[k] = ld16<NT>(reinterpret_cast<const u32x4*>((const uint16_t*)grad_ + base + e));
                bv[k] = ld16<NT>(reinterpret_cast<const u32x4*>((const uint16_t*)buf_ + base + e));
            }
        }
#pragma unroll
        for (int k = 0; k < kStreamGroups; ++k) {
            const int64_t e = lo + (int64_t)threadIdx.x * 8 + (int64_t)k * 256 * 8;
            if (e >= hi) continue;
            u32x4 bo, uo;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float bn32[2], uv[2];
                uint16_t bn16[2], ub[2];
                momentum_elem(__uint_as_float(gv[k][q] << 16), __uint_as_float(bv[k][q] << 16), mu, nu, bn32[0],
                              bn16[0], ub[0], false, uv[0]);
                momentum_elem(__uint_as_float(gv[k][q] & 0xFFFF0000u), __uint_as_float(bv[k][q] & 0xFFFF0000u), mu, nu,
                              bn32[1], bn16[1], ub[1], false, uv[1]);
                acc = add_sq(acc, uv[0]);
                acc = add_sq(acc, uv[1]);
                bo[q] = (uint32_t)bn16[0] | ((uint32_t)bn16[1] << 16);
                uo[q] = (uint32_t)ub[0] | ((uint32_t)ub[1] << 16);
            }
            st16<NT>(reinterpret_cast<u32x4*>((uint16_t*)buf_ + base + e), bo);
            *reinterpret_cast<u32x4*>(u + base + e) = uo;
        }
    } else if (VEC) {
        // 8 consecutive elements per thread per step; slot_numel % 8 == 0 and bases are 16-byte aligned
        for (int64_t e = lo + (int64_t)threadIdx.x * 8; e < hi; e += 256 * 8) {
            const int64_t idx = base + e;
            float g[8], b[8];
            if (F32) {
                const float4* gp = reinterpret_cast<const float4*>((const float*)grad_ + idx);
                const float4* bp = reinterpret_cast<const float4*>((const float*)buf_ + idx);
                float4 g0 = gp[0], g1 = gp[1], b0 = bp[0], b1 = bp[1];
                g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w; g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
                b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w; b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
            } else {
                u32x4 gv = *reinterpret_cast<const u32x4*>((const uint16_t*)grad_ + idx);
                u32x4 bv = *reinterpret_cast<const u32x4*>((const uint16_t*)buf_ + idx);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    g[2 * q] = __uint_as_float(gv[q] << 16);
                    g[2 * q + 1] = __uint_as_float(gv[q] & 0xFFFF0000u);
                    b[2 * q] = __uint_as_float(bv[q] << 16);
                    b[2 * q + 1] = __uint_as_float(bv[q] & 0xFFFF0000u);
                }
            }
            float bn32[8];
            uint16_t bn16[8], ub[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                float uv;
                momentum_elem(g[q], b[q], mu, nu, bn32[q], bn16[q], ub[q], F32, uv);
                acc = add_sq(acc, uv);
            }
            if (F32) {
                float4* bp = reinterpret_cast<float4*>((float*)buf_ + idx);
                bp[0] = make_float4(bn32[0], bn32[1], bn32[2], bn32[3]);
                bp[1] = make_float4(bn32[4], bn32[5], bn32[6], bn32[7]);
            } else {
                u32x4 bo;
#pragma unroll
                for (int q = 0; q < 4; ++q) bo[q] = (uint32_t)bn16[2 * q] | ((uint32_t)bn16[2 * q + 1] << 16);
                *reinterpret_cast<u32x4*>((uint16_t*)buf_ + idx) = bo;
            }
            u32x4 uo;
#pragma unroll
            for (int q = 0; q < 4; ++q) uo[q] = (uint32_t)ub[2 * q] | ((uint32_t)ub[2 * q + 1] << 16);
            *reinterpret_cast<u32x4*>(u + idx) = uo;
        }
    } else {
        for (int64_t e = lo + threadIdx.x; e < hi; e += 256) {
            const int64_t idx = base + e;
            float g, b;
            if (F32) {
                g = ((const float*)grad_)[idx];
                b = ((const float*)buf_)[idx];
            } else {
                g = bf16_to_f32(((const uint16_t*)grad_)[idx]);
                b = bf16_to_f32(((const uint16_t*)buf_)[idx]);
            }
            float bn32, uv;
            uint16_t bn16, ub;
            momentum_elem(g, b, mu, nu, bn32, bn16, ub, F32, uv);
            acc = add_sq(acc, uv);
            if (F32) ((float*)buf_)[idx] = bn32;
            else ((uint16_t*)buf_)[idx] = bn16;
            u[idx] = ub;
        }
    }
    return block_sum256(acc, red);
}

// The bank of workgroup `blk` in a multi-bank launch (banks in increasing first_block; wave-uniform).
__device__ __forceinline__ int find_bank(const StreamArgs& p, int64_t blk) {
    int b = 0;
    for (int i = 1; i < p.nbanks; ++i)
        if (blk >= p.bank[i].first_block) b = i;
    return __builtin_amdgcn_readfirstlane(b);
}

template <bool NT>
__global__ void __launch_bounds__(256) momentum_kernel(StreamArgs p) {
    const int64_t blk = blockIdx.x;
    const StreamBank& bk = p.bank[find_bank(p, blk)];
    const int64_t local = blk - bk.first_block;
    const int64_t slot = local / bk.nchunks, chunk = local - slot * bk.nchunks;
    float mu = bk.mu, nu = bk.nu;
    if (p.slot_scalars) {
        const f32x4 sc = p.slot_scalars[bk.slot_base + slot];
        mu = sc[0];
        nu = sc[1];
    }
    __shared__ double red[4];
    double sum;
    if (bk.f32) {
        sum = bk.vec ? momentum_chunk<true, true, NT>(bk.grad, bk.buf, bk.u, slot, chunk, bk.slot_numel, mu, nu, red)
                     : momentum_chunk<true, false, NT>(bk.grad, bk.buf, bk.u, slot, chunk, bk.slot_numel, mu, nu, red);
    } else {
        sum = bk.vec ? momentum_chunk<false, true, NT>(bk.grad, bk.buf, bk.u, slot, chunk, bk.slot_numel, mu, nu, red)
                     : momentum_chunk<false, false, NT>(bk.grad, bk.buf, bk.u, slot, chunk, bk.slot_numel, mu, nu, red);
    }
    if (threadIdx.x == 0 && bk.partials) bk.partials[slot * bk.nchunks + chunk] = sum;
}

// ---------------------------------------------------------------------------
// sum of squares of a bf16 bank (Frobenius norm of the input of a stand-alone NS)
// ---------------------------------------------------------------------------

template <bool VEC>
__global__ void __launch_bounds__(256) sumsq_kernel(const uint16_t* __restrict__ x, double* __restrict__ partials,
                                                    int64_t slot_numel, int64_t chunk_elems) {
    const int64_t slot = blockIdx.y;
    const int64_t chunk = blockIdx.x;
    const int64_t base = slot * slot_numel;
    const int64_t lo = chunk * chunk_elems;
    const int64_t hi = min(lo + chunk_elems, slot_numel);
    double acc = 0.0;
    if (VEC) {
        for (int64_t e = lo + (int64_t)threadIdx.x * 8; e < hi; e += 256 * 8) {
            u32x4 v = *reinterpret_cast<const u32x4*>(x + base + e);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = add_sq(acc, __uint_as_float(v[q] << 16));
                acc = add_sq(acc, __uint_as_float(v[q] & 0xFFFF0000u));
            }
        }
    } else {
        for (int64_t e = lo + threadIdx.x; e < hi; e += 256) acc = add_sq(acc, bf16_to_f32(x[base + e]));
    }
    __shared__ double red[4];
    acc = block_sum256(acc, red);
    if (threadIdx.x == 0) partials[slot * gridDim.x + chunk] = acc;
}

// ---------------------------------------------------------------------------
// per-slot scale and live word; pre-scaled copy of slots outside the folded range
// ---------------------------------------------------------------------------

// The Frobenius scale s = 1 / (||u||_F + eps) is folded into the first round (the Gram of the unscaled u
// times s^2, the update times s).  That is safe while the bf16 products of u stay normal in fp32 and s^2
// stays finite: ||u||_F in [2^kFoldMinExp, 2^kFoldMaxExp].  A live slot outside that range gets an exact
// power-of-two copy X0 = u * 2^k with ||X0||_F in [1, 2) (k = -floor(log2 ||u||_F)), which the first round
// reads instead of u, and scale = 2^-k / (||u||_F + eps), so that scale * X0 = s * u as before.
constexpr int kFoldMinExp = -45;
constexpr int kFoldMaxExp = 60;
constexpr int kScaleParts = 4;          // workgroups per slot (they share the copy of a pre-scaled slot)

__global__ void __launch_bounds__(256) ns_scale_kernel(ScaleArgs p) {
    const int gslot = blockIdx.x;
    int b = 0;
    for (int i = 1; i < p.nbanks; ++i)
        if (gslot >= p.bank[i].first_slot) b = i;
    const ScaleBank& bk = p.bank[__builtin_amdgcn_readfirstlane(b)];
    const int slot = gslot - bk.first_slot;
    const int part = blockIdx.y;
    const int tid = threadIdx.x;
    // persistent kernel state: queue heads, error word and exit count, and this slot's counter
    if (part == 0) {
        if (bk.heads && slot == 0 && tid < 32) bk.heads[tid] = 0;
        if (bk.ctr && tid == 0) bk.ctr[slot] = 0;
    }
    // every workgroup of the slot forms the same sum in the same order
    double acc = 0.0;
    for (int i = tid; i < bk.nchunks; i += 256) acc += bk.partials[(int64_t)slot * bk.nchunks + i];
    __shared__ double red[4];
    __shared__ int s_word;
    acc = block_sum256(acc, red);
    if (tid == 0) {
        const double nrm = sqrt(acc);
        int word = 0;
        float sc = 0.f;
        if (acc > 0.0) {
            const int e = ilogb(nrm);
            if (e >= kFoldMinExp && e < kFoldMaxExp) {
                word = kLiveBit;
                sc = (float)(1.0 / (nrm + p.eps));
            } else {
                const int k = -e;
                word = kLiveBit | kPrescaledBit | ((k + kPrescaleBias) << kPrescaleShift);
                sc = (float)(ldexp(1.0, -k) / (nrm + p.eps));
            }
        }
        s_word = word;
        if (part == 0) {
            bk.scale[slot] = sc;
            bk.live[slot] = word;
        }
    }
    __syncthreads();
    const int word = s_word;
    if (!(word & kPrescaledBit)) return;
    const int k = prescale_exp(word);
    const uint16_t* src = bk.x0 + (int64_t)slot * bk.slot_numel;
    uint16_t* dst = bk.xpre + (int64_t)slot * bk.slot_numel;
    const int64_t per = (bk.slot_numel + kScaleParts - 1) / kScaleParts;
    const int64_t lo = (int64_t)part * per, hi = min(lo + per, bk.slot_numel);
    // exact: |X0| < 2, and only elements below 2^-126 of the norm can lose bits
    for (int64_t e = lo + tid; e < hi; e += 256) dst[e] = f32_to_bf16_rne(ldexpf(bf16_to_f32(src[e]), k));
}

// ---------------------------------------------------------------------------
// mixed-precision apply
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t apply_elem(uint32_t hi, uint32_t lo, uint32_t v, float eta, float decay) {
    float w = __uint_as_float((hi << 16) | lo);
    float t = __fmul_rn(w, decay);
    float r = __fmaf_rn(-eta, __uint_as_float(v << 16), t);
    return __float_as_uint(r);
}

// One chunk of one slot.  VEC: 8 elements per thread per step (slot_numel % 8 == 0, 16-byte aligned bases).
template <bool VEC, bool NT>
__device__ __forceinline__ void apply_chunk(uint16_t* __restrict__ w_hi, uint16_t* __restrict__ w_lo,
                                            const uint16_t* __restrict__ v, int64_t slot, int64_t chunk,
                                            int64_t slot_numel, float eta, float decay) {
    const int64_t base = slot * slot_numel;
    const int64_t lo = chunk * kStreamChunk;
    const int64_t hi = min(lo + kStreamChunk, slot_numel);
    if (VEC && NT) {
        // a stream larger than the last-level cache: every load of the thread's groups before the first
        // store, all accesses non-temporal, since each element is read and written once (a 2 GB bank: 5.34
        // TB/s with cached accesses one group at a time, 5.88 TB/s like this)
        u32x4 h[kStreamGroups], l[kStreamGroups], vv[kStreamGroups];
#pragma unroll
        for (int k = 0; k < kStreamGroups; ++k) {
            const int64_t idx = base + lo + (int64_t)threadIdx.x * 8 + (int64_t)k * 256 * 8;
            if (idx < base + hi) {
                h[k] = ld16<NT>(reinterpret_cast<const u32x4*>(w_hi + idx));
                l[k] = ld16<NT>(reinterpret_cast<const u32x4*>(w_lo + idx));
                vv[k] = ld16<NT>(reinterpret_cast<const u32x4*>(v + idx));
            }
        }
#pragma unroll
        for (int k = 0; k < kStreamGroups; ++k) {
            const int64_t idx = base + lo + (int64_t)threadIdx.x * 8 + (int64_t)k * 256 * 8;
            if (idx >= base + hi) continue;
            u32x4 ho, lo2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t r0 = apply_elem(h[k][q] & 0xFFFFu, l[k][q] & 0xFFFFu, vv[k][q] & 0xFFFFu, eta, decay);
                uint32_t r1 = apply_elem(h[k][q] >> 16, l[k][q] >> 16, vv[k][q] >> 16, eta, decay);
                ho[q] = (r0 >> 16) | (r1 & 0xFFFF0000u);
                lo2[q] = (r0 & 0xFFFFu) | (r1 << 16);
            }
            st16<NT>(reinterpret_cast<u32x4*>(w_hi + idx), ho);
            st16<NT>(reinterpret_cast<u32x4*>(w_lo + idx), lo2);
        }
    } else if (VEC) {
        for (int64_t e = lo + (int64_t)threadIdx.x * 8; e < hi; e += 256 * 8) {
            const int64_t idx = base + e;
            u32x4 h = *reinterpret_cast<const u32x4*>(w_hi + idx);
            u32x4 l = *reinterpret_cast<const u32x4*>(w_lo + idx);
            u32x4 vv = *reinterpret_cast<const u32x4*>(v + idx);
            u32x4 ho, lo2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t r0 = apply_elem(h[q] & 0xFFFFu, l[q] & 0xFFFFu, vv[q] & 0xFFFFu, eta, decay);
                uint32_t r1 = apply_elem(h[q] >> 16, l[q] >> 16, vv[q] >> 16, eta, decay);
                ho[q] = (r0 >> 16) | (r1 & 0xFFFF0000u);
                lo2[q] = (r0 & 0xFFFFu) | (r1 << 16);
            }
            *reinterpret_cast<u32x4*>(w_hi + idx) = ho;
            *reinterpret_cast<u32x4*>(w_lo + idx) = lo2;
        }
    } else {
        for (int64_t e = lo + threadIdx.x; e < hi; e += 256) {
            const int64_t idx = base + e;
            uint32_t r = apply_elem(w_hi[idx], w_lo[idx], v[idx], eta, decay);
            w_hi[idx] = (uint16_t)(r >> 16);
            w_lo[idx] = (uint16_t)(r & 0xFFFFu);
        }
    }
}

template <bool NT>
__global__ void __launch_bounds__(256) apply_kernel(StreamArgs p) {
    const int64_t blk = blockIdx.x;
    const StreamBank& bk = p.bank[find_bank(p, blk)];
    const int64_t local = blk - bk.first_block;
    const int64_t slot = local / bk.nchunks, chunk = local - slot * bk.nchunks;
    float eta = bk.eta, decay = bk.decay;
    if (p.slot_scalars) {
        const f32x4 sc = p.slot_scalars[bk.slot_base + slot];
        decay = sc[2];
        eta = sc[3];
    } else if (bk.lr_mul_per_slot) {
        eta = __fmul_rn(eta, bk.lr_mul_per_slot[slot]);
    }
    if (bk.vec) apply_chunk<true, NT>(bk.w_hi, bk.w_lo, bk.v, slot, chunk, bk.slot_numel, eta, decay);
    else apply_chunk<false, NT>(bk.w_hi, bk.w_lo, bk.v, slot, chunk, bk.slot_numel, eta, decay);
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------

int stream_chunks(int64_t slot_numel) {
    // fixed chunks of kStreamChunk elements (a multiple of 8), so every thread's 8-element group stays
    // inside one slot and one chunk
    int64_t n = (slot_numel + kStreamChunk - 1) / kStreamChunk;
    return (int)(n < 1 ? 1 : n);
}

namespace {

// Bytes a launch must stream before its accesses go non-temporal (and all its loads first): the 256 MB
// last-level cache (MALL) of the MI355X.  A smaller stream can stay resident from one step to the next
// and gains from cached accesses one 8-element group at a time (attention bank, 189 MB of momentum
// traffic: 4.4 TB/s non-temporal, 4.3 cached with the loads first, 4.7-4.8 cached a group at a time); a
// larger one is evicted anyway (350M banks: momentum 5.26 -> 5.79 TB/s, apply 5.51 -> 5.80 TB/s).
constexpr int64_t kNonTemporalBytes = (int64_t)256 << 20;

// Banks [i, i + count) of one launch: their workgroups numbered bank after bank.
template <class Fill>
hipError_t launch_streams(int nbanks, const float* slot_scalars, hipStream_t stream, Fill fill, int bytes_per_elem,
                          void (*kernel)(StreamArgs), void (*kernel_nt)(StreamArgs)) {
    for (int i0 = 0; i0 < nbanks; i0 += kMaxStreamBanks) {
        StreamArgs p{};
        p.nbanks = nbanks - i0 < kMaxStreamBanks ? nbanks - i0 : kMaxStreamBanks;
        p.slot_scalars = reinterpret_cast<const f32x4*>(slot_scalars);
        int64_t blocks = 0, bytes = 0;
        for (int j = 0; j < p.nbanks; ++j) {
            StreamBank& b = p.bank[j];
            fill(i0 + j, b);
            b.nchunks = stream_chunks(b.slot_numel);
            b.first_block = blocks;
            blocks += (int64_t)b.batch * b.nchunks;
            bytes += (int64_t)b.batch * b.slot_numel * bytes_per_elem * (b.f32 ? 2 : 1);
        }
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL(bytes >= kNonTemporalBytes ? kernel_nt : kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_momentum(const MomentumBank* banks, int nbanks, const float* slot_scalars, hipStream_t stream) {
    return launch_streams(nbanks, slot_scalars, stream, [&](int i, StreamBank& b) {
        const MomentumBank& m = banks[i];
        b.grad = m.grad;
        b.buf = m.buf;
        b.u = m.u;
        b.partials = m.partials;
        b.slot_numel = m.slot_numel;
        b.batch = (int)m.batch;
        b.slot_base = m.slot_base;
        b.f32 = m.f32 ? 1 : 0;
        b.vec = m.slot_numel % 8 == 0 ? 1 : 0;
        b.mu = m.mu;
        b.nu = m.nu;
    }, 8, momentum_kernel<false>, momentum_kernel<true>);
}

hipError_t launch_apply(const ApplyBank* banks, int nbanks, const float* slot_scalars, hipStream_t stream) {
    return launch_streams(nbanks, slot_scalars, stream, [&](int i, StreamBank& b) {
        const ApplyBank& a = banks[i];
        b.w_hi = a.w_hi;
        b.w_lo = a.w_lo;
        b.v = a.v;
        b.lr_mul_per_slot = a.lr_mul_per_slot;
        b.slot_numel = a.slot_numel;
        b.batch = (int)a.batch;
        b.slot_base = a.slot_base;
        b.vec = a.slot_numel % 8 == 0 ? 1 : 0;
        b.eta = a.eta;
        b.decay = a.decay;
    }, 10, apply_kernel<false>, apply_kernel<true>);
}

hipError_t launch_sumsq(const uint16_t* x, double* partials, int64_t batch, int64_t slot_numel, hipStream_t stream) {
    dim3 grid((unsigned)stream_chunks(slot_numel), (unsigned)batch);
    if (slot_numel % 8 == 0) sumsq_kernel<true><<<grid, 256, 0, stream>>>(x, partials, slot_numel, kStreamChunk);
    else sumsq_kernel<false><<<grid, 256, 0, stream>>>(x, partials, slot_numel, kStreamChunk);
    return hipGetLastError();
}

hipError_t launch_ns_scale(const ScaleBank* banks, int nbanks, double eps, hipStream_t stream) {
    for (int i0 = 0; i0 < nbanks; i0 += kMaxStreamBanks) {
        ScaleArgs p{};
        p.nbanks = nbanks - i0 < kMaxStreamBanks ? nbanks - i0 : kMaxStreamBanks;
        p.eps = eps;
        int slots = 0;
        for (int j = 0; j < p.nbanks; ++j) {
            p.bank[j] = banks[i0 + j];
            p.bank[j].first_slot = slots;
            slots += (int)banks[i0 + j].batch;
        }
        ns_scale_kernel<<<dim3((unsigned)slots, kScaleParts), 256, 0, stream>>>(p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mb
