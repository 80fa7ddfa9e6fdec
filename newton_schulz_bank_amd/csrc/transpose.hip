// Tiled transposes for the tied embedding on gfx950 ("Unified zero-copy
// optimizer and transposed LM head", section 2.2): the LM head is stored
// transposed, (768, 50304), against the embedding's (50304, 768), and the
// optimizer step needs
//     transpose_copy:  dst[j][i] = src[i][j]
//     transpose_add:   dst[j][i] = RN(dst[j][i] + src[i][j])
// for src [rows, cols], dst [cols, rows].  Both are bound by HBM: every
// element is read once (twice for the add: src and dst) and written once.
//
// A workgroup moves one 64 x 64 tile: 16-byte row reads of src into LDS, then
// 16-byte row writes of dst, so both ends move whole rows.  For 2-byte
// elements the column read out of LDS is the gfx950 transposing read
// ds_read_b64_tr_b16 (two of them give a lane 8 consecutive elements of a dst
// row); for 4-byte elements a padded tile is read a dword at a time.  The add
// loads its dst chunks before the tile arrives, so their latency overlaps.
// Shapes whose rows are not whole 16-byte chunks take an element-wise kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace mb {

namespace {

constexpr int kT = 64;          // tile edge (elements)
constexpr int kThreads = 256;

// ---- 2-byte elements ------------------------------------------------------
constexpr int kP16 = kT + 8;    // LDS row pitch (elements): 144 B, so the 4 rows a transposing read touches use distinct banks

template <bool ADD, bool BF16>
__global__ void __launch_bounds__(kThreads) transpose16_kernel(uint16_t* __restrict__ dst, const uint16_t* __restrict__ src,
                                                               int rows, int cols, int tiles_c) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[kT * kP16];
    const int tr = blockIdx.x / tiles_c, tc = blockIdx.x - tr * tiles_c;
    const int i0 = tr * kT, j0 = tc * kT;           // src rows i0.., src cols j0..
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // store side: 16-lane group g of wave w handles dst rows j0 + 16*jg + t, dst cols i0 + 8*ig .. +8
    // (unit u = it*16 + 4*wave + g: jg = u / 8, ig = u % 8)
    const int g = lane >> 4, t16 = lane & 15, s4 = t16 >> 2, q4 = t16 & 3;
    u32x4 old[2];
    if (ADD) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int u = it * 16 + 4 * wave + g, jg = u >> 3, ig = u & 7;
            const int jr = j0 + 16 * jg + t16, ic = i0 + 8 * ig;
            old[it] = (jr < cols && ic < rows) ? *reinterpret_cast<const u32x4*>(dst + (int64_t)jr * rows + ic)
                                               : u32x4{0u, 0u, 0u, 0u};
        }
    }
    // load side: thread -> src row i0 + r, 8 elements from column j0 + 8c
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int v = it * kThreads + tid, r = v >> 3, c = v & 7;
        const int gi = i0 + r, gj = j0 + 8 * c;
        u32x4 x = u32x4{0u, 0u, 0u, 0u};
        if (gi < rows && gj < cols) x = *reinterpret_cast<const u32x4*>(src + (int64_t)gi * cols + gj);
        *reinterpret_cast<u32x4*>(tile + r * kP16 + 8 * c) = x;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int u = it * 16 + 4 * wave + g, jg = u >> 3, ig = u & 7;
        // lane 4s + q addresses tile row 8*ig + s (then + 4), columns 16*jg + 4q .. +3; lane t receives
        // column 16*jg + t of those rows: 8 consecutive src rows of one src column
        const uint16_t* pa = tile + (8 * ig + s4) * kP16 + 16 * jg + 4 * q4;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(pa));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(pa + 4 * kP16));
        u32x4 w;
        w[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
        w[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
        w[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
        w[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
        const int jr = j0 + 16 * jg + t16, ic = i0 + 8 * ig;
        if (jr < cols && ic < rows) {
            if (ADD) {
                // bf16 + bf16 in fp32, then one rounding to bf16 (the fp32 sum is exact unless the
                // exponents differ by more than 16, and then the result is the larger term either way)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t a = old[it][e], b = w[e];
                    const float s0 = __fadd_rn(__uint_as_float(a << 16), __uint_as_float(b << 16));
                    const float s1 = __fadd_rn(__uint_as_float(a & 0xFFFF0000u), __uint_as_float(b & 0xFFFF0000u));
                    w[e] = f32x2_to_bf16x2_rne(s0, s1);
                }
            }
            *reinterpret_cast<u32x4*>(dst + (int64_t)jr * rows + ic) = w;
        }
    }
}

// ---- 4-byte elements ------------------------------------------------------
constexpr int kP32 = kT + 1;    // LDS row pitch (dwords): column reads hit distinct banks

template <bool ADD>
__global__ void __launch_bounds__(kThreads) transpose32_kernel(uint32_t* __restrict__ dst, const uint32_t* __restrict__ src,
                                                               int rows, int cols, int tiles_c) {
    __shared__ uint32_t tile[kT * kP32];
    const int tr = blockIdx.x / tiles_c, tc = blockIdx.x - tr * tiles_c;
    const int i0 = tr * kT, j0 = tc * kT;
    const int tid = threadIdx.x;
    // store side: thread -> dst row j0 + (v >> 4), 4 elements from dst column i0 + 4*(v & 15)
    u32x4 old[4];
    if (ADD) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int v = it * kThreads + tid, jr = j0 + (v >> 4), ic = i0 + 4 * (v & 15);
            old[it] = (jr < cols && ic < rows) ? *reinterpret_cast<const u32x4*>(dst + (int64_t)jr * rows + ic)
                                               : u32x4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int v = it * kThreads + tid, r = v >> 4, c = v & 15;
        const int gi = i0 + r, gj = j0 + 4 * c;
        u32x4 x = u32x4{0u, 0u, 0u, 0u};
        if (gi < rows && gj < cols) x = *reinterpret_cast<const u32x4*>(src + (int64_t)gi * cols + gj);
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[r * kP32 + 4 * c + e] = x[e];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int v = it * kThreads + tid, jl = v >> 4, il = 4 * (v & 15);
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = tile[(il + e) * kP32 + jl];
        const int jr = j0 + jl, ic = i0 + il;
        if (jr < cols && ic < rows) {
            if (ADD) {
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(__fadd_rn(__uint_as_float(old[it][e]), __uint_as_float(w[e])));
            }
            *reinterpret_cast<u32x4*>(dst + (int64_t)jr * rows + ic) = w;
        }
    }
}

// ---- any shape, any alignment: one element per thread and step --------------
template <bool ADD, int ES, bool BF16>
__global__ void __launch_bounds__(kThreads) transpose_any_kernel(void* __restrict__ dst_, const void* __restrict__ src_,
                                                                 int rows, int cols, int tiles_c) {
    typedef typename std::conditional<ES == 2, uint16_t, uint32_t>::type T;
    __shared__ T tile[kT * (kT + 1)];
    T* dst = static_cast<T*>(dst_);
    const T* src = static_cast<const T*>(src_);
    const int tr = blockIdx.x / tiles_c, tc = blockIdx.x - tr * tiles_c;
    const int i0 = tr * kT, j0 = tc * kT;
    for (int v = threadIdx.x; v < kT * kT; v += kThreads) {
        const int r = v / kT, c = v % kT;
        if (i0 + r < rows && j0 + c < cols) tile[r * (kT + 1) + c] = src[(int64_t)(i0 + r) * cols + j0 + c];
    }
    __syncthreads();
    for (int v = threadIdx.x; v < kT * kT; v += kThreads) {
        const int jl = v / kT, il = v % kT;
        const int jr = j0 + jl, ic = i0 + il;
        if (jr >= cols || ic >= rows) continue;
        T x = tile[il * (kT + 1) + jl];
        T* d = dst + (int64_t)jr * rows + ic;
        if (ADD) {
            if (ES == 4) {
                x = __float_as_uint(__fadd_rn(__uint_as_float(*d), __uint_as_float(x)));
            } else {
                const float s = __fadd_rn(bf16_to_f32(*d), bf16_to_f32(x));
                x = f32_to_bf16_rne(s);
            }
        }
        *d = x;
    }
}

}  // namespace

hipError_t launch_transpose(void* dst, const void* src, int64_t rows, int64_t cols, int elem_bytes, bool add,
                            hipStream_t stream) {
    const int tiles_r = (int)((rows + kT - 1) / kT), tiles_c = (int)((cols + kT - 1) / kT);
    const dim3 grid((unsigned)((int64_t)tiles_r * tiles_c));
    const bool vec = ((uintptr_t)dst & 15) == 0 && ((uintptr_t)src & 15) == 0 && (rows * elem_bytes) % 16 == 0 &&
                     (cols * elem_bytes) % 16 == 0;
    const int r = (int)rows, c = (int)cols;
    if (elem_bytes == 2) {
        if (vec) {
            if (add) transpose16_kernel<true, true><<<grid, kThreads, 0, stream>>>((uint16_t*)dst, (const uint16_t*)src, r, c, tiles_c);
            else transpose16_kernel<false, true><<<grid, kThreads, 0, stream>>>((uint16_t*)dst, (const uint16_t*)src, r, c, tiles_c);
        } else {
            if (add) transpose_any_kernel<true, 2, true><<<grid, kThreads, 0, stream>>>(dst, src, r, c, tiles_c);
            else transpose_any_kernel<false, 2, true><<<grid, kThreads, 0, stream>>>(dst, src, r, c, tiles_c);
        }
    } else {
        if (vec) {
            if (add) transpose32_kernel<true><<<grid, kThreads, 0, stream>>>((uint32_t*)dst, (const uint32_t*)src, r, c, tiles_c);
            else transpose32_kernel<false><<<grid, kThreads, 0, stream>>>((uint32_t*)dst, (const uint32_t*)src, r, c, tiles_c);
        } else {
            if (add) transpose_any_kernel<true, 4, false><<<grid, kThreads, 0, stream>>>(dst, src, r, c, tiles_c);
            else transpose_any_kernel<false, 4, false><<<grid, kThreads, 0, stream>>>(dst, src, r, c, tiles_c);
        }
    }
    return hipGetLastError();
}

}  // namespace mb
