// Every Newton-Schulz round of a bank of small slots in one launch on gfx950.
//
// For slots whose Gram side m is at most 64 and whose m x n fits 4096 elements
// (the 1 x 12 and 6 x 12 gates, for instance) the contractions are a few
// thousand multiply-adds: one launch per contraction would be all launch cost.
// Here one workgroup holds a slot in LDS and runs every round ("Muon Custom
// Sizing", section 2.3; Record 7 walkthrough, section 4.2):
//     A = sig_A * X X^T,  B = c*(A A) + b*A,  X' = RN(sig_X * (a*X + B X))
// with fp32 accumulation in increasing k (sig_A = s^2 and sig_X = s on the
// first round, s the slot's Frobenius scale, else 1).  The iterate X is
// rounded to bf16 (round to nearest even) after every round, as in the tiled
// kernels; A and B, which here are never MFMA operands, stay fp32: on slots
// this small their bf16 roundings alone would take the relative error of the
// result to about 3 % on some inputs.  Tall slots are loaded transposed
// (X = G^T) and stored back transposed.
#include "common.hpp"
#include "kernels.hpp"

namespace mb {

namespace {

constexpr int kSmallThreads = 256;
constexpr int kSmallMaxM = 64;
constexpr int kSmallMaxElems = 4096;

struct SmallBank {
    const uint16_t* x0;     // input slots [batch][rows][cols], bf16 bits (unscaled)
    uint16_t* dest;         // output slots, same layout (may equal x0)
    const float* scale;
    const int* live;
    int rows, cols, m, n;
    int tall;
    int first_slot;         // the bank's first workgroup in the launch
};

struct SmallArgs {
    SmallBank bank[kMaxSmallBanks];
    int nbanks;
    int steps;
    float coef[kMaxRounds][3];
};

__device__ __forceinline__ float round_bf16(float y) { return bf16_to_f32(f32_to_bf16_rne(y)); }

__global__ void __launch_bounds__(kSmallThreads) ns_small_kernel(SmallArgs args) {
    extern __shared__ float sm[];
    int bi = 0;
    for (int i = 1; i < args.nbanks; ++i)
        if ((int)blockIdx.x >= args.bank[i].first_slot) bi = i;
    const SmallBank& p = args.bank[__builtin_amdgcn_readfirstlane(bi)];
    const int m = p.m, n = p.n, mn = m * n, mm = m * m;
    float* X = sm;                 // [m][n]
    float* Y = X + mn;             // [m][n], next round
    float* A = Y + mn;             // [m][m]
    float* B = A + mm;             // [m][m]
    const int slot = (int)blockIdx.x - p.first_slot;
    const int tid = threadIdx.x;
    const uint16_t* src = p.x0 + (int64_t)slot * mn;
    uint16_t* dst = p.dest + (int64_t)slot * mn;
    const int lword = p.live[slot];
    if (lword == 0) {
        // a zero slot's result is exactly zero (dest may alias x0: nothing was read)
        for (int e = tid; e < mn; e += kSmallThreads) dst[e] = 0;
        return;
    }
    // X[i][k] = u[i][k] (wide) or u[k][i] (tall: u is n x m); a pre-scaled slot takes X = u * 2^k,
    // exact in fp32, with the inverse power of two in its scale
    const int pk = (lword & kPrescaledBit) ? prescale_exp(lword) : 0;
    for (int e = tid; e < mn; e += kSmallThreads) {
        const int i = e / n, k = e - i * n;
        X[e] = ldexpf(bf16_to_f32(p.tall ? src[(int64_t)k * m + i] : src[e]), pk);
    }
    const float s = p.scale[slot];
    __syncthreads();
    for (int t = 0; t < args.steps; ++t) {
        const float a = args.coef[t][0], b = args.coef[t][1], c = args.coef[t][2];
        const float sig_a = t == 0 ? s * s : 1.f, sig_x = t == 0 ? s : 1.f;
        for (int e = tid; e < mm; e += kSmallThreads) {
            const int i = e / m, j = e - i * m;
            float acc = 0.f;
            for (int k = 0; k < n; ++k) acc = __fmaf_rn(X[i * n + k], X[j * n + k], acc);
            A[e] = sig_a * acc;
        }
        __syncthreads();
        for (int e = tid; e < mm; e += kSmallThreads) {
            const int i = e / m, j = e - i * m;
            float acc = 0.f;
            for (int k = 0; k < m; ++k) acc = __fmaf_rn(A[i * m + k], A[k * m + j], acc);
            B[e] = __fmaf_rn(b, A[e], c * acc);
        }
        __syncthreads();
        for (int e = tid; e < mn; e += kSmallThreads) {
            const int i = e / n, j = e - i * n;
            float acc = 0.f;
            for (int k = 0; k < m; ++k) acc = __fmaf_rn(B[i * m + k], X[k * n + j], acc);
            Y[e] = round_bf16(sig_x * __fmaf_rn(a, X[e], acc));
        }
        __syncthreads();
        float* tmp = X;
        X = Y;
        Y = tmp;
    }
    // every read of the input happened before the first barrier, so dest may alias x0
    for (int e = tid; e < mn; e += kSmallThreads) {
        const int i = e / n, k = e - i * n;
        const uint16_t h = f32_to_bf16_rne(X[e]);
        if (p.tall) dst[(int64_t)k * m + i] = h;
        else dst[e] = h;
    }
}

}  // namespace

bool ns_small_eligible(int64_t rows, int64_t cols, int steps) {
    const int64_t m = rows < cols ? rows : cols;
    return steps >= 1 && steps <= kMaxRounds && m <= kSmallMaxM && rows * cols <= kSmallMaxElems;
}

hipError_t ns_small(const NsSmall* banks, int nbanks, int steps, const NsCoef* coef, hipStream_t stream) {
    if (steps < 1 || steps > kMaxRounds) return hipErrorInvalidValue;
    for (int i0 = 0; i0 < nbanks; i0 += kMaxSmallBanks) {
        SmallArgs p{};
        p.nbanks = nbanks - i0 < kMaxSmallBanks ? nbanks - i0 : kMaxSmallBanks;
        p.steps = steps;
        for (int t = 0; t < steps; ++t) {
            p.coef[t][0] = coef[t].a;
            p.coef[t][1] = coef[t].b;
            p.coef[t][2] = coef[t].c;
        }
        int slots = 0;
        size_t lds = 0;
        for (int j = 0; j < p.nbanks; ++j) {
            const NsSmall& r = banks[i0 + j];
            SmallBank& b = p.bank[j];
            b.x0 = r.x0;
            b.dest = r.dest;
            b.scale = r.scale;
            b.live = r.live;
            b.rows = (int)r.rows;
            b.cols = (int)r.cols;
            b.tall = r.rows > r.cols ? 1 : 0;
            b.m = (int)(b.tall ? r.cols : r.rows);
            b.n = (int)(b.tall ? r.rows : r.cols);
            b.first_slot = slots;
            slots += (int)r.batch;
            const size_t need = (size_t)(2 * b.m * b.n + 2 * b.m * b.m) * sizeof(float);
            lds = need > lds ? need : lds;
        }
        ns_small_kernel<<<dim3((unsigned)slots), kSmallThreads, lds, stream>>>(p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mb
