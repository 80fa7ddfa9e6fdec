// All Newton-Schulz rounds of a bank in one persistent launch on gfx950.
//
// The rounds ("Muon Custom Sizing", section 2.3; Record 7 walkthrough, section
// 4.2) chain three contractions per slot and round,
//     A = X X^T,   B = b*A + c*A A,   X' = a*X + B X      (wide or square X)
//     A = G^T G,   B as above,        G' = a*G + G B      (tall G),
// and the slots are independent.  Instead of one launch per contraction (whose
// last wave of tiles leaves most CUs idle and whose boundary writes back the
// whole L2), every 256x256 output tile of every contraction is a task, and the
// workgroups of one launch take tasks from a queue while they last.
//
// Placement.  Workgroups are spread over the XCDs, each with its own L2, and
// the L2s are not coherent with each other inside a kernel.  Slot s belongs to
// XCD s % nq: its tasks sit in that XCD's queue, and only workgroups running on
// that XCD (read from the XCC_ID hardware register) take them, so a slot's
// intermediate results are produced and consumed through one L2.
//
// Ordering.  A queue lists the tasks round by round, contraction by
// contraction, slot by slot.  A task needs every tile of the previous
// contraction of its slot: its slot's counter of finished tasks must have
// reached the number of tasks that come before it in that slot's chain.  A
// producer waits until its stores are acknowledged (they are then in the L2),
// then bumps the counter with a device-scope atomic; a consumer polls the
// counter, and loads every operand with the sc1 policy, which misses the CU's
// L1 (possibly stale) and reads the L2.  Tasks are claimed in queue order, so
// everything a task waits for was claimed earlier by a running workgroup:
// progress never depends on how many workgroups are resident.  A wait longer
// than kWaitCapTicks (a fault, never a normal schedule) sets the error word and
// gives up instead of spinning forever.
#include "common.hpp"
#include "kernels.hpp"
#include "ns_tile.hpp"

namespace mb {

namespace {

constexpr uint64_t kWaitCapTicks = 20000000;   // 200 ms of the 100 MHz constant clock
constexpr int kXccIdReg = 20 | (0 << 6) | (15 << 11);   // hwreg(HW_REG_XCC_ID, 0, 16)

struct PersistArgs {
    const uint16_t* x0;     // round input of round 0 (unscaled)
    uint16_t* xa;           // outputs of rounds 0, 2, 4, ... (except the last)
    uint16_t* xb;           // outputs of rounds 1, 3, 5, ...
    uint16_t* dest;         // output of the last round
    uint16_t* A;
    uint16_t* Bm;
    const float* scale;
    const int* live;
    int* sync;              // [0, 16) queue heads, [16] error word, [32, 32 + batch) per-slot counters
    int64_t slot;           // elements per slot of X
    int64_t mm;             // elements per slot of A, B
    int m, n;               // Gram size and long side (m <= n)
    int tm, tn;             // tiles along m and along n
    int batch, steps, nq;
    float coef[kMaxRounds][3];   // (a, b, c) of each round
};

__device__ __forceinline__ int ld_relaxed(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool TALL, class C>
__global__ void __launch_bounds__(C::NT, 2) ns_persist_kernel(PersistArgs p) {
    static_assert(C::BM == C::BN, "square tiles");
    constexpr int kTile = C::BM;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[C::RING];
    __shared__ int s_task;
    int* heads = p.sync;
    int* err = p.sync + 16;
    int* ctr = p.sync + 32;
    const int tid = threadIdx.x;
    const int q = (int)(__builtin_amdgcn_s_getreg(kXccIdReg) & 0xFFFF) % p.nq;
    const int ls = q < p.batch ? (p.batch - q + p.nq - 1) / p.nq : 0;    // slots q, q + nq, ...
    const int nG = p.tm * (p.tm + 1) / 2, nP = nG, nU = p.tm * p.tn;
    const int chain = nG + nP + nU;                                       // tasks per slot and round
    const int per_round = ls * chain;
    const int total = p.steps * per_round;

    // Every branch in this loop is wave-uniform: the queue and counter traffic is done by all
    // 64 lanes of wavefront 0 together (lane 0 adds 1, the others 0) and every loop condition
    // is a readfirstlane value.  A branch on (threadIdx.x == 0) here would let the compiler
    // restructure the loop so that lane 0 and the other lanes of wavefront 0 reach the
    // workgroup barriers in different iterations.
    const bool leader = __builtin_amdgcn_readfirstlane(tid >> 6) == 0;
    const int one = (tid & 63) == 0 ? 1 : 0;
    if (leader) {
        const int got = __hip_atomic_fetch_add(heads + q, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_task = __builtin_amdgcn_readfirstlane(got);
    }
    __syncthreads();
    int idx = __builtin_amdgcn_readfirstlane(s_task);
    while (idx >= 0 && idx < total) {
        const int t = idx / per_round;
        int r = idx - t * per_round;
        int phase, l, tile;
        if (r < ls * nG) { phase = 0; l = r / nG; tile = r - l * nG; }
        else if ((r -= ls * nG) < ls * nP) { phase = 1; l = r / nP; tile = r - l * nP; }
        else { r -= ls * nP; phase = 2; l = r / nU; tile = r - l * nU; }
        const int slot = q + l * p.nq;
        const int need = t * chain + (phase == 0 ? 0 : phase == 1 ? nG : nG + nP);

        if (leader && need > 0 && __builtin_amdgcn_readfirstlane(ld_relaxed(ctr + slot)) < need) {
            const uint64_t t0 = wall_clock64();
            for (int spin = 0;; ++spin) {
                __builtin_amdgcn_s_sleep(2);
                if (__builtin_amdgcn_readfirstlane(ld_relaxed(ctr + slot)) >= need) break;
                if ((spin & 63) == 63 && (__builtin_amdgcn_readfirstlane(ld_relaxed(err)) != 0 ||
                                          wall_clock64() - t0 > kWaitCapTicks)) {
                    __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        __syncthreads();
        int ltid = tid;
        asm volatile("" : "+v"(ltid));

        const bool last = t == p.steps - 1;
        const uint16_t* xin = t == 0 ? p.x0 : ((t & 1) ? p.xa : p.xb);
        uint16_t* xout = last ? p.dest : ((t & 1) ? p.xb : p.xa);
        const uint16_t* xs = xin + (int64_t)slot * p.slot;
        uint16_t* As = p.A + (int64_t)slot * p.mm;
        uint16_t* Bs = p.Bm + (int64_t)slot * p.mm;
        const bool live = p.live[slot] != 0;
        const uint32_t xbytes = (uint32_t)(p.slot * 2), abytes = (uint32_t)(p.mm * 2);

        TileJob jb;
        jb.alpha = 1.f;
        jb.beta = 0.f;
        jb.sig = 1.f;
        if (phase == 0) {
            if (live) {
                int ti, tj;
                sym_tile(tile, p.tm, ti, tj);
                jb.P = make_rsrc(xs, xbytes);
                jb.Q = jb.P;
                jb.X = jb.P;
                jb.ldp = jb.ldq = TALL ? p.m : p.n;
                jb.ldx = jb.ldp;
                jb.ldo = p.m;
                jb.K = p.n;
                jb.i0 = ti * kTile;
                jb.j0 = tj * kTile;
                jb.out = As;
                jb.mirror = ti != tj;
                if (t == 0) {
                    const float s = p.scale[slot];
                    jb.sig = s * s;
                }
                gemm_tile<!TALL, !TALL, EPI_GRAM, C, POL_SC1>(jb, smem, ltid);
            }
        } else if (phase == 1) {
            if (live) {
                int ti, tj;
                sym_tile(tile, p.tm, ti, tj);
                jb.P = make_rsrc(As, abytes);
                jb.Q = jb.P;
                jb.X = jb.P;
                jb.ldp = jb.ldq = jb.ldx = jb.ldo = p.m;
                jb.K = p.m;
                jb.i0 = ti * kTile;
                jb.j0 = tj * kTile;
                jb.out = Bs;
                jb.mirror = ti != tj;
                jb.alpha = p.coef[t][2];
                jb.beta = p.coef[t][1];
                gemm_tile<true, true, EPI_POLY, C, POL_SC1>(jb, smem, ltid);
            }
        } else {
            // wide: X' (m x n) = a*X + B X;  tall: G' (n x m) = a*G + G B
            const int nt_cols = TALL ? p.tm : p.tn;
            const int ti = tile / nt_cols, tj = tile - ti * nt_cols;
            const int ld = TALL ? p.m : p.n;
            uint16_t* os = xout + (int64_t)slot * p.slot;
            if (live) {
                const i32x4 rx = make_rsrc(xs, xbytes);
                const i32x4 rb = make_rsrc(Bs, abytes);
                jb.P = TALL ? rx : rb;
                jb.Q = TALL ? rb : rx;
                jb.X = rx;
                jb.ldp = p.m;
                jb.ldq = TALL ? p.m : p.n;
                jb.ldx = jb.ldo = ld;
                jb.K = p.m;
                jb.i0 = ti * kTile;
                jb.j0 = tj * kTile;
                jb.out = os;
                jb.mirror = false;
                jb.beta = p.coef[t][0];
                if (t == 0) jb.sig = p.scale[slot];
                gemm_tile<true, TALL, EPI_UPDATE, C, POL_SC1>(jb, smem, ltid);
            } else if (last) {
                // a zero slot's result is exactly zero
                const int i0 = ti * kTile, j0 = tj * kTile;
                for (int v = tid; v < kTile * kTile / 8; v += C::NT) {
                    const int i = v / (kTile / 8), c8 = v % (kTile / 8);
                    *reinterpret_cast<u32x4*>(os + (int64_t)(i0 + i) * ld + j0 + c8 * 8) = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }

        // publish: every store of this workgroup is in the L2 before the counter moves; then
        // claim the next task (claiming earlier, while a tile is still running, holds back
        // tasks that another workgroup could start at once)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (leader) {
            __hip_atomic_fetch_add(ctr + slot, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_task = __builtin_amdgcn_readfirstlane(
                __hip_atomic_fetch_add(heads + q, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
        __syncthreads();
        idx = __builtin_amdgcn_readfirstlane(s_task);
    }
}

struct DeviceShape {
    int cus = 0, xccs = 0;
};

hipError_t device_shape(DeviceShape* out) {
    static thread_local int cached_dev = -1;
    static thread_local DeviceShape cached;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev != cached_dev) {
        DeviceShape d;
        if ((e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&d.xccs, hipDeviceAttributeNumberOfXccs, dev)) != hipSuccess) return e;
        if (d.xccs < 1 || d.xccs > 16 || d.cus % d.xccs != 0) d.xccs = 1;
        cached = d;
        cached_dev = dev;
    }
    *out = cached;
    return hipSuccess;
}

// Tile edge of the persistent kernel for a slot of m x n (m <= n), 0 if it cannot run it.
int persist_tile(int64_t m, int64_t n) {
    if (m % 256 == 0 && n % 256 == 0) return 256;
    if (m % 128 == 0 && n % 128 == 0) return 128;
    return 0;
}

}  // namespace

bool ns_persist_eligible(int64_t rows, int64_t cols, int steps) {
    const int64_t m = rows < cols ? rows : cols, n = rows < cols ? cols : rows;
    return steps >= 1 && steps <= kMaxRounds && persist_tile(m, n) != 0 && m * n <= ((int64_t)1 << 30) && m * m <= ((int64_t)1 << 30);
}

int ns_persist_sync_ints(int64_t batch) { return 32 + (int)batch; }

hipError_t ns_persist(const NsPersist& r, hipStream_t stream) {
    DeviceShape d;
    hipError_t e = device_shape(&d);
    if (e != hipSuccess) return e;
    const bool tall = r.rows > r.cols;
    PersistArgs p{};
    p.x0 = r.x0;
    p.xa = r.xa;
    p.xb = r.xb;
    p.dest = r.dest;
    p.A = r.A;
    p.Bm = r.Bm;
    p.scale = r.scale;
    p.live = r.live;
    p.sync = r.sync;
    p.slot = r.rows * r.cols;
    p.m = (int)(tall ? r.cols : r.rows);
    p.n = (int)(tall ? r.rows : r.cols);
    p.mm = (int64_t)p.m * p.m;
    const int tile = persist_tile(p.m, p.n);
    p.tm = p.m / tile;
    p.tn = p.n / tile;
    p.batch = (int)r.batch;
    p.steps = r.steps;
    p.nq = d.xccs;
    for (int t = 0; t < r.steps && t < kMaxRounds; ++t) {
        p.coef[t][0] = r.coef[t].a;
        p.coef[t][1] = r.coef[t].b;
        p.coef[t][2] = r.coef[t].c;
    }
    if (tile == 256) {
        // one 8-wavefront workgroup per CU (its 128 KiB ring fills the LDS)
        const dim3 grid((unsigned)d.cus);
        if (tall) ns_persist_kernel<true, Cfg256><<<grid, Cfg256::NT, 0, stream>>>(p);
        else ns_persist_kernel<false, Cfg256><<<grid, Cfg256::NT, 0, stream>>>(p);
    } else {
        // two 4-wavefront workgroups per CU
        const dim3 grid((unsigned)(2 * d.cus));
        if (tall) ns_persist_kernel<true, Cfg128><<<grid, Cfg128::NT, 0, stream>>>(p);
        else ns_persist_kernel<false, Cfg128><<<grid, Cfg128::NT, 0, stream>>>(p);
    }
    return hipGetLastError();
}

}  // namespace mb
