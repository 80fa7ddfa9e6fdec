// All Newton-Schulz rounds of one or more banks in one persistent launch on gfx950.
//
// The rounds ("Muon Custom Sizing", section 2.3; Record 7 walkthrough, section
// 4.2) chain three contractions per slot and round,
//     A = X X^T,   B = b*A + c*A A,   X' = a*X + B X      (wide or square X)
//     A = G^T G,   B as above,        G' = a*G + G B      (tall G),
// and the slots are independent.  Instead of one launch per contraction (whose
// last wave of tiles leaves most CUs idle and whose boundary writes back the
// whole L2), every 256x256 (or 128x128) output tile of every contraction of every bank is a
// task, and the workgroups of one launch take tasks from a queue while they
// last: the short contractions of one bank fill the gaps of another's.
//
// Placement.  Workgroups are spread over the XCDs, each with its own L2, and
// the L2s are not coherent with each other inside a kernel.  The slots of all
// banks are numbered in one sequence; slot g belongs to XCD g % nq: its tasks
// sit in that XCD's queue, and only workgroups running on that XCD (read from
// the XCC_ID hardware register) take them, so a slot's intermediate results
// are produced and consumed through one L2.
//
// Ordering.  A queue lists the tasks round by round, contraction by
// contraction, bank by bank, slot by slot.  A task needs every tile of the previous
// contraction of its slot: its slot's counter of finished tasks must have
// reached the number of tasks that come before it in that slot's chain.  A
// producer waits until its stores are acknowledged (they are then in the L2),
// then bumps the counter with a device-scope atomic; a consumer polls the
// counter, and loads every operand with the sc1 policy, which misses the CU's
// L1 (possibly stale) and reads the L2.  Tasks are claimed in queue order, so
// everything a task waits for was claimed earlier by a running workgroup:
// progress never depends on how many workgroups are resident.  A wait longer
// than kWaitCapTicks (a fault, never a normal schedule) sets the error word and
// gives up instead of spinning forever.  The last workgroup to leave checks that
// every queue was drained (a queue that no workgroup served would leave its
// tasks undone) and sets the error word otherwise.
#include <atomic>
#include <cstdio>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"
#include "ns_persist_plan.hpp"
#include "ns_tile.hpp"

namespace mb {

// Set (never cleared by a kernel) when a dependency wait of any persistent launch on this device hits
// its time cap; read and cleared from the host through ns_persist_fault.
__device__ int g_persist_fault;

namespace {

constexpr uint64_t kWaitCapTicks = 20000000;   // 200 ms of the 100 MHz constant clock
// test hook (ns_persist_test_faults): a shorter wait cap, and queues beyond the XCDs that nothing serves
std::atomic<uint64_t> g_test_wait_cap{0};
std::atomic<int> g_test_extra_queues{0};
// A 256-tile launch takes the three-slot ring from this many bytes of X (all slots of all its banks) on
constexpr int64_t kAheadMinBytes = (int64_t)128 << 20;
// Tasks of one round per queue, in units of the queue's workgroups, from which a launch claims early
constexpr int kEarlyClaimDepth = 2;
constexpr int kXccIdReg = 20 | (0 << 6) | (15 << 11);   // hwreg(HW_REG_XCC_ID, 0, 16)

__device__ __forceinline__ int ld_relaxed(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Which operand of each contraction the 256-tile ring copies two stages ahead (false: P, true: Q).
constexpr bool kQAheadGram = true;
constexpr bool kQAheadPoly = true;
constexpr bool kQAheadWideUpdate = true;

template <class C>
__global__ void __launch_bounds__(C::NT, 2) ns_persist_kernel(PersistArgs p) {
    static_assert(C::BM == C::BN, "square tiles");
    constexpr int kTile = C::BM;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[C::RING];
    // The claimed task's index is handed to every wavefront through an LDS word.  The three-slot ring
    // fills the LDS, so there the word is the ring's last: it belongs to the second slot of the operand
    // copied one stage ahead, which no copy writes before the first k step of a tile, and every wavefront
    // reads the index before the barrier ahead of the tile; it lies beyond the epilogue's staging tile.
    int* task_word;
    if constexpr (C::PAHEAD) {
        static_assert(C::RING * 2 - 4 >= C::BM * C::BN * 2, "the task word lies outside the staging tile");
        task_word = reinterpret_cast<int*>(smem + C::RING) - 1;
    } else {
        __shared__ int word;
        task_word = &word;
    }
    int& s_task = *task_word;
    const int tid = threadIdx.x;
    const int q = (int)(__builtin_amdgcn_s_getreg(kXccIdReg) & 0xFFFF) % p.nq;
    const int per_round = p.per_round[q];
    const int total = p.steps * per_round;

    // Every branch in this loop is wave-uniform: the queue and counter traffic is done by all
    // 64 lanes of wavefront 0 together (lane 0 adds 1, the others 0) and every loop condition
    // is a readfirstlane value.  A branch on (threadIdx.x == 0) here would let the compiler
    // restructure the loop so that lane 0 and the other lanes of wavefront 0 reach the
    // workgroup barriers in different iterations.
    const bool leader = __builtin_amdgcn_readfirstlane(tid >> 6) == 0;
    const int one = (tid & 63) == 0 ? 1 : 0;
    if (leader) {
        const int got = __hip_atomic_fetch_add(p.heads + q, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_task = __builtin_amdgcn_readfirstlane(got);
    }
    __syncthreads();
    int idx = __builtin_amdgcn_readfirstlane(s_task);
    while (idx >= 0 && idx < total) {
        // ---- decode: round t, contraction (phase), bank, slot, tile, and the slot's finished-task
        // count this task waits for
        // (every field is wave-uniform: readfirstlane keeps them in scalar registers)
        const PersistTask task = decode_task(p, q, idx);
        const int t = __builtin_amdgcn_readfirstlane(task.t), phase = __builtin_amdgcn_readfirstlane(task.phase);
        const int slot = __builtin_amdgcn_readfirstlane(task.slot), tile = __builtin_amdgcn_readfirstlane(task.tile);
        const int need = __builtin_amdgcn_readfirstlane(task.need);
        const PersistBank& bk = p.bank[__builtin_amdgcn_readfirstlane(task.b)];
        int* ctr = p.ctr + bk.base + slot;

        if (leader && need > 0 && __builtin_amdgcn_readfirstlane(ld_relaxed(ctr)) < need) {
            const uint64_t t0 = wall_clock64();
            for (int spin = 0;; ++spin) {
                __builtin_amdgcn_s_sleep(2);
                if (__builtin_amdgcn_readfirstlane(ld_relaxed(ctr)) >= need) break;
                if ((spin & 63) == 63 && (__builtin_amdgcn_readfirstlane(ld_relaxed(p.err)) != 0 ||
                                          wall_clock64() - t0 > p.wait_cap)) {
                    __hip_atomic_store(p.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(&g_persist_fault, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    break;
                }
            }
        }
        __syncthreads();
        int ltid = tid;
        asm volatile("" : "+v"(ltid));

        const bool tall = bk.tall != 0;
        const bool last = t == p.steps - 1;
        const int lword = bk.live[slot];
        const bool live = lword != 0;
        const uint16_t* xin = t == 0 ? ((lword & kPrescaledBit) ? bk.xpre : bk.x0) : ((t & 1) ? bk.xa : bk.xb);
        uint16_t* xout = last ? bk.dest : ((t & 1) ? bk.xb : bk.xa);
        const uint16_t* xs = xin + (int64_t)slot * bk.slot;
        uint16_t* As = bk.A + (int64_t)slot * bk.mm;
        uint16_t* Bs = bk.Bm + (int64_t)slot * bk.mm;
        const uint32_t xbytes = (uint32_t)(bk.slot * 2), abytes = (uint32_t)(bk.mm * 2);

        TileJob jb;
        jb.alpha = 1.f;
        jb.beta = 0.f;
        jb.sig = 1.f;
        if (phase == 0) {
            if (live) {
                int ti, tj;
                sym_tile(tile, bk.tm, ti, tj);
                jb.P = make_rsrc(xs, xbytes);
                jb.Q = jb.P;
                jb.X = jb.P;
                jb.ldp = jb.ldq = tall ? bk.m : bk.n;
                jb.ldx = jb.ldp;
                jb.ldo = bk.m;
                jb.K = bk.n;
                jb.i0 = ti * kTile;
                jb.j0 = tj * kTile;
                jb.out = As;
                jb.mirror = ti != tj;
                if (t == 0) {
                    const float sc = bk.scale[slot];
                    jb.sig = sc * sc;
                }
                if (tall) gemm_tile<false, false, EPI_GRAM, C, POL_SC1, C::PAHEAD && kQAheadGram>(jb, (lds_u16*)smem, ltid);
                else gemm_tile<true, true, EPI_GRAM, C, POL_SC1, C::PAHEAD && kQAheadGram>(jb, (lds_u16*)smem, ltid);
            }
        } else if (phase == 1) {
            if (live) {
                int ti, tj;
                sym_tile(tile, bk.tm, ti, tj);
                jb.P = make_rsrc(As, abytes);
                jb.Q = jb.P;
                jb.X = jb.P;
                jb.ldp = jb.ldq = jb.ldx = jb.ldo = bk.m;
                jb.K = bk.m;
                jb.i0 = ti * kTile;
                jb.j0 = tj * kTile;
                jb.out = Bs;
                jb.mirror = ti != tj;
                jb.alpha = p.coef[t][2];
                jb.beta = p.coef[t][1];
                gemm_tile<true, true, EPI_POLY, C, POL_SC1, C::PAHEAD && kQAheadPoly>(jb, (lds_u16*)smem, ltid);
            }
        } else {
            // wide: X' (m x n) = a*X + B X;  tall: G' (n x m) = a*G + G B
            const int nt_cols = tall ? bk.tm : bk.tn;
            const int ti = tile / nt_cols, tj = tile - ti * nt_cols;
            const int ld = tall ? bk.m : bk.n;
            uint16_t* os = xout + (int64_t)slot * bk.slot;
            if (live) {
                const i32x4 rx = make_rsrc(xs, xbytes);
                const i32x4 rb = make_rsrc(Bs, abytes);
                jb.P = tall ? rx : rb;
                jb.Q = tall ? rb : rx;
                jb.X = rx;
                jb.ldp = bk.m;
                jb.ldq = tall ? bk.m : bk.n;
                jb.ldx = jb.ldo = ld;
                jb.K = bk.m;
                jb.i0 = ti * kTile;
                jb.j0 = tj * kTile;
                jb.out = os;
                jb.mirror = false;
                jb.beta = p.coef[t][0];
                if (t == 0) jb.sig = bk.scale[slot];
                if (tall) gemm_tile<true, true, EPI_UPDATE, C, POL_SC1>(jb, (lds_u16*)smem, ltid);
                else gemm_tile<true, false, EPI_UPDATE, C, POL_SC1, C::PAHEAD && kQAheadWideUpdate>(jb, (lds_u16*)smem, ltid);
            } else if (last) {
                // a zero slot's result is exactly zero
                const int i0 = ti * kTile, j0 = tj * kTile;
                for (int v = tid; v < kTile * kTile / 8; v += C::NT) {
                    const int i = v / (kTile / 8), c8 = v % (kTile / 8);
                    *reinterpret_cast<u32x4*>(os + (int64_t)(i0 + i) * ld + j0 + c8 * 8) = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }

        // publish: every store of this workgroup is in the L2 before the counter moves; and claim
        // the next task.  With claim_early the claim goes out while this tile's stores drain, so
        // its round trip and their acknowledgements overlap (and one barrier goes); the next task
        // may wait for this one, and this workgroup moves the counter before it checks the next
        // task's dependency.  Claiming early holds a task back for the length of the drain, which
        // costs a launch whose queues are short (idle workgroups could have started it at once),
        // so those claim after the drain.
        if (p.claim_early) {
            int got = 0;
            if (leader)
                got = __hip_atomic_fetch_add(p.heads + q, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (leader) s_task = __builtin_amdgcn_readfirstlane(got);
            __syncthreads();
            if (leader) __hip_atomic_fetch_add(ctr, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (leader) {
                __hip_atomic_fetch_add(ctr, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_task = __builtin_amdgcn_readfirstlane(
                    __hip_atomic_fetch_add(p.heads + q, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            }
            __syncthreads();
        }
        idx = __builtin_amdgcn_readfirstlane(s_task);
    }

    // every claim of this workgroup is made; the last workgroup out checks that each queue's head
    // passed its task count (claimed tasks always run, so a queue is drained exactly when it did)
    if (leader) {
        const int out = __builtin_amdgcn_readfirstlane(
            __hip_atomic_fetch_add(p.exits, one, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT));
        if (out == (int)gridDim.x - 1) {
            bool short_ = false;
            for (int qq = 0; qq < p.nq; ++qq)
                short_ |= __builtin_amdgcn_readfirstlane(ld_relaxed(p.heads + qq)) < p.steps * p.per_round[qq];
            if (short_) {
                __hip_atomic_store(p.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&g_persist_fault, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            }
        }
    }
}

struct DeviceShape {
    int cus = 0, xccs = 0;
    bool understood = false;    // one queue per XCD is possible: 1..kMaxQueues XCDs of equal CU count
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
        // a layout outside this (one queue for several L2s would hand intermediate results between
        // non-coherent caches) runs the per-contraction path instead
        d.understood = d.xccs >= 1 && d.xccs <= kMaxQueues && d.cus > 0 && d.cus % d.xccs == 0;
        cached = d;
        cached_dev = dev;
    }
    *out = cached;
    return hipSuccess;
}

}  // namespace

void ns_persist_test_faults(uint64_t wait_cap_ticks, int extra_queues) {
    g_test_wait_cap.store(wait_cap_ticks);
    g_test_extra_queues.store(extra_queues);
}

hipError_t ns_persist_fault(int* flag, bool clear) {
    hipError_t e = hipMemcpyFromSymbol(flag, HIP_SYMBOL(g_persist_fault), sizeof(int), 0, hipMemcpyDeviceToHost);
    if (e != hipSuccess || !clear || *flag == 0) return e;
    const int zero = 0;
    return hipMemcpyToSymbol(HIP_SYMBOL(g_persist_fault), &zero, sizeof(int), 0, hipMemcpyHostToDevice);
}

bool ns_persist_check(const NsPersistBank* banks, int nbanks, int tile, int steps, int nq, char* why, size_t why_len) {
    auto bad = [&](const char* fmt, int a, int b2, int c) {
        if (why && why_len) snprintf(why, why_len, fmt, a, b2, c);
        return false;
    };
    if (nbanks < 1 || nbanks > kMaxPersistBanks || (tile != 256 && tile != 128) || steps < 1 || steps > kMaxRounds ||
        nq < 1 || nq > kMaxQueues)
        return bad("launch arguments out of range (banks %d, tile %d, queues %d)", nbanks, tile, nq);
    PersistArgs p;
    fill_persist_args(p, banks, nbanks, tile, nullptr, steps, nq, nullptr);
    // seen[b][(slot * steps + t) * chain + position in the round's chain]
    std::vector<std::vector<unsigned char>> seen((size_t)nbanks);
    std::vector<std::vector<int>> count((size_t)nbanks);
    for (int b = 0; b < nbanks; ++b) {
        const PersistBank& k = p.bank[b];
        if (k.tm < 1 || k.tn < 1 || k.m % tile || k.n % tile) return bad("bank %d: sides not multiples of the tile %d%c", b, tile, ' ');
        const int chain = 2 * sym_count(k.tm) + k.tm * k.tn;
        seen[(size_t)b].assign((size_t)k.batch * steps * chain, 0);
        count[(size_t)b].assign((size_t)k.batch, 0);
    }
    for (int q = 0; q < nq; ++q) {
        const int total = steps * p.per_round[q];
        for (int idx = 0; idx < total; ++idx) {
            const PersistTask k = decode_task(p, q, idx);
            if (k.b < 0 || k.b >= nbanks) return bad("queue %d position %d: bank %d out of range", q, idx, k.b);
            const PersistBank& bk = p.bank[k.b];
            if (k.slot < 0 || k.slot >= bk.batch) return bad("queue %d position %d: slot %d out of range", q, idx, k.slot);
            if ((bk.base + k.slot) % nq != q) return bad("queue %d position %d: slot %d belongs to another queue", q, idx, k.slot);
            const int nG = sym_count(bk.tm), chain = 2 * nG + bk.tm * bk.tn;
            const int ntile = k.phase == 2 ? bk.tm * bk.tn : nG;
            if (k.t < 0 || k.t >= steps || k.phase < 0 || k.phase > 2 || k.tile < 0 || k.tile >= ntile)
                return bad("queue %d position %d: round, contraction or tile %d out of range", q, idx, k.tile);
            const int pos = k.t * chain + (k.phase == 0 ? 0 : k.phase == 1 ? nG : 2 * nG) + k.tile;
            unsigned char& mark = seen[(size_t)k.b][(size_t)k.slot * steps * chain + pos];
            if (mark) return bad("queue %d position %d: a task of slot %d listed twice", q, idx, k.slot);
            mark = 1;
            // the slot's tasks come in chain order, so everything this task waits for (need tasks) was
            // listed, and therefore claimed, before it on the same queue
            int& c = count[(size_t)k.b][(size_t)k.slot];
            if (pos != c || k.need > pos || k.need != pos - k.tile)
                return bad("queue %d position %d: slot %d out of chain order", q, idx, k.slot);
            ++c;
        }
    }
    for (int b = 0; b < nbanks; ++b)
        for (size_t i = 0; i < seen[(size_t)b].size(); ++i)
            if (!seen[(size_t)b][i]) return bad("bank %d: task %d of the chains never listed%c", b, (int)i, ' ');
    return true;
}

bool ns_persist_supported() {
    DeviceShape d;
    return device_shape(&d) == hipSuccess && d.understood;
}

bool ns_persist_fits256(int64_t rows, int64_t cols) {
    const int64_t m = rows < cols ? rows : cols, n = rows < cols ? cols : rows;
    // a 256-sided Gram is a single 256-tile, so each contraction would be one task per slot: 128-tiles
    // give four (three for the symmetric ones) and a chain of shorter tasks (four 256^2 slots: -24 % per step)
    return m % 256 == 0 && n % 256 == 0 && m >= 512;
}

int ns_persist_tile(int64_t rows, int64_t cols, int steps, int64_t slots) {
    const int64_t m = rows < cols ? rows : cols, n = rows < cols ? cols : rows;
    if (steps < 1 || steps > kMaxRounds || m * n > ((int64_t)1 << 30) || m * m > ((int64_t)1 << 30)) return 0;
    // 256-tiles need more than one slot per XCD (8 on gfx950): with one or none, a slot's chain of 256-tile
    // tasks (six to nine per contraction for an XCD's 32 CUs) sets the launch time, and 128-tiles, four
    // times as many tasks of a quarter of the work, shorten it (8 slots of 768^2, 3072 x 768, 1024^2:
    // -13 %, -14 %, -5 %; from 10 slots on 256-tiles are faster on all three, 768^2: 387 against 423 us)
    if (ns_persist_fits256(rows, cols) && slots >= kMinSlots256) return 256;
    if (m % 128 == 0 && n % 128 == 0) return 128;
    return 0;
}

// A 128-tile launch whose slots' long side is at most 768 runs one 16-wavefront workgroup per CU (its tasks
// are short); longer ones two 4-wavefront workgroups per CU.
static bool short128(const PersistArgs& p) {
    int nmax = 0;
    for (int b = 0; b < p.nbanks; ++b) nmax = p.bank[b].n > nmax ? p.bank[b].n : nmax;
    return nmax <= 768;
}

static PersistLaunch launch_of(const PersistArgs& p, const NsPersistBank* banks, int nbanks, int tile, int cus,
                               int xccs) {
    PersistLaunch l{};
    if (tile == 256) {
        // one 16-wavefront workgroup per CU; the three-slot ring (160 KiB) when the launch's X alone is
        // well beyond what the MALL keeps between a slot's contractions, the two-stage one (128 KiB)
        // otherwise (350M banks, 708 MB of X: 3 % faster; attention bank, 47 MB: 2 % slower)
        int64_t xbytes = 0;
        for (int b = 0; b < nbanks; ++b) xbytes += (int64_t)banks[b].batch * banks[b].rows * banks[b].cols * 2;
        l.ring = xbytes >= kAheadMinBytes ? 3 : 2;
        l.wavefronts = Cfg256::NW;
        l.wg_per_queue = cus / xccs;
    } else if (short128(p)) {
        // short contractions: one 16-wavefront workgroup per CU finishes each task sooner (four 256^2
        // slots -16 %, six 384^2 -20 %, five 768^2 -2 %; all bit-identical)
        l.ring = 2;
        l.wavefronts = Cfg128w16::NW;
        l.wg_per_queue = cus / xccs;
    } else {
        // two 4-wavefront workgroups per CU (three 3072 x 768 slots: 9 % faster than 16 wavefronts, eight
        // 1024^2: 15 %)
        l.ring = 2;
        l.wavefronts = Cfg128::NW;
        l.wg_per_queue = 2 * cus / xccs;
    }
    // claim early only when every queue holds at least kEarlyClaimDepth rounds of tasks for its
    // workgroups (350M banks: -4.5 %; four 256^2 slots, one per XCD: +24 % when claiming early)
    int min_round = 1 << 30;
    for (int q = 0; q < p.nq; ++q) min_round = p.per_round[q] < min_round ? p.per_round[q] : min_round;
    l.claim_early = min_round >= kEarlyClaimDepth * l.wg_per_queue ? 1 : 0;
    return l;
}

PersistLaunch ns_persist_launch(const NsPersistBank* banks, int nbanks, int tile, int steps, int cus, int xccs) {
    PersistArgs p{};
    fill_persist_args(p, banks, nbanks, tile, nullptr, steps, xccs, nullptr);
    return launch_of(p, banks, nbanks, tile, cus, xccs);
}

hipError_t ns_persist(const NsPersistBank* banks, int nbanks, int tile, const NsCoef* coef, int steps, int* sync,
                      hipStream_t stream) {
    if (nbanks < 1 || nbanks > kMaxPersistBanks || (tile != 256 && tile != 128) || steps < 1 || steps > kMaxRounds)
        return hipErrorInvalidValue;
    DeviceShape d;
    hipError_t e = device_shape(&d);
    if (e != hipSuccess) return e;
    if (!d.understood) return hipErrorNotSupported;
    // (the test hook's extra queues take the slots g with g % nq >= the XCD count: no workgroup serves
    // them, so they never run, nothing waits for them, and the drain check reports them)
    const int nq = d.xccs + g_test_extra_queues.load();
    if (nq > kMaxQueues) return hipErrorInvalidValue;
    PersistArgs p{};
    fill_persist_args(p, banks, nbanks, tile, coef, steps, nq, sync);
    const PersistLaunch l = launch_of(p, banks, nbanks, tile, d.cus, d.xccs);
    p.claim_early = l.claim_early;
    const uint64_t cap = g_test_wait_cap.load();
    p.wait_cap = cap ? cap : kWaitCapTicks;
    const dim3 grid((unsigned)(l.wg_per_queue * d.xccs));
    if (tile == 256 && l.ring == 3)
        ns_persist_kernel<Cfg256><<<grid, Cfg256::NT, 0, stream>>>(p);
    else if (tile == 256)
        ns_persist_kernel<Cfg256r2><<<grid, Cfg256r2::NT, 0, stream>>>(p);
    else if (l.wavefronts == Cfg128w16::NW)
        ns_persist_kernel<Cfg128w16><<<grid, Cfg128w16::NT, 0, stream>>>(p);
    else
        ns_persist_kernel<Cfg128><<<grid, Cfg128::NT, 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace mb
