// The task list of the persistent Newton-Schulz launch: its arguments, how they are filled on the
// host, and how a queue position decodes to a task (shared by the kernel and a host-side check of the
// plan, so that what the check verifies is what the kernel runs).
//
// A launch carries up to kMaxPersistBanks banks whose slots are numbered in one sequence; slot g runs
// on queue g % nq (one queue per XCD).  A queue lists its tasks round by round; within a round the
// Gram tiles of all its slots, then the polynomial tiles, then the update tiles; within a contraction
// bank by bank, slot by slot, tile by tile.  Symmetric contractions have one task per upper-triangle
// tile (tm(tm+1)/2), the update one per output tile (tm * tn).
#pragma once

#include <stdint.h>

#include "kernels.hpp"

namespace mb {

constexpr int kMaxQueues = 16;

struct PersistBank {
    const uint16_t* x0;     // round input of round 0 (unscaled)
    const uint16_t* xpre;   // round input of round 0 for pre-scaled slots (their live word says which)
    uint16_t* xa;           // outputs of rounds 0, 2, 4, ... (except the last)
    uint16_t* xb;           // outputs of rounds 1, 3, 5, ...
    uint16_t* dest;         // output of the last round
    uint16_t* A;
    uint16_t* Bm;
    const float* scale;
    const int* live;
    int64_t slot;           // elements per slot of X
    int64_t mm;             // elements per slot of A, B
    int m, n;               // Gram size and long side (m <= n)
    int tm, tn;             // tiles along m and along n
    int batch;
    int base;               // number of the bank's first slot in the launch's slot sequence
    int tall;
};

struct PersistArgs {
    PersistBank bank[kMaxPersistBanks];
    int nbanks, steps, nq;
    int* heads;             // [nq] next task of each queue
    int* err;               // set when a dependency wait hits its time cap or a queue is left undrained
    int* exits;             // workgroups that have left the task loop
    int* ctr;               // [total slots] tasks finished per slot
    // per queue: tasks of one round, of its Gram block and of its polynomial block, and the
    // number of slots of each bank on the queue
    int per_round[kMaxQueues], blk_g[kMaxQueues], blk_p[kMaxQueues];
    int ls[kMaxQueues][kMaxPersistBanks];
    float coef[kMaxRounds][3];   // (a, b, c) of each round
    int claim_early;        // claim the next task while a finished tile's stores drain (set at launch)
    uint64_t wait_cap;      // constant-clock ticks after which a dependency wait gives up (set at launch)
};

__host__ __device__ __forceinline__ int sym_count(int tm) { return tm * (tm + 1) / 2; }

// The bank's first slot (in its own numbering) on queue q.
__host__ __device__ __forceinline__ int first_slot_on(const PersistArgs& p, const PersistBank& bk, int q) {
    return ((q - bk.base) % p.nq + p.nq) % p.nq;
}

struct PersistTask {
    int t;          // round
    int phase;      // 0 Gram, 1 polynomial, 2 update
    int b;          // bank
    int slot;       // slot within the bank
    int tile;       // upper-triangle tile (phases 0, 1) or row-major output tile (phase 2)
    int need;       // tasks of this slot that must have finished first: every task of its earlier contractions
};

// Queue q's task at position idx (0 <= idx < steps * per_round[q]).
__host__ __device__ __forceinline__ PersistTask decode_task(const PersistArgs& p, int q, int idx) {
    PersistTask k;
    k.t = idx / p.per_round[q];
    int r = idx - k.t * p.per_round[q];
    if (r < p.blk_g[q]) k.phase = 0;
    else if ((r -= p.blk_g[q]) < p.blk_p[q]) k.phase = 1;
    else { r -= p.blk_p[q]; k.phase = 2; }
    int b = 0, ntile = 1;
    for (; b < p.nbanks - 1; ++b) {
        ntile = k.phase == 2 ? p.bank[b].tm * p.bank[b].tn : sym_count(p.bank[b].tm);
        const int cnt = p.ls[q][b] * ntile;
        if (r < cnt) break;
        r -= cnt;
    }
    const PersistBank& bk = p.bank[b];
    ntile = k.phase == 2 ? bk.tm * bk.tn : sym_count(bk.tm);
    const int l = r / ntile;
    k.b = b;
    k.tile = r - l * ntile;
    k.slot = first_slot_on(p, bk, q) + l * p.nq;
    const int nG = sym_count(bk.tm);
    const int chain = 2 * nG + bk.tm * bk.tn;                      // tasks per slot and round
    k.need = k.t * chain + (k.phase == 0 ? 0 : k.phase == 1 ? nG : 2 * nG);
    return k;
}

// The launch's arguments for these banks, `tile`-sided tiles and nq queues (sync as in ns_persist;
// the plan check passes NULL).
inline void fill_persist_args(PersistArgs& p, const NsPersistBank* banks, int nbanks, int tile, const NsCoef* coef,
                              int steps, int nq, int* sync) {
    p = PersistArgs{};
    p.nbanks = nbanks;
    p.steps = steps;
    p.nq = nq;
    p.heads = sync;
    p.err = sync ? sync + 16 : nullptr;
    p.exits = sync ? sync + 17 : nullptr;
    p.ctr = sync ? sync + 32 : nullptr;
    int base = 0;
    for (int b = 0; b < nbanks; ++b) {
        const NsPersistBank& r = banks[b];
        PersistBank& k = p.bank[b];
        k.tall = r.rows > r.cols ? 1 : 0;
        k.x0 = r.x0;
        k.xpre = ns_prescale_buffer(r.xa, r.xb, steps);
        k.xa = r.xa;
        k.xb = r.xb;
        k.dest = r.dest;
        k.A = r.A;
        k.Bm = r.Bm;
        k.scale = r.scale;
        k.live = r.live;
        k.slot = r.rows * r.cols;
        k.m = (int)(k.tall ? r.cols : r.rows);
        k.n = (int)(k.tall ? r.rows : r.cols);
        k.mm = (int64_t)k.m * k.m;
        k.tm = k.m / tile;
        k.tn = k.n / tile;
        k.batch = (int)r.batch;
        k.base = base;
        base += k.batch;
    }
    for (int q = 0; q < nq; ++q) {
        int g = 0, pp = 0, u = 0;
        for (int b = 0; b < nbanks; ++b) {
            const PersistBank& k = p.bank[b];
            const int first = first_slot_on(p, k, q);
            const int ls = first < k.batch ? (k.batch - first + nq - 1) / nq : 0;
            p.ls[q][b] = ls;
            g += ls * sym_count(k.tm);
            pp += ls * sym_count(k.tm);
            u += ls * k.tm * k.tn;
        }
        p.blk_g[q] = g;
        p.blk_p[q] = pp;
        p.per_round[q] = g + pp + u;
    }
    for (int t = 0; t < steps && coef; ++t) {
        p.coef[t][0] = coef[t].a;
        p.coef[t][1] = coef[t].b;
        p.coef[t][2] = coef[t].c;
    }
}

}  // namespace mb
