// Host-side launchers of the gfx950 kernels (implemented in stream_kernels.hip
// and ns_gemm.hip), used by the C ABI in muonbank.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mb {

// Brackets kernel launches with events when kernel timing is on.
struct RoundTimer {
    virtual void begin(const char* name, hipStream_t stream) = 0;
    virtual void end(hipStream_t stream) = 0;
    virtual ~RoundTimer() = default;
};

// Elements per workgroup of the streaming kernels (and per partial sum of u^2): two 8-element groups
// per thread of 256, so that many short workgroups are in flight (16384 per workgroup measured 9 %
// slower for momentum, 4 % for the apply).
constexpr int64_t kStreamChunk = 4096;
constexpr int kStreamGroups = (int)(kStreamChunk / (256 * 8));   // 8-element groups per thread and chunk
// Banks per launch of the streaming kernels (momentum, scale, apply); more take several launches.
constexpr int kMaxStreamBanks = 16;
int stream_chunks(int64_t slot_numel);

// buf' and u of one bank (and, if partials is non-null, per-(slot, chunk) sums of u^2 in binary64).
// slot_base: the bank's first row in the call's per-slot scalar table.
struct MomentumBank {
    const void* grad;
    void* buf;
    uint16_t* u;
    double* partials;
    int64_t batch, slot_numel;
    bool f32;
    float mu, nu;
    int slot_base;
};
// Momentum of several banks, one launch per kMaxStreamBanks.  slot_scalars: NULL, or a device table
// of 4 floats (mu, nu, decay, eta) per slot of the call, whose mu and nu replace the banks' own.
hipError_t launch_momentum(const MomentumBank* banks, int nbanks, const float* slot_scalars, hipStream_t stream);

// The mixed-precision apply on one bank [batch, slot_numel]: eta per slot is eta, or
// RN32(eta * lr_mul_per_slot[i]), or (with a scalar table) the table's eta; decay likewise.
struct ApplyBank {
    uint16_t* w_hi;
    uint16_t* w_lo;
    const uint16_t* v;
    const float* lr_mul_per_slot;
    int64_t batch, slot_numel;
    float eta, decay;
    int slot_base;
};
hipError_t launch_apply(const ApplyBank* banks, int nbanks, const float* slot_scalars, hipStream_t stream);

// Per-(slot, chunk) sums of x^2 of a bf16 bank, in binary64.
hipError_t launch_sumsq(const uint16_t* x, double* partials, int64_t batch, int64_t slot_numel, hipStream_t stream);

// Per slot i of one bank, from the sum S of its partials: live[i] = 0 if S == 0 (every element zero),
// else a live word (common.hpp); scale[i] = 1 / (sqrt(S) + eps), or for a pre-scaled slot
// 2^-k / (sqrt(S) + eps) with xpre's slot i = x0's slot i * 2^k.  Also clears, if non-null, heads[0, 32)
// (queue heads, error word and exit count of a persistent launch) and ctr[i].  first_slot is set by
// the launcher.
struct ScaleBank {
    const double* partials;
    int nchunks;
    int64_t batch;
    float* scale;
    int* live;
    int* heads;
    int* ctr;
    const uint16_t* x0;
    uint16_t* xpre;
    int64_t slot_numel;
    int first_slot;
};
hipError_t launch_ns_scale(const ScaleBank* banks, int nbanks, double eps, hipStream_t stream);

// One Newton-Schulz round on a bank: x_out = round(x_in), with A and Bm as scratch.
struct NsRound {
    const uint16_t* x_in;
    uint16_t* x_out;
    uint16_t* A;
    uint16_t* Bm;
    int64_t batch, rows, cols;
    float a, b, c;
    bool first;            // apply the Frobenius scale (x_in is the unscaled input)
    const float* scale;
    const int* live;
    const uint16_t* x_pre; // first round: pre-scaled slots read X from here instead of x_in
};
hipError_t ns_round(const NsRound& r, hipStream_t stream, RoundTimer* timer);

// Where the pre-scaled copy of a slot's first-round input goes (see launch_ns_scale): a ping-pong
// buffer that the first round neither writes nor, with a single round, has as its output.
inline uint16_t* ns_prescale_buffer(uint16_t* x1, uint16_t* x2, int steps) { return steps == 1 ? x1 : x2; }

// Coefficients of one Newton-Schulz round, X' = a*X + (b*A + c*A A) X.
struct NsCoef {
    float a, b, c;
};
constexpr int kMaxRounds = 64;

// Every Newton-Schulz round of up to kMaxPersistBanks banks in one persistent launch: per bank
// x0 -> ... -> dest, with xa, xb as ping-pong buffers and A, Bm as scratch; the banks' slots
// are numbered in one sequence in the order given.  sync holds the queue heads ([0, 16)), the
// error word ([16]) and one counter per slot ([32, 32 + total slots)), all cleared before the
// launch (launch_ns_scale does it).
constexpr int kMaxPersistBanks = 8;
constexpr int64_t kMinSlots256 = 9;    // slots a persistent launch needs before it takes 256-tiles
struct NsPersistBank {
    const uint16_t* x0;
    uint16_t* xa;
    uint16_t* xb;
    uint16_t* dest;
    uint16_t* A;
    uint16_t* Bm;
    const float* scale;
    const int* live;
    int64_t batch, rows, cols;
};
// Tile edge the persistent kernel uses for a slot shape (256 or 128), 0 if it cannot run it; `slots` is
// the number of slots of that launch whose shape would take 256-tiles.
int ns_persist_tile(int64_t rows, int64_t cols, int steps, int64_t slots);
// Whether the current device's XCD layout allows the persistent launch (else it returns
// hipErrorNotSupported and callers take one launch per contraction).
bool ns_persist_supported();
// Whether a slot shape may take 256-tiles at all.
bool ns_persist_fits256(int64_t rows, int64_t cols);
hipError_t ns_persist(const NsPersistBank* banks, int nbanks, int tile, const NsCoef* coef, int steps, int* sync,
                      hipStream_t stream);
// How a persistent launch runs on a device of `cus` compute units in `xccs` XCDs: the ring of its
// tiles (slots of the operand copied ahead: 3 for the 256-tiles of launches whose X is at least
// 128 MiB, else 2), its workgroups per XCD queue, its wavefronts per workgroup, and whether its
// workgroups claim their next task while a finished tile's stores drain.
struct PersistLaunch {
    int ring, wg_per_queue, wavefronts, claim_early;
};
PersistLaunch ns_persist_launch(const NsPersistBank* banks, int nbanks, int tile, int steps, int cus, int xccs);
// Host check of one persistent launch's task lists with nq queues, by the kernel's own decode: every
// task of every slot's chains listed exactly once, on its slot's queue, each after every task it waits
// for.  On failure returns false with a reason in why.
bool ns_persist_check(const NsPersistBank* banks, int nbanks, int tile, int steps, int nq, char* why, size_t why_len);
// The current device's persistent-launch fault flag (1: a dependency wait hit its time cap since the
// flag was last cleared); blocking; clears it when `clear` is set.
hipError_t ns_persist_fault(int* flag, bool clear);
// Test hook for the failure paths of the persistent launch: a dependency-wait cap in constant-clock ticks
// (0: the default 200 ms) and a number of extra queues that no XCD serves (0: none).  Process-wide.
void ns_persist_test_faults(uint64_t wait_cap_ticks, int extra_queues);

// Every Newton-Schulz round of banks of small slots (Gram side <= 64, <= 4096 elements) in one launch
// per kMaxSmallBanks banks, one workgroup per slot (x0 -> dest; dest may equal x0).
constexpr int kMaxSmallBanks = 8;
struct NsSmall {
    const uint16_t* x0;
    uint16_t* dest;
    const float* scale;
    const int* live;
    int64_t batch, rows, cols;
};
bool ns_small_eligible(int64_t rows, int64_t cols, int steps);
hipError_t ns_small(const NsSmall* banks, int nbanks, int steps, const NsCoef* coef, hipStream_t stream);

// dst [cols, rows] = src^T (add: dst += src^T, one rounding), elements of 2 or 4 bytes.
hipError_t launch_transpose(void* dst, const void* src, int64_t rows, int64_t cols, int elem_bytes, bool add,
                            hipStream_t stream);

}  // namespace mb
