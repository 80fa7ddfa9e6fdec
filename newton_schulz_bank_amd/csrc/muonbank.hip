// C ABI of libmuonbank.so: argument validation, host scalars, workspace
// layout and the launch sequence of the Muon bank step on one HIP stream.
// The operations are stated in include/muonbank.h.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "muonbank.h"

namespace {

thread_local std::string g_last_error;

mb_status fail(mb_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mb_status fail(mb_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

mb_status ok() {
    g_last_error.clear();
    return MB_OK;
}

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------

struct TimedLaunch {
    std::string name;
    hipEvent_t start, stop;
};

std::mutex g_timing_mu;
std::atomic<bool> g_timing_on{false};   // read without the lock by every launch
std::vector<TimedLaunch> g_timed;
// Events are pooled: created when timing is switched on (and on demand), handed back by
// mb_timing_read, so a timed loop records events without creating any.
std::vector<hipEvent_t> g_event_pool;
constexpr size_t kEventPoolInit = 16384;

bool take_event(hipEvent_t* e) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (!g_event_pool.empty()) {
        *e = g_event_pool.back();
        g_event_pool.pop_back();
        return true;
    }
    return hipEventCreate(e) == hipSuccess;
}

struct Timer final : mb::RoundTimer {
    TimedLaunch cur;
    bool open = false;
    void begin(const char* name, hipStream_t stream) override {
        if (!g_timing_on) return;
        cur.name = name;
        if (!take_event(&cur.start)) return;
        if (!take_event(&cur.stop)) {
            std::lock_guard<std::mutex> lk(g_timing_mu);
            g_event_pool.push_back(cur.start);
            return;
        }
        (void)hipEventRecord(cur.start, stream);
        open = true;
    }
    void end(hipStream_t stream) override {
        if (!open) return;
        (void)hipEventRecord(cur.stop, stream);
        std::lock_guard<std::mutex> lk(g_timing_mu);
        g_timed.push_back(cur);
        open = false;
    }
};

// ---------------------------------------------------------------------------
// validation helpers
// ---------------------------------------------------------------------------

constexpr int64_t kMaxBatch = 65535;          // grid y dimension
constexpr int64_t kMaxDim = (int64_t)1 << 30;   // rows, cols fit int with tile padding

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

mb_status check_shape(int64_t batch, int64_t rows, int64_t cols, const char* what) {
    if (batch <= 0 || rows <= 0 || cols <= 0)
        return fail(MB_ERR_SHAPE, "%s: batch, rows and cols must be positive (got %lld, %lld, %lld)", what,
                    (long long)batch, (long long)rows, (long long)cols);
    if (batch > kMaxBatch || rows > kMaxDim || cols > kMaxDim)
        return fail(MB_ERR_SHAPE, "%s: shape (%lld, %lld, %lld) beyond the supported range (batch <= %lld, dims <= 2^30)",
                    what, (long long)batch, (long long)rows, (long long)cols, (long long)kMaxBatch);
    const int64_t slot = rows * cols;      // < 2^60
    if (slot > ((int64_t)1 << 62) / batch)
        return fail(MB_ERR_SHAPE, "%s: element count overflows", what);
    // the contraction grids enumerate batch x 128x128 output tiles in 32-bit indices
    const int64_t m = rows < cols ? rows : cols, n = rows < cols ? cols : rows;
    const int64_t tiles = ((m + 127) / 128) * ((n + 127) / 128);
    if (tiles > ((int64_t)1 << 30) / batch)
        return fail(MB_ERR_SHAPE, "%s: shape (%lld, %lld, %lld) has too many 128x128 tiles", what, (long long)batch,
                    (long long)rows, (long long)cols);
    return MB_OK;
}

struct Range {
    uintptr_t lo, hi;
    const char* name;
};

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

mb_status check_no_overlap(const std::vector<Range>& rs) {
    for (size_t i = 0; i < rs.size(); ++i)
        for (size_t j = i + 1; j < rs.size(); ++j)
            if (overlap(rs[i], rs[j]))
                return fail(MB_ERR_ALIAS, "buffers %s and %s overlap", rs[i].name, rs[j].name);
    return MB_OK;
}

bool is_finite(double v) { return std::isfinite(v); }

mb_status check_schedule(const double* schedule, int steps, const char* what) {
    for (int i = 0; schedule && i < 3 * steps; ++i)
        if (!is_finite(schedule[i])) return fail(MB_ERR_VALUE, "%s: schedule entry %d is not finite", what, i);
    return MB_OK;
}

mb_status check_hparams(const mb_hparams& hp) {
    if (!is_finite(hp.lr) || !is_finite(hp.weight_decay) || !is_finite(hp.momentum) || !is_finite(hp.a) || !is_finite(hp.b) ||
        !is_finite(hp.c) || !is_finite(hp.eps))
        return fail(MB_ERR_VALUE, "hyper-parameters must be finite");
    if (hp.ns_steps < 1 || hp.ns_steps > mb::kMaxRounds)
        return fail(MB_ERR_VALUE, "ns_steps must be in 1..%d (got %d)", mb::kMaxRounds, hp.ns_steps);
    if (check_schedule(hp.ns_schedule, hp.ns_steps, "hparams") != MB_OK) return MB_ERR_VALUE;
    if (hp.eps < 0) return fail(MB_ERR_VALUE, "eps must be >= 0");
    return MB_OK;
}

size_t round_up(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace of one bank: u, two ping-pong X buffers, A, B, partial sums, scale, live, and the
// persistent kernel's queue heads, error word and slot counters (32 ints + one per slot).
struct BankWs {
    size_t u, x1, x2, A, Bm, partials, scale, live, sync, total;
};

BankWs bank_ws_layout(int64_t batch, int64_t rows, int64_t cols, bool vec) {
    const int64_t m = rows < cols ? rows : cols;
    BankWs w{};
    size_t off = 0;
    const size_t xb = round_up((size_t)(batch * rows * cols) * 2);
    const size_t ab = round_up((size_t)(batch * m * m) * 2);
    w.u = off; off += xb;
    w.x1 = off; off += xb;
    w.x2 = off; off += xb;
    w.A = off; off += ab;
    w.Bm = off; off += ab;
    w.partials = off; off += round_up((size_t)batch * mb::stream_chunks(rows * cols) * 8);
    w.scale = off; off += round_up((size_t)batch * 4);
    w.live = off; off += round_up((size_t)batch * 4);
    w.sync = off; off += round_up((size_t)(32 + batch) * 4);
    w.total = off;
    return w;
}

float f32(double v) { return (float)v; }

// The persistent launches of one muon_bank_step: banks whose slots the persistent kernel can run,
// grouped by tile edge, in chunks of at most kMaxPersistBanks banks.  Each chunk has its own
// sync block (queue heads and error word, then one counter per slot of the chunk) in the step's
// trailing sync region.
struct PersistChunk {
    int tile;
    std::vector<int32_t> banks;
    size_t sync_off;        // ints from the start of the sync region
    std::vector<int> base;  // number of each bank's first slot within the chunk
};

struct StepPlan {
    std::vector<PersistChunk> chunks;
    std::vector<int> chunk_of;     // per bank: its chunk, or -1
    size_t sync_ints = 0;
};

StepPlan plan_step(const mb_bank* banks, int32_t num_banks) {
    StepPlan pl;
    pl.chunk_of.assign((size_t)num_banks, -1);
    // the slots that could take 256-tiles decide together whether they do
    int64_t slots256 = 0;
    for (int32_t i = 0; i < num_banks; ++i)
        if (mb::ns_persist_fits256(banks[i].rows, banks[i].cols)) slots256 += banks[i].batch;
    for (int tile : {256, 128}) {
        PersistChunk cur{tile, {}, 0, {}};
        int slots = 0;
        auto flush = [&]() {
            if (cur.banks.empty()) return;
            cur.sync_off = pl.sync_ints;
            pl.sync_ints += 32 + (size_t)slots;
            for (int32_t bi : cur.banks) pl.chunk_of[(size_t)bi] = (int)pl.chunks.size();
            pl.chunks.push_back(cur);
            cur = PersistChunk{tile, {}, 0, {}};
            slots = 0;
        };
        for (int32_t i = 0; i < num_banks; ++i) {
            if (mb::ns_persist_tile(banks[i].rows, banks[i].cols, 1, slots256) != tile) continue;
            cur.base.push_back(slots);
            cur.banks.push_back(i);
            slots += (int)banks[i].batch;
            if ((int)cur.banks.size() == mb::kMaxPersistBanks) flush();
        }
        flush();
    }
    return pl;
}

// 0: every round of a bank in one persistent launch where the shape allows it; 1: one launch per
// contraction.
std::atomic<int> g_ns_path{0};

// The float32 scalars of one bank, each from double arithmetic rounded once ("Muon Custom Sizing",
// section 4: eff_lr = lr * max(1, rows/cols)^0.5 * lr_mul, eff_wd = lr * wd * wd_mul, and the
// momentum's two lerp weights).
struct BankScalars {
    float mu, nu, decay, eta;
};
BankScalars bank_scalars(const mb_bank& b, const mb_hparams& hp) {
    return {f32(hp.momentum), f32(1.0 - hp.momentum), f32(1.0 - hp.lr * hp.weight_decay * b.wd_mul),
            f32(hp.lr * std::sqrt(std::max(1.0, (double)b.rows / (double)b.cols)) * b.lr_mul)};
}

// Newton-Schulz rounds on scaled input: x_first -> ... -> dest.  x1, x2 are ping-pong buffers
// distinct from x_first and dest; sync (cleared by the ns_scale launch) serves the persistent
// kernel.
// The per-round coefficients, each rounded once to float32: the schedule (3*steps doubles) if
// given, else (a, b, c) in every round.
std::vector<mb::NsCoef> ns_coefs(int steps, double a, double b, double c, const double* schedule) {
    std::vector<mb::NsCoef> v((size_t)steps);
    for (int t = 0; t < steps; ++t)
        v[(size_t)t] = schedule ? mb::NsCoef{f32(schedule[3 * t]), f32(schedule[3 * t + 1]), f32(schedule[3 * t + 2])}
                                : mb::NsCoef{f32(a), f32(b), f32(c)};
    return v;
}

// Whether this call may use the persistent launch: the process-wide path setting and the device's XCD
// layout (see mb_ns_set_path).
bool persist_path() { return g_ns_path.load() == 0 && mb::ns_persist_supported(); }

mb_status run_ns(const uint16_t* x_first, uint16_t* dest, uint16_t* x1, uint16_t* x2, uint16_t* A, uint16_t* Bm,
                 int64_t batch, int64_t rows, int64_t cols, const std::vector<mb::NsCoef>& coef,
                 const float* scale, const int* live, int* sync, hipStream_t stream, Timer& timer) {
    const int steps = (int)coef.size();
    const int tile = mb::ns_persist_tile(rows, cols, steps, batch);
    if (tile != 0 && sync && persist_path()) {
        const mb::NsPersistBank r{x_first, x1, x2, dest, A, Bm, scale, live, batch, rows, cols};
        timer.begin("ns_persist", stream);
        hipError_t e = mb::ns_persist(&r, 1, tile, coef.data(), steps, sync, stream);
        timer.end(stream);
        if (e != hipSuccess) return fail(MB_ERR_HIP, "Newton-Schulz launch: %s", hipGetErrorString(e));
        return MB_OK;
    }
    if (g_ns_path.load() == 0 && mb::ns_small_eligible(rows, cols, steps)) {
        const mb::NsSmall r{x_first, dest, scale, live, batch, rows, cols};
        timer.begin("ns_small", stream);
        hipError_t e = mb::ns_small(&r, 1, steps, coef.data(), stream);
        timer.end(stream);
        if (e != hipSuccess) return fail(MB_ERR_HIP, "Newton-Schulz launch: %s", hipGetErrorString(e));
        return MB_OK;
    }
    const uint16_t* in = x_first;
    for (int s = 0; s < steps; ++s) {
        const bool last = s == steps - 1;
        uint16_t* out = last ? dest : ((s & 1) ? x2 : x1);
        const mb::NsCoef& k = coef[(size_t)s];
        mb::NsRound r{in, out, A, Bm, batch, rows, cols, k.a, k.b, k.c, s == 0, scale, live,
                      mb::ns_prescale_buffer(x1, x2, steps)};
        hipError_t e = mb::ns_round(r, stream, &timer);
        if (e != hipSuccess) return fail(MB_ERR_HIP, "Newton-Schulz round %d: %s", s, hipGetErrorString(e));
        in = out;
    }
    return MB_OK;
}

}  // namespace

extern "C" {

void mb_default_hparams(mb_hparams* hp) {
    if (!hp) return;
    hp->lr = 0.02;
    hp->weight_decay = 0.01;
    hp->momentum = 0.95;
    hp->ns_steps = 5;
    hp->a = 3.4445;
    hp->b = -4.7750;
    hp->c = 2.0315;
    hp->eps = 1e-7;
    hp->ns_schedule = nullptr;
    hp->slot_scalars = nullptr;
}

const char* mb_status_string(int32_t s) {
    switch (s) {
        case MB_OK: return "ok";
        case MB_ERR_NULL: return "null pointer";
        case MB_ERR_SHAPE: return "bad shape";
        case MB_ERR_DTYPE: return "bad dtype";
        case MB_ERR_ALIGN: return "misaligned pointer";
        case MB_ERR_WORKSPACE: return "workspace too small";
        case MB_ERR_ALIAS: return "overlapping buffers";
        case MB_ERR_VALUE: return "bad scalar argument";
        case MB_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* mb_last_error(void) { return g_last_error.c_str(); }

const char* mb_version(void) { return "muonbank 0.1 gfx950"; }

size_t mb_ns_workspace_bytes(int64_t batch, int64_t rows, int64_t cols) {
    if (check_shape(batch, rows, cols, "mb_ns_workspace_bytes") != MB_OK) return 0;
    const bool vec = (rows * cols) % 8 == 0;
    return bank_ws_layout(batch, rows, cols, vec).total;
}

mb_status mb_slot_scalars_fill(const mb_bank* banks, int32_t num_banks, const mb_hparams* hp_in, float* host_table,
                               int64_t capacity) {
    if (!banks || !host_table) return fail(MB_ERR_NULL, "mb_slot_scalars_fill: null pointer");
    if (num_banks <= 0 || num_banks > 1024) return fail(MB_ERR_SHAPE, "mb_slot_scalars_fill: num_banks must be in 1..1024");
    mb_hparams hp;
    if (hp_in) hp = *hp_in;
    else mb_default_hparams(&hp);
    mb_status s = check_hparams(hp);
    if (s != MB_OK) return s;
    int64_t slots = 0;
    for (int32_t i = 0; i < num_banks; ++i) {
        const mb_bank& b = banks[i];
        s = check_shape(b.batch, b.rows, b.cols, "mb_slot_scalars_fill");
        if (s != MB_OK) return s;
        if (!is_finite(b.lr_mul) || !is_finite(b.wd_mul)) return fail(MB_ERR_VALUE, "mb_slot_scalars_fill: bank %d multipliers", i);
        if (b.lr_mul_per_slot)
            return fail(MB_ERR_VALUE, "mb_slot_scalars_fill: bank %d has lr_mul_per_slot (a device vector): fold it "
                        "into the table's eta", i);
        slots += b.batch;
    }
    if (capacity < 4 * slots)
        return fail(MB_ERR_WORKSPACE, "mb_slot_scalars_fill: %lld floats needed, %lld given", (long long)(4 * slots),
                    (long long)capacity);
    float* out = host_table;
    for (int32_t i = 0; i < num_banks; ++i) {
        const BankScalars bs = bank_scalars(banks[i], hp);
        for (int64_t k = 0; k < banks[i].batch; ++k, out += 4) {
            out[0] = bs.mu;
            out[1] = bs.nu;
            out[2] = bs.decay;
            out[3] = bs.eta;
        }
    }
    return ok();
}

mb_status mb_step_plan(const mb_bank* banks, int32_t num_banks, const mb_hparams* hp_in, int32_t num_cus,
                       int32_t num_xcds, mb_step_plan_info* out) {
    if (!banks || !out) return fail(MB_ERR_NULL, "mb_step_plan: null pointer");
    if (num_banks <= 0 || num_banks > 1024) return fail(MB_ERR_SHAPE, "mb_step_plan: num_banks must be in 1..1024");
    mb_hparams hp;
    if (hp_in) hp = *hp_in;
    else mb_default_hparams(&hp);
    mb_status s = check_hparams(hp);
    if (s != MB_OK) return s;
    for (int32_t i = 0; i < num_banks; ++i) {
        s = check_shape(banks[i].batch, banks[i].rows, banks[i].cols, "mb_step_plan");
        if (s != MB_OK) return s;
    }
    mb_step_plan_info info{};
    const int groups = (num_banks + mb::kMaxStreamBanks - 1) / mb::kMaxStreamBanks;
    info.momentum = info.ns_scale = info.apply = groups;
    const bool persist = g_ns_path.load() == 0 && num_xcds >= 1 && num_xcds <= 16 && num_cus >= num_xcds &&
                         num_cus % num_xcds == 0;
    const StepPlan plan = plan_step(banks, num_banks);
    int small = 0;
    for (int32_t i = 0; i < num_banks; ++i) {
        const mb_bank& b = banks[i];
        if (hp.ns_steps == 1 && !b.v_out) ++info.copies;
        if (persist && plan.chunk_of[(size_t)i] >= 0) continue;
        if (g_ns_path.load() == 0 && mb::ns_small_eligible(b.rows, b.cols, hp.ns_steps)) ++small;
        else info.ns_per_contraction += 3 * hp.ns_steps;
    }
    info.ns_small = (small + mb::kMaxSmallBanks - 1) / mb::kMaxSmallBanks;
    if (persist) {
        char why[256];
        for (const PersistChunk& c : plan.chunks) {
            std::vector<mb::NsPersistBank> pb;
            for (int32_t i : c.banks)
                pb.push_back({nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, banks[i].batch,
                              banks[i].rows, banks[i].cols});
            if (!mb::ns_persist_check(pb.data(), (int)pb.size(), c.tile, hp.ns_steps, num_xcds, why, sizeof why))
                return fail(MB_ERR_VALUE, "mb_step_plan: persistent launch of %zu banks, %d-tiles: %s", c.banks.size(),
                            c.tile, why);
            const mb::PersistLaunch l = mb::ns_persist_launch(pb.data(), (int)pb.size(), c.tile, hp.ns_steps, num_cus,
                                                              num_xcds);
            if (info.ns_persist < 8) {
                info.persist_tile[info.ns_persist] = c.tile;
                info.persist_ring[info.ns_persist] = l.ring;
                info.persist_workgroups[info.ns_persist] = l.wg_per_queue * num_xcds;
                info.persist_claim_early[info.ns_persist] = l.claim_early;
            }
            ++info.ns_persist;
        }
    }
    info.total = info.momentum + info.ns_scale + info.ns_persist + info.ns_small + info.ns_per_contraction + info.apply;
    *out = info;
    return ok();
}

size_t mb_step_workspace_bytes(const mb_bank* banks, int32_t num_banks) {
    if (!banks || num_banks <= 0) return 0;
    size_t total = 0;
    for (int32_t i = 0; i < num_banks; ++i) {
        const mb_bank& b = banks[i];
        if (check_shape(b.batch, b.rows, b.cols, "mb_step_workspace_bytes") != MB_OK) return 0;
        total += bank_ws_layout(b.batch, b.rows, b.cols, (b.rows * b.cols) % 8 == 0).total;
    }
    total += round_up(plan_step(banks, num_banks).sync_ints * 4);
    return total;
}

mb_status muon_momentum_update(const void* grad, void* momentum, uint16_t* u_out, int64_t batch, int64_t rows,
                               int64_t cols, int32_t dtype, float mu, float nu, void* stream) {
    if (!grad || !momentum || !u_out) return fail(MB_ERR_NULL, "muon_momentum_update: null tensor pointer");
    mb_status s = check_shape(batch, rows, cols, "muon_momentum_update");
    if (s != MB_OK) return s;
    if (dtype != MB_F32 && dtype != MB_BF16) return fail(MB_ERR_DTYPE, "muon_momentum_update: dtype %d", dtype);
    if (!aligned16(grad) || !aligned16(momentum) || !aligned16(u_out))
        return fail(MB_ERR_ALIGN, "muon_momentum_update: tensors must be 16-byte aligned");
    if (!std::isfinite(mu) || !std::isfinite(nu)) return fail(MB_ERR_VALUE, "muon_momentum_update: mu, nu must be finite");
    const int64_t n = batch * rows * cols;
    const size_t es = dtype == MB_F32 ? 4 : 2;
    s = check_no_overlap({{(uintptr_t)grad, (uintptr_t)grad + n * es, "grad"},
                          {(uintptr_t)momentum, (uintptr_t)momentum + n * es, "momentum"},
                          {(uintptr_t)u_out, (uintptr_t)u_out + n * 2, "u_out"}});
    if (s != MB_OK) return s;
    Timer timer;
    timer.begin("momentum", (hipStream_t)stream);
    const mb::MomentumBank mbk{grad, momentum, u_out, nullptr, batch, rows * cols, dtype == MB_F32, mu, nu, 0};
    hipError_t e = mb::launch_momentum(&mbk, 1, nullptr, (hipStream_t)stream);
    timer.end((hipStream_t)stream);
    if (e != hipSuccess) return fail(MB_ERR_HIP, "momentum launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

namespace {

mb_status ns_orthogonalize_impl(const uint16_t* x, uint16_t* y, int64_t batch, int64_t rows, int64_t cols,
                                int32_t steps, double a, double b, double c, const double* schedule, double eps,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !y) return fail(MB_ERR_NULL, "ns_orthogonalize_batched: null tensor pointer");
    mb_status s = check_shape(batch, rows, cols, "ns_orthogonalize_batched");
    if (s != MB_OK) return s;
    if (!aligned16(x) || !aligned16(y) || (workspace && !aligned16(workspace)))
        return fail(MB_ERR_ALIGN, "ns_orthogonalize_batched: pointers must be 16-byte aligned");
    if (steps < 1 || steps > mb::kMaxRounds)
        return fail(MB_ERR_VALUE, "ns_orthogonalize_batched: steps must be in 1..%d", mb::kMaxRounds);
    if (!is_finite(a) || !is_finite(b) || !is_finite(c) || !is_finite(eps) || eps < 0)
        return fail(MB_ERR_VALUE, "ns_orthogonalize_batched: coefficients must be finite and eps >= 0");
    if (check_schedule(schedule, steps, "ns_orthogonalize_batched") != MB_OK) return MB_ERR_VALUE;
    const bool vec = (rows * cols) % 8 == 0;
    const BankWs L = bank_ws_layout(batch, rows, cols, vec);
    if (!workspace || workspace_bytes < L.total)
        return fail(MB_ERR_WORKSPACE, "ns_orthogonalize_batched: workspace of %zu bytes needed, %zu given", L.total,
                    workspace ? workspace_bytes : (size_t)0);
    const int64_t n = batch * rows * cols;
    const Range rx{(uintptr_t)x, (uintptr_t)x + n * 2, "x"};
    const Range ry{(uintptr_t)y, (uintptr_t)y + n * 2, "y"};
    const Range rw{(uintptr_t)workspace, (uintptr_t)workspace + L.total, "workspace"};
    if (x != y) {
        s = check_no_overlap({rx, ry, rw});
    } else {
        s = check_no_overlap({rx, rw});
    }
    if (s != MB_OK) return s;

    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    double* partials = (double*)(ws + L.partials);
    float* scale = (float*)(ws + L.scale);
    int* live = (int*)(ws + L.live);
    uint16_t* x1 = (uint16_t*)(ws + L.x1);
    uint16_t* x2 = (uint16_t*)(ws + L.x2);
    Timer timer;
    timer.begin("sumsq", st);
    hipError_t e = mb::launch_sumsq(x, partials, batch, rows * cols, st);
    timer.end(st);
    if (e != hipSuccess) return fail(MB_ERR_HIP, "sumsq launch: %s", hipGetErrorString(e));
    timer.begin("ns_scale", st);
    int* sync = (int*)(ws + L.sync);
    const mb::ScaleBank sb{partials, mb::stream_chunks(rows * cols), batch, scale, live, sync, sync + 32, x,
                           mb::ns_prescale_buffer(x1, x2, steps), rows * cols, 0};
    e = mb::launch_ns_scale(&sb, 1, eps, st);
    timer.end(st);
    if (e != hipSuccess) return fail(MB_ERR_HIP, "ns_scale launch: %s", hipGetErrorString(e));
    // in place with a single round: write the round to scratch, then copy
    uint16_t* dest = (x == y && steps == 1) ? (uint16_t*)(ws + L.u) : y;
    s = run_ns(x, dest, x1, x2, (uint16_t*)(ws + L.A), (uint16_t*)(ws + L.Bm), batch, rows, cols,
               ns_coefs(steps, a, b, c, schedule), scale, live, sync, st, timer);
    if (s != MB_OK) return s;
    if (dest != y) {
        e = hipMemcpyAsync(y, dest, n * 2, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return fail(MB_ERR_HIP, "copy: %s", hipGetErrorString(e));
    }
    return ok();
}

// ---------------------------------------------------------------------------
// the allocation-free variant: its scratch is a static device array
// ---------------------------------------------------------------------------

}  // namespace

// Every device the library runs on holds one copy of this array until the process ends.  Host code
// never uses its name as an address (on the host that name is a stand-in, not device memory): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[MB_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on the first call on that device).
mb_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MB_ERR_HIP, "ns_orthogonalize_batched_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MB_ERR_HIP, "ns_orthogonalize_batched_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(MB_ERR_HIP, "ns_orthogonalize_batched_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MB_OK;
}

}  // namespace

extern "C" {

mb_status ns_orthogonalize_batched_noalloc(const uint16_t* x, uint16_t* y, int64_t batch, int64_t rows, int64_t cols,
                                           int32_t steps, double a, double b, double c, double eps, void* stream) {
    // the size check comes first, before anything touches the device
    if (check_shape(batch, rows, cols, "ns_orthogonalize_batched_noalloc") != MB_OK) return MB_ERR_SHAPE;
    const size_t need = bank_ws_layout(batch, rows, cols, (rows * cols) % 8 == 0).total;
    if (need > (size_t)MB_NOALLOC_SCRATCH_BYTES)
        return fail(MB_ERR_WORKSPACE,
                    "ns_orthogonalize_batched_noalloc: shape (%lld, %lld, %lld) needs %zu bytes of scratch; the static "
                    "scratch holds %zu (use ns_orthogonalize_batched with a workspace)",
                    (long long)batch, (long long)rows, (long long)cols, need, (size_t)MB_NOALLOC_SCRATCH_BYTES);
    if (!x || !y) return fail(MB_ERR_NULL, "ns_orthogonalize_batched_noalloc: null tensor pointer");
    void* ws = nullptr;
    mb_status s = scratch_address(&ws);
    if (s != MB_OK) return s;
    return ns_orthogonalize_impl(x, y, batch, rows, cols, steps, a, b, c, nullptr, eps, ws, need, stream);
}

mb_status ns_orthogonalize_batched(const uint16_t* x, uint16_t* y, int64_t batch, int64_t rows, int64_t cols,
                                   int32_t steps, double a, double b, double c, double eps, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    return ns_orthogonalize_impl(x, y, batch, rows, cols, steps, a, b, c, nullptr, eps, workspace, workspace_bytes,
                                 stream);
}

mb_status ns_orthogonalize_batched_sched(const uint16_t* x, uint16_t* y, int64_t batch, int64_t rows, int64_t cols,
                                         int32_t steps, const double* schedule, double eps, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    if (!schedule) return fail(MB_ERR_NULL, "ns_orthogonalize_batched_sched: null schedule");
    return ns_orthogonalize_impl(x, y, batch, rows, cols, steps, 1.0, 0.0, 0.0, schedule, eps, workspace,
                                 workspace_bytes, stream);
}

mb_status mp_apply_update(uint16_t* w_hi, uint16_t* w_lo, const uint16_t* v, int64_t batch, int64_t slot_numel,
                          float eff_lr, float decay, const float* lr_mul_per_slot, void* stream) {
    if (!w_hi || !w_lo || !v) return fail(MB_ERR_NULL, "mp_apply_update: null tensor pointer");
    mb_status s = check_shape(batch, 1, slot_numel, "mp_apply_update");
    if (s != MB_OK) return s;
    if (!aligned16(w_hi) || !aligned16(w_lo) || !aligned16(v) || ((uintptr_t)lr_mul_per_slot & 3u))
        return fail(MB_ERR_ALIGN, "mp_apply_update: tensors must be 16-byte aligned (lr_mul_per_slot 4-byte)");
    if (!std::isfinite(eff_lr) || !std::isfinite(decay))
        return fail(MB_ERR_VALUE, "mp_apply_update: eff_lr and decay must be finite");
    const int64_t n = batch * slot_numel;
    std::vector<Range> rs = {{(uintptr_t)w_hi, (uintptr_t)w_hi + n * 2, "w_hi"},
                             {(uintptr_t)w_lo, (uintptr_t)w_lo + n * 2, "w_lo"},
                             {(uintptr_t)v, (uintptr_t)v + n * 2, "v"}};
    if (lr_mul_per_slot) rs.push_back({(uintptr_t)lr_mul_per_slot, (uintptr_t)lr_mul_per_slot + batch * 4, "lr_mul_per_slot"});
    s = check_no_overlap(rs);
    if (s != MB_OK) return s;
    Timer timer;
    timer.begin("apply", (hipStream_t)stream);
    const mb::ApplyBank ab{w_hi, w_lo, v, lr_mul_per_slot, batch, slot_numel, eff_lr, decay, 0};
    hipError_t e = mb::launch_apply(&ab, 1, nullptr, (hipStream_t)stream);
    timer.end((hipStream_t)stream);
    if (e != hipSuccess) return fail(MB_ERR_HIP, "apply launch: %s", hipGetErrorString(e));
    return ok();
}

mb_status muon_bank_step(const mb_bank* banks, int32_t num_banks, const mb_hparams* hp_in, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (!banks) return fail(MB_ERR_NULL, "muon_bank_step: banks is null");
    if (num_banks <= 0 || num_banks > 1024) return fail(MB_ERR_SHAPE, "muon_bank_step: num_banks must be in 1..1024");
    mb_hparams hp;
    if (hp_in) hp = *hp_in;
    else mb_default_hparams(&hp);
    mb_status s = check_hparams(hp);
    if (s != MB_OK) return s;

    // ---- validate every bank before enqueueing anything
    std::vector<Range> ranges;
    size_t need = 0;
    int64_t total_slots = 0;
    for (int32_t i = 0; i < num_banks; ++i) {
        const mb_bank& b = banks[i];
        if (!b.grad || !b.momentum || !b.w_hi || !b.w_lo)
            return fail(MB_ERR_NULL, "muon_bank_step: bank %d has a null tensor pointer", i);
        s = check_shape(b.batch, b.rows, b.cols, "muon_bank_step");
        if (s != MB_OK) return s;
        if (b.grad_dtype != MB_F32 && b.grad_dtype != MB_BF16)
            return fail(MB_ERR_DTYPE, "muon_bank_step: bank %d dtype %d", i, b.grad_dtype);
        if (!aligned16(b.grad) || !aligned16(b.momentum) || !aligned16(b.w_hi) || !aligned16(b.w_lo) ||
            !aligned16(b.v_out) || !aligned16(b.u_out) || ((uintptr_t)b.lr_mul_per_slot & 3u))
            return fail(MB_ERR_ALIGN, "muon_bank_step: bank %d tensors must be 16-byte aligned", i);
        if (!is_finite(b.lr_mul) || !is_finite(b.wd_mul)) return fail(MB_ERR_VALUE, "muon_bank_step: bank %d multipliers", i);
        const int64_t n = b.batch * b.rows * b.cols;
        const size_t es = b.grad_dtype == MB_F32 ? 4 : 2;
        ranges.push_back({(uintptr_t)b.grad, (uintptr_t)b.grad + n * es, "grad"});
        ranges.push_back({(uintptr_t)b.momentum, (uintptr_t)b.momentum + n * es, "momentum"});
        ranges.push_back({(uintptr_t)b.w_hi, (uintptr_t)b.w_hi + n * 2, "w_hi"});
        ranges.push_back({(uintptr_t)b.w_lo, (uintptr_t)b.w_lo + n * 2, "w_lo"});
        if (b.v_out) ranges.push_back({(uintptr_t)b.v_out, (uintptr_t)b.v_out + n * 2, "v_out"});
        if (b.u_out) ranges.push_back({(uintptr_t)b.u_out, (uintptr_t)b.u_out + n * 2, "u_out"});
        if (b.lr_mul_per_slot)
            ranges.push_back({(uintptr_t)b.lr_mul_per_slot, (uintptr_t)b.lr_mul_per_slot + b.batch * 4, "lr_mul_per_slot"});
        need += bank_ws_layout(b.batch, b.rows, b.cols, (b.rows * b.cols) % 8 == 0).total;
        total_slots += b.batch;
    }
    if (hp.slot_scalars) {
        if ((uintptr_t)hp.slot_scalars & 15u)
            return fail(MB_ERR_ALIGN, "muon_bank_step: slot_scalars must be 16-byte aligned");
        for (int32_t i = 0; i < num_banks; ++i)
            if (banks[i].lr_mul_per_slot)
                return fail(MB_ERR_VALUE, "muon_bank_step: bank %d has lr_mul_per_slot, but slot_scalars already "
                            "holds every slot's eta", i);
        ranges.push_back({(uintptr_t)hp.slot_scalars, (uintptr_t)hp.slot_scalars + (size_t)total_slots * 16,
                          "slot_scalars"});
    }
    const StepPlan plan = plan_step(banks, num_banks);
    const size_t banks_bytes = need;
    need += round_up(plan.sync_ints * 4);
    if (!workspace || workspace_bytes < need)
        return fail(MB_ERR_WORKSPACE, "muon_bank_step: workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(MB_ERR_ALIGN, "muon_bank_step: workspace must be 16-byte aligned");
    ranges.push_back({(uintptr_t)workspace, (uintptr_t)workspace + need, "workspace"});
    s = check_no_overlap(ranges);
    if (s != MB_OK) return s;

    // ---- enqueue, all on the caller's stream: momentum and scale of every bank, the persistent
    // Newton-Schulz launches (each over several banks), the other banks' Newton-Schulz rounds,
    // then every apply
    hipStream_t st = (hipStream_t)stream;
    Timer timer;
    char* ws = (char*)workspace;
    int* sync = (int*)(ws + banks_bytes);
    const std::vector<mb::NsCoef> coef = ns_coefs(hp.ns_steps, hp.a, hp.b, hp.c, hp.ns_schedule);
    const bool persist = persist_path();
    struct Run {
        int64_t slot;
        bool vec;
        int nch;
        uint16_t *u, *v, *x1, *x2, *A, *Bm, *dest;
        double* partials;
        float* scale;
        int* live;
    };
    std::vector<Run> runs((size_t)num_banks);
    size_t off = 0;
    for (int32_t i = 0; i < num_banks; ++i) {
        const mb_bank& b = banks[i];
        Run& r = runs[(size_t)i];
        r.slot = b.rows * b.cols;
        r.vec = r.slot % 8 == 0;
        r.nch = mb::stream_chunks(r.slot);
        const BankWs L = bank_ws_layout(b.batch, b.rows, b.cols, r.vec);
        char* bw = ws + off;
        off += L.total;
        r.u = b.u_out ? b.u_out : (uint16_t*)(bw + L.u);
        r.v = b.v_out ? b.v_out : (uint16_t*)(bw + L.u);    // u is dead once the first round read it
        r.x1 = (uint16_t*)(bw + L.x1);
        r.x2 = (uint16_t*)(bw + L.x2);
        r.A = (uint16_t*)(bw + L.A);
        r.Bm = (uint16_t*)(bw + L.Bm);
        r.partials = (double*)(bw + L.partials);
        r.scale = (float*)(bw + L.scale);
        r.live = (int*)(bw + L.live);
        // with one round and no v_out, the round would read u while writing v in the same buffer
        r.dest = (hp.ns_steps == 1 && r.v == r.u) ? r.x2 : r.v;
    }
    // momentum of every bank in one launch (per kMaxStreamBanks banks), then the scale
    const float mu = f32(hp.momentum);
    const float nu = f32(1.0 - hp.momentum);
    std::vector<mb::MomentumBank> mbk;
    std::vector<mb::ScaleBank> sbk;
    int slot_base = 0;
    for (int32_t i = 0; i < num_banks; ++i) {
        const mb_bank& b = banks[i];
        const Run& r = runs[(size_t)i];
        mbk.push_back({b.grad, b.momentum, r.u, r.partials, b.batch, r.slot, b.grad_dtype == MB_F32, mu, nu, slot_base});
        slot_base += (int)b.batch;
        // a bank in a persistent launch clears its slot counters; the chunk's first bank clears
        // the chunk's queue heads, error word and exit count
        int *heads = nullptr, *ctr = nullptr;
        const int ch = plan.chunk_of[(size_t)i];
        if (persist && ch >= 0) {
            const PersistChunk& c = plan.chunks[(size_t)ch];
            int* cs = sync + c.sync_off;
            size_t k = 0;
            while (c.banks[k] != i) ++k;
            if (k == 0) heads = cs;
            ctr = cs + 32 + c.base[k];
        }
        sbk.push_back({r.partials, r.nch, b.batch, r.scale, r.live, heads, ctr, r.u,
                       mb::ns_prescale_buffer(r.x1, r.x2, hp.ns_steps), r.slot, 0});
    }
    timer.begin("momentum", st);
    hipError_t e = mb::launch_momentum(mbk.data(), num_banks, hp.slot_scalars, st);
    timer.end(st);
    if (e != hipSuccess) return fail(MB_ERR_HIP, "momentum launch: %s", hipGetErrorString(e));
    timer.begin("ns_scale", st);
    e = mb::launch_ns_scale(sbk.data(), num_banks, hp.eps, st);
    timer.end(st);
    if (e != hipSuccess) return fail(MB_ERR_HIP, "ns_scale launch: %s", hipGetErrorString(e));
    if (persist) {
        for (const PersistChunk& c : plan.chunks) {
            std::vector<mb::NsPersistBank> pb;
            for (int32_t i : c.banks) {
                const mb_bank& b = banks[i];
                const Run& r = runs[(size_t)i];
                pb.push_back({r.u, r.x1, r.x2, r.dest, r.A, r.Bm, r.scale, r.live, b.batch, b.rows, b.cols});
            }
            timer.begin("ns_persist", st);
            hipError_t e = mb::ns_persist(pb.data(), (int)pb.size(), c.tile, coef.data(), hp.ns_steps,
                                          sync + c.sync_off, st);
            timer.end(st);
            if (e != hipSuccess) return fail(MB_ERR_HIP, "Newton-Schulz launch: %s", hipGetErrorString(e));
        }
    }
    // banks of small slots: every round of all of them in one launch; the rest one launch per contraction
    std::vector<mb::NsSmall> small;
    for (int32_t i = 0; i < num_banks; ++i) {
        if (persist && plan.chunk_of[(size_t)i] >= 0) continue;
        const mb_bank& b = banks[i];
        const Run& r = runs[(size_t)i];
        if (g_ns_path.load() == 0 && mb::ns_small_eligible(b.rows, b.cols, hp.ns_steps)) {
            small.push_back({r.u, r.dest, r.scale, r.live, b.batch, b.rows, b.cols});
            continue;
        }
        s = run_ns(r.u, r.dest, r.x1, r.x2, r.A, r.Bm, b.batch, b.rows, b.cols, coef, r.scale, r.live, nullptr, st,
                   timer);
        if (s != MB_OK) return s;
    }
    if (!small.empty()) {
        timer.begin("ns_small", st);
        e = mb::ns_small(small.data(), (int)small.size(), hp.ns_steps, coef.data(), st);
        timer.end(st);
        if (e != hipSuccess) return fail(MB_ERR_HIP, "Newton-Schulz launch: %s", hipGetErrorString(e));
    }
    // every apply in one launch (per kMaxStreamBanks banks); host scalars in double, rounded once to
    // float32
    std::vector<mb::ApplyBank> abk;
    slot_base = 0;
    for (int32_t i = 0; i < num_banks; ++i) {
        const mb_bank& b = banks[i];
        const Run& r = runs[(size_t)i];
        const BankScalars bs = bank_scalars(b, hp);
        abk.push_back({b.w_hi, b.w_lo, r.dest, b.lr_mul_per_slot, b.batch, r.slot, bs.eta, bs.decay, slot_base});
        slot_base += (int)b.batch;
    }
    timer.begin("apply", st);
    e = mb::launch_apply(abk.data(), num_banks, hp.slot_scalars, st);
    timer.end(st);
    if (e != hipSuccess) return fail(MB_ERR_HIP, "apply launch: %s", hipGetErrorString(e));
    for (int32_t i = 0; i < num_banks; ++i) {
        const Run& r = runs[(size_t)i];
        if (r.dest != r.v) {
            e = hipMemcpyAsync(r.v, r.dest, (size_t)(banks[i].batch * r.slot) * 2, hipMemcpyDeviceToDevice, st);
            if (e != hipSuccess) return fail(MB_ERR_HIP, "copy: %s", hipGetErrorString(e));
        }
    }
    return ok();
}

}  // extern "C"

namespace {

mb_status transpose_impl(void* dst, const void* src, int64_t rows, int64_t cols, int es, bool add, const char* what,
                         void* stream) {
    if (!dst || !src) return fail(MB_ERR_NULL, "%s: null pointer", what);
    mb_status s = check_shape(1, rows, cols, what);
    if (s != MB_OK) return s;
    if (((uintptr_t)dst | (uintptr_t)src) % (uintptr_t)es != 0)
        return fail(MB_ERR_ALIGN, "%s: pointers must be aligned to the %d-byte element", what, es);
    const int64_t bytes = rows * cols * es;
    s = check_no_overlap({{(uintptr_t)dst, (uintptr_t)dst + bytes, "dst"}, {(uintptr_t)src, (uintptr_t)src + bytes, "src"}});
    if (s != MB_OK) return s;
    Timer timer;
    timer.begin(add ? "transpose_add" : "transpose_copy", (hipStream_t)stream);
    hipError_t e = mb::launch_transpose(dst, src, rows, cols, es, add, (hipStream_t)stream);
    timer.end((hipStream_t)stream);
    if (e != hipSuccess) return fail(MB_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

mb_status transpose_copy(void* dst, const void* src, int64_t rows, int64_t cols, int32_t elem_bytes, void* stream) {
    if (elem_bytes != 2 && elem_bytes != 4)
        return fail(MB_ERR_DTYPE, "transpose_copy: elem_bytes must be 2 or 4 (got %d)", elem_bytes);
    return transpose_impl(dst, src, rows, cols, elem_bytes, false, "transpose_copy", stream);
}

mb_status transpose_add(void* dst, const void* src, int64_t rows, int64_t cols, int32_t dtype, void* stream) {
    if (dtype != MB_F32 && dtype != MB_BF16) return fail(MB_ERR_DTYPE, "transpose_add: dtype %d", dtype);
    return transpose_impl(dst, src, rows, cols, dtype == MB_F32 ? 4 : 2, true, "transpose_add", stream);
}

int32_t mb_ns_set_path(int32_t path) {
    if (path != 0 && path != 1) return -1;
    return g_ns_path.exchange(path);
}

int32_t mb_device_fault(int32_t clear) {
    int flag = 0;
    const hipError_t e = mb::ns_persist_fault(&flag, clear != 0);
    if (e != hipSuccess) {
        fail(MB_ERR_HIP, "mb_device_fault: %s", hipGetErrorString(e));
        return -1;
    }
    return flag != 0 ? 1 : 0;
}

mb_status mb_test_persist_faults(int64_t wait_cap_ticks, int32_t extra_queues) {
    if (wait_cap_ticks < 0 || extra_queues < 0 || extra_queues > 8)
        return fail(MB_ERR_VALUE, "mb_test_persist_faults: wait cap %lld, extra queues %d", (long long)wait_cap_ticks,
                    extra_queues);
    mb::ns_persist_test_faults((uint64_t)wait_cap_ticks, extra_queues);
    return MB_OK;
}

void mb_timing_enable(int32_t on) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    g_timing_on = on != 0;
    // refill only when the pool runs low, so that switching timing on between steps creates no events
    if (on == 0 || g_event_pool.size() >= kEventPoolInit / 2) return;
    while (g_event_pool.size() < kEventPoolInit) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) break;
        g_event_pool.push_back(e);
    }
}

int32_t mb_timing_read(mb_kernel_time* out, int32_t max_entries) {
    std::vector<TimedLaunch> launches;
    {
        std::lock_guard<std::mutex> lk(g_timing_mu);
        launches.swap(g_timed);
    }
    std::vector<mb_kernel_time> agg;
    int32_t rc = 0;
    for (auto& t : launches) {
        float ms = 0.f;
        if (hipEventSynchronize(t.stop) != hipSuccess || hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess) rc = -1;
        {
            std::lock_guard<std::mutex> lk(g_timing_mu);
            g_event_pool.push_back(t.start);
            g_event_pool.push_back(t.stop);
        }
        size_t k = 0;
        for (; k < agg.size(); ++k)
            if (t.name == agg[k].name) break;
        if (k == agg.size()) {
            mb_kernel_time z{};
            std::snprintf(z.name, sizeof z.name, "%s", t.name.c_str());
            agg.push_back(z);
        }
        agg[k].launches += 1;
        agg[k].total_ms += ms;
    }
    if (rc < 0) return -1;
    const int32_t n = (int32_t)agg.size();
    for (int32_t i = 0; i < n && i < max_entries && out; ++i) out[i] = agg[i];
    return n;
}

}  // extern "C"
