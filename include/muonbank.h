/*
 * muonbank.h -- C ABI of libmuonbank.so, the MI355X (gfx950) Muon bank step.
 *
 * The step follows the modded-nanogpt record walkthroughs:
 *   - banks: stacked parameters viewed zero-copy as [batch, rows, cols]
 *     ("Unified zero-copy optimizer and transposed LM head", section 1.1);
 *   - momentum and Nesterov lerps, eff_lr / eff_wd ("Muon Custom Sizing",
 *     section 4);
 *   - five quintic Newton-Schulz rounds with coefficients 3.4445, -4.7750,
 *     2.0315 after a norm scaling ("Muon Custom Sizing", section 2.3;
 *     GPT-2 Medium Record 7 walkthrough, section 4.2);
 *   - the mixed-precision apply on bf16 weights plus a uint16 low mantissa
 *     (Record 7 walkthrough, section 4.1).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer, owned by the caller; tensors
 *     are dense and row-major.  The library keeps no pointer after returning.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is enqueued on it; no entry point synchronizes the host.
 *   - The library never allocates device memory on these paths: scratch
 *     comes from the caller's `workspace`, sized by the *_workspace_bytes
 *     queries.  Concurrent calls are safe on distinct workspaces.
 *   - Errors are return codes (mb_status).  Every argument is validated
 *     before anything is enqueued: on any status other than MB_OK nothing
 *     was launched and no buffer changed, except MB_ERR_HIP, which reports
 *     a failed launch (detail in mb_last_error()).  Faults inside kernels
 *     surface at the caller's next synchronization, as with any HIP work.
 *   - Device pointers must be 16-byte aligned (MB_ERR_ALIGN otherwise).
 *   - Results are deterministic: repeated calls on the same inputs give the
 *     same bits (fixed reduction orders, no atomics in value paths).
 */
#ifndef MUONBANK_H
#define MUONBANK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MB_OK = 0,
    MB_ERR_NULL = 1,       /* a required pointer is NULL                                   */
    MB_ERR_SHAPE = 2,      /* batch/rows/cols <= 0, or the element count overflows          */
    MB_ERR_DTYPE = 3,      /* unknown dtype code                                            */
    MB_ERR_ALIGN = 4,      /* a device pointer is not 16-byte aligned                       */
    MB_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than the matching query returns     */
    MB_ERR_ALIAS = 6,      /* two buffers overlap where they must not                       */
    MB_ERR_VALUE = 7,      /* a scalar argument is out of its domain (non-finite, steps<0) */
    MB_ERR_HIP = 8         /* the HIP runtime rejected a launch                             */
} mb_status;

typedef enum { MB_F32 = 0, MB_BF16 = 1 } mb_dtype;

/* Hyper-parameters shared by every bank of one call.  Host scalars are taken
 * in double and rounded once to float32 on the host:
 *   mu = RN32(momentum), nu = RN32(1 - momentum),
 *   decay = RN32(1 - lr*weight_decay*wd_mul)               (left to right),
 *   eta   = RN32(lr*sqrt(max(1, rows/cols))*lr_mul)        (left to right),
 * the shape-scaled learning rate and decoupled weight decay of "Muon Custom
 * Sizing", section 4.  Defaults (mb_default_hparams) are Muon's constructor
 * defaults lr=0.02, weight_decay=0.01, momentum=0.95 (same page, section 2.2)
 * and the five-round quintic a, b, c = 3.4445, -4.7750, 2.0315 (section 2.3),
 * eps = 1e-7 in the norm scaling X / (||X||_F + eps). */
typedef struct {
    double lr;
    double weight_decay;
    double momentum;
    int32_t ns_steps;
    double a, b, c;
    double eps;
    /* Optional per-round coefficients: NULL (the default) applies (a, b, c) in
     * every round; otherwise a host array of 3*ns_steps doubles, (a_t, b_t, c_t)
     * for round t, read during the call only.  Orthogonalizers with per-round
     * coefficients are named on the "Unified zero-copy optimizer" page
     * (sections 1.3, 4) without values, so the caller supplies them. */
    const double *ns_schedule;
    /* Optional per-slot scalar table, the one device buffer of bank scalars that the "Unified zero-copy
     * optimizer and transposed LM head" page (section 4) uploads once per step and graph replays read:
     * NULL (the default) uses the scalars above and each bank's multipliers; otherwise a DEVICE array
     * of 4 floats per slot, (mu, nu, decay, eta), for the slots of all banks of the call in bank order,
     * 16-byte aligned.  The kernels read it when they run, so a captured step sees the values in the
     * buffer at each replay.  The banks' lr_mul_per_slot must then be NULL (MB_ERR_VALUE).
     * mb_slot_scalars_fill writes the table that reproduces the call's own scalars. */
    const float *slot_scalars;
} mb_hparams;

/* One viewed bank [batch, rows, cols] (e.g. attention QKVO (10, 3072, 768)
 * viewed as (40, 768, 768); MLP (12, 2, 3072, 768) as (24, 3072, 768)).
 * Slots whose gradient and momentum are all zero (padding, dead layers)
 * stay exactly zero and their Newton-Schulz work is skipped. */
typedef struct {
    int64_t batch, rows, cols;
    int32_t grad_dtype;              /* MB_F32 or MB_BF16; momentum has the same dtype          */
    double lr_mul, wd_mul;           /* per-parameter multipliers (1.0 = none)                  */
    const void *grad;                /* [batch, rows, cols], read only                          */
    void *momentum;                  /* [batch, rows, cols], updated in place                   */
    uint16_t *w_hi;                  /* bf16 weight bits (high half of the fp32 master), in place */
    uint16_t *w_lo;                  /* uint16 low mantissa (low half), in place                */
    const float *lr_mul_per_slot;    /* optional [batch] float32: eta_slot = RN32(eta*m[i])     */
    uint16_t *v_out;                 /* optional [batch, rows, cols] bf16: the Newton-Schulz output */
    uint16_t *u_out;                 /* optional [batch, rows, cols] bf16: the Nesterov update u  */
} mb_bank;

void mb_default_hparams(mb_hparams *hp);
const char *mb_status_string(int32_t status);
/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char *mb_last_error(void);
/* Library version string. */
const char *mb_version(void);

/* Host helper for hp.slot_scalars: for each slot i of the banks in order, writes (mu, nu, decay, eta)
 * into host_table[4i .. 4i+3], as muon_bank_step derives them from hp (NULL = defaults) and each bank's
 * lr_mul and wd_mul: binary64 arithmetic rounded once to float32.  capacity is the number of floats at
 * host_table (at least 4 per slot, else MB_ERR_WORKSPACE).  A bank with lr_mul_per_slot (a device
 * vector the host cannot read) is MB_ERR_VALUE: fold the multiplier into the table's eta instead.  The
 * caller edits the rows it wants (schedules, per-matrix rates) and uploads the table. */
mb_status mb_slot_scalars_fill(const mb_bank *banks, int32_t num_banks, const mb_hparams *hp,
                               float *host_table, int64_t capacity);

/* What muon_bank_step would enqueue for these banks on a device of num_cus compute units in num_xcds
 * XCDs (MI355X: 256 and 8), under the current mb_ns_set_path setting: kernel launches by kind (total
 * excludes the device-to-device copies of one-round calls) and, for each persistent launch (the first
 * 8), its tile edge, its ring (3: the 256-tile ring that copies one operand two stages ahead, taken
 * when the launch's X is at least 128 MiB; 2: the two-stage ring), its workgroups, and whether they
 * claim their next task while a finished tile's stores drain (when every XCD queue holds at least two
 * rounds of tasks per workgroup).  Every persistent launch's task lists are checked on the host with
 * the kernel's own decode: each task of each slot listed exactly once, on its slot's queue, after
 * every task it waits for (MB_ERR_VALUE with the reason if not).  A device whose CU count is not a
 * multiple of its XCD count (or with more than 16 XCDs) gets no persistent launch.  Host only;
 * touches no device. */
typedef struct {
    int32_t momentum, ns_scale, ns_persist, ns_small, ns_per_contraction, apply, copies, total;
    int32_t persist_tile[8];
    int32_t persist_ring[8];
    int32_t persist_workgroups[8];
    int32_t persist_claim_early[8];
} mb_step_plan_info;
mb_status mb_step_plan(const mb_bank *banks, int32_t num_banks, const mb_hparams *hp, int32_t num_cus,
                       int32_t num_xcds, mb_step_plan_info *out);

/* Workspace bytes needed by muon_bank_step for these banks (0 on invalid shapes). */
size_t mb_step_workspace_bytes(const mb_bank *banks, int32_t num_banks);
/* Workspace bytes needed by ns_orthogonalize_batched for this shape (0 on invalid shapes). */
size_t mb_ns_workspace_bytes(int64_t batch, int64_t rows, int64_t cols);

/* The full Muon step on `num_banks` banks, enqueued on one stream:
 *   1. buf' = RN_M(mu*buf + nu*g) and u = RN_bf16(nu*g + mu*buf'), each
 *      correctly rounded from the exact value (M = the momentum dtype);
 *   2. v = NS(u): per slot, on X = u (u^T when rows > cols), X /= ||X||_F + eps,
 *      then ns_steps times A = X X^T, B = b*A + c*A A, X = a*X + B X;
 *      bf16 operands on MFMA with fp32 accumulation; A, B, X rounded to bf16
 *      (round-to-nearest-even) between contractions (slots whose Gram side is
 *      at most 64, with at most 4096 elements, run on fp32 vector units and
 *      keep A and B in fp32); ||u||_F is summed in binary64, so a slot is
 *      skipped (and stays zero) exactly when all its elements are zero, and
 *      any finite scale of u gives the result of the scaled problem;
 *   3. w = fp32(w_hi << 16 | w_lo); t = RN32(w*decay); r = RN32(t - eta_slot*v)
 *      (one fused multiply-add); w_hi = r >> 16, w_lo = r & 0xFFFF.
 * Banks must not overlap each other.  hp NULL = defaults. */
mb_status muon_bank_step(const mb_bank *banks, int32_t num_banks, const mb_hparams *hp,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Stage 1 alone (momentum + Nesterov): grad, momentum as in mb_bank, u_out
 * [batch, rows, cols] bf16.  mu and nu are the float32 coefficients
 * (normally RN32(momentum) and RN32(1 - momentum)).  No workspace. */
mb_status muon_momentum_update(const void *grad, void *momentum, uint16_t *u_out,
                               int64_t batch, int64_t rows, int64_t cols, int32_t dtype,
                               float mu, float nu, void *stream);

/* Stage 2 alone: y = NS(x) for x, y [batch, rows, cols] bf16 (y may equal x
 * exactly; partial overlap is MB_ERR_ALIAS).  Same arithmetic as stage 2 of
 * muon_bank_step, with `steps` rounds of (a, b, c) and the given eps. */
mb_status ns_orthogonalize_batched(const uint16_t *x, uint16_t *y,
                                   int64_t batch, int64_t rows, int64_t cols,
                                   int32_t steps, double a, double b, double c, double eps,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Largest scratch ns_orthogonalize_batched_noalloc can use: mb_ns_workspace_bytes of the shape must not
 * exceed it (the attention bank (40, 768, 768) needs about 236 MB). */
#define MB_NOALLOC_SCRATCH_BYTES (256u << 20)

/* ns_orthogonalize_batched for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same kernels and results, with the scratch
 * in a static device array of MB_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends.  Makes no device allocation and frees nothing; the caller passes x and y as for
 * ns_orthogonalize_batched (y may equal x).  Shapes whose scratch would exceed the array are rejected with
 * MB_ERR_WORKSPACE before the device is touched.  Every call on one device shares that device's array:
 * calls that overlap on one device (other streams, other threads) race and give undefined results;
 * serialize them.  The array's state from the previous call never matters: whatever must start at zero
 * is cleared by the call's own kernels. */
mb_status ns_orthogonalize_batched_noalloc(const uint16_t *x, uint16_t *y,
                                           int64_t batch, int64_t rows, int64_t cols,
                                           int32_t steps, double a, double b, double c, double eps,
                                           void *stream);

/* ns_orthogonalize_batched with per-round coefficients: round t (0-based) uses
 * schedule[3t], schedule[3t+1], schedule[3t+2] as (a, b, c); `schedule` is a
 * host array of 3*steps finite doubles (NULL is MB_ERR_NULL), read during the
 * call only.  Same workspace as ns_orthogonalize_batched.  Each coefficient is
 * rounded once to float32 for the kernels. */
mb_status ns_orthogonalize_batched_sched(const uint16_t *x, uint16_t *y,
                                         int64_t batch, int64_t rows, int64_t cols,
                                         int32_t steps, const double *schedule, double eps,
                                         void *workspace, size_t workspace_bytes, void *stream);

/* Stage 3 alone (Record 7 walkthrough, section 4.1): on every element of
 * [batch, slot_numel], w = fp32(w_hi << 16 | w_lo); t = RN32(w*decay);
 * r = RN32(t - eta_slot*v) with one fused multiply-add, eta_slot = eff_lr or,
 * with lr_mul_per_slot, RN32(eff_lr*lr_mul_per_slot[i]); then w_hi = r >> 16,
 * w_lo = r & 0xFFFF (a bit slice).  eff_lr and decay are float32, already
 * rounded.  v is bf16 bits.  No workspace. */
mb_status mp_apply_update(uint16_t *w_hi, uint16_t *w_lo, const uint16_t *v,
                          int64_t batch, int64_t slot_numel, float eff_lr, float decay,
                          const float *lr_mul_per_slot, void *stream);

/* The tied-embedding transposes of the "Unified zero-copy optimizer and
 * transposed LM head" page, section 2.2 (LM head stored as (768, 50304), the
 * embedding as (50304, 768)): for src [rows, cols] and dst [cols, rows], both
 * dense row-major device buffers that must not overlap,
 *   transpose_copy:  dst[j][i] = src[i][j], elem_bytes 2 or 4 (the bits are copied);
 *   transpose_add:   dst[j][i] = RN(dst[j][i] + src[i][j]), dtype MB_F32 or MB_BF16,
 *                    one round-to-nearest-even of the exact sum.
 * Pointers must be aligned to the element size (16-byte aligned buffers whose
 * rows are whole 16-byte chunks take the tiled fast path).  Enqueued on
 * `stream`; no workspace. */
mb_status transpose_copy(void *dst, const void *src, int64_t rows, int64_t cols, int32_t elem_bytes, void *stream);
mb_status transpose_add(void *dst, const void *src, int64_t rows, int64_t cols, int32_t dtype, void *stream);

/* How stage 2 is scheduled (process-wide; the arithmetic is the same either way).
 *   0 (default): when both sides of a slot are multiples of 128, every round of a
 *     bank runs in one persistent launch: the output tiles (256x256 when both sides
 *     are multiples of 256, the short side is at least 512 and the launch holds
 *     more than 8 such slots, else 128x128) of all
 *     three contractions of all rounds are tasks in per-XCD queues, and a task starts
 *     as soon as the previous contraction of its own slot has finished.  Each slot's
 *     tasks run on one XCD (slot s on XCD s % number of XCDs), so its intermediate
 *     results stay coherent through that XCD's L2.
 *   1: one launch per contraction and round.
 * Returns the previous value, or -1 (nothing changed) for any other value.  Calls
 * already enqueued are not affected. */
int32_t mb_ns_set_path(int32_t path);

/* Fault flag of the persistent Newton-Schulz launches on the current device.  A
 * task of that launch waits for the previous contraction of its slot; the wait
 * gives up after 200 ms (no correct schedule comes near it), the launch then
 * finishes with undefined values in the affected slots, and this flag is set.
 * It is also set when a launch ends with tasks of some XCD queue never claimed
 * (a queue no workgroup served).
 * Returns 1 if any launch on the device has set it since it was last cleared, 0
 * if none has, -1 on a HIP error (detail in mb_last_error()); clears it when
 * `clear` is nonzero.  Blocking: it reads device memory on the null stream, so
 * call it after synchronizing the streams the steps were enqueued on. */
int32_t mb_device_fault(int32_t clear);

/* Test hook (for tests of the two failure paths above; not for use in a
 * step): wait_cap_ticks > 0 replaces the 200 ms cap of a dependency wait
 * (ticks of the 100 MHz constant clock; 1 gives up a wait at its first timed
 * check), and extra_queues > 0 (at most 8) adds that many XCD queues beyond the
 * device's XCDs: no workgroup serves them, so their slots' tasks never run and
 * the launch's drain check reports them.  Either way the launch still finishes
 * (nothing waits for a task of an unserved queue), sets the fault flag, and
 * leaves undefined values in the affected slots.  Zero for both restores the
 * defaults.  Process-wide, host only; applies to launches enqueued after the
 * call.  MB_ERR_VALUE for a negative cap or extra_queues outside 0..8. */
mb_status mb_test_persist_faults(int64_t wait_cap_ticks, int32_t extra_queues);

/* Kernel timing (off by default).  While enabled, every kernel the library
 * launches is bracketed by two hipEvents on its stream; mb_timing_read waits
 * for them and returns, per kernel name, the launch count and the summed
 * duration in milliseconds.  Enabling creates a pool of events that reads hand
 * back, so a timed loop records events without creating them; switching timing
 * on and off between calls (to bracket only some of them) creates none either
 * until half the pool is in use.  Each event pair costs the stream a few
 * microseconds.  Timing never changes a result. */
typedef struct {
    char name[48];
    int64_t launches;
    double total_ms;
} mb_kernel_time;

void mb_timing_enable(int32_t on);
/* Fills up to max_entries records, returns how many kinds were recorded (or
 * -1 on a HIP error), and clears the recorded events. */
int32_t mb_timing_read(mb_kernel_time *out, int32_t max_entries);

#ifdef __cplusplus
}
#endif

#endif /* MUONBANK_H */
