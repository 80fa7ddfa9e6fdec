// One output tile of a Newton-Schulz contraction on gfx950, shared by the
// per-phase kernels and the persistent dataflow kernel.
//
// A tile computes C[i][j] = sum_k P(i,k) Q(k,j) for one slot, with each operand
// stored either K-major (row i holds P(i, 0..K)) or MN-major (row k holds
// P(0..M, k)), then applies one of three fp32 epilogues and rounds once to bf16
// (round to nearest even):
//   GRAM   out = sig*acc              symmetric, mirrored
//   POLY   out = alpha*acc + beta*A   symmetric, mirrored
//   UPDATE out = sig*(acc + beta*X)
// Operand tiles are copied global -> LDS with MUBUF buffer_load ... lds (16 B
// per lane) into a ring, so the copies of later k stages overlap the MFMAs of
// stage k with no register staging.  The 128x128 tiles use a two-stage ring
// (the copy of stage k+1 in flight during stage k).  The 256x256 tiles of
// launches that stream far more than the MALL holds fill the 160 KiB of LDS
// with three slots for one operand and two for the other: the first is copied
// two stages ahead, so its rows that miss the L2 have twice the time to arrive
// (350M banks: 3 % faster).  (A ring of four 32-k slots, three in flight, measured slower:
// twice the barriers and half-line row segments cost more than the deeper
// prefetch gains.)  The LDS layouts are XOR-swizzled so the
// 16-byte fragment reads and the transposing reads (ds_read_b64_tr_b16) hit
// distinct banks.  Every global load takes a cache policy: 0, or sc1 so that a
// load misses the CU's L1 and reads the XCD's L2, which is what a consumer of
// data written during the same kernel by another CU of the same XCD needs.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace mb {

constexpr int kBK = 64;                 // k per ring stage
enum { EPI_GRAM = 0, EPI_POLY = 1, EPI_UPDATE = 2 };
enum { POL_DEFAULT = 0, POL_SC1 = 16 }; // cache-policy bits of MUBUF loads (bit 4 = sc1 on gfx940+)

template <int BM_, int BN_, int WM_, int WN_, bool PAHEAD_ = false>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NW = WM * WN, NT = 64 * NW;
    static constexpr int TM = BM / WM, TN = BN / WN;      // outputs per wavefront
    static constexpr int FM = TM / 32, FN = TN / 32;      // 32x32 MFMA blocks per wavefront
    // PAHEAD: three slots for the operand copied two stages ahead (P, or Q when the tile asks for it),
    // then two for the other; otherwise two slots for each (P's first)
    static constexpr bool PAHEAD = PAHEAD_;
    static constexpr int PSLOT = BM * kBK, QSLOT = BN * kBK;             // elements per operand slot
    static constexpr int NPS = PAHEAD ? 3 : 2;                            // slots of the first group
    static constexpr int RING = NPS * PSLOT + 2 * QSLOT;                  // elements of the whole ring
    // copy instructions per wavefront of one operand tile (P's; Q's too when the tile is square, which
    // copying Q ahead requires)
    static constexpr int NIP = BM / 8 / NW;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tiles are whole MFMA blocks");
    static_assert((BM / 8) % NW == 0 && (BN / 8) % NW == 0, "copy instructions split evenly");
    static_assert(BM * BN <= RING, "the epilogue staging tile fits the ring");
    static_assert(RING * 2 <= 160 * 1024, "the ring fits the LDS");
};
using Cfg128 = Cfg<128, 128, 2, 2>;
// 16 wavefronts of 32x32 on a 128x128 tile: twice the LDS reads per MFMA of 64x64 wave tiles, but a
// task finishes about four times sooner on one CU, which is what a chain of short contractions
// (slots whose long side is at most 768) waits for.
using Cfg128w16 = Cfg<128, 128, 4, 4>;
// 16 wavefronts of 64x64 (four per SIMD, at most 128 VGPRs each): a third more LDS reads per MFMA
// than 8 wavefronts of 128x64, but four wavefronts per SIMD cover each other's waits, and the
// epilogue's LDS round trips and stores are spread over twice the wavefronts.
using Cfg256 = Cfg<256, 256, 4, 4, true>;
// The same tiles with the two-stage ring: when a launch's operands mostly come from the MALL, copying
// further ahead only adds requests in flight (attention bank, 40 x 768^2: 2 % slower with three slots).
using Cfg256r2 = Cfg<256, 256, 4, 4>;

// K-major tile [rows][8 chunks of 8 k]: chunk c of row R sits at entry R*8 + (c ^ ks(R)),
// conflict-free for the 16 lanes a 16-byte read serves per cycle.
__device__ __forceinline__ int ks(int R) { return (R & 7) ^ ((R >> 3) & 1); }
// MN-major tile [64 k rows][rows/8 chunks of 8 mn]: chunk c of row k sits at entry
// k*(rows/8) + (c ^ ms(k)).  A transposing read serves 32 lanes per cycle (4 k rows x 4
// chunks x 2 halves), which the XOR with 4*(k & 3) spreads over all 64 banks.
__device__ __forceinline__ int ms(int k) { return 4 * (k & 3); }

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// MUBUF load of 16 bytes per lane straight into LDS (lane l -> LDS base + 16*l; M0 holds the LDS
// base, saved and restored around the copy).  Unlike the FLAT-encoded global_load_lds it is
// tracked by vmcnt alone, so waiting for LDS reads never waits for copies still in flight; reads
// past the descriptor's size return zeros.  It is issued from inline assembly so that the compiler
// does not see an LDS write: seeing one, it orders later LDS reads after it with vmcnt(0) whenever
// its alias analysis cannot separate the two ring stages (it could not in some of the tile's
// instantiations, which then waited for every next-stage copy right after issuing it).  Every wait
// on these copies is the explicit one the caller places.
template <int POL>
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, const lds_u16* lds, int voffset) {
    const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    // the descriptor is uniform; readfirstlane states it, so the "s" constraints always hold
#pragma unroll
    for (int w = 0; w < 4; ++w) rsrc[w] = __builtin_amdgcn_readfirstlane(rsrc[w]);
    int save;
    if (POL == POL_SC1)
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen sc1 lds\n\ts_mov_b32 m0, %0\n\ts_nop 0"
            : "=&s"(save) : "s"(a), "v"(voffset), "s"(rsrc) : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0\n\ts_nop 0"
            : "=&s"(save) : "s"(a), "v"(voffset), "s"(rsrc) : "memory");
}

// Buffer descriptor of `bytes` bytes at `base` (raw buffer, stride 0; word 3 as for every gfx9 part).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r[0] = (int32_t)(uint32_t)a;
    r[1] = (int32_t)(uint32_t)((a >> 32) & 0xFFFFu);
    r[2] = (int32_t)bytes;
    r[3] = 0x00020000;
    return r;
}

// Copy one ROWS (mn) x 64 (k) operand tile into LDS: ROWS/8 instructions of 64 lanes x 16 B,
// instruction q filling entries [64q, 64q + 64).
template <bool KMAJOR, int ROWS, int NW, int POL>
__device__ __forceinline__ void load_tile_lds(i32x4 rsrc, int ld, int mn0, int k0, lds_u16* lds, int wave,
                                              int lane) {
    constexpr int NI = ROWS / 8 / NW;
    constexpr int CPR = ROWS / 8;                         // chunks per k row (MN-major)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int q = wave * NI + j;
        int elem;
        if (KMAJOR) {
            const int R = q * 8 + (lane >> 3);
            const int c = (lane & 7) ^ ks(R);
            elem = (mn0 + R) * ld + k0 + c * 8;
        } else {
            const int k = q * (64 / CPR) + lane / CPR;
            const int c = (lane % CPR) ^ ms(k);
            elem = (k0 + k) * ld + mn0 + c * 8;
        }
        lds_dma16<POL>(rsrc, lds + q * 512, elem * 2);
    }
}

// MFMA fragment (32 rows x 16 k; lane l holds row l%32, k = kk*16 + 8*(l/32) + 0..7) from a swizzled tile.
template <bool KMAJOR, int ROWS>
__device__ __forceinline__ bf16x8 read_frag_fast(const lds_u16* lds, int mn_base, int kk, int lane) {
    if (KMAJOR) {
        const int R = mn_base + (lane & 31);
        const int c = 2 * kk + (lane >> 5);
        return *(const MB_LDS bf16x8*)(lds + (R * 8 + (c ^ ks(R))) * 8);
    } else {
        constexpr int CPR = ROWS / 8;
        // ds_read_b64_tr_b16: within each 16-lane group, source lane 4s+q names k row s, columns
        // 4q..4q+3 of a 4 x 16 block; result lane t receives column t of the four rows
        const int g = lane >> 4, t = lane & 15, s = t >> 2, q = t & 3;
        const int mn = mn_base + 16 * (g & 1) + 4 * q;
        const int k = kk * 16 + 8 * (g >> 1) + s;
        const int c = mn >> 3, half = (mn >> 2) & 1;
        const lds_u16* p0 = lds + (k * CPR + (c ^ ms(k))) * 8 + half * 4;
        const int k4 = k + 4;
        const lds_u16* p1 = lds + (k4 * CPR + (c ^ ms(k4))) * 8 + half * 4;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MB_LDS i16x4*)p0);
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MB_LDS i16x4*)p1);
        i16x4 both[2] = {lo, hi};
        bf16x8 out;
        __builtin_memcpy(&out, both, 16);
        return out;
    }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // s_waitcnt with vmcnt = N (bits 3:0 and 15:14), expcnt and lgkmcnt left at their maxima (no wait)
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    // vmcnt = N, expcnt = 0, lgkmcnt = 0 (N = 0 is s_waitcnt 0)
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14));
}

// Upper-triangle tile t (row-major over the triangle of a T x T tile grid) -> (I, J), I <= J.
__device__ __forceinline__ void sym_tile(int t, int T, int& I, int& J) {
    int i = 0;
    while (t >= T - i) { t -= T - i; ++i; }
    I = i;
    J = i + t;
}

// What one tile needs: buffer descriptors of the slot's operands and aux, leading dimensions
// (elements), the contraction length, the tile origin, and the epilogue scalars.
struct TileJob {
    i32x4 P, Q, X;          // operand P, operand Q, aux (A for POLY, X for UPDATE; unused for GRAM)
    int ldp, ldq, ldx, ldo;
    int K;                  // multiple of 64
    int i0, j0;
    uint16_t* out;          // the slot's output
    bool mirror;            // also write the transposed tile (off-diagonal symmetric tiles)
    float alpha, beta, sig;
};

// tid is the thread's index in the workgroup.  A caller that runs tiles in a loop passes it
// through an opaque copy made inside the loop, so the per-lane address arithmetic is recomputed
// per tile instead of being hoisted out of the loop and held in registers across it.
// QAHEAD (256-tile ring only): Q, not P, takes the three slots and is copied two stages ahead.  The
// operand to copy ahead is the one whose rows the tiles that run next to each other do not share
// (for a tile order that walks j fastest, Q), so that more of its first-touch L2 misses have time.
template <bool P_KMAJOR, bool Q_KMAJOR, int EPI, class C, int POL, bool QAHEAD = false>
__device__ __forceinline__ void gemm_tile(const TileJob& jb, lds_u16* smem, int tid) {
    const int lane = tid & 63;
    // the wavefront's index is uniform: in scalar registers, its row and column offsets cost no VGPRs
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i0 = jb.i0, j0 = jb.j0;
    // a diagonal tile of a symmetric product (X X^T, A A) has P == Q: its operand is copied once
    // and both fragment sets read it
    const bool same = P_KMAJOR == Q_KMAJOR && C::BM == C::BN &&
                      __builtin_amdgcn_readfirstlane((int)(i0 == j0 && jb.P[0] == jb.Q[0] && jb.P[1] == jb.Q[1] &&
                                                           jb.ldp == jb.ldq)) != 0;
    // Such a tile computes only the wavefront blocks on and above its diagonal, one per wavefront in
    // row-major order (10 of 16 with a 4 x 4 grid; with the wavefronts placed on the four SIMDs in
    // turn, at most three per SIMD instead of four, so its K-loop needs three quarters of the MFMA
    // time), and stores the blocks below the diagonal as the transposes of those above it.  These are
    // the same bits: a block below the diagonal holds the same exact bf16 products, summed in the same
    // order, as its mirror image, and the polynomial's aux A is symmetric.  The other wavefronts copy
    // and wait at the barriers but compute nothing.  (256-tiles only: the 128-tiles serve short
    // chains, whose tasks gain less than the transposing stores and the second copy of the K-loop cost.)
    constexpr bool kTri = C::BM == 256 && C::WM == C::WN;
    const bool tri = kTri && EPI != EPI_UPDATE && same;
    int wm = wave / C::WN, wn = wave % C::WN;
    bool active = true;
    if constexpr (kTri) {
        if (tri) {
            active = wave < C::WM * (C::WM + 1) / 2;
            if (active) sym_tile(wave, C::WM, wm, wn);
            wm = __builtin_amdgcn_readfirstlane(wm);
            wn = __builtin_amdgcn_readfirstlane(wn);
        }
    }

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int a = 0; a < C::FM; ++a)
#pragma unroll
        for (int b = 0; b < C::FN; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

    const int KT = jb.K / kBK;
    // The ring: NPS slots of the operand copied ahead (P, or Q with QAHEAD; a diagonal tile copies
    // only P and always ahead), then two slots of the other.  Stage kt's operands sit in slot kt % NPS
    // of the first group and slot kt % 2 of the second.
    static_assert(!QAHEAD || (C::PAHEAD && C::BM == C::BN), "Q ahead needs the three-slot ring of square tiles");
    const bool qa = QAHEAD && !same;
    auto slot3 = [&](int s) { return smem + s * C::PSLOT; };
    auto slot2 = [&](int s) { return smem + C::NPS * C::PSLOT + s * C::QSLOT; };
    auto pslot = [&](int s3, int s2) { return qa ? slot2(s2) : slot3(s3); };
    auto qslot = [&](int s3, int s2) { return same ? slot3(s3) : (qa ? slot3(s3) : slot2(s2)); };
    auto copy_p = [&](int kt, lds_u16* dst) {
        load_tile_lds<P_KMAJOR, C::BM, C::NW, POL>(jb.P, jb.ldp, i0, kt * kBK, dst, wave, lane);
    };
    auto copy_q = [&](int kt, lds_u16* dst) {
        if (!same) load_tile_lds<Q_KMAJOR, C::BN, C::NW, POL>(jb.Q, jb.ldq, j0, kt * kBK, dst, wave, lane);
    };
    // copies of one stage's operand ahead of the other's, and of the other's (the ahead operand's
    // instruction count is what a wait that leaves it in flight allows)
    auto copy_ahead = [&](int kt, int s3) {
        if (qa) copy_q(kt, slot3(s3));
        else copy_p(kt, slot3(s3));
    };
    auto copy_other = [&](int kt, int s2) {
        if (qa) copy_p(kt, slot2(s2));
        else copy_q(kt, slot2(s2));
    };
    copy_ahead(0, 0);
    copy_other(0, 0);
    if (C::PAHEAD && KT > 1) {
        // the ahead operand of stage 1 stays in flight: the wait below covers everything issued before it
        copy_ahead(1, 1);
        wait_vmcnt<C::NIP>();
    } else {
        wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();

    // fragments double-buffered in registers: the reads of step kk+1 are issued before
    // the MFMAs of step kk, and the first reads of the next stage right after the barrier,
    // ahead of the last MFMAs of the current one
    bf16x8 pf[2][C::FM], qf[2][C::FN];
    if (active) {
#pragma unroll
        for (int a = 0; a < C::FM; ++a)
            pf[0][a] = read_frag_fast<P_KMAJOR, C::BM>(pslot(0, 0), wm * C::TM + a * 32, 0, lane);
#pragma unroll
        for (int b = 0; b < C::FN; ++b)
            qf[0][b] = read_frag_fast<Q_KMAJOR, C::BN>(qslot(0, 0), wn * C::TN + b * 32, 0, lane);
    }

    // One ring stage.  The last stage is a separate instantiation: were both kinds one loop body, the
    // compiler would merge the path that read the next stage's first fragments after the barrier with
    // the path that did not, and wait for those reads before the last MFMAs of the stage (every
    // wavefront of the workgroup, just past the barrier, would then leave its SIMD idle for the LDS
    // latency of the whole workgroup's reads).
    int s3 = 0;                                          // kt % NPS
    auto stage = [&](int kt, auto has_next, auto computes) {
        constexpr bool more = decltype(has_next)::value;
        constexpr bool mf = decltype(computes)::value;   // false: an idle wavefront (copies and barriers only)
        const int s2 = kt & 1;
        const int n3 = s3 + 1 == C::NPS ? 0 : s3 + 1;    // (kt + 1) % NPS
        const lds_u16* lp = pslot(s3, s2);
        const lds_u16* lq = qslot(s3, s2);
        // the slots of stage kt - 1 are free (every wave passed the barrier after reading them)
        bool ahead = false;
        if constexpr (more) {
            if (C::PAHEAD) {
                copy_other(kt + 1, s2 ^ 1);
                ahead = kt + 2 < KT;
                if (ahead) copy_ahead(kt + 2, n3 + 1 == C::NPS ? 0 : n3 + 1);
            } else {
                copy_ahead(kt + 1, n3);
                copy_other(kt + 1, s2 ^ 1);
            }
        }
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int fb = kk & 1, nb = fb ^ 1;
            if (kk + 1 < kBK / 16) {
                if constexpr (mf) {
#pragma unroll
                    for (int a = 0; a < C::FM; ++a)
                        pf[nb][a] = read_frag_fast<P_KMAJOR, C::BM>(lp, wm * C::TM + a * 32, kk + 1, lane);
#pragma unroll
                    for (int b = 0; b < C::FN; ++b)
                        qf[nb][b] = read_frag_fast<Q_KMAJOR, C::BN>(lq, wn * C::TN + b * 32, kk + 1, lane);
                }
            } else if constexpr (more) {
                // every wave's reads of this stage are done and the next stage has landed (with the
                // three-slot ring, the copy of stage kt + 2's ahead operand, issued last, may still be
                // in flight)
                if (ahead) wait_vmcnt_lgkm0<C::NIP>();
                else wait_vmcnt_lgkm0<0>();
                __builtin_amdgcn_s_barrier();
                const lds_u16* np = pslot(n3, s2 ^ 1);
                const lds_u16* nq = qslot(n3, s2 ^ 1);
                if constexpr (mf) {
#pragma unroll
                    for (int a = 0; a < C::FM; ++a)
                        pf[nb][a] = read_frag_fast<P_KMAJOR, C::BM>(np, wm * C::TM + a * 32, 0, lane);
#pragma unroll
                    for (int b = 0; b < C::FN; ++b)
                        qf[nb][b] = read_frag_fast<Q_KMAJOR, C::BN>(nq, wn * C::TN + b * 32, 0, lane);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (mf) {
#pragma unroll
                for (int a = 0; a < C::FM; ++a)
#pragma unroll
                    for (int b = 0; b < C::FN; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[fb][b], pf[fb][a], acc[a][b], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        s3 = n3;
    };
    // two copies of the loop, so that no branch on the wavefront's role sits inside it
    auto kloop = [&](auto computes) {
        for (int kt = 0; kt + 1 < KT; ++kt) stage(kt, std::true_type{}, computes);
        if (KT > 0) stage(KT - 1, std::false_type{}, computes);
    };
    if constexpr (kTri) {
        if (active) kloop(std::true_type{});
        else kloop(std::false_type{});
    } else {
        kloop(std::true_type{});
    }

    // ---- epilogue, staged through LDS so that every global access is a full coalesced row:
    //   1. (polynomial, update) the aux tile A or X is copied into LDS with buffer_load ... lds;
    //   2. each lane computes y for its accumulators (lane holds C[i][j..j+3] for
    //      i = i_base + lane%32, j = j_base + 8g + 4*(lane/32)), reading aux from LDS and
    //      writing y in place;
    //   3. the tile is stored row by row with 16-byte stores;
    //   4. off-diagonal symmetric tiles are also stored transposed: transposing LDS reads
    //      (ds_read_b64_tr_b16) of the same staged tile hand each lane 8 consecutive
    //      elements of a transposed row, stored with one 16-byte store.
    // Tile rows hold BN/8 16-byte chunks; chunk c of row i sits at chunk position c ^ (i % CW),
    // so the 32 rows an accumulator access touches spread over the banks.
    constexpr int CPRO = C::BN / 8;                     // 16-byte chunks per tile row
    constexpr int CW = CPRO < 32 ? CPRO : 32;
    constexpr int CH = C::BM * CPRO;                    // 16-byte chunks per tile
    static_assert(C::BM == C::BN || EPI == EPI_UPDATE, "symmetric tiles are square");
    static_assert(CH % (64 * C::NW) == 0, "the aux copy splits evenly over the wavefronts");
    lds_u16* st = smem;                                  // BM x BN bf16 staging tile (fits the ring)
    auto spos = [&](int i, int c) { return i * C::BN + ((c ^ (i % CW)) << 3); };
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    if (EPI != EPI_GRAM) {
        // LDS entry e = 64q + lane is row i = e / CPRO, position pc = e % CPRO, which holds
        // global chunk c = pc ^ (i % CW) of that row
        constexpr int NI = CH / 64 / C::NW;
#pragma unroll
        for (int jq = 0; jq < NI; ++jq) {
            const int q = wave * NI + jq;
            const int e = q * 64 + lane;
            const int i = e / CPRO, c = (e % CPRO) ^ (i % CW);
            const int elem = (i0 + i) * jb.ldx + j0 + c * 8;
            lds_dma16<POL>(jb.X, st + q * 512, elem * 2);
        }
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
    }
    // (the idle wavefronts of a diagonal tile have no block)
    if (active) {
#pragma unroll
        for (int a = 0; a < C::FM; ++a) {
            const int i = wm * C::TM + a * 32 + (lane & 31);
#pragma unroll
            for (int b = 0; b < C::FN; ++b) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int j = wn * C::TN + b * 32 + 8 * g + 4 * (lane >> 5);
                    lds_u16* p = st + spos(i, j >> 3) + (j & 4);
                    float av[4] = {0.f, 0.f, 0.f, 0.f};
                    if (EPI != EPI_GRAM) {
                        const u32x2 wv = *(const MB_LDS u32x2*)p;
                        av[0] = __uint_as_float(wv[0] << 16);
                        av[1] = __uint_as_float(wv[0] & 0xFFFF0000u);
                        av[2] = __uint_as_float(wv[1] << 16);
                        av[3] = __uint_as_float(wv[1] & 0xFFFF0000u);
                    }
                    float y[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = acc[a][b][4 * g + r];
                        if (EPI == EPI_GRAM) y[r] = jb.sig * x;
                        else if (EPI == EPI_POLY) y[r] = __fmaf_rn(jb.beta, av[r], jb.alpha * x);
                        else y[r] = jb.sig * __fmaf_rn(jb.beta, av[r], x);
                    }
                    u32x2 wv;
                    wv[0] = f32x2_to_bf16x2_rne(y[0], y[1]);
                    wv[1] = f32x2_to_bf16x2_rne(y[2], y[3]);
                    *(MB_LDS u32x2*)p = wv;
                }
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int v = tid; v < CH; v += C::NT) {
        const int i = v / CPRO, c = v % CPRO;
        if (tri && i / C::TM > c * 8 / C::TN) continue;     // below the diagonal: stored transposed below
        *reinterpret_cast<u32x4*>(jb.out + (int64_t)(i0 + i) * jb.ldo + j0 + c * 8) =
            *(const MB_LDS u32x4*)(st + spos(i, c));
    }
    if (EPI != EPI_UPDATE && (jb.mirror || tri)) {
        // unit (ib, jb16): tile rows [32 ib, 32 ib + 32) x columns [16 jb16, 16 jb16 + 16); the four
        // 16-lane groups of a wave take 8 rows each.  In a group, lane 4s + q addresses row s
        // (then s + 4) at columns 4q..4q+3, and lane t receives column t of those rows: elements
        // (i..i+7, j + t) = transposed row j + t, columns i..i+7.
        constexpr int UNITS = (C::BM / 32) * (C::BN / 16);
        static_assert(UNITS % C::NW == 0, "transposed units split evenly over the wavefronts");
        const int grp = lane >> 4, t16 = lane & 15, s4 = t16 >> 2, q4 = t16 & 3;
#pragma unroll
        for (int u = wave; u < UNITS; u += C::NW) {
            const int ib = u % (C::BM / 32), jb16 = u / (C::BM / 32);
            // a diagonal tile transposes only its blocks above the diagonal, into those below it
            if (tri && ib * 32 / C::TM >= jb16 * 16 / C::TN) continue;
            const int i = ib * 32 + grp * 8;
            const int jc = jb16 * 16 + 4 * q4;
            const lds_u16* pa = st + spos(i + s4, jc >> 3) + (jc & 7);
            const lds_u16* pb = st + spos(i + 4 + s4, jc >> 3) + (jc & 7);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MB_LDS i16x4*)pa);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MB_LDS i16x4*)pb);
            u32x4 w;
            w[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
            w[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
            w[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
            w[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
            *reinterpret_cast<u32x4*>(jb.out + (int64_t)(j0 + jb16 * 16 + t16) * jb.ldo + i0 + i) = w;
        }
    }
}

}  // namespace mb
