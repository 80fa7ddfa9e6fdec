// Batched bf16 MFMA contractions of one quintic Newton-Schulz round on gfx950.
//
// One round ("Muon Custom Sizing", section 2.3; Record 7 walkthrough,
// section 4.2) on a slot X (m x n, m <= n) is
//     A = X X^T,   B = b*A + c*A A,   X' = a*X + B X.
// A tall slot G (n x m, stored row-major) is never transposed in memory:
//     A = G^T G,   B as above,        G' = a*G + G B,
// which is the same map (p(G^T) = p(G)^T for the odd polynomial p).
//
// Every contraction is C[i][j] = sum_k P(i,k) Q(k,j) on one slot, with each
// operand stored either K-major (row i holds P(i, 0..K)) or MN-major (row k
// holds P(0..M, k)).  Tiles of 128 x 128 outputs, K in steps of 64, four
// wavefronts each owning 64 x 64 outputs as 2 x 2 v_mfma_f32_32x32x16_bf16
// blocks with fp32 accumulators.  Operand tiles go global -> registers ->
// LDS (double-buffered, one barrier per K step).  K-major fragments are read
// with 16-byte LDS reads; MN-major fragments with the gfx950 transposing LDS
// read ds_read_b64_tr_b16, so no operand is ever transposed in memory.
//
// Epilogues (fp32, then one round-to-nearest-even to bf16):
//   GRAM   out = alpha*acc            (alpha = s^2 on the first round, s = the
//                                      slot's Frobenius scale, else 1); symmetric
//   POLY   out = c*acc + b*A          symmetric
//   UPDATE out = sigma*(a*X + acc)    (sigma = s on the first round, else 1)
// Symmetric outputs are computed on the upper tile triangle only and each
// off-diagonal tile is also written mirrored.  Slots with a zero norm are
// skipped; the update writes zeros for them.  In the first round a slot whose
// live word marks it pre-scaled reads X from the pre-scaled copy (the scale
// then includes the inverse power of two).

#include <cmath>

#include "common.hpp"
#include "kernels.hpp"
#include "ns_tile.hpp"

namespace mb {

namespace {

constexpr int BM = 128;          // output tile rows (i)
constexpr int BN = 128;          // output tile cols (j)
constexpr int BK = 64;           // k per stage
constexpr int NT = 256;          // threads per workgroup (4 wavefronts)
constexpr int KP = BK + 8;       // K-major LDS row pitch in elements (144 B: conflict-free 16-B reads)
constexpr int MP = BM + 16;      // MN-major LDS row pitch in elements (288 B: conflict-free transposing reads)
constexpr int TILE_ELEMS = 128 * KP;   // == 64 * MP == 9216 elements per operand tile
static_assert(TILE_ELEMS == BK * MP, "both LDS layouts use the same footprint");

struct GemmArgs {
    const uint16_t* P; int64_t ldp; int64_t p_stride;   // operand P (rows i)
    const uint16_t* Q; int64_t ldq; int64_t q_stride;   // operand Q (cols j)
    const uint16_t* aux; int64_t ld_aux; int64_t aux_stride;   // A (poly) or X (update) at the output position
    uint16_t* out; int64_t ldo; int64_t o_stride;
    int M, N, K;
    int tiles_m, tiles_n;
    int batch;
    float alpha, beta;          // GRAM: alpha; POLY: c, b; UPDATE: 1, a
    const float* scale;         // per-slot Frobenius scale (first round only), else null
    const int* live;            // per-slot live word
    const uint16_t* x_in;       // first round: the round's input X (P, Q or aux may be it) ...
    const uint16_t* x_pre;      // ... and, if non-null, where pre-scaled slots read it instead
};

// An operand's base for one slot: the pre-scaled copy of X for a pre-scaled slot in the first round.
__device__ __forceinline__ const uint16_t* slot_base(const GemmArgs& a, const uint16_t* p, int slot) {
    return (a.x_pre && p == a.x_in && (a.live[slot] & kPrescaledBit)) ? a.x_pre : p;
}

// Registers staging one 128 (mn) x 64 (k) operand tile: four 16-byte vectors per thread.
template <bool KMAJOR, bool VEC>
struct Stage {
    u32x4 r[4];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld, int mn0, int k0, int MN, int K,
                                         int tid) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int v = tid + NT * it;
            int mn, k;
            if (KMAJOR) { mn = v >> 3; k = (v & 7) * 8; }
            else { k = v >> 4; mn = (v & 15) * 8; }
            const int gmn = mn0 + mn, gk = k0 + k;
            if (VEC) {
                const bool ok = (gmn < MN) && (gk < K);
                if (ok) {
                    const uint16_t* p = KMAJOR ? base + (int64_t)gmn * ld + gk : base + (int64_t)gk * ld + gmn;
                    r[it] = *reinterpret_cast<const u32x4*>(p);
                } else {
                    r[it] = u32x4{0u, 0u, 0u, 0u};
                }
            } else {
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    int a = KMAJOR ? gmn : gmn + e;
                    int b = KMAJOR ? gk + e : gk;
                    bool ok = (a < MN) && (b < K);
                    h[e] = ok ? (uint32_t)(KMAJOR ? base[(int64_t)a * ld + b] : base[(int64_t)b * ld + a]) : 0u;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) r[it][q] = h[2 * q] | (h[2 * q + 1] << 16);
            }
        }
    }

    __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int v = tid + NT * it;
            int off = KMAJOR ? (v >> 3) * KP + (v & 7) * 8 : (v >> 4) * MP + (v & 15) * 8;
            *reinterpret_cast<u32x4*>(lds + off) = r[it];
        }
    }
};

// MFMA fragment of 32 rows (mn) x 16 k: lane l holds row (l % 32), k = kk*16 + 8*(l/32) + 0..7.
template <bool KMAJOR>
__device__ __forceinline__ bf16x8 read_frag(const uint16_t* lds, int mn_base, int kk, int lane) {
    if (KMAJOR) {
        const int row = mn_base + (lane & 31);
        const int k = kk * 16 + 8 * (lane >> 5);
        return *reinterpret_cast<const bf16x8*>(lds + row * KP + k);
    } else {
        // ds_read_b64_tr_b16: within each 16-lane group, source lane 4s+q names row s, columns 4q..4q+3
        // of a 4 x 16 block; result lane t receives column t of the four rows.
        const int g = lane >> 4;            // group: bit0 -> columns +16, bit1 -> k +8
        const int t = lane & 15;
        const int s = t >> 2, q = t & 3;
        const int col = mn_base + 16 * (g & 1) + 4 * q;
        const int krow = kk * 16 + 8 * (g >> 1) + s;
        const uint16_t* p0 = lds + krow * MP + col;
        const uint16_t* p1 = p0 + 4 * MP;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(p0));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(p1));
        i16x4 both[2] = {lo, hi};
        bf16x8 out;
        __builtin_memcpy(&out, both, 16);
        return out;
    }
}

template <bool P_KMAJOR, bool Q_KMAJOR, int EPI, bool VEC>
__global__ void __launch_bounds__(NT, 2) ns_gemm_kernel(GemmArgs args) {
    // XCD-aware mapping: workgroups are dispatched round-robin over the 8 XCDs, so
    // workgroup L runs on XCD L % 8.  Give XCD x the contiguous range
    // [x*per, (x+1)*per) of the slot-major work list, so all tiles of a slot share
    // one XCD's L2 and the operand panels they re-read stay cached there.
    const int per_slot = (EPI == EPI_UPDATE) ? args.tiles_m * args.tiles_n : args.tiles_m * (args.tiles_m + 1) / 2;
    const int total = args.batch * per_slot;
    const int per_xcd = (total + 7) >> 3;
    const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (w >= total) return;
    const int slot = w / per_slot;
    const int tile = w - slot * per_slot;
    if (!args.live[slot]) {
        if (EPI != EPI_UPDATE) return;
    }
    int ti, tj;
    if (EPI == EPI_UPDATE) {
        ti = tile / args.tiles_n;
        tj = tile % args.tiles_n;
    } else {
        sym_tile(tile, args.tiles_m, ti, tj);
    }
    const int i0 = ti * BM, j0 = tj * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    uint16_t* out = args.out + (int64_t)slot * args.o_stride;

    if (EPI == EPI_UPDATE && !args.live[slot]) {
        // dead slot: the round's output is exactly zero
        for (int v = tid; v < BM * BN; v += NT) {
            int i = i0 + v / BN, j = j0 + v % BN;
            if (i < args.M && j < args.N) out[(int64_t)i * args.ldo + j] = 0;
        }
        return;
    }

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE_ELEMS];
    // stage buffer b: P tile at smem + 2*b*TILE_ELEMS, Q tile right after it

    const uint16_t* P = slot_base(args, args.P, slot) + (int64_t)slot * args.p_stride;
    const uint16_t* Q = slot_base(args, args.Q, slot) + (int64_t)slot * args.q_stride;

    Stage<P_KMAJOR, VEC> sp;
    Stage<Q_KMAJOR, VEC> sq;
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

    const int KT = (args.K + BK - 1) / BK;
    sp.load(P, args.ldp, i0, 0, args.M, args.K, tid);
    sq.load(Q, args.ldq, j0, 0, args.N, args.K, tid);
    sp.store(smem, tid);
    sq.store(smem + TILE_ELEMS, tid);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) {
            sp.load(P, args.ldp, i0, (kt + 1) * BK, args.M, args.K, tid);
            sq.load(Q, args.ldq, j0, (kt + 1) * BK, args.N, args.K, tid);
        }
        const uint16_t* lp = smem + 2 * cur * TILE_ELEMS;
        const uint16_t* lq = lp + TILE_ELEMS;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 pf[2], qf[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) pf[a] = read_frag<P_KMAJOR>(lp, wm * 64 + a * 32, kk, lane);
#pragma unroll
            for (int b = 0; b < 2; ++b) qf[b] = read_frag<Q_KMAJOR>(lq, wn * 64 + b * 32, kk, lane);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[b], pf[a], acc[a][b], 0, 0, 0);
        }
        if (more) {
            uint16_t* np = smem + 2 * (cur ^ 1) * TILE_ELEMS;
            sp.store(np, tid);
            sq.store(np + TILE_ELEMS, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds C[i][j] for i = i_base + lane%32, j = j_base + 8g + 4*(lane/32) + 0..3
    float sig = 1.f;
    if (args.scale) {
        const float s = args.scale[slot];
        sig = (EPI == EPI_GRAM) ? s * s : s;
    }
    const uint16_t* aux = args.aux ? slot_base(args, args.aux, slot) + (int64_t)slot * args.aux_stride : nullptr;
    const bool mirror = (EPI != EPI_UPDATE) && (ti != tj);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int i = i0 + wm * 64 + a * 32 + (lane & 31);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int jb = j0 + wn * 64 + b * 32 + 8 * g + 4 * (lane >> 5);
                float x[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = acc[a][b][4 * g + r];
                float av[4] = {0.f, 0.f, 0.f, 0.f};
                if (EPI != EPI_GRAM) {
                    if (VEC) {
                        if (i < args.M && jb < args.N) {
                            u32x2 w = *reinterpret_cast<const u32x2*>(aux + (int64_t)i * args.ld_aux + jb);
                            av[0] = __uint_as_float(w[0] << 16);
                            av[1] = __uint_as_float(w[0] & 0xFFFF0000u);
                            av[2] = __uint_as_float(w[1] << 16);
                            av[3] = __uint_as_float(w[1] & 0xFFFF0000u);
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (i < args.M && jb + r < args.N) av[r] = bf16_to_f32(aux[(int64_t)i * args.ld_aux + jb + r]);
                    }
                }
                uint16_t hb[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float y;
                    if (EPI == EPI_GRAM) y = sig * x[r];
                    else if (EPI == EPI_POLY) y = __fmaf_rn(args.beta, av[r], args.alpha * x[r]);
                    else y = sig * __fmaf_rn(args.beta, av[r], x[r]);
                    hb[r] = f32_to_bf16_rne(y);
                }
                if (VEC) {
                    if (i < args.M && jb < args.N) {
                        u32x2 w;
                        w[0] = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
                        w[1] = (uint32_t)hb[2] | ((uint32_t)hb[3] << 16);
                        *reinterpret_cast<u32x2*>(out + (int64_t)i * args.ldo + jb) = w;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (i < args.M && jb + r < args.N) out[(int64_t)i * args.ldo + jb + r] = hb[r];
                }
                if (mirror) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (i < args.M && jb + r < args.N) out[(int64_t)(jb + r) * args.ldo + i] = hb[r];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Fast path for M, N multiples of the tile and K a multiple of 64 (every bank
// shape): one workgroup per output tile, the tile body shared with the
// persistent kernel.  Tile shapes: 128x128 with four wavefronts (two
// workgroups per CU) or 256x256 with sixteen (one per CU, twice the flops per
// byte moved out of L2).
// ---------------------------------------------------------------------------

template <bool P_KMAJOR, bool Q_KMAJOR, int EPI, class C>
__global__ void __launch_bounds__(C::NT, 2) ns_gemm_fast(GemmArgs args) {
    const int per_slot = (EPI == EPI_UPDATE) ? args.tiles_m * args.tiles_n : args.tiles_m * (args.tiles_m + 1) / 2;
    const int total = args.batch * per_slot;
    const int per_xcd = (total + 7) >> 3;
    const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (w >= total) return;
    const int slot = w / per_slot;
    const int tile = w - slot * per_slot;
    const bool live = args.live[slot] != 0;
    if (!live && EPI != EPI_UPDATE) return;
    int ti, tj;
    if (EPI == EPI_UPDATE) {
        ti = tile / args.tiles_n;
        tj = tile % args.tiles_n;
    } else {
        sym_tile(tile, args.tiles_m, ti, tj);
    }
    const int i0 = ti * C::BM, j0 = tj * C::BN;
    uint16_t* out = args.out + (int64_t)slot * args.o_stride;

    if (!live) {
        for (int v = threadIdx.x; v < C::BM * C::BN; v += C::NT) {
            int i = i0 + v / C::BN, j = j0 + v % C::BN;
            out[(int64_t)i * args.ldo + j] = 0;
        }
        return;
    }

    __shared__ __attribute__((aligned(1024))) uint16_t smem[C::RING];
    TileJob jb;
    jb.P = make_rsrc(slot_base(args, args.P, slot) + (int64_t)slot * args.p_stride, (uint32_t)(args.p_stride * 2));
    jb.Q = make_rsrc(slot_base(args, args.Q, slot) + (int64_t)slot * args.q_stride, (uint32_t)(args.q_stride * 2));
    jb.X = EPI == EPI_GRAM ? jb.P
                           : make_rsrc(slot_base(args, args.aux, slot) + (int64_t)slot * args.aux_stride,
                                       (uint32_t)(args.aux_stride * 2));
    jb.ldp = (int)args.ldp;
    jb.ldq = (int)args.ldq;
    jb.ldx = (int)args.ld_aux;
    jb.ldo = (int)args.ldo;
    jb.K = args.K;
    jb.i0 = i0;
    jb.j0 = j0;
    jb.out = out;
    jb.mirror = (EPI != EPI_UPDATE) && (ti != tj);
    jb.alpha = args.alpha;
    jb.beta = args.beta;
    float sig = 1.f;
    if (args.scale) {
        const float s = args.scale[slot];
        sig = (EPI == EPI_GRAM) ? s * s : s;
    }
    jb.sig = sig;
    gemm_tile<P_KMAJOR, Q_KMAJOR, EPI, C, POL_DEFAULT>(jb, (lds_u16*)smem, (int)threadIdx.x);
}

// Tile configuration of one contraction: 256x256 tiles move half the bytes per flop out of L2
// but come in quarter the number; take them unless that leaves most of the chip idle.
enum TileChoice { TILE_GENERIC = 0, TILE_128 = 1, TILE_256 = 2 };

TileChoice pick_tile(int M, int N, int K, int batch, bool symmetric, bool transposed, bool vec) {
    if (!vec || K % BK != 0) return TILE_GENERIC;
    const bool fit256 = M % 256 == 0 && N % 256 == 0;
    const bool fit128 = M % 128 == 0 && N % 128 == 0;
    if (!fit128) return TILE_GENERIC;
    if (!fit256) return TILE_128;
    auto tiles = [&](int t) {
        const int64_t tm = M / t, tn = N / t;
        return (int64_t)batch * (symmetric ? tm * (tm + 1) / 2 : tm * tn);
    };
    // rounds of the whole grid over 256 CUs (128-tiles: two per CU) times the measured cost of
    // one round: a round of 256-tiles (four times the work) takes about 1.4x a round of
    // 128-tiles, 1.5x when an operand goes through the transposing LDS reads
    const double r128 = std::ceil(tiles(128) / 512.0);
    const double r256 = std::ceil(tiles(256) / 256.0) * (transposed ? 1.5 : 1.4);
    return r256 <= r128 ? TILE_256 : TILE_128;
}

template <bool PK, bool QK, int EPI>
hipError_t launch_gemm(GemmArgs a, int batch, bool vec, hipStream_t stream) {
    const bool sym = EPI != EPI_UPDATE;
    const TileChoice tc = pick_tile(a.M, a.N, a.K, batch, sym, !(PK && QK), vec);
    const int t = tc == TILE_256 ? 256 : 128;
    a.tiles_m = (a.M + t - 1) / t;
    a.tiles_n = (a.N + t - 1) / t;
    a.batch = batch;
    const int tiles = sym ? a.tiles_m * (a.tiles_m + 1) / 2 : a.tiles_m * a.tiles_n;
    const int64_t total = (int64_t)tiles * batch;
    dim3 grid((unsigned)(((total + 7) / 8) * 8));
    if (tc == TILE_256) ns_gemm_fast<PK, QK, EPI, Cfg256><<<grid, Cfg256::NT, 0, stream>>>(a);
    else if (tc == TILE_128) ns_gemm_fast<PK, QK, EPI, Cfg128><<<grid, Cfg128::NT, 0, stream>>>(a);
    else if (vec) ns_gemm_kernel<PK, QK, EPI, true><<<grid, NT, 0, stream>>>(a);
    else ns_gemm_kernel<PK, QK, EPI, false><<<grid, NT, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

// One Newton-Schulz round on every slot of a bank.  x_in/x_out are [batch, rows, cols]
// bf16 in the stored orientation; A and Bm are [batch, m, m] bf16 scratch.
hipError_t ns_round(const NsRound& r, hipStream_t stream, RoundTimer* timer) {
    const int64_t rows = r.rows, cols = r.cols;
    const bool tall = rows > cols;
    const int m = (int)(tall ? cols : rows);
    const int n = (int)(tall ? rows : cols);
    const int64_t slot = rows * cols;
    const int64_t mm = (int64_t)m * m;
    const bool vec = (m % 8 == 0) && (n % 8 == 0);
    const int tm = (m + BM - 1) / BM;
    hipError_t e;

    // A = X X^T (wide) or G^T G (tall)
    GemmArgs g{};
    g.P = r.x_in; g.p_stride = slot;
    g.Q = r.x_in; g.q_stride = slot;
    g.ldp = g.ldq = tall ? m : n;
    g.out = r.A; g.ldo = m; g.o_stride = mm;
    g.M = m; g.N = m; g.K = n;
    g.tiles_m = tm; g.tiles_n = tm;
    g.alpha = 1.f;
    g.scale = r.first ? r.scale : nullptr;
    g.live = r.live;
    g.x_in = r.x_in;
    g.x_pre = r.first ? r.x_pre : nullptr;
    if (timer) timer->begin("ns_gram", stream);
    e = tall ? launch_gemm<false, false, EPI_GRAM>(g, (int)r.batch, vec, stream)
             : launch_gemm<true, true, EPI_GRAM>(g, (int)r.batch, vec, stream);
    if (timer) timer->end(stream);
    if (e != hipSuccess) return e;

    // B = b*A + c*A A  (A symmetric: Q(k, j) = A[j][k])
    GemmArgs p{};
    p.P = r.A; p.Q = r.A; p.ldp = p.ldq = m; p.p_stride = p.q_stride = mm;
    p.aux = r.A; p.ld_aux = m; p.aux_stride = mm;
    p.out = r.Bm; p.ldo = m; p.o_stride = mm;
    p.M = m; p.N = m; p.K = m;
    p.tiles_m = tm; p.tiles_n = tm;
    p.alpha = r.c; p.beta = r.b;
    p.scale = nullptr;
    p.live = r.live;
    if (timer) timer->begin("ns_poly", stream);
    e = launch_gemm<true, true, EPI_POLY>(p, (int)r.batch, vec, stream);
    if (timer) timer->end(stream);
    if (e != hipSuccess) return e;

    // X' = a*X + B X (wide: Q(k, j) = X[k][j], MN-major) or G' = a*G + G B (tall: both K-major)
    GemmArgs u{};
    u.live = r.live;
    u.scale = r.first ? r.scale : nullptr;
    u.x_in = r.x_in;
    u.x_pre = r.first ? r.x_pre : nullptr;
    u.alpha = 1.f; u.beta = r.a;
    u.aux = r.x_in; u.aux_stride = slot;
    u.out = r.x_out; u.o_stride = slot;
    if (tall) {
        u.P = r.x_in; u.ldp = m; u.p_stride = slot;     // G (n x m), K-major over k = the m columns
        u.Q = r.Bm; u.ldq = m; u.q_stride = mm;         // Q(k, j) = B[k][j] = B[j][k]
        u.M = n; u.N = m; u.K = m;
        u.ld_aux = m; u.ldo = m;
    } else {
        u.P = r.Bm; u.ldp = m; u.p_stride = mm;
        u.Q = r.x_in; u.ldq = n; u.q_stride = slot;     // Q(k, j) = X[k][j]: MN-major
        u.M = m; u.N = n; u.K = m;
        u.ld_aux = n; u.ldo = n;
    }
    u.tiles_m = (u.M + BM - 1) / BM;
    u.tiles_n = (u.N + BN - 1) / BN;
    if (timer) timer->begin("ns_update", stream);
    e = tall ? launch_gemm<true, true, EPI_UPDATE>(u, (int)r.batch, vec, stream)
             : launch_gemm<true, false, EPI_UPDATE>(u, (int)r.batch, vec, stream);
    if (timer) timer->end(stream);
    return e;
}

}  // namespace mb
