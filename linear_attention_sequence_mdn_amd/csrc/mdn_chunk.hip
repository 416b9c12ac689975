// mdn_chunk.hip -- chunkwise-parallel forward of Momentum DeltaNet (gfx950).
//
// Algorithm (MDN summary at paper.rainbus.top, method walk-through steps
// 2-5).  Chunk n holds tokens r = 0..C-1 (chunk-local, all cumulative
// quantities restart per chunk); S, M are the chunk-start states.
//
//   coefficients (step 5, log domain):
//     LA_r = sum_{s<=r} log alpha_s, LM_r = sum_{s<=r} log mu_s,
//     log c_r = logcumsumexp_{j<=r}(log beta_j + LM_j - LA_j),
//     abar_r = exp(LA_r), b_r = exp(LA_r + log c_r),
//     Gamma_{r,i} = eta_i sum_{j=i..r} beta_j (abar_r/abar_j)(mubar_j/mubar_i)
//   intra-chunk (steps 3-4):
//     A = (P K^T) o Gamma^-,  P = Diag(alpha) K,  Gamma^-_{r,i} = Gamma_{r-1,i} (i < r)
//     T = (I + A)^{-1}                       (unit lower, forward substitution)
//     Aqk = (Q K^T) o Gamma                  (lower, diagonal included)
//   inter-chunk (step 4 and the closed form of step 2 at r and at r = C-1):
//     W      = V - Diag(abar) K S + Diag(alpha_r b_{r-1}) K M
//     vtilde = T W                           (= U - Y S + Z M with U = TV,
//                                             Y = T Diag(abar_{r-1}) P,
//                                             Z = T Diag(b_{r-1}) P)
//     O      = Diag(abar) Q S - Diag(b) Q M + Aqk vtilde
//     S     <- abar_{C-1} S - b_{C-1} M + K^T Diag(gS) vtilde
//     M     <- mubar_{C-1} M - K^T Diag(gM) vtilde
//
// Kernel split:
//   mdn_intra_kernel  (mdn_intra.hip) one workgroup per chunk tile, fully
//                     parallel: coefficients, Gamma, T, Aqk.
//   mdn_inter_kernel  (this file) one workgroup per (head, slab of state
//                     columns), sequential over the chunks: vtilde, O (fused)
//                     and the fp32 S/M carry.  State columns are independent,
//                     so the slab split needs no communication.
#include "mdn_device.h"
#include "mdn_internal.h"
#include "mdn_lds.h"
#include "../../include/mdn.h"

namespace mdn {

// ---------------------------------------------------------------------------
// mdn_inter_kernel
//
// One workgroup owns a slab of 16*NCOL state columns of one head and runs
// the chunks of that head in order.  For every 16-column tile there are two
// waves that split the work of a chunk by state:
//   S-wave: W = V - Diag(abar) K S + Diag(alpha b_prev) K M, vtilde = T W,
//           S <- abar_C S - b_C M + K^T Diag(gS) vtilde        (S in registers)
//   M-wave: Q S and Q M for the output, M <- mubar_C M - K^T Diag(gM) vtilde,
//           O = Diag(abar) Q S - Diag(b) Q M + Aqk vtilde     (M in registers)
// The two exchange the chunk-start states (bf16 S, fp32 M) and vtilde through
// LDS, with two workgroup barriers per chunk.
//
// Every per-chunk input (K, Q, T, Aqk, the coefficient rows and the V slab)
// is copied to LDS by direct global->LDS loads, 16 bytes per lane, into one
// of two buffers: chunk n+1 is in flight while chunk n is computed.  K, Q, T
// and Aqk rows are XOR-swizzled by 16-byte piece (piece p of row r lives at
// p ^ (r mod pieces-per-row)) so that the 16 rows an operand read touches
// fall in different LDS banks.  K^T, the A operand of the state updates, is
// read from the row-major K tile with the LDS transpose read (bf16).
// vtilde and O go through an LDS tile so that they leave as full 16-byte
// stores.  Rows past the end of a ragged last chunk are copied from the last
// valid row: they only ever meet zero weights (T and Aqk are lower
// triangular, gS = gM = 0 there) and are never stored.
// ---------------------------------------------------------------------------
template <typename Tr, int D, int C, int NCOL, int NBUF>
struct InterLayout {
    using E = typename Tr::elem;
    using frag = typename Tr::frag;
    static constexpr int ES = sizeof(E);
    static constexpr int PK = D * ES / 16;            // 16-byte pieces per K/Q row
    static constexpr int PT = C * ES / 16;            // pieces per T/Aqk row
    static constexpr int PV = 16 * NCOL * ES / 16;    // pieces per V-slab / out row
    static constexpr int PC = MDN_COEF_ROWS * C * 4 / 16;
    static_assert((PK & (PK - 1)) == 0 && (PT & (PT - 1)) == 0, "power-of-two rows");
    // regions of one stage buffer (bytes)
    static constexpr int K0 = 0;
    static constexpr int Q0 = K0 + C * PK * 16;
    static constexpr int T0 = Q0 + C * PK * 16;
    static constexpr int A0 = T0 + C * PT * 16;
    static constexpr int CF0 = A0 + C * PT * 16;
    static constexpr int V0 = CF0 + PC * 16;
    static constexpr int BUF = V0 + C * PV * 16;
    // exchange areas and out tiles
    static constexpr int KSD = D / Tr::KW;
    static constexpr int XCH = NCOL * 64 * (KSD * (int)sizeof(frag) + (D / 16) * 16 + (C / 16) * 16);
    static constexpr int OUT = 2 * C * PV * 16;
    static constexpr int TOTAL = NBUF * BUF + XCH + OUT;
};

template <typename Tr, int D, int C>
struct InterPick {
    static constexpr int LIMIT = 160 * 1024 - 1024;
    static constexpr int NCOL = (D >= 32 && InterLayout<Tr, D, C, 2, 1>::TOTAL <= LIMIT) ? 2 : 1;
    static constexpr int NBUF = InterLayout<Tr, D, C, NCOL, 2>::TOTAL <= LIMIT ? 2 : 1;
};

// K^T operand of the state update for d-tile td, contraction step ks.
template <typename Tr, int P> struct KtOperand;
template <int P> struct KtOperand<TraitsBf16, P> {
    static __device__ __forceinline__ bf16x8 load(const char* Kt, int td, int ks, int lane) {
        // Transpose read: in each 16-lane group, result lane i takes element
        // i%4 of source lane 4j + i/4.  Source lane s of group g points at
        // row 32ks + 8g + s/4 (+4 for the second half) and columns
        // perm(16td) + 8(s%4) .. +3, so lane i receives
        // K[32ks + 8g + j][perm(16td + i)] for j = 0..3: the contraction
        // slots j (and 4 + j) of lane group g, for state row 16td + i.
        const int g = lane >> 4, s = lane & 15;
        const int r0 = 32 * ks + 8 * g + (s >> 2);
        const int b = 2 * (Slots<TraitsBf16>::perm(16 * td) + 8 * (s & 3));
        union { shortx4 h[2]; bf16x8 v; } f;
        f.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(Kt + swz<P>(r0, b)));
        f.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(Kt + swz<P>(r0 + 4, b)));
        return f.v;
    }
};
template <int P> struct KtOperand<TraitsF32, P> {
    static __device__ __forceinline__ float load(const char* Kt, int td, int ks, int lane) {
        const int g = lane >> 4, m = lane & 15;
        const int r = 16 * (ks >> 2) + 4 * g + (ks & 3);
        return *reinterpret_cast<const float*>(Kt + swz<P>(r, 4 * (16 * td + m)));
    }
};

// Issue part of the direct global->LDS copies of one chunk into the buffer at
// LDS byte address `buf`, by one wave: PART 0 K, PART 1 Q, PART 2 T and the coefficients,
// PART 3 Aqk and the V slab.  Rows past `valid` (ragged last chunk) repeat
// the last valid row.
template <typename LT, typename E, int D, int C, int PART>
__device__ __forceinline__ void stage_chunk(uint32_t buf, const E* __restrict__ k, const E* __restrict__ q,
                                            const E* __restrict__ v, const E* __restrict__ Tm,
                                            const E* __restrict__ Aqk, const float* __restrict__ coef,
                                            size_t rowbase, int valid, size_t tile, int col0, int lane)
{
    constexpr unsigned RB = D * LT::ES;              // bytes per K/Q/V row
    const unsigned vlast = (unsigned)valid - 1;
    auto seq_row = [&](unsigned r) { return (r < vlast ? r : vlast) * RB; };
    auto t_row = [](unsigned r) { return r * (unsigned)(C * LT::ES); };
    if constexpr (PART == 0) {
        dma_tile<C, LT::PK>(buf + LT::K0, reinterpret_cast<const char*>(k + rowbase * D), seq_row, lane);
    } else if constexpr (PART == 1) {
        dma_tile<C, LT::PK>(buf + LT::Q0, reinterpret_cast<const char*>(q + rowbase * D), seq_row, lane);
    } else if constexpr (PART == 2) {
        dma_tile<C, LT::PT>(buf + LT::T0, reinterpret_cast<const char*>(Tm + tile * C * C), t_row, lane);
        dma_plain<1, LT::PC>(buf + LT::CF0, reinterpret_cast<const char*>(coef + tile * MDN_COEF_ROWS * C),
                             [](unsigned) { return 0u; }, lane);
    } else {
        dma_tile<C, LT::PT>(buf + LT::A0, reinterpret_cast<const char*>(Aqk + tile * C * C), t_row, lane);
        dma_plain<C, LT::PV>(buf + LT::V0, reinterpret_cast<const char*>(v + rowbase * D + col0), seq_row, lane);
    }
}

// Copy an out tile (C rows x 16*NCOL elements in LDS) to rows [0, valid) of
// a row-major [.., D] output, by one wave; `dst` points at the chunk's first row.
template <typename LT, typename E, int D, int C>
__device__ __forceinline__ void copy_out(const char* tile, E* __restrict__ dst, int valid, int col0, int lane)
{
    constexpr int EPS = 16 / LT::ES;
    for (int s = lane; s < C * LT::PV; s += 64) {
        const int r = s / LT::PV, p = s % LT::PV;
        if (r < valid)
            *reinterpret_cast<uint4*>(dst + (size_t)r * D + col0 + p * EPS) =
                *reinterpret_cast<const uint4*>(tile + s * 16);
    }
}

template <typename Tr, int D, int C, int NCOL, int NBUF>
__global__ __launch_bounds__(64 * (2 * NCOL + 2))
void mdn_inter_kernel(const typename Tr::elem* __restrict__ q,
                      const typename Tr::elem* __restrict__ k,
                      const typename Tr::elem* __restrict__ v,
                      const typename Tr::elem* __restrict__ Tm,
                      const typename Tr::elem* __restrict__ Aqk,
                      const float* __restrict__ coef,
                      const float* __restrict__ S0, const float* __restrict__ M0,
                      typename Tr::elem* __restrict__ O,
                      float* __restrict__ ST, float* __restrict__ MT,
                      typename Tr::elem* __restrict__ Vt,
                      int64_t T, int64_t NT, int BH)
{
    using E = typename Tr::elem;
    using SL = Slots<Tr>;
    using LT = InterLayout<Tr, D, C, NCOL, NBUF>;
    using frag = typename Tr::frag;
    constexpr int NSL = SL::NSLOT;
    constexpr int NW = 2 * NCOL;                      // compute waves; waves NW, NW+1 load
    constexpr int NDT = D / 16, NCT = C / 16, KSD = D / Tr::KW, KSC = C / Tr::KW;
    constexpr int SLABS = D / (16 * NCOL);
    constexpr int OW = 16 * NCOL;                     // out-tile row length (elements)
    // Distinct LDS objects, so that the compiler can tell the buffer being
    // prefetched from every buffer being read.
    __shared__ __attribute__((aligned(16))) char stA[LT::BUF];
    __shared__ __attribute__((aligned(16))) char stB[NBUF == 2 ? LT::BUF : 16];
    __shared__ __attribute__((aligned(16))) frag xs[NCOL][KSD][64];      // S operands (S-wave -> M-wave)
    __shared__ __attribute__((aligned(16))) floatx4 xm[NCOL][NDT][64];   // M accumulators (M -> S)
    __shared__ __attribute__((aligned(16))) floatx4 xv[NCOL][NCT][64];   // vtilde (S -> M)
    __shared__ __attribute__((aligned(16))) E ov[C * OW];                // vtilde out tile
    __shared__ __attribute__((aligned(16))) E oo[C * OW];                // O out tile

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, nn = lane & 15;
    int bh, slab;
    xcd_head_map(blockIdx.x, SLABS, BH, bh, slab);
    const int col0 = slab * OW;
    auto valid_of = [&](int64_t n) { return (int)((T - n * C) < C ? (T - n * C) : C); };

    if (wave >= NW) {
        // ---- two loader waves: every global->LDS copy and every output store ----
        // Loader 0 copies K (before the mid-chunk barrier), then T and the
        // coefficients, and writes O; loader 1 copies Q, then Aqk and the V
        // slab, and writes vtilde.
        const int lw = wave - NW;
        auto issue = [&](uint32_t buf, int64_t m, int half) __attribute__((always_inline)) {
            const size_t tile = (size_t)bh * NT + m;
            const size_t rb = (size_t)bh * T + m * C;
            const int vm = valid_of(m);
            if (half == 0) {
                if (lw == 0) stage_chunk<LT, E, D, C, 0>(buf, k, q, v, Tm, Aqk, coef, rb, vm, tile, col0, lane);
                else stage_chunk<LT, E, D, C, 1>(buf, k, q, v, Tm, Aqk, coef, rb, vm, tile, col0, lane);
            } else {
                if (lw == 0) stage_chunk<LT, E, D, C, 2>(buf, k, q, v, Tm, Aqk, coef, rb, vm, tile, col0, lane);
                else stage_chunk<LT, E, D, C, 3>(buf, k, q, v, Tm, Aqk, coef, rb, vm, tile, col0, lane);
            }
        };
        const uint32_t aA = lds_addr(stA), aB = lds_addr(stB);
        if (NBUF == 2 && NT > 0) {
            issue(aA, 0, 0);
            issue(aA, 0, 1);
        }
        auto load = [&](uint32_t cur, uint32_t nxt, int64_t n) __attribute__((always_inline)) {
            const size_t rowbase = (size_t)bh * T + n * C;
            const bool more = n + 1 < NT;
            if constexpr (NBUF == 2) {
                __builtin_amdgcn_s_waitcnt(0);          // chunk n has landed (and earlier stores left)
                lds_barrier();                          // B0
                if (more) issue(nxt, n + 1, 0);
            } else {
                lds_barrier();                          // B0': the previous chunk's reads are done
                issue(cur, n, 0);
                issue(cur, n, 1);
                __builtin_amdgcn_s_waitcnt(0);
                lds_barrier();                          // B0
            }
            if (lw == 0 && n > 0)                       // O of chunk n-1 (written before B0)
                copy_out<LT, E, D, C>(reinterpret_cast<const char*>(oo), O + (rowbase - C) * D, C, col0, lane);
            lds_barrier();                              // B1
            if (NBUF == 2 && more) issue(nxt, n + 1, 1);
            if (lw == 1)
                copy_out<LT, E, D, C>(reinterpret_cast<const char*>(ov), Vt + rowbase * D, valid_of(n), col0, lane);
        };
        if constexpr (NBUF == 2) {
            for (int64_t n = 0; n < NT; n += 2) {
                load(aA, aB, n);
                if (n + 1 < NT) load(aB, aA, n + 1);
            }
        } else {
            for (int64_t n = 0; n < NT; ++n) load(aA, aA, n);
        }
        lds_barrier();
        if (lw == 0 && NT > 0)
            copy_out<LT, E, D, C>(reinterpret_cast<const char*>(oo), O + ((size_t)bh * T + (NT - 1) * C) * D,
                                  valid_of(NT - 1), col0, lane);
        return;
    }

    // ---- compute waves ----
    const bool swave = wave < NCOL;                   // S-wave or M-wave
    const int ct = swave ? wave : wave - NCOL;        // column tile within the slab
    const int col = col0 + 16 * ct + nn;

    // the wave's own state: S (S-wave) or M (M-wave)
    const size_t sbase = (size_t)bh * D * D;
    const float* X0 = swave ? S0 : M0;
    floatx4 X[NDT];
    if (X0) {
#pragma unroll
        for (int td = 0; td < NDT; ++td)
#pragma unroll
            for (int e = 0; e < 4; ++e) X[td][e] = X0[sbase + (size_t)SL::perm(16 * td + 4 * g + e) * D + col];
    } else {
#pragma unroll
        for (int td = 0; td < NDT; ++td) X[td] = zero4();
    }
    if (swave) {
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) xs[ct][ks][lane] = SL::from_acc(X, ks);
    } else {
#pragma unroll
        for (int td = 0; td < NDT; ++td) xm[ct][td][lane] = X[td];
    }

    auto chunk = [&](const char* cur, int64_t n) __attribute__((always_inline)) {
        if constexpr (NBUF == 1) lds_barrier();         // B0'
        lds_barrier();                                  // B0: chunk n staged, exchanges visible

        const char* Kl = cur + LT::K0;
        const char* Ql = cur + LT::Q0;
        const char* Tl = cur + LT::T0;
        const float* cf = reinterpret_cast<const float*>(cur + LT::CF0);
        const E* Vl = reinterpret_cast<const E*>(cur + LT::V0) + 16 * ct + nn;
        // coefficient of accumulator rows perm(16tc + 4g) + e, e = 0..3 (contiguous)
        auto crow = [&](int which, int tc) __attribute__((always_inline)) {
            return *reinterpret_cast<const floatx4*>(cf + which * C + SL::perm(16 * tc + 4 * g));
        };

        frag Sb[KSD], Mb[KSD];
        floatx4 Vx[NCT];      // S-wave: vtilde
        floatx4 Op[NCT];      // M-wave: Diag(abar) Q S - Diag(b) Q M
        if (swave) {
            floatx4 Mf[NDT];
#pragma unroll
            for (int td = 0; td < NDT; ++td) Mf[td] = xm[ct][td][lane];
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) { Sb[ks] = SL::from_acc(X, ks); Mb[ks] = SL::from_acc(Mf, ks); }
            {   // first half of the S update: abar_C S - b_C M (the chunk-start M is no longer needed)
                const float abarC = cf[MDN_COEF_ABAR * C + C - 1];
                const float bC = cf[MDN_COEF_B * C + C - 1];
#pragma unroll
                for (int td = 0; td < NDT; ++td)
#pragma unroll
                    for (int e = 0; e < 4; ++e) X[td][e] = abarC * X[td][e] - bC * Mf[td][e];
            }
            // W = V - Diag(abar) K S + Diag(alpha b_prev) K M
            floatx4 W[NCT], KSa[NCT], KMa[NCT];
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) { KSa[tc] = zero4(); KMa[tc] = zero4(); }
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                frag a[NCT];
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) a[tc] = LdsA<Tr, LT::PK>::load(Kl, SL::perm(16 * tc + nn), ks, g);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) {
                    KSa[tc] = Tr::mma(a[tc], Sb[ks], KSa[tc]);
                    KMa[tc] = Tr::mma(a[tc], Mb[ks], KMa[tc]);
                }
            }
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) {
                const floatx4 ca = crow(MDN_COEF_ABAR, tc), cb = crow(MDN_COEF_ABP, tc);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float vv = Tr::to_f(Vl[(SL::perm(16 * tc + 4 * g) + e) * OW]);
                    W[tc][e] = vv - ca[e] * KSa[tc][e] + cb[e] * KMa[tc][e];
                }
            }
            // vtilde = T W
            frag Wb[KSC];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) Wb[ks] = SL::from_acc(W, ks);
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) Vx[tc] = zero4();
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                frag a[NCT];
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) a[tc] = LdsA<Tr, LT::PT>::load(Tl, SL::perm(16 * tc + nn), ks, g);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) Vx[tc] = Tr::mma(a[tc], Wb[ks], Vx[tc]);
            }
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) {
                xv[ct][tc][lane] = Vx[tc];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ov[(SL::perm(16 * tc + 4 * g) + e) * OW + 16 * ct + nn] = Tr::from_f(Vx[tc][e]);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) { Sb[ks] = xs[ct][ks][lane]; Mb[ks] = SL::from_acc(X, ks); }
            floatx4 QSa[NCT], QMa[NCT];
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) { QSa[tc] = zero4(); QMa[tc] = zero4(); }
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                frag a[NCT];
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) a[tc] = LdsA<Tr, LT::PK>::load(Ql, SL::perm(16 * tc + nn), ks, g);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) {
                    QSa[tc] = Tr::mma(a[tc], Sb[ks], QSa[tc]);
                    QMa[tc] = Tr::mma(a[tc], Mb[ks], QMa[tc]);
                }
            }
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) {
                const floatx4 ca = crow(MDN_COEF_ABAR, tc), cb = crow(MDN_COEF_B, tc);
#pragma unroll
                for (int e = 0; e < 4; ++e) Op[tc][e] = ca[e] * QSa[tc][e] - cb[e] * QMa[tc][e];
            }
        }
        lds_barrier();                                  // B1: vtilde and the states of chunk n visible

        if (swave) {
            // S <- (abar_C S - b_C M) + K^T Diag(gS) vtilde
            frag VS[KSC];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                float sc[NSL];
#pragma unroll
                for (int j = 0; j < NSL; ++j) sc[j] = cf[MDN_COEF_GS * C + SL::row(ks, g, j)];
                VS[ks] = SL::from_acc_scaled(Vx, ks, sc);
            }
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                frag a[NDT];
#pragma unroll
                for (int td = 0; td < NDT; ++td) a[td] = KtOperand<Tr, LT::PK>::load(Kl, td, ks, lane);
#pragma unroll
                for (int td = 0; td < NDT; ++td) X[td] = Tr::mma(a[td], VS[ks], X[td]);
            }
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) xs[ct][ks][lane] = SL::from_acc(X, ks);
        } else {
            floatx4 Vv[NCT];
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) Vv[tc] = xv[ct][tc][lane];
            frag VM[KSC], Vb[KSC];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                float sc[NSL];
#pragma unroll
                for (int j = 0; j < NSL; ++j) sc[j] = -cf[MDN_COEF_GM * C + SL::row(ks, g, j)];
                VM[ks] = SL::from_acc_scaled(Vv, ks, sc);
                Vb[ks] = SL::from_acc(Vv, ks);
            }
            // M <- mubar_C M - K^T Diag(gM) vtilde
            const float mubarC = expf(cf[MDN_COEF_LM * C + C - 1]);
#pragma unroll
            for (int td = 0; td < NDT; ++td)
#pragma unroll
                for (int e = 0; e < 4; ++e) X[td][e] = mubarC * X[td][e];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                frag a[NDT];
#pragma unroll
                for (int td = 0; td < NDT; ++td) a[td] = KtOperand<Tr, LT::PK>::load(Kl, td, ks, lane);
#pragma unroll
                for (int td = 0; td < NDT; ++td) X[td] = Tr::mma(a[td], VM[ks], X[td]);
            }
#pragma unroll
            for (int td = 0; td < NDT; ++td) xm[ct][td][lane] = X[td];
            // O = Op + Aqk vtilde
            const char* Al = cur + LT::A0;
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                frag a[NCT];
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) a[tc] = LdsA<Tr, LT::PT>::load(Al, SL::perm(16 * tc + nn), ks, g);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) Op[tc] = Tr::mma(a[tc], Vb[ks], Op[tc]);
            }
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    oo[(SL::perm(16 * tc + 4 * g) + e) * OW + 16 * ct + nn] = Tr::from_f(Op[tc][e]);
        }
    };

    if constexpr (NBUF == 2) {
        for (int64_t n = 0; n < NT; n += 2) {
            chunk(stA, n);
            if (n + 1 < NT) chunk(stB, n + 1);
        }
    } else {
        for (int64_t n = 0; n < NT; ++n) chunk(stA, n);
    }
    lds_barrier();

    float* Xo = swave ? ST : MT;
#pragma unroll
    for (int td = 0; td < NDT; ++td)
#pragma unroll
        for (int e = 0; e < 4; ++e) Xo[sbase + (size_t)SL::perm(16 * td + 4 * g + e) * D + col] = X[td][e];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename Tr, int D, int C>
static hipError_t launch_inter_nw(const ChunkArgs& a)
{
    using E = typename Tr::elem;
    using P = InterPick<Tr, D, C>;
    constexpr int NCOL = P::NCOL, NBUF = P::NBUF;
    const int64_t grid = a.BH * (D / (16 * NCOL));
    hipLaunchKernelGGL((mdn_inter_kernel<Tr, D, C, NCOL, NBUF>), dim3((unsigned)grid), dim3(64 * (2 * NCOL + 2)), 0,
                       (hipStream_t)a.stream, (const E*)a.q, (const E*)a.k, (const E*)a.v,
                       (const E*)a.Tmat, (const E*)a.Aqk, a.coef, a.S0, a.M0,
                       (E*)a.O, a.ST, a.MT, (E*)a.Vt, a.T, a.NT, (int)a.BH);
    return hipGetLastError();
}

template <typename Tr>
static hipError_t inter_dispatch(const ChunkArgs& a)
{
    if constexpr (std::is_same<Tr, TraitsBf16>::value) {
        switch (a.dk * 1000 + a.C) {
        case 32032: return launch_inter_nw<Tr, 32, 32>(a);
        case 32064: return launch_inter_nw<Tr, 32, 64>(a);
        case 64032: return launch_inter_nw<Tr, 64, 32>(a);
        case 64064: return launch_inter_nw<Tr, 64, 64>(a);
        case 128032: return launch_inter_nw<Tr, 128, 32>(a);
        case 128064: return launch_inter_nw<Tr, 128, 64>(a);
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (a.dk * 1000 + a.C) {
        case 16016: return launch_inter_nw<Tr, 16, 16>(a);
        case 16032: return launch_inter_nw<Tr, 16, 32>(a);
        case 16064: return launch_inter_nw<Tr, 16, 64>(a);
        case 32016: return launch_inter_nw<Tr, 32, 16>(a);
        case 32032: return launch_inter_nw<Tr, 32, 32>(a);
        case 32064: return launch_inter_nw<Tr, 32, 64>(a);
        case 64016: return launch_inter_nw<Tr, 64, 16>(a);
        case 64032: return launch_inter_nw<Tr, 64, 32>(a);
        case 64064: return launch_inter_nw<Tr, 64, 64>(a);
        case 128016: return launch_inter_nw<Tr, 128, 16>(a);
        case 128032: return launch_inter_nw<Tr, 128, 32>(a);
        case 128064: return launch_inter_nw<Tr, 128, 64>(a);
        default: return hipErrorInvalidValue;
        }
    }
}

hipError_t launch_chunk_inter(const ChunkArgs& a)
{
    if (a.BH == 0) return hipSuccess;
    return a.dtype == MDN_BF16 ? inter_dispatch<TraitsBf16>(a) : inter_dispatch<TraitsF32>(a);
}

}  // namespace mdn
