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

// Whether row tile t of a lower-triangular C x C matrix (T, Aqk), read as a
// matrix-core A operand, can be nonzero in contraction step ks.  bf16: step
// ks covers columns 32ks .. 32ks + 31 and the rows perm(16t + x) of tile t
// all lie in the 32-row half t/2; fp32: step ks covers the columns
// 16(ks/4) + ks%4 + 4g and tile t holds rows 16t .. 16t + 15.
template <typename Tr>
constexpr bool lower_step(int t, int ks)
{
    return std::is_same<Tr, TraitsBf16>::value ? ks <= (t >> 1) : (ks >> 2) <= t;
}

// ---------------------------------------------------------------------------
// mdn_inter_kernel
//
// One workgroup owns a slab of 16*NCOL state columns of one head and runs
// the chunks of that head in order.  State columns are independent.
//
// Chain waves (NCOL*RS of them) carry the state.  For every 16-column tile,
// RS chain waves split the dk state rows into RS parts: wave (ct, h) holds
// rows [h*D/RS, (h+1)*D/RS) of both S and M for column tile ct in fp32
// registers.  Per chunk:
//   phase 1: vtilde starts as T V; the partial products over its own rows,
//              P_h = -Diag(abar) K S_h + Diag(alpha b_prev) K M_h,
//            are exchanged with the partner wave (one barrier), and the
//            first half of the state update (abar_C S_h - b_C M_h,
//            mubar_C M_h) is done while the chunk-start M_h is at hand;
//   phase 2: vtilde += T (P_0 + P_1) (both waves, so that no second
//            exchange is needed), the vtilde operands go to LDS, and the
//            wave's rows are updated, S_h += K_h^T Diag(gS) vtilde,
//            M_h -= K_h^T Diag(gM) vtilde, which needs nothing from the
//            partner; the new state's bf16 operands go to LDS.
// With RS = 1 one wave per column tile does all of it and nothing is
// exchanged.  The output is off the state chain: nothing of it is computed
// by the chain waves.
//
// Four loader waves issue every global->LDS copy (K, Q, T, Aqk, the
// coefficient rows and the V slab of the next chunk, 16 bytes per lane, into
// one of two buffers) and every output store, and they compute the output:
// after the mid-chunk barrier of chunk n each forms, for its token tile and
// column tiles, R = Diag(abar) Q S - Diag(b) Q M from the chunk-start state
// operands (all dk rows, so no partial sums are exchanged; the operands are
// kept per chunk parity, so the chain waves can store the next chunk's
// meanwhile); after the next chunk barrier it adds Aqk vtilde, and writes O and vtilde to LDS out tiles
// that are copied out with 16-byte stores.  K, Q, T and Aqk rows are
// XOR-swizzled by 16-byte piece so that the 16 rows an operand read touches
// fall in different LDS banks.  K^T, the A operand of the state updates, and
// V, the B operand of T V, are read with the LDS transpose read (bf16).  Rows
// past the end of a ragged last chunk are copies of the last valid row: they
// only ever meet zero weights (T and Aqk are lower triangular, gS = gM = 0
// there) and are never stored.
// ---------------------------------------------------------------------------
template <typename Tr, int D, int C, int NCOL, int RS, int NBUF>
struct InterLayout {
    using E = typename Tr::elem;
    using frag = typename Tr::frag;
    static constexpr int ES = sizeof(E);
    static constexpr int FS = sizeof(frag);
    static constexpr int PK = D * ES / 16;            // 16-byte pieces per K/Q row
    static constexpr int PT = C * ES / 16;            // pieces per T/Aqk row
    static constexpr int PV = 16 * NCOL * ES / 16;    // pieces per V-slab / out row
    static constexpr int PC = MDN_COEF_ROWS * C * 4 / 16;
    static constexpr bool QUAD = quad_unread<Tr, C>();  // T, Aqk staged without their zero quadrant
    static_assert((PK & (PK - 1)) == 0 && (PT & (PT - 1)) == 0, "power-of-two rows");
    // regions of one stage buffer (bytes)
    static constexpr int K0 = 0;
    static constexpr int Q0 = K0 + C * PK * 16;
    static constexpr int T0 = Q0 + C * PK * 16;
    static constexpr int A0 = T0 + C * PT * 16;
    static constexpr int CF0 = A0 + C * PT * 16;
    static constexpr int V0 = CF0 + PC * 16;
    static constexpr int BUF = V0 + C * PV * 16;
    static constexpr int NCT = C / 16;
    static constexpr int KSH = D / RS / Tr::KW;       // contraction steps of one row part
    static constexpr int KSC = C / Tr::KW;
    // partial-product exchange (RS > 1): 4 fp32 values per lane and row tile
    static constexpr int XP = RS > 1 ? NCOL * RS * NCT * 64 * 16 : 0;
    // chain -> output waves: chunk-start S, M operands and vtilde operands
    static constexpr int SM = 2 * NCOL * RS * 2 * KSH * 64 * FS;   // two chunk parities
    static constexpr int VB = NCOL * KSC * 64 * FS;
    static constexpr int OUT = 2 * C * PV * 16;
    static constexpr int TOTAL = NBUF * BUF + XP + SM + VB + OUT;
};

template <typename Tr, int D, int C>
struct InterPick {
    static constexpr int LIMIT = 160 * 1024 - 1024;
    // One chain wave per column tile holds all dk rows.  Splitting the rows
    // over two waves (one per SIMD, with the partial products of K S and
    // K M exchanged through LDS every chunk) measured slower once the output
    // moved to the loader waves: the exchange puts a second workgroup
    // barrier on the chain and four waves read every T operand.  fp32
    // operands at dk >= 64 keep the split, which halves the registers a
    // chain wave holds.
    static constexpr bool BF = std::is_same<Tr, TraitsBf16>::value;
    static constexpr int RS = (!BF && D >= 64 && C >= 32) ? 2 : 1;
    static constexpr int NCOL = (D >= 32 && InterLayout<Tr, D, C, 2, RS, 1>::TOTAL <= LIMIT) ? 2 : 1;
    static constexpr int NBUF = InterLayout<Tr, D, C, NCOL, RS, 2>::TOTAL <= LIMIT ? 2 : 1;
    static_assert(InterLayout<Tr, D, C, NCOL, RS, NBUF>::TOTAL <= LIMIT, "LDS");
};

// Issue one loader wave's share of the direct global->LDS copies of one
// chunk into the stage buffer `buf`.  HALF 0 (needed first):
// the K and Q rows, split by rows over the NLD loaders; HALF 1: T, Aqk, the
// V slab and the coefficient rows.  A single wave sustains only a fraction
// of a CU's L2 bandwidth, so the copies are spread over all loaders.  Rows
// past `valid` (ragged last chunk) repeat the last valid row.  `vr` points
// at the chunk's first V row; when it is NULL the V slab is not copied (the
// buffer's V region then holds zeros, written once at the start).
template <typename LT, typename E, int D, int C, int NLD, int HALF>
__device__ __forceinline__ void stage_chunk(int lw, lds_char* buf, const E* __restrict__ k, const E* __restrict__ q,
                                            const E* __restrict__ vr, const E* __restrict__ Tm,
                                            const E* __restrict__ Aqk, const float* __restrict__ coef,
                                            size_t rowbase, int valid, size_t tile, int col0, int lane)
{
    static_assert(NLD == 4, "four loader waves");
    constexpr unsigned RB = D * LT::ES;              // bytes per K/Q/V row
    const unsigned vlast = (unsigned)valid - 1;
    auto seq_row = [&](unsigned r) { return (r < vlast ? r : vlast) * RB; };
    auto t_row = [](unsigned r) { return r * (unsigned)(C * LT::ES); };
    auto cf_row = [](unsigned) { return 0u; };
    if constexpr (HALF == 0) {
        constexpr int NH = NLD / 2, RPL = C / NH;    // loaders per matrix, rows per loader
        const bool isq = lw >= NH;
        const int part = lw % NH;
        if (isq)      // Q is read only by the loader waves: swizzle key 1
            dma_tile_p<RPL, LT::PK, 1>(buf + LT::Q0, reinterpret_cast<const char*>(q + rowbase * D), seq_row, lane,
                                       part * RPL);
        else
            dma_tile_p<RPL, LT::PK>(buf + LT::K0, reinterpret_cast<const char*>(k + rowbase * D), seq_row, lane,
                                    part * RPL);
    } else {
        constexpr int QS = LT::QUAD ? 1 : 0;          // the intra stage leaves that quadrant unwritten
        if (lw == 0)
            dma_tile_p<C, LT::PT, 0, QS, C>(buf + LT::T0, reinterpret_cast<const char*>(Tm + tile * C * C), t_row, lane);
        else if (lw == 1)
            dma_tile_p<C, LT::PT, 1, QS, C>(buf + LT::A0, reinterpret_cast<const char*>(Aqk + tile * C * C), t_row,
                                            lane);
        else if (lw == 2) {
            if (vr) dma_plain_p<C, LT::PV>(buf + LT::V0, reinterpret_cast<const char*>(vr + col0), seq_row, lane);
        }
        else
            dma_plain_p<1, LT::PC>(buf + LT::CF0, reinterpret_cast<const char*>(coef + tile * MDN_COEF_ROWS * C),
                                   cf_row, lane);
    }
}

// Row r of an out tile is stored at row out_row(r): the accumulator rows a
// lane group writes with one 2-byte store (rows 8 apart) then fall in
// different LDS banks.  The map is its own inverse.
__device__ __forceinline__ int out_row(int r) { return r ^ ((r >> 3) & 3); }

// Copy an out tile (C rows x 16*NCOL elements in LDS, rows placed by
// out_row) to rows [0, valid) of a row-major [.., D] output, by one wave;
// `dst` points at the chunk's first row.  Every LDS read is issued before
// the first store.
template <typename LT, typename E, int D, int C>
__device__ __forceinline__ void copy_out(const char* tile, E* __restrict__ dst, int valid, int col0, int lane)
{
    constexpr int EPS = 16 / LT::ES;
    constexpr int NP = C * LT::PV, NI = (NP + 63) / 64;
    uint4 val[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int s = i * 64 + lane;
        if (NP % 64 == 0 || s < NP) val[i] = *reinterpret_cast<const uint4*>(tile + s * 16);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int s = i * 64 + lane;
        const int r = out_row(s / LT::PV), p = s % LT::PV;
        if ((NP % 64 == 0 || s < NP) && r < valid)
            *reinterpret_cast<uint4*>(dst + (size_t)r * D + col0 + p * EPS) = val[i];
    }
}

template <typename Tr, int D, int C, int NCOL, int RS, int NBUF, int NLD, bool SEG>
__global__ __launch_bounds__(64 * (NCOL * RS + NLD))
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
                      int64_t T, int64_t NT, int BH, const int32_t* __restrict__ cu,
                      const int32_t* __restrict__ perm, int H, InterSeg seg)
{
    using E = typename Tr::elem;
    using SL = Slots<Tr>;
    using LT = InterLayout<Tr, D, C, NCOL, RS, NBUF>;
    using frag = typename Tr::frag;
    constexpr int NSL = SL::NSLOT;
    constexpr int NW = NCOL * RS;                     // chain waves; waves NW .. NW+NLD-1 load and output
    constexpr int NCT = C / 16, KSC = C / Tr::KW, KSD = D / Tr::KW;
    constexpr int DH = D / RS;                        // state rows per chain wave
    constexpr int NDH = DH / 16, KSH = DH / Tr::KW;   // its accumulator tiles / contraction steps
    constexpr int SLABS = D / (16 * NCOL);
    constexpr int OW = 16 * NCOL;                     // out-tile row length (elements)
    static_assert(DH % 16 == 0 && DH % Tr::KW == 0 && NLD == 4 && NLD % NCT == 0, "row split, output tasks");
    // Distinct LDS objects, so that the compiler can tell the buffer being
    // prefetched from every buffer being read.
    __shared__ __attribute__((aligned(16))) char stA[LT::BUF];
    __shared__ __attribute__((aligned(16))) char stB[NBUF == 2 ? LT::BUF : 16];
    __shared__ __attribute__((aligned(16))) floatx4 xp[RS > 1 ? NCOL * RS * NCT * 64 : 1];   // P_h
    __shared__ __attribute__((aligned(16))) frag sm[2][NCOL * RS * 2 * KSH * 64];          // S_h, M_h operands, by chunk parity
    __shared__ __attribute__((aligned(16))) frag vb[NCOL * KSC * 64];                       // vtilde operands
    __shared__ __attribute__((aligned(16))) E ov[C * OW];                // vtilde out tile
    __shared__ __attribute__((aligned(16))) E oo[C * OW];                // O out tile

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, nn = lane & 15;
    const InterUnit unit = inter_unit<SEG>(blockIdx.x, SLABS, BH, T, NT, C, cu, perm, H, D, seg);
    const int slab = unit.slab;
    const int64_t row0 = unit.row0, tile0 = unit.tile0, len = unit.len;
    const int col0 = slab * OW;
    const int64_t NTu = (len + C - 1) / C;
    auto valid_of = [&](int64_t n) { return (int)((len - n * C) < C ? (len - n * C) : C); };
    // coefficient of accumulator rows perm(16tc + 4g) + e, e = 0..3 (contiguous)
    auto crow = [&](const float* cf, int which, int tc) __attribute__((always_inline)) {
        return *reinterpret_cast<const floatx4*>(cf + which * C + SL::perm(16 * tc + 4 * g));
    };

    if (wave >= NW) {
        // ---- loader / output waves ----
        // Copies: the K and Q rows of chunk n+1 are issued right after the
        // chunk barrier, T, Aqk, the V slab and the coefficients after the
        // mid-chunk barrier.  Output: wave lw owns token tile tc = lw % NCT
        // of the column tiles lw / NCT + i * (NLD / NCT).  Between the
        // barrier of chunk n and its mid-chunk barrier it finishes O and
        // vtilde of chunk n-1 into the out tiles (the vtilde operands of
        // chunk n-1 were stored before the barrier, and its Aqk is still
        // staged) and forms R of chunk n (its chunk-start state operands
        // were stored before the barrier too).  The out tiles are copied
        // out after the mid-chunk barrier, O by loader 2 and vtilde by
        // loader 3 (loaders 0 and 1 issue the larger copies).
        // The wave index is a template constant of the wave's code, so that
        // the token tile and every choice of which copy to issue are too.
        auto loader = [&](auto lwc) __attribute__((always_inline)) {
        constexpr int lw = decltype(lwc)::value;
        constexpr int OCS = NLD / NCT;                 // output waves per token tile
        constexpr int NOC = (NCOL + OCS - 1) / OCS;    // column tiles per output wave
        constexpr int tc = lw % NCT, oc0 = lw / NCT;
        auto issue = [&](lds_char* buf, int64_t m, int half) __attribute__((always_inline)) {
            const size_t tile = (size_t)(tile0 + m);
            const size_t rb = (size_t)(row0 + m * C);
            const int vm = valid_of(m);
            const E* vr = (SEG && unit.vzero) ? nullptr : v + rb * D;
            if (half == 0) stage_chunk<LT, E, D, C, NLD, 0>(lw, buf, k, q, vr, Tm, Aqk, coef, rb, vm, tile, col0, lane);
            else stage_chunk<LT, E, D, C, NLD, 1>(lw, buf, k, q, vr, Tm, Aqk, coef, rb, vm, tile, col0, lane);
        };
        auto copy_outs = [&](int64_t m) __attribute__((always_inline)) {
            if (SEG && !unit.ostore) return;
            if (lw == 2)
                copy_out<LT, E, D, C>(reinterpret_cast<const char*>(oo), O + (size_t)(row0 + m * C) * D, valid_of(m), col0, lane);
            else if (lw == 3)
                copy_out<LT, E, D, C>(reinterpret_cast<const char*>(ov), Vt + (size_t)(row0 + m * C) * D, valid_of(m), col0, lane);
        };
        floatx4 R[NOC];
        // R = Diag(abar) Q S - Diag(b) Q M of the chunk staged in `cur`, over all dk rows
        auto out_r = [&](const char* cur, int64_t n) __attribute__((always_inline)) {
            const frag* smp = sm[n & 1];
            const char* Ql = cur + LT::Q0;
            const float* cf = reinterpret_cast<const float*>(cur + LT::CF0);
            frag qa[KSD];
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) qa[ks] = LdsA<Tr, LT::PK, 1>::load(Ql, SL::perm(16 * tc + nn), ks, g);
            const floatx4 ca = crow(cf, MDN_COEF_ABAR, tc), cb = crow(cf, MDN_COEF_B, tc);
#pragma unroll
            for (int i = 0; i < NOC; ++i) {
                const int oct = oc0 + i * OCS;
                if (oct >= NCOL) continue;
                floatx4 qs = zero4(), qm = zero4();
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    const int base = ((oct * RS + ks / KSH) * 2) * KSH * 64 + (ks % KSH) * 64 + lane;
                    qs = Tr::mma(qa[ks], smp[base], qs);
                    qm = Tr::mma(qa[ks], smp[base + KSH * 64], qm);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) R[i][e] = ca[e] * qs[e] - cb[e] * qm[e];
            }
        };
        // O = R + Aqk vtilde and the vtilde rows of the chunk staged in `cur`, into the out tiles
        auto out_o = [&](const char* cur) __attribute__((always_inline)) {
            const char* Al = cur + LT::A0;
            frag aa[KSC];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
                if (lower_step<Tr>(tc, ks)) aa[ks] = LdsA<Tr, LT::PT, 1>::load(Al, SL::perm(16 * tc + nn), ks, g);
#pragma unroll
            for (int i = 0; i < NOC; ++i) {
                const int oct = oc0 + i * OCS;
                if (oct >= NCOL) continue;
                frag vf[KSC];
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) vf[ks] = vb[(oct * KSC + ks) * 64 + lane];
                floatx4 o = R[i];
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks)
                    if (lower_step<Tr>(tc, ks)) o = Tr::mma(aa[ks], vf[ks], o);
                const int r0 = SL::perm(16 * tc + 4 * g), c = 16 * oct + nn;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    oo[out_row(r0 + e) * OW + c] = Tr::from_f(o[e]);
                    ov[out_row(r0 + e) * OW + c] = SL::acc_elem(vf, tc, e);
                }
            }
        };
        lds_char* const aA = lds_ptr(stA);
        lds_char* const aB = lds_ptr(stB);
        if (SEG && lw == 2 && unit.vzero) {                    // ordered before any read by the first chunk barrier
            constexpr int NV = C * LT::PV;              // 16-byte pieces of one V region
            for (int i = lane; i < NV; i += 64) {
                reinterpret_cast<uint4*>(stA + LT::V0)[i] = uint4{0u, 0u, 0u, 0u};
                if constexpr (NBUF == 2) reinterpret_cast<uint4*>(stB + LT::V0)[i] = uint4{0u, 0u, 0u, 0u};
            }
        }
        if constexpr (NBUF == 2) {
            if (NTu > 0) {
                issue(aA, 0, 0);
                issue(aA, 0, 1);
            }
            auto step = [&](lds_char* nxt, const char* cur, const char* prev, int64_t n) __attribute__((always_inline)) {
                const bool more = n + 1 < NTu;
                __builtin_amdgcn_s_waitcnt(0);          // chunk n has landed (and earlier stores left)
                lds_barrier();                          // B0
                // chunk n-1 (its Aqk rows are in the buffer refilled next):
                // read before the copies into that buffer are issued, which
                // later reads of the buffer would have to wait for
                if (n > 0) out_o(prev);
                if (more) issue(nxt, n + 1, 0);
                lds_barrier();                          // X
                if (more) issue(nxt, n + 1, 1);
                out_r(cur, n);                          // chunk n (its state operands stay until chunk n + 2)
                if (n > 0) copy_outs(n - 1);
            };
            for (int64_t n = 0; n < NTu; n += 2) {
                step(aB, stA, stB, n);
                if (n + 1 < NTu) step(aA, stB, stA, n + 1);
            }
        } else {
            for (int64_t n = 0; n < NTu; ++n) {
                lds_barrier();                          // B0': the chain waves are done with chunk n-1
                if (n > 0) out_o(stA);                  // chunk n-1, before its Aqk is overwritten
                lds_barrier();                          // B0'': every read of chunk n-1 is done
                issue(aA, n, 0);
                issue(aA, n, 1);
                if (n > 0) copy_outs(n - 1);
                __builtin_amdgcn_s_waitcnt(0);
                lds_barrier();                          // B0
                lds_barrier();                          // X
                out_r(stA, n);
            }
        }
        lds_barrier();                                  // E1: vtilde operands of the last chunk stored
        if (NTu > 0) out_o(NBUF == 2 && ((NTu - 1) & 1) ? stB : stA);
        lds_barrier();                                  // E2: out tiles of the last chunk written
        if (NTu > 0) copy_outs(NTu - 1);
        };
        switch (__builtin_amdgcn_readfirstlane(wave - NW)) {
        case 0: loader(std::integral_constant<int, 0>{}); break;
        case 1: loader(std::integral_constant<int, 1>{}); break;
        case 2: loader(std::integral_constant<int, 2>{}); break;
        default: loader(std::integral_constant<int, 3>{}); break;
        }
        return;
    }

    // ---- chain waves ----
    // The row part is a template constant of the wave's code, so that the
    // code of a chunk is straight-line (uniform branches on it would split
    // the chunk into small blocks, each waiting for its own LDS reads).
    const int cw = __builtin_amdgcn_readfirstlane(wave);
    const int ct = cw / RS;                           // column tile
    auto chain = [&](auto hc) __attribute__((always_inline)) {
    constexpr int h = decltype(hc)::value;            // row part
    const int col = col0 + 16 * ct + nn;
    const int td0 = h * NDH, ks0 = h * KSH;           // first state tile / contraction step owned

    // the wave's rows of S and M (fp32 accumulators; tile t holds state rows perm(16 (td0 + t) + 4g + e))
    // (split units: start state at unit.sin, or zero, or an identity block)
    const size_t sbase = SEG ? 0 : (size_t)unit.bh * D * D;
    floatx4 XS[NDH], XM[NDH];
    if constexpr (SEG) {
        const float* S0u = (S0 && unit.sin >= 0) ? S0 + unit.sin : nullptr;
        const float* M0u = (M0 && unit.sin >= 0) ? M0 + unit.sin : nullptr;
#pragma unroll
        for (int t = 0; t < NDH; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = SL::perm(16 * (td0 + t) + 4 * g + e);
                const size_t off = (size_t)row * D + col;
                XS[t][e] = S0u ? S0u[off] : (unit.ident == 1 && row == col ? 1.f : 0.f);
                XM[t][e] = M0u ? M0u[off] : (unit.ident == 2 && row == col ? 1.f : 0.f);
            }
    } else {
#pragma unroll
        for (int t = 0; t < NDH; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const size_t off = sbase + (size_t)SL::perm(16 * (td0 + t) + 4 * g + e) * D + col;
                XS[t][e] = S0 ? S0[off] : 0.f;
                XM[t][e] = M0 ? M0[off] : 0.f;
            }
    }
    int64_t spar = 0;                                 // parity of the chunk whose start state is stored next
    const int smo = ((ct * RS + h) * 2) * KSH * 64 + lane;
    // chunk-start state operands, for P and for the output waves; stored
    // before the chunk barrier, at the end of the previous chunk
    frag Sb[KSH], Mb[KSH];
    auto state_operands = [&]() __attribute__((always_inline)) {
        frag* const smS = sm[spar & 1] + smo;
        frag* const smM = smS + KSH * 64;
#pragma unroll
        for (int ks = 0; ks < KSH; ++ks) {
            Sb[ks] = SL::from_acc(XS, ks);
            Mb[ks] = SL::from_acc(XM, ks);
            smS[ks * 64] = Sb[ks];
            smM[ks * 64] = Mb[ks];
        }
        ++spar;
    };
    state_operands();

    auto chunk = [&](const char* cur) __attribute__((always_inline)) {
        if constexpr (NBUF == 1) {
            lds_barrier();                              // B0'
            lds_barrier();                              // B0''
        }
        lds_barrier();                                  // B0: chunk n staged
        const char* Kl = cur + LT::K0;
        const char* Tl = cur + LT::T0;
        const char* Vl = cur + LT::V0;
        const float* cf = reinterpret_cast<const float*>(cur + LT::CF0);

        // -- phase 1 --
        // T operands (for T V now and T W in phase 2); vtilde starts as T V
        frag tA[KSC][NCT];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc)
                if (lower_step<Tr>(tc, ks)) tA[ks][tc] = LdsA<Tr, LT::PT>::load(Tl, SL::perm(16 * tc + nn), ks, g);
        floatx4 Vx[NCT];
#pragma unroll
        for (int tc = 0; tc < NCT; ++tc) Vx[tc] = zero4();
        floatx4 P[NCT];
        {
            // P_h = -Diag(abar) K S_h + Diag(alpha b_prev) K M_h over the wave's rows
            floatx4 KSa[NCT], KMa[NCT];
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) { KSa[tc] = zero4(); KMa[tc] = zero4(); }
#pragma unroll
            for (int ks = 0; ks < KSH; ++ks) {
                frag a[NCT];
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) a[tc] = LdsA<Tr, LT::PK>::load(Kl, SL::perm(16 * tc + nn), ks0 + ks, g);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) {
                    KSa[tc] = Tr::mma(a[tc], Sb[ks], KSa[tc]);
                    KMa[tc] = Tr::mma(a[tc], Mb[ks], KMa[tc]);
                }
                if constexpr (KSH > 2) {                // bounds the K operands held at once
                    if (ks % 2 == 1) __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                const frag vB = VOperand<Tr, OW>::load(Vl, ct, ks, lane);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc)
                    if (lower_step<Tr>(tc, ks)) Vx[tc] = Tr::mma(tA[ks][tc], vB, Vx[tc]);
            }
            // first half of the state updates, while the chunk-start M is at hand
            {
                const float abarC = cf[MDN_COEF_ABAR * C + C - 1];
                const float bC = cf[MDN_COEF_B * C + C - 1];
                const float mubarC = expf(cf[MDN_COEF_LM * C + C - 1]);
#pragma unroll
                for (int t = 0; t < NDH; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        XS[t][e] = abarC * XS[t][e] - bC * XM[t][e];
                        XM[t][e] = mubarC * XM[t][e];
                    }
            }
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) {
                const floatx4 ca = crow(cf, MDN_COEF_ABAR, tc), cp = crow(cf, MDN_COEF_ABP, tc);
#pragma unroll
                for (int e = 0; e < 4; ++e) P[tc][e] = cp[e] * KMa[tc][e] - ca[e] * KSa[tc][e];
            }
        }
        if constexpr (RS > 1) {
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) xp[((ct * RS + h) * NCT + tc) * 64 + lane] = P[tc];
        }
        // gS, gM of the contraction slots, K^T operands of the wave's rows (for
        // phase 2; read before the barrier where the registers allow)
        float gs[KSC][NSL], gm[KSC][NSL];
        frag kT[KSC][NDH];
        auto read_update_operands = [&](int ks) __attribute__((always_inline)) {
            SL::load_row(cf + MDN_COEF_GS * C, ks, g, gs[ks]);
            SL::load_row(cf + MDN_COEF_GM * C, ks, g, gm[ks]);
#pragma unroll
            for (int t = 0; t < NDH; ++t) kT[ks][t] = KtOperand<Tr, LT::PK>::load(Kl, td0 + t, ks, lane);
        };
        constexpr bool EARLY = KSC * (NDH * sizeof(frag) / 4 + 2 * NSL) <= 64;
        if constexpr (EARLY) {
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) read_update_operands(ks);
        }
        lds_barrier();                                  // X: partial products visible

        // -- phase 2 --
        if constexpr (RS > 1) {                         // W - V = P_0 + P_1
#pragma unroll
            for (int h2 = 0; h2 < RS; ++h2) {
                if (h2 == h) continue;                  // uniform
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) {
                    const floatx4 o = xp[((ct * RS + h2) * NCT + tc) * 64 + lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e) P[tc][e] += o[e];
                }
            }
        }
        // vtilde = T V + T (W - V)
        {
            frag Wb[KSC];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) Wb[ks] = SL::from_acc(P, ks);
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc)
                    if (lower_step<Tr>(tc, ks)) Vx[tc] = Tr::mma(tA[ks][tc], Wb[ks], Vx[tc]);
        }
        // S_h += K_h^T Diag(gS) vtilde;  M_h -= K_h^T Diag(gM) vtilde, one
        // contraction step at a time (with the operands read just before
        // where they were not read ahead)
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            if constexpr (!EARLY) read_update_operands(ks);
#pragma unroll
            for (int j = 0; j < NSL; ++j) gm[ks][j] = -gm[ks][j];
            const frag VS = SL::from_acc_scaled(Vx, ks, gs[ks]);
            const frag VM = SL::from_acc_scaled(Vx, ks, gm[ks]);
#pragma unroll
            for (int t = 0; t < NDH; ++t) {
                XS[t] = Tr::mma(kT[ks][t], VS, XS[t]);
                XM[t] = Tr::mma(kT[ks][t], VM, XM[t]);
            }
            if constexpr (!EARLY) __builtin_amdgcn_sched_barrier(0);
        }
        // vtilde operands for the output waves (the row parts share the steps)
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks)
            if (ks % RS == h) vb[(ct * KSC + ks) * 64 + lane] = SL::from_acc(Vx, ks);
        state_operands();                               // of the next chunk
    };

    if constexpr (NBUF == 2) {
        for (int64_t n = 0; n < NTu; n += 2) {
            chunk(stA);
            if (n + 1 < NTu) chunk(stB);
        }
    } else {
        for (int64_t n = 0; n < NTu; ++n) chunk(stA);
    }
    lds_barrier();                                      // E1
    lds_barrier();                                      // E2

    // (the identity replicas of the split store theirs transposed, [col][row],
    // the layout the combine step reads them in)
    if (!SEG || unit.sout >= 0) {
        const size_t obase = SEG ? (size_t)unit.sout : sbase;
        const bool tr = SEG && unit.ident != 0;
#pragma unroll
        for (int t = 0; t < NDH; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const size_t row = (size_t)SL::perm(16 * (td0 + t) + 4 * g + e);
                const size_t off = obase + (tr ? (size_t)col * D + row : row * D + col);
                ST[off] = XS[t][e];
                MT[off] = XM[t][e];
            }
    }
    };
    if constexpr (RS == 1) {
        chain(std::integral_constant<int, 0>{});
    } else {
        if (cw % RS == 0) chain(std::integral_constant<int, 0>{});
        else chain(std::integral_constant<int, 1>{});
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// Compute units of the current device.  Queried on every call (a lookup in
// the runtime's device properties), so the library keeps no mutable state.
static int device_cus()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}
int device_compute_units() { return device_cus(); }

// One launch of the inter stage.  `units` is the number of state units the
// grid covers: heads of a [B, H, T] batch, (sequence, head) pairs of a packed
// batch, or the units of one pass of the sequence split (seg.P > 0), whose
// start and end states are read from S0/M0 and written to ST/MT at the
// offsets the unit map gives.
struct InterLaunch {
    int64_t units;
    InterSeg seg;
    const float *S0, *M0;
    float *ST, *MT;
};

template <typename Tr, int D, int C, int NCOL, int RS>
static hipError_t launch_inter_cols(const ChunkArgs& a, const InterLaunch& l)
{
    using E = typename Tr::elem;
    using P = InterPick<Tr, D, C>;
    constexpr int NLD = 4;
    constexpr int NBUF = InterLayout<Tr, D, C, NCOL, RS, 2>::TOTAL <= P::LIMIT ? 2 : 1;
    static_assert(InterLayout<Tr, D, C, NCOL, RS, NBUF>::TOTAL <= P::LIMIT, "LDS");
    const int64_t grid = l.units * (D / (16 * NCOL));
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * (NCOL * RS + NLD)), 0, (hipStream_t)a.stream,
                           (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.Tmat, (const E*)a.Aqk, a.coef,
                           l.S0, l.M0, (E*)a.O, l.ST, l.MT, (E*)a.Vt, a.T, a.NT, (int)l.units, a.cu, a.perm,
                           (int)a.BH, l.seg);
    };
    if (l.seg.P > 0) go(mdn_inter_kernel<Tr, D, C, NCOL, RS, NBUF, NLD, true>);
    else go(mdn_inter_kernel<Tr, D, C, NCOL, RS, NBUF, NLD, false>);
    return hipGetLastError();
}

// When the grid of two-tile slabs would occupy at most half of the compute
// units (few heads), the launch takes one-tile slabs, so that each chain
// wave has a compute unit's loaders and LDS to itself, and at dk >= 64 it
// splits each tile's rows over two chain waves, which shortens the per-chunk
// chain that bounds such a launch.  The price is reading K, Q, T and Aqk
// once more per head and the partial-product exchange of the row split.
template <typename Tr, int D, int C>
static hipError_t launch_inter_nw(const ChunkArgs& a, const InterLaunch& l)
{
    using P = InterPick<Tr, D, C>;
    if constexpr (P::NCOL == 2 && P::RS == 1) {
        if (2 * l.units * (D / 32) <= device_cus()) return launch_inter_cols<Tr, D, C, 1, (D >= 64 ? 2 : 1)>(a, l);
    }
    return launch_inter_cols<Tr, D, C, P::NCOL, P::RS>(a, l);
}

template <typename Tr>
static hipError_t inter_dispatch(const ChunkArgs& a, const InterLaunch& l)
{
    if constexpr (std::is_same<Tr, TraitsBf16>::value) {
        switch (a.dk * 1000 + a.C) {
        case 32032: return launch_inter_nw<Tr, 32, 32>(a, l);
        case 32064: return launch_inter_nw<Tr, 32, 64>(a, l);
        case 64032: return launch_inter_nw<Tr, 64, 32>(a, l);
        case 64064: return launch_inter_nw<Tr, 64, 64>(a, l);
        case 128032: return launch_inter_nw<Tr, 128, 32>(a, l);
        case 128064: return launch_inter_nw<Tr, 128, 64>(a, l);
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (a.dk * 1000 + a.C) {
        case 16016: return launch_inter_nw<Tr, 16, 16>(a, l);
        case 16032: return launch_inter_nw<Tr, 16, 32>(a, l);
        case 16064: return launch_inter_nw<Tr, 16, 64>(a, l);
        case 32016: return launch_inter_nw<Tr, 32, 16>(a, l);
        case 32032: return launch_inter_nw<Tr, 32, 32>(a, l);
        case 32064: return launch_inter_nw<Tr, 32, 64>(a, l);
        case 64016: return launch_inter_nw<Tr, 64, 16>(a, l);
        case 64032: return launch_inter_nw<Tr, 64, 32>(a, l);
        case 64064: return launch_inter_nw<Tr, 64, 64>(a, l);
        case 128016: return launch_inter_nw<Tr, 128, 16>(a, l);
        case 128032: return launch_inter_nw<Tr, 128, 32>(a, l);
        case 128064: return launch_inter_nw<Tr, 128, 64>(a, l);
        default: return hipErrorInvalidValue;
        }
    }
}

hipError_t launch_chunk_inter(const ChunkArgs& a)
{
    if (a.BH == 0 || (a.cu && a.nseq == 0)) return hipSuccess;
    const InterLaunch l{a.cu ? a.BH * a.nseq : a.BH, InterSeg{0, 0}, a.S0, a.M0, a.ST, a.MT};
    return a.dtype == MDN_BF16 ? inter_dispatch<TraitsBf16>(a, l) : inter_dispatch<TraitsF32>(a, l);
}

// ---------------------------------------------------------------------------
// Sequence split: the combine step between the two passes.  Per sequence s
// and middle segment p - 1 (p = 2 .. P-1), in order of p:
//   [S; M]_p = Phi [S; M]_{p-1} + offset,   Phi = [[A_S, B_S], [A_M, B_M]]
// where (A_S, A_M), (B_S, B_M) and the offset are the end states of pass-1
// replicas 1, 2 and 0 of segment p - 1 (the replicas' stored transposed,
// A^T[k][r]), and [S; M]_1 is the end state of segment 0.  One workgroup per
// (sequence, 16 state columns) keeps the columns' [S; M]_{p-1} (2D x 16,
// fp32) in LDS; thread r forms row r of the result, so for each k the
// threads read consecutive elements of A^T[k] and B^T[k], and every thread
// reads the same X row (an LDS broadcast).  Slots are D x D fp32 blocks of
// `segS` / `segM`: pass-1 slot s U1 + j, the results at H U1 + s (P - 2) +
// p - 2.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(2 * D * 4) void mdn_seg_combine_kernel(float* __restrict__ segS, float* __restrict__ segM,
                                                                    int H, int P)
{
    constexpr int CB = 16, NB = D / CB;
    constexpr int KQ = 4, KL = D / KQ;                 // contraction quarters, steps per quarter
    __shared__ __attribute__((aligned(16))) float X[2 * D][CB];
    __shared__ __attribute__((aligned(16))) float red[KQ - 1][2 * D][CB];   // partial sums of quarters 1..3
    const int s = blockIdx.x / NB, c0 = (blockIdx.x % NB) * CB;
    const int U1 = 1 + 3 * (P - 2);
    const int64_t DD = (int64_t)D * D;
    const int tid = threadIdx.x;
    const int r = tid % (2 * D), kq = tid / (2 * D);   // row of [S; M], contraction quarter
    float* const base = r < D ? segS : segM;
    const int rr = r % D;
    for (int i = tid; i < 2 * D * CB; i += 2 * D * KQ) {
        const int xr = i / CB, c = i % CB;
        X[xr][c] = (xr < D ? segS : segM)[(int64_t)s * U1 * DD + (int64_t)(xr % D) * D + c0 + c];
    }
    for (int p = 2; p < P; ++p) {
        const int64_t j0 = (int64_t)s * U1 + 1 + 3 * (p - 2);
        // this quarter's A^T[k][rr], B^T[k][rr], all in flight at once
        const float* aT = base + (j0 + 1) * DD + rr + (int64_t)kq * KL * D;
        const float* bT = base + (j0 + 2) * DD + rr + (int64_t)kq * KL * D;
        float av[KL], bv[KL];
#pragma unroll
        for (int k = 0; k < KL; ++k) {
            av[k] = aT[(int64_t)k * D];
            bv[k] = bT[(int64_t)k * D];
        }
        float acc[CB];
        if (kq == 0) {
            const float* off = base + j0 * DD + (int64_t)rr * D + c0;
#pragma unroll
            for (int c = 0; c < CB; c += 4) {
                const float4 o = *reinterpret_cast<const float4*>(off + c);
                acc[c] = o.x; acc[c + 1] = o.y; acc[c + 2] = o.z; acc[c + 3] = o.w;
            }
        } else {
#pragma unroll
            for (int c = 0; c < CB; ++c) acc[c] = 0.f;
        }
        __syncthreads();                               // X_{p-1} complete
#pragma unroll
        for (int k = 0; k < KL; ++k) {
            const int kk = kq * KL + k;
#pragma unroll
            for (int c = 0; c < CB; c += 4) {
                const float4 xs = *reinterpret_cast<const float4*>(&X[kk][c]);
                const float4 xm = *reinterpret_cast<const float4*>(&X[D + kk][c]);
                acc[c] = fmaf(av[k], xs.x, fmaf(bv[k], xm.x, acc[c]));
                acc[c + 1] = fmaf(av[k], xs.y, fmaf(bv[k], xm.y, acc[c + 1]));
                acc[c + 2] = fmaf(av[k], xs.z, fmaf(bv[k], xm.z, acc[c + 2]));
                acc[c + 3] = fmaf(av[k], xs.w, fmaf(bv[k], xm.w, acc[c + 3]));
            }
        }
        if (kq > 0) {
#pragma unroll
            for (int c = 0; c < CB; c += 4)
                *reinterpret_cast<float4*>(&red[kq - 1][r][c]) = float4{acc[c], acc[c + 1], acc[c + 2], acc[c + 3]};
        }
        __syncthreads();                               // partial sums written, every read of X_{p-1} done
        if (kq == 0) {
            const int64_t out = (int64_t)H * U1 + (int64_t)s * (P - 2) + p - 2;
            float* dst = base + out * DD + (int64_t)rr * D + c0;
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                const float v = acc[c] + red[0][r][c] + red[1][r][c] + red[2][r][c];
                X[r][c] = v;
                dst[c] = v;
            }
        }
    }
}

hipError_t launch_chunk_inter_split(const ChunkArgs& a, int P, float* segS, float* segM)
{
    if (a.BH == 0) return hipSuccess;
    auto run = [&](const InterLaunch& l) {
        return a.dtype == MDN_BF16 ? inter_dispatch<TraitsBf16>(a, l) : inter_dispatch<TraitsF32>(a, l);
    };
    const int U1 = 1 + 3 * (P - 2);
    hipError_t e = run(InterLaunch{a.BH * U1, InterSeg{P, 1}, a.S0, a.M0, segS, segM});
    if (e != hipSuccess) return e;
    if (P > 2) {
        const int NB = a.dk / 16;
        switch (a.dk) {
        case 16: hipLaunchKernelGGL(mdn_seg_combine_kernel<16>, dim3((unsigned)(a.BH * NB)), dim3(2 * a.dk * 4), 0, (hipStream_t)a.stream, segS, segM, (int)a.BH, P); break;
        case 32: hipLaunchKernelGGL(mdn_seg_combine_kernel<32>, dim3((unsigned)(a.BH * NB)), dim3(2 * a.dk * 4), 0, (hipStream_t)a.stream, segS, segM, (int)a.BH, P); break;
        case 64: hipLaunchKernelGGL(mdn_seg_combine_kernel<64>, dim3((unsigned)(a.BH * NB)), dim3(2 * a.dk * 4), 0, (hipStream_t)a.stream, segS, segM, (int)a.BH, P); break;
        case 128: hipLaunchKernelGGL(mdn_seg_combine_kernel<128>, dim3((unsigned)(a.BH * NB)), dim3(2 * a.dk * 4), 0, (hipStream_t)a.stream, segS, segM, (int)a.BH, P); break;
        default: return hipErrorInvalidValue;
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return run(InterLaunch{a.BH * (P - 1), InterSeg{P, 2}, segS, segM, a.ST, a.MT});
}

}  // namespace mdn
