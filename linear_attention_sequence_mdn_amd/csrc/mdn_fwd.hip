// mdn_fwd.hip -- the chunkwise Momentum DeltaNet forward in one kernel
// (gfx950; bf16 operands, chunk size 64, dk = dv in {64, 128}).
//
// It computes what mdn_intra_kernel followed by mdn_inter_kernel computes
// (the MDN summary at paper.rainbus.top, method walk-through steps 2-5; the
// equations are listed at the top of mdn_chunk.hip), but the per-chunk
// intermediates -- the coefficient rows, Gamma, A, T and Aqk -- never leave
// the compute unit: HBM sees q, k, v and the gates once, O and vtilde once,
// and the states, and no workspace is needed.
//
// One workgroup owns a slab of 32 state columns of one head and runs the
// chunks of the head in order with eight waves (wave w on SIMD w % 4):
//   waves 0, 1  the chains of column tiles 0, 1: S and M in fp32 registers,
//               vtilde and the state update of chunk m as in the inter
//               kernel, reading T, K, V and the coefficient rows of chunk m
//               from LDS;
//   waves 2, 3  copies and output for token tiles {w, w + 2}: the global ->
//               LDS copies of K (two chunks ahead) and the V slab (one
//               ahead), the gates (wave 2, three chunks ahead, with their
//               wave scans), then per chunk O = R + Aqk vtilde of chunk m-1,
//               and Aqk = (K Q^T) o Gamma and R = Diag(abar) Q S - Diag(b) Q M
//               of chunk m from Q rows loaded into registers;
//   waves 4-7   the intra step of chunk m+1 while the chains run chunk m:
//               the coefficient rows, column block w - 4 of Gamma (a
//               per-column recurrence whose every term is non-negative), of
//               A = (Diag(alpha) K K^T) o Gamma^- and of T = (I + A)^{-1}
//               (the diagonal block by forward substitution in registers, the
//               blocks below it by block forward substitution on the matrix
//               cores).
// One workgroup barrier per chunk.  The intra waves also meet among
// themselves on a counter in LDS (the other waves never wait on it), and
// they overwrite Gamma only after both output waves have counted that they
// read it.  Those waits are bounded spins.
//
// Measured on the 400M-layer shape it takes 0.257-0.265 ms against 0.20-0.21
// ms for the two-kernel forward: each of a head's four workgroups runs the
// head's whole intra step, and the workgroup's LDS traffic (about 450 KB per
// chunk) slows every stage.  It is the forward for callers that cannot give
// a workspace or want the HBM traffic of the path's own bytes.
#include "mdn_device.h"
#include "mdn_internal.h"
#include "mdn_lds.h"
#include "../../include/mdn.h"

namespace mdn {

template <int D, int C, int NCOL, int RS>
struct FwdLayout {
    using Tr = TraitsBf16;
    using frag = bf16x8;
    static constexpr int ES = 2, FS = 16;
    static constexpr int PK = D * ES / 16;            // 16-byte pieces per K row
    static constexpr int PT = C * ES / 16;            // pieces per T row
    static constexpr int PV = 16 * NCOL * ES / 16;    // pieces per V-slab / out row
    static constexpr int NCT = C / 16, KSC = C / 32, KSD = D / 32;
    static constexpr int KSH = D / RS / 32;
    static constexpr int KB = C * PK * 16;            // one staged K tile
    static constexpr int VB = C * PV * 16;            // one staged V slab
    static constexpr int GB = 4 * C * 4;              // one chunk's gates: alpha, mu, beta, eta rows
    static constexpr int TB = C * PT * 16;            // one T tile (bf16, swizzled rows)
    static constexpr int CFB = MDN_COEF_ROWS * C * 4; // one chunk's coefficient rows
    static constexpr int GAMB = C * C * 4;            // Gamma, fp32, column-major
    static constexpr int AB = C * C * 4;              // A, fp32, row-major, XOR-swizzled by row
    static constexpr int SMB = NCOL * RS * 2 * KSH * 64 * FS;   // chunk-start S, M operands (one parity)
    static constexpr int VTB = NCOL * KSC * 64 * FS;            // vtilde operands (one parity)
    static constexpr int OUTB = C * PV * 16;                    // one out tile
    static constexpr int XPB = RS > 1 ? NCOL * RS * NCT * 64 * 16 : 16;
    static constexpr int TOTAL = 3 * KB + 2 * VB + 2 * GB + 2 * TB + 2 * CFB + GAMB + AB + 2 * SMB + 2 * VTB +
                                 2 * OUTB + XPB + 16;
    static constexpr int LIMIT = 160 * 1024;
};

// A[r][i] (fp32) sits at word r*C + (i ^ ((r & 15) << 2)): the 16 rows that
// one matrix-core operand read touches fall in different bank groups, and
// every aligned group of four columns stays contiguous.
template <int C>
__device__ __forceinline__ int a_idx(int r, int i) { return r * C + (i ^ ((r & 15) << 2)); }

// Row r of an out tile is stored at row fwd_out_row(r), so that the 2-byte
// column writes of the four lane groups (rows 8 apart) fall in different
// banks.  The map is its own inverse.
__device__ __forceinline__ int fwd_out_row(int r) { return r ^ ((r >> 3) & 3); }

// Barrier of the four intra waves alone: they meet on a counter in LDS.
// Every intra wave calls it the same number of times; `target` is four
// times the number of calls so far.  The spin is bounded, so that a wave
// never waits forever whatever happens.
// The data these counters order lives in LDS, whose operations complete in
// order per wave: waiting for this wave's LDS operations (lgkmcnt) before
// the increment is the release, and issuing the later LDS operations after
// the count is seen is the acquire.  (A release atomic would also wait for
// every outstanding global load and copy of the wave.)
__device__ __forceinline__ void count_up(unsigned* ctr, int lane)
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");      // this wave's LDS reads and writes are done
    if (lane == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    asm volatile("" ::: "memory");
}

// Waits (bounded) until a counter in LDS reaches `target`.
__device__ __forceinline__ void wait_count(unsigned* ctr, unsigned target)
{
    for (int it = 0; it < (1 << 24); ++it) {
        if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

__device__ __forceinline__ void group_sync(unsigned* ctr, unsigned target, int lane)
{
    count_up(ctr, lane);
    wait_count(ctr, target);
}

// out[t] = x of lane t of this lane's 16-lane row (DPP row broadcast)
template <int... Q>
__device__ __forceinline__ void row_bcast_all(float x, float (&out)[16], std::integer_sequence<int, Q...>)
{
    ((out[Q] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + Q, 0xf, 0xf, false))), ...);
}

// Orders this wave's earlier LDS writes before its later LDS reads of data
// that other lanes of the same wave wrote.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int D, int C, int NCOL, int RS>
__global__ __launch_bounds__(64 * (NCOL * RS + 6))
void mdn_fwd_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                    const float* __restrict__ alpha, const float* __restrict__ mu,
                    const float* __restrict__ beta, const float* __restrict__ eta,
                    const float* __restrict__ S0, const float* __restrict__ M0,
                    __bf16* __restrict__ O, float* __restrict__ ST, float* __restrict__ MT,
                    __bf16* __restrict__ Vt, int64_t T, int BH)
{
    using Tr = TraitsBf16;
    using E = __bf16;
    using SL = Slots<Tr>;
    using L = FwdLayout<D, C, NCOL, RS>;
    using frag = bf16x8;
    constexpr int NLD = 4;
    constexpr int NW = NCOL * RS;                     // chain waves
    constexpr int NCT = L::NCT, KSC = L::KSC, KSD = L::KSD;
    constexpr int DH = D / RS, NDH = DH / 16, KSH = DH / 32;
    constexpr int SLABS = D / (16 * NCOL);
    constexpr int OW = 16 * NCOL;                     // out-tile row length (elements)
    static_assert(C == 64 && NCT == NLD, "one column block of Gamma, A and T per intra wave");
    static_assert(L::TOTAL <= L::LIMIT, "LDS");
    static_assert(RS == 1, "row split not built in the single-kernel forward");

    __shared__ __attribute__((aligned(16))) char kst[3 * L::KB];       // K tiles of chunks m, m+1, m+2
    __shared__ __attribute__((aligned(16))) char vst[2 * L::VB];       // V slabs by chunk parity
    __shared__ __attribute__((aligned(16))) float gst[2][4][C];        // gates by chunk parity
    __shared__ __attribute__((aligned(16))) float sst[2][3][C];        // their scans: LA, LM, b
    __shared__ __attribute__((aligned(16))) char tst[2 * L::TB];       // T by chunk parity
    __shared__ __attribute__((aligned(16))) float cst[2][MDN_COEF_ROWS * C];   // coefficient rows by parity
    __shared__ __attribute__((aligned(16))) float gam[C * C];          // Gamma of the chunk being prepared
    __shared__ __attribute__((aligned(16))) float amat[C * C];         // A, then T's diagonal blocks
    __shared__ __attribute__((aligned(16))) frag sm[2][NW * 2 * KSH * 64];   // chunk-start S, M operands
    __shared__ __attribute__((aligned(16))) frag vb[2][NCOL * KSC * 64];      // vtilde operands
    __shared__ __attribute__((aligned(16))) E oo[C * OW];              // O out tile
    __shared__ __attribute__((aligned(16))) E ov[C * OW];              // vtilde out tile
    __shared__ unsigned lbar;                                          // intra-wave barrier counter
    __shared__ unsigned gfree;                                         // output waves done reading Gamma

    const int tid = threadIdx.x, lane = tid & 63, hw = tid >> 6;
    const int g = lane >> 4, nn = lane & 15;
    // Roles: waves 0 .. NW-1 carry the chains, waves NW, NW+1 copy and form
    // the output, waves NW+2 .. NW+5 run the intra step.  Waves go to the four
    // SIMDs round robin (wave w on SIMD w % 4): the output waves have SIMDs 2
    // and 3, and every SIMD runs one intra wave.
    const int role = __builtin_amdgcn_readfirstlane(hw);   // 0..NW-1: chain wave, then output and intra waves

    int bh, slab;
    xcd_head_map(blockIdx.x, SLABS, BH, bh, slab);
    const int64_t row0 = (int64_t)bh * T;
    const int col0 = slab * OW;
    const int64_t NTu = (T + C - 1) / C;
    auto valid_of = [&](int64_t n) { return (int)((T - n * C) < C ? (T - n * C) : C); };
    auto crow = [&](const float* cf, int which, int tc) __attribute__((always_inline)) {
        return *reinterpret_cast<const floatx4*>(cf + which * C + SL::perm(16 * tc + 4 * g));
    };

    if (role == NW && lane == 0) {
        lbar = 0u;
        gfree = 0u;
    }
    lds_barrier();                                    // B_init

    if (role >= NW) {
        // waves NW, NW+1: output (SIMDs 2, 3); waves NW+2 .. NW+5: intra
        // waves of column blocks 0..3, one on each SIMD
        const int r2 = role - NW;
        if (r2 < 2) {
        // =========================== output waves ===========================
        auto output = [&](auto owc) __attribute__((always_inline)) {
        constexpr int ow = decltype(owc)::value;
        constexpr int TT[2] = {ow, ow + 2};           // token tiles (one light, one heavy in Aqk)
        // K rows [32 ow, 32 ow + 32) of chunk n into K buffer n % 3 (rows past
        // the end repeat the last valid row)
        auto issue_k = [&](int64_t n) __attribute__((always_inline)) {
            const unsigned vlast = (unsigned)valid_of(n) - 1;
            auto seq_row = [&](unsigned r) { return (r < vlast ? r : vlast) * (unsigned)(D * 2); };
            dma_tile_p<32, L::PK>(lds_ptr(kst) + (n % 3) * L::KB,
                                  reinterpret_cast<const char*>(k + (row0 + n * C) * D), seq_row, lane, 32 * ow);
        };
        // the V slab of chunk n: rows [32 ow, 32 ow + 32)
        auto issue_v = [&](int64_t n) __attribute__((always_inline)) {
            const unsigned vlast = (unsigned)valid_of(n) - 1;
            auto seq_row = [&](unsigned r) { r += 32 * ow; return (r < vlast ? r : vlast) * (unsigned)(D * 2); };
            dma_plain_p<32, L::PV>(lds_ptr(vst) + (n & 1) * L::VB + 32 * ow * L::PV * 16,
                                   reinterpret_cast<const char*>(v + (row0 + n * C) * D + col0), seq_row, lane);
        };
        // the Q rows perm(16 tc + nn) of both token tiles of chunk n, as
        // matrix-core operands
        auto load_q = [&](frag (&qa)[2][KSD], int64_t n) __attribute__((always_inline)) {
            const int vl = valid_of(n);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                int r = SL::perm(16 * TT[u] + nn);
                r = r < vl ? r : vl - 1;
                const E* qr = q + (row0 + n * C + r) * D;
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) qa[u][ks] = Contig<Tr>::load(qr, ks, g);
            }
        };
        // the gates of chunk n, one token per lane (output wave 0 only); the
        // loads are only issued here and consumed a chunk later
        auto load_gates = [&](int64_t n, floatx4& x) __attribute__((always_inline)) {
            const int vl = valid_of(n);
            const int64_t off = row0 + n * C + (lane < vl ? lane : vl - 1);
            x[0] = alpha[off];
            x[1] = mu[off];
            x[2] = beta[off];
            x[3] = eta[off];
        };
        // stores chunk n's gates, with the neutral values alpha = mu = 1,
        // beta = eta = 0 past the end (they leave every quantity unchanged),
        // and their 64-lane scans (parity par): the cumulative logs LA, LM and
        // b_r = alpha_r b_{r-1} + beta_r mubar_r (an affine scan, every term
        // non-negative)
        auto put_gates = [&](int par, int64_t n, floatx4 x) __attribute__((always_inline)) {
            if (lane >= valid_of(n)) x = floatx4{1.f, 1.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 4; ++u) gst[par][u][lane] = x[u];
            const float la = wave_scan_add(logf(x[0]));
            const float lm = wave_scan_add(logf(x[1]));
            float Aa = x[0], Bv = x[2] * expf(lm);
            wave_scan_affine(Aa, Bv);
            sst[par][0][lane] = la;
            sst[par][1][lane] = lm;
            sst[par][2][lane] = Bv;
        };

        floatx4 gsl[2][NCT];                           // Gamma[query][key] of the chunk being output
        floatx4 R[2][NCOL];
        frag aa[2][KSC];                               // Aqk of both token tiles (A operands)
        // Gamma[perm(16 tc + nn)][perm(16 t + 4 g) + e] for the token tiles'
        // Aqk.  Under the slot map, key tiles 0 and 1 hold rows 0..31 and
        // tiles 2 and 3 rows 32..63, so a query tile meets the key tiles of
        // its own half and of the halves before it (keys after the query are
        // zero in Gamma).
        auto read_gamma = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tc = TT[u];
#pragma unroll
                for (int t = 0; t < NCT; ++t) {
                    if ((t >> 1) <= (tc >> 1)) {
                        const int rq = SL::perm(16 * tc + nn), i0 = SL::perm(16 * t + 4 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e) gsl[u][t][e] = gam[(i0 + e) * C + rq];
                    }
                }
            }
        };
        // Aqk of chunk n: (K Q^T) o Gamma, keys perm(16 t + x) as accumulator
        // rows; key tiles of later halves are zero
        auto aqk = [&](int64_t n, const frag (&qn)[2][KSD]) __attribute__((always_inline)) {
            const char* Kl = kst + (n % 3) * L::KB;
            floatx4 Dk[2][NCT];
#pragma unroll
            for (int t = 0; t < NCT; ++t) {
                Dk[0][t] = zero4();
                Dk[1][t] = zero4();
                // key tile t meets token tile TT[u] when (t >> 1) <= (TT[u] >> 1);
                // TT[1] = ow + 2 meets every key tile
                const bool both = (t >> 1) <= (TT[0] >> 1);
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    const frag kk = LdsA<Tr, L::PK>::load(Kl, SL::perm(16 * t + nn), ks, g);
                    if (both) Dk[0][t] = Tr::mma(kk, qn[0][ks], Dk[0][t]);
                    Dk[1][t] = Tr::mma(kk, qn[1][ks], Dk[1][t]);
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int t = 0; t < NCT; ++t)
                    if ((t >> 1) <= (TT[u] >> 1)) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) Dk[u][t][e] *= gsl[u][t][e];
                    }
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) aa[u][ks] = SL::from_acc(Dk[u], ks);
            }
        };
        // R = Diag(abar) Q S - Diag(b) Q M of chunk n over all dk rows; each
        // state operand read once for both token tiles
        auto out_r = [&](int64_t n, const frag (&qn)[2][KSD]) __attribute__((always_inline)) {
            const frag* smp = sm[n & 1];
            const float* cf = cst[n & 1];
#pragma unroll
            for (int oct = 0; oct < NCOL; ++oct) {
                floatx4 qs[2] = {zero4(), zero4()}, qm[2] = {zero4(), zero4()};
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    const int base = ((oct * RS + ks / KSH) * 2) * KSH * 64 + (ks % KSH) * 64 + lane;
                    const frag sS = smp[base], sM = smp[base + KSH * 64];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        qs[u] = Tr::mma(qn[u][ks], sS, qs[u]);
                        qm[u] = Tr::mma(qn[u][ks], sM, qm[u]);
                    }
                }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const floatx4 ca = crow(cf, MDN_COEF_ABAR, TT[u]), cb = crow(cf, MDN_COEF_B, TT[u]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) R[u][oct][e] = ca[e] * qs[u][e] - cb[e] * qm[u][e];
                }
            }
        };
        // O = R + Aqk vtilde and vtilde of chunk n for both token tiles: into
        // the out tiles, then these rows to HBM
        auto out_o = [&](int64_t n) __attribute__((always_inline)) {
            const frag* vbp = vb[n & 1];
#pragma unroll
            for (int oct = 0; oct < NCOL; ++oct) {
                frag vf[KSC];
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) vf[ks] = vbp[(oct * KSC + ks) * 64 + lane];
                const int c = 16 * oct + nn;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    floatx4 o = R[u][oct];
#pragma unroll
                    for (int ks = 0; ks < KSC; ++ks) o = Tr::mma(aa[u][ks], vf[ks], o);
                    const int r0 = SL::perm(16 * TT[u] + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        oo[fwd_out_row(r0 + e) * OW + c] = Tr::from_f(o[e]);
                        ov[fwd_out_row(r0 + e) * OW + c] = SL::acc_elem(vf, TT[u], e);
                    }
                }
            }
            wave_lds_sync();
            // rows perm(16 tc + x), x = 0..15, of both tiles: PV pieces each
            constexpr int NP = 16 * L::PV;
            const int vl = valid_of(n);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (NP == 64 || lane < NP) {
                    const int x = lane / L::PV, p = lane % L::PV;
                    const int r = SL::perm(16 * TT[u] + x), ro = fwd_out_row(r);
                    const uint4 po = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(oo) + (ro * L::PV + p) * 16);
                    const uint4 pv = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(ov) + (ro * L::PV + p) * 16);
                    if (r < vl) {
                        const size_t off = (size_t)(row0 + n * C + r) * D + col0 + p * 8;
                        *reinterpret_cast<uint4*>(O + off) = po;
                        *reinterpret_cast<uint4*>(Vt + off) = pv;
                    }
                }
            }
        };

        // -- prologue: chunks 0 and 1 staged (K, gates), V and Q of chunk 0 --
        floatx4 gn = zero4();                          // gates of chunk m + 2, stored at B0(m)
        if (NTu > 0) {
            issue_k(0);
            if (NTu > 1) issue_k(1);
            issue_v(0);
            if constexpr (ow == 0) {
                floatx4 g0 = zero4(), g1 = zero4();
                load_gates(0, g0);
                if (NTu > 1) load_gates(1, g1);
                if (NTu > 2) load_gates(2, gn);
                __builtin_amdgcn_s_waitcnt(0);
                put_gates(0, 0, g0);
                if (NTu > 1) put_gates(1, 1, g1);
            }
            __builtin_amdgcn_s_waitcnt(0);
        }
        lds_barrier();                                 // B_pro: chunk 0 staged for the intra waves
        auto step = [&](int64_t m, auto par) __attribute__((always_inline)) {
            constexpr int P = decltype(par)::value;    // m & 1
            __builtin_amdgcn_s_waitcnt(0);             // this wave's copies, loads and stores are done
            lds_barrier();                             // B0(m)
            read_gamma();                              // chunk m's Gamma, before the intra waves overwrite it
            count_up(&gfree, lane);
            frag qa[2][KSD];                           // this chunk's Q rows of both token tiles
            load_q(qa, m);                             // in flight while chunk m-1 is finished
            if (m > 0) out_o(m - 1);
            aqk(m, qa);
            out_r(m, qa);
            if constexpr (ow == 0) {
                if (m + 2 < NTu) put_gates(P, m + 2, gn);   // chunk m + 2 (parity P)
            }
            // The copies go out after this step's LDS work: the compiler
            // makes every later LDS access of the wave wait for them.
            if (m + 2 < NTu) issue_k(m + 2);
            if (m + 1 < NTu) issue_v(m + 1);
            if constexpr (ow == 0) {
                if (m + 3 < NTu) load_gates(m + 3, gn);
            }
        };
        for (int64_t m = 0; m < NTu; m += 2) {
            step(m, std::integral_constant<int, 0>{});
            if (m + 1 < NTu) step(m + 1, std::integral_constant<int, 1>{});
        }
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();                                 // E1: vtilde operands of the last chunk stored
        if (NTu > 0) out_o(NTu - 1);
        };
        if (r2 == 0) output(std::integral_constant<int, 0>{});
        else output(std::integral_constant<int, 1>{});
        return;
        }

        // ============================ intra waves ============================
        auto intra_wave = [&](auto wc) __attribute__((always_inline)) {
        constexpr int w = decltype(wc)::value;        // column block of Gamma, A and T
        unsigned nsync = 0;
        auto lsync = [&]() __attribute__((always_inline)) { nsync += NLD; group_sync(&lbar, nsync, lane); };
        auto intra = [&](int64_t n) __attribute__((always_inline)) {
            const char* Kl = kst + (n % 3) * L::KB;
            const float (*G)[C] = gst[n & 1];
            const int vl = valid_of(n);
            float* cf = cst[n & 1];
            // the gate scans of this chunk, stored with its gates (lane = token)
            const float (*Sc)[C] = sst[n & 1];
            if constexpr (w == 0) {
                const float a = G[0][lane], la = Sc[0][lane], lm = Sc[1][lane], b = Sc[2][lane];
                const float bprev = lane > 0 ? Sc[2][lane - 1] : 0.f;
                cf[MDN_COEF_ABAR * C + lane] = expf(la);
                cf[MDN_COEF_ABP * C + lane] = a * bprev;
                cf[MDN_COEF_B * C + lane] = b;
                cf[MDN_COEF_LA * C + lane] = la;
                cf[MDN_COEF_LM * C + lane] = lm;
                cf[MDN_COEF_LOGC * C + lane] = logf(b) - la;
            }
            // K K^T, column block w: tiles (a, w), a = w .. NCT-1, rows and
            // columns in natural order (issued first: the matrix cores work
            // while the Gamma recurrence below runs on the vector units)
            floatx4 acc[NCT];
            {
                frag bk[KSD];
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) bk[ks] = LdsA<Tr, L::PK>::load(Kl, 16 * w + nn, ks, g);
#pragma unroll
                for (int a2 = w; a2 < NCT; ++a2) {
                    acc[a2] = zero4();
                    frag ak[KSD];
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks)
                        ak[ks] = a2 == w ? bk[ks] : LdsA<Tr, L::PK>::load(Kl, 16 * a2 + nn, ks, g);
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks) acc[a2] = Tr::mma(ak[ks], bk[ks], acc[a2]);
                }
            }
            // Gamma, column block w: lane (j, rb) runs column i = 16 w + j over
            // rows 16 rb .. 16 rb + 15, then adds the carry of the earlier row
            // blocks scaled by the running product of alpha:
            //   gamma_{r,i} = alpha_r gamma_{r-1,i} + beta_r mubar_r / mubar_i
            // The 16 rows run as two independent halves of 8 from zero, the
            // second then taking the first's end value scaled the same way.
            const int j = nn, rb = g, i = 16 * w + j;
            const float lmi = Sc[1][i], ei = G[3][i], lmC = Sc[1][C - 1];
            const float lms0 = Sc[1][16 * rb > 0 ? 16 * rb - 1 : 0], lms1 = Sc[1][16 * rb + 7];
            // alpha, beta, mu of row 16 rb + t sit in lane t of this lane's
            // 16-lane row: every row of lanes gets them by row broadcast
            float ga[16], gb[16], gmu[16];
            {
                const float xa = G[0][lane], xm = G[1][lane], xb = G[2][lane];
                row_bcast_all(xa, ga, std::make_integer_sequence<int, 16>{});
                row_bcast_all(xm, gmu, std::make_integer_sequence<int, 16>{});
                row_bcast_all(xb, gb, std::make_integer_sequence<int, 16>{});
            }
            float wv0 = 16 * rb > i ? expf(lms0 - lmi) : 0.f;
            float wv1 = 16 * rb + 8 > i ? expf(lms1 - lmi) : 0.f;
            float loc0 = 0.f, d0 = 1.f, loc1 = 0.f, d1 = 1.f;
            float lv[16], dv[16];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int t1 = t + 8;
                const float ar0 = ga[t], br0 = gb[t], mr0 = gmu[t];
                const float ar1 = ga[t1], br1 = gb[t1], mr1 = gmu[t1];
                wv0 = (16 * rb + t == i) ? 1.f : wv0 * mr0;
                wv1 = (16 * rb + t1 == i) ? 1.f : wv1 * mr1;
                loc0 = fmaf(ar0, loc0, br0 * wv0);
                loc1 = fmaf(ar1, loc1, br1 * wv1);
                d0 *= ar0;
                d1 *= ar1;
                lv[t] = loc0;
                dv[t] = d0;
                lv[t1] = loc1;
                dv[t1] = d1;
            }
#pragma unroll
            for (int t = 8; t < 16; ++t) {
                lv[t] = fmaf(dv[t], lv[7], lv[t]);
                dv[t] *= dv[7];
            }
            const float loc = lv[15], d = dv[15];
            float G0 = 0.f;
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) {
                const float xe = __shfl(loc, j + 16 * bb, 64), xd = __shfl(d, j + 16 * bb, 64);
                if (bb < rb) G0 = fmaf(xd, G0, xe);
            }
            // the output waves read chunk n-1's Gamma at the start of this
            // step; wait until both have before overwriting it
            wait_count(&gfree, 2u * (unsigned)n);
            {
                float* gcol = gam + i * C + 16 * rb;
#pragma unroll
                for (int t = 0; t < 16; t += 4) {
                    floatx4 o;
#pragma unroll
                    for (int u = 0; u < 4; ++u) o[u] = ei * fmaf(dv[t + u], G0, lv[t + u]);
                    *reinterpret_cast<floatx4*>(gcol + t) = o;
                }
                if (rb == NCT - 1) {
                    cf[MDN_COEF_GS * C + i] = ei * fmaf(dv[15], G0, lv[15]);
                    cf[MDN_COEF_GM * C + i] = ei * expf(lmC - lmi);
                }
            }
            wave_lds_sync();                           // this wave's Gamma columns are written
            // A_{r,i} = alpha_r (k_r . k_i) Gamma_{r-1,i}: zero on and above the
            // diagonal (Gamma_{r-1,i} = 0 for i >= r) and on rows past the end.
#pragma unroll
            for (int a2 = w; a2 < NCT; ++a2) {
                const int RK = 16 * a2 + 4 * g;
                const float* gc = gam + i * C;
                const floatx4 g4 = *reinterpret_cast<const floatx4*>(gc + RK);
                const float gp = RK > 0 ? gc[RK - 1] : 0.f;
                const floatx4 gm = floatx4{gp, g4[0], g4[1], g4[2]};
                const floatx4 al = *reinterpret_cast<const floatx4*>(&G[0][RK]);
                floatx4 av;
#pragma unroll
                for (int e = 0; e < 4; ++e) av[e] = RK + e < vl ? al[e] * acc[a2][e] * gm[e] : 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) amat[a_idx<C>(RK + e, i)] = av[e];
            }
            wave_lds_sync();
            // T_ww = (I + A_ww)^{-1} by forward substitution in registers: lane
            // (r, g) holds row r of T_ww at columns 4g .. 4g+3 and row r of A_ww
            floatx4 Tc[NCT];
            {
                const int r = nn;
                floatx4 lrow[4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    lrow[q4] = *reinterpret_cast<const floatx4*>(amat + a_idx<C>(16 * w + r, 16 * w + 4 * q4));
                float t[4];
                unit_lower_inv16(t, lrow, lane);
                wave_lds_sync();                       // every lane has read A_ww
                *reinterpret_cast<floatx4*>(amat + a_idx<C>(16 * w + r, 16 * w + 4 * g)) = floatx4{t[0], t[1], t[2], t[3]};
                char* Tl = tst + (n & 1) * L::TB;
                bf16x4 tb;
#pragma unroll
                for (int c = 0; c < 4; ++c) tb[c] = Tr::from_f(t[c]);
                *reinterpret_cast<bf16x4*>(Tl + swz<L::PT>(16 * w + r, 2 * (16 * w + 4 * g))) = tb;
                wave_lds_sync();
                // T_ww in the accumulator layout (rows 4g + e, column nn), the B
                // operand of the products below
#pragma unroll
                for (int e = 0; e < 4; ++e) Tc[w][e] = amat[a_idx<C>(16 * w + 4 * g + e, 16 * w + nn)];
            }
            lsync();                                   // A below the diagonal and every T_aa visible
            // column block w of T below the diagonal:
            //   T_aw = -T_aa X_aw,  X_aw = sum_{c=w}^{a-1} A_ac T_cw,
            // on the bf16 matrix cores with fp32 accumulation (the bf16 path's
            // operand precision; T_ww above is exact fp32).  One K = 32 step
            // takes the c blocks in pairs: slots 0-3 of lane group g are rows
            // 4g .. 4g+3 of block c, slots 4-7 the same rows of block c+1, and
            // the A operand reads the same columns of A_ac and A_a(c+1).  A
            // lone block, and T_aa X, leave slots 4-7 zero.
            {
                char* Tl = tst + (n & 1) * L::TB;
                auto pack = [](const floatx4& lo, const floatx4& hi) __attribute__((always_inline)) {
                    bf16x8 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        r[e] = (__bf16)lo[e];
                        r[4 + e] = (__bf16)hi[e];
                    }
                    return r;
                };
                // every A_ac and T_aa this column block needs, read at once
                floatx4 Ao[NCT][NCT], To[NCT];
#pragma unroll
                for (int a2 = w + 1; a2 < NCT; ++a2) {
#pragma unroll
                    for (int c = w; c < a2; ++c)
                        Ao[a2][c] = *reinterpret_cast<const floatx4*>(amat + a_idx<C>(16 * a2 + nn, 16 * c + 4 * g));
                    To[a2] = *reinterpret_cast<const floatx4*>(amat + a_idx<C>(16 * a2 + nn, 16 * a2 + 4 * g));
                }
#pragma unroll
                for (int a2 = w + 1; a2 < NCT; ++a2) {
                    floatx4 X = zero4();
#pragma unroll
                    for (int c = w; c < a2; c += 2) {
                        const bool two = c + 1 < a2;
                        X = Tr::mma(pack(Ao[a2][c], two ? Ao[a2][c + 1] : zero4()),
                                    pack(Tc[c], two ? Tc[c + 1] : zero4()), X);
                    }
                    const floatx4 Y = Tr::mma(pack(To[a2], zero4()), pack(X, zero4()), zero4());
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        Tc[a2][e] = -Y[e];
                        *reinterpret_cast<E*>(Tl + swz<L::PT>(16 * a2 + 4 * g + e, 2 * (16 * w + nn))) =
                            Tr::from_f(-Y[e]);
                    }
                }
            }
        };


        // -- prologue: T buffers zeroed (their upper blocks are never written
        // again), then the intra step of chunk 0 --
        {
            constexpr int NZ = 2 * L::TB / 16;
            for (int p = w * 64 + lane; p < NZ; p += NLD * 64)
                reinterpret_cast<uint4*>(tst)[p] = uint4{0u, 0u, 0u, 0u};
        }
        lds_barrier();                                 // B_pro: chunk 0's K rows and gates staged
        if (NTu > 0) {
            lsync();                                   // every T buffer zeroed
            intra(0);
        }
        for (int64_t m = 0; m < NTu; ++m) {
            lds_barrier();                             // B0(m)
            if (m + 1 < NTu) intra(m + 1);
        }
        lds_barrier();                                 // E1
        };
        switch (r2) {
        case 2: intra_wave(std::integral_constant<int, 0>{}); break;
        case 3: intra_wave(std::integral_constant<int, 1>{}); break;
        case 4: intra_wave(std::integral_constant<int, 2>{}); break;
        default: intra_wave(std::integral_constant<int, 3>{}); break;
        }
        return;
    }

    // ============================ chain waves ============================
    const int cw = role;
    const int ct = cw / RS;                           // column tile
    constexpr int h = 0;                              // row part (no row split)
    const int col = col0 + 16 * ct + nn;
    const int td0 = h * NDH, ks0 = h * KSH;

    const size_t sbase = (size_t)bh * D * D;
    floatx4 XS[NDH], XM[NDH];
#pragma unroll
    for (int t = 0; t < NDH; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t off = sbase + (size_t)SL::perm(16 * (td0 + t) + 4 * g + e) * D + col;
            XS[t][e] = S0 ? S0[off] : 0.f;
            XM[t][e] = M0 ? M0[off] : 0.f;
        }
    const int smo = ((ct * RS + h) * 2) * KSH * 64 + lane;
    frag Sb[KSH], Mb[KSH];
    // chunk-start state operands of chunk n, for P and for the output waves
    auto state_operands = [&](int par) __attribute__((always_inline)) {
        frag* const smS = sm[par] + smo;
        frag* const smM = smS + KSH * 64;
#pragma unroll
        for (int ks = 0; ks < KSH; ++ks) {
            Sb[ks] = SL::from_acc(XS, ks);
            Mb[ks] = SL::from_acc(XM, ks);
            smS[ks * 64] = Sb[ks];
            smM[ks * 64] = Mb[ks];
        }
    };
    state_operands(0);
    lds_barrier();                                    // B_pro

    auto chunk = [&](auto mod6) __attribute__((always_inline)) {
        constexpr int P = decltype(mod6)::value & 1;    // m & 1
        constexpr int KBI = decltype(mod6)::value % 3;  // m % 3
        lds_barrier();                                  // B0(m)
        const char* Kl = kst + KBI * L::KB;
        const char* Tl = tst + P * L::TB;
        const char* Vl = vst + P * L::VB;
        const float* cf = cst[P];

        // -- phase 1 --
        frag tA[KSC][NCT];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) tA[ks][tc] = LdsA<Tr, L::PT>::load(Tl, SL::perm(16 * tc + nn), ks, g);
        floatx4 Vx[NCT];
#pragma unroll
        for (int tc = 0; tc < NCT; ++tc) Vx[tc] = zero4();
        floatx4 Pm[NCT];
        {
            floatx4 KSa[NCT], KMa[NCT];
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) { KSa[tc] = zero4(); KMa[tc] = zero4(); }
#pragma unroll
            for (int ks = 0; ks < KSH; ++ks) {
                frag a[NCT];
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) a[tc] = LdsA<Tr, L::PK>::load(Kl, SL::perm(16 * tc + nn), ks0 + ks, g);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) {
                    KSa[tc] = Tr::mma(a[tc], Sb[ks], KSa[tc]);
                    KMa[tc] = Tr::mma(a[tc], Mb[ks], KMa[tc]);
                }
                if constexpr (KSH > 2) {
                    if (ks % 2 == 1) __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                const frag vB = VOperand<Tr, OW>::load(Vl, ct, ks, lane);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) Vx[tc] = Tr::mma(tA[ks][tc], vB, Vx[tc]);
            }
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
                for (int e = 0; e < 4; ++e) Pm[tc][e] = cp[e] * KMa[tc][e] - ca[e] * KSa[tc][e];
            }
        }
        // -- phase 2 --
        {
            frag Wb[KSC];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) Wb[ks] = SL::from_acc(Pm, ks);
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) Vx[tc] = Tr::mma(tA[ks][tc], Wb[ks], Vx[tc]);
        }
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            float gs[8], gm[8];
            SL::load_row(cf + MDN_COEF_GS * C, ks, g, gs);
            SL::load_row(cf + MDN_COEF_GM * C, ks, g, gm);
            frag kT[NDH];
#pragma unroll
            for (int t = 0; t < NDH; ++t) kT[t] = KtOperand<Tr, L::PK>::load(Kl, td0 + t, ks, lane);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) gm[jj] = -gm[jj];
            const frag VS = SL::from_acc_scaled(Vx, ks, gs);
            const frag VM = SL::from_acc_scaled(Vx, ks, gm);
#pragma unroll
            for (int t = 0; t < NDH; ++t) {
                XS[t] = Tr::mma(kT[t], VS, XS[t]);
                XM[t] = Tr::mma(kT[t], VM, XM[t]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) vb[P][(ct * KSC + ks) * 64 + lane] = SL::from_acc(Vx, ks);
        state_operands(P ^ 1);                          // of chunk m + 1
    };
    // six chunks per iteration, so that every buffer of a chunk (K by m % 3,
    // the others by m % 2) sits at a compile-time LDS offset
    for (int64_t m = 0; m < NTu; m += 6) {
        chunk(std::integral_constant<int, 0>{});
        if (m + 1 >= NTu) break;
        chunk(std::integral_constant<int, 1>{});
        if (m + 2 >= NTu) break;
        chunk(std::integral_constant<int, 2>{});
        if (m + 3 >= NTu) break;
        chunk(std::integral_constant<int, 3>{});
        if (m + 4 >= NTu) break;
        chunk(std::integral_constant<int, 4>{});
        if (m + 5 >= NTu) break;
        chunk(std::integral_constant<int, 5>{});
    }
    lds_barrier();                                      // E1

#pragma unroll
    for (int t = 0; t < NDH; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t off = sbase + (size_t)SL::perm(16 * (td0 + t) + 4 * g + e) * D + col;
            ST[off] = XS[t][e];
            MT[off] = XM[t][e];
        }
}

template <int D, int C, int NCOL>
static hipError_t launch_fwd_cols(const ChunkArgs& a)
{
    constexpr int RS = 1;
    const int64_t grid = a.BH * (D / (16 * NCOL));
    hipLaunchKernelGGL((mdn_fwd_kernel<D, C, NCOL, RS>), dim3((unsigned)grid), dim3(64 * (NCOL * RS + 6)), 0,
                       (hipStream_t)a.stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                       a.alpha, a.mu, a.beta, a.eta, a.S0, a.M0, (__bf16*)a.O, a.ST, a.MT, (__bf16*)a.Vt, a.T,
                       (int)a.BH);
    return hipGetLastError();
}

bool fwd_fused_supported(const ChunkArgs& a)
{
    return a.dtype == MDN_BF16 && !a.cu && a.C == 64 && a.dk == a.dv && (a.dk == 64 || a.dk == 128);
}

hipError_t launch_chunk_fwd_fused(const ChunkArgs& a)
{
    if (a.BH == 0) return hipSuccess;
    switch (a.dk) {
    case 64: return launch_fwd_cols<64, 64, 2>(a);
    case 128: return launch_fwd_cols<128, 64, 2>(a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mdn
