// mdn_intra.hip -- coefficient and intra-chunk stage of the chunkwise
// Momentum DeltaNet forward (gfx950).
//
// For every chunk tile (head, chunk n), independently of all others (MDN
// summary at paper.rainbus.top, method walk-through steps 3-5):
//   coefficient rows   LA, LM (cumulative log gates), log c (log-domain
//                      cumulative sum), abar = exp(LA), b = exp(LA + log c),
//                      alpha_r b_{r-1}, gS_i = Gamma_{C-1,i},
//                      gM_i = eta_i exp(LM_{C-1} - LM_i)
//   Gamma_{r,i}        = eta_i gamma_{r,i},
//                      gamma_{r,i} = alpha_r gamma_{r-1,i} + beta_r exp(LM_r - LM_i)  (r >= i)
//   A                  = (Diag(alpha) K K^T) o Gamma^-   (Gamma^-_{r,i} = Gamma_{r-1,i}, i < r)
//   T                  = (I + A)^{-1}
//   Aqk                = (Q K^T) o Gamma                 (i <= r)
// and writes T, Aqk (element type) and the coefficient rows to the workspace.
//
// One workgroup of four waves per tile:
//   1. waves 1-3 copy the K and Q rows of the chunk into LDS (direct
//      global->LDS loads, swizzled) while wave 0 loads the gates and runs the
//      three 64-lane scans;
//   2. Gamma by a two-level scan over rows: each thread runs the recurrence
//      over one block of rows for one column from zero, and the block carries
//      are combined afterwards (every term is non-negative, every exponent
//      <= 0, so nothing overflows or cancels);
//   3. K K^T and Q K^T on the matrix cores: a wave keeps the A operands of
//      one 16-row block of K and Q in registers and sweeps the column blocks
//      of the (block-)lower triangle, so each K row block is read once per
//      wave and serves both products;
//   4. T = (I + A)^{-1} blockwise in fp32: the 16 x 16 diagonal blocks by
//      forward substitution (one wave each), then column block b of T by
//      block forward substitution, T_ab = -T_aa sum_{c=b..a-1} A_ac T_cb, on
//      the fp32 matrix cores, one wave per column block;
//   5. T and Aqk leave through LDS tiles as full 16-byte stores (or, for the
//      backward, T^T and Aqk^T), without the all-zero quadrant that no
//      product reads (quad_unread).
#include "mdn_device.h"
#include "mdn_internal.h"
#include "mdn_lds.h"
#include "../../include/mdn.h"

namespace mdn {

// A operand read straight from a global row, in the contraction order of
// LdsA (bf16: lane group g of step ks holds columns 32ks + 8g .. +7; fp32:
// column 16(ks/4) + 4g + ks%4).
template <typename Tr, int KSD> struct RowA;
template <int KSD> struct RowA<TraitsBf16, KSD> {
    static __device__ __forceinline__ void load(bf16x8 (&a)[KSD], const __bf16* row, int g) {
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            union { uint4 u; bf16x8 v; } f;
            f.u = *reinterpret_cast<const uint4*>(row + 32 * ks + 8 * g);
            a[ks] = f.v;
        }
    }
    static __device__ __forceinline__ void zero(bf16x8 (&a)[KSD]) {
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) a[ks] = Slots<TraitsBf16>::zero();
    }
};
template <int KSD> struct RowA<TraitsF32, KSD> {
    static __device__ __forceinline__ void load(float (&a)[KSD], const float* row, int g) {
#pragma unroll
        for (int m = 0; m < KSD / 4; ++m) {
            const floatx4 v = *reinterpret_cast<const floatx4*>(row + 16 * m + 4 * g);
#pragma unroll
            for (int u = 0; u < 4; ++u) a[4 * m + u] = v[u];
        }
    }
    static __device__ __forceinline__ void zero(float (&a)[KSD]) {
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) a[ks] = 0.f;
    }
};

template <typename Tr, int DK, int C>
struct IntraLayout {
    using E = typename Tr::elem;
    static constexpr int ES = sizeof(E);
    static constexpr int NCT = C / 16;               // 16-row blocks
    static constexpr int PK = DK * ES / 16;          // 16-byte pieces per K/Q row
    static constexpr int KT = C * PK * 16;           // one K or Q tile (bytes)
    static constexpr int AS = C + 4;                 // row stride of A (floats)
    static constexpr int ABYTES = C * AS * 4;
    static constexpr int OUT = C * C * ES;           // one out tile (T or Aqk)
    // Gamma, column-major: column i at floats [i*GS, (i+1)*GS), 4 zeros then
    // rows 0..C-1, so that rows r-4..r-1 (the shifted Gamma^-) sit just
    // before rows r..r+3 and both are aligned 16-byte reads
    static constexpr int GS = C + 4;
    static constexpr int GBYTES = C * GS * 4;
    // region X: the K tile; then the T out tile and the Aqk out tile
    static constexpr int OT = 0, OQ = OUT;
    static constexpr int RX = KT > 2 * OUT ? KT : 2 * OUT;
    // region Y: Gamma; then A (fp32), whose diagonal blocks are replaced by
    // the inverses T_aa once those are known
    static constexpr int RY = GBYTES > ABYTES ? GBYTES : ABYTES;
    // Gamma scan: NB row blocks of RB rows, one thread per (block, column)
    static constexpr int NB = 256 / C;
    static constexpr int RB = C / NB;
    static constexpr int KSD = DK / Tr::KW;
    static_assert(NB * C == 256 && RB * NB == C, "256 threads cover the C x C Gamma scan");
};

// One wave's share of K K^T and Q K^T: row block TRK of K K^T (if DOK) and
// row block TRQ of Q K^T (if DOQ), over the column blocks of the lower
// triangle, then the decay weights
//   A_{r,i}   = alpha_r (K K^T)_{r,i} Gamma_{r-1,i}   (i < r)
//   Aqk_{r,i} = (Q K^T)_{r,i} Gamma_{r,i}             (i <= r).
// Accumulator row x of block t stands for chunk row perm(16t + x) (bf16
// slot map; identity for fp32), so the 16 rows of an operand read get
// distinct swizzle keys.  The B operands (K rows of column block tc) are
// read once and serve both products.  Gamma is column-major (see
// IntraLayout), so the four rows of a lane are one 16-byte read.
template <typename Tr, typename L>
struct IntraProducts {
    using frag = typename Tr::frag;
    using SL = Slots<Tr>;
    static constexpr int NCT = L::NCT, KSD = L::KSD;
    static constexpr bool lower(int rb, int cb) {
        return std::is_same<Tr, TraitsBf16>::value ? ((cb >> 1) <= (rb >> 1)) : (cb <= rb);
    }
    template <int TRK, int TRQ, bool DOK, bool DOQ>
    static __device__ __forceinline__ void run(const char* Kl, const frag (&aQ)[KSD], const float* Gt,
                                               const float* sal, int g, int nn,
                                               floatx4 (&accK)[NCT], floatx4 (&accQ)[NCT]) {
        frag aK[KSD];
        if constexpr (DOK) {
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) aK[ks] = LdsA<Tr, L::PK>::load(Kl, SL::perm(16 * TRK + nn), ks, g);
        }
#pragma unroll
        for (int tc = 0; tc < NCT; ++tc) {
            const bool uk = DOK && lower(TRK, tc), uq = DOQ && lower(TRQ, tc);
            if (uk || uq) {
                frag bk[KSD];
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) bk[ks] = LdsA<Tr, L::PK>::load(Kl, SL::perm(16 * tc + nn), ks, g);
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    if (uk) accK[tc] = Tr::mma(aK[ks], bk[ks], accK[tc]);
                    if (uq) accQ[tc] = Tr::mma(aQ[ks], bk[ks], accQ[tc]);
                }
            }
        }
        constexpr int GS = L::GS;
        const int RK = SL::perm(16 * TRK + 4 * g), RQ = SL::perm(16 * TRQ + 4 * g);
        const floatx4 al = *reinterpret_cast<const floatx4*>(sal + RK);
#pragma unroll
        for (int tc = 0; tc < NCT; ++tc) {
            const int i = SL::perm(16 * tc + nn);
            const float* gc = Gt + i * GS + 4;
            if (DOK && lower(TRK, tc)) {
                const floatx4 g4 = *reinterpret_cast<const floatx4*>(gc + RK);
                const floatx4 gp = *reinterpret_cast<const floatx4*>(gc + RK - 4);
                const floatx4 gm = floatx4{gp[3], g4[0], g4[1], g4[2]};
#pragma unroll
                for (int e = 0; e < 4; ++e) accK[tc][e] = (i < RK + e) ? al[e] * accK[tc][e] * gm[e] : 0.f;
            }
            if (DOQ && lower(TRQ, tc)) {
                const floatx4 g4 = *reinterpret_cast<const floatx4*>(gc + RQ);
#pragma unroll
                for (int e = 0; e < 4; ++e) accQ[tc][e] = (i <= RQ + e) ? accQ[tc][e] * g4[e] : 0.f;
            }
        }
    }
};

template <typename Tr, int DK, int C, bool COEF_ONLY, bool TRANS = false>
__global__ __launch_bounds__(256)
void mdn_intra_kernel(const typename Tr::elem* __restrict__ q,
                      const typename Tr::elem* __restrict__ k,
                      const float* __restrict__ alpha, const float* __restrict__ mu,
                      const float* __restrict__ beta, const float* __restrict__ eta,
                      int64_t T, int64_t NT, const int2* __restrict__ tab,
                      typename Tr::elem* __restrict__ Tout,
                      typename Tr::elem* __restrict__ Aqk,
                      float* __restrict__ coef,
                      float* __restrict__ gamma)
{
    using E = typename Tr::elem;
    using SL = Slots<Tr>;
    using L = IntraLayout<Tr, DK, C>;
    using frag = typename Tr::frag;
    constexpr int NCT = L::NCT, KSD = DK / Tr::KW, NB = L::NB, RB = L::RB, GS = L::GS;

    __shared__ __attribute__((aligned(16))) char rx[COEF_ONLY ? 16 : L::RX];
    __shared__ __attribute__((aligned(16))) char ry[L::RY];
    __shared__ __attribute__((aligned(16))) floatx4 sg[C];     // (alpha, beta, mu, eta) per row
    __shared__ __attribute__((aligned(16))) float sal[C];      // alpha per row
    __shared__ float slm[C];                                   // LM (cumulative log mu)
    __shared__ float xe[NB][C];                                // Gamma scan: block ends
    __shared__ float xd[NB];                                   // Gamma scan: alpha product per block

    const int64_t tile = blockIdx.x;
    const int64_t bh = tile / NT, n = tile % NT;
    size_t rowbase;
    int valid;
    if (tab) {
        // packed batch: slot n of head bh covers rows [first, first + rows)
        // of the head's packed sequence; empty slots have no work.  Clamped,
        // so that a malformed table can only give wrong values, never an
        // access outside the head's rows.
        const int2 e = tab[n];
        const int64_t vmax = T < C ? T : C;
        valid = (int)(e.y < 0 ? 0 : (e.y > vmax ? vmax : e.y));
        if (valid == 0) return;
        const int64_t f = e.x < 0 ? 0 : (e.x > T - valid ? T - valid : e.x);
        rowbase = (size_t)(bh * T + f);
    } else {
        rowbase = (size_t)(bh * T + n * C);
        valid = (int)((T - n * C) < C ? (T - n * C) : C);
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, nn = lane & 15;
    float* cf = coef + tile * MDN_COEF_ROWS * C;

    // Product roles.  Accumulator row x of block t stands for chunk row
    // perm(16t + x) (bf16 slot map; identity for fp32), so the 16 rows of an
    // operand read get distinct swizzle keys.  With four row blocks wave w
    // owns row block w of K K^T and row block 3-w of Q K^T (equal numbers of
    // lower tiles); otherwise wave w owns row block w % NCT of product w / NCT.
    constexpr bool BOTH = NCT >= 4;
    const int trK = BOTH ? wave : wave % NCT;
    const int trQ = BOTH ? NCT - 1 - wave : wave % NCT;
    const int mat = BOTH ? 0 : wave / NCT;
    const bool doK = BOTH || mat == 0, doQ = BOTH || mat == 1;
    // The Q rows of a wave's block are used by that wave alone: they go
    // straight from global memory into A-operand registers (zero past the end).
    frag aQ[KSD];
    auto load_q = [&]() __attribute__((always_inline)) {
        const int row = SL::perm(16 * trQ + nn);
        if (row < valid) RowA<Tr, KSD>::load(aQ, q + (rowbase + row) * DK, g);
        else RowA<Tr, KSD>::zero(aQ);
    };

    // ---- 1. K -> LDS (waves 1-3), Q -> registers; gates and scans (wave 0) ---
    if constexpr (!COEF_ONLY) {
        if (wave > 0) {
            // NCT blocks of 16 K rows, dealt to waves 1-3; rows past `valid`
            // repeat the last valid row (zeroed below)
            const unsigned vlast = (unsigned)valid - 1;
            auto seq_row = [&](unsigned r) { return (r < vlast ? r : vlast) * (unsigned)(DK * L::ES); };
            const uint32_t base = lds_addr(rx);
#pragma unroll
            for (int j = 0; j < NCT; ++j)
                if (j % 3 == wave - 1)
                    dma_tile<16, L::PK>(base, reinterpret_cast<const char*>(k + rowbase * DK), seq_row, lane, 16 * j);
            if (doQ) load_q();
        }
    }
    if (wave == 0) {
        float a = 1.f, m = 1.f, bt = 0.f, e = 0.f;   // neutral padding past the end
        if (lane < valid) {
            const size_t gi = rowbase + lane;
            a = alpha[gi]; m = mu[gi]; bt = beta[gi]; e = eta[gi];
        }
        if constexpr (!COEF_ONLY)
            if (doQ) load_q();                       // after the gate loads
        const float la = wave_scan_add(logf(a));
        const float lm = wave_scan_add(logf(m));
        // b_r = alpha_r b_{r-1} + beta_r mubar_r (b_{-1} = 0): a scan of the
        // affine maps x -> A x + B, every term non-negative
        float A = a, Bv = bt * expf(lm);
        wave_scan_affine(A, Bv);
        const float b = Bv;
        float bprev = __shfl_up(b, 1, 64);
        if (lane == 0) bprev = 0.f;
        if (lane < C) {
            sg[lane] = floatx4{a, bt, m, e};
            sal[lane] = a;
            slm[lane] = lm;
            cf[MDN_COEF_ABAR * C + lane] = expf(la);
            cf[MDN_COEF_ABP * C + lane] = a * bprev;
            cf[MDN_COEF_B * C + lane] = b;
            cf[MDN_COEF_LA * C + lane] = la;
            cf[MDN_COEF_LM * C + lane] = lm;
            cf[MDN_COEF_LOGC * C + lane] = logf(b) - la;   // log c_r = log(b_r / abar_r)
        }
    }
    lds_barrier();

    // ---- 2. Gamma: column i, rows [r0, r0 + RB) per thread -------------------
    // gamma_{r,i} = alpha_r gamma_{r-1,i} + beta_r w_{r,i},  w_{r,i} = mubar_r / mubar_i
    // (w_{i,i} = 1, w_{r,i} = mu_r w_{r-1,i}).  Each thread runs the recurrence
    // from zero over its block; the carry gamma_{r0-1,i} from the earlier
    // blocks enters scaled by the running product of alpha.
    float* Gt = reinterpret_cast<float*>(ry);
    {
        const int i = tid % C, bk = tid / C, r0 = bk * RB;
        const float lmi = slm[i], ei = sg[i][3];
        float w = (r0 > i) ? expf(slm[r0 > 0 ? r0 - 1 : 0] - lmi) : 0.f;
        float loc = 0.f, d = 1.f;
        float lv[RB], dv[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const floatx4 gr = sg[r0 + j];
            w = (r0 + j == i) ? 1.f : w * gr[2];
            loc = fmaf(gr[0], loc, gr[1] * w);
            d *= gr[0];
            lv[j] = loc;
            dv[j] = d;
        }
        xe[bk][i] = loc;
        if (i == 0) xd[bk] = d;
        lds_barrier();
        float G = 0.f;
#pragma unroll
        for (int bb = 0; bb < NB - 1; ++bb)
            if (bb < bk) G = fmaf(xd[bb], G, xe[bb][i]);
        float* col = Gt + i * GS + 4 + r0;
        if (bk == 0) *reinterpret_cast<floatx4*>(Gt + i * GS) = zero4();   // Gamma^- of row 0
        if constexpr (RB % 4 == 0) {
#pragma unroll
            for (int j = 0; j < RB; j += 4) {
                floatx4 o;
#pragma unroll
                for (int u = 0; u < 4; ++u) o[u] = ei * fmaf(dv[j + u], G, lv[j + u]);
                *reinterpret_cast<floatx4*>(col + j) = o;
            }
        } else {
#pragma unroll
            for (int j = 0; j < RB; ++j) col[j] = ei * fmaf(dv[j], G, lv[j]);
        }
        if (bk == NB - 1) {                          // this thread holds row C-1
            cf[MDN_COEF_GS * C + i] = ei * fmaf(dv[RB - 1], G, lv[RB - 1]);
            cf[MDN_COEF_GM * C + i] = ei * expf(slm[C - 1] - lmi);
        }
    }
    if constexpr (COEF_ONLY) {
        lds_barrier();
        if (gamma) {
            float* gp = gamma + tile * C * C;
            for (int idx = tid; idx < C * C; idx += 256) gp[idx] = Gt[(idx % C) * GS + 4 + idx / C];
        }
        return;
    }

    __builtin_amdgcn_s_waitcnt(0);                   // this wave's K/Q copies have landed
    lds_barrier();                                   // Gamma and the K/Q tiles visible
    const char* Kl = rx;
    if (valid < C) {                                 // ragged last chunk: zero K rows past the end
        constexpr int W = L::PK;                     // 16-byte words per row
        for (int w = valid * W + tid; w < C * W; w += 256)
            reinterpret_cast<uint4*>(rx)[w] = uint4{0u, 0u, 0u, 0u};
        lds_barrier();
    }

    // ---- 3. K K^T and Q K^T on the matrix cores --------------------------------
    // The role of each wave is a template argument, so that the product code
    // is straight-line (no uniform branches between the matrix-core ops).
    floatx4 accK[NCT], accQ[NCT];
#pragma unroll
    for (int tc = 0; tc < NCT; ++tc) { accK[tc] = zero4(); accQ[tc] = zero4(); }
    const int RK = SL::perm(16 * trK + 4 * g), RQ = SL::perm(16 * trQ + 4 * g);   // first of 4 rows
    {
        using P = IntraProducts<Tr, L>;
        if constexpr (NCT >= 4) {
            switch (wave) {
            case 0: P::template run<0, 3, true, true>(Kl, aQ, Gt, sal, g, nn, accK, accQ); break;
            case 1: P::template run<1, 2, true, true>(Kl, aQ, Gt, sal, g, nn, accK, accQ); break;
            case 2: P::template run<2, 1, true, true>(Kl, aQ, Gt, sal, g, nn, accK, accQ); break;
            default: P::template run<3, 0, true, true>(Kl, aQ, Gt, sal, g, nn, accK, accQ); break;
            }
        } else if constexpr (NCT == 2) {
            switch (wave) {
            case 0: P::template run<0, 0, true, false>(Kl, aQ, Gt, sal, g, nn, accK, accQ); break;
            case 1: P::template run<1, 1, true, false>(Kl, aQ, Gt, sal, g, nn, accK, accQ); break;
            case 2: P::template run<0, 0, false, true>(Kl, aQ, Gt, sal, g, nn, accK, accQ); break;
            default: P::template run<1, 1, false, true>(Kl, aQ, Gt, sal, g, nn, accK, accQ); break;
            }
        } else {
            if (wave == 0) P::template run<0, 0, true, false>(Kl, aQ, Gt, sal, g, nn, accK, accQ);
            else if (wave == 1) P::template run<0, 0, false, true>(Kl, aQ, Gt, sal, g, nn, accK, accQ);
        }
    }
    lds_barrier();                                   // K and Gamma reads done

    float* sA = reinterpret_cast<float*>(ry);        // A, fp32, row stride AS (then T_aa on the diagonal)
    E* oT = reinterpret_cast<E*>(rx + L::OT);        // T out tile, row-major C x C
    E* oAq = reinterpret_cast<E*>(rx + L::OQ);       // Aqk out tile, row-major C x C
    if (doK || doQ) {
#pragma unroll
        for (int tc = 0; tc < NCT; ++tc) {
            const int i = SL::perm(16 * tc + nn);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (doK) sA[(RK + e) * L::AS + i] = accK[tc][e];
                if (doQ) oAq[(RQ + e) * C + i] = Tr::from_f(accQ[tc][e]);
            }
        }
    }
    lds_barrier();

    // ---- 4a. diagonal blocks of T: wave a inverts block a -------------------
    // T_aa = (I + A_aa)^{-1} by forward substitution in registers (lane (r, g)
    // holds row r of A_aa and returns row r of T_aa at columns 4g .. 4g+3),
    // written over A's diagonal block and to the T out tile
    if (wave < NCT) {
        const int a = wave, r = nn;
        floatx4 arow[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            arow[q4] = *reinterpret_cast<const floatx4*>(sA + (16 * a + r) * L::AS + 16 * a + 4 * q4);
        float t[4];
        unit_lower_inv16(t, arow, lane);
        // the wave's reads of A_aa have returned (t depends on them)
        *reinterpret_cast<floatx4*>(sA + (16 * a + r) * L::AS + 16 * a + 4 * g) = floatx4{t[0], t[1], t[2], t[3]};
#pragma unroll
        for (int c = 0; c < 4; ++c) oT[(16 * a + r) * C + 16 * a + 4 * g + c] = Tr::from_f(t[c]);
    }
    {
        // strictly upper blocks (a < b) of T are zero: 16-byte stores
        constexpr int PB = 16 * L::ES / 16;          // 16-byte pieces per block row
        constexpr int NU = NCT * (NCT - 1) / 2;
        for (int idx = tid; idx < NU * 16 * PB; idx += 256) {
            int blk = idx / (16 * PB), a = 0;
            while (blk >= NCT - 1 - a) { blk -= NCT - 1 - a; ++a; }
            const int b = a + 1 + blk, rem = idx % (16 * PB);
            const int row = 16 * a + rem / PB;
            *reinterpret_cast<uint4*>(reinterpret_cast<char*>(oT) + (row * C + 16 * b) * L::ES + (rem % PB) * 16) =
                uint4{0u, 0u, 0u, 0u};
        }
    }
    lds_barrier();

    // ---- 4b. column block b of T below the diagonal (fp32 matrix cores) -------
    // Wave w >= 1 owns column block b = NCT-1-w.  Contraction slot map: in
    // step ks, lane group g carries inner index 4g + ks of the 16-block, so
    // an accumulator (rows 4g + e) is the next product's B operand as it stands.
    if (wave >= 1 && wave < NCT) {
        const int b = NCT - 1 - wave;
        floatx4 Tc[NCT];
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
            Tc[c] = zero4();
            if (c == b)
#pragma unroll
                for (int e = 0; e < 4; ++e) Tc[c][e] = sA[(16 * c + 4 * g + e) * L::AS + 16 * c + nn];
        }
#pragma unroll
        for (int a = 1; a < NCT; ++a) {
            if (a > b) {
                floatx4 X = zero4();
#pragma unroll
                for (int c = 0; c < a; ++c) {
                    if (c >= b) {
                        const floatx4 Ao = *reinterpret_cast<const floatx4*>(sA + (16 * a + nn) * L::AS + 16 * c + 4 * g);
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) X = TraitsF32::mma(Ao[ks], Tc[c][ks], X);
                    }
                }
                const floatx4 To = *reinterpret_cast<const floatx4*>(sA + (16 * a + nn) * L::AS + 16 * a + 4 * g);
                floatx4 Y = zero4();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) Y = TraitsF32::mma(To[ks], X[ks], Y);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Tc[a][e] = -Y[e];
                    oT[(16 * a + 4 * g + e) * C + 16 * b + nn] = Tr::from_f(-Y[e]);
                }
            }
        }
    }
    lds_barrier();

    // ---- 5. T and Aqk -> workspace ------------------------------------------
    constexpr int NP = L::OUT / 16;
    constexpr int EPS = 16 / L::ES;                  // elements per 16-byte piece
    constexpr bool QS = quad_unread<Tr, C>();
    uint4* gT = reinterpret_cast<uint4*>(Tout + tile * C * C);
    uint4* gA = reinterpret_cast<uint4*>(Aqk + tile * C * C);
    if constexpr (!TRANS) {
        for (int p = tid; p < NP; p += 256) {
            const int r = p / (C / EPS), c0 = (p % (C / EPS)) * EPS;
            if (QS && r < C / 2 && c0 >= C / 2) continue;   // upper-right quadrant
            gT[p] = reinterpret_cast<const uint4*>(oT)[p];
            gA[p] = reinterpret_cast<const uint4*>(oAq)[p];
        }
    } else {
        // T^T and Aqk^T (the backward's A operands): piece p holds row c of
        // the transpose, columns r0 .. r0 + EPS - 1
        for (int p = tid; p < NP; p += 256) {
            const int c = p / (C / EPS), r0 = (p % (C / EPS)) * EPS;
            if (QS && c >= C / 2 && r0 < C / 2) continue;   // lower-left quadrant of the transpose
            union { uint4 u; E e[EPS]; } t, a;
#pragma unroll
            for (int j = 0; j < EPS; ++j) {
                t.e[j] = oT[(r0 + j) * C + c];
                a.e[j] = oAq[(r0 + j) * C + c];
            }
            gT[p] = t.u;
            gA[p] = a.u;
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename Tr, int DK, int C, bool COEF_ONLY>
static hipError_t launch_intra_t(const ChunkArgs& a)
{
    using E = typename Tr::elem;
    const int64_t tiles = a.BH * a.NT;
    if (!COEF_ONLY && a.trans)
        hipLaunchKernelGGL((mdn_intra_kernel<Tr, DK, C, false, true>), dim3((unsigned)tiles), dim3(256), 0,
                           (hipStream_t)a.stream, (const E*)a.q, (const E*)a.k,
                           a.alpha, a.mu, a.beta, a.eta, a.T, a.NT, reinterpret_cast<const int2*>(a.tab),
                           (E*)a.Tmat, (E*)a.Aqk, a.coef, a.gamma);
    else
        hipLaunchKernelGGL((mdn_intra_kernel<Tr, DK, C, COEF_ONLY>), dim3((unsigned)tiles), dim3(256), 0,
                           (hipStream_t)a.stream, (const E*)a.q, (const E*)a.k,
                           a.alpha, a.mu, a.beta, a.eta, a.T, a.NT, reinterpret_cast<const int2*>(a.tab),
                           (E*)a.Tmat, (E*)a.Aqk, a.coef, a.gamma);
    return hipGetLastError();
}

template <typename Tr>
static hipError_t intra_dispatch(const ChunkArgs& a)
{
    if constexpr (std::is_same<Tr, TraitsBf16>::value) {
        switch (a.dk * 1000 + a.C) {
        case 32032: return launch_intra_t<Tr, 32, 32, false>(a);
        case 32064: return launch_intra_t<Tr, 32, 64, false>(a);
        case 64032: return launch_intra_t<Tr, 64, 32, false>(a);
        case 64064: return launch_intra_t<Tr, 64, 64, false>(a);
        case 128032: return launch_intra_t<Tr, 128, 32, false>(a);
        case 128064: return launch_intra_t<Tr, 128, 64, false>(a);
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (a.dk * 1000 + a.C) {
        case 16016: return launch_intra_t<Tr, 16, 16, false>(a);
        case 16032: return launch_intra_t<Tr, 16, 32, false>(a);
        case 16064: return launch_intra_t<Tr, 16, 64, false>(a);
        case 32016: return launch_intra_t<Tr, 32, 16, false>(a);
        case 32032: return launch_intra_t<Tr, 32, 32, false>(a);
        case 32064: return launch_intra_t<Tr, 32, 64, false>(a);
        case 64016: return launch_intra_t<Tr, 64, 16, false>(a);
        case 64032: return launch_intra_t<Tr, 64, 32, false>(a);
        case 64064: return launch_intra_t<Tr, 64, 64, false>(a);
        case 128016: return launch_intra_t<Tr, 128, 16, false>(a);
        case 128032: return launch_intra_t<Tr, 128, 32, false>(a);
        case 128064: return launch_intra_t<Tr, 128, 64, false>(a);
        default: return hipErrorInvalidValue;
        }
    }
}

hipError_t launch_chunk_intra(const ChunkArgs& a)
{
    if (a.BH * a.NT == 0) return hipSuccess;
    return a.dtype == MDN_BF16 ? intra_dispatch<TraitsBf16>(a) : intra_dispatch<TraitsF32>(a);
}

// Preparation of a packed variable-length batch, one thread per sequence.
//
// Slot table.  Sequence i (tokens [cu[i], cu[i+1]) of every head) owns the
// slots [cu[i] / C + i, cu[i+1] / C + i + 1) of each head's NT = T / C + nseq
// tile slots: its chunks first, then at most one empty slot.  For ordered
// bounds these ranges tile [0, NT) and hold every chunk.  Thread i writes
// sequence i's range, thread 0 also any slots before sequence 0's.  Entries
// are (first row, rows), (0, 0) if empty.
//
// Dispatch order.  perm[r] is the sequence of rank r, lengths descending
// (ties by index): the inter-chunk workgroups of long sequences start first,
// so that the short ones fill in behind them.  Each thread ranks its
// sequence against all others, reading the lengths through LDS in tiles.
//
// Every bound is clamped into [0, T] and ordered first, as the inter kernel
// does, so a malformed cu gives wrong values, never an access out of range.
__device__ __forceinline__ void seq_bounds(const int32_t* __restrict__ cu, int64_t i, int64_t T,
                                           int64_t& c0, int64_t& c1)
{
    c0 = cu[i];
    c1 = cu[i + 1];
    c0 = c0 < 0 ? 0 : (c0 > T ? T : c0);
    c1 = c1 < c0 ? c0 : (c1 > T ? T : c1);
}

__global__ __launch_bounds__(256)
void mdn_varlen_prep_kernel(const int32_t* __restrict__ cu, int64_t nseq, int64_t T, int C, int64_t NT,
                            int2* __restrict__ tab, int32_t* __restrict__ perm)
{
    constexpr int TILE = 2048;
    __shared__ int lens[TILE];
    const int tid = threadIdx.x;
    const int64_t i = (int64_t)blockIdx.x * 256 + tid;
    int li = 0;
    if (i < nseq) {
        int64_t c0, c1;
        seq_bounds(cu, i, T, c0, c1);
        li = (int)(c1 - c0);
        int64_t cn = cu[i + 1];
        cn = cn < 0 ? 0 : (cn > T ? T : cn);
        const int64_t next = i + 1 < nseq ? cn / C + i + 1 : NT;
        const int64_t base = c0 / C + i, nt = (c1 - c0 + C - 1) / C;
        if (i == 0)
            for (int64_t j = 0; j < base && j < NT; ++j) tab[j] = make_int2(0, 0);
        for (int64_t j = base; j < next && j < NT; ++j) {
            const int64_t n = j - base;
            tab[j] = n < nt ? make_int2((int)(c0 + n * C), (int)((c1 - c0 - n * C) < C ? (c1 - c0 - n * C) : C))
                            : make_int2(0, 0);
        }
    }
    int64_t rank = 0;
    for (int64_t t0 = 0; t0 < nseq; t0 += TILE) {
        const int n = (int)(nseq - t0 < TILE ? nseq - t0 : TILE);
        __syncthreads();
        for (int j = tid; j < n; j += 256) {
            int64_t c0, c1;
            seq_bounds(cu, t0 + j, T, c0, c1);
            lens[j] = (int)(c1 - c0);
        }
        __syncthreads();
        if (i < nseq)
            for (int j = 0; j < n; ++j) {
                const int lj = lens[j];
                rank += (lj > li) || (lj == li && t0 + j < i);
            }
    }
    if (i < nseq) perm[rank] = (int32_t)i;
}

hipError_t launch_varlen_prep(const ChunkArgs& a)
{
    if (a.nseq == 0) return hipSuccess;
    const int64_t blocks = (a.nseq + 255) / 256;
    hipLaunchKernelGGL(mdn_varlen_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)a.stream,
                       a.cu, a.nseq, a.T, a.C, a.NT, reinterpret_cast<int2*>(a.tab), a.perm);
    return hipGetLastError();
}

hipError_t launch_chunk_coef(const ChunkArgs& a)
{
    if (a.BH * a.NT == 0) return hipSuccess;
    // the coefficients depend on neither dk nor the element type
    switch (a.C) {
    case 16: return launch_intra_t<TraitsF32, 16, 16, true>(a);
    case 32: return launch_intra_t<TraitsF32, 16, 32, true>(a);
    case 64: return launch_intra_t<TraitsF32, 16, 64, true>(a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mdn
