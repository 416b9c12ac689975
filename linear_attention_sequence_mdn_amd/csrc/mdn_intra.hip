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
//   5. T and Aqk leave through LDS tiles as full 16-byte stores.
#include "mdn_device.h"
#include "mdn_internal.h"
#include "mdn_lds.h"
#include "../../include/mdn.h"

namespace mdn {

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
    static constexpr int DS = 20;                    // row stride of a diagonal inverse (floats)
    static constexpr int TD = NCT * 16 * DS * 4;
    // region X: K, Q tiles; then A (fp32) and the Aqk out tile
    static constexpr int RX = 2 * KT > ABYTES + OUT ? 2 * KT : ABYTES + OUT;
    // region Y: Gamma (fp32); then the T out tile and the diagonal inverses
    static constexpr int RY = C * C * 4 > OUT + 2 * TD ? C * C * 4 : OUT + 2 * TD;
    // Gamma scan: NB row blocks of RB rows, one thread per (block, column)
    static constexpr int NB = 256 / C;
    static constexpr int RB = C / NB;
    static_assert(NB * C == 256 && RB * NB == C, "256 threads cover the C x C Gamma scan");
};

template <typename Tr, int DK, int C, bool COEF_ONLY>
__global__ __launch_bounds__(256)
void mdn_intra_kernel(const typename Tr::elem* __restrict__ q,
                      const typename Tr::elem* __restrict__ k,
                      const float* __restrict__ alpha, const float* __restrict__ mu,
                      const float* __restrict__ beta, const float* __restrict__ eta,
                      int64_t T, int64_t NT,
                      typename Tr::elem* __restrict__ Tout,
                      typename Tr::elem* __restrict__ Aqk,
                      float* __restrict__ coef,
                      float* __restrict__ gamma)
{
    using E = typename Tr::elem;
    using SL = Slots<Tr>;
    using L = IntraLayout<Tr, DK, C>;
    using frag = typename Tr::frag;
    constexpr int NCT = L::NCT, KSD = DK / Tr::KW, NB = L::NB, RB = L::RB;
    constexpr bool BF16 = std::is_same<Tr, TraitsBf16>::value;

    __shared__ __attribute__((aligned(16))) char rx[COEF_ONLY ? 16 : L::RX];
    __shared__ __attribute__((aligned(16))) char ry[L::RY];
    __shared__ float sa[C], sbt[C], slm[C], sla[C], se[C];
    __shared__ float xe[NB][C];                      // Gamma block carries

    const int64_t tile = blockIdx.x;
    const int64_t bh = tile / NT, n = tile % NT;
    const size_t rowbase = (size_t)(bh * T + n * C);
    const int valid = (int)((T - n * C) < C ? (T - n * C) : C);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, nn = lane & 15;
    float* cf = coef + tile * MDN_COEF_ROWS * C;

    // ---- 1. K, Q -> LDS (waves 1-3); gates and scans (wave 0) ----------------
    if constexpr (!COEF_ONLY) {
        if (wave > 0) {
            // 2*NCT blocks of 16 rows (K blocks, then Q blocks), dealt to waves 1-3;
            // rows past `valid` repeat the last valid row (zeroed below)
            const unsigned vlast = (unsigned)valid - 1;
            auto seq_row = [&](unsigned r) { return (r < vlast ? r : vlast) * (unsigned)(DK * L::ES); };
            const uint32_t base = lds_addr(rx);
#pragma unroll
            for (int j = 0; j < 2 * NCT; ++j) {
                if (j % 3 == wave - 1) {
                    const E* src = (j < NCT ? k : q) + rowbase * DK;
                    dma_tile<16, L::PK>(base + (j < NCT ? 0 : L::KT), reinterpret_cast<const char*>(src), seq_row,
                                        lane, 16 * (j % NCT));
                }
            }
        }
    }
    if (wave == 0) {
        float a = 1.f, m = 1.f, bt = 0.f, e = 0.f;   // neutral padding past the end
        if (lane < valid) {
            const size_t gi = rowbase + lane;
            a = alpha[gi]; m = mu[gi]; bt = beta[gi]; e = eta[gi];
        }
        const float la = wave_scan_add(logf(a), lane);
        const float lm = wave_scan_add(logf(m), lane);
        const float lc = wave_scan_logaddexp(logf(bt) + lm - la, lane);
        const float b = expf(la + lc);
        float bprev = __shfl_up(b, 1, 64);
        if (lane == 0) bprev = 0.f;
        if (lane < C) {
            sa[lane] = a; sbt[lane] = bt; slm[lane] = lm; sla[lane] = la; se[lane] = e;
            cf[MDN_COEF_ABAR * C + lane] = expf(la);
            cf[MDN_COEF_ABP * C + lane] = a * bprev;
            cf[MDN_COEF_B * C + lane] = b;
            cf[MDN_COEF_LA * C + lane] = la;
            cf[MDN_COEF_LM * C + lane] = lm;
            cf[MDN_COEF_LOGC * C + lane] = lc;
        }
    }
    lds_barrier();

    // ---- 2. Gamma (fp32, row-major C x C in region Y) ------------------------
    float* Gm = reinterpret_cast<float*>(ry);
    {
        const int i = tid % C, bk = tid / C, r0 = bk * RB;
        const float lmi = slm[i], ei = se[i];
        float lv[RB];
        float loc = 0.f;
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const int r = r0 + j;
            loc = sa[r] * loc + (r >= i ? sbt[r] * expf(slm[r] - lmi) : 0.f);
            lv[j] = loc;
        }
        xe[bk][i] = loc;
        lds_barrier();
        // gamma_{r0-1,i}: carries of the earlier blocks, each decayed by the
        // product of alpha over the next block
        float G = 0.f, lprev = 0.f;
#pragma unroll
        for (int bb = 0; bb < NB - 1; ++bb) {
            if (bb < bk) {
                const float lend = sla[bb * RB + RB - 1];
                G = expf(lend - lprev) * G + xe[bb][i];
                lprev = lend;
            }
        }
        float last = 0.f;
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const int r = r0 + j;
            last = ei * (lv[j] + expf(sla[r] - lprev) * G);
            Gm[r * C + i] = last;
        }
        if (bk == NB - 1) {                          // this thread holds row C-1
            cf[MDN_COEF_GS * C + i] = last;
            cf[MDN_COEF_GM * C + i] = ei * expf(slm[C - 1] - lmi);
        }
    }
    if constexpr (COEF_ONLY) {
        lds_barrier();
        if (gamma) {
            float* gp = gamma + tile * C * C;
            for (int idx = tid; idx < C * C; idx += 256) gp[idx] = Gm[idx];
        }
        return;
    }

    __builtin_amdgcn_s_waitcnt(0);                   // this wave's K/Q copies have landed
    lds_barrier();                                   // Gamma and the K/Q tiles visible
    const char* Kl = rx;
    const char* Ql = rx + L::KT;
    if (valid < C) {                                 // ragged last chunk: zero rows past the end
        constexpr int W = L::PK;                     // 16-byte words per row
        for (int w = valid * W + tid; w < C * W; w += 256) {
            reinterpret_cast<uint4*>(rx)[w] = uint4{0u, 0u, 0u, 0u};
            reinterpret_cast<uint4*>(rx + L::KT)[w] = uint4{0u, 0u, 0u, 0u};
        }
        lds_barrier();
    }

    // ---- 3. K K^T and Q K^T on the matrix cores --------------------------------
    // Accumulator row x of block t stands for chunk row perm(16t + x) (bf16
    // slot map; identity for fp32), so the 16 rows of an operand read get
    // distinct swizzle keys.  With four or more row blocks a wave owns row
    // block `tr` of both products; otherwise wave w owns product w / NCT.
    constexpr bool BOTH = NCT >= 4;
    const int tr = BOTH ? wave : wave % NCT;
    const int mat = BOTH ? 0 : wave / NCT;
    const bool doK = BOTH || mat == 0, doQ = BOTH || mat == 1;
    auto lower = [&](int rb, int cb) { return BF16 ? ((cb >> 1) <= (rb >> 1)) : (cb <= rb); };
    floatx4 accK[NCT], accQ[NCT];
#pragma unroll
    for (int tc = 0; tc < NCT; ++tc) { accK[tc] = zero4(); accQ[tc] = zero4(); }
    if (doK || doQ) {
        frag aK[KSD], aQ[KSD];
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            if (doK) aK[ks] = LdsA<Tr, L::PK>::load(Kl, SL::perm(16 * tr + nn), ks, g);
            if (doQ) aQ[ks] = LdsA<Tr, L::PK>::load(Ql, SL::perm(16 * tr + nn), ks, g);
        }
#pragma unroll
        for (int tc = 0; tc < NCT; ++tc) {
            if (lower(tr, tc)) {
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    const frag bk = LdsA<Tr, L::PK>::load(Kl, SL::perm(16 * tc + nn), ks, g);
                    if (doK) accK[tc] = Tr::mma(aK[ks], bk, accK[tc]);
                    if (doQ) accQ[tc] = Tr::mma(aQ[ks], bk, accQ[tc]);
                }
            }
        }
        // apply the decay weights (Gamma is still in region Y)
#pragma unroll
        for (int tc = 0; tc < NCT; ++tc) {
            const int i = SL::perm(16 * tc + nn);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = SL::perm(16 * tr + 4 * g) + e;
                accK[tc][e] = (i < r) ? sa[r] * accK[tc][e] * Gm[(r > 0 ? r - 1 : 0) * C + i] : 0.f;
                accQ[tc][e] = (i <= r) ? accQ[tc][e] * Gm[r * C + i] : 0.f;
            }
        }
    }
    lds_barrier();                                   // K, Q and Gamma reads done

    float* sA = reinterpret_cast<float*>(rx);        // A, fp32, row stride AS
    E* oAq = reinterpret_cast<E*>(rx + L::ABYTES);   // Aqk out tile, row-major C x C
    E* oT = reinterpret_cast<E*>(ry);                // T out tile, row-major C x C
    float* sTd = reinterpret_cast<float*>(ry + L::OUT);   // T_aa, row-major, stride DS
    float* sTt = sTd + NCT * 16 * L::DS;                  // T_aa transposed
    if (doK || doQ) {
#pragma unroll
        for (int tc = 0; tc < NCT; ++tc) {
            const int i = SL::perm(16 * tc + nn);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = SL::perm(16 * tr + 4 * g) + e;
                if (doK) sA[r * L::AS + i] = accK[tc][e];
                if (doQ) oAq[r * C + i] = Tr::from_f(accQ[tc][e]);
            }
        }
    }
    lds_barrier();

    // ---- 4a. diagonal blocks of T: forward substitution, lane = column -------
    if (wave < NCT) {
        const int a = wave, j = nn;
        float tcol[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float* Ar = sA + (16 * a + r) * L::AS + 16 * a;
            float s = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) s = fmaf(-Ar[i], tcol[i], s);
            tcol[r] = s;
        }
        if (g == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sTd[(16 * a + r) * L::DS + j] = tcol[r];
                sTt[(16 * a + j) * L::DS + r] = tcol[r];
                oT[(16 * a + r) * C + 16 * a + j] = Tr::from_f(tcol[r]);
            }
        }
    }
    for (int idx = tid; idx < C * C; idx += 256) {   // strictly upper blocks are zero
        const int r = idx / C, c = idx % C;
        if ((r >> 4) < (c >> 4)) oT[idx] = Tr::from_f(0.f);
    }
    lds_barrier();

    // ---- 4b. column block b of T below the diagonal (fp32 matrix cores) -------
    // Contraction slot map: in step ks, lane group g carries inner index
    // 4g + ks of the 16-block, so an accumulator (rows 4g + e) is the next
    // product's B operand as it stands.
    if (wave < NCT - 1) {
        const int b = wave;
        floatx4 Tc[NCT];
#pragma unroll
        for (int c = 0; c < NCT; ++c)
            Tc[c] = (c == b) ? *reinterpret_cast<const floatx4*>(sTt + (16 * c + nn) * L::DS + 4 * g) : zero4();
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
                const floatx4 To = *reinterpret_cast<const floatx4*>(sTd + (16 * a + nn) * L::DS + 4 * g);
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
    uint4* gT = reinterpret_cast<uint4*>(Tout + tile * C * C);
    uint4* gA = reinterpret_cast<uint4*>(Aqk + tile * C * C);
    for (int p = tid; p < NP; p += 256) {
        gT[p] = reinterpret_cast<const uint4*>(oT)[p];
        gA[p] = reinterpret_cast<const uint4*>(oAq)[p];
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
    hipLaunchKernelGGL((mdn_intra_kernel<Tr, DK, C, COEF_ONLY>), dim3((unsigned)tiles), dim3(256), 0,
                       (hipStream_t)a.stream, (const E*)a.q, (const E*)a.k,
                       a.alpha, a.mu, a.beta, a.eta, a.T, a.NT,
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
