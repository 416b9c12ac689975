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
//   mdn_intra_kernel  one workgroup per chunk tile (fully parallel): the
//                     coefficient scans, Gamma, the two C x C score products
//                     on the matrix cores, T by forward substitution in LDS;
//                     writes T, Aqk and the coefficient rows.
//   mdn_inter_kernel  one workgroup per (head, slab of 16*NW state columns),
//                     sequential over the chunks: vtilde, O (fused) and the
//                     fp32 S/M carry.  State columns are independent, so the
//                     slab split needs no communication.
#include "mdn_device.h"
#include "mdn_internal.h"
#include "../../include/mdn.h"

namespace mdn {

// ---------------------------------------------------------------------------
// mdn_intra_kernel
// ---------------------------------------------------------------------------
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
    constexpr int NCT = C / 16;
    constexpr int NJOB = NCT * (NCT + 1) / 2;      // lower-triangular 16x16 tiles
    constexpr int KSD = DK / Tr::KW;
    constexpr int GS = C + 4;                       // LDS row stride (floats)
    __shared__ float sA[C * GS];                    // A = (P K^T) o Gamma^-
    __shared__ float sG[C * GS];                    // Gamma
    __shared__ float sa[C], sbt[C], slm[C], se[C];

    const int64_t tile = blockIdx.x;
    const int64_t bh = tile / NT, n = tile % NT;
    const int64_t t0 = n * C;
    const int valid = (int)((T - t0) < C ? (T - t0) : C);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, nn = lane & 15;
    float* cf = coef + tile * MDN_COEF_ROWS * C;

    // -- coefficient scans (wave 0, lane r = token r) ----------------------
    if (wave == 0) {
        float a = 1.f, m = 1.f, bt = 0.f, e = 0.f;   // neutral padding
        if (lane < valid) {
            const size_t gi = (size_t)(bh * T + t0 + lane);
            a = alpha[gi]; m = mu[gi]; bt = beta[gi]; e = eta[gi];
        }
        const float la = wave_scan_add(logf(a), lane);
        const float lm = wave_scan_add(logf(m), lane);
        const float x = logf(bt) + lm - la;          // log beta_j + LM_j - LA_j
        const float lc = wave_scan_logaddexp(x, lane);
        const float b = expf(la + lc);
        float bprev = __shfl_up(b, 1, 64);
        if (lane == 0) bprev = 0.f;
        if (lane < C) {
            sa[lane] = a; sbt[lane] = bt; slm[lane] = lm; se[lane] = e;
            cf[MDN_COEF_ABAR * C + lane] = expf(la);
            cf[MDN_COEF_ABP * C + lane] = a * bprev;
            cf[MDN_COEF_B * C + lane] = b;
            cf[MDN_COEF_LA * C + lane] = la;
            cf[MDN_COEF_LM * C + lane] = lm;
            cf[MDN_COEF_LOGC * C + lane] = lc;
        }
    }
    __syncthreads();

    // -- Gamma, one column per lane (wave 0) --------------------------------
    // gamma_{r,i} = alpha_r gamma_{r-1,i} + beta_r exp(LM_r - LM_i), r >= i:
    // the mu ratio is a broadcast difference of the log cumsum (exponent
    // <= 0), the alpha ratio is applied as the running decay, and every term
    // is non-negative, so nothing overflows or cancels.
    if (wave == 0 && lane < C) {
        const float lmi = slm[lane], ei = se[lane];
        float gam = 0.f;
        for (int r = 0; r < C; ++r) {
            const float w = (r >= lane) ? expf(slm[r] - lmi) : 0.f;
            gam = sa[r] * gam + sbt[r] * w;
            sG[r * GS + lane] = ei * gam;
        }
        cf[MDN_COEF_GS * C + lane] = ei * gam;
        cf[MDN_COEF_GM * C + lane] = ei * expf(slm[C - 1] - lmi);
    }
    __syncthreads();

    if (gamma) {
        float* gp = gamma + tile * C * C;
        for (int idx = tid; idx < C * C; idx += 256) gp[idx] = sG[(idx / C) * GS + (idx % C)];
    }
    if constexpr (COEF_ONLY) return;

    // -- score products on the matrix cores ---------------------------------
    // job < NJOB: K K^T tile -> A (LDS);  job >= NJOB: Q K^T tile -> Aqk.
    const E* qh = q + (size_t)(bh * T + t0) * DK;
    const E* kh = k + (size_t)(bh * T + t0) * DK;
    E* Aq = Aqk + tile * C * C;
    for (int job = wave; job < 2 * NJOB; job += 4) {
        const int mat = job / NJOB;
        int idx = job % NJOB, tr = 0;
        while (idx > tr) { idx -= tr + 1; ++tr; }
        const int tc = idx;
        const int ra = 16 * tr + nn, rb = 16 * tc + nn;
        const E* xa = (mat == 0 ? kh : qh) + (size_t)ra * DK;
        const E* xb = kh + (size_t)rb * DK;
        floatx4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            const auto fa = ra < valid ? Contig<Tr>::load(xa, ks, g) : Contig<Tr>::zero();
            const auto fb = rb < valid ? Contig<Tr>::load(xb, ks, g) : Contig<Tr>::zero();
            acc = Tr::mma(fa, fb, acc);
        }
        const int i = 16 * tc + nn;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * tr + 4 * g + e;
            if (mat == 0) {
                sA[r * GS + i] = (i < r) ? sa[r] * acc[e] * sG[(r - 1) * GS + i] : 0.f;
            } else {
                Aq[r * C + i] = Tr::from_f((i <= r) ? acc[e] * sG[r * GS + i] : 0.f);
            }
        }
    }
    // upper tiles of Aqk are zero
    for (int idx = tid; idx < C * C; idx += 256) {
        const int r = idx / C, i = idx % C;
        if ((i >> 4) > (r >> 4)) Aq[idx] = Tr::from_f(0.f);
    }
    __syncthreads();

    // -- T = (I + A)^{-1} by forward substitution (wave 0, lane = column) ---
    // T[r][j] = delta_rj - sum_{i<r} A[r][i] T[i][j]
    if (wave == 0) {
        E* Tt = Tout + tile * C * C;
        float tcol[C];
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float s = (r == lane) ? 1.f : 0.f;
            const float* Ar = sA + r * GS;
#pragma unroll
            for (int i = 0; i < r; ++i) s = fmaf(-Ar[i], tcol[i], s);
            tcol[r] = s;
            if (lane < C) Tt[r * C + lane] = Tr::from_f(s);
        }
    }
}

// ---------------------------------------------------------------------------
// mdn_inter_kernel
// ---------------------------------------------------------------------------
template <typename Tr, int DK, int DV, int C, int NW>
__global__ __launch_bounds__(64 * NW)
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
    using frag = typename Tr::frag;
    constexpr int KW = Tr::KW, NSL = SL::NSLOT;
    constexpr int NDT = DK / 16, NCT = C / 16, KSD = DK / KW, KSC = C / KW;
    constexpr int KTS = C + 8;                       // row stride of the K^T tile
    constexpr int VEC = 16 / sizeof(E);              // elements per 16-byte load
    constexpr int SLABS = DV / (16 * NW);
    __shared__ __attribute__((aligned(16))) E sKt[DK * KTS];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = lane >> 4, nn = lane & 15;
    int bh, slab;
    xcd_head_map(blockIdx.x, SLABS, BH, bh, slab);
    const int col = (slab * NW + wave) * 16 + nn;

    const size_t sbase = (size_t)bh * DK * DV;
    floatx4 S[NDT], M[NDT];
#pragma unroll
    for (int td = 0; td < NDT; ++td)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t off = sbase + (size_t)(16 * td + 4 * g + e) * DV + col;
            S[td][e] = S0 ? S0[off] : 0.f;
            M[td][e] = M0 ? M0[off] : 0.f;
        }

    for (int64_t n = 0; n < NT; ++n) {
        const int64_t t0 = n * C;
        const int valid = (int)((T - t0) < C ? (T - t0) : C);
        const size_t tile = (size_t)bh * NT + n;
        const size_t rowbase = (size_t)bh * T + t0;
        const float* cf = coef + tile * MDN_COEF_ROWS * C;
        const E* kc = k + rowbase * DK;
        const E* qc = q + rowbase * DK;

        // K chunk -> LDS, transposed: sKt[d][c] = K[c][d]
        __syncthreads();
        for (int idx = threadIdx.x; idx < C * (DK / VEC); idx += 64 * NW) {
            const int c = idx / (DK / VEC), d0 = (idx % (DK / VEC)) * VEC;
            union { uint4 u; E x[VEC]; } ld;
            ld.u = c < valid ? *reinterpret_cast<const uint4*>(kc + (size_t)c * DK + d0)
                             : uint4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < VEC; ++i) sKt[(d0 + i) * KTS + c] = ld.x[i];
        }
        __syncthreads();

        // state as B operands (contraction over the dk rows)
        frag Sb[KSD], Mb[KSD];
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) { Sb[ks] = SL::from_acc(S, ks); Mb[ks] = SL::from_acc(M, ks); }

        // W = V - Diag(abar) K S + Diag(alpha b_prev) K M
        floatx4 W[NCT];
#pragma unroll
        for (int tc = 0; tc < NCT; ++tc) {
            const int r = 16 * tc + nn;
            floatx4 ks_ = zero4(), km_ = zero4();
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const frag a = r < valid ? SL::load_row(kc + (size_t)r * DK, ks, g) : SL::zero();
                ks_ = Tr::mma(a, Sb[ks], ks_);
                km_ = Tr::mma(a, Mb[ks], km_);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 16 * tc + 4 * g + e;
                const float vv = rr < valid ? Tr::to_f(v[(rowbase + rr) * DV + col]) : 0.f;
                W[tc][e] = vv - cf[MDN_COEF_ABAR * C + rr] * ks_[e] + cf[MDN_COEF_ABP * C + rr] * km_[e];
            }
        }

        // vtilde = T W
        frag Wb[KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) Wb[ks] = SL::from_acc(W, ks);
        floatx4 Vx[NCT];
        const E* Tt = Tm + tile * C * C;
#pragma unroll
        for (int tc = 0; tc < NCT; ++tc) {
            floatx4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
                acc = Tr::mma(SL::load_row(Tt + (16 * tc + nn) * C, ks, g), Wb[ks], acc);
            Vx[tc] = acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 16 * tc + 4 * g + e;
                if (rr < valid) Vt[(rowbase + rr) * DV + col] = Tr::from_f(acc[e]);
            }
        }

        // O = Diag(abar) Q S - Diag(b) Q M + Aqk vtilde   (chunk-start S, M)
        frag Vb[KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) Vb[ks] = SL::from_acc(Vx, ks);
        const E* Aq = Aqk + tile * C * C;
#pragma unroll
        for (int tc = 0; tc < NCT; ++tc) {
            const int r = 16 * tc + nn;
            floatx4 qs = zero4(), qm = zero4(), ai = zero4();
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const frag a = r < valid ? SL::load_row(qc + (size_t)r * DK, ks, g) : SL::zero();
                qs = Tr::mma(a, Sb[ks], qs);
                qm = Tr::mma(a, Mb[ks], qm);
            }
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
                ai = Tr::mma(SL::load_row(Aq + (16 * tc + nn) * C, ks, g), Vb[ks], ai);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 16 * tc + 4 * g + e;
                if (rr < valid) {
                    const float o = cf[MDN_COEF_ABAR * C + rr] * qs[e] - cf[MDN_COEF_B * C + rr] * qm[e] + ai[e];
                    O[(rowbase + rr) * DV + col] = Tr::from_f(o);
                }
            }
        }

        // S <- abar_C S - b_C M + K^T Diag(gS) vtilde ; M <- mubar_C M - K^T Diag(gM) vtilde
        const float abarC = cf[MDN_COEF_ABAR * C + C - 1];
        const float bC = cf[MDN_COEF_B * C + C - 1];
        const float mubarC = expf(cf[MDN_COEF_LM * C + C - 1]);
        frag VS[KSC], VM[KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            float sS[NSL], sM[NSL];
#pragma unroll
            for (int j = 0; j < NSL; ++j) {
                const int rr = SL::row(ks, g, j);
                sS[j] = cf[MDN_COEF_GS * C + rr];
                sM[j] = -cf[MDN_COEF_GM * C + rr];
            }
            VS[ks] = SL::from_acc_scaled(Vx, ks, sS);
            VM[ks] = SL::from_acc_scaled(Vx, ks, sM);
        }
#pragma unroll
        for (int td = 0; td < NDT; ++td) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float s_ = abarC * S[td][e] - bC * M[td][e];
                M[td][e] = mubarC * M[td][e];
                S[td][e] = s_;
            }
            const E* ktr = sKt + (16 * td + nn) * KTS;
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                const frag a = SL::load_row(ktr, ks, g);
                S[td] = Tr::mma(a, VS[ks], S[td]);
                M[td] = Tr::mma(a, VM[ks], M[td]);
            }
        }
    }

#pragma unroll
    for (int td = 0; td < NDT; ++td)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t off = sbase + (size_t)(16 * td + 4 * g + e) * DV + col;
            ST[off] = S[td][e];
            MT[off] = M[td][e];
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

template <typename Tr, int DK, int C, int NW>
static hipError_t launch_inter_t(const ChunkArgs& a)
{
    using E = typename Tr::elem;
    const int64_t grid = a.BH * (a.dv / (16 * NW));
    hipLaunchKernelGGL((mdn_inter_kernel<Tr, DK, DK, C, NW>), dim3((unsigned)grid), dim3(64 * NW), 0,
                       (hipStream_t)a.stream, (const E*)a.q, (const E*)a.k, (const E*)a.v,
                       (const E*)a.Tmat, (const E*)a.Aqk, a.coef, a.S0, a.M0,
                       (E*)a.O, a.ST, a.MT, (E*)a.Vt, a.T, a.NT, (int)a.BH);
    return hipGetLastError();
}

// Workgroups of two waves share one staged K^T tile; fall back to one wave
// per workgroup when two-wave slabs would leave fewer than 256 workgroups
// (one per compute unit) or the head has a single 16-column slab.
template <typename Tr, int DK, int C>
static hipError_t launch_inter_nw(const ChunkArgs& a)
{
    if constexpr (DK >= 32) {
        if (a.BH * (DK / 32) >= 256) return launch_inter_t<Tr, DK, C, 2>(a);
    }
    return launch_inter_t<Tr, DK, C, 1>(a);
}

template <typename Tr, bool COEF_ONLY>
static hipError_t intra_dispatch(const ChunkArgs& a)
{
    if constexpr (std::is_same<Tr, TraitsBf16>::value) {
        switch (a.dk * 1000 + a.C) {
        case 32032: return launch_intra_t<Tr, 32, 32, COEF_ONLY>(a);
        case 32064: return launch_intra_t<Tr, 32, 64, COEF_ONLY>(a);
        case 64032: return launch_intra_t<Tr, 64, 32, COEF_ONLY>(a);
        case 64064: return launch_intra_t<Tr, 64, 64, COEF_ONLY>(a);
        case 128032: return launch_intra_t<Tr, 128, 32, COEF_ONLY>(a);
        case 128064: return launch_intra_t<Tr, 128, 64, COEF_ONLY>(a);
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (a.dk * 1000 + a.C) {
        case 16016: return launch_intra_t<Tr, 16, 16, COEF_ONLY>(a);
        case 16032: return launch_intra_t<Tr, 16, 32, COEF_ONLY>(a);
        case 16064: return launch_intra_t<Tr, 16, 64, COEF_ONLY>(a);
        case 32016: return launch_intra_t<Tr, 32, 16, COEF_ONLY>(a);
        case 32032: return launch_intra_t<Tr, 32, 32, COEF_ONLY>(a);
        case 32064: return launch_intra_t<Tr, 32, 64, COEF_ONLY>(a);
        case 64016: return launch_intra_t<Tr, 64, 16, COEF_ONLY>(a);
        case 64032: return launch_intra_t<Tr, 64, 32, COEF_ONLY>(a);
        case 64064: return launch_intra_t<Tr, 64, 64, COEF_ONLY>(a);
        case 128016: return launch_intra_t<Tr, 128, 16, COEF_ONLY>(a);
        case 128032: return launch_intra_t<Tr, 128, 32, COEF_ONLY>(a);
        case 128064: return launch_intra_t<Tr, 128, 64, COEF_ONLY>(a);
        default: return hipErrorInvalidValue;
        }
    }
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

hipError_t launch_chunk_intra(const ChunkArgs& a)
{
    if (a.BH * a.NT == 0) return hipSuccess;
    return a.dtype == MDN_BF16 ? intra_dispatch<TraitsBf16, false>(a) : intra_dispatch<TraitsF32, false>(a);
}

hipError_t launch_chunk_coef(const ChunkArgs& a)
{
    if (a.BH * a.NT == 0) return hipSuccess;
    // coefficients do not depend on dk or the element type
    ChunkArgs b = a;
    b.dk = 16;
    switch (a.C) {
    case 16: return launch_intra_t<TraitsF32, 16, 16, true>(b);
    case 32: return launch_intra_t<TraitsF32, 16, 32, true>(b);
    case 64: return launch_intra_t<TraitsF32, 16, 64, true>(b);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_inter(const ChunkArgs& a)
{
    if (a.BH == 0) return hipSuccess;
    return a.dtype == MDN_BF16 ? inter_dispatch<TraitsBf16>(a) : inter_dispatch<TraitsF32>(a);
}

}  // namespace mdn
