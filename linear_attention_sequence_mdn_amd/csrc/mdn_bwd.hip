// mdn_bwd.hip -- chunkwise backward of the Momentum DeltaNet forward (gfx950).
//
// The pages give the forward only; the backward is the chain rule applied
// to the chunk equations the forward kernels use (chunk n, chunk-local rows
// r, S and M the chunk-start states, L the chunk's last row):
//
//   W = V - Diag(abar) K S + Diag(ab) K M,  vtilde = T W,  ab_r = alpha_r b_{r-1}
//   O = Diag(abar) Q S - Diag(b) Q M + Aqk vtilde
//   S' = abar_L S - b_L M + K^T Diag(gS) vtilde,   M' = mubar_L M - K^T Diag(gM) vtilde
//
// Four launches after the intra stage (which recomputes T^T, Aqk^T and the
// coefficient rows):
//   replay  one workgroup per (head, column slab), forward over the chunks:
//           the chunk-start S[n], M[n] from the stored vtilde (state update
//           only; T is not needed), written to the workspace;
//   carry   one workgroup per (head, column slab), backward over the chunks,
//           with dS, dM the adjoints of the chunk-end states:
//             dvt = Aqk^T dO + Diag(gS) K dS - Diag(gM) K dM
//             dW  = T^T dvt                           (= dV, written out)
//             dS <- abar_L dS + Q^T Diag(abar) dO - K^T Diag(abar) dW
//             dM <- mubar_L dM - b_L dS + -Q^T Diag(b) dO + K^T Diag(ab) dW
//           the chunk-end adjoints of every chunk go to the workspace;
//   sgrad   one workgroup per chunk tile: the products with the states,
//             dq += Diag(abar) dO S^T - Diag(b) dO M^T
//             dk += -Diag(abar) dW S^T + Diag(ab) dW M^T + Diag(gS) vtilde dS'^T - Diag(gM) vtilde dM'^T
//           and the coefficient adjoints they give (row dots with q and k);
//   cgrad   one workgroup per chunk tile: the products inside the chunk
//           (dAqk = dO vtilde^T, dA = -dW vtilde^T, their weights Gamma and
//           Gamma^-), then the gate gradients through the coefficient
//           definitions, and the final dq, dk.
#include "mdn_device.h"
#include "mdn_internal.h"
#include "mdn_lds.h"
#include "../../include/mdn.h"

namespace mdn {

// K^T (or Q^T) operand of a state-row product for d-tile td, contraction
// step ks over chunk rows (natural order 32ks + 8g + j), from a swizzled
// tile of P pieces per row.
template <typename Tr, int P> struct TrOperand;
template <int P> struct TrOperand<TraitsBf16, P> {
    static __device__ __forceinline__ bf16x8 load(const char* X, int td, int ks, int lane) {
        const int g = lane >> 4, s = lane & 15;
        const int r0 = 32 * ks + 8 * g + (s >> 2);
        const int b = 2 * (Slots<TraitsBf16>::perm(16 * td) + 8 * (s & 3));
        union { shortx4 h[2]; bf16x8 v; } f;
        f.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(X + swz<P>(r0, b)));
        f.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(X + swz<P>(r0 + 4, b)));
        return f.v;
    }
};
template <int P> struct TrOperand<TraitsF32, P> {
    static __device__ __forceinline__ float load(const char* X, int td, int ks, int lane) {
        const int g = lane >> 4, m = lane & 15;
        const int r = 16 * (ks >> 2) + 4 * g + (ks & 3);
        return *reinterpret_cast<const float*>(X + swz<P>(r, 4 * (16 * td + m)));
    }
};

// Plain row-major tile of OW elements per row as the B operand of a product
// over its rows, column tile ct, contraction step ks (natural row order).
template <typename Tr, int OW> struct ColOperand;
template <int OW> struct ColOperand<TraitsBf16, OW> {
    static __device__ __forceinline__ bf16x8 load(const char* X, int ct, int ks, int lane) {
        const int g = lane >> 4, s = lane & 15;
        const int r0 = 32 * ks + 8 * g + (s >> 2);
        const int b = 2 * (16 * ct + 4 * (s & 3));
        union { shortx4 h[2]; bf16x8 v; } f;
        f.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(X + r0 * OW * 2 + b));
        f.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(X + (r0 + 4) * OW * 2 + b));
        return f.v;
    }
};
template <int OW> struct ColOperand<TraitsF32, OW> {
    static __device__ __forceinline__ float load(const char* X, int ct, int ks, int lane) {
        const int g = lane >> 4, m = lane & 15;
        const int r = 16 * (ks >> 2) + 4 * g + (ks & 3);
        return *reinterpret_cast<const float*>(X + 4 * (r * OW + 16 * ct + m));
    }
};

// A operand from a plain row (contraction index contiguous) in the slot
// order of ColOperand and TrOperand: for bf16 the natural order, for fp32
// contraction index 16(ks/4) + 4g + ks%4 in step ks.
template <typename Tr> struct SlotRow;
template <> struct SlotRow<TraitsBf16> {
    static __device__ __forceinline__ bf16x8 load(const __bf16* rowp, int ks, int g) {
        return Contig<TraitsBf16>::load(rowp, ks, g);
    }
};
template <> struct SlotRow<TraitsF32> {
    static __device__ __forceinline__ float load(const float* rowp, int ks, int g) {
        return rowp[Slots<TraitsF32>::row(ks, g, 0)];
    }
};

// Each contraction slot of an operand scaled by its own factor.
template <typename Tr> struct FragScale;
template <> struct FragScale<TraitsBf16> {
    static __device__ __forceinline__ bf16x8 apply(bf16x8 v, const float (&s)[8]) {
        bf16x8 r;
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = (__bf16)((float)v[j] * s[j]);
        return r;
    }
};
template <> struct FragScale<TraitsF32> {
    static __device__ __forceinline__ float apply(float v, const float (&s)[1]) { return v * s[0]; }
};

// ---------------------------------------------------------------------------
// replay: chunk-start states from vtilde
// ---------------------------------------------------------------------------
template <typename Tr, int D, int C, int NCOL>
struct ReplayLayout {
    using E = typename Tr::elem;
    static constexpr int ES = sizeof(E);
    static constexpr int PK = D * ES / 16;
    static constexpr int PV = 16 * NCOL * ES / 16;
    static constexpr int PC = MDN_COEF_ROWS * C * 4 / 16;
    static constexpr int K0 = 0;
    static constexpr int V0 = K0 + C * PK * 16;
    static constexpr int CF0 = V0 + C * PV * 16;
    static constexpr int BUF = CF0 + PC * 16;
};

template <typename Tr, int D, int C, int NCOL>
__global__ __launch_bounds__(64 * (NCOL + 2))
void mdn_bwd_replay_kernel(const typename Tr::elem* __restrict__ k, const typename Tr::elem* __restrict__ Vt,
                           const float* __restrict__ coef, const float* __restrict__ S0,
                           const float* __restrict__ M0, typename Tr::elem* __restrict__ Sst,
                           typename Tr::elem* __restrict__ Mst, int64_t T, int64_t NT, int BH)
{
    using E = typename Tr::elem;
    using SL = Slots<Tr>;
    using LT = ReplayLayout<Tr, D, C, NCOL>;
    using frag = typename Tr::frag;
    constexpr int NSL = SL::NSLOT, KSC = C / Tr::KW, NDH = D / 16, SLABS = D / (16 * NCOL), OW = 16 * NCOL;
    __shared__ __attribute__((aligned(16))) char stA[LT::BUF];
    __shared__ __attribute__((aligned(16))) char stB[LT::BUF];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, nn = lane & 15;
    int bh, slab;
    xcd_head_map(blockIdx.x, SLABS, BH, bh, slab);
    const int col0 = slab * OW;
    auto valid_of = [&](int64_t n) { return (int)((T - n * C) < C ? (T - n * C) : C); };

    if (wave >= NCOL) {
        const int lw = wave - NCOL;
        auto issue = [&](uint32_t buf, int64_t m) __attribute__((always_inline)) {
            const size_t rb = (size_t)bh * T + m * C, tile = (size_t)bh * NT + m;
            const unsigned vlast = (unsigned)valid_of(m) - 1;
            auto seq_row = [&](unsigned r) { return (r < vlast ? r : vlast) * (unsigned)(D * LT::ES); };
            auto cf_row = [](unsigned) { return 0u; };
            if (lw == 0) {
                dma_tile<C, LT::PK>(buf + LT::K0, reinterpret_cast<const char*>(k + rb * D), seq_row, lane);
            } else {
                dma_plain<C, LT::PV>(buf + LT::V0, reinterpret_cast<const char*>(Vt + rb * D + col0), seq_row, lane);
                dma_plain<1, LT::PC>(buf + LT::CF0, reinterpret_cast<const char*>(coef + tile * MDN_COEF_ROWS * C),
                                     cf_row, lane);
            }
        };
        const uint32_t aA = lds_addr(stA), aB = lds_addr(stB);
        if (NT > 0) issue(aA, 0);
        for (int64_t n = 0; n < NT; ++n) {
            __builtin_amdgcn_s_waitcnt(0);
            lds_barrier();                              // chunk n staged; buffer of chunk n-1 free
            if (n + 1 < NT) issue((n & 1) ? aA : aB, n + 1);
        }
        return;
    }

    const int ct = wave;
    const int col = col0 + 16 * ct + nn;
    const size_t sbase = (size_t)bh * D * D;
    floatx4 XS[NDH], XM[NDH];
#pragma unroll
    for (int t = 0; t < NDH; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t off = sbase + (size_t)SL::perm(16 * t + 4 * g + e) * D + col;
            XS[t][e] = S0 ? S0[off] : 0.f;
            XM[t][e] = M0 ? M0[off] : 0.f;
        }
    for (int64_t n = 0; n < NT; ++n) {
        lds_barrier();
        const char* cur = (n & 1) ? stB : stA;
        const char* Kl = cur + LT::K0;
        const char* Vl = cur + LT::V0;
        const float* cf = reinterpret_cast<const float*>(cur + LT::CF0);
        // the chunk-start state of chunk n
        E* so = Sst + ((size_t)bh * NT + n) * D * D;
        E* mo = Mst + ((size_t)bh * NT + n) * D * D;
#pragma unroll
        for (int t = 0; t < NDH; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const size_t off = (size_t)SL::perm(16 * t + 4 * g + e) * D + col;
                so[off] = Tr::from_f(XS[t][e]);
                mo[off] = Tr::from_f(XM[t][e]);
            }
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
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            float gs[NSL], gm[NSL];
            SL::load_row(cf + MDN_COEF_GS * C, ks, g, gs);
            SL::load_row(cf + MDN_COEF_GM * C, ks, g, gm);
#pragma unroll
            for (int j = 0; j < NSL; ++j) gm[j] = -gm[j];
            const frag vb = ColOperand<Tr, OW>::load(Vl, ct, ks, lane);
            const frag VS = FragScale<Tr>::apply(vb, gs), VM = FragScale<Tr>::apply(vb, gm);
#pragma unroll
            for (int t = 0; t < NDH; ++t) {
                const frag kT = TrOperand<Tr, LT::PK>::load(Kl, t, ks, lane);
                XS[t] = Tr::mma(kT, VS, XS[t]);
                XM[t] = Tr::mma(kT, VM, XM[t]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// carry: reverse pass of the state adjoints
// ---------------------------------------------------------------------------
template <typename Tr, int D, int C, int NCOL, int NBUF>
struct CarryLayout {
    using E = typename Tr::elem;
    static constexpr int ES = sizeof(E);
    static constexpr int PK = D * ES / 16;
    static constexpr int PT = C * ES / 16;
    static constexpr int PV = 16 * NCOL * ES / 16;
    static constexpr int PC = MDN_COEF_ROWS * C * 4 / 16;
    static constexpr int K0 = 0;
    static constexpr int Q0 = K0 + C * PK * 16;
    static constexpr int TT0 = Q0 + C * PK * 16;
    static constexpr int AT0 = TT0 + C * PT * 16;
    static constexpr int O0 = AT0 + C * PT * 16;
    static constexpr int CF0 = O0 + C * PV * 16;
    static constexpr int BUF = CF0 + PC * 16;
    static constexpr int TOTAL = NBUF * BUF;
};

template <typename Tr, int D, int C>
struct CarryPick {
    static constexpr int LIMIT = 160 * 1024 - 1024;
    static constexpr int NCOL = D >= 32 ? 2 : 1;
    static constexpr int NBUF = CarryLayout<Tr, D, C, NCOL, 2>::TOTAL <= LIMIT ? 2 : 1;
    static_assert(CarryLayout<Tr, D, C, NCOL, NBUF>::TOTAL <= LIMIT, "LDS");
};

template <typename Tr, int D, int C, int NCOL, int NBUF>
__global__ __launch_bounds__(64 * (NCOL + 2))
void mdn_bwd_carry_kernel(const typename Tr::elem* __restrict__ q, const typename Tr::elem* __restrict__ k,
                          const typename Tr::elem* __restrict__ TT, const typename Tr::elem* __restrict__ AT,
                          const float* __restrict__ coef, const typename Tr::elem* __restrict__ dO,
                          const float* __restrict__ dST, const float* __restrict__ dMT,
                          typename Tr::elem* __restrict__ dv, typename Tr::elem* __restrict__ dSst,
                          typename Tr::elem* __restrict__ dMst, float* __restrict__ dS0,
                          float* __restrict__ dM0, int64_t T, int64_t NT, int BH)
{
    using E = typename Tr::elem;
    using SL = Slots<Tr>;
    using LT = CarryLayout<Tr, D, C, NCOL, NBUF>;
    using frag = typename Tr::frag;
    constexpr int NSL = SL::NSLOT, KSC = C / Tr::KW, KSD = D / Tr::KW, NCT = C / 16, NDH = D / 16;
    constexpr int SLABS = D / (16 * NCOL), OW = 16 * NCOL;
    __shared__ __attribute__((aligned(16))) char stA[LT::BUF];
    __shared__ __attribute__((aligned(16))) char stB[NBUF == 2 ? LT::BUF : 16];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, nn = lane & 15;
    int bh, slab;
    xcd_head_map(blockIdx.x, SLABS, BH, bh, slab);
    const int col0 = slab * OW;
    auto valid_of = [&](int64_t n) { return (int)((T - n * C) < C ? (T - n * C) : C); };

    if (wave >= NCOL) {
        const int lw = wave - NCOL;
        // iteration it handles chunk NT - 1 - it
        auto issue = [&](uint32_t buf, int64_t m) __attribute__((always_inline)) {
            const size_t rb = (size_t)bh * T + m * C, tile = (size_t)bh * NT + m;
            const unsigned vlast = (unsigned)valid_of(m) - 1;
            auto seq_row = [&](unsigned r) { return (r < vlast ? r : vlast) * (unsigned)(D * LT::ES); };
            auto t_row = [](unsigned r) { return r * (unsigned)(C * LT::ES); };
            auto cf_row = [](unsigned) { return 0u; };
            if (lw == 0) {
                dma_tile<C, LT::PK>(buf + LT::K0, reinterpret_cast<const char*>(k + rb * D), seq_row, lane);
                dma_tile<C, LT::PK>(buf + LT::Q0, reinterpret_cast<const char*>(q + rb * D), seq_row, lane);
                dma_plain<1, LT::PC>(buf + LT::CF0, reinterpret_cast<const char*>(coef + tile * MDN_COEF_ROWS * C),
                                     cf_row, lane);
            } else {
                dma_tile<C, LT::PT>(buf + LT::TT0, reinterpret_cast<const char*>(TT + tile * C * C), t_row, lane);
                dma_tile<C, LT::PT>(buf + LT::AT0, reinterpret_cast<const char*>(AT + tile * C * C), t_row, lane);
                dma_plain<C, LT::PV>(buf + LT::O0, reinterpret_cast<const char*>(dO + rb * D + col0), seq_row, lane);
            }
        };
        const uint32_t aA = lds_addr(stA), aB = lds_addr(stB);
        if constexpr (NBUF == 2) {
            if (NT > 0) issue(aA, NT - 1);
            for (int64_t it = 0; it < NT; ++it) {
                __builtin_amdgcn_s_waitcnt(0);
                lds_barrier();
                if (it + 1 < NT) issue((it & 1) ? aA : aB, NT - 2 - it);
            }
        } else {
            for (int64_t it = 0; it < NT; ++it) {
                lds_barrier();                          // the chain waves are done with the buffer
                issue(aA, NT - 1 - it);
                __builtin_amdgcn_s_waitcnt(0);
                lds_barrier();                          // staged
            }
        }
        return;
    }

    const int ct = wave;
    const int col = col0 + 16 * ct + nn;
    const size_t sbase = (size_t)bh * D * D;
    floatx4 XS[NDH], XM[NDH];                          // dS, dM (rows perm(16t + 4g + e))
#pragma unroll
    for (int t = 0; t < NDH; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t off = sbase + (size_t)SL::perm(16 * t + 4 * g + e) * D + col;
            XS[t][e] = dST ? dST[off] : 0.f;
            XM[t][e] = dMT ? dMT[off] : 0.f;
        }
    auto crow = [&](const float* cf, int which, int tc) __attribute__((always_inline)) {
        return *reinterpret_cast<const floatx4*>(cf + which * C + SL::perm(16 * tc + 4 * g));
    };
    for (int64_t it = 0; it < NT; ++it) {
        const int64_t n = NT - 1 - it;
        if constexpr (NBUF == 1) lds_barrier();
        lds_barrier();
        const char* cur = (NBUF == 2 && (it & 1)) ? stB : stA;
        const char* Kl = cur + LT::K0;
        const char* Ql = cur + LT::Q0;
        const char* TTl = cur + LT::TT0;
        const char* ATl = cur + LT::AT0;
        const char* Ol = cur + LT::O0;
        const float* cf = reinterpret_cast<const float*>(cur + LT::CF0);
        const int vm = valid_of(n);
        const size_t tile = (size_t)bh * NT + n;

        // the chunk-end adjoints of chunk n
        {
            E* so = dSst + tile * D * D;
            E* mo = dMst + tile * D * D;
#pragma unroll
            for (int t = 0; t < NDH; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const size_t off = (size_t)SL::perm(16 * t + 4 * g + e) * D + col;
                    so[off] = Tr::from_f(XS[t][e]);
                    mo[off] = Tr::from_f(XM[t][e]);
                }
        }
        // dvt = Aqk^T dO + Diag(gS) K dS - Diag(gM) K dM
        floatx4 dV[NCT];
        {
            floatx4 KS[NCT], KM[NCT];
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) { KS[tc] = zero4(); KM[tc] = zero4(); dV[tc] = zero4(); }
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const frag sb = SL::from_acc(XS, ks), mb = SL::from_acc(XM, ks);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) {
                    const frag a = LdsA<Tr, LT::PK>::load(Kl, SL::perm(16 * tc + nn), ks, g);
                    KS[tc] = Tr::mma(a, sb, KS[tc]);
                    KM[tc] = Tr::mma(a, mb, KM[tc]);
                }
            }
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                const frag ob = ColOperand<Tr, OW>::load(Ol, ct, ks, lane);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc)
                    dV[tc] = Tr::mma(LdsA<Tr, LT::PT>::load(ATl, SL::perm(16 * tc + nn), ks, g), ob, dV[tc]);
            }
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) {
                const floatx4 gs = crow(cf, MDN_COEF_GS, tc), gm = crow(cf, MDN_COEF_GM, tc);
#pragma unroll
                for (int e = 0; e < 4; ++e) dV[tc][e] += gs[e] * KS[tc][e] - gm[e] * KM[tc][e];
            }
        }
        // dW = T^T dvt, which is dV of the chunk
        floatx4 dW[NCT];
        {
            frag vb[KSC];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) vb[ks] = SL::from_acc(dV, ks);
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc) {
                dW[tc] = zero4();
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks)
                    dW[tc] = Tr::mma(LdsA<Tr, LT::PT>::load(TTl, SL::perm(16 * tc + nn), ks, g), vb[ks], dW[tc]);
            }
        }
        {
            E* dst = dv + ((size_t)bh * T + n * C) * D + col;
#pragma unroll
            for (int tc = 0; tc < NCT; ++tc)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = SL::perm(16 * tc + 4 * g + e);
                    if (r < vm) dst[(size_t)r * D] = Tr::from_f(dW[tc][e]);
                }
        }
        // chunk-start adjoints
        const float abarC = cf[MDN_COEF_ABAR * C + C - 1];
        const float bC = cf[MDN_COEF_B * C + C - 1];
        const float mubarC = expf(cf[MDN_COEF_LM * C + C - 1]);
#pragma unroll
        for (int t = 0; t < NDH; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                XM[t][e] = mubarC * XM[t][e] - bC * XS[t][e];
                XS[t][e] = abarC * XS[t][e];
            }
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            float sa[NSL], sb[NSL], sab[NSL], nsa[NSL];
            SL::load_row(cf + MDN_COEF_ABAR * C, ks, g, sa);
            SL::load_row(cf + MDN_COEF_B * C, ks, g, sb);
            SL::load_row(cf + MDN_COEF_ABP * C, ks, g, sab);
#pragma unroll
            for (int j = 0; j < NSL; ++j) {
                nsa[j] = -sa[j];
                // the staged dO rows past the end repeat the last row: weight 0
                const bool in = SL::row(ks, g, j) < vm;
                sa[j] = in ? sa[j] : 0.f;
                sb[j] = in ? -sb[j] : 0.f;
            }
            const frag ob = ColOperand<Tr, OW>::load(Ol, ct, ks, lane);
            const frag dOa = FragScale<Tr>::apply(ob, sa), dOb = FragScale<Tr>::apply(ob, sb);
            const frag dWa = SL::from_acc_scaled(dW, ks, nsa), dWab = SL::from_acc_scaled(dW, ks, sab);
#pragma unroll
            for (int t = 0; t < NDH; ++t) {
                const frag qT = TrOperand<Tr, LT::PK>::load(Ql, t, ks, lane);
                const frag kT = TrOperand<Tr, LT::PK>::load(Kl, t, ks, lane);
                XS[t] = Tr::mma(qT, dOa, XS[t]);
                XS[t] = Tr::mma(kT, dWa, XS[t]);
                XM[t] = Tr::mma(qT, dOb, XM[t]);
                XM[t] = Tr::mma(kT, dWab, XM[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NDH; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t off = sbase + (size_t)SL::perm(16 * t + 4 * g + e) * D + col;
            dS0[off] = XS[t][e];
            dM0[off] = XM[t][e];
        }
}

// ---------------------------------------------------------------------------
// sgrad: the products with the states, one workgroup per chunk tile
//
// Wave w owns chunk rows 16w .. 16w+15 (natural order; its A operands come
// straight from global memory, zero past the end of a ragged chunk) and all
// dk columns.  For each state X of the chunk the B operand X^T is read from
// the workspace (rows of X are contiguous in the contraction index).  Row
// dots with q and k give the coefficient adjoints; the state inner products
// <S, dS'>, <M, dS'>, <M, dM'> are summed by the whole workgroup.
// ---------------------------------------------------------------------------
template <typename Tr, int D, int C>
__global__ __launch_bounds__(256)
void mdn_bwd_sgrad_kernel(const typename Tr::elem* __restrict__ q, const typename Tr::elem* __restrict__ k,
                          const typename Tr::elem* __restrict__ Vt, const typename Tr::elem* __restrict__ dO,
                          const typename Tr::elem* __restrict__ dW, const float* __restrict__ coef,
                          const typename Tr::elem* __restrict__ Sst, const typename Tr::elem* __restrict__ Mst,
                          const typename Tr::elem* __restrict__ dSst, const typename Tr::elem* __restrict__ dMst,
                          float* __restrict__ dqp, float* __restrict__ dkp, float* __restrict__ vec,
                          int64_t T, int64_t NT)
{
    using E = typename Tr::elem;
    using frag = typename Tr::frag;
    constexpr int NCT = C / 16, NDH = D / 16, KSD = D / Tr::KW;
    __shared__ float red[4][3];

    const int64_t tile = blockIdx.x;
    const int64_t bh = tile / NT, n = tile % NT;
    const int vm = (int)((T - n * C) < C ? (T - n * C) : C);
    const size_t rowbase = (size_t)(bh * T + n * C);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, nn = lane & 15;
    const E* S = Sst + tile * D * D;
    const E* M = Mst + tile * D * D;
    const E* dS = dSst + tile * D * D;
    const E* dM = dMst + tile * D * D;
    const float* cf = coef + tile * MDN_COEF_ROWS * C;
    float* vt = vec + tile * MDN_BWD_VEC_ROWS * C;

    // the state inner products (all threads)
    {
        constexpr int EPV = 16 / sizeof(E);
        float s0 = 0.f, s1 = 0.f, s2 = 0.f;
        for (int p = tid; p < D * D / EPV; p += 256) {
            union U { uint4 u; E e[EPV]; };
            U a, b, c, d;
            a.u = reinterpret_cast<const uint4*>(S)[p];
            b.u = reinterpret_cast<const uint4*>(M)[p];
            c.u = reinterpret_cast<const uint4*>(dS)[p];
            d.u = reinterpret_cast<const uint4*>(dM)[p];
#pragma unroll
            for (int j = 0; j < EPV; ++j) {
                const float xs = Tr::to_f(a.e[j]), xm = Tr::to_f(b.e[j]);
                const float ys = Tr::to_f(c.e[j]), ym = Tr::to_f(d.e[j]);
                s0 = fmaf(xs, ys, s0);
                s1 = fmaf(xm, ys, s1);
                s2 = fmaf(xm, ym, s2);
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            s0 += __shfl_xor(s0, m, 64);
            s1 += __shfl_xor(s1, m, 64);
            s2 += __shfl_xor(s2, m, 64);
        }
        if (lane == 0) { red[wave][0] = s0; red[wave][1] = s1; red[wave][2] = s2; }
    }
    __syncthreads();
    if (tid < 3) vt[5 * C + tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];

    if (wave >= NCT) return;
    const int rA = 16 * wave + nn;                    // A-operand row of this lane
    frag aO[KSD], aW[KSD], aV[KSD];
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
        if (rA < vm) {
            aO[ks] = Contig<Tr>::load(dO + (rowbase + rA) * D, ks, g);
            aW[ks] = Contig<Tr>::load(dW + (rowbase + rA) * D, ks, g);
            aV[ks] = Contig<Tr>::load(Vt + (rowbase + rA) * D, ks, g);
        } else {
            aO[ks] = Contig<Tr>::zero();
            aW[ks] = Contig<Tr>::zero();
            aV[ks] = Contig<Tr>::zero();
        }
    }
    const int r0 = 16 * wave + 4 * g;                 // accumulator rows r0 + e
    const floatx4 ca = *reinterpret_cast<const floatx4*>(cf + MDN_COEF_ABAR * C + r0);
    const floatx4 cb = *reinterpret_cast<const floatx4*>(cf + MDN_COEF_B * C + r0);
    const floatx4 cab = *reinterpret_cast<const floatx4*>(cf + MDN_COEF_ABP * C + r0);
    const floatx4 cgs = *reinterpret_cast<const floatx4*>(cf + MDN_COEF_GS * C + r0);
    const floatx4 cgm = *reinterpret_cast<const floatx4*>(cf + MDN_COEF_GM * C + r0);
    floatx4 dq[NDH], dk[NDH];
    float pa[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f}, pab[4] = {0.f, 0.f, 0.f, 0.f};
    float pgs[4] = {0.f, 0.f, 0.f, 0.f}, pgm[4] = {0.f, 0.f, 0.f, 0.f};
    auto qk_at = [&](const E* x, int e, int c) __attribute__((always_inline)) {
        return (r0 + e < vm) ? Tr::to_f(x[(rowbase + r0 + e) * D + c]) : 0.f;
    };
#pragma unroll
    for (int ct = 0; ct < NDH; ++ct) {
        const int c = 16 * ct + nn;
        floatx4 oS = zero4(), wS = zero4(), oM = zero4(), wM = zero4(), vS = zero4(), vM = zero4();
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            const frag bS = Contig<Tr>::load(S + (size_t)c * D, ks, g);
            const frag bM = Contig<Tr>::load(M + (size_t)c * D, ks, g);
            const frag bdS = Contig<Tr>::load(dS + (size_t)c * D, ks, g);
            const frag bdM = Contig<Tr>::load(dM + (size_t)c * D, ks, g);
            oS = Tr::mma(aO[ks], bS, oS);
            wS = Tr::mma(aW[ks], bS, wS);
            oM = Tr::mma(aO[ks], bM, oM);
            wM = Tr::mma(aW[ks], bM, wM);
            vS = Tr::mma(aV[ks], bdS, vS);
            vM = Tr::mma(aV[ks], bdM, vM);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dq[ct][e] = ca[e] * oS[e] - cb[e] * oM[e];
            dk[ct][e] = -ca[e] * wS[e] + cab[e] * wM[e] + cgs[e] * vS[e] - cgm[e] * vM[e];
            const float qv = qk_at(q, e, c), kv = qk_at(k, e, c);
            pa[e] += qv * oS[e] - kv * wS[e];
            pb[e] -= qv * oM[e];
            pab[e] += kv * wM[e];
            pgs[e] += kv * vS[e];
            pgm[e] -= kv * vM[e];
        }
    }
    float* qo = dqp + (tile * C + r0) * D;
    float* ko = dkp + (tile * C + r0) * D;
#pragma unroll
    for (int ct = 0; ct < NDH; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qo[e * D + 16 * ct + nn] = dq[ct][e];
            ko[e * D + 16 * ct + nn] = dk[ct][e];
        }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) {
            pa[e] += __shfl_xor(pa[e], m, 64);
            pb[e] += __shfl_xor(pb[e], m, 64);
            pab[e] += __shfl_xor(pab[e], m, 64);
            pgs[e] += __shfl_xor(pgs[e], m, 64);
            pgm[e] += __shfl_xor(pgm[e], m, 64);
        }
    }
    if (nn == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vt[0 * C + r0 + e] = pa[e];
            vt[1 * C + r0 + e] = pb[e];
            vt[2 * C + r0 + e] = pab[e];
            vt[3 * C + r0 + e] = pgs[e];
            vt[4 * C + r0 + e] = pgm[e];
        }
    }
}

// ---------------------------------------------------------------------------
// cgrad: the products inside the chunk and the gate gradients, one
// workgroup per chunk tile
//
// With E[r,j] = abar_r/abar_j (j <= r), F[j,i] = mubar_j/mubar_i (i <= j),
// Psi = E Diag(beta) F and Gamma = Psi Diag(eta), b = E (beta mubar):
//   X1 = (dO vtilde^T) o Gamma,  X2 = -(dW vtilde^T) o Gamma^-   (dA = -dW vtilde^T)
//   dq += X1 K;   dk += X1^T Q + (Diag(alpha) X2)^T K + Diag(alpha) X2 K
//   DGamma = (dO vtilde^T) o (Q K^T) + shift_up(dA o (P K^T)) + e_L DgS^T
//   dbeta_j = Z_j = sum_{r>=j,i<=j} E[r,j] (DGamma eta)[r,i] F[j,i] + mubar_j sum_{r>=j} E[r,j] Db_r
//   dLA_m = rowsum(DGamma Diag(eta) o Psi)_m + Db_m b_m - beta_m Z_m + Dabar_m abar_m
//   dLM_m = beta_m Z_m - eta_m colsum(DGamma o Psi)_m - DgM_m gM_m (+ the L terms)
//   deta_i = colsum(DGamma o Psi)_i + DgM_i F[L,i]
//   dalpha = revcumsum(dLA) / alpha + rowdot(K, X2 K) + Dab b_prev,  dmu = revcumsum(dLM) / mu
// (LA, LM the chunk's inclusive cumulative logs).  The C x C products over
// chunk rows run on the fp32 matrix cores with E and F formed on the fly
// from LA and LM (every exponent <= 0).
// ---------------------------------------------------------------------------
template <typename Tr, int D, int C>
struct CgradLayout {
    using E = typename Tr::elem;
    static constexpr int ES = sizeof(E);
    static constexpr int FS = C + 4;                  // fp32 C x C row stride (floats)
    static constexpr int XS = C + 16 / ES;            // element C x C row stride (elements)
    static constexpr int FB = C * FS * 4;
    static constexpr int XB = C * XS * ES;
    static constexpr int QT = C * D * ES;             // Q or K tile (plain rows of D)
    // fp32 C x C: QK -> DGamma, PK, dAqk, dA', Psi;  element C x C: X1, X1^T, X2, X2a^T
    static constexpr int F0 = 0, F1 = FB, F2 = 2 * FB, F3 = 3 * FB, F4 = 4 * FB;
    static constexpr int X0 = 5 * FB;
    static constexpr int Q0 = X0 + 4 * XB, K0 = Q0 + QT;
    static constexpr int V0 = K0 + QT;
    static constexpr int NV = 20;                     // vectors of C floats
    static constexpr int TOTAL = V0 + NV * C * 4;
};

template <typename Tr, int D, int C>
__global__ __launch_bounds__(256)
void mdn_bwd_cgrad_kernel(const typename Tr::elem* __restrict__ q, const typename Tr::elem* __restrict__ k,
                          const float* __restrict__ alpha, const float* __restrict__ mu,
                          const float* __restrict__ beta, const float* __restrict__ eta,
                          const typename Tr::elem* __restrict__ Vt, const typename Tr::elem* __restrict__ dO,
                          const typename Tr::elem* __restrict__ dW, const float* __restrict__ coef,
                          const float* __restrict__ dqp, const float* __restrict__ dkp,
                          const float* __restrict__ vec, typename Tr::elem* __restrict__ dq,
                          typename Tr::elem* __restrict__ dk, float* __restrict__ dalpha,
                          float* __restrict__ dmu, float* __restrict__ dbeta, float* __restrict__ deta,
                          int64_t T, int64_t NT)
{
    using E = typename Tr::elem;
    using frag = typename Tr::frag;
    using L = CgradLayout<Tr, D, C>;
    using F32 = TraitsF32;
    constexpr int NCT = C / 16, NDH = D / 16, KSD = D / Tr::KW, KSC = C / Tr::KW, FS = L::FS, XS = L::XS;
    __shared__ __attribute__((aligned(16))) char lds[L::TOTAL];
    float* fQK = reinterpret_cast<float*>(lds + L::F0);     // Q K^T, then DGamma
    float* fPK = reinterpret_cast<float*>(lds + L::F1);     // P K^T
    float* fAq = reinterpret_cast<float*>(lds + L::F2);     // dO vtilde^T
    float* fAw = reinterpret_cast<float*>(lds + L::F3);     // dW vtilde^T
    float* fPs = reinterpret_cast<float*>(lds + L::F4);     // Psi
    E* x1 = reinterpret_cast<E*>(lds + L::X0);
    E* x1t = reinterpret_cast<E*>(lds + L::X0 + L::XB);
    E* x2 = reinterpret_cast<E*>(lds + L::X0 + 2 * L::XB);
    E* x2t = reinterpret_cast<E*>(lds + L::X0 + 3 * L::XB);
    E* Ql = reinterpret_cast<E*>(lds + L::Q0);
    E* Kl = reinterpret_cast<E*>(lds + L::K0);
    float* vv = reinterpret_cast<float*>(lds + L::V0);
    float* sLA = vv + 0 * C; float* sLM = vv + 1 * C; float* sAl = vv + 2 * C; float* sMu = vv + 3 * C;
    float* sBe = vv + 4 * C; float* sEt = vv + 5 * C; float* sAb = vv + 6 * C; float* sB = vv + 7 * C;
    float* sGM = vv + 8 * C; float* sDa = vv + 9 * C; float* sDb = vv + 10 * C; float* sDab = vv + 11 * C;
    float* sDgM = vv + 12 * C; float* sDgS = vv + 13 * C; float* sZ = vv + 14 * C; float* sAd = vv + 15 * C;
    float* sMisc = vv + 16 * C;

    const int64_t tile = blockIdx.x;
    const int64_t bh = tile / NT, n = tile % NT;
    const int vm = (int)((T - n * C) < C ? (T - n * C) : C);
    const size_t rowbase = (size_t)(bh * T + n * C);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, nn = lane & 15;
    const float* cf = coef + tile * MDN_COEF_ROWS * C;
    const float* vt = vec + tile * MDN_BWD_VEC_ROWS * C;
    constexpr int LR = C - 1;

    // ---- 1. Q, K tiles and the row vectors -----------------------------------
    {
        constexpr int EPV = 16 / L::ES, PR = D / EPV;
        for (int p = tid; p < C * PR; p += 256) {
            const int r = p / PR, c = p % PR;
            uint4 a = uint4{0u, 0u, 0u, 0u}, b = a;
            if (r < vm) {
                a = reinterpret_cast<const uint4*>(q + (rowbase + r) * D)[c];
                b = reinterpret_cast<const uint4*>(k + (rowbase + r) * D)[c];
            }
            reinterpret_cast<uint4*>(Ql)[p] = a;
            reinterpret_cast<uint4*>(Kl)[p] = b;
        }
        if (tid < C) {
            const int r = tid;
            const bool in = r < vm;
            sLA[r] = cf[MDN_COEF_LA * C + r];
            sLM[r] = cf[MDN_COEF_LM * C + r];
            sAl[r] = in ? alpha[rowbase + r] : 1.f;
            sMu[r] = in ? mu[rowbase + r] : 1.f;
            sBe[r] = in ? beta[rowbase + r] : 0.f;
            sEt[r] = in ? eta[rowbase + r] : 0.f;
            sAb[r] = cf[MDN_COEF_ABAR * C + r];
            sB[r] = cf[MDN_COEF_B * C + r];
            sGM[r] = cf[MDN_COEF_GM * C + r];
            sDa[r] = vt[0 * C + r];
            sDab[r] = vt[2 * C + r];
            sDgS[r] = vt[3 * C + r];
            sDgM[r] = vt[4 * C + r];
            sAd[r] = 0.f;
        }
        if (tid < 3) sMisc[tid] = vt[5 * C + tid];    // <S,dS'>, <M,dS'>, <M,dM'>
    }
    __syncthreads();
    if (tid < C) {
        // Db_r: its own row dot, -<M,dS'> at the last row, and the b_{r-1} of ab_{r+1}
        const int r = tid;
        float db = vt[1 * C + r];
        if (r == LR) db -= sMisc[1];
        if (r + 1 < C) db += sDab[r + 1] * sAl[r + 1];
        sDb[r] = db;
        if (r == LR) sDa[r] += sMisc[0];
    }

    // ---- 2. Q K^T, K K^T, dO vtilde^T, dW vtilde^T (row block = wave) -----------
    if (wave < NCT) {
        const int rA = 16 * wave + nn;
        frag aQ[KSD], aK[KSD], aO[KSD], aW[KSD];
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            aQ[ks] = Contig<Tr>::load(Ql + rA * D, ks, g);
            aK[ks] = Contig<Tr>::load(Kl + rA * D, ks, g);
            if (rA < vm) {
                aO[ks] = Contig<Tr>::load(dO + (rowbase + rA) * D, ks, g);
                aW[ks] = Contig<Tr>::load(dW + (rowbase + rA) * D, ks, g);
            } else {
                aO[ks] = Contig<Tr>::zero();
                aW[ks] = Contig<Tr>::zero();
            }
        }
        const int r0 = 16 * wave + 4 * g;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            floatx4 aqk = zero4(), akk = zero4(), ao = zero4(), aw = zero4();
            if (ct <= wave) {
                const int cB = 16 * ct + nn;
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    const frag bK = Contig<Tr>::load(Kl + cB * D, ks, g);
                    const frag bV = (cB < vm) ? Contig<Tr>::load(Vt + (rowbase + cB) * D, ks, g) : Contig<Tr>::zero();
                    aqk = Tr::mma(aQ[ks], bK, aqk);
                    akk = Tr::mma(aK[ks], bK, akk);
                    ao = Tr::mma(aO[ks], bV, ao);
                    aw = Tr::mma(aW[ks], bV, aw);
                }
            }
            const int i = 16 * ct + nn;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = r0 + e;
                fQK[r * FS + i] = aqk[e];
                fPK[r * FS + i] = sAl[r] * akk[e];
                fAq[r * FS + i] = ao[e];
                fAw[r * FS + i] = aw[e];
            }
        }
    }
    // ---- 3. Psi = E Diag(beta) F on the fp32 matrix cores ----------------------
    if (wave < NCT) {
        const int rA = 16 * wave + nn, r0 = 16 * wave + 4 * g;
        const float laA = sLA[rA];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            floatx4 acc = zero4();
            if (ct <= wave) {
                const int i = 16 * ct + nn;
                const float lmi = sLM[i];
                for (int ks = 4 * ct; ks < 4 * wave + 4; ++ks) {
                    const int j = 4 * ks + g;
                    const float a = (j <= rA) ? expf(laA - sLA[j]) : 0.f;
                    const float b = (i <= j) ? sBe[j] * expf(sLM[j] - lmi) : 0.f;
                    acc = F32::mma(a, b, acc);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) fPs[(r0 + e) * FS + 16 * ct + nn] = acc[e];
        }
    }
    __syncthreads();

    // ---- 4. X1, X2 and DGamma (values first, then the stores) -----------------
    {
        constexpr int PER = C * C / 256 > 0 ? C * C / 256 : 1;
        float vX1[PER], vX2[PER], vDG[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int idx = tid + 256 * m;
            vX1[m] = vX2[m] = vDG[m] = 0.f;
            if (idx < C * C) {
                const int r = idx / C, i = idx % C;
                const float et = sEt[i];
                if (i <= r) {
                    const float gam = fPs[r * FS + i] * et;
                    vX1[m] = fAq[r * FS + i] * gam;
                    float dg = fAq[r * FS + i] * fQK[r * FS + i];
                    if (r + 1 < C) dg -= fAw[(r + 1) * FS + i] * fPK[(r + 1) * FS + i];
                    if (r == LR) dg += sDgS[i];
                    vDG[m] = dg;
                }
                if (i < r) vX2[m] = -fAw[r * FS + i] * fPs[(r - 1) * FS + i] * et;
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int idx = tid + 256 * m;
            if (idx < C * C) {
                const int r = idx / C, i = idx % C;
                fQK[r * FS + i] = vDG[m];
                x1[r * XS + i] = Tr::from_f(vX1[m]);
                x1t[i * XS + r] = Tr::from_f(vX1[m]);
                x2[r * XS + i] = Tr::from_f(vX2[m]);
                x2t[i * XS + r] = Tr::from_f(vX2[m] * sAl[r]);
            }
        }
    }
    __syncthreads();
    float* fDG = fQK;

    // ---- 5. Z: G = E^T (DGamma Diag(eta)) on the fp32 matrix cores, G o F row sums
    if (wave < NCT) {
        const int mA = 16 * wave + nn, m0 = 16 * wave + 4 * g;
        const float laA = sLA[mA];
        float zp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            if (ct > wave) continue;
            const int i = 16 * ct + nn;
            const float et = sEt[i], lmi = sLM[i];
            floatx4 acc = zero4();
            for (int ks = 4 * wave; ks < C / 4; ++ks) {
                const int r = 4 * ks + g;
                const float a = (r >= mA) ? expf(sLA[r] - laA) : 0.f;
                acc = F32::mma(a, fDG[r * FS + i] * et, acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + e;
                zp[e] += (i <= m) ? acc[e] * expf(sLM[m] - lmi) : 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int s = 8; s >= 1; s >>= 1) zp[e] += __shfl_xor(zp[e], s, 64);
            if (nn == 0) sZ[m0 + e] = zp[e];
        }
    }

    // ---- 6. dq, dk: X1 K, X1^T Q + (Diag(alpha) X2)^T K + Diag(alpha) X2 K ------
    if (wave < NCT) {
        const int rA = 16 * wave + nn, r0 = 16 * wave + 4 * g;
        frag a1[KSC], a1t[KSC], a2[KSC], a2t[KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            a1[ks] = SlotRow<Tr>::load(x1 + rA * XS, ks, g);
            a1t[ks] = SlotRow<Tr>::load(x1t + rA * XS, ks, g);
            a2[ks] = SlotRow<Tr>::load(x2 + rA * XS, ks, g);
            a2t[ks] = SlotRow<Tr>::load(x2t + rA * XS, ks, g);
        }
        const char* Qc = reinterpret_cast<const char*>(Ql);
        const char* Kc = reinterpret_cast<const char*>(Kl);
        float pad[4] = {0.f, 0.f, 0.f, 0.f};
        const float* qp = dqp + (tile * C + r0) * D;
        const float* kp = dkp + (tile * C + r0) * D;
#pragma unroll
        for (int ct = 0; ct < NDH; ++ct) {
            floatx4 aq = zero4(), ak = zero4(), x2k = zero4();
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                const frag bK = ColOperand<Tr, D>::load(Kc, ct, ks, lane);
                const frag bQ = ColOperand<Tr, D>::load(Qc, ct, ks, lane);
                aq = Tr::mma(a1[ks], bK, aq);
                ak = Tr::mma(a1t[ks], bQ, ak);
                ak = Tr::mma(a2t[ks], bK, ak);
                x2k = Tr::mma(a2[ks], bK, x2k);
            }
            const int c = 16 * ct + nn;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = r0 + e;
                const float kv = Tr::to_f(Kl[r * D + c]);
                pad[e] += kv * x2k[e];
                const float vq = aq[e] + qp[e * D + c];
                const float vk = ak[e] + sAl[r] * x2k[e] + kp[e * D + c];
                if (r < vm) {
                    dq[(rowbase + r) * D + c] = Tr::from_f(vq);
                    dk[(rowbase + r) * D + c] = Tr::from_f(vk);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int s = 8; s >= 1; s >>= 1) pad[e] += __shfl_xor(pad[e], s, 64);
            if (nn == 0) sAd[r0 + e] = pad[e];
        }
    }
    __syncthreads();

    // ---- 7. the gate gradients ------------------------------------------------
    // row sums of DGamma Diag(eta) o Psi (threads 0..C-1), column sums of
    // DGamma o Psi (threads 64..64+C-1), the b part of Z (threads 128..)
    if (tid < C) {
        const int m = tid;
        float s = 0.f;
        for (int i = 0; i <= m; ++i) s += fDG[m * FS + i] * sEt[i] * fPs[m * FS + i];
        sMisc[8 + m] = s;
    } else if (tid >= 64 && tid < 64 + C) {
        const int i = tid - 64;
        float s = 0.f;
        for (int r = i; r < C; ++r) s += fDG[r * FS + i] * fPs[r * FS + i];
        sMisc[8 + C + i] = s;
    } else if (tid >= 128 && tid < 128 + C) {
        const int m = tid - 128;
        float s = 0.f;
        for (int r = m; r < C; ++r) s += expf(sLA[r] - sLA[m]) * sDb[r];
        sMisc[8 + 2 * C + m] = s * expf(sLM[m]);
    }
    __syncthreads();
    if (wave == 0) {
        const int m = lane;
        const bool in = m < C;
        float dla = 0.f, dlm = 0.f, z = 0.f, de = 0.f;
        float tail = 0.f;
        if (in) {
            z = sZ[m] + sMisc[8 + 2 * C + m];
            const float cs = sMisc[8 + C + m];
            const float gmL = expf(sLM[LR] - sLM[m]);
            de = cs + sDgM[m] * gmL;
            dla = sMisc[8 + m] + sDb[m] * sB[m] - sBe[m] * z + sDa[m] * sAb[m];
            dlm = sBe[m] * z - sEt[m] * cs - sDgM[m] * sGM[m];
            tail = sDgM[m] * sGM[m];
        }
        // the last row's terms: sum_i DgM_i gM_i + Dmubar_L mubar_L
        float tsum = tail;
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) tsum += __shfl_xor(tsum, s, 64);
        if (m == LR) dlm += tsum + sMisc[2] * expf(sLM[LR]);
        // suffix sums over rows: total - inclusive prefix + own
        const float pla = wave_scan_add(dla), plm = wave_scan_add(dlm);
        const float tla = __shfl(pla, 63, 64), tlm = __shfl(plm, 63, 64);
        const float sla = tla - pla + dla, slm = tlm - plm + dlm;
        if (in && m < vm) {
            const float bprev = m > 0 ? sB[m - 1] : 0.f;
            const size_t gi = rowbase + m;
            dalpha[gi] = sla / sAl[m] + sAd[m] + sDab[m] * bprev;
            dmu[gi] = slm / sMu[m];
            dbeta[gi] = z;
            deta[gi] = de;
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename Tr, int D, int C>
static hipError_t launch_bwd_t(const BwdArgs& a)
{
    using E = typename Tr::elem;
    const ChunkArgs& f = a.f;
    constexpr int NCOL = D >= 32 ? 2 : 1;
    const int64_t grid = f.BH * (D / (16 * NCOL));
    hipLaunchKernelGGL((mdn_bwd_replay_kernel<Tr, D, C, NCOL>), dim3((unsigned)grid), dim3(64 * (NCOL + 2)), 0,
                       (hipStream_t)f.stream, (const E*)f.k, (const E*)a.Vt, f.coef, f.S0, f.M0,
                       (E*)a.Sst, (E*)a.Mst, f.T, f.NT, (int)f.BH);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    using CP = CarryPick<Tr, D, C>;
    hipLaunchKernelGGL((mdn_bwd_carry_kernel<Tr, D, C, CP::NCOL, CP::NBUF>), dim3((unsigned)grid),
                       dim3(64 * (CP::NCOL + 2)), 0, (hipStream_t)f.stream, (const E*)f.q, (const E*)f.k,
                       (const E*)f.Tmat, (const E*)f.Aqk, f.coef, (const E*)a.dO, a.dST, a.dMT, (E*)a.dv,
                       (E*)a.dSst, (E*)a.dMst, a.dS0, a.dM0, f.T, f.NT, (int)f.BH);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t tiles = f.BH * f.NT;
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL((mdn_bwd_sgrad_kernel<Tr, D, C>), dim3((unsigned)tiles), dim3(256), 0, (hipStream_t)f.stream,
                       (const E*)f.q, (const E*)f.k, (const E*)a.Vt, (const E*)a.dO, (const E*)a.dv, f.coef,
                       (const E*)a.Sst, (const E*)a.Mst, (const E*)a.dSst, (const E*)a.dMst, a.dqp, a.dkp, a.vec,
                       f.T, f.NT);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    static_assert(CgradLayout<Tr, D, C>::TOTAL <= 160 * 1024 - 1024, "LDS");
    hipLaunchKernelGGL((mdn_bwd_cgrad_kernel<Tr, D, C>), dim3((unsigned)tiles), dim3(256), 0, (hipStream_t)f.stream,
                       (const E*)f.q, (const E*)f.k, f.alpha, f.mu, f.beta, f.eta, (const E*)a.Vt, (const E*)a.dO,
                       (const E*)a.dv, f.coef, a.dqp, a.dkp, a.vec, (E*)a.dq, (E*)a.dk, a.dalpha, a.dmu, a.dbeta,
                       a.deta, f.T, f.NT);
    return hipGetLastError();
}

template <typename Tr>
static hipError_t bwd_dispatch(const BwdArgs& a)
{
    if constexpr (std::is_same<Tr, TraitsBf16>::value) {
        switch (a.f.dk * 1000 + a.f.C) {
        case 32032: return launch_bwd_t<Tr, 32, 32>(a);
        case 32064: return launch_bwd_t<Tr, 32, 64>(a);
        case 64032: return launch_bwd_t<Tr, 64, 32>(a);
        case 64064: return launch_bwd_t<Tr, 64, 64>(a);
        case 128032: return launch_bwd_t<Tr, 128, 32>(a);
        case 128064: return launch_bwd_t<Tr, 128, 64>(a);
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (a.f.dk * 1000 + a.f.C) {
        case 16016: return launch_bwd_t<Tr, 16, 16>(a);
        case 16032: return launch_bwd_t<Tr, 16, 32>(a);
        case 32016: return launch_bwd_t<Tr, 32, 16>(a);
        case 32032: return launch_bwd_t<Tr, 32, 32>(a);
        case 64016: return launch_bwd_t<Tr, 64, 16>(a);
        case 64032: return launch_bwd_t<Tr, 64, 32>(a);
        default: return hipErrorInvalidValue;
        }
    }
}

hipError_t launch_bwd(const BwdArgs& a)
{
    if (a.f.BH == 0) return hipSuccess;
    if (a.f.T > 0) {
        hipError_t e = launch_chunk_intra(a.f);
        if (e != hipSuccess) return e;
    }
    return a.f.dtype == MDN_BF16 ? bwd_dispatch<TraitsBf16>(a) : bwd_dispatch<TraitsF32>(a);
}

}  // namespace mdn
