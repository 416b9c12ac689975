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

// Whether row tile t of an upper-triangular C x C matrix (T^T, Aqk^T), read
// as a matrix-core A operand, can be nonzero in contraction step ks.  bf16:
// step ks covers columns 32ks .. 32ks + 31 and the rows perm(16t + x) of tile
// t all lie in the 32-row half t/2; fp32: step ks covers the columns
// 16(ks/4) + ks%4 + 4g and tile t holds rows 16t .. 16t + 15.
template <typename Tr>
constexpr bool upper_step(int t, int ks)
{
    return std::is_same<Tr, TraitsBf16>::value ? ks >= (t >> 1) : (ks >> 2) >= t;
}

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

// Sum over the 16 lanes of a row (lanes 16g .. 16g+15) on DPP row shifts:
// lane 16g + 15 ends with the row's sum.
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp_move<DPP_ROW_SHR1>(x, 0.f);
    x += dpp_move<DPP_ROW_SHR2>(x, 0.f);
    x += dpp_move<DPP_ROW_SHR4>(x, 0.f);
    x += dpp_move<DPP_ROW_SHR8>(x, 0.f);
    return x;
}

// A chain wave's 16-column slice of a D x D state (accumulator tiles t,
// rows perm(16t + 4g + e), column nn) to rows of a row-major [D][D] array,
// through an LDS tile so that every global store is 16 bytes.
template <typename Tr, int D>
__device__ __forceinline__ void store_slice(const floatx4 (&X)[D / 16], typename Tr::elem* __restrict__ lt,
                                            typename Tr::elem* __restrict__ dst, int lane)
{
    using E = typename Tr::elem;
    using SL = Slots<Tr>;
    constexpr int EPV = 16 / sizeof(E), PPR = 16 / EPV, NP = D * PPR;
    const int g = lane >> 4, nn = lane & 15;
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) lt[SL::perm(16 * t + 4 * g + e) * 16 + nn] = Tr::from_f(X[t][e]);
#pragma unroll
    for (int i = 0; i < (NP + 63) / 64; ++i) {
        const int p = i * 64 + lane;
        if (NP % 64 == 0 || p < NP) {
            const int r = p / PPR, c = (p % PPR) * EPV;
            *reinterpret_cast<uint4*>(dst + (size_t)r * D + c) = reinterpret_cast<const uint4*>(lt)[p];
        }
    }
}

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

// Hand-off of a chain wave's 16-column slice of an R-row matrix (accumulator
// tiles t, rows perm(16t + 4g + e), column nn) to the loader waves through an
// LDS tile: the chain wave only writes it, and after the next barrier the
// loader waves copy it to its row-major destination.
//   bf16: the tile is column-major with column stride RS = R + 4, so a lane's
//   four rows (consecutive in the slot order) are one 8-byte write.  The
//   copy reads it back with the LDS transpose read: a lane group addresses a
//   4-column x 16-row block and each lane receives one row's 4 columns,
//   which is an 8-byte piece of the destination row.
//   fp32: the tile is row-major with row stride 20, so the four rows a lane
//   group writes per instruction (4 apart in the fp32 slot order) start 16
//   banks apart; the copy moves 8-byte pieces.
template <typename Tr, int R> struct HandTile;
template <int R> struct HandTile<TraitsBf16, R> {
    static constexpr int RS = R + 4;
    static constexpr int BYTES = 16 * RS * 2;
    // tiles t0 .. t0 + NX - 1 of the slice (all of it by default)
    template <int NX>
    static __device__ __forceinline__ void write(const floatx4 (&X)[NX], __bf16* __restrict__ lt, int lane, int t0 = 0) {
        const int g = lane >> 4, nn = lane & 15;
#pragma unroll
        for (int t = 0; t < NX; ++t) {
            const int r = Slots<TraitsBf16>::perm(16 * (t0 + t) + 4 * g);
            union { __bf16 h[4]; uint2 u; } v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v.h[e] = (__bf16)X[t][e];
            *reinterpret_cast<uint2*>(lt + nn * RS + r) = v.u;
        }
    }
    // the whole tile to dst (row stride ld) by the NW waves of threads
    // tid < 64 NW; rows >= nrows are not stored
    template <int NW>
    static __device__ __forceinline__ void copy(const char* lt, __bf16* __restrict__ dst, int ld, int nrows, int tid) {
        const int lane = tid & 63, gq = lane >> 4, s = lane & 15;
#pragma unroll
        for (int i = 0; i < (R / 16 + NW - 1) / NW; ++i) {
            const int rb = i * NW + (tid >> 6);
            if (rb < R / 16) {
                const int c = 4 * gq + (s >> 2), r = 16 * rb + 4 * (s & 3);
                const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) shortx4*)(lt + (c * RS + r) * 2));
                const int row = 16 * rb + s;
                if (row < nrows) *reinterpret_cast<shortx4*>(dst + (size_t)row * ld + 4 * gq) = v;
            }
        }
    }
};
template <int R> struct HandTile<TraitsF32, R> {
    static constexpr int SS = 20;
    static constexpr int BYTES = R * SS * 4;
    template <int NX>
    static __device__ __forceinline__ void write(const floatx4 (&X)[NX], float* __restrict__ lt, int lane, int t0 = 0) {
        const int g = lane >> 4, nn = lane & 15;
#pragma unroll
        for (int t = 0; t < NX; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) lt[Slots<TraitsF32>::perm(16 * (t0 + t) + 4 * g + e) * SS + nn] = X[t][e];
    }
    template <int NW>
    static __device__ __forceinline__ void copy(const char* lt, float* __restrict__ dst, int ld, int nrows, int tid) {
        for (int p = tid; p < R * 8; p += 64 * NW) {
            const int r = p >> 3, c = 2 * (p & 7);
            if (r < nrows)
                *reinterpret_cast<uint2*>(dst + (size_t)r * ld + c) =
                    *reinterpret_cast<const uint2*>(lt + (r * SS + c) * 4);
        }
    }
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
__global__ __launch_bounds__(64 * (NCOL + 4))
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
    __shared__ __attribute__((aligned(16))) E stg[NCOL][2][D * 16];   // state slices on their way out

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
            // four loaders: K by rows, the vtilde slab and the coefficients
            constexpr int RPL = C / 4;
            dma_tile<RPL, LT::PK>(buf + LT::K0, reinterpret_cast<const char*>(k + rb * D), seq_row, lane, lw * RPL);
            if (lw == 0)
                dma_plain<C, LT::PV>(buf + LT::V0, reinterpret_cast<const char*>(Vt + rb * D + col0), seq_row, lane);
            else if (lw == 1)
                dma_plain<1, LT::PC>(buf + LT::CF0, reinterpret_cast<const char*>(coef + tile * MDN_COEF_ROWS * C),
                                     cf_row, lane);
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
        {
            const size_t off = ((size_t)bh * NT + n) * D * D + col0 + 16 * ct;
            store_slice<Tr, D>(XS, stg[ct][0], Sst + off, lane);
            store_slice<Tr, D>(XM, stg[ct][1], Mst + off, lane);
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
//
// One workgroup per (head, slab of 16 NCOL state columns), backward over the
// chunks: NCOL chain waves carry dS and dM of their 16 columns in registers,
// four loader waves stage each chunk's K, Q, T^T, Aqk^T, dO slab and
// coefficient rows.  Each chunk's dS', dM' slices and dV rows leave the chain
// waves as LDS writes into hand-off tiles; two of the loader waves copy them
// to HBM after the next barrier, and the other two stage (where the LDS
// budget has no room for the hand-off tiles, the chain waves store them
// through staging tiles themselves and all four loaders stage).
//
// Row split (RS = 2, where the LDS has room for it): each column tile has two
// chain waves, h = 0 and 1, holding dk rows [h D/2, (h+1) D/2) of dS and dM.
// Per chunk, wave h forms the part of K dS', K dM' over its own rows; wave 1
// adds Aqk^T dO to its part and hands it to wave 0 through an LDS exchange
// tile; wave 0 completes dvt and dW = T^T dvt and hands dW back through the
// same tile.  Meanwhile both scale their rows to the chunk start and add the
// products with dO, which need no dW; the products with dW follow.  Each
// wave's in-order share per chunk drops from about 112 to about 60 matrix-core
// products.  The two hand-offs are ordered by counters in LDS (release after
// the tile is written, acquire before it is read), not by workgroup barriers,
// so the loader waves and the other column tile never wait for them.
// ---------------------------------------------------------------------------

// Release and acquire of a per-chunk counter in LDS between two waves of one
// workgroup.  The wait is bounded (about 2^22 polls, tens of milliseconds):
// a handshake that never completes ends the kernel with wrong values instead
// of hanging it.
__device__ __forceinline__ void pair_release(int* f, int v)
{
    __hip_atomic_store(f, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void pair_wait(int* f, int v)
{
    for (int i = 0; i < (1 << 22); ++i) {
        if (__hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= v) return;
        __builtin_amdgcn_s_sleep(1);
    }
}

template <typename Tr, int D, int C, int NCOL, int NBUF, int RS = 1>
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
    static constexpr int SR = D > C ? D : C;          // staging rows: adjoint slices and dV rows
    static constexpr int STG = NCOL * 2 * SR * 16 * ES;
    // with two stage buffers and room to spare, the adjoint slices and the dV
    // rows go to the loaders instead: per parity and column tile a dS' and a
    // dM' slice tile, then C x 16 dV rows
    static constexpr int SLB = HandTile<Tr, D>::BYTES, DVB = HandTile<Tr, C>::BYTES, CTB = 2 * SLB + DVB;
    static constexpr int PAR = NCOL * CTB, HAND = 2 * PAR;
    // row split: per column tile one C x 16 fp32 exchange tile (4 values per
    // lane and row tile)
    static constexpr int XB = RS > 1 ? NCOL * (C / 16) * 64 * 16 : 0;
    static constexpr bool OFF = NBUF == 2 && 2 * BUF + HAND + XB <= 160 * 1024 - 1024;
    static constexpr int TOTAL = NBUF * BUF + (OFF ? HAND : STG) + XB;
};

template <typename Tr, int D, int C>
struct CarryPick {
    static constexpr int LIMIT = 160 * 1024 - 1024;
    static constexpr int NCOL = D >= 32 ? 2 : 1;
    // the row split only with double-buffered staging and the hand-off tiles
    static constexpr int RS = (D >= 64 && CarryLayout<Tr, D, C, NCOL, 2, 2>::OFF) ? 2 : 1;
    static constexpr int NBUF = CarryLayout<Tr, D, C, NCOL, 2, RS>::TOTAL <= LIMIT ? 2 : 1;
    static_assert(CarryLayout<Tr, D, C, NCOL, NBUF, RS>::TOTAL <= LIMIT, "LDS");
    static_assert(RS == 1 || (NBUF == 2 && CarryLayout<Tr, D, C, NCOL, NBUF, RS>::OFF), "row split layout");
    // loader waves, of which NST stage (with the hand-off tiles) and the rest
    // copy the hand-off tiles out.  The split chain is short enough that two
    // staging waves (their copies in flight bound the bytes per chunk) and
    // two copying waves would set the pace; with four of each, twelve waves,
    // the chain does again.
    static constexpr int NLD = RS > 1 ? 8 : 4;
    static constexpr int NST = RS > 1 ? 4 : 2;
};

template <typename Tr, int D, int C, int NCOL, int NBUF, int RS, int NLD, int NST>
__global__ __launch_bounds__(64 * (NCOL * RS + NLD))
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
    using LT = CarryLayout<Tr, D, C, NCOL, NBUF, RS>;
    using frag = typename Tr::frag;
    constexpr int NSL = SL::NSLOT, KSC = C / Tr::KW, KSD = D / Tr::KW, NCT = C / 16, NDH = D / 16;
    constexpr int SLABS = D / (16 * NCOL), OW = 16 * NCOL;
    constexpr int NW = NCOL * RS;                      // chain waves
    constexpr int NDL = NDH / RS, KSH = KSD / RS;      // a chain wave's d tiles and contraction steps over d
    static_assert(NDH % RS == 0 && KSD % RS == 0, "row split");
    __shared__ __attribute__((aligned(16))) char stA[LT::BUF];
    __shared__ __attribute__((aligned(16))) char stB[NBUF == 2 ? LT::BUF : 16];
    constexpr bool OFF = LT::OFF;
    constexpr int NDMA = OFF ? NST : NLD;              // staging loader waves
    // adjoint slices and dV rows on their way out (hand-off tiles, or per
    // column tile two staging tiles of the chain wave)
    __shared__ __attribute__((aligned(16))) char stg[OFF ? LT::HAND : LT::STG];
    // row split: the exchange tiles and, per column tile, the counters of the
    // two hand-offs (partial dvt to wave 0, dW to wave 1)
    __shared__ __attribute__((aligned(16))) floatx4 xb[RS > 1 ? NCOL * NCT * 64 : 1];
    __shared__ int xflag[RS > 1 ? 2 * NCOL : 1];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, nn = lane & 15;
    int bh, slab;
    xcd_head_map(blockIdx.x, SLABS, BH, bh, slab);
    const int col0 = slab * OW;
    auto valid_of = [&](int64_t n) { return (int)((T - n * C) < C ? (T - n * C) : C); };

    if (wave >= NW) {
        const int lw = wave - NW;
        // iteration it handles chunk NT - 1 - it
        auto issue = [&](uint32_t buf, int64_t m) __attribute__((always_inline)) {
            const size_t rb = (size_t)bh * T + m * C, tile = (size_t)bh * NT + m;
            const unsigned vlast = (unsigned)valid_of(m) - 1;
            auto seq_row = [&](unsigned r) { return (r < vlast ? r : vlast) * (unsigned)(D * LT::ES); };
            auto t_row = [](unsigned r) { return r * (unsigned)(C * LT::ES); };
            auto cf_row = [](unsigned) { return 0u; };
            // the staging loaders: K, Q, T^T and Aqk^T by rows; the dO slab; the
            // coefficients
            constexpr int RPL = C / NDMA;
            const int r0 = lw * RPL;
            dma_tile<RPL, LT::PK>(buf + LT::K0, reinterpret_cast<const char*>(k + rb * D), seq_row, lane, r0);
            dma_tile<RPL, LT::PK>(buf + LT::Q0, reinterpret_cast<const char*>(q + rb * D), seq_row, lane, r0);
            // whole rows, the quadrant the intra stage leaves unwritten
            // included (no product reads it; leaving it out of the copies
            // measured slower here, 876 against 865 us for the whole call)
            dma_tile<RPL, LT::PT>(buf + LT::TT0, reinterpret_cast<const char*>(TT + tile * C * C), t_row, lane, r0);
            dma_tile<RPL, LT::PT>(buf + LT::AT0, reinterpret_cast<const char*>(AT + tile * C * C), t_row, lane, r0);
            if (lw == NDMA - 2)
                dma_plain<C, LT::PV>(buf + LT::O0, reinterpret_cast<const char*>(dO + rb * D + col0), seq_row, lane);
            else if (lw == NDMA - 1)
                dma_plain<1, LT::PC>(buf + LT::CF0, reinterpret_cast<const char*>(coef + tile * MDN_COEF_ROWS * C),
                                     cf_row, lane);
        };
        // what the chain waves handed over in iteration j (chunk NT - 1 - j):
        // the dS', dM' slices to dSst, dMst and the dV rows to dv
        auto flush = [&](int64_t j) __attribute__((always_inline)) {
            const int64_t m = NT - 1 - j;
            const char* hb = stg + (j & 1) * LT::PAR;
            const size_t off = ((size_t)bh * NT + m) * D * D + col0;
            constexpr int NCP = NLD - NDMA;             // copying waves
            const int ft = (lw - NDMA) * 64 + lane, vm = valid_of(m);
            E* dvd = dv + ((size_t)bh * T + m * C) * D + col0;
#pragma unroll
            for (int c = 0; c < NCOL; ++c) {
                const char* cb = hb + c * LT::CTB;
                HandTile<Tr, D>::template copy<NCP>(cb, dSst + off + 16 * c, D, D, ft);
                HandTile<Tr, D>::template copy<NCP>(cb + LT::SLB, dMst + off + 16 * c, D, D, ft);
                HandTile<Tr, C>::template copy<NCP>(cb + 2 * LT::SLB, dvd + 16 * c, D, vm, ft);
            }
        };
        // with the hand-off, waves 0-1 stage and waves 2-3 copy out: the copying
        // waves never wait for their stores, so store latency stays off the
        // chunk barrier
        const uint32_t aA = lds_addr(stA), aB = lds_addr(stB);
        const bool stager = lw < NDMA;
        if constexpr (NBUF == 2) {
            if (stager && NT > 0) issue(aA, NT - 1);
            for (int64_t it = 0; it < NT; ++it) {
                if (stager) __builtin_amdgcn_s_waitcnt(0);
                lds_barrier();
                if (stager) {
                    if (it + 1 < NT) issue((it & 1) ? aA : aB, NT - 2 - it);
                } else if constexpr (OFF) {
                    if (it > 0) flush(it - 1);
                }
            }
            if constexpr (OFF) {
                lds_barrier();                          // the last chunk's hand-off
                if (!stager && NT > 0) flush(NT - 1);
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

    const int ct = wave / RS, h = wave % RS;          // column tile; part of the dk rows
    const int col = col0 + 16 * ct + nn;
    const size_t sbase = (size_t)bh * D * D;
    floatx4 XS[NDL], XM[NDL];                          // dS, dM (rows perm(16 (t + h NDL) + 4g + e))
#pragma unroll
    for (int t = 0; t < NDL; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t off = sbase + (size_t)SL::perm(16 * (t + h * NDL) + 4 * g + e) * D + col;
            XS[t][e] = dST ? dST[off] : 0.f;
            XM[t][e] = dMT ? dMT[off] : 0.f;
        }
    if constexpr (RS > 1) {
        if (h == 0 && lane < 2) xflag[2 * ct + lane] = 0;   // the first barrier orders it before any use
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
        // OFF: this iteration's hand-off tiles; otherwise the wave's staging tiles
        char* hand = OFF ? stg + (it & 1) * LT::PAR + ct * LT::CTB : stg;
        E* sg = OFF ? reinterpret_cast<E*>(stg) : reinterpret_cast<E*>(stg) + ct * 2 * LT::SR * 16;
        if constexpr (OFF) {
            HandTile<Tr, D>::write(XS, reinterpret_cast<E*>(hand), lane, h * NDL);
            HandTile<Tr, D>::write(XM, reinterpret_cast<E*>(hand + LT::SLB), lane, h * NDL);
        } else {
            static_assert(RS == 1, "row split needs the hand-off tiles");
            const size_t off = tile * D * D + col0 + 16 * ct;
            store_slice<Tr, D>(XS, sg, dSst + off, lane);
            store_slice<Tr, D>(XM, sg + LT::SR * 16, dMst + off, lane);
        }
        if constexpr (RS == 1) {
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
                        if (upper_step<Tr>(tc, ks))
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
                        if (upper_step<Tr>(tc, ks))
                            dW[tc] = Tr::mma(LdsA<Tr, LT::PT>::load(TTl, SL::perm(16 * tc + nn), ks, g), vb[ks], dW[tc]);
                }
            }
            {
                // dV rows of the chunk: C x 16 into the hand-off tile, or through
                // the first staging tile
                if constexpr (OFF) {
                    HandTile<Tr, C>::write(dW, reinterpret_cast<E*>(hand + 2 * LT::SLB), lane);
                } else {
                    E* lt = sg;
#pragma unroll
                    for (int tc = 0; tc < NCT; ++tc)
#pragma unroll
                        for (int e = 0; e < 4; ++e) lt[SL::perm(16 * tc + 4 * g + e) * 16 + nn] = Tr::from_f(dW[tc][e]);
                    constexpr int EPV = 16 / sizeof(E), PPR = 16 / EPV, NP = C * PPR;
                    E* dst = dv + ((size_t)bh * T + n * C) * D + col0 + 16 * ct;
#pragma unroll
                    for (int i = 0; i < (NP + 63) / 64; ++i) {
                        const int p = i * 64 + lane;
                        const int r = p / PPR, c = (p % PPR) * EPV;
                        if ((NP % 64 == 0 || p < NP) && r < vm)
                            *reinterpret_cast<uint4*>(dst + (size_t)r * D + c) = reinterpret_cast<const uint4*>(lt)[p];
                    }
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
        } else {
            // this wave's part of K dS', K dM' (its dk rows), weighted by the
            // gates: P = Diag(gS) K dS - Diag(gM) K dM over those rows
            floatx4 P[NCT];
            {
                floatx4 KS[NCT], KM[NCT];
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) { KS[tc] = zero4(); KM[tc] = zero4(); }
#pragma unroll
                for (int kl = 0; kl < KSH; ++kl) {
                    const frag sb = SL::from_acc(XS, kl), mb = SL::from_acc(XM, kl);
#pragma unroll
                    for (int tc = 0; tc < NCT; ++tc) {
                        const frag a = LdsA<Tr, LT::PK>::load(Kl, SL::perm(16 * tc + nn), kl + h * KSH, g);
                        KS[tc] = Tr::mma(a, sb, KS[tc]);
                        KM[tc] = Tr::mma(a, mb, KM[tc]);
                    }
                }
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) {
                    const floatx4 gs = crow(cf, MDN_COEF_GS, tc), gm = crow(cf, MDN_COEF_GM, tc);
#pragma unroll
                    for (int e = 0; e < 4; ++e) P[tc][e] = gs[e] * KS[tc][e] - gm[e] * KM[tc][e];
                }
            }
            frag ob[KSC];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) ob[ks] = ColOperand<Tr, OW>::load(Ol, ct, ks, lane);
            floatx4* xt = xb + ct * NCT * 64 + lane;
            if (h == 1) {
                // Aqk^T dO joins this part, which goes to wave 0
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
                    for (int tc = 0; tc < NCT; ++tc)
                        if (upper_step<Tr>(tc, ks))
                            P[tc] = Tr::mma(LdsA<Tr, LT::PT>::load(ATl, SL::perm(16 * tc + nn), ks, g), ob[ks], P[tc]);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) xt[tc * 64] = P[tc];
                if (lane == 0) pair_release(&xflag[2 * ct], (int)it + 1);
            }
            // chunk-start adjoints of this wave's rows, and their products with dO
            const float abarC = cf[MDN_COEF_ABAR * C + C - 1];
            const float bC = cf[MDN_COEF_B * C + C - 1];
            const float mubarC = expf(cf[MDN_COEF_LM * C + C - 1]);
#pragma unroll
            for (int t = 0; t < NDL; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    XM[t][e] = mubarC * XM[t][e] - bC * XS[t][e];
                    XS[t][e] = abarC * XS[t][e];
                }
            auto dO_products = [&](int k0, int k1) __attribute__((always_inline)) {
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) {
                    if (ks < k0 || ks >= k1) continue;
                    float sa[NSL], sb[NSL];
                    SL::load_row(cf + MDN_COEF_ABAR * C, ks, g, sa);
                    SL::load_row(cf + MDN_COEF_B * C, ks, g, sb);
#pragma unroll
                    for (int j = 0; j < NSL; ++j) {
                        // the staged dO rows past the end repeat the last row: weight 0
                        const bool in = SL::row(ks, g, j) < vm;
                        sa[j] = in ? sa[j] : 0.f;
                        sb[j] = in ? -sb[j] : 0.f;
                    }
                    const frag dOa = FragScale<Tr>::apply(ob[ks], sa), dOb = FragScale<Tr>::apply(ob[ks], sb);
#pragma unroll
                    for (int t = 0; t < NDL; ++t) {
                        const frag qT = TrOperand<Tr, LT::PK>::load(Ql, t + h * NDL, ks, lane);
                        XS[t] = Tr::mma(qT, dOa, XS[t]);
                        XM[t] = Tr::mma(qT, dOb, XM[t]);
                    }
                }
            };
            // wave 1 takes all its products with dO before it waits for dW;
            // wave 0 the first half of the contraction steps before it waits
            // for the partner's part, the rest after it has handed dW over, so
            // that dW reaches wave 1 sooner (the accumulation order is the same)
            constexpr int DOS = KSC / 2;
            // dvt = P_0 + P_1 (with Aqk^T dO) and dW = T^T dvt on wave 0, which
            // hands dW to wave 1 and dW (the chunk's dV rows) to the loaders
            floatx4 dW[NCT];
            if (h == 0) {
                dO_products(0, DOS);
                pair_wait(&xflag[2 * ct], (int)it + 1);
                floatx4 dV[NCT];
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) dV[tc] = P[tc] + xt[tc * 64];
                frag vb[KSC];
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) vb[ks] = SL::from_acc(dV, ks);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) {
                    dW[tc] = zero4();
#pragma unroll
                    for (int ks = 0; ks < KSC; ++ks)
                        if (upper_step<Tr>(tc, ks))
                            dW[tc] = Tr::mma(LdsA<Tr, LT::PT>::load(TTl, SL::perm(16 * tc + nn), ks, g), vb[ks], dW[tc]);
                }
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) xt[tc * 64] = dW[tc];
                if (lane == 0) pair_release(&xflag[2 * ct + 1], (int)it + 1);
                HandTile<Tr, C>::write(dW, reinterpret_cast<E*>(hand + 2 * LT::SLB), lane);
                dO_products(DOS, KSC);
            } else {
                dO_products(0, KSC);
                pair_wait(&xflag[2 * ct + 1], (int)it + 1);
#pragma unroll
                for (int tc = 0; tc < NCT; ++tc) dW[tc] = xt[tc * 64];
            }
            // the products with dW
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                float nsa[NSL], sab[NSL];
                SL::load_row(cf + MDN_COEF_ABAR * C, ks, g, nsa);
                SL::load_row(cf + MDN_COEF_ABP * C, ks, g, sab);
#pragma unroll
                for (int j = 0; j < NSL; ++j) nsa[j] = -nsa[j];
                const frag dWa = SL::from_acc_scaled(dW, ks, nsa), dWab = SL::from_acc_scaled(dW, ks, sab);
#pragma unroll
                for (int t = 0; t < NDL; ++t) {
                    const frag kT = TrOperand<Tr, LT::PK>::load(Kl, t + h * NDL, ks, lane);
                    XS[t] = Tr::mma(kT, dWa, XS[t]);
                    XM[t] = Tr::mma(kT, dWab, XM[t]);
                }
            }
        }
    }
    if constexpr (OFF) lds_barrier();                   // the loaders copy the last chunk's hand-off
#pragma unroll
    for (int t = 0; t < NDL; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t off = sbase + (size_t)SL::perm(16 * (t + h * NDL) + 4 * g + e) * D + col;
            dS0[off] = XS[t][e];
            dM0[off] = XM[t][e];
        }
}

// ---------------------------------------------------------------------------
// sgrad: the products with the states, one workgroup per chunk tile
//
// The A operands (the chunk's dO, dW and vtilde rows) are staged in LDS by
// direct loads; wave w owns dk-column tiles w, w + 4, ... of the outputs
// (in each pass the four waves read adjacent q and k columns, so a line of
// q or k is fetched once), and each state row (the B operand X^T: rows of X are contiguous
// in the contraction index) is read from memory once per workgroup.  For
// one column tile the four states' operands are held while the chunk's
// row tiles run; each 16 x 16 output tile is folded and stored as soon as
// its six products are done.  Row dots with q and k give the coefficient
// adjoints (rows past a ragged end stage copies of the last row and meet
// zero q and k; q and k of all row tiles are loaded with the column tile's
// state operands, so their latency is paid once per column tile); the state inner products <S, dS'>, <M, dS'>, <M, dM'> come from
// the same operands.
// ---------------------------------------------------------------------------
// Workgroups of the sgrad kernel that fit one compute unit's LDS (at most
// three): the occupancy its register allocation targets (one wave per SIMD
// each).
template <typename Tr, int D, int C>
struct SgradOcc {
    static constexpr int LDS = 3 * C * D * (int)sizeof(typename Tr::elem) + MDN_COEF_ROWS * C * 4 + 5 * C * 4 + 48;
    static constexpr int FIT = (160 * 1024) / LDS;
    static constexpr int W = FIT < 1 ? 1 : (FIT > 3 ? 3 : FIT);
};

template <typename Tr, int D, int C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SgradOcc<Tr, D, C>::W)))
void mdn_bwd_sgrad_kernel(const typename Tr::elem* __restrict__ q, const typename Tr::elem* __restrict__ k,
                          const typename Tr::elem* __restrict__ Vt, const typename Tr::elem* __restrict__ dO,
                          const typename Tr::elem* __restrict__ dW, const float* __restrict__ coef,
                          const typename Tr::elem* __restrict__ Sst, const typename Tr::elem* __restrict__ Mst,
                          const typename Tr::elem* __restrict__ dSst, const typename Tr::elem* __restrict__ dMst,
                          typename Tr::elem* __restrict__ dqp, typename Tr::elem* __restrict__ dkp,
                          float* __restrict__ vec,
                          int64_t T, int64_t NT)
{
    using E = typename Tr::elem;
    using frag = typename Tr::frag;
    constexpr int ES = sizeof(E);
    constexpr int NCT = C / 16, NDH = D / 16, KSD = D / Tr::KW;
    constexpr int CPW = NDH >= 4 ? NDH / 4 : 1;       // column tiles per wave
    constexpr int PK = D * ES / 16, TB = C * PK * 16, PC = MDN_COEF_ROWS * C * 4 / 16;
    __shared__ __attribute__((aligned(16))) char st[3 * TB + PC * 16];   // dO, dW, vtilde rows (swizzled), coefficients
    __shared__ float rv[5][C];                                   // row dots
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

    {
        const unsigned vlast = (unsigned)vm - 1;
        auto seq_row = [&](unsigned r) { return (r < vlast ? r : vlast) * (unsigned)(D * ES); };
        const uint32_t base = lds_addr(st);
        if (wave == 0) dma_tile<C, PK>(base, reinterpret_cast<const char*>(dO + rowbase * D), seq_row, lane);
        else if (wave == 1) dma_tile<C, PK>(base + TB, reinterpret_cast<const char*>(dW + rowbase * D), seq_row, lane);
        else if (wave == 2) dma_tile<C, PK>(base + 2 * TB, reinterpret_cast<const char*>(Vt + rowbase * D), seq_row, lane);
        else dma_plain<1, PC>(base + 3 * TB, reinterpret_cast<const char*>(cf), [](unsigned) { return 0u; }, lane);
    }
    const float* cfl = reinterpret_cast<const float*>(st + 3 * TB);
    for (int i = tid; i < 5 * C; i += 256) (&rv[0][0])[i] = 0.f;
    // the first column tile's state operands are issued before the wait, so
    // that they travel with the staging copies
    frag bS[KSD], bM[KSD], bdS[KSD], bdM[KSD];
    // q, k at this lane's output positions for all row tiles, two rows per
    // vector (one register in the bf16 path), issued with the state operands
    typedef E e2 __attribute__((ext_vector_type(2)));
    e2 qa[NCT][2], ka[NCT][2];
    auto load_states = [&](int ct) __attribute__((always_inline)) {
        const int c = 16 * ct + nn;
#pragma unroll
        for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + 4 * g + e;
                qa[rt][e >> 1][e & 1] = r < vm ? q[(rowbase + r) * D + c] : Tr::from_f(0.f);
                ka[rt][e >> 1][e & 1] = r < vm ? k[(rowbase + r) * D + c] : Tr::from_f(0.f);
            }
        const size_t ro = (size_t)(16 * ct + nn) * D;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            bS[ks] = SlotRow<Tr>::load(S + ro, ks, g);
            bM[ks] = SlotRow<Tr>::load(M + ro, ks, g);
            bdS[ks] = SlotRow<Tr>::load(dS + ro, ks, g);
            bdM[ks] = SlotRow<Tr>::load(dM + ro, ks, g);
        }
    };
    if (wave < NDH) load_states(wave);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    float ip0 = 0.f, ip1 = 0.f, ip2 = 0.f;
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
        const int ct = wave + 4 * cc;                 // interleaved: the four waves read one q, k line
        if (ct >= NDH) break;                         // uniform
        const int c = 16 * ct + nn;                   // dk column of this lane's outputs / state row
        if (cc > 0) load_states(ct);
        // the state inner products over these rows
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            if constexpr (std::is_same<Tr, TraitsBf16>::value) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float xs = (float)bS[ks][j], xm = (float)bM[ks][j];
                    const float ys = (float)bdS[ks][j], ym = (float)bdM[ks][j];
                    ip0 = fmaf(xs, ys, ip0);
                    ip1 = fmaf(xm, ys, ip1);
                    ip2 = fmaf(xm, ym, ip2);
                }
            } else {
                ip0 = fmaf(bS[ks], bdS[ks], ip0);
                ip1 = fmaf(bM[ks], bdS[ks], ip1);
                ip2 = fmaf(bM[ks], bdM[ks], ip2);
            }
        }
#pragma unroll
        for (int rt = 0; rt < NCT; ++rt) {
            float qcur[4], kcur[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qcur[e] = Tr::to_f(qa[rt][e >> 1][e & 1]);
                kcur[e] = Tr::to_f(ka[rt][e >> 1][e & 1]);
            }
            floatx4 oS = zero4(), wS = zero4(), oM = zero4(), wM = zero4(), vS = zero4(), vM = zero4();
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const frag aO = LdsA<Tr, PK>::load(st, 16 * rt + nn, ks, g);
                const frag aW = LdsA<Tr, PK>::load(st + TB, 16 * rt + nn, ks, g);
                const frag aV = LdsA<Tr, PK>::load(st + 2 * TB, 16 * rt + nn, ks, g);
                oS = Tr::mma(aO, bS[ks], oS);
                oM = Tr::mma(aO, bM[ks], oM);
                wS = Tr::mma(aW, bS[ks], wS);
                wM = Tr::mma(aW, bM[ks], wM);
                vS = Tr::mma(aV, bdS[ks], vS);
                vM = Tr::mma(aV, bdM[ks], vM);
            }
            const int r0 = 16 * rt + 4 * g;
            const floatx4 ca = *reinterpret_cast<const floatx4*>(cfl + MDN_COEF_ABAR * C + r0);
            const floatx4 cb = *reinterpret_cast<const floatx4*>(cfl + MDN_COEF_B * C + r0);
            const floatx4 cab = *reinterpret_cast<const floatx4*>(cfl + MDN_COEF_ABP * C + r0);
            const floatx4 cgs = *reinterpret_cast<const floatx4*>(cfl + MDN_COEF_GS * C + r0);
            const floatx4 cgm = *reinterpret_cast<const floatx4*>(cfl + MDN_COEF_GM * C + r0);
            E* qo = dqp + (tile * C + r0) * D + c;
            E* ko = dkp + (tile * C + r0) * D + c;
            float pd[5][4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // rows past a ragged end: their q and k are zero, so they add
                // nothing to the row dots, and their partial rows are never read
                const float os = oS[e], om = oM[e], ws = wS[e], wm = wM[e];
                const float vs = vS[e], vmm = vM[e];
                qo[e * D] = Tr::from_f(ca[e] * os - cb[e] * om);
                ko[e * D] = Tr::from_f(-ca[e] * ws + cab[e] * wm + cgs[e] * vs - cgm[e] * vmm);
                const float qv = qcur[e], kv = kcur[e];
                pd[0][e] = qv * os - kv * ws;
                pd[1][e] = -qv * om;
                pd[2][e] = kv * wm;
                pd[3][e] = kv * vs;
                pd[4][e] = -kv * vmm;
            }
#pragma unroll
            for (int a = 0; a < 5; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e) pd[a][e] = row_sum16(pd[a][e]);
            if (nn == 15) {
#pragma unroll
                for (int a = 0; a < 5; ++a)
#pragma unroll
                    for (int e = 0; e < 4; ++e) atomicAdd(&rv[a][r0 + e], pd[a][e]);
            }
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        ip0 += __shfl_xor(ip0, m, 64);
        ip1 += __shfl_xor(ip1, m, 64);
        ip2 += __shfl_xor(ip2, m, 64);
    }
    if (lane == 0) { red[wave][0] = ip0; red[wave][1] = ip1; red[wave][2] = ip2; }
    __syncthreads();
    for (int i = tid; i < 5 * C; i += 256) vt[i] = (&rv[0][0])[i];
    if (tid < 3) vt[5 * C + tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
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
// (LA, LM the chunk's inclusive cumulative logs).  Psi comes from its column
// recurrence (products of alpha and mu only); the Z contraction over chunk
// rows runs on the fp32 matrix cores with E formed on the fly from LA (every
// exponent <= 0).
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
    static constexpr int G0 = 0;                      // DGamma (fp32)
    static constexpr int X0 = FB;                     // X1, then Diag(alpha) X2 (elements)
    static constexpr int Q0 = X0 + 2 * XB, K0 = Q0 + QT;
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
                          const typename Tr::elem* __restrict__ dqp, const typename Tr::elem* __restrict__ dkp,
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
    float* fDG = reinterpret_cast<float*>(lds + L::G0);
    E* x1 = reinterpret_cast<E*>(lds + L::X0);
    E* x2a = reinterpret_cast<E*>(lds + L::X0 + L::XB);
    E* Ql = reinterpret_cast<E*>(lds + L::Q0);
    E* Kl = reinterpret_cast<E*>(lds + L::K0);
    float* vv = reinterpret_cast<float*>(lds + L::V0);
    float* sLM = vv + 1 * C; float* sAl = vv + 2 * C; float* sMu = vv + 3 * C;   // (slot 0 unused)
    float* sBe = vv + 4 * C; float* sEt = vv + 5 * C; float* sAb = vv + 6 * C; float* sB = vv + 7 * C;
    float* sGM = vv + 8 * C; float* sDa = vv + 9 * C; float* sDb = vv + 10 * C; float* sDab = vv + 11 * C;
    float* sDgM = vv + 12 * C; float* sDgS = vv + 13 * C; float* sZ = vv + 14 * C; float* sAd = vv + 15 * C;
    float* sRow = vv + 16 * C; float* sCol = vv + 17 * C; float* sZb = vv + 18 * C; float* sMisc = vv + 19 * C;
    // LA, LM again in fp64, for the factors E[r,m] = exp(LA_r - LA_m) and
    // F[m,i] = exp(LM_m - LM_i) formed from differences of the cumulative
    // logs: in fp32 such a difference keeps only the absolute precision of
    // the larger sum (about 1e-5 at |LA| ~ 100), while Psi comes from
    // running products; the gate gradients subtract terms built from the two
    // (rowsum(DPsi o Psi) against beta Z), which then disagree by that much
    __shared__ double sLAd[C], sLMd[C];

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
            sRow[r] = 0.f;
            sCol[r] = 0.f;
        }
        if (tid < 3) sMisc[tid] = vt[5 * C + tid];    // <S,dS'>, <M,dS'>, <M,dM'>
        if (wave == 0) {                              // inclusive fp64 scans of log alpha, log mu
            double pa = lane < C ? log((double)sAl[lane]) : 0.0;
            double pm = lane < C ? log((double)sMu[lane]) : 0.0;
#pragma unroll
            for (int s = 1; s < 64; s <<= 1) {
                const double ya = __shfl_up(pa, s, 64), ym = __shfl_up(pm, s, 64);
                if (lane >= s) {
                    pa += ya;
                    pm += ym;
                }
            }
            if (lane < C) {
                sLAd[lane] = pa;
                sLMd[lane] = pm;
            }
        }
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

    // ---- 1b. Psi = E Diag(beta) F by its column recurrence ---------------------
    // Psi[r][i] = alpha_r Psi[r-1][i] + beta_r w_{r,i},  w_{r,i} = mubar_r / mubar_i
    // (w_{i,i} = 1, w_{r,i} = mu_r w_{r-1,i}); wave w runs rows [16w, 16w + 16)
    // of column i = lane from zero and the carry of the blocks above enters
    // scaled by their alpha products.  Psi is lower triangular with diagonal
    // beta, DGamma is lower triangular: Psi[r][i] (r > i) is kept at
    // fDG[i][r], the strictly upper triangle of the DGamma table.
    {
        float* xe = reinterpret_cast<float*>(lds + L::X0);    // [NCT][C] block ends (X1 comes later)
        float* xd = xe + NCT * C;                             // [NCT] block alpha products
        const int i = lane, rb = 16 * wave;
        const bool act = wave < NCT && i < C;
        float lv[16], dv[16];
        if (act) {
            float w = (rb > i) ? expf((float)(sLMd[rb - 1] - sLMd[i])) : 0.f;
            float loc = 0.f, d = 1.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int r = rb + j;
                const float al = sAl[r];
                w = (r == i) ? 1.f : w * sMu[r];
                loc = fmaf(al, loc, sBe[r] * w);
                d *= al;
                lv[j] = loc;
                dv[j] = d;
            }
            xe[wave * C + i] = loc;
            if (i == 0) xd[wave] = d;
        }
        __syncthreads();
        if (act) {
            float G = 0.f;
#pragma unroll
            for (int bb = 0; bb < NCT - 1; ++bb)
                if (bb < wave) G = fmaf(xd[bb], G, xe[bb * C + i]);
            // entries r <= i land in the lower triangle of row i, which the
            // DGamma writes below cover before anything reads them as DGamma
            floatx4* row = reinterpret_cast<floatx4*>(fDG + i * FS + rb);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                floatx4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = fmaf(dv[4 * u + e], G, lv[4 * u + e]);
                row[u] = o;
            }
        }
    }
    __syncthreads();

    // ---- 2. per row block (wave): the C x C products and what they feed -------
    float apv[NCT][4];                                // dA o (P K^T) of the wave's rows, for DGamma of the row above
    if (wave < NCT) {
        const int rA = 16 * wave + nn, r0 = 16 * wave + 4 * g;
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
        float rowd[4] = {0.f, 0.f, 0.f, 0.f}, rsum[4] = {0.f, 0.f, 0.f, 0.f}, rsp[4] = {0.f, 0.f, 0.f, 0.f};
        frag bVc[KSD];                                 // vtilde rows of column tile ct (B operand)
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
            bVc[ks] = (nn < vm) ? Contig<Tr>::load(Vt + (rowbase + nn) * D, ks, g) : Contig<Tr>::zero();
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
            for (int e = 0; e < 4; ++e) apv[ct][e] = 0.f;
            const int i = 16 * ct + nn;
            if (ct > wave) {                           // uniform: above the diagonal blocks
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x1[(r0 + e) * XS + i] = Tr::from_f(0.f);
                    x2a[(r0 + e) * XS + i] = Tr::from_f(0.f);
                }
                continue;
            }
            const float eti = sEt[i];
            // the vtilde rows of the next column tile, in flight meanwhile
            frag bVn[KSD];
            if (ct + 1 <= wave) {
                const int inx = i + 16;
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
                    bVn[ks] = (inx < vm) ? Contig<Tr>::load(Vt + (rowbase + inx) * D, ks, g) : Contig<Tr>::zero();
            }
            // Psi rows r and r - 1 from the transposed table (diagonal beta_i)
            floatx4 ps, pp;
            {
                const float bi = sBe[i];
                const floatx4 raw = *reinterpret_cast<const floatx4*>(fDG + i * FS + r0);
                const float rm = fDG[i * FS + (r0 > 0 ? r0 - 1 : 0)];
#pragma unroll
                for (int e = 0; e < 4; ++e) ps[e] = (r0 + e > i) ? raw[e] : (r0 + e == i ? bi : 0.f);
                pp[0] = (r0 - 1 > i) ? rm : (r0 - 1 == i ? bi : 0.f);
#pragma unroll
                for (int e = 1; e < 4; ++e) pp[e] = ps[e - 1];
            }
            floatx4 aqk = zero4(), akk = zero4(), ao = zero4(), aw = zero4();
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const frag bK = Contig<Tr>::load(Kl + i * D, ks, g);
                aqk = Tr::mma(aQ[ks], bK, aqk);
                akk = Tr::mma(aK[ks], bK, akk);
                ao = Tr::mma(aO[ks], bVc[ks], ao);
                aw = Tr::mma(aW[ks], bVc[ks], aw);
            }
            if (ct + 1 <= wave) {
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) bVc[ks] = bVn[ks];
            }
            float csum = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = r0 + e;
                const float al = sAl[r];
                const bool low = i <= r, strict = i < r;
                const float x1v = low ? ao[e] * ps[e] * eti : 0.f;
                const float x2v = strict ? -aw[e] * pp[e] * eti : 0.f;
                const float dg0 = low ? ao[e] * aqk[e] : 0.f;
                const float ap = strict ? -aw[e] * al * akk[e] : 0.f;
                x1[r * XS + i] = Tr::from_f(x1v);
                x2a[r * XS + i] = Tr::from_f(al * x2v);
                if (low) fDG[r * FS + i] = dg0;        // the upper triangle holds Psi
                apv[ct][e] = ap;
                rowd[e] += x2v * akk[e];               // k_r . (X2 K)_r
                // DGamma o Psi: the own entry, and the row-above entry of ap
                rsum[e] += dg0 * eti * ps[e];
                rsp[e] += ap * eti * pp[e];
                csum += dg0 * ps[e] + ap * pp[e];
                if (r == LR && low) {                  // DgS enters DGamma at the last row
                    rsum[e] += sDgS[i] * eti * ps[e];
                    csum += sDgS[i] * ps[e];
                }
            }
            atomicAdd(&sCol[i], csum);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            rowd[e] = row_sum16(rowd[e]);
            rsum[e] = row_sum16(rsum[e]);
            rsp[e] = row_sum16(rsp[e]);
        }
        if (nn == 15) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sAd[r0 + e] = rowd[e];
                atomicAdd(&sRow[r0 + e], rsum[e]);
                if (r0 + e > 0) atomicAdd(&sRow[r0 + e - 1], rsp[e]);
            }
        }
    }
    __syncthreads();
    // DGamma[r-1][i] += (dA o P K^T)[r][i];  DGamma[L][i] += DgS_i
    if (wave < NCT) {
        const int r0 = 16 * wave + 4 * g;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            if (ct > wave) continue;
            const int i = 16 * ct + nn;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = r0 + e;
                if (i < r) fDG[(r - 1) * FS + i] += apv[ct][e];
                if (r == LR) fDG[r * FS + i] += sDgS[i];
            }
        }
    }
    __syncthreads();

    // the state-product parts of dq and dk for step 4, all column tiles, two
    // rows per vector: issued here so that their latency hides behind Z
    typedef E e2 __attribute__((ext_vector_type(2)));
    e2 pqa[NDH][2], pka[NDH][2];
    if (wave < NCT) {
        const E* qp = dqp + (tile * C + 16 * wave + 4 * g) * D + nn;
        const E* kp = dkp + (tile * C + 16 * wave + 4 * g) * D + nn;
#pragma unroll
        for (int ct = 0; ct < NDH; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pqa[ct][e >> 1][e & 1] = qp[e * D + 16 * ct];
                pka[ct][e >> 1][e & 1] = kp[e * D + 16 * ct];
            }
    }

    // ---- 3. Z: G = E^T (DGamma Diag(eta)) on the fp32 matrix cores, G o F row sums
    // (the E entries of a k-step are shared by the column tiles; DGamma is
    // read from the lower triangle only)
    if (wave < NCT) {
        const int mA = 16 * wave + nn, m0 = 16 * wave + 4 * g;
        const double laA = sLAd[mA];
        floatx4 acc[NCT];
        float etc[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            acc[ct] = zero4();
            etc[ct] = sEt[16 * ct + nn];
        }
#pragma unroll
        for (int ks = 0; ks < C / 4; ++ks) {
            if (ks < 4 * wave) continue;               // uniform: rows above the wave's block
            const int r = 4 * ks + g;
            const float a = (r >= mA) ? expf((float)(sLAd[r] - laA)) : 0.f;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                if (ct > wave) continue;
                const int i = 16 * ct + nn;
                const float dg = (i <= r) ? fDG[r * FS + i] : 0.f;
                acc[ct] = F32::mma(a, dg * etc[ct], acc[ct]);
            }
        }
        float zp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            if (ct > wave) continue;
            const int i = 16 * ct + nn;
            const double lmi = sLMd[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + e;
                zp[e] += (i <= m) ? acc[ct][e] * expf((float)(sLMd[m] - lmi)) : 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            zp[e] = row_sum16(zp[e]);
            if (nn == 15) sZ[m0 + e] = zp[e];
        }
    }
    // the b part of Z, mubar_m sum_{r >= m} E[r,m] Db_r: x_m = Db_m + alpha_{m+1}
    // x_{m+1} as a scan of affine maps with the rows reversed over the lanes,
    // on a spare wave or the last one (which has the fewest Z steps)
    if (wave == (NCT < 4 ? NCT : 3)) {
        const int m = C - 1 - lane;
        float A = 1.f, B = 0.f;
        if (m >= 0) {
            A = (m + 1 < C) ? sAl[m + 1] : 1.f;
            B = sDb[m];
        }
        wave_scan_affine(A, B);
        if (m >= 0) sZb[m] = B * expf(sLM[m]);
    }

    // ---- 4. dq, dk: X1 K, X1^T Q + (Diag(alpha) X2)^T K + Diag(alpha) X2 K -----
    if (wave < NCT) {
        const int rA = 16 * wave + nn, r0 = 16 * wave + 4 * g;
        const char* X1c = reinterpret_cast<const char*>(x1);
        const char* X2c = reinterpret_cast<const char*>(x2a);
        frag a1[KSC], a1t[KSC], a2[KSC], a2t[KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            a1[ks] = SlotRow<Tr>::load(x1 + rA * XS, ks, g);
            a2[ks] = SlotRow<Tr>::load(x2a + rA * XS, ks, g);
            a1t[ks] = ColOperand<Tr, XS>::load(X1c, wave, ks, lane);
            a2t[ks] = ColOperand<Tr, XS>::load(X2c, wave, ks, lane);
        }
        const char* Qc = reinterpret_cast<const char*>(Ql);
        const char* Kc = reinterpret_cast<const char*>(Kl);
#pragma unroll
        for (int ct = 0; ct < NDH; ++ct) {
            float pq[4], pk[4];                        // the state-product parts (loaded before Z)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pq[e] = Tr::to_f(pqa[ct][e >> 1][e & 1]);
                pk[e] = Tr::to_f(pka[ct][e >> 1][e & 1]);
            }
            floatx4 aq = zero4(), ak = zero4();
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) {
                const frag bK = ColOperand<Tr, D>::load(Kc, ct, ks, lane);
                const frag bQ = ColOperand<Tr, D>::load(Qc, ct, ks, lane);
                aq = Tr::mma(a1[ks], bK, aq);
                ak = Tr::mma(a1t[ks], bQ, ak);
                ak = Tr::mma(a2t[ks], bK, ak);
                ak = Tr::mma(a2[ks], bK, ak);
            }
            const int c = 16 * ct + nn;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = r0 + e;
                if (r < vm) {
                    dq[(rowbase + r) * D + c] = Tr::from_f(aq[e] + pq[e]);
                    dk[(rowbase + r) * D + c] = Tr::from_f(ak[e] + pk[e]);
                }
            }
        }
    }
    __syncthreads();

    // ---- 5. the gate gradients ------------------------------------------------
    if (wave == 0) {
        const int m = lane;
        const bool in = m < C;
        float dla = 0.f, dlm = 0.f, z = 0.f, de = 0.f, tail = 0.f;
        if (in) {
            z = sZ[m] + sZb[m];
            const float cs = sCol[m];
            de = cs + sDgM[m] * expf((float)(sLMd[LR] - sLMd[m]));
            dla = sRow[m] + sDb[m] * sB[m] - sBe[m] * z + sDa[m] * sAb[m];
            dlm = sBe[m] * z - sEt[m] * cs - sDgM[m] * sGM[m];
            tail = sDgM[m] * sGM[m];
        }
        // the last row's terms: sum_i DgM_i gM_i + Dmubar_L mubar_L
        float tsum = tail;
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) tsum += __shfl_xor(tsum, s, 64);
        if (m == LR) dlm += tsum + sMisc[2] * expf(sLM[LR]);
        // suffix sums over rows, as inclusive scans over the reversed rows
        // (forming them as the total minus a prefix cancels when the suffix is
        // small against the total, and dalpha then divides by a small alpha)
        const float sla = __shfl(wave_scan_add(__shfl(dla, 63 - m, 64)), 63 - m, 64);
        const float slm = __shfl(wave_scan_add(__shfl(dlm, 63 - m, 64)), 63 - m, 64);
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
    hipLaunchKernelGGL((mdn_bwd_replay_kernel<Tr, D, C, NCOL>), dim3((unsigned)grid), dim3(64 * (NCOL + 4)), 0,
                       (hipStream_t)f.stream, (const E*)f.k, (const E*)a.Vt, f.coef, f.S0, f.M0,
                       (E*)a.Sst, (E*)a.Mst, f.T, f.NT, (int)f.BH);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    using CP = CarryPick<Tr, D, C>;
    hipLaunchKernelGGL((mdn_bwd_carry_kernel<Tr, D, C, CP::NCOL, CP::NBUF, CP::RS, CP::NLD, CP::NST>), dim3((unsigned)grid),
                       dim3(64 * (CP::NCOL * CP::RS + CP::NLD)), 0, (hipStream_t)f.stream, (const E*)f.q, (const E*)f.k,
                       (const E*)f.Tmat, (const E*)f.Aqk, f.coef, (const E*)a.dO, a.dST, a.dMT, (E*)a.dv,
                       (E*)a.dSst, (E*)a.dMst, a.dS0, a.dM0, f.T, f.NT, (int)f.BH);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t tiles = f.BH * f.NT;
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL((mdn_bwd_sgrad_kernel<Tr, D, C>), dim3((unsigned)tiles), dim3(256), 0, (hipStream_t)f.stream,
                       (const E*)f.q, (const E*)f.k, (const E*)a.Vt, (const E*)a.dO, (const E*)a.dv, f.coef,
                       (const E*)a.Sst, (const E*)a.Mst, (const E*)a.dSst, (const E*)a.dMst, (E*)a.dqp, (E*)a.dkp, a.vec,
                       f.T, f.NT);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    static_assert(CgradLayout<Tr, D, C>::TOTAL <= 160 * 1024 - 1024, "LDS");
    hipLaunchKernelGGL((mdn_bwd_cgrad_kernel<Tr, D, C>), dim3((unsigned)tiles), dim3(256), 0, (hipStream_t)f.stream,
                       (const E*)f.q, (const E*)f.k, f.alpha, f.mu, f.beta, f.eta, (const E*)a.Vt, (const E*)a.dO,
                       (const E*)a.dv, f.coef, (const E*)a.dqp, (const E*)a.dkp, a.vec, (E*)a.dq, (E*)a.dk, a.dalpha, a.dmu, a.dbeta,
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
        case 16064: return launch_bwd_t<Tr, 16, 64>(a);
        case 32016: return launch_bwd_t<Tr, 32, 16>(a);
        case 32032: return launch_bwd_t<Tr, 32, 32>(a);
        case 32064: return launch_bwd_t<Tr, 32, 64>(a);
        case 64016: return launch_bwd_t<Tr, 64, 16>(a);
        case 64032: return launch_bwd_t<Tr, 64, 32>(a);
        case 64064: return launch_bwd_t<Tr, 64, 64>(a);
        case 128016: return launch_bwd_t<Tr, 128, 16>(a);
        case 128032: return launch_bwd_t<Tr, 128, 32>(a);
        case 128064: return launch_bwd_t<Tr, 128, 64>(a);
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
