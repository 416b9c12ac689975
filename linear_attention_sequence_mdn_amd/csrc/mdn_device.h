// mdn_device.h -- device-side building blocks shared by the MDN kernels (gfx950).
//
// Matrix-core fragments.  Every product in the chunk kernels runs on 16x16
// output tiles:
//   bf16 path: v_mfma_f32_16x16x32_bf16 (8 bf16 of A and of B per lane, K = 32)
//   fp32 path: v_mfma_f32_16x16x4_f32   (1 fp32 of A and of B per lane, K = 4)
// Accumulator layout (both): lane l, register e holds D[4*(l/16) + e][l%16].
// Operand layout: lane l holds row (A) / column (B) l%16 and a group of K
// values selected by l/16.  Which K index a given (lane group, slot) carries
// only has to agree between A and B, so the kernels pick the order that lets
// an accumulator be reused as the next product's B operand without leaving
// registers ("slot map" below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace mdn {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// Element traits
// ---------------------------------------------------------------------------
struct TraitsBf16 {
    using elem = __bf16;
    using frag = bf16x8;
    static constexpr int KW = 32;   // contraction length of one matrix-core op

    static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float to_f(elem x) { return (float)x; }
    static __device__ __forceinline__ elem from_f(float x) { return (__bf16)x; }
};

struct TraitsF32 {
    using elem = float;
    using frag = float;
    static constexpr int KW = 4;

    static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float to_f(elem x) { return x; }
    static __device__ __forceinline__ elem from_f(float x) { return x; }
};

// ---------------------------------------------------------------------------
// Slot map for products whose B operand is an accumulator.
//
// An accumulator "column" is a stack of 16-row tiles acc[0..R/16) along the
// contraction dimension.  Lane group g = l/16 of tile t holds accumulator
// rows 16t + 4g + e, e = 0..3.
//   bf16 (K = 32 per step ks): slots 0..3 <- tile 2ks, slots 4..7 <- tile
//   2ks+1.  Accumulator row x does not stand for index x of the dimension
//   but for perm(x) = 32(x/32) + 8((x/4)%4) + 4((x/16)%2) + x%4, which maps
//   the 8 rows slot-feeding lane group g onto the contiguous indices
//   32ks + 8g .. 32ks + 8g + 7.  A row-major A operand (contraction index
//   contiguous) is then a single 16-byte read.  Every producer and consumer
//   of such a dimension (state rows, chunk rows) applies the same perm.
//   fp32 (K = 4 per step ks): the single slot of group g is accumulator row
//   16(ks/4) + 4g + ks%4, and perm is the identity.
// ---------------------------------------------------------------------------
// T and Aqk are lower triangular, so their upper-right C/2 x C/2 quadrant is
// zero.  Where every matrix-core contraction step is at most C/2 columns wide
// (bf16 at C = 64: steps of 32; fp32 at C >= 32: steps of 16), the products
// that read T and Aqk (and T^T, Aqk^T in the backward) skip the steps that
// fall in that quadrant, so the intra stage does not write it.
template <typename Tr, int C>
constexpr bool quad_unread()
{
    return std::is_same<Tr, TraitsBf16>::value ? C == 64 : C >= 32;
}

template <typename Tr> struct Slots;

template <> struct Slots<TraitsBf16> {
    using Tr = TraitsBf16;
    static constexpr int NSLOT = 8;
    static __device__ __forceinline__ int perm(int x) {
        return (x & ~31) | ((x & 12) << 1) | ((x & 16) >> 2) | (x & 3);
    }
    // index (after perm) carried by slot j of step ks, lane group g
    static __device__ __forceinline__ int row(int ks, int g, int j) { return 32 * ks + 8 * g + j; }
    // B operand from accumulator tiles
    static __device__ __forceinline__ bf16x8 from_acc(const floatx4* acc, int ks) {
        const floatx4 a = acc[2 * ks], b = acc[2 * ks + 1];
        bf16x8 r;
        r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
        r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
        return r;
    }
    // same, each slot j scaled by s[j]
    static __device__ __forceinline__ bf16x8 from_acc_scaled(const floatx4* acc, int ks, const float* s) {
        const floatx4 a = acc[2 * ks], b = acc[2 * ks + 1];
        bf16x8 r;
        r[0] = (__bf16)(a[0] * s[0]); r[1] = (__bf16)(a[1] * s[1]);
        r[2] = (__bf16)(a[2] * s[2]); r[3] = (__bf16)(a[3] * s[3]);
        r[4] = (__bf16)(b[0] * s[4]); r[5] = (__bf16)(b[1] * s[5]);
        r[6] = (__bf16)(b[2] * s[6]); r[7] = (__bf16)(b[3] * s[7]);
        return r;
    }
    static __device__ __forceinline__ bf16x8 zero() {
        union { uint4 u; bf16x8 v; } f;
        f.u = uint4{0u, 0u, 0u, 0u};
        return f.v;
    }
    // element e of accumulator tile t, read back from the B operands that
    // from_acc built from the whole column
    static __device__ __forceinline__ __bf16 acc_elem(const bf16x8* b, int t, int e) {
        return b[t >> 1][4 * (t & 1) + e];
    }
    // the per-slot factors p[row(ks, g, j)], j = 0..7, of a row vector p
    // (16-byte aligned): two 16-byte reads
    static __device__ __forceinline__ void load_row(const float* p, int ks, int g, float (&out)[NSLOT]) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(p + 32 * ks + 8 * g);
        const floatx4 b = *reinterpret_cast<const floatx4*>(p + 32 * ks + 8 * g + 4);
        out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
        out[4] = b[0]; out[5] = b[1]; out[6] = b[2]; out[7] = b[3];
    }
};

template <> struct Slots<TraitsF32> {
    using Tr = TraitsF32;
    static constexpr int NSLOT = 1;
    static __device__ __forceinline__ int perm(int x) { return x; }
    static __device__ __forceinline__ int row(int ks, int g, int /*j*/) {
        return 16 * (ks >> 2) + 4 * g + (ks & 3);
    }
    static __device__ __forceinline__ float from_acc(const floatx4* acc, int ks) {
        return acc[ks >> 2][ks & 3];
    }
    static __device__ __forceinline__ float from_acc_scaled(const floatx4* acc, int ks, const float* s) {
        return acc[ks >> 2][ks & 3] * s[0];
    }
    static __device__ __forceinline__ float zero() { return 0.f; }
    static __device__ __forceinline__ float acc_elem(const float* b, int t, int e) { return b[4 * t + e]; }
    static __device__ __forceinline__ void load_row(const float* p, int ks, int g, float (&out)[NSLOT]) {
        out[0] = p[row(ks, g, 0)];
    }
};

// Operand with contiguous contraction index, natural order (both operands
// read from memory): lane group g holds K values [KW*ks + (KW/4)*g, +KW/4).
template <typename Tr> struct Contig;
template <> struct Contig<TraitsBf16> {
    static __device__ __forceinline__ bf16x8 load(const __bf16* rowp, int ks, int g) {
        union { uint4 u; bf16x8 v; } f;
        f.u = *reinterpret_cast<const uint4*>(rowp + 32 * ks + 8 * g);
        return f.v;
    }
    static __device__ __forceinline__ bf16x8 zero() {
        union { uint4 u; bf16x8 v; } f;
        f.u = uint4{0u, 0u, 0u, 0u};
        return f.v;
    }
};
template <> struct Contig<TraitsF32> {
    static __device__ __forceinline__ float load(const float* rowp, int ks, int g) {
        return rowp[4 * ks + g];
    }
    static __device__ __forceinline__ float zero() { return 0.f; }
};

// ---------------------------------------------------------------------------
// Wave-wide (64-lane) inclusive scans on DPP lane moves: row_shr 1, 2, 4, 8
// inside each 16-lane row, then the broadcasts of lane 15 into rows 1 and 3
// and of lane 31 into rows 2 and 3.  A lane whose source lies outside its
// row, or whose row is masked off, receives the identity `ident`.
// ---------------------------------------------------------------------------
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_move(float x, float ident) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(ident), __float_as_int(x), CTRL, ROWS, 0xf,
                                                      false));
}
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118;
constexpr int DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;

__device__ __forceinline__ float wave_scan_add(float x) {
    x += dpp_move<DPP_ROW_SHR1>(x, 0.f);
    x += dpp_move<DPP_ROW_SHR2>(x, 0.f);
    x += dpp_move<DPP_ROW_SHR4>(x, 0.f);
    x += dpp_move<DPP_ROW_SHR8>(x, 0.f);
    x += dpp_move<DPP_ROW_BCAST15, 0xa>(x, 0.f);
    x += dpp_move<DPP_ROW_BCAST31, 0xc>(x, 0.f);
    return x;
}

// Inclusive scan of the affine maps x -> A x + B in lane order: afterwards
// lane r holds the composition of the maps of lanes 0..r (applied in that
// order), so B is the value reached from x = 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ void affine_step(float& A, float& B) {
    const float Ap = dpp_move<CTRL, ROWS>(A, 1.f), Bp = dpp_move<CTRL, ROWS>(B, 0.f);
    B = fmaf(A, Bp, B);
    A *= Ap;
}
__device__ __forceinline__ void wave_scan_affine(float& A, float& B) {
    affine_step<DPP_ROW_SHR1>(A, B);
    affine_step<DPP_ROW_SHR2>(A, B);
    affine_step<DPP_ROW_SHR4>(A, B);
    affine_step<DPP_ROW_SHR8>(A, B);
    affine_step<DPP_ROW_BCAST15, 0xa>(A, B);
    affine_step<DPP_ROW_BCAST31, 0xc>(A, B);
}

// ---------------------------------------------------------------------------
// Inverse of a 16 x 16 unit lower-triangular matrix I + A by forward
// substitution in registers, one wave: lane (r, g) (r = lane % 16, g =
// lane / 16) holds row r of A in a[0..3] (columns 4q .. 4q+3 in a[q]) and
// returns row r of (I + A)^{-1} at columns 4g .. 4g+3 in t.  Only A's
// strictly lower part is used.  Step Q takes row Q, final after the steps
// before it, to every row of the lane's 16-lane row group by a DPP row
// broadcast (row_newbcast) and subtracts A[r][Q] times it from rows r > Q.
// ---------------------------------------------------------------------------
template <int Q>
__device__ __forceinline__ void unit_lower_inv16_step(float (&t)[4], const floatx4 (&a)[4], int r)
{
    const float lq = Q < r ? a[Q / 4][Q % 4] : 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float tq = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(t[c]), 0x150 + Q, 0xf, 0xf,
                                                                    false));
        t[c] = fmaf(-lq, tq, t[c]);
    }
}
template <int... Q>
__device__ __forceinline__ void unit_lower_inv16_steps(float (&t)[4], const floatx4 (&a)[4], int r,
                                                       std::integer_sequence<int, Q...>)
{
    (unit_lower_inv16_step<Q>(t, a, r), ...);
}
__device__ __forceinline__ void unit_lower_inv16(float (&t)[4], const floatx4 (&a)[4], int lane)
{
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) t[c] = (r == 4 * g + c) ? 1.f : 0.f;
    unit_lower_inv16_steps(t, a, r, std::make_integer_sequence<int, 15>{});
}

// ---------------------------------------------------------------------------
// Workgroup -> (head, column slab) map that keeps the slabs of one head on
// one XCD.  Workgroups are dispatched round-robin over the 8 XCDs in order
// of their linear id, so ids with equal (id % 8) share an XCD and its L2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void xcd_head_map(int id, int slabs, int BH, int& bh, int& slab) {
    if ((BH & 7) == 0) {
        const int x = id & 7, l = id >> 3;
        bh = x * (BH >> 3) + l / slabs;
        slab = l % slabs;
    } else {
        bh = id / slabs;
        slab = id % slabs;
    }
}

// The sequence a workgroup of the inter-chunk stage carries: state index
// bh, column slab, first row, first tile slot and length.  Without cu the
// batch is [BH, T] and workgroup id covers head bh (xcd_head_map).  With cu
// it is a packed batch of BH = nseq * H units (sequence, head); states are
// [nseq, H, D, D].  Units are taken longest sequence first (perm): unit rank
// r = (sequence rank) * H + head.  Workgroups go to the XCDs round robin in
// launch order, so rank r runs on XCD r % 8, all its slabs there, and each
// XCD meets its units longest first.  The bounds read from cu are clamped
// into [0, T] and ordered, which keeps every row and tile slot in range
// whatever the table holds.
//
// Sequence split (seg.P > 0, [BH, T] layout): each sequence is cut at chunk
// boundaries into P segments, segment p holding chunks [P0(p), P0(p + 1))
// with P0(p) = p NT / P.  Each chunk's map of the state [S; M] is affine, so
// a segment's is too; the columns of the state evolve independently under
// one 2D x 2D map.  Pass 1 (seg.pass == 1) runs, per sequence, segment 0
// from the true start state (its outputs are final) and, for each middle
// segment 1 .. P-2, three replicas from chunk P0(p): the data from a zero
// state (the map's offset), and V = 0 from S = I, M = 0 and from S = 0,
// M = I (the columns of the map); replicas store no O or vtilde.  Units are
// (sequence, j) with j = 0 for segment 0 and j = 1 + 3 (p - 1) + replica;
// the end states go to slot unit.  Pass 2 reruns segments 1 .. P-1, unit
// (sequence, p - 1), from the start states the combine step placed at
// unit.sin; only the last segment stores its end state (at the sequence's
// own slot).
struct InterSeg {
    int P, pass;
};
struct InterUnit {
    int bh, slab;
    int64_t row0, tile0, len;
    int64_t sin, sout;      // state element offsets of the start / end states (-1: zero start / no store)
    int ident;              // 1: start from S = I, M = 0; 2: from S = 0, M = I
    bool vzero, ostore;     // V read as zero; O and vtilde stored
};
__device__ __forceinline__ int64_t seg_first_chunk(int p, int P, int64_t NT) { return (int64_t)p * NT / P; }
// SEG: the kernel is the sequence split's (seg.P > 0); the other kernels
// are compiled without the split's unit fields.
template <bool SEG>
__device__ __forceinline__ InterUnit inter_unit(int id, int slabs, int BH, int64_t T, int64_t NT, int C,
                                                const int32_t* __restrict__ cu, const int32_t* __restrict__ perm,
                                                int H, int D, InterSeg seg)
{
    InterUnit u;
    u.ident = 0;
    u.vzero = false;
    u.ostore = true;
    if constexpr (SEG) {
        // BH counts the units of the pass here; H the sequences
        const int U = seg.pass == 1 ? 1 + 3 * (seg.P - 2) : seg.P - 1;
        int un;
        xcd_head_map(id, slabs, BH, un, u.slab);
        const int s = un / U, j = un % U;
        const int p = seg.pass == 1 ? (j == 0 ? 0 : 1 + (j - 1) / 3) : 1 + j;
        const int64_t c0 = seg_first_chunk(p, seg.P, NT), c1 = seg_first_chunk(p + 1, seg.P, NT);
        u.bh = s;
        u.row0 = (int64_t)s * T + c0 * C;
        u.tile0 = (int64_t)s * NT + c0;
        u.len = (c1 * C < T ? c1 * C : T) - c0 * C;
        const int64_t DD = (int64_t)D * D;
        if (seg.pass == 1) {
            const int rep = j == 0 ? 0 : (j - 1) % 3;
            u.sin = j == 0 ? s * DD : -1;
            u.ident = rep;
            u.vzero = rep > 0;
            u.ostore = j == 0;
            u.sout = (int64_t)un * DD;
        } else {
            // start states: segment 1 from the end state of segment 0 (pass-1
            // slot (s, 0)); segment p >= 2 from the combine step's slot
            // H U1 + s (P - 2) + p - 2 (U1 = 1 + 3 (P - 2))
            const int U1 = 1 + 3 * (seg.P - 2);
            u.sin = (p == 1 ? (int64_t)s * U1 : (int64_t)H * U1 + (int64_t)s * (seg.P - 2) + p - 2) * DD;
            u.sout = p == seg.P - 1 ? s * DD : -1;
        }
        return u;
    }
    if (!cu) {
        xcd_head_map(id, slabs, BH, u.bh, u.slab);
        u.row0 = (int64_t)u.bh * T;
        u.tile0 = (int64_t)u.bh * NT;
        u.len = T;
        u.sin = u.sout = (int64_t)u.bh * D * D;
        return u;
    }
    int r;
    if ((BH & 7) == 0) {
        const int x = id & 7, l = id >> 3;
        r = (l / slabs) * 8 + x;
        u.slab = l % slabs;
    } else {
        r = id / slabs;
        u.slab = id % slabs;
    }
    const int64_t nseq = BH / H, h = r % H;
    int64_t i = perm[r / H];
    i = i < 0 ? 0 : (i >= nseq ? nseq - 1 : i);
    u.bh = (int)(i * H + h);
    int64_t c0 = cu[i], c1 = cu[i + 1];
    c0 = c0 < 0 ? 0 : (c0 > T ? T : c0);
    c1 = c1 < c0 ? c0 : (c1 > T ? T : c1);
    u.row0 = h * T + c0;
    u.tile0 = h * NT + c0 / C + i;
    u.len = c1 - c0;
    u.sin = u.sout = (int64_t)u.bh * D * D;
    return u;
}

}  // namespace mdn
