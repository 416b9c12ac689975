// mdn_lds.h -- LDS staging helpers shared by the chunk kernels (gfx950):
// LDS addresses and barriers, the XOR swizzle of 16-byte pieces, matrix-core
// operand reads from swizzled tiles, and direct global->LDS tile copies.
#pragma once

#include "mdn_device.h"

namespace mdn {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroup barrier that orders LDS only.  __syncthreads() would also wait
// for every outstanding global load and store (including the next chunk's
// LDS prefetch); here the chunk-boundary wait is explicit instead.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Swizzle key of row r for rows of P 16-byte pieces.  Key 0 gives the 16
// rows an operand read touches (perm of 16 consecutive accumulator rows, or
// the 4 x 4 row/column pattern of the transpose read) distinct keys, and
// does not depend on the bit of the row that tells even from odd row tiles,
// so the reads of all row tiles share their lane addresses up to a constant.
// Key 1 was chosen by measuring bank conflicts on gfx950: with it the
// 16-byte operand reads of 16 rows perm(16t + i) are conflict-free, where
// key 0 measures two-way conflicts; it costs address registers, so it is
// used for the tiles that only waves with registers to spare read.
template <int P, int KEY = 0>
__device__ __forceinline__ int swz_key(int r) {
    static_assert(P >= 4 && (P & (P - 1)) == 0, "rows of 4, 8, 16, ... pieces");
    if constexpr (KEY == 0) return ((r & 3) * (P / 4)) | ((r >> 3) & (P / 4 - 1));
    else return ((r & 3) * (P / 4)) ^ ((r >> 2) & (P / 2 - 1));
}

// byte offset of (row r, byte b) in a row of P 16-byte pieces; piece p of
// row r is stored at piece p ^ key(r)
template <int P, int KEY = 0>
__device__ __forceinline__ int swz(int r, int b) {
    return r * P * 16 + ((((b >> 4) ^ swz_key<P, KEY>(r))) << 4) + (b & 15);
}

// A operand of a product whose B operand comes from accumulators (slot map),
// from a swizzled LDS tile whose rows hold the contraction index.
template <typename Tr, int P, int KEY = 0> struct LdsA;
template <int P, int KEY> struct LdsA<TraitsBf16, P, KEY> {
    // slots of lane group g are the contiguous columns 32ks + 8g .. +7
    static __device__ __forceinline__ bf16x8 load(const char* tile, int row, int ks, int g) {
        union { uint4 u; bf16x8 v; } f;
        f.u = *reinterpret_cast<const uint4*>(tile + swz<P, KEY>(row, 2 * (32 * ks + 8 * g)));
        return f.v;
    }
};
template <int P, int KEY> struct LdsA<TraitsF32, P, KEY> {
    static __device__ __forceinline__ float load(const char* tile, int row, int ks, int g) {
        const int c = 16 * (ks >> 2) + 4 * g + (ks & 3);
        return *reinterpret_cast<const float*>(tile + swz<P, KEY>(row, 4 * c));
    }
};

// Copy rows [r0, r0 + R) of a tile of P 16-byte pieces per row from global
// memory into LDS, swizzled (piece p of row r lands at piece p ^ key(r)), by
// one wave; `dst` is the LDS byte address of the tile's row 0.  Instruction
// i covers rows r0 + [i*64/P, (i+1)*64/P): lane l takes row r0 + i*64/P + l/P
// and physical piece l%P, so its source offset is a per-lane constant plus a
// per-instruction constant.  `rowoff(r)` gives the byte offset of global row
// r relative to `base`.
//
// QS leaves out the all-zero quadrant of a triangular tile of RT rows (its
// LDS pieces keep whatever they held; no product reads them): 1 = the
// upper-right quadrant (rows < RT/2, pieces >= P/2: T, Aqk), 2 = the
// lower-left one (rows >= RT/2, pieces < P/2: T^T, Aqk^T).
template <int QS, int RT, int P>
__device__ __forceinline__ bool quad_piece(unsigned r, unsigned p)
{
    if constexpr (QS == 1) return r < (unsigned)RT / 2 && p >= (unsigned)P / 2;
    else if constexpr (QS == 2) return r >= (unsigned)RT / 2 && p < (unsigned)P / 2;
    else return false;
}

template <int R, int P, int KEY = 0, int QS = 0, int RT = 0, typename RowOff>
__device__ __forceinline__ void dma_tile(uint32_t dst, const char* __restrict__ base, RowOff rowoff, int lane,
                                         int r0 = 0)
{
    static_assert(P <= 64 && 64 % P == 0, "rows of at most 64 pieces");
    constexpr int RPI = 64 / P;                       // rows per instruction
    constexpr int NI = (R * P + 63) / 64;
    const unsigned lr = (unsigned)lane / P, lp = (unsigned)lane % P;
    const uint32_t d0 = dst + (uint32_t)r0 * P * 16;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const unsigned rl = i * RPI + lr;             // row within the copied range
        const unsigned r = (unsigned)r0 + rl;
        const unsigned p = lp ^ (unsigned)swz_key<P, KEY>((int)r);
        if ((R * P % 64 == 0 || rl < (unsigned)R) && !quad_piece<QS, RT, P>(r, p))
            __builtin_amdgcn_global_load_lds(base + rowoff(r) + p * 16, (lds_void*)(uintptr_t)(d0 + i * 1024), 16, 0, 0);
    }
}

// The same copies with the destination given as a pointer into a named LDS
// array (not as an integer address), so that the compiler can tell which
// array a copy writes and need not wait for it before LDS accesses to other
// arrays.
typedef __attribute__((address_space(3))) char lds_char;
template <typename T>
__device__ __forceinline__ lds_char* lds_ptr(T* p) { return (lds_char*)(__attribute__((address_space(3))) void*)p; }

template <int R, int P, int KEY = 0, int QS = 0, int RT = 0, typename RowOff>
__device__ __forceinline__ void dma_tile_p(lds_char* dst, const char* __restrict__ base, RowOff rowoff, int lane,
                                           int r0 = 0)
{
    static_assert(P <= 64 && 64 % P == 0, "rows of at most 64 pieces");
    constexpr int RPI = 64 / P;
    constexpr int NI = (R * P + 63) / 64;
    const unsigned lr = (unsigned)lane / P, lp = (unsigned)lane % P;
    lds_char* d0 = dst + r0 * P * 16;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const unsigned rl = i * RPI + lr;
        const unsigned r = (unsigned)r0 + rl;
        const unsigned p = lp ^ (unsigned)swz_key<P, KEY>((int)r);
        if ((R * P % 64 == 0 || rl < (unsigned)R) && !quad_piece<QS, RT, P>(r, p))
            __builtin_amdgcn_global_load_lds(base + rowoff(r) + p * 16, (lds_void*)(d0 + i * 1024), 16, 0, 0);
    }
}

template <int R, int P, typename RowOff>
__device__ __forceinline__ void dma_plain_p(lds_char* dst, const char* __restrict__ base, RowOff rowoff, int lane)
{
    constexpr int NI = (R * P + 63) / 64;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const unsigned s = i * 64 + (unsigned)lane;
        const unsigned r = s / P, p = s % P;
        if (R * P % 64 == 0 || r < (unsigned)R)
            __builtin_amdgcn_global_load_lds(base + rowoff(r) + p * 16, (lds_void*)(dst + i * 1024), 16, 0, 0);
    }
}

// Copy R rows of P plain 16-byte pieces (no swizzle).
template <int R, int P, typename RowOff>
__device__ __forceinline__ void dma_plain(uint32_t dst, const char* __restrict__ base, RowOff rowoff, int lane)
{
    constexpr int NI = (R * P + 63) / 64;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const unsigned s = i * 64 + (unsigned)lane;
        const unsigned r = s / P, p = s % P;
        if (R * P % 64 == 0 || r < (unsigned)R)
            __builtin_amdgcn_global_load_lds(base + rowoff(r) + p * 16, (lds_void*)(uintptr_t)(dst + i * 1024), 16, 0, 0);
    }
}


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

// V slab (plain rows of OW elements) as the B operand of T V for column tile
// ct, contraction step ks.
template <typename Tr, int OW> struct VOperand;
template <int OW> struct VOperand<TraitsBf16, OW> {
    static __device__ __forceinline__ bf16x8 load(const char* Vs, int ct, int ks, int lane) {
        // Transpose read: source lane s of group g points at row
        // 32ks + 8g + s/4 (+4 for the second half) and columns
        // 16ct + 4(s%4) .. +3, so lane i receives V[32ks + 8g + j][16ct + i]
        // for j = 0..3 (4..7): the contraction slots of lane group g.
        const int g = lane >> 4, s = lane & 15;
        const int r0 = 32 * ks + 8 * g + (s >> 2);
        const int b = 2 * (16 * ct + 4 * (s & 3));
        union { shortx4 h[2]; bf16x8 v; } f;
        f.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(Vs + r0 * OW * 2 + b));
        f.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(Vs + (r0 + 4) * OW * 2 + b));
        return f.v;
    }
};
template <int OW> struct VOperand<TraitsF32, OW> {
    static __device__ __forceinline__ float load(const char* Vs, int ct, int ks, int lane) {
        const int g = lane >> 4, m = lane & 15;
        const int r = 16 * (ks >> 2) + 4 * g + (ks & 3);
        return *reinterpret_cast<const float*>(Vs + 4 * (r * OW + 16 * ct + m));
    }
};

}  // namespace mdn
