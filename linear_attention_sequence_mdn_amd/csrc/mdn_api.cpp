// mdn_api.cpp -- C entry points declared in include/mdn.h.
//
// Every argument is validated here, on the host, before any HIP call: sizes,
// the compiled (dtype, head dim, chunk size) set, NULL pointers, 16-byte
// alignment, overlap between outputs and inputs, and workspace size.  A
// failed check returns its status and enqueues nothing.  Validated calls are
// handed to the launchers in mdn_step.hip / mdn_chunk.hip.
#include <algorithm>
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/mdn.h"
#include "mdn_internal.h"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;   // per tensor; keeps every offset in range

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
    const uintptr_t a = (uintptr_t)p;
    return Range{a, a + (uintptr_t)bytes};
}

bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > kMaxElems / a) return false;
    *out = a * b;
    return *out <= kMaxElems;
}

int64_t elem_size(int dtype) { return dtype == MDN_BF16 ? 2 : 4; }

// Shapes the chunk kernels are compiled for in the given element type.  The
// bf16 kernels tile every contraction in steps of 32 (the bf16 matrix-core
// op), so they need dk and C of at least 32.
bool dims_native_chunk(int dtype, int dk, int dv, int C) {
    if (dk != dv) return false;
    if (dtype == MDN_F32)
        return (dk == 16 || dk == 32 || dk == 64 || dk == 128) && (C == 16 || C == 32 || C == 64);
    if (dtype == MDN_BF16)
        return (dk == 32 || dk == 64 || dk == 128) && (C == 32 || C == 64);
    return false;
}

// bf16 calls at dk = 16 or C = 16: the fp32 kernels run on fp32 copies of
// the bf16 inputs (exact), and the outputs are rounded back to bf16.  The
// copies live in the workspace, after the fp32 call's own sections.
bool dims_widened_chunk(int dtype, int dk, int dv, int C) {
    return dtype == MDN_BF16 && !dims_native_chunk(dtype, dk, dv, C) && dims_native_chunk(MDN_F32, dk, dv, C);
}

bool dims_supported_chunk(int dtype, int dk, int dv, int C) {
    return dims_native_chunk(dtype, dk, dv, C) || dims_widened_chunk(dtype, dk, dv, C);
}

bool dims_supported_step(int dtype, int dk, int dv) {
    if (dtype != MDN_F32 && dtype != MDN_BF16) return false;
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct ChunkSizes {
    int64_t BH, NT, tok;         // tok = BH * T
    int64_t qk_elems, v_elems, g_elems, st_elems, tiles;
    int64_t nseq;                // packed batch: number of sequences; -1 for the [B,H,T,.] layout
};

int chunk_sizes(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, ChunkSizes* s) {
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0 || C <= 0) return MDN_ERR_BAD_SHAPE;
    if (!mul_ok(B, H, &s->BH) || !mul_ok(s->BH, T, &s->tok)) return MDN_ERR_BAD_SHAPE;
    s->NT = (T + C - 1) / C;
    if (!mul_ok(s->tok, dk, &s->qk_elems) || !mul_ok(s->tok, dv, &s->v_elems)) return MDN_ERR_BAD_SHAPE;
    s->g_elems = s->tok;
    int64_t dd;
    if (!mul_ok((int64_t)dk, (int64_t)dv, &dd) || !mul_ok(s->BH, dd, &s->st_elems)) return MDN_ERR_BAD_SHAPE;
    int64_t cc;
    if (!mul_ok(s->BH, s->NT, &s->tiles) || !mul_ok(s->tiles, (int64_t)C * C, &cc)) return MDN_ERR_BAD_SHAPE;
    // one workgroup per chunk tile / per column slab: keep the grids in range
    if (s->tiles > INT32_MAX || s->BH > INT32_MAX / 8) return MDN_ERR_BAD_SHAPE;
    s->nseq = -1;
    return MDN_OK;
}

// Packed variable-length batch: H heads of T packed tokens, nseq sequences;
// NT = T / C + nseq tile slots per head, states [nseq, H, dk, dv].
int varlen_sizes(int64_t H, int64_t T, int64_t nseq, int dk, int dv, int C, ChunkSizes* s) {
    if (H < 0 || T < 0 || nseq < 0 || dk <= 0 || dv <= 0 || C <= 0) return MDN_ERR_BAD_SHAPE;
    if (T > INT32_MAX || nseq > INT32_MAX - 1) return MDN_ERR_BAD_SHAPE;   // int32 sequence bounds
    s->BH = H;
    if (!mul_ok(H, T, &s->tok)) return MDN_ERR_BAD_SHAPE;
    s->NT = T / C + nseq;
    if (!mul_ok(s->tok, dk, &s->qk_elems) || !mul_ok(s->tok, dv, &s->v_elems)) return MDN_ERR_BAD_SHAPE;
    s->g_elems = s->tok;
    int64_t dd, units, cc;
    if (!mul_ok(nseq, H, &units) || !mul_ok((int64_t)dk, (int64_t)dv, &dd) || !mul_ok(units, dd, &s->st_elems))
        return MDN_ERR_BAD_SHAPE;
    if (!mul_ok(H, s->NT, &s->tiles) || !mul_ok(s->tiles, (int64_t)C * C, &cc)) return MDN_ERR_BAD_SHAPE;
    if (s->tiles > INT32_MAX || units > INT32_MAX / 8) return MDN_ERR_BAD_SHAPE;
    s->nseq = nseq;
    return MDN_OK;
}

// workspace: T and Aqk per tile slot, the coefficients, and for a packed
// batch the slot table and the dispatch order
size_t workspace_of(const ChunkSizes& s, int C, int dtype) {
    const size_t mat = align256((size_t)s.tiles * C * C * elem_size(dtype));
    const size_t cf = align256((size_t)s.tiles * MDN_COEF_ROWS * C * sizeof(float));
    const size_t tab = s.nseq >= 0 ? align256((size_t)s.NT * 2 * sizeof(int32_t)) : 0;
    const size_t perm = s.nseq >= 0 ? align256((size_t)s.nseq * sizeof(int32_t)) : 0;
    return 2 * mat + cf + tab + perm;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MDN_OK : MDN_ERR_HIP; }

// Widened forward (dims_widened_chunk): the fp32 call's workspace, then fp32
// q, k, v, O and vtilde (byte offsets).
struct WideFwd {
    size_t base, q, k, v, O, Vt, total;
};
WideFwd wide_fwd_sections(const ChunkSizes& s, int C) {
    WideFwd w;
    const size_t qk = align256((size_t)s.qk_elems * 4), vv = align256((size_t)s.v_elems * 4);
    w.base = workspace_of(s, C, MDN_F32);
    w.q = w.base;
    w.k = w.q + qk;
    w.v = w.k + qk;
    w.O = w.v + vv;
    w.Vt = w.O + vv;
    w.total = w.Vt + vv;
    return w;
}

size_t fwd_workspace(const ChunkSizes& s, int dk, int dv, int C, int dtype) {
    return dims_widened_chunk(dtype, dk, dv, C) ? wide_fwd_sections(s, C).total : workspace_of(s, C, dtype);
}

// Sequence split into P segments: after the forward's sections, two arrays
// (S, then M) of D x D fp32 state slots, BH (1 + 3 (P - 2)) written by the
// first pass and BH (P - 2) by the combine step: the bytes of one array in
// *out; false when the sizes do not fit.
bool split_state_bytes(const ChunkSizes& s, int dk, int dv, int P, size_t* out) {
    int64_t slots, elems;
    if (!mul_ok(s.BH, (int64_t)(1 + 4 * (P - 2)), &slots) || !mul_ok(slots, (int64_t)dk * dv, &elems) ||
        elems > kMaxElems)
        return false;
    *out = align256((size_t)elems * sizeof(float));
    return true;
}

// Segments mdn_chunk_fwd cuts each sequence into by itself (0: none).  The
// split pays where one pass leaves compute units idle.  Its first pass runs
// 1 + 3 (P - 2) units per head in slabs of two column tiles, d / 32
// workgroups per unit.  Measured (bf16, C = 64, d = 128 and d = 64, 1 to 32
// heads of 4096 to 65536 tokens), the best P is about the largest whose first
// pass fits the device in one round of workgroups, with segments of at
// least 32 chunks, or 64 where the three-segment first pass would fill more
// than half of the device (short segments then lose to the slower rate of a
// full device), and at most 12 (beyond, the combine steps in sequence cost
// more); two segments never paid.  E.g. on 256 compute units, d = 128: 16
// heads of 16384 tokens take 3 segments (0.40 against 0.44 ms), 4 heads of
// 32768 take 7 (0.36 against 0.65 ms), 2 of 65536 take 12 (0.47 against
// 1.27 ms); 16 heads of 8192 tokens keep the single pass.  d = 64: 16 heads
// of 8192 take 4 (0.13 against 0.15 ms), 8 of 32768 take 7 (about 0.30
// against 0.54 ms).  Taken for those two families only.
int auto_segments(const ChunkSizes& s, int dk, int dv, int C, int dtype) {
    if (s.nseq >= 0 || dtype != MDN_BF16 || dk != dv || (dk != 128 && dk != 64) || C != 64 || s.BH <= 0) return 0;
    const int64_t cus = mdn::device_compute_units();
    const int64_t w = dk / 32;                         // first-pass workgroups per unit
    const int64_t units = cus / (w * s.BH);            // first-pass units per head that fit one round
    int64_t P = units >= 1 ? (units - 1) / 3 + 2 : 0;
    const int64_t floor_chunks = 2 * (4 * w * s.BH) > cus ? 64 : 32;
    P = std::min<int64_t>(P, s.NT / floor_chunks);
    P = std::min<int64_t>(P, 12);
    return P >= 3 ? (int)P : 0;
}

}  // namespace

extern "C" {

const char* mdn_status_string(int status)
{
    switch (status) {
    case MDN_OK: return "MDN_OK";
    case MDN_ERR_NULL_ARG: return "MDN_ERR_NULL_ARG: a required pointer is NULL";
    case MDN_ERR_BAD_SHAPE: return "MDN_ERR_BAD_SHAPE: negative or overflowing size";
    case MDN_ERR_UNSUPPORTED: return "MDN_ERR_UNSUPPORTED: dtype, head dim or chunk size not compiled";
    case MDN_ERR_ALIAS: return "MDN_ERR_ALIAS: an output overlaps an input or another output";
    case MDN_ERR_WORKSPACE: return "MDN_ERR_WORKSPACE: workspace missing or too small";
    case MDN_ERR_ALIGN: return "MDN_ERR_ALIGN: a pointer is not 16-byte aligned";
    case MDN_ERR_HIP: return "MDN_ERR_HIP: a HIP launch or runtime call failed";
    case MDN_ERR_TOO_LARGE:
        return "MDN_ERR_TOO_LARGE: the problem needs more than the allocation-free entry point's static scratch";
    default: return "unknown mdn status";
    }
}

int mdn_abi_version(void) { return MDN_ABI_VERSION; }

size_t mdn_chunk_fwd_workspace_bytes(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype)
{
    ChunkSizes s;
    if (chunk_sizes(B, H, T, dk, dv, C, &s) != MDN_OK) return (size_t)-1;
    if (!dims_supported_chunk(dtype, dk, dv, C)) return (size_t)-1;
    const int P = auto_segments(s, dk, dv, C, dtype);
    size_t st;
    if (P > 0 && split_state_bytes(s, dk, dv, P, &st)) return workspace_of(s, C, dtype) + 2 * st;
    return fwd_workspace(s, dk, dv, C, dtype);
}

size_t mdn_chunk_fwd_varlen_workspace_bytes(int64_t H, int64_t T, int64_t nseq, int dk, int dv, int C, int dtype)
{
    ChunkSizes s;
    if (varlen_sizes(H, T, nseq, dk, dv, C, &s) != MDN_OK) return (size_t)-1;
    if (!dims_supported_chunk(dtype, dk, dv, C)) return (size_t)-1;
    return fwd_workspace(s, dk, dv, C, dtype);
}

// Backward workspace: the forward's sections (T^T and Aqk^T in place of T and
// Aqk, the coefficients), then per tile the chunk-start states S, M and the
// chunk-end adjoints dS, dM and the state-product parts of dq and dk (element
// type), and the coefficient adjoints (fp32).
struct BwdSections {
    size_t mat, cf, st, part, vec, total;
};

BwdSections bwd_sections(const ChunkSizes& s, int dk, int C, int dtype);

// Widened backward (dims_widened_chunk): the fp32 call's workspace, then fp32
// q, k, vtilde, dO (inputs) and dq, dk, dv (outputs), as byte offsets.
struct WideBwd {
    size_t base, q, k, Vt, dO, dq, dk, dv, total;
};
WideBwd wide_bwd_sections(const ChunkSizes& s, int dk, int C) {
    WideBwd w;
    const size_t qk = align256((size_t)s.qk_elems * 4), vv = align256((size_t)s.v_elems * 4);
    w.base = bwd_sections(s, dk, C, MDN_F32).total;
    w.q = w.base;
    w.k = w.q + qk;
    w.Vt = w.k + qk;
    w.dO = w.Vt + vv;
    w.dq = w.dO + vv;
    w.dk = w.dq + qk;
    w.dv = w.dk + qk;
    w.total = w.dv + vv;
    return w;
}

BwdSections bwd_sections(const ChunkSizes& s, int dk, int C, int dtype) {
    BwdSections b;
    const size_t es = (size_t)elem_size(dtype);
    b.mat = align256((size_t)s.tiles * C * C * es);
    b.cf = align256((size_t)s.tiles * MDN_COEF_ROWS * C * sizeof(float));
    b.st = align256((size_t)s.tiles * dk * dk * es);
    b.part = align256((size_t)s.tiles * C * dk * es);
    b.vec = align256((size_t)s.tiles * mdn::MDN_BWD_VEC_ROWS * C * sizeof(float));
    b.total = 2 * b.mat + b.cf + 4 * b.st + 2 * b.part + b.vec;
    return b;
}

// Validation shared by mdn_chunk_fwd, its two stages and the packed-batch
// forward (s.nseq >= 0, sequence bounds cu).  `stage` is 3 (both), 1 (intra
// only) or 2 (inter only); only the pointers a stage reads or writes are
// required.  With `wide` the call is a widened bf16 forward: it is checked
// against the widened workspace size, and the kernel arguments are not used
// (the fp32 call is prepared from the workspace copies).
static int chunk_prepare(int stage, const ChunkSizes& s, int64_t T, int dk, int dv, int C, int dtype,
                         const int32_t* cu,
                         const void* q, const void* k, const void* v,
                         const float* alpha, const float* mu, const float* beta, const float* eta,
                         const float* S0, const float* M0,
                         void* O, float* S_T, float* M_T, void* Vtilde,
                         void* workspace, size_t workspace_bytes, void* stream,
                         mdn::ChunkArgs* a, bool* empty, bool wide = false, bool no_workspace = false,
                         size_t extra = 0)
{
    if (wide ? !dims_widened_chunk(dtype, dk, dv, C) : !dims_native_chunk(dtype, dk, dv, C))
        return MDN_ERR_UNSUPPORTED;
    const bool packed = s.nseq >= 0;
    *empty = s.BH == 0 || s.nseq == 0;
    if (*empty) return MDN_OK;
    if (packed && !cu) return MDN_ERR_NULL_ARG;
    if (packed && ((uintptr_t)cu & 3u) != 0) return MDN_ERR_ALIGN;

    const int64_t es = elem_size(dtype);
    const bool seq = s.tok > 0;
    const bool inter = (stage & 2) != 0;
    if (inter && (!S_T || !M_T)) return MDN_ERR_NULL_ARG;
    if (seq && (!q || !k || !alpha || !mu || !beta || !eta)) return MDN_ERR_NULL_ARG;
    if (seq && inter && (!v || !O || !Vtilde)) return MDN_ERR_NULL_ARG;
    const size_t need = (no_workspace ? 0 : wide ? wide_fwd_sections(s, C).total : workspace_of(s, C, dtype)) + extra;
    if (need > 0 && (!workspace || workspace_bytes < need)) return MDN_ERR_WORKSPACE;

    const void* all[] = {q, k, v, alpha, mu, beta, eta, S0, M0, O, S_T, M_T, Vtilde, workspace};
    for (const void* p : all)
        if (p && !aligned16(p)) return MDN_ERR_ALIGN;

    const Range rq = range_of(q, s.qk_elems * es), rk = range_of(k, s.qk_elems * es);
    const Range rv = range_of(v, s.v_elems * es);
    const Range ra = range_of(alpha, s.g_elems * 4), rm = range_of(mu, s.g_elems * 4);
    const Range rb = range_of(beta, s.g_elems * 4), re = range_of(eta, s.g_elems * 4);
    const Range rs0 = range_of(S0, S0 ? s.st_elems * 4 : 0), rm0 = range_of(M0, M0 ? s.st_elems * 4 : 0);
    const Range rO = range_of(O, O ? s.v_elems * es : 0), rVt = range_of(Vtilde, Vtilde ? s.v_elems * es : 0);
    const Range rST = range_of(S_T, S_T ? s.st_elems * 4 : 0), rMT = range_of(M_T, M_T ? s.st_elems * 4 : 0);
    const Range rW = range_of(workspace, (int64_t)need);
    const Range rcu = range_of(cu, packed ? (s.nseq + 1) * 4 : 0);
    const Range ins[] = {rq, rk, rv, ra, rm, rb, re, rs0, rm0, rcu};
    const Range outs[] = {rO, rVt, rST, rMT, rW};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 10; ++j) {
            if (!overlap(outs[i], ins[j])) continue;
            // the states may be updated in place, as exact aliases only
            if (i == 2 && j == 7 && (const void*)S_T == (const void*)S0) continue;
            if (i == 3 && j == 8 && (const void*)M_T == (const void*)M0) continue;
            return MDN_ERR_ALIAS;
        }
        for (int j = i + 1; j < 5; ++j)
            if (overlap(outs[i], outs[j])) return MDN_ERR_ALIAS;
    }

    memset(a, 0, sizeof(*a));
    a->BH = s.BH; a->T = T; a->NT = s.NT;
    a->cu = packed ? cu : nullptr;
    a->nseq = packed ? s.nseq : 0;
    a->dk = dk; a->dv = dv; a->C = C; a->dtype = dtype;
    a->q = q; a->k = k; a->v = v;
    a->alpha = alpha; a->mu = mu; a->beta = beta; a->eta = eta;
    a->S0 = S0; a->M0 = M0;
    a->O = O; a->ST = S_T; a->MT = M_T; a->Vt = Vtilde;
    const size_t mat = align256((size_t)s.tiles * C * C * es);
    a->Tmat = workspace;
    a->Aqk = workspace ? (char*)workspace + mat : nullptr;
    a->coef = workspace ? (float*)((char*)workspace + 2 * mat) : nullptr;
    const size_t cfb = align256((size_t)s.tiles * MDN_COEF_ROWS * C * sizeof(float));
    a->tab = packed ? (int32_t*)((char*)workspace + 2 * mat + cfb) : nullptr;
    a->perm = packed ? (int32_t*)((char*)workspace + 2 * mat + cfb + align256((size_t)s.NT * 2 * sizeof(int32_t)))
                     : nullptr;
    a->gamma = nullptr;
    a->stream = stream;
    return MDN_OK;
}

// The launches of a prepared forward (plain or packed batch).
static int fwd_launch(const mdn::ChunkArgs& a, int64_t T)
{
    int st;
    if (a.cu) {
        st = hip_status(mdn::launch_varlen_prep(a));
        if (st != MDN_OK) return st;
    }
    if (T > 0) {
        st = hip_status(mdn::launch_chunk_intra(a));
        if (st != MDN_OK) return st;
    }
    return hip_status(mdn::launch_chunk_inter(a));
}

// Widened bf16 forward: the caller's arguments are checked as a bf16 call,
// q, k and v are widened into the workspace, the fp32 forward runs on them
// (its own workspace sections first), and O and vtilde are rounded back.
static int fwd_widened(const ChunkSizes& s, int64_t T, int dk, int dv, int C, const int32_t* cu,
                       const void* q, const void* k, const void* v,
                       const float* alpha, const float* mu, const float* beta, const float* eta,
                       const float* S0, const float* M0,
                       void* O, float* S_T, float* M_T, void* Vtilde,
                       void* workspace, size_t workspace_bytes, void* stream)
{
    mdn::ChunkArgs a;
    bool empty = false;
    int st = chunk_prepare(3, s, T, dk, dv, C, MDN_BF16, cu, q, k, v, alpha, mu, beta, eta, S0, M0,
                           O, S_T, M_T, Vtilde, workspace, workspace_bytes, stream, &a, &empty, true);
    if (st != MDN_OK || empty) return st;
    const WideFwd w = wide_fwd_sections(s, C);
    char* ws = (char*)workspace;
    const bool seq = s.tok > 0;
    float* q32 = seq ? (float*)(ws + w.q) : nullptr;
    float* k32 = seq ? (float*)(ws + w.k) : nullptr;
    float* v32 = seq ? (float*)(ws + w.v) : nullptr;
    float* O32 = seq ? (float*)(ws + w.O) : nullptr;
    float* Vt32 = seq ? (float*)(ws + w.Vt) : nullptr;
    if (seq) {
        st = hip_status(mdn::launch_convert(q, MDN_BF16, q32, s.qk_elems, stream));
        if (st == MDN_OK) st = hip_status(mdn::launch_convert(k, MDN_BF16, k32, s.qk_elems, stream));
        if (st == MDN_OK) st = hip_status(mdn::launch_convert(v, MDN_BF16, v32, s.v_elems, stream));
        if (st != MDN_OK) return st;
    }
    mdn::ChunkArgs b;
    st = chunk_prepare(3, s, T, dk, dv, C, MDN_F32, cu, q32, k32, v32, alpha, mu, beta, eta, S0, M0,
                       O32, S_T, M_T, Vt32, w.base ? ws : nullptr, w.base, stream, &b, &empty);
    if (st != MDN_OK || empty) return st;
    st = fwd_launch(b, T);
    if (st != MDN_OK || !seq) return st;
    st = hip_status(mdn::launch_convert(O32, MDN_F32, O, s.v_elems, stream));
    if (st != MDN_OK) return st;
    return hip_status(mdn::launch_convert(Vt32, MDN_F32, Vtilde, s.v_elems, stream));
}

// The split forward on validated sizes (native dims, 2 <= nseg <= max).
static int fwd_split(const ChunkSizes& s, int64_t T, int dk, int dv, int C, int dtype, int nseg,
                     const void* q, const void* k, const void* v,
                     const float* alpha, const float* mu, const float* beta, const float* eta,
                     const float* S0, const float* M0,
                     void* O, float* S_T, float* M_T, void* Vtilde,
                     void* workspace, size_t workspace_bytes, void* stream)
{
    int64_t units;
    if (!mul_ok(s.BH, (int64_t)(1 + 3 * (nseg - 2)), &units) || units > INT32_MAX / 8) return MDN_ERR_BAD_SHAPE;
    size_t stb;
    if (!split_state_bytes(s, dk, dv, nseg, &stb)) return MDN_ERR_BAD_SHAPE;
    mdn::ChunkArgs a;
    bool empty = false;
    int st = chunk_prepare(3, s, T, dk, dv, C, dtype, nullptr, q, k, v, alpha, mu, beta, eta, S0, M0,
                           O, S_T, M_T, Vtilde, workspace, workspace_bytes, stream, &a, &empty, false, false, 2 * stb);
    if (st != MDN_OK || empty) return st;
    float* segS = (float*)((char*)workspace + workspace_of(s, C, dtype));
    float* segM = (float*)((char*)segS + stb);
    if (T > 0) {
        st = hip_status(mdn::launch_chunk_intra(a));
        if (st != MDN_OK) return st;
    }
    return hip_status(mdn::launch_chunk_inter_split(a, nseg, segS, segM));
}

// mdn_chunk_fwd; with allow_split it takes the sequence split where
// auto_segments chooses it and the workspace holds the split's state slots.
static int chunk_fwd_impl(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                          const void* q, const void* k, const void* v,
                          const float* alpha, const float* mu, const float* beta, const float* eta,
                          const float* S0, const float* M0,
                          void* O, float* S_T, float* M_T, void* Vtilde,
                          void* workspace, size_t workspace_bytes, void* stream, bool allow_split)
{
    mdn::ChunkArgs a;
    bool empty = false;
    ChunkSizes s;
    int st = chunk_sizes(B, H, T, dk, dv, C, &s);
    if (st != MDN_OK) return st;
    if (allow_split && dims_native_chunk(dtype, dk, dv, C)) {
        const int P = auto_segments(s, dk, dv, C, dtype);
        size_t stb;
        if (P > 0 && split_state_bytes(s, dk, dv, P, &stb) && workspace_bytes >= workspace_of(s, C, dtype) + 2 * stb)
            return fwd_split(s, T, dk, dv, C, dtype, P, q, k, v, alpha, mu, beta, eta, S0, M0, O, S_T, M_T, Vtilde,
                             workspace, workspace_bytes, stream);
    }
    if (dims_widened_chunk(dtype, dk, dv, C))
        return fwd_widened(s, T, dk, dv, C, nullptr, q, k, v, alpha, mu, beta, eta, S0, M0, O, S_T, M_T, Vtilde,
                           workspace, workspace_bytes, stream);
    st = chunk_prepare(3, s, T, dk, dv, C, dtype, nullptr, q, k, v, alpha, mu, beta, eta, S0, M0,
                       O, S_T, M_T, Vtilde, workspace, workspace_bytes, stream, &a, &empty);
    if (st != MDN_OK || empty) return st;
    return fwd_launch(a, T);
}

int mdn_chunk_fwd(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                  const void* q, const void* k, const void* v,
                  const float* alpha, const float* mu, const float* beta, const float* eta,
                  const float* S0, const float* M0,
                  void* O, float* S_T, float* M_T, void* Vtilde,
                  void* workspace, size_t workspace_bytes, void* stream)
{
    return chunk_fwd_impl(B, H, T, dk, dv, C, dtype, q, k, v, alpha, mu, beta, eta, S0, M0, O, S_T, M_T, Vtilde,
                          workspace, workspace_bytes, stream, true);
}

size_t mdn_chunk_fwd_split_workspace_bytes(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                                           int nseg)
{
    ChunkSizes s;
    if (chunk_sizes(B, H, T, dk, dv, C, &s) != MDN_OK) return (size_t)-1;
    if (!dims_native_chunk(dtype, dk, dv, C) || nseg < 2 || nseg > MDN_SPLIT_MAX_SEGMENTS) return (size_t)-1;
    size_t st;
    if (!split_state_bytes(s, dk, dv, nseg, &st)) return (size_t)-1;
    return workspace_of(s, C, dtype) + 2 * st;
}

// The forward with each sequence cut into nseg segments that run side by
// side: pass 1, the combine step, pass 2 (launch_chunk_inter_split).
int mdn_chunk_fwd_split(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype, int nseg,
                        const void* q, const void* k, const void* v,
                        const float* alpha, const float* mu, const float* beta, const float* eta,
                        const float* S0, const float* M0,
                        void* O, float* S_T, float* M_T, void* Vtilde,
                        void* workspace, size_t workspace_bytes, void* stream)
{
    ChunkSizes s;
    int st = chunk_sizes(B, H, T, dk, dv, C, &s);
    if (st != MDN_OK) return st;
    if (!dims_native_chunk(dtype, dk, dv, C) || nseg < 2 || nseg > MDN_SPLIT_MAX_SEGMENTS)
        return MDN_ERR_UNSUPPORTED;
    return fwd_split(s, T, dk, dv, C, dtype, nseg, q, k, v, alpha, mu, beta, eta, S0, M0, O, S_T, M_T, Vtilde,
                     workspace, workspace_bytes, stream);
}

// The whole forward in one kernel (no workspace): bf16, C = 64, dk = dv in
// {64, 128}.
int mdn_chunk_fwd_fused(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                        const void* q, const void* k, const void* v,
                        const float* alpha, const float* mu, const float* beta, const float* eta,
                        const float* S0, const float* M0,
                        void* O, float* S_T, float* M_T, void* Vtilde, void* stream)
{
    mdn::ChunkArgs a;
    bool empty = false;
    ChunkSizes s;
    int st = chunk_sizes(B, H, T, dk, dv, C, &s);
    if (st != MDN_OK) return st;
    if (!(dtype == MDN_BF16 && C == 64 && dk == dv && (dk == 64 || dk == 128))) return MDN_ERR_UNSUPPORTED;
    st = chunk_prepare(3, s, T, dk, dv, C, dtype, nullptr, q, k, v, alpha, mu, beta, eta, S0, M0,
                       O, S_T, M_T, Vtilde, nullptr, 0, stream, &a, &empty, false, true);
    if (st != MDN_OK || empty) return st;
    if (!mdn::fwd_fused_supported(a)) return MDN_ERR_UNSUPPORTED;
    return hip_status(mdn::launch_chunk_fwd_fused(a));
}

// ---------------------------------------------------------------------------
// Allocation-free forward.  The chunk forward's workspace (T, Aqk and the
// coefficient rows of every chunk tile) lives in a file-scope device array
// instead of a caller buffer.  Each GPU holds its own copy of the array, at
// its own address, for the life of the process.  In host code `scratch`
// names a host-side stand-in, never the device memory: the device address
// is taken once per device with hipGetSymbolAddress (with that device
// current) and only that address is handed to the kernels.
// ---------------------------------------------------------------------------
static __device__ __attribute__((aligned(256))) unsigned char scratch[MDN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void* scratch_dev[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// Device address of this device's `scratch` (looked up on the first call
// on the device, then kept).
int scratch_of_current_device(void** p) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MDN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MDN_ERR_UNSUPPORTED;
    std::call_once(scratch_once[dev], [dev]() {
        void* ptr = nullptr;
        scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        scratch_dev[dev] = scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    if (scratch_err[dev] != hipSuccess || !scratch_dev[dev]) return MDN_ERR_HIP;
    *p = scratch_dev[dev];
    return MDN_OK;
}
}  // namespace

int mdn_chunk_fwd_noalloc(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                          const void* q, const void* k, const void* v,
                          const float* alpha, const float* mu, const float* beta, const float* eta,
                          const float* S0, const float* M0,
                          void* O, float* S_T, float* M_T, void* Vtilde, void* stream)
{
    ChunkSizes s;
    int st = chunk_sizes(B, H, T, dk, dv, C, &s);
    if (st != MDN_OK) return st;
    if (!dims_supported_chunk(dtype, dk, dv, C)) return MDN_ERR_UNSUPPORTED;
    const size_t need = fwd_workspace(s, dk, dv, C, dtype);
    if (need > (size_t)MDN_NOALLOC_SCRATCH_BYTES) return MDN_ERR_TOO_LARGE;
    void* ws = nullptr;
    if (need > 0) {
        st = scratch_of_current_device(&ws);
        if (st != MDN_OK) return st;
    }
    // the kernels write every byte of the workspace they read, so nothing
    // left by an earlier call needs clearing
    return chunk_fwd_impl(B, H, T, dk, dv, C, dtype, q, k, v, alpha, mu, beta, eta, S0, M0, O, S_T, M_T, Vtilde,
                          ws, ws ? (size_t)MDN_NOALLOC_SCRATCH_BYTES : 0, stream, false);
}

int mdn_chunk_intra(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                    const void* q, const void* k,
                    const float* alpha, const float* mu, const float* beta, const float* eta,
                    void* workspace, size_t workspace_bytes, void* stream)
{
    mdn::ChunkArgs a;
    bool empty = false;
    ChunkSizes s;
    int st = chunk_sizes(B, H, T, dk, dv, C, &s);
    if (st != MDN_OK) return st;
    st = chunk_prepare(1, s, T, dk, dv, C, dtype, nullptr, q, k, nullptr, alpha, mu, beta, eta,
                       nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                       workspace, workspace_bytes, stream, &a, &empty);
    if (st != MDN_OK || empty || T == 0) return st;
    return hip_status(mdn::launch_chunk_intra(a));
}

int mdn_chunk_inter(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                    const void* q, const void* k, const void* v,
                    const float* alpha, const float* mu, const float* beta, const float* eta,
                    const float* S0, const float* M0,
                    void* O, float* S_T, float* M_T, void* Vtilde,
                    void* workspace, size_t workspace_bytes, void* stream)
{
    mdn::ChunkArgs a;
    bool empty = false;
    ChunkSizes s;
    int st = chunk_sizes(B, H, T, dk, dv, C, &s);
    if (st != MDN_OK) return st;
    st = chunk_prepare(2, s, T, dk, dv, C, dtype, nullptr, q, k, v, alpha, mu, beta, eta, S0, M0,
                       O, S_T, M_T, Vtilde, workspace, workspace_bytes, stream, &a, &empty);
    if (st != MDN_OK || empty) return st;
    return hip_status(mdn::launch_chunk_inter(a));
}

size_t mdn_chunk_bwd_workspace_bytes(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype)
{
    ChunkSizes s;
    if (chunk_sizes(B, H, T, dk, dv, C, &s) != MDN_OK) return (size_t)-1;
    if (!dims_supported_chunk(dtype, dk, dv, C)) return (size_t)-1;
    int64_t x;
    if (!mul_ok(s.tiles, (int64_t)dk * dk, &x)) return (size_t)-1;
    return dims_widened_chunk(dtype, dk, dv, C) ? wide_bwd_sections(s, dk, C).total : bwd_sections(s, dk, C, dtype).total;
}

// The launches of a checked backward call (element type dtype, natively
// compiled shape); `workspace` holds bwd_sections(s, dk, C, dtype).
static int bwd_launch(const ChunkSizes& s, int64_t T, int dk, int dv, int C, int dtype,
                      const void* q, const void* k,
                      const float* alpha, const float* mu, const float* beta, const float* eta,
                      const float* S0, const float* M0, const void* Vtilde,
                      const void* dO, const float* dS_T, const float* dM_T,
                      void* dq, void* dk_out, void* dv_out,
                      float* dalpha, float* dmu, float* dbeta, float* deta, float* dS0, float* dM0,
                      void* workspace, void* stream)
{
    const BwdSections sec = bwd_sections(s, dk, C, dtype);
    mdn::BwdArgs a;
    memset(&a, 0, sizeof(a));
    mdn::ChunkArgs& f = a.f;
    f.BH = s.BH; f.T = T; f.NT = s.NT;
    f.dk = dk; f.dv = dv; f.C = C; f.dtype = dtype;
    f.q = q; f.k = k;
    f.alpha = alpha; f.mu = mu; f.beta = beta; f.eta = eta;
    f.S0 = S0; f.M0 = M0;
    char* w = (char*)workspace;
    f.Tmat = w;
    f.Aqk = w + sec.mat;
    f.coef = (float*)(w + 2 * sec.mat);
    f.trans = true;
    f.stream = stream;
    char* st0 = w + 2 * sec.mat + sec.cf;
    a.Sst = st0; a.Mst = st0 + sec.st; a.dSst = st0 + 2 * sec.st; a.dMst = st0 + 3 * sec.st;
    a.dqp = st0 + 4 * sec.st;
    a.dkp = st0 + 4 * sec.st + sec.part;
    a.vec = (float*)(st0 + 4 * sec.st + 2 * sec.part);
    a.Vt = Vtilde; a.dO = dO; a.dST = dS_T; a.dMT = dM_T;
    a.dq = dq; a.dk = dk_out; a.dv = dv_out;
    a.dalpha = dalpha; a.dmu = dmu; a.dbeta = dbeta; a.deta = deta;
    a.dS0 = dS0; a.dM0 = dM0;
    return hip_status(mdn::launch_bwd(a));
}

int mdn_chunk_bwd(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                  const void* q, const void* k,
                  const float* alpha, const float* mu, const float* beta, const float* eta,
                  const float* S0, const float* M0, const void* Vtilde,
                  const void* dO, const float* dS_T, const float* dM_T,
                  void* dq, void* dk_out, void* dv_out,
                  float* dalpha, float* dmu, float* dbeta, float* deta, float* dS0, float* dM0,
                  void* workspace, size_t workspace_bytes, void* stream)
{
    ChunkSizes s;
    int st = chunk_sizes(B, H, T, dk, dv, C, &s);
    if (st != MDN_OK) return st;
    const bool wide = dims_widened_chunk(dtype, dk, dv, C);
    if (!wide && !dims_native_chunk(dtype, dk, dv, C)) return MDN_ERR_UNSUPPORTED;
    int64_t x;
    if (!mul_ok(s.tiles, (int64_t)dk * dk, &x)) return MDN_ERR_BAD_SHAPE;
    if (s.BH == 0) return MDN_OK;
    const bool seq = s.tok > 0;
    if (!dS0 || !dM0) return MDN_ERR_NULL_ARG;
    if (seq && (!q || !k || !alpha || !mu || !beta || !eta || !Vtilde || !dO || !dq || !dk_out || !dv_out ||
                !dalpha || !dmu || !dbeta || !deta))
        return MDN_ERR_NULL_ARG;
    const size_t need = wide ? wide_bwd_sections(s, dk, C).total : bwd_sections(s, dk, C, dtype).total;
    if (need > 0 && (!workspace || workspace_bytes < need)) return MDN_ERR_WORKSPACE;
    const void* all[] = {q, k, alpha, mu, beta, eta, S0, M0, Vtilde, dO, dS_T, dM_T,
                         dq, dk_out, dv_out, dalpha, dmu, dbeta, deta, dS0, dM0, workspace};
    for (const void* p : all)
        if (p && !aligned16(p)) return MDN_ERR_ALIGN;
    const int64_t es = elem_size(dtype);
    const Range ins[] = {range_of(q, s.qk_elems * es), range_of(k, s.qk_elems * es),
                         range_of(alpha, s.g_elems * 4), range_of(mu, s.g_elems * 4),
                         range_of(beta, s.g_elems * 4), range_of(eta, s.g_elems * 4),
                         range_of(S0, S0 ? s.st_elems * 4 : 0), range_of(M0, M0 ? s.st_elems * 4 : 0),
                         range_of(Vtilde, s.v_elems * es), range_of(dO, s.v_elems * es),
                         range_of(dS_T, dS_T ? s.st_elems * 4 : 0), range_of(dM_T, dM_T ? s.st_elems * 4 : 0)};
    const Range outs[] = {range_of(dq, s.qk_elems * es), range_of(dk_out, s.qk_elems * es),
                          range_of(dv_out, s.v_elems * es), range_of(dalpha, s.g_elems * 4),
                          range_of(dmu, s.g_elems * 4), range_of(dbeta, s.g_elems * 4),
                          range_of(deta, s.g_elems * 4), range_of(dS0, s.st_elems * 4),
                          range_of(dM0, s.st_elems * 4), range_of(workspace, (int64_t)need)};
    constexpr int NI = sizeof(ins) / sizeof(ins[0]), NO = sizeof(outs) / sizeof(outs[0]);
    for (int i = 0; i < NO; ++i) {
        for (int j = 0; j < NI; ++j)
            if (overlap(outs[i], ins[j])) return MDN_ERR_ALIAS;
        for (int j = i + 1; j < NO; ++j)
            if (overlap(outs[i], outs[j])) return MDN_ERR_ALIAS;
    }

    if (!wide)
        return bwd_launch(s, T, dk, dv, C, dtype, q, k, alpha, mu, beta, eta, S0, M0, Vtilde, dO, dS_T, dM_T,
                          dq, dk_out, dv_out, dalpha, dmu, dbeta, deta, dS0, dM0, workspace, stream);
    // widened bf16 call: fp32 copies of q, k, vtilde and dO, the fp32
    // backward on them, and dq, dk, dv rounded back
    const WideBwd w = wide_bwd_sections(s, dk, C);
    char* ws = (char*)workspace;
    void* q32 = seq ? ws + w.q : nullptr;
    void* k32 = seq ? ws + w.k : nullptr;
    void* Vt32 = seq ? ws + w.Vt : nullptr;
    void* dO32 = seq ? ws + w.dO : nullptr;
    void* dq32 = seq ? ws + w.dq : nullptr;
    void* dk32 = seq ? ws + w.dk : nullptr;
    void* dv32 = seq ? ws + w.dv : nullptr;
    int st2 = MDN_OK;
    if (seq) {
        st2 = hip_status(mdn::launch_convert(q, MDN_BF16, q32, s.qk_elems, stream));
        if (st2 == MDN_OK) st2 = hip_status(mdn::launch_convert(k, MDN_BF16, k32, s.qk_elems, stream));
        if (st2 == MDN_OK) st2 = hip_status(mdn::launch_convert(Vtilde, MDN_BF16, Vt32, s.v_elems, stream));
        if (st2 == MDN_OK) st2 = hip_status(mdn::launch_convert(dO, MDN_BF16, dO32, s.v_elems, stream));
        if (st2 != MDN_OK) return st2;
    }
    st2 = bwd_launch(s, T, dk, dv, C, MDN_F32, q32, k32, alpha, mu, beta, eta, S0, M0, Vt32, dO32, dS_T, dM_T,
                     dq32, dk32, dv32, dalpha, dmu, dbeta, deta, dS0, dM0, w.base ? ws : nullptr, stream);
    if (st2 != MDN_OK || !seq) return st2;
    st2 = hip_status(mdn::launch_convert(dq32, MDN_F32, dq, s.qk_elems, stream));
    if (st2 == MDN_OK) st2 = hip_status(mdn::launch_convert(dk32, MDN_F32, dk_out, s.qk_elems, stream));
    if (st2 == MDN_OK) st2 = hip_status(mdn::launch_convert(dv32, MDN_F32, dv_out, s.v_elems, stream));
    return st2;
}

int mdn_chunk_fwd_varlen(int64_t H, int64_t T, int64_t nseq, const int32_t* cu_seqlens,
                         int dk, int dv, int C, int dtype,
                         const void* q, const void* k, const void* v,
                         const float* alpha, const float* mu, const float* beta, const float* eta,
                         const float* S0, const float* M0,
                         void* O, float* S_T, float* M_T, void* Vtilde,
                         void* workspace, size_t workspace_bytes, void* stream)
{
    mdn::ChunkArgs a;
    bool empty = false;
    ChunkSizes s;
    int st = varlen_sizes(H, T, nseq, dk, dv, C, &s);
    if (st != MDN_OK) return st;
    if (dims_widened_chunk(dtype, dk, dv, C))
        return fwd_widened(s, T, dk, dv, C, cu_seqlens, q, k, v, alpha, mu, beta, eta, S0, M0, O, S_T, M_T,
                           Vtilde, workspace, workspace_bytes, stream);
    st = chunk_prepare(3, s, T, dk, dv, C, dtype, cu_seqlens, q, k, v, alpha, mu, beta, eta, S0, M0,
                       O, S_T, M_T, Vtilde, workspace, workspace_bytes, stream, &a, &empty);
    if (st != MDN_OK || empty) return st;
    return fwd_launch(a, T);
}

int mdn_step(int64_t B, int64_t H, int dk, int dv, int dtype,
             const void* q, const void* k, const void* v,
             const float* alpha, const float* mu, const float* beta, const float* eta,
             float* S, float* M, void* o, void* stream)
{
    int64_t BH, qe, ve, se, dd;
    if (B < 0 || H < 0 || dk <= 0 || dv <= 0) return MDN_ERR_BAD_SHAPE;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, dk, &qe) || !mul_ok(BH, dv, &ve)) return MDN_ERR_BAD_SHAPE;
    if (!mul_ok((int64_t)dk, (int64_t)dv, &dd) || !mul_ok(BH, dd, &se)) return MDN_ERR_BAD_SHAPE;
    if (BH > INT32_MAX) return MDN_ERR_BAD_SHAPE;
    if (!dims_supported_step(dtype, dk, dv)) return MDN_ERR_UNSUPPORTED;
    if (BH == 0) return MDN_OK;
    if (!q || !k || !v || !alpha || !mu || !beta || !eta || !S || !M || !o) return MDN_ERR_NULL_ARG;
    const void* all[] = {q, k, v, alpha, mu, beta, eta, S, M, o};
    for (const void* p : all)
        if (!aligned16(p)) return MDN_ERR_ALIGN;
    const int64_t es = elem_size(dtype);
    const Range rS = range_of(S, se * 4), rM = range_of(M, se * 4), ro = range_of(o, ve * es);
    const Range others[] = {range_of(q, qe * es), range_of(k, qe * es), range_of(v, ve * es),
                            range_of(alpha, BH * 4), range_of(mu, BH * 4), range_of(beta, BH * 4),
                            range_of(eta, BH * 4)};
    if (overlap(rS, rM) || overlap(rS, ro) || overlap(rM, ro)) return MDN_ERR_ALIAS;
    for (const Range& r : others)
        if (overlap(rS, r) || overlap(rM, r) || overlap(ro, r)) return MDN_ERR_ALIAS;

    mdn::StepArgs a;
    a.BH = BH; a.dk = dk; a.dv = dv; a.dtype = dtype;
    a.q = q; a.k = k; a.v = v;
    a.alpha = alpha; a.mu = mu; a.beta = beta; a.eta = eta;
    a.S = S; a.M = M; a.o = o; a.stream = stream;
    return hip_status(mdn::launch_step(a));
}

int mdn_stream_rw(void* buf, int64_t bytes, float scale, void* stream)
{
    if (bytes < 0 || bytes % 16 != 0 || bytes / 16 > (int64_t)INT32_MAX * 4096) return MDN_ERR_BAD_SHAPE;
    if (bytes == 0) return MDN_OK;
    if (!buf) return MDN_ERR_NULL_ARG;
    if (!aligned16(buf)) return MDN_ERR_ALIGN;
    return hip_status(mdn::launch_stream_rw(buf, bytes / 16, scale, stream));
}

int mdn_gates(int64_t B, int64_t H, int64_t T, int dk, int dtype, float s, float mu_log_min,
              const float* x, const float* a, const float* b, const float* mu_log,
              float* alpha, float* mu, float* beta, float* eta,
              const void* q, const void* k, const float* d, void* q_out, void* stream)
{
    int64_t BH, N;
    if (B < 0 || H < 0 || T < 0 || !mul_ok(B, H, &BH) || !mul_ok(BH, T, &N)) return MDN_ERR_BAD_SHAPE;
    if (!(s > 0.f) || !(s < INFINITY) || !(mu_log_min <= 0.f) || !(mu_log_min > -INFINITY)) return MDN_ERR_BAD_SHAPE;
    if (dtype != MDN_F32 && dtype != MDN_BF16) return MDN_ERR_UNSUPPORTED;
    const bool corr = q || k || d || q_out;
    if (corr && (!q || !k || !d || !q_out)) return MDN_ERR_NULL_ARG;
    if (corr && dk != 16 && dk != 32 && dk != 64 && dk != 128) return MDN_ERR_UNSUPPORTED;
    if (N == 0) return MDN_OK;
    if (!x || !a || !b || !mu_log || !alpha || !mu || !beta || !eta) return MDN_ERR_NULL_ARG;
    const void* all[] = {x, a, b, mu_log, alpha, mu, beta, eta, q, k, d, q_out};
    for (const void* p : all)
        if (p && !aligned16(p)) return MDN_ERR_ALIGN;
    int64_t nq = 0;
    if (corr && !mul_ok(N, (int64_t)dk, &nq)) return MDN_ERR_BAD_SHAPE;
    const int64_t es = elem_size(dtype);
    const Range ins[] = {range_of(x, N * 4), range_of(a, N * 4), range_of(b, N * 4), range_of(mu_log, N * 4),
                         range_of(q, nq * es), range_of(k, nq * es), range_of(d, corr ? H * 4 : 0)};
    const Range outs[] = {range_of(alpha, N * 4), range_of(mu, N * 4), range_of(beta, N * 4),
                          range_of(eta, N * 4), range_of(q_out, nq * es)};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 7; ++j) {
            if (!overlap(outs[i], ins[j])) continue;
            if (i == 4 && j == 4 && q_out == q) continue;      // in-place correction
            return MDN_ERR_ALIAS;
        }
        for (int j = i + 1; j < 5; ++j)
            if (overlap(outs[i], outs[j])) return MDN_ERR_ALIAS;
    }
    mdn::GateArgs g;
    memset(&g, 0, sizeof(g));
    g.N = N; g.T = T; g.H = H; g.dk = dk; g.dtype = dtype; g.s = s; g.mu_log_min = mu_log_min;
    g.x = x; g.a = a; g.b = b; g.mu_log = mu_log;
    g.alpha = alpha; g.mu = mu; g.beta = beta; g.eta = eta;
    g.q = q; g.k = k; g.d = d; g.qo = q_out; g.stream = stream;
    return hip_status(mdn::launch_gates(g));
}

int mdn_chunk_coef(int64_t B, int64_t H, int64_t T, int C,
                   const float* alpha, const float* mu, const float* beta, const float* eta,
                   float* coef, float* gamma, void* stream)
{
    ChunkSizes s;
    int st = chunk_sizes(B, H, T, 16, 16, C, &s);
    if (st != MDN_OK) return st;
    if (C != 16 && C != 32 && C != 64) return MDN_ERR_UNSUPPORTED;
    if (s.tiles == 0) return MDN_OK;
    if (!alpha || !mu || !beta || !eta || !coef) return MDN_ERR_NULL_ARG;
    const void* all[] = {alpha, mu, beta, eta, coef, gamma};
    for (const void* p : all)
        if (p && !aligned16(p)) return MDN_ERR_ALIGN;
    const Range rc = range_of(coef, s.tiles * MDN_COEF_ROWS * C * 4);
    const Range rg = range_of(gamma, gamma ? s.tiles * C * C * 4 : 0);
    const Range ins[] = {range_of(alpha, s.tok * 4), range_of(mu, s.tok * 4),
                         range_of(beta, s.tok * 4), range_of(eta, s.tok * 4)};
    if (overlap(rc, rg)) return MDN_ERR_ALIAS;
    for (const Range& r : ins)
        if (overlap(rc, r) || overlap(rg, r)) return MDN_ERR_ALIAS;

    mdn::ChunkArgs a;
    memset(&a, 0, sizeof(a));
    a.BH = s.BH; a.T = T; a.NT = s.NT; a.dk = 16; a.dv = 16; a.C = C; a.dtype = MDN_F32;
    a.alpha = alpha; a.mu = mu; a.beta = beta; a.eta = eta;
    a.coef = coef; a.gamma = gamma; a.stream = stream;
    return hip_status(mdn::launch_chunk_coef(a));
}

}  // extern "C"
