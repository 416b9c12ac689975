// mdn_step.hip -- one recurrent decode step of Momentum DeltaNet (gfx950).
//
// Recurrent form used for generation (ijyty.com article on MDN, section 6;
// update equations of the MDN summary at paper.rainbus.top, method
// walk-through step 1), per (batch, head), in fp32:
//     vtilde = v - alpha * S^T k
//     M      = mu * M - eta * k vtilde^T
//     S      = alpha * S - beta * M
//     o      = S^T q
// The step is bound by HBM: S and M (dk x dv fp32 each) are read once and
// written once; everything else is a few hundred bytes per head.  One
// workgroup owns one head and keeps its whole S and M slab in registers:
//   thread t: column group cg = t % CG (4 adjacent columns, one float4),
//             row group    rg = t / CG (rows rg, rg + RG, rg + 2RG, ...).
// A wave therefore reads whole 4*dv-byte rows with dwordx4 accesses.
// The two reductions over dk (S^T k before the update, S^T q after it) go
// through LDS.
#include "mdn_device.h"
#include "mdn_internal.h"

namespace mdn {

#ifndef MDN_STEP_SPLIT
#define MDN_STEP_SPLIT 2
#endif

template <typename Tr, int DK, int DV, int NSPLIT>
struct StepCfg {
    static constexpr int DVW = DV / NSPLIT;                 // columns per workgroup
    static constexpr int CG = DVW / 4;                      // float4 column groups
    static constexpr int RG = (256 / CG) < DK ? (256 / CG) : DK;  // row groups
    static constexpr int RPT = DK / RG;                     // rows per thread
    static constexpr int NTHR = CG * RG;
    static_assert(DK % RG == 0, "row groups must tile dk");
};

template <typename Tr, int DK, int DV, int NSPLIT>
__global__ __launch_bounds__(256)
void mdn_step_kernel(const typename Tr::elem* __restrict__ q,
                     const typename Tr::elem* __restrict__ k,
                     const typename Tr::elem* __restrict__ v,
                     const float* __restrict__ alpha, const float* __restrict__ mu,
                     const float* __restrict__ beta, const float* __restrict__ eta,
                     float* __restrict__ S, float* __restrict__ M,
                     typename Tr::elem* __restrict__ o)
{
    using Cfg = StepCfg<Tr, DK, DV, NSPLIT>;
    constexpr int CG = Cfg::CG, RG = Cfg::RG, RPT = Cfg::RPT;
    __shared__ float4 red[RG][CG];

    // workgroup = (head, block of DV / NSPLIT columns); columns are independent
    const int bh = blockIdx.x / NSPLIT;
    const int cb = (blockIdx.x % NSPLIT) * Cfg::DVW;
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;

    float* Sh = S + (size_t)bh * DK * DV + cb;
    float* Mh = M + (size_t)bh * DK * DV + cb;

    // Issue the state loads first: they are the whole cost of the step.
    // The state streams through once per step and is far larger than the
    // caches, so loads and stores are non-temporal.
    floatx4 s[RPT], m[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(Sh + (size_t)row * DV + 4 * cg));
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        m[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(Mh + (size_t)row * DV + 4 * cg));
    }
    const float a = alpha[bh], mm = mu[bh], b = beta[bh], e = eta[bh];
    float kk[RPT], qq[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        kk[i] = Tr::to_f(k[(size_t)bh * DK + row]);
        qq[i] = Tr::to_f(q[(size_t)bh * DK + row]);
    }
    float vv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) vv[c] = Tr::to_f(v[(size_t)bh * DV + cb + 4 * cg + c]);

    // u = S^T k over this thread's rows, then across row groups.
    float4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        u.x += s[i][0] * kk[i]; u.y += s[i][1] * kk[i];
        u.z += s[i][2] * kk[i]; u.w += s[i][3] * kk[i];
    }
    red[rg][cg] = u;
    __syncthreads();
    float4 ut = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        const float4 p = red[r][cg];
        ut.x += p.x; ut.y += p.y; ut.z += p.z; ut.w += p.w;
    }
    const float vt0 = vv[0] - a * ut.x, vt1 = vv[1] - a * ut.y;
    const float vt2 = vv[2] - a * ut.z, vt3 = vv[3] - a * ut.w;

    // M <- mu M - eta k vtilde^T ;  S <- alpha S - beta M ;  partial o = S^T q
    float4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float ek = e * kk[i];
        floatx4 mn, sn;
        mn[0] = mm * m[i][0] - ek * vt0; mn[1] = mm * m[i][1] - ek * vt1;
        mn[2] = mm * m[i][2] - ek * vt2; mn[3] = mm * m[i][3] - ek * vt3;
        sn[0] = a * s[i][0] - b * mn[0]; sn[1] = a * s[i][1] - b * mn[1];
        sn[2] = a * s[i][2] - b * mn[2]; sn[3] = a * s[i][3] - b * mn[3];
        const int row = rg + RG * i;
        __builtin_nontemporal_store(mn, reinterpret_cast<floatx4*>(Mh + (size_t)row * DV + 4 * cg));
        __builtin_nontemporal_store(sn, reinterpret_cast<floatx4*>(Sh + (size_t)row * DV + 4 * cg));
        w.x += sn[0] * qq[i]; w.y += sn[1] * qq[i]; w.z += sn[2] * qq[i]; w.w += sn[3] * qq[i];
    }
    __syncthreads();          // every thread has read red[] for u
    red[rg][cg] = w;
    __syncthreads();
    if (rg == 0) {
        float4 ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const float4 p = red[r][cg];
            ot.x += p.x; ot.y += p.y; ot.z += p.z; ot.w += p.w;
        }
        typename Tr::elem* op = o + (size_t)bh * DV + cb + 4 * cg;
        op[0] = Tr::from_f(ot.x); op[1] = Tr::from_f(ot.y);
        op[2] = Tr::from_f(ot.z); op[3] = Tr::from_f(ot.w);
    }
}

template <typename Tr, int DK, int DV>
static hipError_t launch_step_t(const StepArgs& a)
{
    constexpr int NSPLIT = DV >= 64 ? MDN_STEP_SPLIT : 1;
    using Cfg = StepCfg<Tr, DK, DV, NSPLIT>;
    using E = typename Tr::elem;
    hipLaunchKernelGGL((mdn_step_kernel<Tr, DK, DV, NSPLIT>), dim3((unsigned)(a.BH * NSPLIT)), dim3(Cfg::NTHR), 0,
                       (hipStream_t)a.stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v,
                       a.alpha, a.mu, a.beta, a.eta, a.S, a.M, (E*)a.o);
    return hipGetLastError();
}

template <typename Tr>
static hipError_t launch_step_d(const StepArgs& a)
{
    switch (a.dk) {
    case 16: return launch_step_t<Tr, 16, 16>(a);
    case 32: return launch_step_t<Tr, 32, 32>(a);
    case 64: return launch_step_t<Tr, 64, 64>(a);
    case 128: return launch_step_t<Tr, 128, 128>(a);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_step(const StepArgs& a)
{
    if (a.BH == 0) return hipSuccess;
    return a.dtype == 1 ? launch_step_d<TraitsBf16>(a) : launch_step_d<TraitsF32>(a);
}

// Bandwidth reference for the decode step: every fp32 of a buffer is read,
// multiplied by `scale` and written back in place, with the step's access
// pattern and none of its arithmetic: 256 threads per workgroup, each
// loading RPT 16-byte pieces (non-temporal) before storing them back, so a
// workgroup streams 64 KiB, as a decode workgroup does with its half of a
// head's S and M.  A scale of 1 leaves the buffer as it was.
template <int RPT>
__global__ __launch_bounds__(256)
void mdn_stream_rw_kernel(floatx4* __restrict__ buf, int64_t n16, float scale)
{
    const int64_t base = (int64_t)blockIdx.x * 256 * RPT + threadIdx.x;
    floatx4 x[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int64_t j = base + (int64_t)i * 256;
        if (j < n16) x[i] = __builtin_nontemporal_load(buf + j);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int64_t j = base + (int64_t)i * 256;
        if (j < n16) {
            floatx4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = x[i][e] * scale;
            __builtin_nontemporal_store(y, buf + j);
        }
    }
}

hipError_t launch_stream_rw(void* buf, int64_t n16, float scale, void* stream)
{
    constexpr int RPT = 16;
    if (n16 == 0) return hipSuccess;
    const int64_t blocks = (n16 + 256 * RPT - 1) / (256 * RPT);
    hipLaunchKernelGGL((mdn_stream_rw_kernel<RPT>), dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<floatx4*>(buf), n16, scale);
    return hipGetLastError();
}

// Element-type conversion of n values (n a multiple of 8): bf16 -> fp32
// (exact) or fp32 -> bf16 (round to nearest even), 8 values per thread.
__global__ __launch_bounds__(256)
void mdn_widen_kernel(const uint4* __restrict__ src, floatx4* __restrict__ dst, int64_t n8)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    union { uint4 u; __bf16 h[8]; } x;
    x.u = src[i];
    dst[2 * i] = floatx4{(float)x.h[0], (float)x.h[1], (float)x.h[2], (float)x.h[3]};
    dst[2 * i + 1] = floatx4{(float)x.h[4], (float)x.h[5], (float)x.h[6], (float)x.h[7]};
}

__global__ __launch_bounds__(256)
void mdn_narrow_kernel(const floatx4* __restrict__ src, uint4* __restrict__ dst, int64_t n8)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const floatx4 a = src[2 * i], b = src[2 * i + 1];
    union { uint4 u; __bf16 h[8]; } y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        y.h[e] = (__bf16)a[e];
        y.h[4 + e] = (__bf16)b[e];
    }
    dst[i] = y.u;
}

hipError_t launch_convert(const void* src, int src_dtype, void* dst, int64_t n, void* stream)
{
    if (n == 0) return hipSuccess;
    if (n % 8 != 0) return hipErrorInvalidValue;
    const int64_t n8 = n / 8, blocks = (n8 + 255) / 256;
    if (src_dtype == 1)
        hipLaunchKernelGGL(mdn_widen_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                           reinterpret_cast<const uint4*>(src), reinterpret_cast<floatx4*>(dst), n8);
    else
        hipLaunchKernelGGL(mdn_narrow_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                           reinterpret_cast<const floatx4*>(src), reinterpret_cast<uint4*>(dst), n8);
    return hipGetLastError();
}

}  // namespace mdn
