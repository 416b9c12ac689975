// mdn_gates.hip -- gate pre-operation and output correction (gfx950).
//
// The elementwise step between a layer's projections and the recurrence
// (MDN summary at paper.rainbus.top, method walk-through steps 6 and 7;
// ijyty.com article on MDN, sections 5 and 8):
//   eta   = tanh(x) + 1
//   theta = arctan(s eta);  alpha_max = cos^2 theta,  beta_max = sin^2 theta
//   alpha = alpha_max sigmoid(a),  beta = beta_max sigmoid(b)
//   mu    = exp(clamp(mu_log, mu_log_min, 0))
//   q'    = q - d_h k                       (query correction, per head h)
// cos^2(arctan u) = 1 / (1 + u^2) and sin^2(arctan u) = u^2 / (1 + u^2), so
// the kernel forms alpha_max and beta_max without trigonometric calls, and
// tanh(x) + 1 = 2 / (1 + exp(-2x)) is evaluated in that form, which keeps its
// relative accuracy where tanh(x) is close to -1 (this is the same function,
// not the 2 sigmoid(x) activation the article's ablation replaces it with).
//
// One launch, two kinds of workgroups: the first `gate_blocks` handle four
// consecutive tokens per thread (16-byte loads and stores of each fp32
// tensor), the rest correct q in 16-byte vectors (a vector never straddles
// two tokens, as a row of dk >= 16 elements is at least 32 bytes).
// Everything is HBM-bound.
#include <algorithm>

#include "mdn_device.h"
#include "mdn_internal.h"
#include "../../include/mdn.h"

namespace mdn {

__device__ __forceinline__ void gate_one(float x, float a, float b, float ml, float s, float mlmin,
                                         float& alpha, float& mu, float& beta, float& eta)
{
    eta = 2.f / (1.f + expf(-2.f * x));          // = tanh(x) + 1, without its cancellation at x << 0
    const float u = s * eta, u2 = u * u;
    const float amax = 1.f / (1.f + u2);
    const float bmax = u2 * amax;
    alpha = amax / (1.f + expf(-a));
    beta = bmax / (1.f + expf(-b));
    mu = expf(fminf(fmaxf(ml, mlmin), 0.f));
}

template <typename E>
__global__ __launch_bounds__(256)
void mdn_gates_kernel(int64_t N, int64_t T, int H, int dk, float s, float mlmin,
                      const float* __restrict__ x, const float* __restrict__ a,
                      const float* __restrict__ b, const float* __restrict__ ml,
                      float* __restrict__ alpha, float* __restrict__ mu,
                      float* __restrict__ beta, float* __restrict__ eta,
                      const E* q, const E* __restrict__ k, const float* __restrict__ d, E* qo,
                      int64_t gate_blocks)
{
    const int64_t nthr = 256;
    if ((int64_t)blockIdx.x < gate_blocks) {
        const int64_t n4 = N / 4;
        for (int64_t i = blockIdx.x * nthr + threadIdx.x; i < n4; i += gate_blocks * nthr) {
            const floatx4 X = reinterpret_cast<const floatx4*>(x)[i];
            const floatx4 A = reinterpret_cast<const floatx4*>(a)[i];
            const floatx4 Bv = reinterpret_cast<const floatx4*>(b)[i];
            const floatx4 L = reinterpret_cast<const floatx4*>(ml)[i];
            floatx4 oa, om, ob, oe;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float ga, gm, gb, ge;
                gate_one(X[u], A[u], Bv[u], L[u], s, mlmin, ga, gm, gb, ge);
                oa[u] = ga; om[u] = gm; ob[u] = gb; oe[u] = ge;
            }
            reinterpret_cast<floatx4*>(alpha)[i] = oa;
            reinterpret_cast<floatx4*>(mu)[i] = om;
            reinterpret_cast<floatx4*>(beta)[i] = ob;
            reinterpret_cast<floatx4*>(eta)[i] = oe;
        }
        // tail of fewer than four tokens
        if (blockIdx.x == 0 && threadIdx.x < N - 4 * n4) {
            const int64_t i = 4 * n4 + threadIdx.x;
            gate_one(x[i], a[i], b[i], ml[i], s, mlmin, alpha[i], mu[i], beta[i], eta[i]);
        }
        return;
    }
    if (!qo) return;
    // query correction: 16-byte vectors of EV elements
    constexpr int EV = 16 / sizeof(E);
    const int64_t nv = N * dk / EV, vpt = dk / EV;          // vectors, vectors per token
    const int64_t qb = (int64_t)gridDim.x - gate_blocks;
    for (int64_t i = (blockIdx.x - gate_blocks) * nthr + threadIdx.x; i < nv; i += qb * nthr) {
        const int64_t tok = i / vpt;
        const float dh = d[(tok / T) % H];
        union { uint4 u; E e[EV]; } Q, K, R;
        Q.u = reinterpret_cast<const uint4*>(q)[i];
        K.u = reinterpret_cast<const uint4*>(k)[i];
#pragma unroll
        for (int j = 0; j < EV; ++j) R.e[j] = (E)((float)Q.e[j] - dh * (float)K.e[j]);
        reinterpret_cast<uint4*>(qo)[i] = R.u;
    }
}

hipError_t launch_gates(const GateArgs& g)
{
    if (g.N == 0) return hipSuccess;
    const int64_t gate_blocks = std::min<int64_t>((g.N / 4 + 255) / 256 + 1, 2048);
    int64_t q_blocks = 0;
    if (g.qo) {
        const int64_t ev = 16 / (g.dtype == MDN_BF16 ? 2 : 4);
        q_blocks = std::min<int64_t>((g.N * g.dk / ev + 255) / 256, 8192);
    }
    const dim3 grid((unsigned)(gate_blocks + q_blocks));
    if (g.dtype == MDN_BF16)
        hipLaunchKernelGGL(mdn_gates_kernel<__bf16>, grid, dim3(256), 0, (hipStream_t)g.stream,
                           g.N, g.T, (int)g.H, g.dk, g.s, g.mu_log_min, g.x, g.a, g.b, g.mu_log,
                           g.alpha, g.mu, g.beta, g.eta, (const __bf16*)g.q, (const __bf16*)g.k, g.d,
                           (__bf16*)g.qo, gate_blocks);
    else
        hipLaunchKernelGGL(mdn_gates_kernel<float>, grid, dim3(256), 0, (hipStream_t)g.stream,
                           g.N, g.T, (int)g.H, g.dk, g.s, g.mu_log_min, g.x, g.a, g.b, g.mu_log,
                           g.alpha, g.mu, g.beta, g.eta, (const float*)g.q, (const float*)g.k, g.d,
                           (float*)g.qo, gate_blocks);
    return hipGetLastError();
}

}  // namespace mdn
