// mdn_internal.h -- argument blocks passed from the validated C entry points
// (mdn_api.cpp) to the kernel launchers (mdn_step.hip, mdn_chunk.hip).
// Everything here has already been checked on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mdn {

struct StepArgs {
    int64_t BH;
    int dk, dv, dtype;
    const void *q, *k, *v;
    const float *alpha, *mu, *beta, *eta;
    float *S, *M;
    void* o;
    void* stream;
};

struct ChunkArgs {
    int64_t BH, T, NT;
    int dk, dv, C, dtype;
    const void *q, *k, *v;
    const float *alpha, *mu, *beta, *eta;
    const float *S0, *M0;
    void* O;
    float *ST, *MT;
    void* Vt;
    // per-chunk intermediates (workspace sections)
    void* Tmat;      // [BH*NT][C][C] elem
    void* Aqk;       // [BH*NT][C][C] elem
    float* coef;     // [BH*NT][8][C]
    float* gamma;    // [BH*NT][C][C] or nullptr (diagnostic only)
    // Packed variable-length batch: nullptr for the [B,H,T,.] layout.  With
    // cu set, BH is the head count H of the [H,T,.] packed layout, T the
    // packed length, nseq the number of sequences, and NT = T / C + nseq the
    // tile slots per head; tab holds (first row, rows) per slot and perm
    // the sequences in dispatch order (longest first).
    const int32_t* cu;   // [nseq + 1] sequence starts (device)
    int64_t nseq;
    int32_t* tab;        // [NT][2] (workspace)
    int32_t* perm;       // [nseq] (workspace)
    bool trans;          // intra stage writes T^T and Aqk^T (for the backward)
    void* stream;
};

// Backward of the chunk forward: the forward's arguments, its vtilde, the
// output gradients and the gradient outputs; workspace sections as listed
// in mdn_api.cpp.
struct BwdArgs {
    ChunkArgs f;          // q, k, gates, S0, M0, sizes; Tmat/Aqk hold T^T, Aqk^T
    const void* Vt;       // [BH][T][D] elem (the forward's vtilde)
    const void* dO;       // [BH][T][D] elem
    const float *dST, *dMT;   // [BH][D][D] or NULL
    void *dq, *dk, *dv;   // [BH][T][D] elem
    float *dalpha, *dmu, *dbeta, *deta;   // [BH][T]
    float *dS0, *dM0;     // [BH][D][D]
    void *Sst, *Mst, *dSst, *dMst;        // [BH*NT][D][D] elem: chunk-start states, chunk-end adjoints
    void *dqp, *dkp;      // [BH*NT][C][D] elem: state-product parts of dq, dk
    float* vec;           // [BH*NT][MDN_BWD_VEC_ROWS][C] fp32: coefficient adjoints from the state products
};
constexpr int MDN_BWD_VEC_ROWS = 8;   // Dabar, Db, Dab, DgS, DgM, then <S,dS'>, <M,dS'>, <M,dM'> in row 5
hipError_t launch_bwd(const BwdArgs& a);

struct GateArgs {
    int64_t N, T, H;          // N = B*H*T tokens
    int dk, dtype;
    float s, mu_log_min;
    const float *x, *a, *b, *mu_log;
    float *alpha, *mu, *beta, *eta;
    const void *q, *k;        // all NULL when the query correction is skipped
    const float* d;
    void* qo;
    void* stream;
};

hipError_t launch_step(const StepArgs& a);
// in-place read, scale and write of n16 16-byte pieces (decode bandwidth reference)
hipError_t launch_stream_rw(void* buf, int64_t n16, float scale, void* stream);
// n values (a multiple of 8) from src to dst: bf16 -> fp32 when src_dtype is
// bf16, else fp32 -> bf16 (round to nearest even)
hipError_t launch_convert(const void* src, int src_dtype, void* dst, int64_t n, void* stream);
// gate pre-operation and query correction
hipError_t launch_gates(const GateArgs& g);
// coefficient + intra-chunk stage (T, (QK^T) o Gamma, coefficients)
hipError_t launch_chunk_intra(const ChunkArgs& a);
// coefficient stage alone (diagnostic entry point)
hipError_t launch_chunk_coef(const ChunkArgs& a);
// sequential inter-chunk stage (vtilde, O, state carry)
hipError_t launch_chunk_inter(const ChunkArgs& a);
// the inter-chunk stage with each sequence cut into P segments ([B, H, T]
// layout): pass 1, the combine step and pass 2, with the state slots in
// segS / segM (BH (1 + 4 (P - 2)) blocks of dk x dv fp32 each)
hipError_t launch_chunk_inter_split(const ChunkArgs& a, int P, float* segS, float* segM);
// compute units of the current device (256 when the query fails)
int device_compute_units();
// the whole forward in one kernel, without a workspace, for the shapes it
// covers (bf16, C = 64, dk = dv in {64, 128}, [B, H, T] layout)
bool fwd_fused_supported(const ChunkArgs& a);
hipError_t launch_chunk_fwd_fused(const ChunkArgs& a);
// slot table and dispatch order of a packed variable-length batch (a.cu set)
hipError_t launch_varlen_prep(const ChunkArgs& a);

}  // namespace mdn
