// backward.h -- private declarations of the backward pass (backward.hip), shared with the
// entry points in essh_api.hip.
#pragma once

#include "essh_internal.h"

namespace essh {

struct BackwardArgs {
    int B, L, K, K_T;
    const void* v;            // forward inputs, as for the prefill
    const float* delta;
    const void* g_w;
    const void* g_r;
    const float* rho;
    const float* theta;
    const float* c;
    const float* zl;          // or null
    const float* state_in;    // or null (zero entering state)
    const void* dy;           // [B, L, K, P] io dtype
    const float* dstate_out;  // [B, K, m, 2, P] or null
    void* dv;                 // [B, L, K, P] io dtype
    float* ddelta;            // [B, L, K]
    float* dg_w;              // [B, L, K] fp32
    float* dg_r;              // [B, L, K] fp32
    float* drho;              // [K, m]
    float* dtheta;            // [K, m]
    float* dc;                // [K, m, 2]
    float* dzl;               // [K, m] or null
    float* dstate_in;         // [B, K, m, 2, P] or null
};

// Work split of the backward pass: nseq = B K_T sequences, each cut into nseg segments of Ls
// positions (nsb sub-blocks of 16), each segment handled by nslice waves of <= 64 value columns.
// Workspace (fp32):
//   ck   [nseq][nseg][nsb][2m][P]  local state (from a zero entering state) after each sub-block
//   sa   [nseq][nseg][2m][P]       local adjoint aggregate, then the arriving adjoint
//   hin  [nseq][nseg][2m][P]       entering state of each segment
//   tpf  [nseq][nseg][nsb][m]      transfer from the segment start to each sub-block's start (complex)
//   lam  [nseq][nseg][m]           segment transfers (complex)
//   pp   [nseq][nseg][nslice][4m+1] mode-table partials (Omega_j, Gamma_j, trace)
//   pc   [nseq][L]                 channel-major controls (delta, g_w, g_r, 0)
//   gc   [nslice][nseq][L]         channel-major control gradients (ddelta, dg_w, dg_r, 0)
constexpr int MAX_BWD_SUBBLOCKS = 128;
struct BwdPlan {
    int P, nslice, nseq, nseg, Ls, nsb, L;
    float* ck;
    float* sa;
    float* hin;
    float2* tpf;
    float2* lam;
    float* pp;
    float4* pc;
    float4* gc;
};

BwdPlan plan_backward(int B, int L, int K, int K_T, int m, int P);
size_t backward_workspace_bytes(int B, int L, int K, int K_T, int m, int P);
void bind_backward_workspace(BwdPlan& plan, void* workspace, int m);
hipError_t launch_prefill_backward(const BackwardArgs& a, int m, const BwdPlan& plan, int io_dtype, hipStream_t s);

}  // namespace essh
