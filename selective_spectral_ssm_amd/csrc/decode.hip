// decode.hip -- fused single-token recurrent decode step.
//
// ESSH paper, Sec. 4.3 "Recurrent decoding" and Sec. 5.3: the mode states are
// updated one token at a time, state update and readout fused, discarded
// channels never touched.  One launch advances n_layers independent mixers.
//
// One thread owns one (layer, b, k < K_T, p) lane and all m modes of it: it
// reads the 2m fp32 state values of the lane once, applies
// h <- rho e^{-delta} e^{i theta} h + g_w v, accumulates g_r Re(c h), writes
// the state back and writes y.  Consecutive lanes are consecutive p, so every
// state plane, v and y access of a wave is one contiguous run.
//
// The grid is (channel groups, batch rows, layers): a workgroup holds
// max(P, 64) lanes, i.e. 64/P channels of one (layer, b) when P < 64 and one
// channel otherwise, so no lane divides to find its indices.  Every global
// load of a lane is issued first; the pole rotations
// rho (cos theta, sin theta), per (layer, k, j) and shared by the P lanes of a
// channel, are evaluated while those loads are in flight, by the first m lanes
// of each channel group in a wave, and broadcast with cross-lane reads.
#include "essh_internal.h"

namespace essh {
namespace {

template <int M, typename IO, bool PER_MODE>
__global__ void __launch_bounds__(128)
decode_kernel(DecodeArgs a, int P) {
    using io = io_traits<IO>;
    const int tpb = P < 64 ? 64 : P;            // lanes of a workgroup
    const int k = blockIdx.x * (tpb / P) + (int)threadIdx.x / P;
    const int p = (int)threadIdx.x % P;
    const int b = blockIdx.y;
    const int l = blockIdx.z;
    const bool active = k < a.K_T;
    const int kk = active ? k : a.K_T - 1;      // inactive lanes mirror a valid channel
    const int K = a.K;

    // Channel group of this lane inside the wave (P >= 16 >= M lanes per group).
    const int lane = threadIdx.x & 63;
    const int G = P < 64 ? P : 64;
    const int base = lane - (lane % G);
    const int jm = (lane % G) < M ? (lane % G) : 0;
    const size_t tab = ((size_t)l * K + kk) * M;                 // (layer, k, j=0) of rho/theta/c
    const size_t row = ((size_t)l * a.B + b) * K + kk;           // (layer, b, k)

    // ---- every load first; the pole parameters first of all, so that waiting
    // for them (loads complete in issue order) does not wait for the state --------------
    const float rr = a.rho[tab + jm];
    const float th = a.theta[tab + jm];
    const IO* vp = static_cast<const IO*>(a.v);
    const IO* gwp = static_cast<const IO*>(a.g_w);
    const IO* grp = static_cast<const IO*>(a.g_r);
    float* st = a.state + row * (size_t)(M * 2 * P) + p;
    float hr[M], hi[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        hr[j] = st[(2 * j) * P];
        hi[j] = st[(2 * j + 1) * P];
    }
    const float x = io::load(vp, row * P + p);
    float dl[PER_MODE ? M : 1], gw[PER_MODE ? M : 1], gr[PER_MODE ? M : 1];
#pragma unroll
    for (int j = 0; j < (PER_MODE ? M : 1); ++j) {
        const size_t cj = PER_MODE ? row * M + j : row;
        dl[j] = a.delta[cj];
        gw[j] = io::load(gwp, cj);
        gr[j] = io::load(grp, cj);
    }
    float cr[M], ci[M], za[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        cr[j] = a.c[(tab + j) * 2 + 0];
        ci[j] = a.c[(tab + j) * 2 + 1];
        za[j] = a.zl ? a.zl[tab + j] : 0.f;   // zero-lag correction (Eq. 24)
    }

    // ---- pole rotations, broadcast over the channel group ------------------------------------
    float my_r, my_i;
    {
        float sn, cs;
        sincosf(th, &sn, &cs);
        my_r = rr * cs;
        my_i = rr * sn;
    }

    float acc = 0.f;
    const float e_ch = PER_MODE ? 0.f : expf(-dl[0]);
    const float w_ch = PER_MODE ? 0.f : gw[0] * x;
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const float pr = __shfl(my_r, base + j);
        const float pi = __shfl(my_i, base + j);
        const float e = PER_MODE ? expf(-dl[PER_MODE ? j : 0]) : e_ch;
        const float w = PER_MODE ? gw[PER_MODE ? j : 0] * x : w_ch;
        const float g = PER_MODE ? gr[PER_MODE ? j : 0] : 1.f;
        const float ar = e * pr, ai = e * pi;
        const float nr = ar * hr[j] - ai * hi[j] + w;
        const float ni = ai * hr[j] + ar * hi[j];
        hr[j] = nr;
        hi[j] = ni;
        acc += g * (cr[j] * nr - ci[j] * ni - za[j] * cr[j] * w);
    }
    if (!PER_MODE) acc *= gr[0];

    if (active) {
#pragma unroll
        for (int j = 0; j < M; ++j) {
            st[(2 * j) * P] = hr[j];
            st[(2 * j + 1) * P] = hi[j];
        }
        io::store(static_cast<IO*>(a.y), row * P + p, acc);
    }
}

template <int M, typename IO>
hipError_t launch_decode_m(const DecodeArgs& a, int P, hipStream_t s) {
    if ((long long)a.n_layers * a.B * a.K_T == 0) return hipSuccess;
    const int tpb = P < 64 ? 64 : P;
    const int cpb = tpb / P;                     // channels per workgroup
    const dim3 grid((unsigned)((a.K_T + cpb - 1) / cpb), (unsigned)a.B, (unsigned)a.n_layers);
    if (a.per_mode)
        hipLaunchKernelGGL((decode_kernel<M, IO, true>), grid, dim3(tpb), 0, s, a, P);
    else
        hipLaunchKernelGGL((decode_kernel<M, IO, false>), grid, dim3(tpb), 0, s, a, P);
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_decode_io(const DecodeArgs& a, int m, int P, hipStream_t s) {
    switch (m) {
        case 1: return launch_decode_m<1, IO>(a, P, s);
        case 2: return launch_decode_m<2, IO>(a, P, s);
        case 4: return launch_decode_m<4, IO>(a, P, s);
        case 8: return launch_decode_m<8, IO>(a, P, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int m, int P, int io_dtype, hipStream_t s) {
    return io_dtype == ESSH_BF16 ? launch_decode_io<uint16_t>(a, m, P, s) : launch_decode_io<float>(a, m, P, s);
}

}  // namespace essh
