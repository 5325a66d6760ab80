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
// The pole rotations rho(cos theta, sin theta) are per (layer, k, j) and
// shared by the P lanes of a channel: the first m lanes of each channel group
// in a wave evaluate one each and the wave broadcasts them with cross-lane
// reads, instead of every lane evaluating m sin/cos pairs.
#include "essh_internal.h"

namespace essh {
namespace {

template <int M, typename IO, bool PER_MODE>
__global__ void __launch_bounds__(256)
decode_kernel(DecodeArgs a, int P) {
    using io = io_traits<IO>;
    const long long total = (long long)a.n_layers * a.B * a.K_T * P;
    const long long tid_raw = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const bool active = tid_raw < total;
    const long long tid = active ? tid_raw : total - 1;   // inactive lanes mirror the last lane
    const int p = (int)(tid % P);
    long long r = tid / P;
    const int k = (int)(r % a.K_T);
    r /= a.K_T;
    const int b = (int)(r % a.B);
    const int l = (int)(r / a.B);
    const int K = a.K;

    // Channel group of this lane inside the wave (P >= 16 >= M lanes per group).
    const int lane = threadIdx.x & 63;
    const int G = P < 64 ? P : 64;
    const int base = lane - (lane % G);
    const int jm = (lane % G) < M ? (lane % G) : 0;
    const size_t tab = ((size_t)l * K + k) * M;   // (layer, k, j=0) of rho/theta/c
    float my_r, my_i;
    {
        const float rr = a.rho[tab + jm];
        float sn, cs;
        sincosf(a.theta[tab + jm], &sn, &cs);
        my_r = rr * cs;
        my_i = rr * sn;
    }

    const size_t row = ((size_t)l * a.B + b) * K + k;            // (layer, b, k)
    const IO* vp = static_cast<const IO*>(a.v);
    const IO* gwp = static_cast<const IO*>(a.g_w);
    const IO* grp = static_cast<const IO*>(a.g_r);
    const float x = io::load(vp, row * P + p);

    float* st = a.state + row * (size_t)(M * 2 * P) + p;
    float hr[M], hi[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        hr[j] = st[(2 * j) * P];
        hi[j] = st[(2 * j + 1) * P];
    }

    float acc = 0.f;
    float e_ch = 0.f, w_ch = 0.f, g_ch = 0.f;
    if (!PER_MODE) {
        e_ch = expf(-a.delta[row]);
        w_ch = io::load(gwp, row) * x;
        g_ch = io::load(grp, row);
    }
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const float pr = __shfl(my_r, base + j);
        const float pi = __shfl(my_i, base + j);
        const float cr = a.c[(tab + j) * 2 + 0];
        const float ci = a.c[(tab + j) * 2 + 1];
        const float za = a.zl ? a.zl[tab + j] * cr : 0.f;   // zero-lag correction (Eq. 24)
        float e, w, g;
        if (PER_MODE) {
            const size_t cj = row * M + j;
            e = expf(-a.delta[cj]);
            w = io::load(gwp, cj) * x;
            g = io::load(grp, cj);
        } else {
            e = e_ch;
            w = w_ch;
            g = 1.f;
        }
        const float ar = e * pr, ai = e * pi;
        const float nr = ar * hr[j] - ai * hi[j] + w;
        const float ni = ai * hr[j] + ar * hi[j];
        hr[j] = nr;
        hi[j] = ni;
        acc += g * (cr * nr - ci * ni - za * w);
    }
    if (!PER_MODE) acc *= g_ch;

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
    const long long total = (long long)a.n_layers * a.B * a.K_T * P;
    if (total == 0) return hipSuccess;
    const int threads = 256;
    const unsigned blocks = (unsigned)((total + threads - 1) / threads);
    if (a.per_mode)
        hipLaunchKernelGGL((decode_kernel<M, IO, true>), dim3(blocks), dim3(threads), 0, s, a, P);
    else
        hipLaunchKernelGGL((decode_kernel<M, IO, false>), dim3(blocks), dim3(threads), 0, s, a, P);
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
