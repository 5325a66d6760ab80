// prefill_seq.hip -- sequential-over-positions prefill kernel.
//
// One thread owns one (batch row b, channel k < K_T, value p) lane and keeps
// the m complex mode states of that lane in registers while it walks the
// positions in order.  This is the recurrence of the ESSH selective mixer
// (Sec. 4.1 Eq. 5, readout Eq. 9) in complex form (App. B.1), evaluated
// exactly as written, in fp32.  It serves fp32 io with per-mode controls, the
// one layout no chunked kernel takes (fp32 io with per-channel controls runs on
// the fp32 matrix cores in prefill_f32.hip, bf16 io in prefill_chunk.hip and
// prefill_wave.hip).
//
// Positions are processed in blocks of SEQ_BLK; the loads of block i+1 are
// issued before the arithmetic of block i so that HBM latency overlaps work.
#include "essh_internal.h"

namespace essh {
namespace {

constexpr int SEQ_BLK = 8;

template <int M, typename IO, bool PER_MODE>
__global__ void __launch_bounds__(256)
prefill_seq_kernel(PrefillArgs a, int P) {
    using io = io_traits<IO>;
    const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)a.B * a.K_T * P;
    if (tid >= total) return;
    const int p = (int)(tid % P);
    const long long bk = tid / P;
    const int k = (int)(bk % a.K_T);
    const int b = (int)(bk / a.K_T);
    const int L = a.L, K = a.K;

    const IO* v = static_cast<const IO*>(a.v);
    const IO* gwp = static_cast<const IO*>(a.g_w);
    const IO* grp = static_cast<const IO*>(a.g_r);
    IO* y = static_cast<IO*>(a.y);

    // Pole and readout of each mode: rho e^{i theta} and c.
    // za: a_j kc_j, the lag-zero term removed by the zero-lag correction (Eq. 24)
    float lr[M], li[M], cr[M], ci[M], hr[M], hi[M], za[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const float r = a.rho[k * M + j];
        float sn, cs;
        sincosf(a.theta[k * M + j], &sn, &cs);
        lr[j] = r * cs;
        li[j] = r * sn;
        cr[j] = a.c[(k * M + j) * 2 + 0];
        ci[j] = a.c[(k * M + j) * 2 + 1];
        za[j] = a.zl ? a.zl[k * M + j] * cr[j] : 0.f;
        if (a.state_in) {
            const size_t s = ((((size_t)b * K + k) * M + j) * 2) * P + p;
            hr[j] = a.state_in[s];
            hi[j] = a.state_in[s + P];
        } else {
            hr[j] = 0.f;
            hi[j] = 0.f;
        }
    }

    constexpr int NC = PER_MODE ? M : 1;   // controls per position
    float xv[SEQ_BLK], xd[SEQ_BLK][NC], xw[SEQ_BLK][NC], xr[SEQ_BLK][NC];

    auto load_block = [&](int t0) {
#pragma unroll
        for (int u = 0; u < SEQ_BLK; ++u) {
            const int t = t0 + u;
            if (t < L) {
                const size_t row = ((size_t)b * L + t) * K + k;
                xv[u] = io::load(v, row * P + p);
#pragma unroll
                for (int q = 0; q < NC; ++q) {
                    const size_t ciq = row * NC + q;
                    xd[u][q] = a.delta[ciq];
                    xw[u][q] = io::load(gwp, ciq);
                    xr[u][q] = io::load(grp, ciq);
                }
            }
        }
    };

    load_block(0);
    for (int t0 = 0; t0 < L; t0 += SEQ_BLK) {
        float cv[SEQ_BLK], cd[SEQ_BLK][NC], cw[SEQ_BLK][NC], crd[SEQ_BLK][NC];
#pragma unroll
        for (int u = 0; u < SEQ_BLK; ++u) {
            cv[u] = xv[u];
#pragma unroll
            for (int q = 0; q < NC; ++q) { cd[u][q] = xd[u][q]; cw[u][q] = xw[u][q]; crd[u][q] = xr[u][q]; }
        }
        if (t0 + SEQ_BLK < L) load_block(t0 + SEQ_BLK);
#pragma unroll
        for (int u = 0; u < SEQ_BLK; ++u) {
            const int t = t0 + u;
            if (t >= L) break;
            float acc = 0.f;
            if (PER_MODE) {
#pragma unroll
                for (int j = 0; j < M; ++j) {
                    const float e = expf(-cd[u][j]);
                    const float ar = e * lr[j], ai = e * li[j];
                    const float w = cw[u][j] * cv[u];
                    const float nr = ar * hr[j] - ai * hi[j] + w;
                    const float ni = ai * hr[j] + ar * hi[j];
                    hr[j] = nr;
                    hi[j] = ni;
                    acc += crd[u][j] * (cr[j] * nr - ci[j] * ni - za[j] * w);
                }
            } else {
                const float e = expf(-cd[u][0]);
                const float w = cw[u][0] * cv[u];
#pragma unroll
                for (int j = 0; j < M; ++j) {
                    const float ar = e * lr[j], ai = e * li[j];
                    const float nr = ar * hr[j] - ai * hi[j] + w;
                    const float ni = ai * hr[j] + ar * hi[j];
                    hr[j] = nr;
                    hi[j] = ni;
                    acc += cr[j] * nr - ci[j] * ni - za[j] * w;
                }
                acc *= crd[u][0];
            }
            const size_t row = ((size_t)b * L + t) * K + k;
            io::store(y, row * P + p, acc);
        }
    }

    if (a.state_out) {
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const size_t s = ((((size_t)b * K + k) * M + j) * 2) * P + p;
            a.state_out[s] = hr[j];
            a.state_out[s + P] = hi[j];
        }
    }
}

template <int M, typename IO>
hipError_t launch_seq_m(const PrefillArgs& a, int P, hipStream_t s) {
    const long long total = (long long)a.B * a.K_T * P;
    if (total == 0) return hipSuccess;
    const int threads = 256;
    const unsigned blocks = (unsigned)((total + threads - 1) / threads);
    if (a.per_mode)
        hipLaunchKernelGGL((prefill_seq_kernel<M, IO, true>), dim3(blocks), dim3(threads), 0, s, a, P);
    else
        hipLaunchKernelGGL((prefill_seq_kernel<M, IO, false>), dim3(blocks), dim3(threads), 0, s, a, P);
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_seq_io(const PrefillArgs& a, int m, int P, hipStream_t s) {
    switch (m) {
        case 1: return launch_seq_m<1, IO>(a, P, s);
        case 2: return launch_seq_m<2, IO>(a, P, s);
        case 4: return launch_seq_m<4, IO>(a, P, s);
        case 8: return launch_seq_m<8, IO>(a, P, s);
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// Fill and state-copy helpers (kernels rather than hipMemset/hipMemcpy so a
// caller may capture them in a HIP graph).
// ---------------------------------------------------------------------------

__global__ void fill_zero_kernel(float4* p, size_t n4, float* tail, size_t ntail) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t j = i; j < n4; j += stride) p[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < ntail) tail[i] = 0.f;
}

// state [B, K, m, 2, P]: copy channels k < K_T from src to dst.
__global__ void copy_state_kernel(const float* src, float* dst, int B, int K, int K_T, int row) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)B * K_T * row;
    if (i >= total) return;
    const int e = (int)(i % row);
    const long long bk = i / row;
    const int k = (int)(bk % K_T);
    const int b = (int)(bk / K_T);
    const size_t off = ((size_t)b * K + k) * row + e;
    dst[off] = src ? src[off] : 0.f;
}

}  // namespace

hipError_t launch_prefill_sequential(const PrefillArgs& a, int m, int P, int io_dtype, hipStream_t s) {
    return io_dtype == ESSH_BF16 ? launch_seq_io<uint16_t>(a, m, P, s) : launch_seq_io<float>(a, m, P, s);
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t n4 = n / 4, ntail = n % 4;
    const int threads = 256;
    size_t want = (n4 + threads - 1) / threads;
    const unsigned blocks = (unsigned)(want < 1 ? 1 : (want > 4096 ? 4096 : want));
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(threads), 0, s,
                       reinterpret_cast<float4*>(p), n4, p + n4 * 4, ntail);
    return hipGetLastError();
}

hipError_t launch_copy_state(const float* src, float* dst, int B, int K, int K_T, int m, int P, hipStream_t s) {
    const int row = m * 2 * P;
    const long long total = (long long)B * K_T * row;
    if (total == 0 || src == dst) return hipSuccess;
    const int threads = 256;
    hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((total + threads - 1) / threads)), dim3(threads), 0, s,
                       src, dst, B, K, K_T, row);
    return hipGetLastError();
}

}  // namespace essh
