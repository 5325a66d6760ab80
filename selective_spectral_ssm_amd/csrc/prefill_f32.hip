// prefill_f32.hip -- the chunked parallel scan for fp32 io with per-channel controls, on the
// fp32 matrix cores (v_mfma_f32_16x16x4f32).
//
// ESSH paper, Sec. 4.3 "Chunked parallel training": within a chunk the source-to-target
// contributions form a dense causal matrix applied by matrix multiplication, and only the
// 2 m P mode-state entries of a channel pass from one piece of the sequence to the next (the
// transition product of Eq. 6 makes the split exact).  Here the pieces are 16-position
// sub-blocks.  For a sub-block [T0, T0 + n), with qs(t) the clock summed from T0 to t
// (inclusive) and lambda_j = rho_j e^{i theta_j}:
//   y(t)   = sum_{s <= t} G[t][s] v(s) + sum_row C[t][row] h[row]
//   G[t][s] = g_r(t) g_w(s) e^{-(qs(t) - qs(s))} psi(t - s),  psi(tau) = sum_j Re(c_j lambda_j^tau)
//   C[t][(j, re/im)] = g_r(t) e^{-qs(t)} {Re, -Im}(c_j lambda_j^{t - T0 + 1})
//   h_j' = lambda_j^n e^{-qs(T0 + n - 1)} h_j + sum_s W[(j, re/im)][s] v(s),
//   W[(j, re/im)][s] = {Re, Im}(lambda_j^{T0 + n - 1 - s}) e^{-(qs(T0 + n - 1) - qs(s))} g_w(s)
// Every clock factor is the exponential of a non-positive difference, so no range limit
// applies; every product is fp32 with fp32 accumulation.  With the zero-lag correction
// (Eq. 24) and per-channel gates the lag-zero coefficient is psi(0) - sum_j a_j Re(c_j).
//
// One 64-lane wave per (batch row, channel) sequence.  MFMA layouts (16x16x4 f32): A operand
// lane l = A[l % 16][l / 16], B operand lane l = B[l / 16][l % 16], result lane l register r =
// D[4 (l / 16) + r][l % 16].  The state h [2m rows][P] is held as P/16 result tiles (rows
// 4g..4g+3 of column col per lane) and mirrored in LDS, from where the carry product reads it
// as a B operand.
#include "essh_internal.h"

namespace essh {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int M, int P>
__global__ void __launch_bounds__(64) prefill_f32_chunk_kernel(PrefillArgs a) {
    constexpr int NT = P / 16;            // 16-column tiles
    constexpr int ROWS = 2 * M;           // state rows (mode, re/im)
    constexpr int KR = (ROWS + 3) / 4;    // K steps of the carry product
    __shared__ float2 pw[17][M];          // lambda_j^tau, tau = 0..16
    __shared__ float2 cpw[17][M];         // c_j lambda_j^tau
    __shared__ float psi[16];
    __shared__ float hs[16][P];           // the state, [row][column]

    const int lane = threadIdx.x;
    const int i = lane & 15;              // A row / B column / result column
    const int g = lane >> 4;              // A column group / B row group / result row group
    const int seq = blockIdx.x;
    const int k = seq % a.K_T, b = seq / a.K_T;
    const int L = a.L, K = a.K;
    const float* v = static_cast<const float*>(a.v);
    const float* gwp = static_cast<const float*>(a.g_w);
    const float* grp = static_cast<const float*>(a.g_r);
    float* y = static_cast<float*>(a.y);

    // ---- pole tables of channel k ----
    for (int idx = lane; idx < 17 * M; idx += 64) {
        const int tau = idx / M, j = idx - tau * M;
        const float r = a.rho[k * M + j], th = a.theta[k * M + j];
        const float mag = tau == 0 ? 1.f : powf(r, (float)tau);
        float sn, cs;
        sincosf(th * (float)tau, &sn, &cs);
        const float pr = mag * cs, pi = mag * sn;
        const float cr = a.c[(k * M + j) * 2], ci = a.c[(k * M + j) * 2 + 1];
        pw[tau][j] = make_float2(pr, pi);
        cpw[tau][j] = make_float2(cr * pr - ci * pi, cr * pi + ci * pr);
    }
    __syncthreads();
    if (lane < 16) {
        float s = 0.f;
        for (int j = 0; j < M; ++j) {
            s += cpw[lane][j].x;
            if (lane == 0 && a.zl) s -= a.zl[k * M + j] * a.c[(k * M + j) * 2];
        }
        psi[lane] = s;
    }

    // ---- entering state (result layout and LDS mirror) ----
    f32x4 st[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * g + r;
            float x = 0.f;
            if (row < ROWS && a.state_in) x = a.state_in[(((size_t)b * K + k) * ROWS + row) * P + nt * 16 + i];
            st[nt][r] = x;
            hs[row][nt * 16 + i] = x;
        }
    }
    __syncthreads();

    for (int t0 = 0; t0 < L; t0 += 16) {
        const int n = min(16, L - t0);
        // controls of the sub-block: position i of every 16-lane group
        const size_t crow = ((size_t)b * L + t0 + (i < n ? i : n - 1)) * K + k;
        const float dl = i < n ? a.delta[crow] : 0.f;
        const float gwi = i < n ? gwp[crow] : 0.f;
        const float gri = i < n ? grp[crow] : 0.f;
        float q = dl;   // inclusive clock sum over the group's positions
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const float o = __shfl_up(q, off, 16);
            if (i >= off) q += o;
        }
        const float qe = __shfl(q, n - 1, 16);

        // A operands: G (intra), C (carry), W (state)
        float ga[4], ca[KR], wa[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int s = 4 * kk + g;
            const float qs = __shfl(q, s, 16), gws = __shfl(gwi, s, 16);
            ga[kk] = (s <= i && i < n) ? gri * gws * expf(qs - q) * psi[i - s < 0 ? 0 : i - s] : 0.f;
            // W: row i (mode i/2, re/im), source s
            float wv = 0.f;
            if (i < ROWS && s < n) {
                const float2 p = pw[n - 1 - s][i >> 1];
                wv = ((i & 1) ? p.y : p.x) * expf(qs - qe) * gws;
            }
            wa[kk] = wv;
        }
#pragma unroll
        for (int kk = 0; kk < KR; ++kk) {
            const int row = 4 * kk + g;
            float cv = 0.f;
            if (row < ROWS && i < n) {
                const float2 cp = cpw[i + 1][row >> 1];
                cv = gri * expf(-q) * ((row & 1) ? -cp.y : cp.x);
            }
            ca[kk] = cv;
        }
        // transfer of the sub-block for this lane's modes 2g, 2g + 1
        float lt[4];
        {
            const float e = expf(-qe);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int j = 2 * g + hh;
                const float2 p = j < M ? pw[n][j] : make_float2(0.f, 0.f);
                lt[2 * hh] = e * p.x;
                lt[2 * hh + 1] = e * p.y;
            }
        }

#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int p = nt * 16 + i;
            // B operands: v[s = 4 kk + g][p]
            float vb[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int s = 4 * kk + g;
                vb[kk] = s < n ? v[(((size_t)b * L + t0 + s) * K + k) * P + p] : 0.f;
            }
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[kk], vb[kk], acc, 0, 0, 0);
#pragma unroll
            for (int kk = 0; kk < KR; ++kk)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ca[kk], hs[4 * kk + g][p], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g + r;
                if (t < n) y[(((size_t)b * L + t0 + t) * K + k) * P + p] = acc[r];
            }
            // state: h' = transfer * h + W v
            f32x4 d;
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                const float hr = st[nt][r], hi = st[nt][r + 1];
                d[r] = lt[r] * hr - lt[r + 1] * hi;
                d[r + 1] = lt[r + 1] * hr + lt[r] * hi;
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) d = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[kk], vb[kk], d, 0, 0, 0);
            st[nt] = d;
        }
        __syncthreads();   // every carry read of hs is done
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) hs[4 * g + r][nt * 16 + i] = (4 * g + r < ROWS) ? st[nt][r] : 0.f;
        }
        __syncthreads();
    }

    if (a.state_out) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * g + r;
                if (row < ROWS) a.state_out[(((size_t)b * K + k) * ROWS + row) * P + nt * 16 + i] = st[nt][r];
            }
        }
    }
}

template <int M>
hipError_t launch_m(const PrefillArgs& a, int P, hipStream_t s) {
    const dim3 grid((unsigned)(a.B * a.K_T)), block(64);
    switch (P) {
        case 16: hipLaunchKernelGGL((prefill_f32_chunk_kernel<M, 16>), grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL((prefill_f32_chunk_kernel<M, 32>), grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL((prefill_f32_chunk_kernel<M, 64>), grid, block, 0, s, a); break;
        case 128: hipLaunchKernelGGL((prefill_f32_chunk_kernel<M, 128>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32_chunked(const PrefillArgs& a, int m, int P, hipStream_t s) {
    if (a.B == 0 || a.K_T == 0 || a.L == 0) return hipSuccess;
    switch (m) {
        case 1: return launch_m<1>(a, P, s);
        case 2: return launch_m<2>(a, P, s);
        case 4: return launch_m<4>(a, P, s);
        case 8: return launch_m<8>(a, P, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace essh
