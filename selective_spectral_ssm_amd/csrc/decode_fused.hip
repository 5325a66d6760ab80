// decode_fused.hip -- one decode token through n_layers independent mixer layers with their
// projections, reading every weight byte once.
//
// ESSH paper, App. C.2 "Projections, gates, and clock": channel k's value is W_in_k u followed
// by the channel-local blend of Eq. 23 (a statistic over channel k's own P coordinates only),
// and three affine rows per (channel, mode) give the write gate 2 sigmoid(.), the read gate
// 2 sigmoid(.) and the clock increment softplus(.).  Sec. 4.1, Eq. 5 (per-mode controls) and
// App. C.3, Eq. 24: the mode update, readout and zero-lag term.  App. C.4: the first K_T P
// columns of W_out applied to the concatenated channel outputs, scaled by K_T^-1/2.
//
// Launch 1, one workgroup per (layer, batch row, retained channel): the P value rows and 3m
// control rows of that channel against u (bf16 weights, fp32 accumulation; u staged in LDS),
// the blend, the controls, and the mode update of the channel's P x m state lanes.  Its
// corrected outputs z go to the caller's z array.  Launch 2, one workgroup per (layer, batch
// row, 64 output rows): those rows of W_out (their first K_T P columns) against z.  Both are
// weight-streaming dot products: each wave walks one row at a time with 16-byte loads, two
// rows interleaved.
#include "essh_internal.h"
#include "lane_ops.h"

namespace essh {
namespace {

constexpr int FT = 256;        // threads per workgroup of launch 2 (4 waves)
constexpr int OUT_ROWS = 64;   // output rows per workgroup of launch 2
// Launch 1 takes 8 waves per channel with 4 chunks per row and lane in flight when its grid is
// about one workgroup per CU or less (few retained channels), else 4 waves with 8 chunks: at
// the 24-layer, d = 4096 decode shape the former is 20% faster at K_T = 8 and the latter at
// K_T = 16 to 32, where 8 waves with 8 chunks each put too many loads in flight per CU.
constexpr int SMALL_GRID = 256;

// dot of 8 bf16 weights (one 16-byte load) with 8 fp32 values in LDS
__device__ __forceinline__ float dot8(uint4 w, const float* s) {
    const float4 a = *reinterpret_cast<const float4*>(s);
    const float4 c = *reinterpret_cast<const float4*>(s + 4);
    float r = __uint_as_float(w.x << 16) * a.x;
    r += __uint_as_float(w.x & 0xffff0000u) * a.y;
    r += __uint_as_float(w.y << 16) * a.z;
    r += __uint_as_float(w.y & 0xffff0000u) * a.w;
    r += __uint_as_float(w.z << 16) * c.x;
    r += __uint_as_float(w.z & 0xffff0000u) * c.y;
    r += __uint_as_float(w.w << 16) * c.z;
    r += __uint_as_float(w.w & 0xffff0000u) * c.w;
    return r;
}

// Two rows (r0, r1 < 0: none) of n bf16 weights each against s[0, n), by one wave; n % 8 == 0.
// Every load of a round (RQ 16-byte chunks of each row per lane) goes out before the first is
// used.
// Returns both sums in every lane.
template <int RQ>
__device__ __forceinline__ float2 rows2(const uint16_t* w0, const uint16_t* w1, bool has1, const float* s, int n,
                                        int lane) {
    float a0 = 0.f, a1 = 0.f;
    for (int e0 = lane * 8; e0 < n; e0 += RQ * 512) {
        uint4 x0[RQ], x1[RQ];
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
            const int e = e0 + q * 512;
            x0[q] = e < n ? *reinterpret_cast<const uint4*>(w0 + e) : make_uint4(0u, 0u, 0u, 0u);
            x1[q] = (has1 && e < n) ? *reinterpret_cast<const uint4*>(w1 + e) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
            const int e = e0 + q * 512;
            if (e < n) {
                a0 += dot8(x0[q], s + e);
                a1 += dot8(x1[q], s + e);
            }
        }
    }
    return make_float2(wave_sum64(a0), wave_sum64(a1));
}

template <int M, int P, typename IO, int FTC, int RQ>
__global__ void __launch_bounds__(FTC) fused_channel_kernel(FusedDecodeArgs a) {
    extern __shared__ float us[];               // u of this (layer, batch row), fp32
    constexpr int R = P + 3 * M;                // value rows, then (mode, {write, read, clock}) rows
    __shared__ float rowv[R];
    __shared__ float ms_sh;
    using io = io_traits<IO>;
    const int k = blockIdx.x, b = blockIdx.y, l = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = a.d_model, K = a.K, B = a.B;

    const IO* u = static_cast<const IO*>(a.u) + ((size_t)l * B + b) * D;
    for (int e = tid; e < D; e += FTC) us[e] = io::load(u, e);
    __syncthreads();

    constexpr int NWC = FTC / 64;               // waves; wave w takes rows w, w + NWC, w + 2 NWC, ...
    const uint16_t* w_in = a.w_in + ((size_t)l * K + k) * P * (size_t)D;
    const uint16_t* w_ctl = a.w_ctl + ((size_t)l * K + k) * (3 * M) * (size_t)D;
    auto row_ptr = [&](int r) { return r < P ? w_in + (size_t)r * D : w_ctl + (size_t)(r - P) * D; };
    for (int r = wave; r < R; r += 2 * NWC) {
        const bool has1 = r + NWC < R;
        const float2 s = rows2<RQ>(row_ptr(r), row_ptr(has1 ? r + NWC : r), has1, us, D, lane);
        if (lane == 0) {
            rowv[r] = s.x;
            if (has1) rowv[r + NWC] = s.y;
        }
    }
    __syncthreads();

    // Eq. 23: statistic over this channel's P values only
    if (wave == 0) {
        float s = 0.f;
        for (int p = lane; p < P; p += 64) s += rowv[p] * rowv[p];
        s = wave_sum64(s);
        if (lane == 0) ms_sh = s / (float)P;
    }
    __syncthreads();
    const float bt = a.beta[(size_t)l * K + k];
    const float vscale = (1.f - bt) + bt * rsqrtf(ms_sh + a.eps_norm);

    if (tid < P) {
        const int p = tid;
        const float v = rowv[p] * vscale;
        const size_t tb = (size_t)l * K + k;   // modal tables of this channel
        float* st = a.state + ((((size_t)l * B + b) * K + k) * M) * 2 * P + p;
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const float* bc = a.b_ctl + (tb * M + j) * 3;
            const float aw = rowv[P + 3 * j] + bc[0];
            const float ar = rowv[P + 3 * j + 1] + bc[1];
            const float ad = rowv[P + 3 * j + 2] + bc[2];
            const float gw = 2.f / (1.f + expf(-aw));
            const float gr = 2.f / (1.f + expf(-ar));
            const float dl = fmaxf(ad, 0.f) + log1pf(expf(-fabsf(ad)));   // softplus
            const float rj = a.rho[tb * M + j] * expf(-dl);
            float sn, cs;
            sincosf(a.theta[tb * M + j], &sn, &cs);
            const float lr = rj * cs, li = rj * sn;
            const float hr = st[(size_t)(2 * j) * P], hi = st[(size_t)(2 * j + 1) * P];
            const float w = gw * v;
            const float nr = lr * hr - li * hi + w;
            const float ni = li * hr + lr * hi;
            st[(size_t)(2 * j) * P] = nr;
            st[(size_t)(2 * j + 1) * P] = ni;
            const float cr = a.c[(tb * M + j) * 2], ci = a.c[(tb * M + j) * 2 + 1];
            z += gr * (cr * nr - ci * ni);
            if (a.zl) z -= a.zl[tb * M + j] * gr * gw * cr * v;   // Eq. 24
        }
        a.z[(((size_t)l * B + b) * K + k) * P + p] = z;
    }
}

__global__ void __launch_bounds__(FT) fused_out_kernel(FusedDecodeArgs a) {
    extern __shared__ float zs[];               // z of the retained channels, [K_T][P]
    const int b = blockIdx.y, l = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = a.d_model, KPt = a.K_T * a.P, KP = a.K * a.P;
    const float* z = a.z + ((size_t)l * a.B + b) * KP;
    for (int i = tid; i < KPt; i += FT) zs[i] = z[i];
    __syncthreads();
    const float scale = rsqrtf((float)a.K_T);
    const int o0 = blockIdx.x * OUT_ROWS;
    for (int r = wave; r < OUT_ROWS; r += 8) {
        const int o = o0 + r;
        if (o >= D) break;
        const bool has1 = r + 4 < OUT_ROWS && o + 4 < D;
        const uint16_t* w0 = a.w_out + ((size_t)l * D + o) * KP;
        const float2 s = rows2<8>(w0, has1 ? w0 + 4 * (size_t)KP : w0, has1, zs, KPt, lane);
        if (lane == 0) {
            a.y[((size_t)l * a.B + b) * D + o] = s.x * scale;
            if (has1) a.y[((size_t)l * a.B + b) * D + o + 4] = s.y * scale;
        }
    }
}

template <int M, typename IO, int FTC, int RQ>
hipError_t launch_channels_shape(const FusedDecodeArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)a.K_T, (unsigned)a.B, (unsigned)a.n_layers);
    const size_t lds = (size_t)a.d_model * sizeof(float);
    switch (a.P) {
        case 16: hipLaunchKernelGGL((fused_channel_kernel<M, 16, IO, FTC, RQ>), grid, dim3(FTC), lds, s, a); break;
        case 32: hipLaunchKernelGGL((fused_channel_kernel<M, 32, IO, FTC, RQ>), grid, dim3(FTC), lds, s, a); break;
        case 64: hipLaunchKernelGGL((fused_channel_kernel<M, 64, IO, FTC, RQ>), grid, dim3(FTC), lds, s, a); break;
        case 128: hipLaunchKernelGGL((fused_channel_kernel<M, 128, IO, FTC, RQ>), grid, dim3(FTC), lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int M, typename IO>
hipError_t launch_channels(const FusedDecodeArgs& a, hipStream_t s) {
    const long long wgs = (long long)a.K_T * a.B * a.n_layers;
    return wgs <= SMALL_GRID ? launch_channels_shape<M, IO, 512, 4>(a, s) : launch_channels_shape<M, IO, 256, 8>(a, s);
}

template <typename IO>
hipError_t launch_channels_io(const FusedDecodeArgs& a, hipStream_t s) {
    switch (a.m) {
        case 1: return launch_channels<1, IO>(a, s);
        case 2: return launch_channels<2, IO>(a, s);
        case 4: return launch_channels<4, IO>(a, s);
        case 8: return launch_channels<8, IO>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_fused(const FusedDecodeArgs& a, int io_dtype, hipStream_t s) {
    if (a.n_layers == 0 || a.B == 0) return hipSuccess;
    const hipError_t e = io_dtype == ESSH_BF16 ? launch_channels_io<uint16_t>(a, s) : launch_channels_io<float>(a, s);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((a.d_model + OUT_ROWS - 1) / OUT_ROWS), (unsigned)a.B, (unsigned)a.n_layers);
    hipLaunchKernelGGL(fused_out_kernel, grid, dim3(FT), (size_t)a.K_T * a.P * sizeof(float), s, a);
    return hipGetLastError();
}

}  // namespace essh
