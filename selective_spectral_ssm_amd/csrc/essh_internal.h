// essh_internal.h -- private declarations shared by the HIP sources of libessh.
//
// Kernels are written for gfx950 (CDNA4): wave64, MFMA bf16 16x16x32 /
// 16x16x16, 160 KB LDS per CU, 8 XCDs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/essh.h"

namespace essh {

// ---------------------------------------------------------------------------
// Small numeric helpers
// ---------------------------------------------------------------------------

// bf16 <-> fp32 on raw 16-bit patterns.  The upcast is exact; the downcast
// rounds to nearest even (gfx950 has a hardware conversion for it).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

template <typename IO> struct io_traits;
template <> struct io_traits<float> {
    __device__ static __forceinline__ float load(const float* p, size_t i) { return p[i]; }
    __device__ static __forceinline__ void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct io_traits<uint16_t> {
    __device__ static __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
    __device__ static __forceinline__ void store(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16(x); }
};

// ---------------------------------------------------------------------------
// Launch descriptions (plain structs passed by value to kernels)
// ---------------------------------------------------------------------------

struct PrefillArgs {
    int B, L, K, K_T, Lc;
    int per_mode;
    const void* v;
    const float* delta;
    const void* g_w;
    const void* g_r;
    const float* rho;
    const float* theta;
    const float* c;
    const float* state_in;
    float* state_out;
    void* y;
    void* workspace;
    size_t workspace_bytes;
};

struct DecodeArgs {
    int n_layers, B, K, K_T;
    int per_mode;
    const void* v;
    const float* delta;
    const void* g_w;
    const void* g_r;
    const float* rho;
    const float* theta;
    const float* c;
    float* state;
    void* y;
};

// Launchers (host side).  Each returns hipSuccess or the launch error.
hipError_t launch_prefill_sequential(const PrefillArgs& a, int m, int P, int io_dtype, hipStream_t s);
hipError_t launch_prefill_chunked(const PrefillArgs& a, int m, int P, hipStream_t s);
bool chunked_supported(int m, int P, int Lc, int io_dtype, int per_mode);
size_t chunked_workspace_bytes(int B, int L, int K_T, int m, int P, int Lc);
hipError_t launch_decode(const DecodeArgs& a, int m, int P, int io_dtype, hipStream_t s);
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s);
hipError_t launch_copy_state(const float* src, float* dst, int B, int K, int K_T, int m, int P, hipStream_t s);

}  // namespace essh
