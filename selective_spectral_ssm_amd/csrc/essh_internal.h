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
    const float* zl;          // zero-lag coefficients [K, m] (Eq. 24) or null
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
    const float* zl;          // zero-lag coefficients [n_layers, K, m] or null
    float* state;
    void* y;
};

struct FusedDecodeArgs {
    int n_layers, B, K, K_T, m, P, d_model;
    float eps_norm;
    const void* u;            // [n_layers, B, d_model] io dtype
    const uint16_t* w_in;     // [n_layers, K, P, d_model] bf16
    const float* beta;        // [n_layers, K]
    const uint16_t* w_ctl;    // [n_layers, K, m, 3, d_model] bf16
    const float* b_ctl;       // [n_layers, K, m, 3]
    const float* rho;
    const float* theta;
    const float* c;
    const float* zl;          // or null
    const uint16_t* w_out;    // [n_layers, d_model, K, P] bf16
    float* state;             // [n_layers, B, K, m, 2, P]
    float* z;                 // [n_layers, B, K, P]
    float* y;                 // [n_layers, B, d_model]
};

// Work split of the chunked prefill.  nseq = B * K_T sequences of nchunks
// chunks; each sequence is cut into nseg segments of seg_chunks chunks, one
// workgroup per (sequence, segment).  With nseg > 1 the workspace holds the
// look-back state of the segmented scan:
//   hdr   [SCAN_HDR_WORDS]          epoch, error bits and completion count (first 128-byte
//                                   line), then 8 ticket and 8 done counters, one line each
//   flags [nseq * nseg]             (epoch tag << 2) | FLAG_AGG / FLAG_INCL
//   lam   [nseq * nseg][2m]         segment transfer Lambda_j (re, im)
//   agg   [nseq * nseg][2m][P]      end state reached from a zero entering state
//   incl  [nseq * nseg][2m][P]      true end state
// The one-wave-per-segment kernel (wave = 1) always has the header, and after the
// arrays above its channel-major controls:
//   cdl   [nseq][L]                 clock delta of sequence b K_T + k
//   cgg   [nseq][L]                 write gate bits | read gate bits << 16
// The header must be zero before the first launch that uses the workspace;
// each launch leaves it re-armed for the next one.
enum {
    SCAN_HDR_EPOCH = 0,
    SCAN_HDR_ERROR = 1,
    SCAN_HDR_XDONE = 2,
    SCAN_HDR_STRIDE = 32,                    // one 128-byte line per counter
    SCAN_HDR_TICKET0 = 1 * SCAN_HDR_STRIDE,
    SCAN_HDR_DONE0 = 9 * SCAN_HDR_STRIDE,
    SCAN_HDR_WORDS = 17 * SCAN_HDR_STRIDE
};
enum : unsigned { SCAN_ERR_TIMEOUT = 1u, SCAN_ERR_TICKET = 2u };

// How a chunked prefill launch covers the sequences (one per batch row and
// retained channel):
//   SCAN_WHOLE     one workgroup streams a whole sequence;
//   SCAN_LOOKBACK  segments of a sequence in one launch, each obtaining its
//                  entering state by a decoupled look-back over its predecessors;
//   SCAN_SPLIT     three launches: segment aggregates, a scan over segments,
//                  then every segment streamed from its entering state.
enum { SCAN_WHOLE = 0, SCAN_LOOKBACK = 1, SCAN_SPLIT = 2 };

struct ScanPlan {
    int mode;
    int wave;                 // 1: the one-wave-per-segment kernel (prefill_wave.hip)
    int L;
    int nseq, nchunks, seg_chunks, nseg, nblocks;
    unsigned* hdr;
    unsigned* flags;
    float* lam;
    float* agg;
    float* incl;
    float* cdl;
    uint32_t* cgg;
};

// Launchers (host side).  Each returns hipSuccess or the launch error.
hipError_t launch_prefill_sequential(const PrefillArgs& a, int m, int P, int io_dtype, hipStream_t s);
hipError_t launch_prefill_f32_chunked(const PrefillArgs& a, int m, int P, hipStream_t s);
bool chunked_supported(int m, int P, int Lc, int io_dtype, int per_mode);
ScanPlan plan_chunked(int B, int L, int K_T, int m, int P, int Lc, int per_mode);
size_t chunked_workspace_bytes(int B, int L, int K_T, int m, int P, int Lc, int per_mode);
void bind_workspace(ScanPlan& plan, void* workspace, int m, int P);
hipError_t launch_prefill_chunked(const PrefillArgs& a, int m, int P, const ScanPlan& plan, hipStream_t s);
hipError_t launch_prefill_chunked_pm(const PrefillArgs& a, int m, int P, const ScanPlan& plan, hipStream_t s);
bool wave_supported(int m, int P, int Lc, int io_dtype, int per_mode);
hipError_t launch_prefill_wave(const PrefillArgs& a, int m, const ScanPlan& plan, hipStream_t s);
hipError_t launch_seg_scan(const ScanPlan& plan, int m, int P, hipStream_t s);
// Leading workspace bytes that must be zero before a prefill with dims d (scan header and
// look-back flags); 0 when the plan keeps no look-back records.
size_t prefill_clear_bytes(const essh_dims* d);
hipError_t launch_decode(const DecodeArgs& a, int m, int P, int io_dtype, hipStream_t s);
hipError_t launch_decode_fused(const FusedDecodeArgs& a, int io_dtype, hipStream_t s);
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s);
hipError_t launch_copy_state(const float* src, float* dst, int B, int K, int K_T, int m, int P, hipStream_t s);

}  // namespace essh
