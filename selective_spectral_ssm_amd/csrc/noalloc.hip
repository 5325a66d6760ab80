// noalloc.hip -- essh_mixer_prefill_noalloc: the chunked prefill with its look-back records and
// control copies in a file-scope device array instead of a caller workspace, for callers that
// cannot allocate device memory.
//
// The array (scratch) exists once per GPU the library runs on and lives until the process
// ends.  Host code never passes its name to a kernel (on the host that name is only a stand-in):
// the first call on a device looks up the array's device address with hipGetSymbolAddress,
// with that device current, and every later call on that device uses the stored address.
// Each call clears what must start at zero (the scan header and the look-back flags) with a
// fill kernel, so it does not depend on what an earlier call left there.
#include <mutex>

#include "essh_internal.h"

namespace {

constexpr size_t SCRATCH_BYTES = ESSH_NOALLOC_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;

__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex g_mu;
void* g_scratch[MAX_DEVICES];   // device address of scratch on each device, once looked up

// Device address of this device's scratch array; null on failure.
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

// *dst |= *src, by one lane (the scan error word of this call into the caller's word)
__global__ void or_word_kernel(const unsigned* src, unsigned* dst) {
    if (threadIdx.x == 0) {
        const unsigned x = *src;
        if (x) *dst |= x;
    }
}

}  // namespace

extern "C" essh_status essh_mixer_prefill_noalloc(const essh_dims* d,
                                                  const void* v, const float* delta, const void* g_w,
                                                  const void* g_r, const float* rho, const float* theta,
                                                  const float* c, const float* zl, const float* state_in,
                                                  float* state_out, void* y, uint32_t* scan_error,
                                                  hipStream_t stream) {
    // Host-side checks come first: invalid dims give need = 0 and are rejected below by the
    // prefill entry point before anything is launched.
    const size_t need = essh_prefill_workspace_bytes(d);
    if (need > SCRATCH_BYTES) return ESSH_ERR_SCRATCH;
    if (scan_error && (reinterpret_cast<uintptr_t>(scan_error) & 3u)) return ESSH_ERR_INVALID_ARG;
    if (need == 0)
        return essh_mixer_prefill(d, v, delta, g_w, g_r, rho, theta, c, zl, state_in, state_out, y, nullptr, 0,
                                  stream);
    void* ws = scratch_ptr();
    if (!ws) return ESSH_ERR_HIP;
    const size_t clear = essh::prefill_clear_bytes(d);
    if (clear > 0 && essh::launch_fill_zero(static_cast<float*>(ws), clear / sizeof(float), stream) != hipSuccess)
        return ESSH_ERR_HIP;
    const essh_status st = essh_mixer_prefill(d, v, delta, g_w, g_r, rho, theta, c, zl, state_in, state_out, y, ws,
                                              SCRATCH_BYTES, stream);
    if (st != ESSH_OK || !scan_error) return st;
    hipLaunchKernelGGL(or_word_kernel, dim3(1), dim3(64), 0, stream,
                       static_cast<const unsigned*>(ws) + essh::SCAN_HDR_ERROR, reinterpret_cast<unsigned*>(scan_error));
    return hipGetLastError() == hipSuccess ? ESSH_OK : ESSH_ERR_HIP;
}
