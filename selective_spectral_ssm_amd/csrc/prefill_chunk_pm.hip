// prefill_chunk_pm.hip -- the chunked parallel scan with clock and gates per mode
// ([B, L, K, m]: the controls of Eq. 5 as the paper writes them, each mode with its own
// clock, write gate and read gate).  Same kernel as the per-channel scan (in
// prefill_chunk_kernel.h), instantiated for its per-mode launch modes: every 16-position
// sub-block forms its MFMA operands per element, summing the modes' contributions with
// their own gates and clocks.  Whole sequences, or the three-launch scan when there are
// few sequences; the segment scan between its launches is the per-channel one (the
// segment records do not depend on how the controls are laid out).
#include "prefill_chunk_kernel.h"

namespace essh {
namespace {

template <int P, int M, int LC>
hipError_t launch_cfg_pm(const PrefillArgs& a, const ScanPlan& plan, hipStream_t s) {
    using C = Cfg<P, M, LC>;
    if (plan.nblocks == 0) return hipSuccess;
    if (plan.mode == SCAN_LOOKBACK) return hipErrorInvalidValue;   // not planned for per-mode controls
    if (plan.mode == SCAN_SPLIT && plan.nseg > 1) {
        const int nagg = plan.nseq * (plan.nseg - 1);   // every segment but the last
        hipLaunchKernelGGL((prefill_chunk_kernel<C, MODE_AGG_PM>), dim3((unsigned)nagg), dim3(C::THREADS), 0, s, a,
                           plan);
        const hipError_t e = launch_seg_scan(plan, M, P, s);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((prefill_chunk_kernel<C, MODE_STREAM_PM>), dim3((unsigned)plan.nblocks), dim3(C::THREADS), 0,
                       s, a, plan);
    return hipGetLastError();
}

template <int P, int M>
hipError_t launch_lc_pm(const PrefillArgs& a, const ScanPlan& plan, hipStream_t s) {
    switch (a.Lc) {
        case 32: return launch_cfg_pm<P, M, 32>(a, plan, s);
        case 64: return launch_cfg_pm<P, M, 64>(a, plan, s);
        case 128: return launch_cfg_pm<P, M, 128>(a, plan, s);
        default: return hipErrorInvalidValue;
    }
}

template <int P>
hipError_t launch_m_pm(const PrefillArgs& a, int m, const ScanPlan& plan, hipStream_t s) {
    switch (m) {
        case 1: return launch_lc_pm<P, 1>(a, plan, s);
        case 2: return launch_lc_pm<P, 2>(a, plan, s);
        case 4: return launch_lc_pm<P, 4>(a, plan, s);
        case 8: return launch_lc_pm<P, 8>(a, plan, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill_chunked_pm(const PrefillArgs& a, int m, int P, const ScanPlan& plan, hipStream_t s) {
    switch (P) {
        case 16: return launch_m_pm<16>(a, m, plan, s);
        case 32: return launch_m_pm<32>(a, m, plan, s);
        case 64: return launch_m_pm<64>(a, m, plan, s);
        case 128: return launch_m_pm<128>(a, m, plan, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace essh
