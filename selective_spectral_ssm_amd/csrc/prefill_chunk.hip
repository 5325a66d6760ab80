// prefill_chunk.hip -- launches of the chunked parallel scan (per-channel controls), the
// segment scan of the three-launch form, the planner that picks the scan form, and the
// workspace layout.  The kernel itself is in prefill_chunk_kernel.h; ESSH paper, Sec. 4.3.
#include "prefill_chunk_kernel.h"

namespace essh {
namespace {

// Aggregates per workgroup of the segment scan.
constexpr int SCAN_PER = 16;

// Entering states of the segments of every sequence from the segment
// aggregates: E_1 = S_0 (segment 0's aggregate starts from state_in) and
// E_{s+1} = Lambda_s E_s + S_s, the composition of Eq. 6's affine maps.  One
// workgroup per (sequence, mode, PC value columns); thread (p, grp) composes the
// aggregates of segments [16 grp, 16 grp + 16) for value column p, the groups'
// compositions are exchanged through LDS, and each group then writes its entering
// states.  Sixteen columns per workgroup spread the launch over more CUs than one
// workgroup per (sequence, mode) would; with few segments per sequence (fewer than 64
// threads at 16 columns) a workgroup takes more columns, up to P.
__global__ void __launch_bounds__(1024) seg_scan_kernel(ScanPlan plan, int m, int P, int PC) {
    __shared__ float4 comp[1024];
    const int ROWS = 2 * m;
    const int seq = blockIdx.x / m, j = blockIdx.x - seq * m;
    const int pl = threadIdx.x % PC, grp = threadIdx.x / PC;
    const int p = blockIdx.y * PC + pl;
    const int nag = plan.nseg - 1;
    const int s0 = grp * SCAN_PER;
    const size_t slot = (size_t)seq * plan.nseg;
    float lr[SCAN_PER], li[SCAN_PER], sr[SCAN_PER], si[SCAN_PER];
#pragma unroll
    for (int i = 0; i < SCAN_PER; ++i) {
        const int sg = s0 + i;
        if (sg < nag) {
            lr[i] = plan.lam[(slot + sg) * ROWS + 2 * j];
            li[i] = plan.lam[(slot + sg) * ROWS + 2 * j + 1];
            sr[i] = plan.agg[((slot + sg) * ROWS + 2 * j) * (size_t)P + p];
            si[i] = plan.agg[((slot + sg) * ROWS + 2 * j + 1) * (size_t)P + p];
        } else {
            lr[i] = 1.f;
            li[i] = 0.f;
            sr[i] = 0.f;
            si[i] = 0.f;
        }
    }
    // composition of this group's maps: x -> A x + Bv
    float ar = 1.f, ai = 0.f, br = 0.f, bi = 0.f;
#pragma unroll
    for (int i = 0; i < SCAN_PER; ++i) {
        const float nar = lr[i] * ar - li[i] * ai, nai = lr[i] * ai + li[i] * ar;
        const float nbr = lr[i] * br - li[i] * bi + sr[i], nbi = lr[i] * bi + li[i] * br + si[i];
        ar = nar;
        ai = nai;
        br = nbr;
        bi = nbi;
    }
    comp[threadIdx.x] = make_float4(ar, ai, br, bi);
    __syncthreads();
    float hr = 0.f, hi = 0.f;   // value entering this group's first segment map
    for (int q = 0; q < grp; ++q) {
        const float4 f = comp[q * PC + pl];
        const float nr = f.x * hr - f.y * hi + f.z, ni = f.x * hi + f.y * hr + f.w;
        hr = nr;
        hi = ni;
    }
#pragma unroll
    for (int i = 0; i < SCAN_PER; ++i) {
        const int sg = s0 + i;
        if (sg < nag) {
            const float nr = lr[i] * hr - li[i] * hi + sr[i], ni = lr[i] * hi + li[i] * hr + si[i];
            hr = nr;
            hi = ni;
            plan.incl[((slot + sg + 1) * ROWS + 2 * j) * (size_t)P + p] = hr;
            plan.incl[((slot + sg + 1) * ROWS + 2 * j + 1) * (size_t)P + p] = hi;
        }
    }
}

template <int P, int M, int LC>
hipError_t launch_cfg(const PrefillArgs& a, const ScanPlan& plan, hipStream_t s) {
    using C = Cfg<P, M, LC>;
    if (plan.nblocks == 0) return hipSuccess;
    if (plan.mode == SCAN_LOOKBACK) {
        hipLaunchKernelGGL((prefill_chunk_kernel<C, MODE_LOOKBACK>), dim3((unsigned)plan.nblocks), dim3(C::THREADS),
                           0, s, a, plan);
        return hipGetLastError();
    }
    if (plan.mode == SCAN_SPLIT && plan.nseg > 1) {
        const int nagg = plan.nseq * (plan.nseg - 1);   // every segment but the last
        hipLaunchKernelGGL((prefill_chunk_kernel<C, MODE_AGG>), dim3((unsigned)nagg), dim3(C::THREADS), 0, s, a,
                           plan);
        const hipError_t e = launch_seg_scan(plan, M, P, s);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((prefill_chunk_kernel<C, MODE_STREAM>), dim3((unsigned)plan.nblocks), dim3(C::THREADS), 0, s,
                       a, plan);
    return hipGetLastError();
}

template <int P, int M>
hipError_t launch_lc(const PrefillArgs& a, const ScanPlan& plan, hipStream_t s) {
    switch (a.Lc) {
        case 32: return launch_cfg<P, M, 32>(a, plan, s);
        case 64: return launch_cfg<P, M, 64>(a, plan, s);
        case 128: return launch_cfg<P, M, 128>(a, plan, s);
        default: return hipErrorInvalidValue;
    }
}

template <int P>
hipError_t launch_m(const PrefillArgs& a, int m, const ScanPlan& plan, hipStream_t s) {
    switch (m) {
        case 1: return launch_lc<P, 1>(a, plan, s);
        case 2: return launch_lc<P, 2>(a, plan, s);
        case 4: return launch_lc<P, 4>(a, plan, s);
        case 8: return launch_lc<P, 8>(a, plan, s);
        default: return hipErrorInvalidValue;
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool chunked_supported(int m, int P, int Lc, int io_dtype, int per_mode) {
    const bool mok = m == 1 || m == 2 || m == 4 || m == 8;
    const bool pok = P == 16 || P == 32 || P == 64 || P == 128;
    const bool lok = Lc == 32 || Lc == 64 || Lc == 128;
    (void)per_mode;   // per-channel and per-mode controls
    return mok && pok && lok && io_dtype == ESSH_BF16;
}

ScanPlan plan_chunked(int B, int L, int K_T, int m, int P, int Lc, int per_mode) {
    ScanPlan p{};
    p.L = L;
    p.nseq = B * K_T;
    p.nchunks = (L + Lc - 1) / Lc;
    if (p.nseq == 0 || p.nchunks == 0) return p;
    constexpr int SPLIT_MAX_SEQ = 32;
    if (p.nseq <= SPLIT_MAX_SEQ && wave_supported(m, P, Lc, ESSH_BF16, per_mode)) {
        // Few, long sequences with P = 64: the three-launch scan with one wave per (sequence,
        // segment) (prefill_wave.hip).  The segment length is picked between the shortest the
        // segment scan composes and twice that, to fill the last round of WAVE_SLOTS resident
        // waves (eight one-wave workgroups per CU on 256 CUs) as fully as possible, the shorter
        // length on a tie: a round that is only started (say 4104 waves on 2048 slots) costs
        // almost a whole round's time, while more and shorter segments cost the aggregate and
        // segment-scan launches little.
        constexpr long long WAVE_SLOTS = 2048;
        p.wave = 1;
        int seg_chunks = p.nchunks;
        p.mode = SCAN_SPLIT;
        {
            const int max_seg = 1 + SCAN_PER * (1024 / P);
            const int lo = (p.nchunks + max_seg - 1) / max_seg;
            double best = -1.0;
            for (int c = lo; c <= 2 * lo && c <= p.nchunks; ++c) {
                const long long waves = (long long)p.nseq * ((p.nchunks + c - 1) / c);
                const long long rounds = (waves + WAVE_SLOTS - 1) / WAVE_SLOTS;
                const double fill = (double)waves / (double)(rounds * WAVE_SLOTS);
                if (fill > best + 1e-9) {
                    best = fill;
                    seg_chunks = c;
                }
            }
        }
        if (seg_chunks < 1) seg_chunks = 1;
        if (seg_chunks > p.nchunks) seg_chunks = p.nchunks;
        p.seg_chunks = seg_chunks;
        p.nseg = (p.nchunks + seg_chunks - 1) / seg_chunks;
        p.nblocks = p.nseq * p.nseg;
        if (p.nseg == 1) p.mode = SCAN_WHOLE;
        return p;
    }
    // With about 1.5 sequences per CU or more (one per CU when P = 128), whole
    // sequences keep the GPU busy.  Below that, sequences are cut into segments of as many chunks as
    // a workgroup keeps resident in LDS, and a look-back scan links them.
    // With very few sequences a round of resident workgroups (about 1000)
    // covers many segments of each sequence, so each look-back would fold
    // dozens of predecessors; there the three-launch scan is used instead,
    // with about SPLIT_TARGET segments overall (at most what one scan
    // workgroup composes per sequence).
    // Whole sequences from SEQ_ENOUGH sequences up: 384, or 256 when P = 128,
    // whose sequences carry twice the work per wave.  Measured on MI355X: P = 128
    // streams 256 whole sequences in 82 us against the look-back's 104 us, and 128
    // in 80 us against 51; P = 64 keeps the look-back at 192 sequences (41 us
    // against 63).
    const int SEQ_ENOUGH = P >= 128 ? 256 : 384;
    constexpr int SPLIT_TARGET = 1536;
    int seg_chunks = p.nchunks;
    p.mode = SCAN_WHOLE;
    // Per-mode controls have no look-back kernel: below SEQ_ENOUGH sequences
    // they always take the three-launch scan.
    if (p.nseq < SEQ_ENOUGH) {
        if (p.nseq <= SPLIT_MAX_SEQ || per_mode) {
            p.mode = SCAN_SPLIT;
            const long long want = ((long long)p.nchunks * p.nseq + SPLIT_TARGET - 1) / SPLIT_TARGET;
            const int max_seg = 1 + SCAN_PER * (1024 / P);
            const int min_chunks = (p.nchunks + max_seg - 1) / max_seg;
            seg_chunks = (int)(want > min_chunks ? want : min_chunks);
            if (per_mode && P >= 64) {
                // Per-mode controls with four-wave workgroups: the segment length that
                // minimises rounds x chunks per segment, where a round is the workgroup slots
                // of 256 CUs at three workgroups per CU (m <= 4) or two (m = 8); on a tie the
                // longer segment, which leaves the aggregate launch less to do.  Measured on
                // MI355X: the 370M-class per-mode call at K_T = 24 took 101 us with segments of
                // 8 chunks (one round) against 114 with 4 (two rounds), the 1.5B-class at
                // K_T = 8 110 against 137.5 with 3.
                const long long slots = 256LL * (m <= 4 ? 3 : 2);
                long long best = -1;
                for (int c = min_chunks; c <= p.nchunks; ++c) {
                    const long long wgs = (long long)p.nseq * ((p.nchunks + c - 1) / c);
                    const long long cost = ((wgs + slots - 1) / slots) * c;
                    if (best < 0 || cost <= best) {
                        best = cost;
                        seg_chunks = c;
                    }
                }
            }
        } else {
            p.mode = SCAN_LOOKBACK;
            seg_chunks = resident_chunks(P, Lc);
        }
    }
    if (seg_chunks < 1) seg_chunks = 1;
    if (seg_chunks > p.nchunks) seg_chunks = p.nchunks;
    p.seg_chunks = seg_chunks;
    p.nseg = (p.nchunks + seg_chunks - 1) / seg_chunks;
    p.nblocks = p.nseq * p.nseg;
    if (p.nseg == 1) p.mode = SCAN_WHOLE;
    // The look-back launch's eight ticket counters each own whole sequences (at
    // most ceil(nseq / 8)); its grid gives every counter as many workgroups as
    // the largest one has segments, the rest exit at once.
    if (p.mode == SCAN_LOOKBACK) p.nblocks = 8 * ((p.nseq + 7) / 8) * p.nseg;
    (void)m;
    return p;
}

// Byte offsets of the workspace arrays (see ScanPlan); an array that the plan does not use
// has none.
struct WsLayout {
    size_t hdr, flags, lam, agg, incl, cdl, cgg, total;
    bool has_hdr, has_scan, has_ctrl;
};

WsLayout ws_layout(const ScanPlan& p, int m, int P) {
    WsLayout w{};
    w.has_scan = p.nseg > 1;
    w.has_ctrl = p.wave != 0;
    w.has_hdr = w.has_scan || w.has_ctrl;
    size_t off = 0;
    if (w.has_hdr) {
        w.hdr = off;
        off += align256(SCAN_HDR_WORDS * sizeof(unsigned));
    }
    if (w.has_scan) {
        const size_t slots = (size_t)p.nseq * p.nseg;
        w.flags = off;
        off += align256(slots * sizeof(unsigned));
        w.lam = off;
        off += align256(slots * 2 * m * sizeof(float));
        w.agg = off;
        off += align256(slots * 2 * (size_t)m * P * sizeof(float));
        w.incl = off;
        off += align256(slots * 2 * (size_t)m * P * sizeof(float));
    }
    if (w.has_ctrl) {
        const size_t n = (size_t)p.nseq * p.L;
        w.cdl = off;
        off += align256(n * sizeof(float));
        w.cgg = off;
        off += align256(n * sizeof(uint32_t));
    }
    w.total = off;
    return w;
}

size_t prefill_clear_bytes(const essh_dims* d) {
    if (!d || essh_prefill_workspace_bytes(d) == 0) return 0;
    const int lc = d->Lc == 0 ? 64 : d->Lc;
    const ScanPlan p = plan_chunked(d->B, d->L, d->K_T, d->m, d->P, lc, d->ctrl_per_mode);
    const WsLayout w = ws_layout(p, d->m, d->P);
    if (w.has_scan) return w.lam;
    return w.has_hdr ? align256(SCAN_HDR_WORDS * sizeof(unsigned)) : 0;
}

size_t chunked_workspace_bytes(int B, int L, int K_T, int m, int P, int Lc, int per_mode) {
    const ScanPlan p = plan_chunked(B, L, K_T, m, P, Lc, per_mode);
    if (p.nblocks == 0) return 0;
    return ws_layout(p, m, P).total;
}

void bind_workspace(ScanPlan& p, void* ws, int m, int P) {
    const WsLayout w = ws_layout(p, m, P);
    char* base = static_cast<char*>(ws);
    if (w.has_hdr) p.hdr = reinterpret_cast<unsigned*>(base + w.hdr);
    if (w.has_scan) {
        p.flags = reinterpret_cast<unsigned*>(base + w.flags);
        p.lam = reinterpret_cast<float*>(base + w.lam);
        p.agg = reinterpret_cast<float*>(base + w.agg);
        p.incl = reinterpret_cast<float*>(base + w.incl);
    }
    if (w.has_ctrl) {
        p.cdl = reinterpret_cast<float*>(base + w.cdl);
        p.cgg = reinterpret_cast<uint32_t*>(base + w.cgg);
    }
}

hipError_t launch_seg_scan(const ScanPlan& plan, int m, int P, hipStream_t s) {
    const int ngrp = (plan.nseg - 1 + SCAN_PER - 1) / SCAN_PER;
    // value columns per workgroup: 16, or more (a power of two dividing P) until the
    // workgroup fills a wave, so that few segments per sequence do not launch thousands of
    // quarter-wave workgroups
    int PC = P < 16 ? P : 16;
    while (2 * PC <= P && PC * ngrp < 64) PC *= 2;
    hipLaunchKernelGGL(seg_scan_kernel, dim3((unsigned)(plan.nseq * m), (unsigned)(P / PC)),
                       dim3((unsigned)(PC * ngrp)), 0, s, plan, m, P, PC);
    return hipGetLastError();
}

hipError_t launch_prefill_chunked(const PrefillArgs& a, int m, int P, const ScanPlan& plan, hipStream_t s) {
    if (a.per_mode) return launch_prefill_chunked_pm(a, m, P, plan, s);
    if (plan.wave) return launch_prefill_wave(a, m, plan, s);
    switch (P) {
        case 16: return launch_m<16>(a, m, plan, s);
        case 32: return launch_m<32>(a, m, plan, s);
        case 64: return launch_m<64>(a, m, plan, s);
        case 128: return launch_m<128>(a, m, plan, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace essh
