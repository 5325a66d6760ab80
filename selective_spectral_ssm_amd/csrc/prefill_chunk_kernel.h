// prefill_chunk_kernel.h -- the chunked parallel scan kernel of the ESSH selective mixer on MFMA
// (included by prefill_chunk.hip, per-channel controls, and prefill_chunk_pm.hip, per-mode
// controls, which instantiate it for their launch modes in separate translation units).
//
// ESSH paper, Sec. 4.3 "Chunked parallel training" and Fig. 2A: positions are
// split into chunks; inside a chunk the source-to-target contributions form a
// dense causal matrix applied by matrix multiplication, and only the 2 m P
// mode-state entries of a channel cross a chunk boundary.  Eq. 6 (the
// transition product rho^{t-s} e^{-sum delta} R(theta (t-s))) makes this exact.
//
// Sub-blocks.  A chunk of Lc positions is processed as 16-position sub-blocks
// [T0, T0+16) carrying the mode state h (complex, per mode j and value p)
// from one to the next.  With lambda_j = rho_j e^{i theta_j}, psi(tau) =
// sum_j Re(c_j lambda_j^tau) and the clock measured from the sub-block start,
//   a(t) = e^{-(qh(t) - qh(T0-1))},   b(s) = e^{qh(s) - qh(T0-1)} g_w(s),
// the recurrence over the sub-block gives, for t, s in [T0, T0+16):
//   y(t) = g_r(t) a(t) [ sum_{s<=t} psi(t-s) b(s) v(s)
//                        + sum_j Re(c_j lambda_j^{t-T0+1} h_j) ]          (intra + carry)
//   h_j' = A_T ( lambda_j^16 h_j + sum_s lambda_j^{T0+15-s} b(s) v(s) ),
//   A_T = e^{-(qh(T0+15) - qh(T0-1))}.
// The matrices psi(t-s) [s<=t], Re/Im(c_j lambda_j^{t-T0+1}) and
// Re/Im(lambda_j^{15-s+T0}) are the same for every sub-block, so they are
// built once per channel as MFMA operands held in registers; per sub-block
// only v is scaled by b(s) and y by g_r(t) a(t).  Per 16 value columns that
// is two v_mfma_f32_16x16x32_bf16:
//   y^T = [b.v ; H_hi]^T [Psi^T ; C^T]         K = 16 positions + 16 state rows
//   M   = [Lpow_hi Lpow_lo] [b.v ; b.v]        K = 16 positions x hi/lo of the
//                                              lambda powers, b.v rounded to bf16 once
// and h' = A_T (lambda^16 h + M) on the VALU.  b(s) grows within a sub-block;
// a sub-block whose clock span could overflow it, and a ragged last one, take
// an exact per-element path instead (same MFMA shapes, operands from exps).
//
// Channels are independent (Sec. 4.1), so a workgroup owns one (batch row,
// channel) and walks the chunks of a segment of positions in order, keeping
// the channel's mode state in registers.
//
// Segmented scan.  When batch rows x retained channels alone cannot fill the
// GPU, each sequence of chunks is cut into segments handled by different
// workgroups.  The state entering a segment is the composition of the affine
// maps h -> Lambda h + S of the chunks before it (the same Eq. 6 algebra one
// level up).  A workgroup (i) sweeps its segment once computing only the end
// state reached from a zero state (its aggregate S_seg and transfer
// Lambda_seg), (ii) publishes it, (iii) obtains its entering state by a
// decoupled look-back over its predecessors' published aggregates / inclusive
// states, publishes its own inclusive state, and (iv) sweeps the segment
// again with the true entering state, now producing y.  The segment's chunks
// stay resident in LDS between the two sweeps, so v is read once.
//
// Three-launch scan.  With very few sequences the look-back chains get long;
// then (i) one launch computes every segment's aggregate (end state from a
// zero entering state, or from state_in for segment 0) and transfer, (ii) a
// small scan composes them per sequence into entering states, and (iii) every
// segment is streamed from its entering state producing y.  v is read twice.
//
// gfx950 mapping
//   * Each wave owns 16*NTW value columns for all positions: its share of the
//     state lives in VGPRs in the 16x16 MFMA accumulator layout (lane (g,col)
//     holds state rows 4g..4g+3 = (mode 2g, re/im), (mode 2g+1, re/im) of
//     column col).  Every product of one accumulation chain has one MFMA shape.
//   * v tiles are loaded with 16-byte loads one chunk ahead (streaming) or
//     copied global-to-LDS up front (look-back) into LDS blocked by 16-column
//     tiles, [P/16][Lc][16], so that one wave's columns are contiguous runs;
//     the MFMA fragments (four consecutive positions of one column) come back
//     with ds_read_b64_tr_b16.
//     y is staged in place and written with 16-byte stores.  The look-back
//     launch's first sweep writes b(s) v(s) back over the fragment it read,
//     and its output sweep reads those values instead of scaling v again.
//   * Look-back messages are written and read with agent-scope atomic
//     accesses (they bypass the per-XCD L2), flags carry a per-launch epoch,
//     and every wait is bounded.
#pragma once

#include <type_traits>

#include "essh_internal.h"

namespace essh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
// Read-only fp32 data addressed uniformly across a workgroup (constant address space).
typedef const __attribute__((address_space(4))) float* cfloat_p;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr float LOG2E = 1.4426950408889634f;
// Largest clock span of a sub-block, in log2 units, that the factored path
// takes: b(s) <= 2^64 g_w(s) keeps b(s) v(s) far from overflow.
constexpr float SPAN2_FAST_MAX = 64.f;
// Largest clock span of a 64-position block, in log2 units, that the block
// path takes: with the clock referenced to the middle of the block, a(t) and
// b(s) stay within 2^{+-64}, the same range the sub-block path allows.
constexpr float SPAN2_BLOCK_MAX = 128.f;

// Look-back flag kinds (low two bits of a flag word; the rest is the epoch tag).
constexpr unsigned FLAG_AGG = 1u;    // aggregate (end state from a zero entering state) and transfer
constexpr unsigned FLAG_INCL = 2u;   // inclusive state (true state after the segment)
// Upper bound on polls of one flag window (each poll is a memory round trip
// plus a short sleep, so this is tens of milliseconds); exceeding it records
// SCAN_ERR_TIMEOUT in the workspace header instead of waiting forever.
constexpr int SPIN_LIMIT = 1 << 16;
// Predecessor records a look-back reads per memory round trip (independent loads, then folded
// in order).
constexpr int LB_BATCH = 2;
// s_waitcnt operand: vector memory counter 0, the other counters unconstrained.
constexpr int WAIT_VMEM0 = 0x0F70;

}  // namespace

// Bytes of one staged chunk (v tile and per-position factors) and the number
// of chunks a segment keeps resident in LDS (a budget of 40 KB per workgroup).
constexpr int stage_bytes(int P, int LC) {
    return LC * P * 2 + 5 * LC * 4 + (LC / 16) * 8 + (LC / 32) * 16;
}
constexpr int resident_chunks(int P, int LC) {
    return 40960 / stage_bytes(P, LC) < 1 ? 1 : (40960 / stage_bytes(P, LC) > 4 ? 4 : 40960 / stage_bytes(P, LC));
}
namespace {

template <int P_, int M_, int LC_>
struct Cfg {
    static constexpr int P = P_, M = M_, LC = LC_;
    static constexpr int NT = P / 16;               // 16-column value tiles
    static constexpr int NW = NT < 4 ? NT : 4;      // waves per workgroup
    static constexpr int NTW = NT / NW;             // value tiles per wave
    static constexpr int THREADS = 64 * NW;
    static constexpr int WCOLS = 16 * NTW;          // value columns per wave
    static constexpr int NSB = LC / 16;             // 16-position sub-blocks per chunk
    // Arithmetic blocks: NB sub-blocks whose state is carried once per block;
    // at most 64 positions (the streamed path), 32 in the segmented path.
    static constexpr int NB = LC >= 64 ? 4 : LC / 16;
    static constexpr int BLK = 16 * NB;
    static constexpr int LPR = WCOLS / 8;           // lanes per v row (16 B each)
    static constexpr int RPI = 64 / LPR;            // v rows per wave load
    static constexpr int NLD = LC / RPI;            // wave loads per chunk
    static constexpr int CPL = (LC + 63) / 64;     // control positions per lane of wave 0
    // v tile in LDS: blocked by 16-column tiles, [P/16][LC][16] bf16, so that
    // the 16 rows of one tile form 512 contiguous bytes (a transposing
    // fragment read, and every copy or read of one wave's columns, is one
    // contiguous run).
    static constexpr int TBLK = LC * 16;            // elements of one 16-column tile block
    // chunks of a segment kept resident in LDS between the two sweeps
    static constexpr int RES = resident_chunks(P, LC);
    static_assert(P % 16 == 0 && NT % NW == 0, "P must be 16, 32, 64 or 128");
    static_assert(LC % 32 == 0 && LC <= 128, "chunk length must be 32, 64 or 128");
    static_assert(M >= 1 && M <= 8, "1..8 modes");
    static_assert(LC % RPI == 0, "v tile loads must tile the chunk");
    static_assert(RES >= 1 && RES <= 4, "one to four resident chunks");
};

// Per-chunk staged data.
template <class C>
struct __align__(16) Stage {
    float q2[C::LC];                 // chunk-local inclusive clock sum * log2(e) (the raw clock
                                     // while the segmented scan's copies are staged)
    float bq[C::LC];                 // b(s) = e^{qh(s)-qh(T0-1)} g_w(s)   (0 beyond the chunk)
    float ag[C::LC];                 // a(t) g_r(t) = e^{-(qh(t)-qh(T0-1))} g_r(t)
    float2 blk[C::NSB];              // per sub-block: (A_T, 1 if the exact path is needed)
    float4 blkB[C::LC / 32];         // per block: (H_s, A_e, Lambda_e, 1 if the sub-block path is needed);
                                     // Lambda_e = e^{-clock span} also on the sub-block path
    // Gates as bf16 bits in the low half of a 32-bit slot: a global-to-LDS copy
    // of 16-bit elements writes one 32-bit slot per lane.
    uint32_t gw[C::LC];              // write gate
    uint32_t gr[C::LC];              // read gate
};

// Per-mode controls of a staged chunk (per-mode launches only): clock sums
// * log2(e) and gates, [mode][position], and the factors of the clock
// referenced to the start T0 of each position's 16-position sub-block:
//   fa[j][t] = g_r,j(t) e^{-(q_j(t) - q_j(T0-1))},  fb[j][s] = g_w,j(s) e^{q_j(s) - q_j(T0-1)}
// (0 past the chunk's valid positions), so that g_r,j(t) e^{-(q_j(t)-q_j(s))} g_w,j(s)
// = fa[j][t] fb[j][s] for t, s in one sub-block; ftr[j][T] = e^{-(q_j(T1) - q_j(T0-1))},
// T1 the sub-block's last valid position; fexact[T] = 1 where some mode's clock
// span over the sub-block is too large to factor.
// For the output operand as a rank-2m product (G = U W^T masked to s <= t, with
// lambda^{t-s} = lambda^{t-T0} lambda^{T0-s}): ipw[e][j] = lambda_j^{-e}, e = 0..15;
// lowrho = 1 where some rho_j^{-15} exceeds 2^40, and the sub-blocks then form G element
// by element.
template <class C>
struct __align__(16) StagePM {
    float q[C::M][C::LC];
    float gw[C::M][C::LC];
    float gr[C::M][C::LC];
    float fa[C::M][C::LC];
    float fb[C::M][C::LC];
    float ftr[C::M][C::NSB];
    int fexact[C::NSB];
    float2 ipw[16][C::M];
    int lowrho;
    // The sub-blocks' operands in MFMA lane order ([G ; C hi], [C lo ; C hi], W hi and lo),
    // formed once per chunk by one wave each and read by every wave; chunks of at most four
    // sub-blocks (a longer chunk forms them in each wave, as LDS is short there).
    static constexpr int NOP = C::NSB <= 4 ? C::NSB : 1;
    bf16x8_t opg[NOP][64];
    bf16x8_t opgx[NOP][64];
    bf16x8_t opw[NOP][64];
};

// v tile of a staged chunk: [P/16][LC][16] bf16; y is staged in place.
template <class C>
struct __align__(16) VTile {
    uint16_t V[C::LC * C::P];
};

template <class C>
struct __align__(16) Smem {
    // lambda_j^tau, tau = 0..16, then (rows 17 + d) lambda_j^{16 d}, d = 0..NB: one
    // array, so that both kinds of entry are written by one store whose target
    // the compiler can still tell apart from the asynchronous tile copies
    float2 pw[17 + C::NB + 1][C::M];
    float2 cpw[17][C::M];            // c_j lambda_j^tau
    float psi[C::BLK];               // sum_j Re(c_j lambda_j^tau), tau = 0..BLK-1
    float4 mtab[C::M];               // (rho_j, theta_j, Re c_j, Im c_j) of the channel
    float mza[C::M];                 // zero-lag coefficients a_j (Eq. 24)
    int ticket;
    unsigned epoch;
    int lb_cnt;
    int lb_found;
};

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Work-item order when there is one segment per sequence: channel fastest,
// then batch row.  When the grid is a multiple of 8 the hardware's round-robin
// XCD assignment is undone so that each XCD receives a contiguous range of
// work items (neighbouring channels share the cache lines of the controls).
__device__ __forceinline__ int remap_xcd(int bid, int nblocks) {
    if ((nblocks & 7) != 0) return bid;
    return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

// Wait until this wave's outstanding memory operations have completed.  The
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void wait_stores_complete() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup barrier that orders LDS accesses only: it waits for this wave's
// LDS operations, not for its outstanding vector memory operations (a full
// __syncthreads also waits for asynchronous global-to-LDS copies still in
// flight).
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until at most N of this wave's vector memory operations are outstanding
// (they complete in issue order for this counter).
template <int N>
__device__ __forceinline__ void wait_vmem_at_most() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Calls f(std::integral_constant<int, I>()) for I = B .. E-1 in order.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>());
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ void st_agent(float* p, float x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_agent_u(const unsigned* p) {
    return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u(unsigned* p, unsigned x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bf16x8_t to_bf16x8(u16x8_t x) { return __builtin_bit_cast(bf16x8_t, x); }
// Two fp32 values -> one dword of two bf16 (round to nearest even), element 0 low.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}
// The low / high bf16 of a dword, exactly, as fp32.
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// Eight bf16 MFMA operand slots from two 4-slot halves.
__device__ __forceinline__ bf16x8_t bf16x8_of(uint2 a, uint2 b) {
    return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}

// Kernel roles (template argument MODE): a whole sequence or a segment streamed
// from its entering state (STREAM), a segment of a look-back scan (LOOKBACK),
// or the end state of a segment from a zero entering state (AGG); STREAM_PM and
// AGG_PM are STREAM and AGG with clock and gates per mode ([B, L, K, m], Eq. 5).
enum { MODE_STREAM = 0, MODE_LOOKBACK = 1, MODE_AGG = 2, MODE_STREAM_PM = 3, MODE_AGG_PM = 4 };

// Workgroups per CU that the register budget is held to.  Look-back launches
// keep a workgroup's chunks resident in LDS (four workgroups per CU would fit);
// with the carry readout's coefficients held in hi and lo halves their operands
// need three workgroups' budget (168 VGPRs): four spilled 80-130 bytes per lane
// and ran 370M-class tiers 15-25% slower, three runs them level with or faster
// than the former four without the lo halves.  Streaming and per-mode launches
// with up to four modes are held to three workgroups too.  The per-channel streaming
// launches fit 168 VGPRs; the per-mode streaming launch with P = 64 and m = 4 spills
// about 120 bytes per lane there (since the carry readout's lo halves and the output
// operand's MFMA form), and ran the 370M-class per-mode scan 6-11% faster than at two
// workgroups per CU when measured (K_T = 24: 156 against 166 us).  Four spilled more and
// was slower.  The per-mode streaming launch with m = 8 is held to two workgroups per CU:
// unbounded it took 259 registers and ran one wave per SIMD.
template <class C, int MODE>
constexpr int min_workgroups_per_cu() {
    if (C::NW == 4 && C::M > 4 && MODE == MODE_STREAM_PM) return 2;
    if (C::NW != 4 || C::M > 4) return 1;
    if (MODE == MODE_LOOKBACK) return 3;
    if (MODE == MODE_STREAM || MODE == MODE_STREAM_PM || MODE == MODE_AGG_PM) return 3;
    return 1;
}

template <class C, int MODE>
__global__ void __launch_bounds__(C::THREADS, (min_workgroups_per_cu<C, MODE>()))
prefill_chunk_kernel(PrefillArgs a, ScanPlan plan) {
    constexpr int LC = C::LC, M = C::M, P = C::P, WCOLS = C::WCOLS, NTW = C::NTW;
    constexpr int ROWS = 2 * M;          // state rows (mode, re/im) per value column
    constexpr bool SEG = MODE == MODE_LOOKBACK;
    constexpr bool AGG = MODE == MODE_AGG || MODE == MODE_AGG_PM;
    constexpr bool PM = MODE == MODE_STREAM_PM || MODE == MODE_AGG_PM;   // per-mode controls
    constexpr bool PM_OPS = PM && C::NSB <= 4;   // per-mode operands formed per chunk, in LDS
    constexpr int NB = C::NB, BLK = C::BLK;   // sub-blocks per arithmetic block
    // The staged chunks are an LDS object of their own, so that accesses to
    // the tables in sm are not ordered behind the asynchronous tile copies.
    __shared__ Smem<C> sm;
    // Each resident chunk's factors and v tile are LDS objects of their own:
    // the compiler orders a read of one only behind the asynchronous copies
    // into that object, so a chunk can be read while later chunks' copies
    // are still in flight.  Objects a launch mode never indexes are dropped.
    __shared__ Stage<C> sc0, sc1, sc2, sc3;
    __shared__ VTile<C> sv0, sv1, sv2, sv3;
    __shared__ StagePM<C> spm;   // per-mode launches only
    auto stage_c = [&](int i) __attribute__((always_inline)) -> Stage<C>* {
        return i == 0 ? &sc0 : i == 1 ? &sc1 : i == 2 ? &sc2 : &sc3;
    };
    auto stage_v = [&](int i) __attribute__((always_inline)) -> uint16_t* {
        return i == 0 ? sv0.V : i == 1 ? sv1.V : i == 2 ? sv2.V : sv3.V;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int col = lane & 15;

    // Launch bookkeeping of the look-back scan (every workgroup, at its end):
    // the last workgroup to finish re-arms the workspace header for the next
    // launch.  The grid is a multiple of 8, so counter x has nblocks / 8
    // workgroups.  The error word is left as it is (it stays set until the
    // caller clears it).
    auto finish_launch = [&]() __attribute__((always_inline)) {
        __syncthreads();
        if (tid == 0) {
            // per-counter completion first, then one count per finished counter
            const int xq = (int)(blockIdx.x & 7u);
            const unsigned cnt = (unsigned)(plan.nblocks >> 3);
            const unsigned done = __hip_atomic_fetch_add(&plan.hdr[SCAN_HDR_DONE0 + SCAN_HDR_STRIDE * xq], 1u,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (done + 1 == cnt) {
                const unsigned xd = __hip_atomic_fetch_add(&plan.hdr[SCAN_HDR_XDONE], 1u, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                if (xd + 1 == 8u) {   // every workgroup of this launch has finished: re-arm
                    for (int x = 0; x < 8; ++x) {
                        st_agent_u(&plan.hdr[SCAN_HDR_TICKET0 + SCAN_HDR_STRIDE * x], 0u);
                        st_agent_u(&plan.hdr[SCAN_HDR_DONE0 + SCAN_HDR_STRIDE * x], 0u);
                    }
                    st_agent_u(&plan.hdr[SCAN_HDR_XDONE], 0u);
                    st_agent_u(&plan.hdr[SCAN_HDR_EPOCH], sm.epoch + 1u);
                }
            }
        }
    };

    // ---- work item ------------------------------------------------------------------
    int seq, seg;
    unsigned tag = 0;
    if (SEG) {
        // Eight ticket counters, one per residue of blockIdx mod 8 (the XCD the
        // hardware's round-robin dispatch sends the workgroup to), so that no
        // single address takes every workgroup's atomic.  Counter x owns the
        // whole sequences [lo_x, lo_{x+1}), lo_x = floor(x nseq / 8), and hands
        // out their segments in segment-major order; the grid has 8 * max_x
        // (items of counter x) workgroups, and a workgroup whose ticket is past
        // its counter's items has nothing to do.  One XCD thus reads all
        // channels of its sequences, whose clock and gate lines (channels
        // innermost) are fetched by one L2.
        // Forward progress: a segment waits only for earlier segments of its own
        // sequence, which its own counter handed out before it, i.e. to
        // workgroups that started before it and are running or finished.  Every
        // wait is therefore on a resident workgroup with a smaller ticket of the
        // same counter, whatever the order in which the hardware starts
        // workgroups.
        const int xq = (int)(blockIdx.x & 7u);
        if (tid == 0) {
            const unsigned ep = ld_agent_u(&plan.hdr[SCAN_HDR_EPOCH]);
            const unsigned t = __hip_atomic_fetch_add(&plan.hdr[SCAN_HDR_TICKET0 + SCAN_HDR_STRIDE * xq], 1u,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sm.ticket = (int)t;
            sm.epoch = ep;
        }
        __syncthreads();
        const int tloc = sm.ticket;
        tag = ((sm.epoch + 1u) & 0x3FFFFFFFu) << 2;
        const int lo = (int)(((long long)xq * plan.nseq) >> 3);
        const int nsx = (int)((((long long)xq + 1) * plan.nseq) >> 3) - lo;   // sequences of counter xq
        if (tloc >= (plan.nblocks >> 3)) {
            // More tickets than workgroups of this residue: only possible with a
            // workspace that was not zero-filled before first use.
            if (tid == 0) __hip_atomic_fetch_or(&plan.hdr[SCAN_HDR_ERROR], SCAN_ERR_TICKET, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        if (tloc >= nsx * plan.nseg) {   // padding workgroup: only the completion count
            finish_launch();
            return;
        }
        seg = tloc / nsx;
        seq = lo + (tloc - seg * nsx);
    } else {
        // segment-major order: neighbouring work items are neighbouring channels
        // of one batch row over the same positions
        const int item = remap_xcd(blockIdx.x, gridDim.x);
        seg = item / plan.nseq;
        seq = item - seg * plan.nseq;
    }
    const int k = seq % a.K_T;
    const int b = seq / a.K_T;
    const int L = a.L, K = a.K;
    const int nchunks = plan.nchunks;
    const int c_begin = seg * plan.seg_chunks;
    const int c_end = min(nchunks, c_begin + plan.seg_chunks);
    const int nseg = plan.nseg;
    const size_t slot = (size_t)seq * nseg;   // look-back slots of this sequence: slot + segment

    const uint16_t* vg = static_cast<const uint16_t*>(a.v);
    const uint16_t* gwg = static_cast<const uint16_t*>(a.g_w);
    const uint16_t* grg = static_cast<const uint16_t*>(a.g_r);
    uint16_t* yg = static_cast<uint16_t*>(a.y);

    const int nck = c_end - c_begin;

    // Mode tables of channel k and the zero-lag coefficients, read through the
    // scalar cache (the channel is the same for the whole workgroup).  Scalar
    // loads are counted apart from vector memory operations, so building the
    // tables does not wait for the tile copies below.
    constexpr int NPOLE = (18 + C::NB) * M;
    float m_rho[M], m_th[M], m_cr[M], m_ci[M], m_za[M];
    {
        const cfloat_p rho_s = (cfloat_p)(a.rho) + k * M;
        const cfloat_p th_s = (cfloat_p)(a.theta) + k * M;
        const cfloat_p c_s = (cfloat_p)(a.c) + 2 * k * M;
        const cfloat_p zl_s = (cfloat_p)(a.zl ? a.zl : a.rho) + k * M;   // never a null base
#pragma unroll
        for (int j = 0; j < M; ++j) {
            m_rho[j] = rho_s[j];
            m_th[j] = th_s[j];
            m_cr[j] = c_s[2 * j];
            m_ci[j] = c_s[2 * j + 1];
            m_za[j] = a.zl ? zl_s[j] : 0.f;
        }
    }

    // ---- state in the accumulator layout ---------------------------------------------
    // The entering state.  Segment 0 reads state_in before any segment of the
    // sequence can finish (a look-back segment before it publishes its
    // inclusive state, which the last segment waits for), so that an aliasing
    // state_out written by the last segment cannot race with it.  In the
    // three-launch scan the aggregate launch copies state_in into the
    // entering-state slot of segment 0 and the streaming launch reads only
    // those slots.  The look-back launch reads it after its first sweep, so
    // that no register load is outstanding while its tile copies land.
    const bool split_stream = (MODE == MODE_STREAM || MODE == MODE_STREAM_PM) && nseg > 1;
    auto load_entering = [&](f32x4_t (&x)[NTW]) __attribute__((always_inline)) {
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int p = wave * WCOLS + nt * 16 + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i, j = row >> 1, cmp = row & 1;
                float v = 0.f;
                if (split_stream) {
                    if (row < ROWS) v = plan.incl[((slot + seg) * ROWS + row) * (size_t)P + p];
                } else if (seg == 0 && a.state_in && j < M) {
                    v = a.state_in[((((size_t)b * K + k) * M + j) * 2 + cmp) * P + p];
                }
                x[nt][i] = v;
            }
        }
    };
    // The streaming launches issue these loads before building the tables, so
    // that the tables' work covers their latency.
    f32x4_t st_in[NTW];
    if (!SEG) load_entering(st_in);

    // ---- segmented scan: every chunk of the segment is requested at once -------------------
    // Asynchronous global-to-LDS copies only (no register loads): first the
    // controls of every resident chunk (clock into q2, gate bits into gw/gr;
    // 64 positions per wave instruction, spread over the waves), then the v
    // tiles of the wave's own columns.  Every wave issues the same number of
    // tile copies per chunk, TLW,
    // after all control copies, so "chunk i has landed" is "at most
    // (RES-1-i) * TLW copies outstanding" in every wave.  Rows past the
    // segment or past L repeat a valid row; their values only reach positions
    // that are never written.
    // A wave's tile copy fills 1 KB of LDS, 32 rows of one 16-column tile
    // block (lane l: row l/2, 8-column half l%2); each wave copies the tiles of
    // its own columns, TLW instructions per chunk.
    constexpr int TLW = NTW * (LC / 32);       // tile copies per wave and chunk
    // one tile copy of local chunk position row base `tb` (first position of the
    // chunk) into the tile block array `dst`; rows at or past `tend` repeat row tend-1
    auto copy_tile = [&](uint16_t* dst, int it, int tb, int tend) __attribute__((always_inline)) {
        const int j = wave * NTW + it / (LC / 32), q = it % (LC / 32);
        const int t = min(tb + 32 * q + (lane >> 1), tend - 1);
        const uint16_t* src = vg + (((size_t)b * L + t) * K + k) * P + j * 16 + (lane & 1) * 8;
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(dst + j * C::TBLK + q * 512), 16, 0, 0);
    };
    if (SEG) {
        constexpr int CIA = (LC + 63) / 64;    // instructions per control array of a chunk
        constexpr int NCI = C::RES * 3 * CIA;
        const int seg_last = min(c_end * LC, L) - 1;   // the segment's last position
#pragma unroll
        for (int ci = 0; ci < NCI; ++ci) {
            const int i = ci / (3 * CIA), arr = (ci / CIA) % 3, u = ci % CIA;
            const int pos = u * 64 + lane;
            if (ci % C::NW == wave && pos < LC) {
                const int t = i < nck ? min((c_begin + i) * LC + pos, L - 1) : seg_last;
                const size_t row = ((size_t)b * L + t) * K + k;
                Stage<C>* sp = stage_c(i);
                if (arr == 0)
                    __builtin_amdgcn_global_load_lds(a.delta + row, (lds_void_t*)(&sp->q2[u * 64]), 4, 0, 0);
                else if (arr == 1)   // 16-bit element -> 32-bit slot per lane
                    __builtin_amdgcn_global_load_lds(gwg + row, (lds_void_t*)(&sp->gw[u * 64]), 2, 0, 0);
                else
                    __builtin_amdgcn_global_load_lds(grg + row, (lds_void_t*)(&sp->gr[u * 64]), 2, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < C::RES; ++i) {
            // rows past L repeat row L-1; a stage past the segment's chunks (never
            // read) gets one row, so that every wave still issues TLW copies per stage
#pragma unroll
            for (int it = 0; it < TLW; ++it)
                copy_tile(stage_v(i), it, i < nck ? (c_begin + i) * LC : seg_last, i < nck ? L : seg_last + 1);
        }
    }

    // ---- pole tables: lambda^tau and c lambda^tau for tau = 0..16, lambda^{16 d} ---------
    // (LDS-only barriers here: the tile copies stay in flight.)
#pragma unroll
    for (int j = 0; j < M; ++j)
        if (tid == j) {
            sm.mtab[j] = make_float4(m_rho[j], m_th[j], m_cr[j], m_ci[j]);
            sm.mza[j] = m_za[j];
        }
    lds_barrier();
    for (int idx = tid; idx < NPOLE; idx += C::THREADS) {
        const bool blk16 = idx >= 17 * M;
        const int id2 = blk16 ? idx - 17 * M : idx;
        const int i0 = id2 / M, j = id2 - i0 * M;
        const int tau = blk16 ? 16 * i0 : i0;
        const float4 mt = sm.mtab[j];
        const float r = mt.x;
        const float th = mt.y;
        const float mag = tau == 0 ? 1.f : exp2f((float)tau * log2f(r));
        float sn, cs;
        sincosf(th * (float)tau, &sn, &cs);   // |theta tau| <= 64 pi
        const float pr = mag * cs, pi = mag * sn;
        sm.pw[blk16 ? 17 + i0 : tau][j] = make_float2(pr, pi);
        if (!blk16) {
            const float cr = mt.z, ci = mt.w;
            // per-mode launches fold the zero-lag term (Eq. 24) into the lag-0
            // coefficient of each mode: Re(c_j) (1 - a_j)
            const float zc = PM && tau == 0 ? sm.mza[j] * cr : 0.f;
            sm.cpw[tau][j] = make_float2(cr * pr - ci * pi - zc, cr * pi + ci * pr);
        }
    }
    lds_barrier();
    // psi(16 d + r) = sum_j Re(c_j lambda_j^r lambda_j^{16 d})
    for (int tau = tid; tau < C::BLK; tau += C::THREADS) {
        const int d = tau >> 4, r = tau & 15;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const float2 cp = sm.cpw[r][j], pd = sm.pw[17 + d][j];
            s += cp.x * pd.x - cp.y * pd.y;
        }
        // zero-lag correction (Eq. 24): with per-channel gates it lowers the
        // lag-zero coefficient by sum_j a_j kc_j
        if (tau == 0) {
#pragma unroll
            for (int j = 0; j < M; ++j) s -= m_za[j] * m_cr[j];
        }
        sm.psi[tau] = s;
    }
    lds_barrier();
    if constexpr (PM && !AGG) {   // tables of the output operands only
        for (int idx = tid; idx < 16 * M; idx += C::THREADS) {
            const int e = idx / M, j = idx - e * M;
            const float4 mt = sm.mtab[j];
            const float mag = e == 0 ? 1.f : exp2f(-(float)e * log2f(mt.x));
            float sn, cs;
            sincosf(-mt.y * (float)e, &sn, &cs);
            spm.ipw[e][j] = make_float2(mag * cs, mag * sn);
        }
        if (tid == 0) {
            int f = 0;
#pragma unroll
            for (int j = 0; j < M; ++j)
                if (!(-15.f * log2f(sm.mtab[j].x) <= 40.f)) f = 1;   // also for rho <= 0 or NaN
            spm.lowrho = f;
        }
        lds_barrier();
    }

    // ---- per-lane constant MFMA operands ------------------------------------------------
    // Output product of target sub-block a of a block (B operands; lane (g, col)
    // is target position t = 16a + col of the block):
    //   yD[a]: slots 0..3: psi(t-s) [s <= t] for s = 16a+4g+e (same for every a);
    //          slots 4..7: {Re, -Im}(c_j lambda_j^{t+1}) for state rows 4g..4g+3, bf16 hi.
    //   yDx[a]: slots 0..3: the bf16 lo halves of those coefficients, slots 4..7: their hi
    //          halves; against [state hi ; state lo] it adds both cross terms of the carry
    //          readout, whose mode terms may cancel (fitted tables carry |c| up to ~30).
    //   yB12:  slots 0..3: psi(16+col-4g-e) (source sub-block a-1),
    //          slots 4..7: psi(32+col-4g-e) (source sub-block a-2).
    //   yB3:   slots 0..3: psi(48+col-4g-e) (source sub-block a-3), slots 4..7: 0.
    // State product of source sub-block a (A operands; lane (g, col) is state
    // row col = (j, re/im)): lpA[a]: {Re, Im}(lambda_j^{BLK-1-16a-4g-e}) split
    // into bf16 hi (slots 0..3) and lo (slots 4..7).
    // lB: lambda_j^BLK and l16: lambda_j^16 for this lane's modes 2g, 2g+1.
    // The sub-block path uses yD[0] (its output operand) and lpA[NB-1] (its
    // state operand).
    // The output operands (yD, yB12, yB3) and the state operands (lpA, lB, l16)
    // are built separately: the look-back launch needs the state operands in
    // its aggregate sweep and the output operands in its output sweep only.
    bf16x8_t yD[NB], yDx[NB], yB12, yB3, lpA[NB];
    float lB[4], l16[4];
    auto make_ydx = [&](int aa) __attribute__((always_inline)) -> bf16x8_t {
        u16x8_t hx;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * g + i, j = row >> 1;
            float val = 0.f;
            if (j < M) {
                const float2 cp = sm.cpw[col + 1][j < M ? j : 0], pd = sm.pw[17 + aa][j < M ? j : 0];
                val = (row & 1) ? -(cp.x * pd.y + cp.y * pd.x) : (cp.x * pd.x - cp.y * pd.y);
            }
            const uint16_t hb = f32_to_bf16(val);
            hx[4 + i] = hb;
            hx[i] = f32_to_bf16(val - bf16_to_f32(hb));
        }
        return to_bf16x8(hx);
    };
    auto make_out_constants = [&]() __attribute__((always_inline)) {
        u16x8_t h;
#pragma unroll
        for (int aa = 0; aa < NB; ++aa) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 4 * g + e;
                h[e] = f32_to_bf16(s <= col ? sm.psi[col - s] : 0.f);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i, j = row >> 1;
                float val = 0.f;
                if (j < M) {
                    const float2 cp = sm.cpw[col + 1][j < M ? j : 0], pd = sm.pw[17 + aa][j < M ? j : 0];
                    val = (row & 1) ? -(cp.x * pd.y + cp.y * pd.x) : (cp.x * pd.x - cp.y * pd.y);
                }
                h[4 + i] = f32_to_bf16(val);
            }
            yD[aa] = to_bf16x8(h);
            yDx[aa] = make_ydx(aa);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = NB >= 2 ? f32_to_bf16(sm.psi[(16 + col - 4 * g - e) & (BLK - 1)]) : 0;
            h[4 + e] = NB >= 3 ? f32_to_bf16(sm.psi[(32 + col - 4 * g - e) & (BLK - 1)]) : 0;
        }
        yB12 = to_bf16x8(h);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = NB >= 4 ? f32_to_bf16(sm.psi[(48 + col - 4 * g - e) & (BLK - 1)]) : 0;
            h[4 + e] = 0;
        }
        yB3 = to_bf16x8(h);
    };
    auto make_state_constants = [&]() __attribute__((always_inline)) {
        u16x8_t h;
        const int jr = col >> 1;
#pragma unroll
        for (int aa = 0; aa < NB; ++aa) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float val = 0.f;
                if (jr < M) {
                    const float2 pw = sm.pw[15 - 4 * g - e][jr < M ? jr : 0];
                    const float2 pd = sm.pw[17 + NB - 1 - aa][jr < M ? jr : 0];
                    val = (col & 1) ? (pw.x * pd.y + pw.y * pd.x) : (pw.x * pd.x - pw.y * pd.y);
                }
                const uint16_t hb = f32_to_bf16(val);
                h[e] = hb;
                h[4 + e] = f32_to_bf16(val - bf16_to_f32(hb));
            }
            lpA[aa] = to_bf16x8(h);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int j = 2 * g + hh;
            const float2 pb = j < M ? sm.pw[17 + NB][j < M ? j : 0] : make_float2(0.f, 0.f);
            const float2 p1 = j < M ? sm.pw[17 + 1][j < M ? j : 0] : make_float2(0.f, 0.f);
            lB[2 * hh] = pb.x;
            lB[2 * hh + 1] = pb.y;
            l16[2 * hh] = p1.x;
            l16[2 * hh + 1] = p1.y;
        }
    };
    // The sub-block path's state operand (lpA[NB-1]) and lambda^16, rebuilt
    // from the tables where the state operands are no longer held.
    auto make_sub_al = [&]() __attribute__((always_inline)) -> bf16x8_t {
        u16x8_t h;
        const int jr = col >> 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float val = 0.f;
            if (jr < M) {
                const float2 pw = sm.pw[15 - 4 * g - e][jr < M ? jr : 0];
                val = (col & 1) ? pw.y : pw.x;
            }
            const uint16_t hb = f32_to_bf16(val);
            h[e] = hb;
            h[4 + e] = f32_to_bf16(val - bf16_to_f32(hb));
        }
        return to_bf16x8(h);
    };
    auto make_l16 = [&](float (&o)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int j = 2 * g + hh;
            const float2 p1 = j < M ? sm.pw[17 + 1][j < M ? j : 0] : make_float2(0.f, 0.f);
            o[2 * hh] = p1.x;
            o[2 * hh + 1] = p1.y;
        }
    };
    make_state_constants();
    if (!SEG) make_out_constants();

    // ---- chunk pipeline helpers ---------------------------------------------------------
    const int vrow_l = lane / C::LPR;          // row of this lane inside a wave load
    const int vunit = lane % C::LPR;           // 16-byte unit of this lane inside a row
    const size_t vcol0 = (size_t)wave * WCOLS + vunit * 8;
    Stage<C>* sgp = stage_c(0);   // staged chunk the helpers work on: factors
    uint16_t* sgv = stage_v(0);   // ... and v tile
    // element offset of (row r, first column of 16-byte unit u) in the v tile
    auto vt_off = [&](int r, int u) __attribute__((always_inline)) {
        return (u >> 1) * C::TBLK + r * 16 + ((u & 1) << 3);
    };

    // Loads of one chunk held in registers until they are staged into LDS.
    // per-mode controls of a chunk spread over every thread: LC * M values each
    constexpr int PMC = PM ? (LC * M + C::THREADS - 1) / C::THREADS : 1;
    struct ChunkRegs {
        uint4 v[C::NLD];
        float cd[C::CPL];                           // controls (wave 0 only); gates as
        uint32_t cw[C::CPL], cr[C::CPL];            // raw bf16 bits, converted when staged
        float md[PMC];                              // per-mode controls (per-mode launches):
        uint32_t mw[PMC], mr[PMC];                  // element tid + u * THREADS = position * M + mode
    };

    auto load_chunk = [&](ChunkRegs& rg, int c) __attribute__((always_inline)) {
        const int t0 = c * LC;
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            const int t = t0 + i * C::RPI + vrow_l;
            if (t < L) {
                const size_t off = (((size_t)b * L + t) * K + k) * P + vcol0;
                rg.v[i] = *reinterpret_cast<const uint4*>(vg + off);
            } else {
                rg.v[i] = make_uint4(0, 0, 0, 0);
            }
        }
        if constexpr (PM) {
#pragma unroll
            for (int u = 0; u < PMC; ++u) {
                const int e = tid + u * C::THREADS;
                const int r = e / M;
                const int t = t0 + r;
                if (e < LC * M && t < L) {
                    const size_t row = (((size_t)b * L + t) * K + k) * M + (e - r * M);
                    rg.md[u] = a.delta[row];
                    rg.mw[u] = gwg[row];
                    rg.mr[u] = grg[row];
                } else {
                    rg.md[u] = 0.f;
                    rg.mw[u] = 0u;
                    rg.mr[u] = 0u;
                }
            }
        } else if (wave == 0) {
#pragma unroll
            for (int u = 0; u < C::CPL; ++u) {
                const int r = lane * C::CPL + u;
                const int t = t0 + r;
                if (r < LC && t < L) {
                    const size_t row = ((size_t)b * L + t) * K + k;
                    rg.cd[u] = a.delta[row];
                    rg.cw[u] = gwg[row];
                    rg.cr[u] = grg[row];
                } else {
                    rg.cd[u] = 0.f;
                    rg.cw[u] = 0u;
                    rg.cr[u] = 0u;
                }
            }
        }
    };

    // One wave: clock sums and per-position factors of the staged chunk (n
    // valid positions) from the controls it holds.
    auto stage_ctrl = [&](const float (&cd)[C::CPL], const uint32_t (&cwb)[C::CPL], const uint32_t (&crb)[C::CPL],
                          int n) __attribute__((always_inline)) {
        {
            float cw[C::CPL], cr[C::CPL];
#pragma unroll
            for (int u = 0; u < C::CPL; ++u) {
                cw[u] = bf16_to_f32((uint16_t)cwb[u]);
                cr[u] = bf16_to_f32((uint16_t)crb[u]);
            }
            float loc[C::CPL];
            float run = 0.f;
#pragma unroll
            for (int u = 0; u < C::CPL; ++u) {
                run += cd[u];
                loc[u] = run;
            }
            float incl = run;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(incl, off);
                if (lane >= off) incl += o;
            }
            const float excl = incl - run;
#pragma unroll
            for (int u = 0; u < C::CPL; ++u) {
                const int idx = lane * C::CPL + u;
                if (idx < LC) {
                    sgp->q2[idx] = (excl + loc[u]) * LOG2E;
                    sgp->gw[idx] = cwb[u];
                    sgp->gr[idx] = crb[u];
                }
            }
            // same wave: its own LDS writes above are visible to these reads
#pragma unroll
            for (int u = 0; u < C::CPL; ++u) {
                const int idx = lane * C::CPL + u;
                if (idx < LC) {
                    const float q = sgp->q2[idx];
                    // block of BLK positions: factored with the clock referenced to
                    // its middle when it is whole and its span allows
                    const int B0 = idx & ~(BLK - 1);
                    const int B1 = min(B0 + BLK - 1, n - 1);
                    const float qs = B0 > 0 ? sgp->q2[B0 - 1] : 0.f;
                    const float qe = sgp->q2[B1 > 0 ? B1 : 0];
                    if (B1 == B0 + BLK - 1 && qe - qs <= SPAN2_BLOCK_MAX) {
                        const float ref = 0.5f * (qs + qe);
                        sgp->bq[idx] = exp2f(q - ref) * cw[u];
                        sgp->ag[idx] = exp2f(ref - q) * cr[u];
                        if (idx == B1)
                            sgp->blkB[B0 / BLK] = make_float4(exp2f(qs - ref), exp2f(ref - qe), exp2f(qs - qe), 0.f);
                    } else {
                        // sub-block factors (clock referenced to each sub-block's start)
                        const int T0 = idx & ~15;
                        const float qp = T0 > 0 ? sgp->q2[T0 - 1] : 0.f;
                        sgp->bq[idx] = idx < n ? exp2f(q - qp) * cw[u] : 0.f;
                        sgp->ag[idx] = exp2f(qp - q) * cr[u];
                        const int T1 = min(T0 + 15, n - 1);
                        if (idx == T1) {
                            const bool exact = (q - qp) > SPAN2_FAST_MAX || T1 - T0 < 15;
                            sgp->blk[idx >> 4] = make_float2(exp2f(qp - q), exact ? 1.f : 0.f);
                        }
                        if (idx == B1) sgp->blkB[B0 / BLK] = make_float4(0.f, 0.f, exp2f(qs - qe), 1.f);
                    }
                }
            }
        }
    };

    // Per-mode controls: 1 where some mode's clock span over sub-block T (n valid positions in
    // the chunk, clock sums staged) is too large for the factored operands.
    auto pm_exact = [&](int T, int n) __attribute__((always_inline)) -> int {
        int ex = 0;
        if constexpr (PM) {
            const int T0 = 16 * T, T1 = min(T0 + 15, n - 1);
            if (T0 < n) {
#pragma unroll
                for (int j = 0; j < M; ++j)
                    if (spm.q[j][T1] - (T0 > 0 ? spm.q[j][T0 - 1] : 0.f) > SPAN2_FAST_MAX) ex = 1;
            }
        }
        return ex;
    };

    // Register path: v tile and controls of the loaded chunk -> LDS, then the
    // loads of chunk `next` (if >= 0) are issued so that they overlap this
    // chunk's arithmetic.  Starts and ends with a barrier.
    auto stage_chunk = [&](ChunkRegs& rg, int n, int next) __attribute__((always_inline)) {
        __syncthreads();   // previous readers of the staged chunk are done
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            const int tr = i * C::RPI + vrow_l;
            *reinterpret_cast<uint4*>(&sgv[vt_off(tr, (int)(vcol0 >> 3))]) = rg.v[i];
        }
        if constexpr (PM) {
            // raw per-mode controls -> [mode][position]; every sub-block takes
            // the exact path (its operands are formed per element and mode)
#pragma unroll
            for (int u = 0; u < PMC; ++u) {
                const int e = tid + u * C::THREADS;
                if (e < LC * M) {
                    const int r = e / M, j = e - r * M;
                    spm.q[j][r] = rg.md[u];
                    spm.gw[j][r] = bf16_to_f32((uint16_t)rg.mw[u]);
                    spm.gr[j][r] = bf16_to_f32((uint16_t)rg.mr[u]);
                }
            }
            for (int i = tid; i < C::NSB; i += C::THREADS) sgp->blk[i] = make_float2(0.f, 1.f);
            for (int i = tid; i < LC / 32; i += C::THREADS) sgp->blkB[i] = make_float4(0.f, 0.f, 0.f, 1.f);
        } else if (wave == 0) {
            stage_ctrl(rg.cd, rg.cw, rg.cr, n);
        }
        if (next >= 0) load_chunk(rg, next);
        __syncthreads();
        if constexpr (PM) {
            // clock sums of each mode over the chunk and, from them, the factors of the clock
            // referenced to each sub-block's start (wave w: modes w, w + NW, ...)
            for (int j = wave; j < M; j += C::NW) {
                float loc[C::CPL];
                float run = 0.f;
#pragma unroll
                for (int u = 0; u < C::CPL; ++u) {
                    const int idx = lane * C::CPL + u;
                    run += idx < LC ? spm.q[j][idx] : 0.f;
                    loc[u] = run;
                }
                float incl = run;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float o = __shfl_up(incl, off);
                    if (lane >= off) incl += o;
                }
                const float excl = incl - run;
                float qv[C::CPL];
#pragma unroll
                for (int u = 0; u < C::CPL; ++u) qv[u] = (excl + loc[u]) * LOG2E;
                // the clock sum just before this lane's sub-block (CPL divides 16, so a lane's
                // positions share one sub-block and position T0 - 1 is a lane's last)
                const int T0 = (lane * C::CPL) & ~15;
                const float qb = __shfl(qv[C::CPL - 1], T0 > 0 ? T0 / C::CPL - 1 : 0);
                const float qp = T0 > 0 ? qb : 0.f;
#pragma unroll
                for (int u = 0; u < C::CPL; ++u) {
                    const int t = lane * C::CPL + u;
                    if (t < LC) {
                        spm.q[j][t] = qv[u];
                        const float d = qv[u] - qp;   // >= 0 (log2 units)
                        if constexpr (!AGG) spm.fa[j][t] = exp2f(-d) * spm.gr[j][t];   // output side only
                        spm.fb[j][t] = t < n ? exp2f(d) * spm.gw[j][t] : 0.f;
                        if (t == min(T0 + 15, n - 1)) spm.ftr[j][t >> 4] = exp2f(-d);
                    }
                }
            }
            if constexpr (!PM_OPS) {
                // sub-blocks whose clock span is too large to factor (with operands formed per
                // chunk, the wave forming a sub-block's operands decides this)
                __syncthreads();
                for (int i = tid; i < C::NSB; i += C::THREADS) spm.fexact[i] = pm_exact(i, n);
            }
            __syncthreads();
        }
    };

    // v fragment of sub-block T for tile nt: positions T0+4g..T0+4g+3 of column
    // p = wave*WCOLS + nt*16 + col, by one transposing LDS read.  Within a group
    // of 16 lanes, ds_read_b64_tr_b16 returns to lane i, element e, the (i%4)-th
    // 16-bit value at the address of lane 4e + i/4; so lane (g, col) supplies
    // the address of row T0 + 4g + col/4, columns 4*(col%4) .. +3 of the tile.
    // Sub-block T is 16 rows = 256 elements further in the tile block.
    int vf_off[NTW], ys_off[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int p0 = wave * WCOLS + nt * 16 + 4 * (col & 3);
        vf_off[nt] = vt_off(4 * g + (col >> 2), p0 >> 3) + (p0 & 7);
        const int p1 = wave * WCOLS + nt * 16 + 4 * g;
        ys_off[nt] = vt_off(col, p1 >> 3) + (p1 & 7);
    }
    auto load_vfrag = [&](int T, int nt) __attribute__((always_inline)) -> uint2 {
        const s16x4_t x =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(&sgv[vf_off[nt] + T * 256]));
        return __builtin_bit_cast(uint2, x);
    };

    // y tile of sub-block T (lane holds y(t = T0+col, p1 + i), i < 4, p1 =
    // wave*WCOLS + nt*16 + 4g) -> staged in the v tile in place: each wave
    // overwrites only its own columns of rows it has already read.
    auto stage_y = [&](int T, int nt, const f32x4_t& acc, float scale) __attribute__((always_inline)) {
        *reinterpret_cast<uint2*>(&sgv[ys_off[nt] + T * 256]) =
            make_uint2(pk_bf16(acc[0] * scale, acc[1] * scale), pk_bf16(acc[2] * scale, acc[3] * scale));
    };

    // b(s) v(s) of fragment (T, nt) kept for a later sweep, in place: the
    // fragment's footprint in the tile (rows T0..T0+15 of one 16-column tile
    // block) is 512 contiguous bytes, and lane l takes the l-th 8 bytes.  Only
    // the wave that read the fragment writes its slots, after reading it.
    int bw_off[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
        bw_off[nt] = (wave * NTW + nt) * C::TBLK + lane * 4;
    auto store_bv = [&](int T, int nt, uint2 x) __attribute__((always_inline)) {
        *reinterpret_cast<uint2*>(&sgv[bw_off[nt] + T * 256]) = x;
    };
    auto load_bv = [&](int T, int nt) __attribute__((always_inline)) -> uint2 {
        return *reinterpret_cast<const uint2*>(&sgv[bw_off[nt] + T * 256]);
    };

    auto hi4 = [&](const f32x4_t& x) __attribute__((always_inline)) -> uint2 {
        return make_uint2(pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3]));
    };
    // The bf16 rounding of what x - (its bf16 rounding h) leaves: x = h + lo4(x, h) to about
    // 16 mantissa bits.  Feeding both halves to an MFMA keeps an fp32-class product.
    auto lo4 = [&](const f32x4_t& x, uint2 h) __attribute__((always_inline)) -> uint2 {
        return make_uint2(pk_bf16(x[0] - lo_f32(h.x), x[1] - hi_f32(h.x)),
                          pk_bf16(x[2] - lo_f32(h.y), x[3] - hi_f32(h.y)));
    };
    // b(s) v(s) of one fragment (four positions of one column) in fp32
    auto bv_f32 = [&](const float4& b4, uint2 vf) __attribute__((always_inline)) -> f32x4_t {
        return f32x4_t{b4.x * lo_f32(vf.x), b4.y * hi_f32(vf.x), b4.z * lo_f32(vf.y), b4.w * hi_f32(vf.y)};
    };

    // Per-mode operands of sub-block T, per element and mode, with the read gate inside the
    // sum over modes:
    //   G[t][s]  = sum_j g_r,j(t) e^{-(qj(t)-qj(s))} g_w,j(s) Re(c_j lambda_j^{t-s})  (s <= t)
    //   C[t][jr] = g_r,j(t) e^{-(qj(t)-qj(T0-1))} {Re, -Im}(c_j lambda_j^{t-T0+1})
    //   W[jr][s] = {Re, Im}(lambda_j^{T1-s}) e^{-(qj(T1)-qj(s))} g_w,j(s)
    // from the staged factors fa, fb, ftr (products, no exponentials), or, where a mode's
    // clock span is too large to factor, from the clock sums.  With out: bx = [G ; C hi] and
    // bxx = [C lo ; C hi] (the carry coefficients in bf16 hi and lo halves, since mode terms
    // may cancel).  wf = W in hi and lo halves.
    auto pm_operands = [&](int T, int n, bool out, bool fac, bf16x8_t& bx, bf16x8_t& bxx,
                           bf16x8_t& wf) __attribute__((always_inline)) {
        if constexpr (PM) {
            const int T0 = T * 16, T1 = min(T0 + 15, n - 1);
            float wv[4];
            if (fac) {
                if (out) {
                    const int t = T0 + col;
                    float gv[4] = {0.f, 0.f, 0.f, 0.f}, av[4] = {0.f, 0.f, 0.f, 0.f};
                    if (!spm.lowrho) {
                        // G^T = W U^T on the fp32 matrix cores, rank 2m: U[t][2j, 2j+1] =
                        // fa_j(t) {Re, -Im}(c_j lambda_j^{t-T0}), W[s][2j, 2j+1] = fb_j(s)
                        // {Re, Im}(lambda_j^{T0-s}); lane (g, col) gives row col of each, columns
                        // 4 kb + g, and gets G[t][s = T0 + 4g + e] in element e.  Row T0 of U
                        // takes c_j itself (the lag-0 coefficient without the zero-lag term);
                        // the diagonal then loses zd.
                        f32x4_t gd = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kb = 0; kb < (2 * M + 3) / 4; ++kb) {
                            const int k = 4 * kb + g, j = k >> 1;
                            float u = 0.f, w = 0.f;
                            if (j < M) {
                                const int jj = j < M ? j : 0;
                                const float4 mt = sm.mtab[jj];
                                const float2 cp = col == 0 ? make_float2(mt.z, mt.w) : sm.cpw[col][jj];
                                const float2 ip = spm.ipw[col][jj];
                                u = spm.fa[jj][t] * ((k & 1) ? -cp.y : cp.x);
                                w = spm.fb[jj][t] * ((k & 1) ? ip.y : ip.x);
                            }
                            gd = __builtin_amdgcn_mfma_f32_16x16x4f32(w, u, gd, 0, 0, 0);
                        }
                        float zdt = 0.f;   // the zero-lag term of the diagonal
#pragma unroll
                        for (int j = 0; j < M; ++j) zdt += spm.gr[j][t] * spm.gw[j][t] * sm.mza[j] * sm.mtab[j].z;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int sl = 4 * g + e;
                            gv[e] = sl < col ? gd[e] : sl == col ? gd[e] - zdt : 0.f;
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < M; ++j) {
                            const float fat = spm.fa[j][t];
                            const float4 fb4 = *reinterpret_cast<const float4*>(&spm.fb[j][T0 + 4 * g]);
                            const float fbs[4] = {fb4.x, fb4.y, fb4.z, fb4.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int sl = 4 * g + e;
                                if (sl <= col) gv[e] += fat * fbs[e] * sm.cpw[col - sl][j].x;
                            }
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 4 * g + i, j = row >> 1;
                        if (j < M) {
                            const int jj = j < M ? j : 0;
                            const float2 cp = sm.cpw[col + 1][jj];
                            av[i] = spm.fa[jj][t] * ((row & 1) ? -cp.y : cp.x);
                        }
                    }
                    const f32x4_t af = f32x4_t{av[0], av[1], av[2], av[3]};
                    const uint2 ah4 = hi4(af);
                    bx = bf16x8_of(make_uint2(pk_bf16(gv[0], gv[1]), pk_bf16(gv[2], gv[3])), ah4);
                    bxx = bf16x8_of(lo4(af, ah4), ah4);
                }
                const int jr = col >> 1;
                const int jj = jr < M ? jr : 0;
                const float trj = spm.ftr[jj][T];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s2 = T0 + 4 * g + e;
                    float val = 0.f;
                    if (jr < M && s2 <= T1) {
                        const float2 pw = sm.pw[T1 - s2][jj];
                        val = ((col & 1) ? pw.y : pw.x) * spm.fb[jj][s2] * trj;
                    }
                    wv[e] = val;
                }
            } else {
                if (out) {
                    const int t = T0 + col;
                    float gv[4] = {0.f, 0.f, 0.f, 0.f}, av[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < M; ++j) {
                        const float qt = spm.q[j][t];
                        const float grt = spm.gr[j][t];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int sl = 4 * g + e;
                            if (sl <= col) {
                                const int s2 = T0 + sl;
                                gv[e] += exp2f(spm.q[j][s2] - qt) * spm.gw[j][s2] * grt * sm.cpw[col - sl][j].x;
                            }
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 4 * g + i, j = row >> 1;
                        if (j < M) {
                            const int jj = j < M ? j : 0;
                            const float qp = T0 > 0 ? spm.q[jj][T0 - 1] : 0.f;
                            const float ea = exp2f(qp - spm.q[jj][t]) * spm.gr[jj][t];
                            const float2 cp = sm.cpw[col + 1][jj];
                            av[i] = ea * ((row & 1) ? -cp.y : cp.x);
                        }
                    }
                    const f32x4_t af = f32x4_t{av[0], av[1], av[2], av[3]};
                    const uint2 ah4 = hi4(af);
                    bx = bf16x8_of(make_uint2(pk_bf16(gv[0], gv[1]), pk_bf16(gv[2], gv[3])), ah4);
                    bxx = bf16x8_of(lo4(af, ah4), ah4);
                }
                const int jr = col >> 1;
                const int jj = jr < M ? jr : 0;
                const float qe = spm.q[jj][T1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s2 = T0 + 4 * g + e;
                    float val = 0.f;
                    if (jr < M && s2 <= T1) {
                        const float2 pw = sm.pw[T1 - s2][jj];
                        val = ((col & 1) ? pw.y : pw.x) * exp2f(spm.q[jj][s2] - qe) * spm.gw[jj][s2];
                    }
                    wv[e] = val;
                }
            }
            const uint32_t w01 = pk_bf16(wv[0], wv[1]), w23 = pk_bf16(wv[2], wv[3]);
            wf = bf16x8_of(make_uint2(w01, w23), make_uint2(pk_bf16(wv[0] - lo_f32(w01), wv[1] - hi_f32(w01)),
                                                           pk_bf16(wv[2] - lo_f32(w23), wv[3] - hi_f32(w23))));
        }
    };

    // One sub-block: optional outputs, then the state update; tr accumulates the
    // sub-block transfers (modes 2g, 2g+1) for the segment aggregate.
    auto subblock = [&](f32x4_t (&st)[NTW], int T, int n, bool out, float (&tr)[4], const bf16x8_t& al,
                        const float (&l16)[4]) __attribute__((always_inline)) {
        const int T0 = T * 16;
        const float2 bk = sgp->blk[T];
        uint2 vfr[NTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) vfr[nt] = load_vfrag(T, nt);
        float lam[4];   // Lambda_T for modes 2g, 2g+1
        if (bk.y == 0.f) {
            // factored path: scale v by b(s), constant operands.  b(s) v(s) is
            // split into a bf16 hi half, which feeds the output product, and a bf16
            // lo half; the state product takes both halves against the hi and lo
            // halves of the lambda powers, and the carry term takes the hi and lo
            // halves of the state, so both state-side contractions keep fp32-class
            // precision.
            const float4 b4 = *reinterpret_cast<const float4*>(&sgp->bq[T0 + 4 * g]);
            uint2 bv[NTW], bvl[NTW];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const f32x4_t f = bv_f32(b4, vfr[nt]);
                bv[nt] = hi4(f);
                bvl[nt] = lo4(f, bv[nt]);
            }
            if (out) {
                const float sc = sgp->ag[T0 + col];
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    const uint2 hh = hi4(st[nt]);
                    f32x4_t acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        bf16x8_of(bv[nt], hh), yD[0], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(hh, lo4(st[nt], hh)), yDx[0], acc, 0,
                                                                  0, 0);
                    stage_y(T, nt, acc, sc);
                }
            }
            const float at = bk.x;
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                f32x4_t mv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bf16x8_of(bv[nt], bv[nt]),
                                                                    f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                mv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bf16x8_of(bvl[nt], bvl[nt]), mv, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const float lr = l16[i], li = l16[i + 1];
                    const float hr = st[nt][i], hi = st[nt][i + 1];
                    st[nt][i] = at * (lr * hr - li * hi + mv[i]);
                    st[nt][i + 1] = at * (li * hr + lr * hi + mv[i + 1]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) lam[i] = at * l16[i];
        } else if constexpr (PM) {
            // per-mode controls: the operands of pm_operands, formed for the whole chunk before
            // its sub-blocks where they are held in LDS, else here
            const int T1 = min(T0 + 15, n - 1);
            bf16x8_t bx, bxx, wf;
            if constexpr (PM_OPS) {
                if (out) {
                    bx = spm.opg[T][lane];
                    bxx = spm.opgx[T][lane];
                }
                wf = spm.opw[T][lane];
            } else {
                pm_operands(T, n, out, spm.fexact[T] == 0, bx, bxx, wf);
            }
            if (out) {
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    const uint2 hh = hi4(st[nt]);
                    f32x4_t acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        bf16x8_of(vfr[nt], hh), bx, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(hh, lo4(st[nt], hh)), bxx, acc, 0, 0,
                                                                  0);
                    stage_y(T, nt, acc, 1.f);
                }
            }
            // Lambda_T of modes 2g, 2g+1: the clock factor of the whole sub-block (staged, or
            // from the clock sums where the span is too large to factor) and lambda^len
            const bool fac = spm.fexact[T] == 0;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int j = 2 * g + hh;
                float2 pn = make_float2(0.f, 0.f);
                float at = 0.f;
                if (j < M) {
                    const int jj = j < M ? j : 0;
                    const float qp = T0 > 0 ? spm.q[jj][T0 - 1] : 0.f;
                    at = fac ? spm.ftr[jj][T] : exp2f(qp - spm.q[jj][T1]);
                    pn = sm.pw[T1 - T0 + 1][jj];
                }
                lam[2 * hh] = at * pn.x;
                lam[2 * hh + 1] = at * pn.y;
            }
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                f32x4_t d;
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const float hr = st[nt][i], hi = st[nt][i + 1];
                    d[i] = lam[i] * hr - lam[i + 1] * hi;
                    d[i + 1] = lam[i + 1] * hr + lam[i] * hi;
                }
                st[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, bf16x8_of(vfr[nt], vfr[nt]), d, 0, 0, 0);
            }
        } else {
            // exact path (ragged sub-block, or a clock span too large to factor):
            // operands evaluated per element from the clock sums.
            const int T1 = min(T0 + 15, n - 1);
            const float qp = T0 > 0 ? sgp->q2[T0 - 1] : 0.f;
            const float qe = sgp->q2[T1];
            if (out) {
                const int t = T0 + col;
                const float qt = sgp->q2[t];
                const float ea = exp2f(qp - qt);
                float gv[4], av[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int sl = 4 * g + e;
                    gv[e] = sl <= col ? exp2f(sgp->q2[T0 + sl] - qt) * bf16_to_f32((uint16_t)sgp->gw[T0 + sl]) *
                                            sm.psi[col - sl]
                                      : 0.f;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 4 * g + i, j = row >> 1;
                    float val = 0.f;
                    if (j < M) {
                        const float2 cp = sm.cpw[col + 1][j < M ? j : 0];
                        val = ea * ((row & 1) ? -cp.y : cp.x);
                    }
                    av[i] = val;
                }
                // carry coefficients in bf16 hi and lo halves (mode terms may cancel)
                const f32x4_t af = f32x4_t{av[0], av[1], av[2], av[3]};
                const uint2 ah4 = hi4(af);
                const bf16x8_t bx = bf16x8_of(make_uint2(pk_bf16(gv[0], gv[1]), pk_bf16(gv[2], gv[3])), ah4);
                const bf16x8_t bxx = bf16x8_of(lo4(af, ah4), ah4);
                const float sc = bf16_to_f32((uint16_t)sgp->gr[t]);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    const uint2 hh = hi4(st[nt]);
                    f32x4_t acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        bf16x8_of(vfr[nt], hh), bx, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(hh, lo4(st[nt], hh)), bxx, acc, 0, 0,
                                                                  0);
                    stage_y(T, nt, acc, sc);
                }
            }
            // W[row = col][s] = {Re,Im}(lambda_j^{T1-s}) e^{-(qh(T1)-qh(s))} g_w(s), hi + lo
            float wv[4];
            {
                const int jr = col >> 1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = T0 + 4 * g + e;
                    float val = 0.f;
                    if (jr < M && s <= T1) {
                        const float2 pw = sm.pw[T1 - s][jr < M ? jr : 0];
                        val = ((col & 1) ? pw.y : pw.x) * exp2f(sgp->q2[s] - qe) * bf16_to_f32((uint16_t)sgp->gw[s]);
                    }
                    wv[e] = val;
                }
            }
            const uint32_t w01 = pk_bf16(wv[0], wv[1]), w23 = pk_bf16(wv[2], wv[3]);
            const bf16x8_t wf = bf16x8_of(make_uint2(w01, w23),
                                          make_uint2(pk_bf16(wv[0] - lo_f32(w01), wv[1] - hi_f32(w01)),
                                                     pk_bf16(wv[2] - lo_f32(w23), wv[3] - hi_f32(w23))));
            const float at = exp2f(qp - qe);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int j = 2 * g + hh;
                const float2 pn = j < M ? sm.pw[T1 - T0 + 1][j < M ? j : 0] : make_float2(0.f, 0.f);
                lam[2 * hh] = at * pn.x;
                lam[2 * hh + 1] = at * pn.y;
            }
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                f32x4_t d;
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const float hr = st[nt][i], hi = st[nt][i + 1];
                    d[i] = lam[i] * hr - lam[i + 1] * hi;
                    d[i + 1] = lam[i + 1] * hr + lam[i] * hi;
                }
                st[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, bf16x8_of(vfr[nt], vfr[nt]), d, 0, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            const float ar = tr[i], ai = tr[i + 1];
            tr[i] = ar * lam[i] - ai * lam[i + 1];
            tr[i + 1] = ar * lam[i + 1] + ai * lam[i];
        }
    };

    // One whole block of NB sub-blocks with the clock referenced to its middle:
    //   y(t) = a(t) g_r(t) [ sum_{s<=t} psi(t-s) b(s) v(s) + sum_j Re(c_j lambda_j^{t+1} H_s h_j) ]
    //   h'   = Lambda_e lambda^BLK h + A_e sum_s lambda^{BLK-1-s} b(s) v(s)
    // (positions relative to the block, H_s = a at the block's entry, A_e = a at
    // its end, Lambda_e = e^{-clock span}).  The state is carried once per block;
    // per sub-block only b(s) v(s) is formed (rounded to bf16) and fed to the
    // constant-operand products.
    auto block_fast = [&](f32x4_t (&st)[NTW], int Bi, bool out, bool wb,
                          float (&tr)[4]) __attribute__((always_inline)) {
        const float4 bk = sgp->blkB[Bi];
        uint2 hh[NTW], hl[NTW];
        if (out) {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const f32x4_t hs = st[nt] * bk.x;
                hh[nt] = hi4(hs);
                hl[nt] = lo4(hs, hh[nt]);
            }
        }
        f32x4_t mv[NTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) mv[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        uint2 bvh[NB][NTW];
        const uint2 z2 = make_uint2(0u, 0u);
#pragma unroll
        for (int aa = 0; aa < NB; ++aa) {
            const int T = Bi * NB + aa, T0 = T * 16;
            const float4 b4 = *reinterpret_cast<const float4*>(&sgp->bq[T0 + 4 * g]);
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const f32x4_t f = bv_f32(b4, load_vfrag(T, nt));
                bvh[aa][nt] = hi4(f);
                const uint2 bvl = lo4(f, bvh[aa][nt]);
                if (wb) store_bv(T, nt, bvh[aa][nt]);
                mv[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lpA[aa], bf16x8_of(bvh[aa][nt], bvh[aa][nt]), mv[nt],
                                                                 0, 0, 0);
                mv[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lpA[aa], bf16x8_of(bvl, bvl), mv[nt], 0, 0, 0);
            }
            if (out) {
                const float sc = sgp->ag[T0 + col];
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    f32x4_t acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(bvh[aa][nt], hh[nt]), yD[aa],
                                                                         f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(hh[nt], hl[nt]), yDx[aa], acc, 0, 0, 0);
                    if (aa >= 1)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            bf16x8_of(bvh[aa >= 1 ? aa - 1 : 0][nt], aa >= 2 ? bvh[aa >= 2 ? aa - 2 : 0][nt] : z2),
                            yB12, acc, 0, 0, 0);
                    if (aa >= 3)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(bvh[aa >= 3 ? aa - 3 : 0][nt], z2),
                                                                     yB3, acc, 0, 0, 0);
                    stage_y(T, nt, acc, sc);
                }
            }
        }
        float lam[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) lam[i] = bk.z * lB[i];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float hr = st[nt][i], hi = st[nt][i + 1];
                st[nt][i] = lam[i] * hr - lam[i + 1] * hi + bk.y * mv[nt][i];
                st[nt][i + 1] = lam[i + 1] * hr + lam[i] * hi + bk.y * mv[nt][i + 1];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            const float ar = tr[i], ai = tr[i + 1];
            tr[i] = ar * lam[i] - ai * lam[i + 1];
            tr[i + 1] = ar * lam[i + 1] + ai * lam[i];
        }
    };

    // Outputs of one whole block on the block path from the true state h
    // entering it; the state itself is not carried (the look-back launch's
    // output sweep knows every block's entering state).  The b(s) v(s)
    // fragments are the ones the first sweep wrote back into the tile.
    auto block_out = [&](const f32x4_t (&h)[NTW], int Bi) __attribute__((always_inline)) {
        const float4 bk = sgp->blkB[Bi];
        uint2 hh[NTW], hl[NTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const f32x4_t hs = h[nt] * bk.x;
            hh[nt] = hi4(hs);
            hl[nt] = lo4(hs, hh[nt]);
        }
        uint2 bvh[NB][NTW];
        const uint2 z2 = make_uint2(0u, 0u);
#pragma unroll
        for (int aa = 0; aa < NB; ++aa) {
            const int T = Bi * NB + aa, T0 = T * 16;
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) bvh[aa][nt] = load_bv(T, nt);
            const float sc = sgp->ag[T0 + col];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                f32x4_t acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(bvh[aa][nt], hh[nt]), yD[aa],
                                                                     f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(hh[nt], hl[nt]), yDx[aa], acc, 0, 0, 0);
                if (aa >= 1)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        bf16x8_of(bvh[aa >= 1 ? aa - 1 : 0][nt], aa >= 2 ? bvh[aa >= 2 ? aa - 2 : 0][nt] : z2), yB12,
                        acc, 0, 0, 0);
                if (aa >= 3)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(bvh[aa >= 3 ? aa - 3 : 0][nt], z2), yB3,
                                                                 acc, 0, 0, 0);
                stage_y(T, nt, acc, sc);
            }
        }
    };

    // All positions of the staged chunk (n valid): whole blocks on the block
    // path, the others (ragged, or a clock span too large) sub-block by sub-block.
    auto chunk_pass = [&](f32x4_t (&st)[NTW], int n, bool out, float (&tr)[4]) __attribute__((always_inline)) {
        if constexpr (PM_OPS) {
            // every sub-block's operands, wave w forming those of sub-blocks w, w + NW, ...
            for (int T = wave; T * 16 < n; T += C::NW) {
                const int ex = pm_exact(T, n);
                if (lane == 0) spm.fexact[T] = ex;
                bf16x8_t bx, bxx, wf;
                pm_operands(T, n, out, ex == 0, bx, bxx, wf);
                if (out) {
                    spm.opg[T][lane] = bx;
                    spm.opgx[T][lane] = bxx;
                }
                spm.opw[T][lane] = wf;
            }
            lds_barrier();
        }
        for (int Bi = 0; Bi * BLK < n; ++Bi) {
            if (sgp->blkB[Bi].w == 0.f) {
                block_fast(st, Bi, out, false, tr);
            } else {
                const int tend = min(n, (Bi + 1) * BLK);
                for (int T = Bi * NB; T * 16 < tend; ++T) subblock(st, T, n, out, tr, lpA[NB - 1], l16);
            }
        }
    };

    // staged y -> global, 16 bytes per lane (the units this lane loaded v from).
    // A streaming launch with P >= 128 (64 bytes of a row per wave) stores
    // non-temporally: measured faster there, slower with narrower rows.
    auto store_y = [&](int t0, int n) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            const int tr = i * C::RPI + vrow_l;
            const int t = t0 + tr;
            const uint4 outv = *reinterpret_cast<const uint4*>(&sgv[vt_off(tr, (int)(vcol0 >> 3))]);
            if (tr < n) {
                const size_t off = (((size_t)b * L + t) * K + k) * P + vcol0;
                if constexpr (P >= 128 && MODE == MODE_STREAM)
                    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, outv),
                                                reinterpret_cast<u32x4_t*>(yg + off));
                else
                    *reinterpret_cast<uint4*>(yg + off) = outv;
            }
        }
    };

    // staged y -> global by whole rows, non-temporally: each 128-byte line is
    // written by one instruction, so none is left dirty in L2 when the kernel
    // ends.  Needs every wave's y of the chunk staged (a barrier before).  Used
    // with P <= 64 by the look-back launch and the streaming launches, per-channel
    // and per-mode (measured faster there; with wider rows the read-back crosses
    // too many tile blocks).  In the per-mode launch, whose address registers
    // spill, the per-wave stores each waited for a reload and so for the store
    // before it: whole rows took the 370M-class per-mode call from 120 to 116 us.
    auto store_y_rows = [&](int t0, int n) __attribute__((always_inline)) {
        constexpr int UPR = P / 8;                     // 16-byte units per row
        constexpr int RPW = 64 / UPR;                  // rows per wave instruction
        constexpr int NI = LC / (RPW * C::NW);         // instructions per wave
        static_assert(LC % (RPW * C::NW) == 0, "rows must divide over the waves");
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = (i * C::NW + wave) * RPW + lane / UPR;
            const int u = lane % UPR;
            const uint4 outv = *reinterpret_cast<const uint4*>(&sgv[vt_off(r, u)]);
            if (r < n) {
                const size_t off = (((size_t)b * L + t0 + r) * K + k) * P + u * 8;
                __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, outv), reinterpret_cast<u32x4_t*>(yg + off));
            }
        }
    };

    // Look-back message rows: rows (j, re/im) of this lane's value columns.
    auto publish = [&](float* dst, const f32x4_t (&s)[NTW], unsigned kind,
                       const float (&trn)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int p = wave * WCOLS + nt * 16 + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                if (row < ROWS) st_agent(&dst[(size_t)row * P + p], s[nt][i]);
            }
        }
        if (kind == FLAG_AGG && wave == 0 && col == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                if (row < ROWS) st_agent(&plan.lam[(slot + seg) * ROWS + row], trn[i]);
            }
        }
        // The message stores are agent-scope (they write through the XCD's L2);
        // wait for their completion before the barrier that precedes the flag.
        // (An agent-scope release fence would also write back every dirty line
        // of this XCD's L2, which the message does not need.)
        wait_stores_complete();
        __syncthreads();
        if (tid == 0) st_agent_u(&plan.flags[slot + seg], tag | kind);
    };

    // Entering state of this segment: compose predecessors' messages backwards
    // until an inclusive state is found (segment 0 always publishes one).  Wave
    // 0 polls the flags of up to 64 predecessors at once; once every
    // predecessor nearer than the nearest inclusive one has its aggregate out,
    // all of those messages are read (independent loads) and folded in order.
    auto lookback = [&](f32x4_t (&e)[NTW]) __attribute__((always_inline)) {
        float cf[4] = {1.f, 0.f, 1.f, 0.f};   // accumulated transfer of modes 2g, 2g+1
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) e[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        int hi = seg - 1;                     // nearest predecessor not folded yet
        while (hi >= 0) {
            if (wave == 0) {
                const int nwin = min(64, hi + 1);
                int cnt = 1;
                bool found = true;
                int it = 0;
                for (; it < SPIN_LIMIT; ++it) {
                    const unsigned f = lane < nwin ? ld_agent_u(&plan.flags[slot + hi - lane]) : 0u;
                    const bool ready = (f & ~3u) == tag && (f & 3u) != 0;
                    const unsigned long long minc = __ballot(ready && (f & 3u) == FLAG_INCL);
                    const unsigned long long mrdy = __ballot(ready);
                    found = minc != 0ull;
                    cnt = found ? __ffsll((long long)minc) : nwin;   // predecessors to fold
                    const unsigned long long need = cnt >= 64 ? ~0ull : ((1ull << cnt) - 1ull);
                    if ((mrdy & need) == need) break;
                    __builtin_amdgcn_s_sleep(2);
                }
                if (it == SPIN_LIMIT) {
                    if (lane == 0)
                        __hip_atomic_fetch_or(&plan.hdr[SCAN_HDR_ERROR], SCAN_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                    cnt = 1;        // give up: treat the (unwritten) nearest state as final
                    found = true;
                }
                if (lane == 0) {
                    sm.lb_cnt = cnt;
                    sm.lb_found = found ? 1 : 0;
                }
            }
            __syncthreads();
            const int cnt = sm.lb_cnt;
            const bool found = sm.lb_found != 0;
            __syncthreads();   // sm.lb_* may be rewritten by the next window
            for (int l0 = 0; l0 < cnt; l0 += LB_BATCH) {
                float sv[LB_BATCH][NTW][4], lv[LB_BATCH][4];
#pragma unroll
                for (int u = 0; u < LB_BATCH; ++u) {
                    const int l = l0 + u;
                    if (l >= cnt) break;
                    const int pred = hi - l;
                    const bool incl = found && l == cnt - 1;
                    const float* src = (incl ? plan.incl : plan.agg) + (slot + pred) * (size_t)ROWS * P;
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt) {
                        const int p = wave * WCOLS + nt * 16 + col;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int row = 4 * g + i;
                            sv[u][nt][i] = row < ROWS ? ld_agent(&src[(size_t)row * P + p]) : 0.f;
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 4 * g + i;
                        lv[u][i] = (!incl && row < ROWS) ? ld_agent(&plan.lam[(slot + pred) * ROWS + row]) : 0.f;
                    }
                }
#pragma unroll
                for (int u = 0; u < LB_BATCH; ++u) {
                    if (l0 + u >= cnt) break;
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
                        for (int i = 0; i < 4; i += 2) {
                            const float sr = sv[u][nt][i], si = sv[u][nt][i + 1];
                            e[nt][i] += cf[i] * sr - cf[i + 1] * si;
                            e[nt][i + 1] += cf[i] * si + cf[i + 1] * sr;
                        }
                    }
                    // compose with this predecessor's transfer: cf <- cf * Lambda_pred
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        const float ar = cf[i], ai = cf[i + 1];
                        cf[i] = ar * lv[u][i] - ai * lv[u][i + 1];
                        cf[i + 1] = ar * lv[u][i + 1] + ai * lv[u][i];
                    }
                }
            }
            if (found) break;
            hi -= cnt;
        }
    };

    // ---- the two sweeps -------------------------------------------------------------------------
    // Sweep 1 (segmented scan, segments with a successor): the end state from a
    // zero entering state, or the true one for segment 0.  Sweep 2: outputs.
    // Each chunk step stages the chunk held in the register buffer and refills
    // it with the loads of the next chunk, which then overlap the arithmetic.
    f32x4_t st[NTW];
    float tr[4] = {1.f, 0.f, 1.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) st[nt] = SEG ? f32x4_t{0.f, 0.f, 0.f, 0.f} : st_in[nt];

    ChunkRegs rb;
    if (SEG) {
        // Segment: its (at most RES) chunks were requested up front and stay in LDS.
        constexpr int NBC = LC / BLK;   // blocks per chunk
        const bool has_succ = seg + 1 < nseg;
        if (!has_succ && seg > 0) {
            // last segment: the entering state first, so that the first sweep
            // already runs from the true state
            f32x4_t e[NTW];
            lookback(e);
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) st[nt] = e[nt];
        }
        // The control copies were issued before every tile copy: they have
        // landed once at most this wave's tile copies are outstanding.  Wave w
        // turns the controls of chunks w, w + NW, ... into the chunk factors.
        wait_vmem_at_most<C::RES * TLW>();
        lds_barrier();
#pragma unroll
        for (int i = 0; i < C::RES; ++i) {
            if (i % C::NW == wave && i < nck) {
                sgp = stage_c(i);
                float cd[C::CPL];
                uint32_t cw[C::CPL], cr[C::CPL];
#pragma unroll
                for (int u = 0; u < C::CPL; ++u) {
                    const int idx = min(lane * C::CPL + u, LC - 1);
                    cd[u] = sgp->q2[idx];
                    cw[u] = sgp->gw[idx];
                    cr[u] = sgp->gr[idx];
                }
                stage_ctrl(cd, cw, cr, min(LC, L - (c_begin + i) * LC));
            }
        }
        // Sweep 1: the state through the segment from a zero entering state (the
        // looked-back state for the last segment), recorded at every block
        // start; each chunk as soon as its tile has landed.
        f32x4_t h0[C::RES][NBC][NTW];
        static_for<0, C::RES>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            wait_vmem_at_most<(C::RES - 1 - i) * TLW>();
            lds_barrier();   // every wave's copies of tile i (and, first, the factors)
            if (i < nck) {
                const int n = min(LC, L - (c_begin + i) * LC);
                sgp = stage_c(i);
                sgv = stage_v(i);
#pragma unroll
                for (int Bi = 0; Bi < NBC; ++Bi) {
                    if (Bi * BLK < n) {
#pragma unroll
                        for (int nt = 0; nt < NTW; ++nt) h0[i][Bi][nt] = st[nt];
                        if (sgp->blkB[Bi].w == 0.f) {
                            block_fast(st, Bi, false, true, tr);
                        } else {
                            const int tend = min(n, (Bi + 1) * BLK);
                            for (int T = Bi * NB; T * 16 < tend; ++T) subblock(st, T, n, false, tr, lpA[NB - 1], l16);
                        }
                    }
                }
            }
        });
        // Entering state, publish, look back.  gc: the entering state carried
        // to the current block by the transfers of the blocks before it; the
        // true state at a block start is h0 + gc (gc = 0 where sweep 1 began
        // from the true state).
        f32x4_t gc[NTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) gc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // st <- Lambda_seg * e + st (the inclusive state from the aggregate)
        auto enter = [&](const f32x4_t (&e)[NTW]) __attribute__((always_inline)) {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const float ir = tr[i] * e[nt][i] - tr[i + 1] * e[nt][i + 1] + st[nt][i];
                    const float ii = tr[i] * e[nt][i + 1] + tr[i + 1] * e[nt][i] + st[nt][i + 1];
                    st[nt][i] = ir;
                    st[nt][i + 1] = ii;
                }
                gc[nt] = e[nt];
            }
        };
        if (seg == 0) {
            f32x4_t e[NTW];
            load_entering(e);   // state_in, or zero
            enter(e);
            if (has_succ) publish(plan.incl + (slot + seg) * (size_t)ROWS * P, st, FLAG_INCL, tr);
        } else if (has_succ) {
            publish(plan.agg + (slot + seg) * (size_t)ROWS * P, st, FLAG_AGG, tr);
            f32x4_t e[NTW];
            lookback(e);
            enter(e);
            publish(plan.incl + (slot + seg) * (size_t)ROWS * P, st, FLAG_INCL, tr);
        }
        // Sweep 2: outputs from the resident chunks.  Each wave reads and
        // overwrites only its own columns; a barrier per chunk precedes the
        // whole-row stores.
        make_out_constants();
#pragma unroll
        for (int i = 0; i < C::RES; ++i) {
            if (i < nck) {
                const int t0 = (c_begin + i) * LC;
                const int n = min(LC, L - t0);
                sgp = stage_c(i);
                sgv = stage_v(i);
#pragma unroll
                for (int Bi = 0; Bi < NBC; ++Bi) {
                    if (Bi * BLK < n) {
                        f32x4_t h[NTW];
#pragma unroll
                        for (int nt = 0; nt < NTW; ++nt) h[nt] = h0[i][Bi][nt] + gc[nt];
                        const float4 bk = sgp->blkB[Bi];
                        if (bk.w == 0.f) {
                            block_out(h, Bi);
                        } else {
                            const bf16x8_t al_r = make_sub_al();
                            float l16_r[4], trd[4] = {1.f, 0.f, 1.f, 0.f};
                            make_l16(l16_r);
                            const int tend = min(n, (Bi + 1) * BLK);
                            for (int T = Bi * NB; T * 16 < tend; ++T) subblock(h, T, n, true, trd, al_r, l16_r);
                        }
                        // carry gc over this (whole) block: lambda^BLK e^{-span}
#pragma unroll
                        for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
                            for (int q = 0; q < 4; q += 2) {
                                const float lr = bk.z * lB[q], li = bk.z * lB[q + 1];
                                const float gr = gc[nt][q], gi = gc[nt][q + 1];
                                gc[nt][q] = lr * gr - li * gi;
                                gc[nt][q + 1] = lr * gi + li * gr;
                            }
                        }
                    }
                }
                if constexpr (P <= 64) {
                    lds_barrier();   // every wave's y of this chunk is staged
                    store_y_rows(t0, n);
                } else {
                    store_y(t0, n);
                }
            }
        }
    } else {
        // Whole sequence or segment, streamed through one staging buffer.  The
        // y of chunk c-1 stays staged until the loads of chunk c have been
        // waited for, so that this wait never includes the stores of y (vector
        // memory operations complete in issue order for the wait counter).
        load_chunk(rb, c_begin);
        int yt0 = -1, yn = 0;
        for (int c = c_begin; c < c_end; ++c) {
            const int t0 = c * LC;
            const int n = min(LC, L - t0);
            __builtin_amdgcn_s_waitcnt(WAIT_VMEM0);   // loads of chunk c, issued a chunk ago
            if (!AGG && yt0 >= 0) {
                if constexpr (P <= 64 && (MODE == MODE_STREAM || MODE == MODE_STREAM_PM)) {
                    lds_barrier();   // every wave's y of chunk c-1 is staged
                    store_y_rows(yt0, yn);
                } else {
                    store_y(yt0, yn);   // each wave reads back only its own columns
                }
            }
            stage_chunk(rb, n, c + 1 < c_end ? c + 1 : -1);
            chunk_pass(st, n, !AGG, tr);
            yt0 = t0;
            yn = n;
        }
        if (!AGG && yt0 >= 0) {
            if constexpr (P <= 64 && (MODE == MODE_STREAM || MODE == MODE_STREAM_PM)) {
                lds_barrier();
                store_y_rows(yt0, yn);
            } else {
                store_y(yt0, yn);
            }
        }
    }

    // ---- segment aggregate (three-launch scan) ----------------------------------------------
    if (AGG) {
        float* dst = plan.agg + (slot + seg) * (size_t)ROWS * P;
        float* ent = plan.incl + slot * (size_t)ROWS * P;   // entering state of segment 0
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int p = wave * WCOLS + nt * 16 + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                if (row < ROWS) {
                    dst[(size_t)row * P + p] = st[nt][i];
                    if (seg == 0) ent[(size_t)row * P + p] = st_in[nt][i];
                }
            }
        }
        if (wave == 0 && col == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                if (row < ROWS) plan.lam[(slot + seg) * ROWS + row] = tr[i];
            }
        }
    }

    // ---- leaving state ----------------------------------------------------------------------
    if (!AGG && seg + 1 >= nseg && a.state_out) {
        const size_t base = ((size_t)b * K + k) * M;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int p = wave * WCOLS + nt * 16 + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i, j = row >> 1, cmp = row & 1;
                if (j < M) a.state_out[((base + j) * 2 + cmp) * P + p] = st[nt][i];
            }
        }
    }

    if (SEG) finish_launch();
}

}  // namespace
}  // namespace essh
