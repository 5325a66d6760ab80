// prefill_wave.hip -- the chunked parallel scan with one wave per (sequence, segment), for
// channels of P = 64 values with per-channel clock and gates (bf16 io).
//
// ESSH paper, Sec. 4.3 "Chunked parallel training": inside a chunk the source-to-target
// contributions form a dense causal matrix applied by matrix multiplication; only the
// 2 m P mode-state entries of a channel cross a chunk boundary (Eq. 6 gives the transition
// product that makes this exact).
//
// The block algebra (64-position blocks of four 16-position sub-blocks, clock referenced to
// the middle of the block, mid = qe / 2 with q the clock sum from the block start and qe
// its value at the block's end):
//   a(t) = e^{-(q(t) - mid)},  b(s) = e^{q(s) - mid} g_w(s),  Hs = e^{-mid},
//   Ae = e^{-(qe - mid)},      Le = e^{-qe},
//   y(t) = g_r(t) a(t) [ sum_{s<=t} psi(t-s) b(s) v(s) + Hs sum_j Re(c_j lambda_j^{t+1} h_j) ]
//   h_j' = Le lambda_j^64 h_j + Ae sum_s lambda_j^{63-s} b(s) v(s)
// with lambda_j = rho_j e^{i theta_j} and psi(tau) = sum_j Re(c_j lambda_j^tau).  A block that
// is ragged or whose clock span exceeds 2^128 (log2 units) is done sub-block by sub-block with
// operands formed from exponentials of clock differences instead (the same function).
//
// gfx950 mapping.  The wave owns all 64 value columns of its channel, as four 16-column
// MFMA tiles.  Every factor of the matrices above depends on the positions only, not on the
// value column, so the operands that carry them are formed once per block and shared by the
// four tiles, and v enters every v_mfma_f32_16x16x32_bf16 exactly as read from LDS:
//   output, target sub-block a (B operands, lane (g, col) = target position t = 16a + col):
//     [ g_r a(t) b(s) psi(t-s) for s in sub-block a ; C hi ] against A = [ v(s) ; state hi ],
//     and [ C lo ; C hi ] against A = [ state hi ; state lo ], with C = g_r a(t) Hs
//     {Re,-Im}(c lambda^{t+1}) split into bf16 halves (the modes' readout terms may cancel);
//     then the pieces of the three preceding sub-blocks against A = [ v ; v ].
//   state, source sub-block a (A operand, lane (g, col) = state row (mode, re/im)):
//     {Re, Im}(lambda^{63-s}) b(s) split into bf16 hi and lo halves, against B = [ v ; v ],
//     so the state product is exact up to the lambda-power and b(s) rounding to ~16 bits.
// Blocks are staged by asynchronous global-to-LDS copies into a ring of two stages (8 KB of v
// plus the block's controls each), one block ahead, so that eight waves fit a CU; y is staged
// in place and written back by whole 128-byte rows.  v is copied by whole 128-byte rows too; the controls come from a
// channel-major copy made by a first launch (pack_ctrl_kernel), so that a block's controls
// are two contiguous 256-byte reads instead of 64-way gathers across the channel rows.
#include "prefill_chunk_kernel.h"

namespace essh {
namespace {

constexpr int WP = 64;            // values per channel (four 16-column tiles)
constexpr int WBLK = 64;          // positions per block
constexpr int WSTV = WBLK * WP;   // bf16 elements of one v stage
// vector memory operations a lane issues per staged block: 8 row copies, 2 control copies
constexpr int WCPY = 8 + 2;

// A v stage is row-major, [64 positions][64 values], with the eight 16-byte units of row r
// permuted: unit u sits at u ^ swz(r).  The transposing fragment reads (8 rows x 32 bytes per
// half wave), the y writes by target row (16 rows x 16 bytes) and the row read-back for the
// global stores then each touch every LDS bank once.
__device__ __forceinline__ int swz(int r) { return (r & 6) | ((r >> 3) & 1); }

// Every LDS access issued so far has completed, and no instruction is moved across this point
// in either direction (a stage's last reads before an asynchronous copy overwrites it).
__device__ __forceinline__ void stage_reads_done() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int M>
struct __align__(16) WTables {
    float2 pw[17 + 5][M];         // lambda_j^tau, tau = 0..16; rows 17 + d: lambda_j^{16 d}, d = 0..4
    float2 cpw[17][M];            // c_j lambda_j^tau
    float psi[WBLK];              // psi(tau), zero-lag corrected at tau = 0
    float4 mtab[M];               // (rho, theta, Re c, Im c)
    float mza[M];                 // zero-lag coefficients a_j
};
struct __align__(16) WStageC {
    float dl[WBLK];               // clock
    uint32_t gg[WBLK];            // write gate bf16 bits | read gate bf16 bits << 16
};
struct __align__(16) WStage {
    uint16_t v[WSTV];
    WStageC c;
};
struct __align__(16) WFactors {   // per-position factors of the sub-block path
    float bq[WBLK];               // clock sum from the block start (log2 units)
    float ag[WBLK];               // write gate
    float gr[WBLK];               // read gate
};

// Channel-major copy of the controls of the retained channels, sequence seq = b K_T + k:
//   cdl[seq][t] = delta(b, t, k),  cgg[seq][t] = g_w bits | g_r bits << 16.
// One workgroup per 64 positions x 32 channels of one batch row, transposed through LDS so
// that both the reads (along the channels of a position) and the writes (along the positions
// of a channel) are contiguous.
__global__ void __launch_bounds__(256) pack_ctrl_kernel(PrefillArgs a, ScanPlan plan) {
    __shared__ float sd[32][WBLK + 1];
    __shared__ uint32_t sg[32][WBLK + 1];
    const int t0 = blockIdx.x * WBLK, k0 = blockIdx.y * 32, b = blockIdx.z;
    const uint16_t* gw = static_cast<const uint16_t*>(a.g_w);
    const uint16_t* gr = static_cast<const uint16_t*>(a.g_r);
    const bool vec4 = (a.K & 3) == 0 && (a.K_T & 3) == 0 && (reinterpret_cast<uintptr_t>(a.delta) & 15) == 0 &&
                      (reinterpret_cast<uintptr_t>(gw) & 7) == 0 && (reinterpret_cast<uintptr_t>(gr) & 7) == 0;
    if (vec4) {
        // four channels per load: 16-byte clock and 8-byte gate reads (rows start at a
        // multiple of four channels)
        for (int i = threadIdx.x; i < 8 * WBLK; i += 256) {
            const int pos = i >> 3, kq = 4 * (i & 7);
            const int t = t0 + pos, k = k0 + kq;
            if (t < a.L && k < a.K_T) {
                const size_t row = ((size_t)b * a.L + t) * a.K + k;
                const float4 d = *reinterpret_cast<const float4*>(a.delta + row);
                const uint2 w = *reinterpret_cast<const uint2*>(gw + row);
                const uint2 r = *reinterpret_cast<const uint2*>(gr + row);
                sd[kq][pos] = d.x;
                sd[kq + 1][pos] = d.y;
                sd[kq + 2][pos] = d.z;
                sd[kq + 3][pos] = d.w;
                sg[kq][pos] = (w.x & 0xffffu) | (r.x << 16);
                sg[kq + 1][pos] = (w.x >> 16) | (r.x & 0xffff0000u);
                sg[kq + 2][pos] = (w.y & 0xffffu) | (r.y << 16);
                sg[kq + 3][pos] = (w.y >> 16) | (r.y & 0xffff0000u);
            }
        }
    } else {
        for (int i = threadIdx.x; i < 32 * WBLK; i += 256) {
            const int pos = i >> 5, kk = i & 31;
            const int t = t0 + pos, k = k0 + kk;
            if (t < a.L && k < a.K_T) {
                const size_t row = ((size_t)b * a.L + t) * a.K + k;
                sd[kk][pos] = a.delta[row];
                sg[kk][pos] = (uint32_t)gw[row] | ((uint32_t)gr[row] << 16);
            }
        }
    }
    __syncthreads();
    if ((a.L & 3) == 0) {
        // four positions per store (a channel's row starts at a multiple of four positions)
        for (int i = threadIdx.x; i < 32 * (WBLK / 4); i += 256) {
            const int kk = i >> 4, pos = 4 * (i & 15);
            const int t = t0 + pos, k = k0 + kk;
            if (t < a.L && k < a.K_T) {   // L % 4 == 0: the four positions are all in range
                const size_t o = ((size_t)b * a.K_T + k) * a.L + t;
                *reinterpret_cast<float4*>(plan.cdl + o) =
                    make_float4(sd[kk][pos], sd[kk][pos + 1], sd[kk][pos + 2], sd[kk][pos + 3]);
                *reinterpret_cast<uint4*>(plan.cgg + o) =
                    make_uint4(sg[kk][pos], sg[kk][pos + 1], sg[kk][pos + 2], sg[kk][pos + 3]);
            }
        }
    } else {
        for (int i = threadIdx.x; i < 32 * WBLK; i += 256) {
            const int kk = i >> 6, pos = i & 63;
            const int t = t0 + pos, k = k0 + kk;
            if (t < a.L && k < a.K_T) {
                const size_t o = ((size_t)b * a.K_T + k) * a.L + t;
                plan.cdl[o] = sd[kk][pos];
                plan.cgg[o] = sg[kk][pos];
            }
        }
    }
}

template <int M, int NS, int MODE>
__global__ void __launch_bounds__(64) wave_prefill_kernel(PrefillArgs a, ScanPlan plan) {
    static_assert(MODE == MODE_STREAM || MODE == MODE_AGG, "streaming or segment-aggregate role");
    static_assert(NS >= 2 && NS <= 4, "two to four stages");
    // The ring's partial waits count outstanding vector memory operations.  Loads complete in
    // issue order, but a store may complete before or after a load issued around it, so a
    // partial count proves nothing once the streaming role's y stores are interleaved with
    // the copies: that role waits for all of them (two stages).
    static_assert(MODE == MODE_AGG || NS == 2, "the streaming role waits with a zero count");
    constexpr bool AGG = MODE == MODE_AGG;
    constexpr int ROWS = 2 * M;
    __shared__ WTables<M> tb;
    __shared__ WFactors fc;
    // Each stage (v and controls together) is an LDS object of its own: the compiler follows
    // the asynchronous copies into LDS per object (a few objects at most), and orders a read
    // of one stage only behind the copies into that stage.
    __shared__ WStage st0, st1, st2, st3;
    // (a stage index past NS - 1 never occurs; the selections name only the NS stages in use,
    // so the others are not allocated even where the index is not a compile-time constant)
    auto stg = [&](int s) __attribute__((always_inline)) -> WStage* {
        return s == 0 ? &st0 : (NS == 2 || s == 1) ? &st1 : (NS == 3 || s == 2) ? &st2 : &st3;
    };
    auto stv = [&](int s) __attribute__((always_inline)) -> uint16_t* { return stg(s)->v; };
    auto stc = [&](int s) __attribute__((always_inline)) -> WStageC* { return &stg(s)->c; };

    const int lane = threadIdx.x;
    const int g = lane >> 4;
    const int col = lane & 15;

    // ---- work item: segment-major order (neighbouring items are neighbouring channels) --------
    const int item = remap_xcd(blockIdx.x, gridDim.x);
    int seg = item / plan.nseq;
    const int seq = item - seg * plan.nseq;
    const int nseg = plan.nseg;
    // A segment streamed from its entering state (three-launch scan) runs last segment
    // first: the aggregate launch read the sequence front to back, so its last segments are
    // the most likely still to sit in the memory-side cache.
    if (!AGG && nseg > 1) seg = nseg - 1 - seg;
    const int k = seq % a.K_T;
    const int b = seq / a.K_T;
    const int L = a.L, K = a.K;
    const int t_beg = seg * plan.seg_chunks * a.Lc;
    const int t_end = min(L, t_beg + plan.seg_chunks * a.Lc);
    const int nblk = (t_end - t_beg + WBLK - 1) / WBLK;
    const size_t slot = (size_t)seq * nseg;

    const uint16_t* vg = static_cast<const uint16_t*>(a.v);
    uint16_t* yg = static_cast<uint16_t*>(a.y);

    // ---- entering state, accumulator layout: lane (g, col) holds rows 4g..4g+3 of column col ----
    // Both sources are [2m rows][P] (row = 2 j + re/im): the segment's slot of the three-launch
    // scan's entering states, or this channel's state_in for segment 0.  Rows past 2m read
    // row 2m-1 and are zeroed, so the sixteen loads go out back to back.
    const float* sbase = !AGG && nseg > 1 ? plan.incl + (slot + seg) * ROWS * (size_t)WP
                         : (seg == 0 && a.state_in) ? a.state_in + ((size_t)b * K + k) * ROWS * WP
                                                    : nullptr;
    f32x4_t st[4], st_in[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * g + i;
            const float x = sbase ? sbase[(row < ROWS ? row : ROWS - 1) * WP + nt * 16 + col] : 0.f;
            st_in[nt][i] = row < ROWS ? x : 0.f;
        }
        st[nt] = st_in[nt];
    }

    // ---- staging of one block: 8 row copies (8 rows x 128 bytes each; lane l fills physical
    // unit l%8 of row l/8, so it reads that row's unit (l%8) ^ swz) and 2 control copies (one
    // position per lane).  Rows past the segment repeat its last row, so every block issues
    // the same WCPY operations.
    const int cp_row = lane >> 3;
    const int cp_u0 = (lane & 7) ^ swz(cp_row);        // rows 8 it + cp_row: it even
    const int cp_u1 = (lane & 7) ^ swz(cp_row + 8);    // it odd
    const float* cdl = plan.cdl + (size_t)seq * L;
    const uint32_t* cgg = plan.cgg + (size_t)seq * L;
    auto copy_block = [&](int s, int blk) __attribute__((always_inline)) {
        const int t0 = t_beg + blk * WBLK;
        uint16_t* dv = stv(s);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int t = min(t0 + 8 * it + cp_row, t_end - 1);
            const uint16_t* src = vg + (((size_t)b * L + t) * K + k) * WP + ((it & 1) ? cp_u1 : cp_u0) * 8;
            __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(dv + it * 512), 16, 0, 0);
        }
        WStageC* dc = stc(s);
        const int t = min(t0 + lane, t_end - 1);
        __builtin_amdgcn_global_load_lds(cdl + t, (lds_void_t*)(&dc->dl[0]), 4, 0, 0);
        __builtin_amdgcn_global_load_lds(cgg + t, (lds_void_t*)(&dc->gg[0]), 4, 0, 0);
    };
    // the copies of the first NS-1 blocks go out before the tables are built
    static_for<0, NS - 1>([&](auto ic) __attribute__((always_inline)) { copy_block(decltype(ic)::value, decltype(ic)::value); });

    // ---- pole tables of channel k (scalar loads of the mode tables; LDS-only barriers) --------
    {
        const cfloat_p rho_s = (cfloat_p)(a.rho) + k * M;
        const cfloat_p th_s = (cfloat_p)(a.theta) + k * M;
        const cfloat_p c_s = (cfloat_p)(a.c) + 2 * k * M;
        const cfloat_p zl_s = (cfloat_p)(a.zl ? a.zl : a.rho) + k * M;   // never a null base
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const float4 mt = make_float4(rho_s[j], th_s[j], c_s[2 * j], c_s[2 * j + 1]);
            const float za = a.zl ? zl_s[j] : 0.f;
            if (lane == j) {
                tb.mtab[j] = mt;
                tb.mza[j] = za;
            }
        }
    }
    lds_barrier();
    for (int idx = lane; idx < 22 * M; idx += 64) {
        const bool blk16 = idx >= 17 * M;
        const int id2 = blk16 ? idx - 17 * M : idx;
        const int i0 = id2 / M, j = id2 - i0 * M;
        const int tau = blk16 ? 16 * i0 : i0;
        const float4 mt = tb.mtab[j];
        const float mag = tau == 0 ? 1.f : exp2f((float)tau * log2f(mt.x));
        float sn, cs;
        sincosf(mt.y * (float)tau, &sn, &cs);   // |theta tau| <= 64 pi
        const float pr = mag * cs, pi = mag * sn;
        tb.pw[blk16 ? 17 + i0 : tau][j] = make_float2(pr, pi);
        if (!blk16) tb.cpw[tau][j] = make_float2(mt.z * pr - mt.w * pi, mt.z * pi + mt.w * pr);
    }
    lds_barrier();
    {
        // psi(16 d + r) = sum_j Re(c_j lambda_j^r lambda_j^{16 d}); the zero-lag correction
        // (Eq. 24) with per-channel gates lowers the lag-0 coefficient by sum_j a_j Re(c_j)
        const int tau = lane, d = tau >> 4, r = tau & 15;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const float2 cp = tb.cpw[r][j], pd = tb.pw[17 + d][j];
            s += cp.x * pd.x - cp.y * pd.y;
            if (tau == 0) s -= tb.mza[j] * tb.mtab[j].z;
        }
        tb.psi[tau] = s;
    }
    lds_barrier();

    // ---- per-lane constants of the block path --------------------------------------------------
    //   psv[d][e] = psi(16 d + col - 4g - e)      (d = 0: zero where 4g + e > col)
    //   c0[a][i]  = {Re, -Im}(c_j lambda_j^{16 a + col + 1}), row 4g + i = (j, re/im)
    //   lw[a][e]  = {Re, Im}(lambda_j^{63 - 16 a - 4g - e}), row col = (j, re/im)
    //   l64[.]    = lambda_j^64 for this lane's modes 2g, 2g + 1
    float psv[4][4], c0[4][4], lw[4][4], l64[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int lag = 16 * d + col - 4 * g - e;
            psv[d][e] = lag >= 0 ? tb.psi[lag < 0 ? 0 : lag] : 0.f;
        }
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * g + i, j = row >> 1, jj = j < M ? j : 0;
            const float2 cp = tb.cpw[col + 1][jj], pd = tb.pw[17 + aa][jj];
            const float re = cp.x * pd.x - cp.y * pd.y, im = cp.x * pd.y + cp.y * pd.x;
            c0[aa][i] = j < M ? ((row & 1) ? -im : re) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int jr = col >> 1, jj = jr < M ? jr : 0;
            const float2 pw = tb.pw[15 - 4 * g - e][jj], pd = tb.pw[17 + 3 - aa][jj];
            const float re = pw.x * pd.x - pw.y * pd.y, im = pw.x * pd.y + pw.y * pd.x;
            lw[aa][e] = jr < M ? ((col & 1) ? im : re) : 0.f;
        }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int j = 2 * g + hh, jj = j < M ? j : 0;
        const float2 p64 = tb.pw[17 + 4][jj];
        l64[2 * hh] = j < M ? p64.x : 0.f;
        l64[2 * hh + 1] = j < M ? p64.y : 0.f;
    }

    auto hi4 = [&](const f32x4_t& x) __attribute__((always_inline)) -> uint2 {
        return make_uint2(pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3]));
    };
    auto lo4 = [&](const f32x4_t& x, uint2 h) __attribute__((always_inline)) -> uint2 {
        return make_uint2(pk_bf16(x[0] - lo_f32(h.x), x[1] - hi_f32(h.x)),
                          pk_bf16(x[2] - lo_f32(h.y), x[3] - hi_f32(h.y)));
    };
    const uint2 z2 = make_uint2(0u, 0u);
    const f32x4_t zf = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // v fragment of sub-block T, tile nt: positions 16T + 4g .. +3 of column 16 nt + col, by one
    // transposing LDS read (lane (g, col) addresses row 16T + 4g + col/4, columns 16 nt + 4 (col % 4)
    // .. +3).  swz of that row does not depend on T, so the per-tile offsets are lane constants.
    int vf_off[4], sy_off[4];
    {
        const int r = 4 * g + (col >> 2), sr = swz(r), sc = swz(col);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            vf_off[nt] = r * WP + (((2 * nt + ((col & 3) >> 1)) ^ sr) << 3) + 4 * (col & 1);
            sy_off[nt] = col * WP + (((2 * nt + (g >> 1)) ^ sc) << 3) + 4 * (g & 1);
        }
    }
    auto vfrag = [&](const uint16_t* sv, int T, int nt) __attribute__((always_inline)) -> uint2 {
        const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(sv + T * 16 * WP + vf_off[nt]));
        return __builtin_bit_cast(uint2, x);
    };
    // y of target rows t (lane (g, col): t = 16T + col, columns 16 nt + 4g .. +3) into the stage
    auto stage_y = [&](uint16_t* sv, int T, int nt, const f32x4_t& acc) __attribute__((always_inline)) {
        *reinterpret_cast<uint2*>(sv + T * 16 * WP + sy_off[nt]) = hi4(acc);
    };
    // staged y of block blk -> global by whole 128-byte rows (lane l: row l/8 + 8 i, 16-byte unit
    // l%8); rows past the segment repeat its last row (same bytes), so every block issues 8 stores
    auto store_y = [&](const uint16_t* sv, int blk) __attribute__((always_inline)) {
        const int t0 = t_beg + blk * WBLK;
        const int n = min(WBLK, t_end - t0);
        const int u = lane & 7;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = min((lane >> 3) + 8 * i, n - 1);
            const uint4 x = *reinterpret_cast<const uint4*>(sv + r * WP + ((u ^ swz(r)) << 3));
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, x),
                                        reinterpret_cast<u32x4_t*>(yg + (((size_t)b * L + t0 + r) * K + k) * WP + u * 8));
        }
    };

    float tr[4] = {1.f, 0.f, 1.f, 0.f};   // transfer of the segment so far, modes 2g, 2g+1

    // ---- one block -------------------------------------------------------------------------------
    auto compute_block = [&](uint16_t* sv, const WStageC* sc, int blk) __attribute__((always_inline)) {
        const int t0 = t_beg + blk * WBLK;
        const int n = min(WBLK, t_end - t0);
        // controls, one position per lane; the inclusive clock sum by a wave scan
        const float dl = lane < n ? sc->dl[lane] : 0.f;
        const uint32_t ggv = sc->gg[lane];
        const float gwv = __uint_as_float(ggv << 16);
        const float grv = __uint_as_float(ggv & 0xffff0000u);
        float q = dl;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(q, off);
            if (lane >= off) q += o;
        }
        const float q2 = q * LOG2E;
        const float qe2 = __shfl(q2, n - 1);
        float lam[4];
        if (n == WBLK && qe2 <= SPAN2_BLOCK_MAX) {
            // ---- block path ----
            const float mid = 0.5f * qe2;
            // b(s) and g_r(t) a(t) stay in registers and are read across lanes: an LDS copy of
            // them would make the compiler wait for every copy in flight before reading it
            const float bql = exp2f(q2 - mid) * gwv;
            const float agl = exp2f(mid - q2) * grv;
            const float Hs = exp2f(-mid), Ae = exp2f(mid - qe2), Le = exp2f(-qe2);
            float4 bq4[4];
#pragma unroll
            for (int aa = 0; aa < 4; ++aa)
                bq4[aa] = make_float4(__shfl(bql, 16 * aa + 4 * g), __shfl(bql, 16 * aa + 4 * g + 1),
                                      __shfl(bql, 16 * aa + 4 * g + 2), __shfl(bql, 16 * aa + 4 * g + 3));
            const float bqv[4][4] = {{bq4[0].x, bq4[0].y, bq4[0].z, bq4[0].w},
                                     {bq4[1].x, bq4[1].y, bq4[1].z, bq4[1].w},
                                     {bq4[2].x, bq4[2].y, bq4[2].z, bq4[2].w},
                                     {bq4[3].x, bq4[3].y, bq4[3].z, bq4[3].w}};
            uint2 hh[4], hl[4];
            if constexpr (!AGG) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    hh[nt] = hi4(st[nt]);
                    hl[nt] = lo4(st[nt], hh[nt]);
                }
            }
            // Sub-blocks last to first: target sub-block aa reads v of sub-blocks aa, aa-1, ..
            // only, so once its y is staged over its own rows no later step needs those rows,
            // and every fragment is read from LDS where it is used.  Source sub-block aa's
            // state product goes in the same step, before its rows are overwritten.
            f32x4_t mv[4] = {zf, zf, zf, zf};
#pragma unroll
            for (int aa = 3; aa >= 0; --aa) {
                const f32x4_t w = f32x4_t{lw[aa][0] * bqv[aa][0], lw[aa][1] * bqv[aa][1], lw[aa][2] * bqv[aa][2],
                                          lw[aa][3] * bqv[aa][3]};
                const uint2 wh = hi4(w);
                const bf16x8_t W = bf16x8_of(wh, lo4(w, wh));
                bf16x8_t Bd, Bx, B12, B3;
                if constexpr (!AGG) {
                    const float at = __shfl(agl, 16 * aa + col);
                    const float ah = at * Hs;
                    // the carry readout's coefficients in bf16 hi and lo halves: the modes'
                    // terms may cancel (fitted tables carry |c| up to ~30 for outputs ~0.1)
                    const f32x4_t cf = f32x4_t{ah * c0[aa][0], ah * c0[aa][1], ah * c0[aa][2], ah * c0[aa][3]};
                    const uint2 ch = hi4(cf);
                    Bd = bf16x8_of(
                        make_uint2(pk_bf16(at * bqv[aa][0] * psv[0][0], at * bqv[aa][1] * psv[0][1]),
                                   pk_bf16(at * bqv[aa][2] * psv[0][2], at * bqv[aa][3] * psv[0][3])),
                        ch);
                    Bx = bf16x8_of(lo4(cf, ch), ch);
                    if (aa >= 1) {
                        const int a1 = aa >= 1 ? aa - 1 : 0, a2 = aa >= 2 ? aa - 2 : 0;
                        const float s2 = aa >= 2 ? at : 0.f;
                        B12 = bf16x8_of(
                            make_uint2(pk_bf16(at * bqv[a1][0] * psv[1][0], at * bqv[a1][1] * psv[1][1]),
                                       pk_bf16(at * bqv[a1][2] * psv[1][2], at * bqv[a1][3] * psv[1][3])),
                            make_uint2(pk_bf16(s2 * bqv[a2][0] * psv[2][0], s2 * bqv[a2][1] * psv[2][1]),
                                       pk_bf16(s2 * bqv[a2][2] * psv[2][2], s2 * bqv[a2][3] * psv[2][3])));
                    }
                    if (aa >= 3)
                        B3 = bf16x8_of(make_uint2(pk_bf16(at * bqv[0][0] * psv[3][0], at * bqv[0][1] * psv[3][1]),
                                                  pk_bf16(at * bqv[0][2] * psv[3][2], at * bqv[0][3] * psv[3][3])),
                                       z2);
                }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const uint2 v0 = vfrag(sv, aa, nt);
                    mv[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(W, bf16x8_of(v0, v0), mv[nt], 0, 0, 0);
                    if constexpr (!AGG) {
                        f32x4_t acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(v0, hh[nt]), Bd, zf, 0, 0, 0);
                        // state hi x coefficient lo + state lo x coefficient hi
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(hh[nt], hl[nt]), Bx, acc, 0, 0, 0);
                        if (aa >= 1) {
                            const uint2 v1 = vfrag(sv, aa >= 1 ? aa - 1 : 0, nt);
                            const uint2 v2 = aa >= 2 ? vfrag(sv, aa >= 2 ? aa - 2 : 0, nt) : z2;
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(v1, v2), B12, acc, 0, 0, 0);
                        }
                        if (aa >= 3)
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(vfrag(sv, 0, nt), z2), B3, acc, 0, 0,
                                                                          0);
                        stage_y(sv, aa, nt, acc);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) lam[i] = Le * l64[i];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const float hr = st[nt][i], hi = st[nt][i + 1];
                    st[nt][i] = lam[i] * hr - lam[i + 1] * hi + Ae * mv[nt][i];
                    st[nt][i + 1] = lam[i + 1] * hr + lam[i] * hi + Ae * mv[nt][i + 1];
                }
            }
        } else {
            // ---- sub-block path (ragged block, or a clock span too large to factor) ----
            fc.bq[lane] = q2;
            fc.ag[lane] = gwv;
            fc.gr[lane] = grv;
            lam[0] = 1.f;
            lam[1] = 0.f;
            lam[2] = 1.f;
            lam[3] = 0.f;
            for (int T = 0; T * 16 < n; ++T) {
                const int T0 = 16 * T, T1 = min(T0 + 15, n - 1);
                const float qp = T0 > 0 ? fc.bq[T0 - 1] : 0.f;
                const float qe = fc.bq[T1];
                uint2 vf[4];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) vf[nt] = vfrag(sv, T, nt);
                if constexpr (!AGG) {
                    // G[s][t] = g_r(t) e^{-(q(t)-q(s))} g_w(s) psi(t-s), s <= t;
                    // C[row][t] = g_r(t) e^{-(q(t)-q(T0-1))} {Re,-Im}(c_j lambda_j^{t-T0+1})
                    const int t = T0 + col;
                    const float qt = fc.bq[t], grt = fc.gr[t];
                    float gv[4], av[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int sl = 4 * g + e, s2 = T0 + sl;
                        gv[e] = (sl <= col && s2 <= T1) ? exp2f(fc.bq[s2] - qt) * fc.ag[s2] * grt * tb.psi[col - sl]
                                                        : 0.f;
                    }
                    const float ea = exp2f(qp - qt) * grt;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 4 * g + i, j = row >> 1;
                        const float2 cp = tb.cpw[col + 1][j < M ? j : 0];
                        av[i] = j < M ? ea * ((row & 1) ? -cp.y : cp.x) : 0.f;
                    }
                    const f32x4_t af = f32x4_t{av[0], av[1], av[2], av[3]};
                    const uint2 ah4 = hi4(af);
                    const bf16x8_t Bo = bf16x8_of(make_uint2(pk_bf16(gv[0], gv[1]), pk_bf16(gv[2], gv[3])), ah4);
                    const bf16x8_t Box = bf16x8_of(lo4(af, ah4), ah4);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        const uint2 hh = hi4(st[nt]);
                        f32x4_t acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(vf[nt], hh), Bo, zf, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16x8_of(hh, lo4(st[nt], hh)), Box, acc, 0, 0,
                                                                      0);
                        stage_y(sv, T, nt, acc);
                    }
                }
                // W[row][s] = {Re,Im}(lambda_j^{T1-s}) e^{-(q(T1)-q(s))} g_w(s), hi and lo
                f32x4_t wv;
                {
                    const int jr = col >> 1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s2 = T0 + 4 * g + e;
                        float val = 0.f;
                        if (jr < M && s2 <= T1) {
                            const float2 pw = tb.pw[T1 - s2][jr < M ? jr : 0];
                            val = ((col & 1) ? pw.y : pw.x) * exp2f(fc.bq[s2] - qe) * fc.ag[s2];
                        }
                        wv[e] = val;
                    }
                }
                const uint2 wh = hi4(wv);
                const bf16x8_t W = bf16x8_of(wh, lo4(wv, wh));
                const float at = exp2f(qp - qe);
                float ls[4];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int j = 2 * g + hh;
                    const float2 pn = j < M ? tb.pw[T1 - T0 + 1][j < M ? j : 0] : make_float2(0.f, 0.f);
                    ls[2 * hh] = at * pn.x;
                    ls[2 * hh + 1] = at * pn.y;
                }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    f32x4_t dd;
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        const float hr = st[nt][i], hi = st[nt][i + 1];
                        dd[i] = ls[i] * hr - ls[i + 1] * hi;
                        dd[i + 1] = ls[i + 1] * hr + ls[i] * hi;
                    }
                    st[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(W, bf16x8_of(vf[nt], vf[nt]), dd, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const float ar = lam[i], ai = lam[i + 1];
                    lam[i] = ar * ls[i] - ai * ls[i + 1];
                    lam[i + 1] = ar * ls[i + 1] + ai * ls[i];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            const float ar = tr[i], ai = tr[i + 1];
            tr[i] = ar * lam[i] - ai * lam[i + 1];
            tr[i + 1] = ar * lam[i + 1] + ai * lam[i];
        }
    };

    // ---- the ring: block blk waits for its copies (issued NS-1 blocks ahead), then the y of
    // block blk-1 is stored and the copies of block blk+NS-1 go into blk-1's stage.  In the
    // aggregate role only loads are in flight and they complete in issue order; the operations
    // issued after block blk's copies are those of blocks blk+1 .. blk+NS-2, so waiting until
    // at most WCPY (NS-2) are outstanding covers block blk.  The streaming role (NS = 2) waits
    // for everything.
    for (int base = 0; base < nblk; base += NS) {
        static_for<0, NS>([&](auto ic) __attribute__((always_inline)) {
            constexpr int s = decltype(ic)::value;
            constexpr int sp = (s + NS - 1) % NS;   // stage of block blk-1 and of block blk+NS-1
            const int blk = base + s;
            if (blk < nblk) {
                wait_vmem_at_most<WCPY * (NS - 2)>();
                if constexpr (!AGG) {
                    if (blk >= 1) store_y(stv(sp), blk - 1);
                }
                // The copies below overwrite stage sp, which the LDS reads just above (the y
                // rows of block blk-1) and those of the block before still read.  The compiler
                // takes an asynchronous copy to write only its base address, so it may move
                // the copies above those reads; a copy that then lands first puts v rows
                // into y.  The reads are completed and the order is pinned here.
                stage_reads_done();
                copy_block(sp, blk + NS - 1);
                compute_block(stv(s), stc(s), blk);
            }
        });
    }
    if constexpr (!AGG) store_y(stv((nblk - 1) % NS), nblk - 1);
    __builtin_amdgcn_s_waitcnt(WAIT_VMEM0);   // no copy into this workgroup's LDS outlives it

    if constexpr (AGG) {
        // segment aggregate (end state from a zero entering state, or from state_in for
        // segment 0) and transfer; segment 0 also records its entering state
        float* dst = plan.agg + (slot + seg) * (size_t)ROWS * WP;
        float* ent = plan.incl + slot * (size_t)ROWS * WP;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int p = nt * 16 + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                if (row < ROWS) {
                    dst[(size_t)row * WP + p] = st[nt][i];
                    if (seg == 0) ent[(size_t)row * WP + p] = st_in[nt][i];
                }
            }
        }
        if (col == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                if (row < ROWS) plan.lam[(slot + seg) * ROWS + row] = tr[i];
            }
        }
    } else if (seg + 1 >= nseg && a.state_out) {
        const size_t base = ((size_t)b * K + k) * M;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int p = nt * 16 + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i, j = row >> 1, cmp = row & 1;
                if (j < M) a.state_out[((base + j) * 2 + cmp) * WP + p] = st[nt][i];
            }
        }
    }
}

// The aggregate role, which stores nothing until its end, can also run a deeper ring (the
// waits above allow it); with three or four stages its LDS halves the waves per CU, and it
// measured 13-15% slower.
#ifndef ESSH_WAVE_STAGES_AGG
#define ESSH_WAVE_STAGES_AGG 2
#endif
constexpr int WNS = 2;
constexpr int WNS_AGG = ESSH_WAVE_STAGES_AGG;

template <int M>
hipError_t launch_wave_m(const PrefillArgs& a, const ScanPlan& plan, hipStream_t s) {
    if (plan.nblocks == 0) return hipSuccess;
    if (!plan.cdl || !plan.cgg) return hipErrorInvalidValue;
    const dim3 pgrid((unsigned)((a.L + WBLK - 1) / WBLK), (unsigned)((a.K_T + 31) / 32), (unsigned)a.B);
    hipLaunchKernelGGL(pack_ctrl_kernel, pgrid, dim3(256), 0, s, a, plan);
    if (plan.mode == SCAN_SPLIT && plan.nseg > 1) {
        const int nagg = plan.nseq * (plan.nseg - 1);   // every segment but the last
        hipLaunchKernelGGL((wave_prefill_kernel<M, WNS_AGG, MODE_AGG>), dim3((unsigned)nagg), dim3(64), 0, s, a, plan);
        const hipError_t e = launch_seg_scan(plan, M, WP, s);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((wave_prefill_kernel<M, WNS, MODE_STREAM>), dim3((unsigned)plan.nblocks), dim3(64), 0, s, a,
                       plan);
    return hipGetLastError();
}

}  // namespace

bool wave_supported(int m, int P, int Lc, int io_dtype, int per_mode) {
    return P == WP && (m == 1 || m == 2 || m == 4 || m == 8) && (Lc == 64 || Lc == 128) && io_dtype == ESSH_BF16 &&
           !per_mode;
}

hipError_t launch_prefill_wave(const PrefillArgs& a, int m, const ScanPlan& plan, hipStream_t s) {
    switch (m) {
        case 1: return launch_wave_m<1>(a, plan, s);
        case 2: return launch_wave_m<2>(a, plan, s);
        case 4: return launch_wave_m<4>(a, plan, s);
        case 8: return launch_wave_m<8>(a, plan, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace essh
