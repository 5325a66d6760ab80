// prefill_chunk.hip -- chunked parallel scan of the ESSH selective mixer on MFMA.
//
// ESSH paper, Sec. 4.3 "Chunked parallel training" and Fig. 2A: positions are
// split into chunks of Lc; inside a chunk the source-to-target contributions
// are a dense causal matrix G_k applied by matrix multiplication, and only the
// 2 m P mode-state entries of a channel cross a chunk boundary.  Eq. 6 (the
// transition product rho^{t-s} e^{-sum delta} R(theta (t-s))) makes this
// exact.  For a chunk [t0, t0+n) and chunk-local inclusive clock sums
// qh(r) = sum_{l<=r} delta(t0+l), with lambda_j = rho_j e^{i theta_j}:
//
//   y(r)   = g_r(r) [ sum_{s<=r} e^{-(qh(r)-qh(s))} g_w(s) psi(r-s) v(s)        (intra, G V)
//                   + e^{-qh(r)} sum_j Re(c_j lambda_j^{r+1} h_j) ]             (carry,  A H)
//   h_j'   = lambda_j^n e^{-qh(n-1)} h_j
//            + sum_s lambda_j^{n-1-s} e^{-(qh(n-1)-qh(s))} g_w(s) v(s)          (end state, W V)
//
// with psi(tau) = sum_j Re(c_j lambda_j^tau).  Channels are independent
// (Sec. 4.1), so a workgroup owns one (batch row, channel) and walks the
// chunks of a segment of positions in order, keeping the channel's mode state
// in registers.
//
// Segmented scan.  When batch rows x retained channels alone cannot fill the
// GPU, each sequence of chunks is cut into segments handled by different
// workgroups.  The state entering a segment is the composition of the affine
// chunk maps h -> Lambda h + S before it (the same Eq. 6 algebra one level
// up).  A workgroup (i) sweeps its segment once computing only the end state
// reached from a zero state (its aggregate S_seg and transfer Lambda_seg),
// (ii) publishes it, (iii) obtains its entering state by a decoupled
// look-back over its predecessors' published aggregates / inclusive states,
// publishes its own inclusive state, and (iv) sweeps the segment again with
// the true entering state, now producing y.  The second sweep re-reads v,
// which the first sweep has just brought into the caches.
//
// gfx950 mapping
//   * Each wave owns 16*NTW value columns for all positions: its share of the
//     state lives in VGPRs in the 16x16 MFMA accumulator layout (lane (g,col)
//     holds state rows 4g..4g+3 = (mode 2g, re/im), (mode 2g+1, re/im) of
//     column col).
//   * All three products use v_mfma_f32_16x16x32_bf16.  The intra-chunk
//     product is computed transposed, Y^T = V^T G^T, so that the V fragment
//     a lane holds (8 consecutive positions of one value column) is the A
//     operand of Y^T and the B operand of the end-state product W V.  The
//     carry product packs (state row, hi/lo half) into its K axis.  Every
//     product of one accumulation chain has the same MFMA shape.
//   * G and the carry matrix A are rounded once to bf16 (the output is bf16);
//     W, which feeds the fp32 state, is split into bf16 hi + lo, and so is
//     the state in the carry product, so the state path keeps ~16 bits.
//   * v is streamed with 16-byte loads one chunk ahead of the arithmetic and
//     written to LDS transposed ([t/8][column][8]) with a bank swizzle; y is
//     staged through the same LDS region and written with 16-byte stores.
//   * Clocks, gates and pole tables are staged in LDS; G, W, A are built
//     cooperatively once per chunk and read by every wave.
//   * Look-back messages are written and read with agent-scope atomic
//     accesses (they bypass the per-XCD L2), flags carry a per-launch epoch,
//     and every wait is bounded.
#include "essh_internal.h"

namespace essh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float LOG2E = 1.4426950408889634f;

// Look-back flag kinds (low two bits of a flag word; the rest is the epoch tag).
constexpr unsigned FLAG_AGG = 1u;    // aggregate (end state from a zero entering state) and transfer
constexpr unsigned FLAG_INCL = 2u;   // inclusive state (true state after the segment)
// Upper bound on polls of one flag (each poll is a memory round trip plus a
// short sleep, so this is tens of milliseconds); exceeding it records
// SCAN_ERR_TIMEOUT in the workspace header instead of waiting forever.
constexpr int SPIN_LIMIT = 1 << 16;

template <int P_, int M_, int LC_>
struct Cfg {
    static constexpr int P = P_, M = M_, LC = LC_;
    static constexpr int NT = P / 16;               // 16-column value tiles
    static constexpr int NW = NT < 4 ? NT : 4;      // waves per workgroup
    static constexpr int NTW = NT / NW;             // value tiles per wave
    static constexpr int THREADS = 64 * NW;
    static constexpr int WCOLS = 16 * NTW;          // value columns per wave
    static constexpr int MT = LC / 16;              // 16-position tiles
    static constexpr int KS = LC / 32;              // 32-deep k steps
    static constexpr int UNITS = LC / 8;            // 16-byte units per G/W row
    static constexpr int GSWZ = (UNITS < 8 ? UNITS : 8) - 1;
    static constexpr int LPR = WCOLS / 8;           // lanes per v row (16 B each)
    static constexpr int RPI = 64 / LPR;            // v rows per wave load
    static constexpr int NLD = LC / RPI;            // wave loads per chunk
    static constexpr int QU = WCOLS / 4;            // 8-byte units per staged y row
    static constexpr int YROWS128 = 64 / WCOLS;     // staged y rows per 128 bytes
    static constexpr int CPL = (LC + 63) / 64;     // control positions per lane of wave 0
    static_assert(P % 16 == 0 && NT % NW == 0, "P must be 16, 32, 64 or 128");
    static_assert(LC % 32 == 0 && LC <= 128, "chunk length must be 32, 64 or 128");
    static_assert(M >= 1 && M <= 8, "1..8 modes");
    static_assert(LC % RPI == 0, "v tile loads must tile the chunk");
};

template <class C>
struct __align__(16) Smem {
    float q2[C::LC];                 // chunk-local inclusive clock sum * log2(e)
    float eq[C::LC];                 // exp(-chunk-local inclusive clock sum)
    float gw[C::LC];                 // write gate
    float gr[C::LC];                 // read gate
    float psi[C::LC];                // sum_j Re(c_j lambda_j^tau)
    float2 pw[C::LC + 1][C::M];      // lambda_j^tau
    float2 cpw[C::LC + 1][C::M];     // c_j lambda_j^tau
    alignas(16) uint16_t G[C::LC * C::LC];        // bf16, row t, swizzled 16-byte units over s
    alignas(16) uint16_t Whi[16 * C::LC];         // bf16, row (j,re/im), swizzled units over s
    alignas(16) uint16_t Wlo[16 * C::LC];
    alignas(16) uint16_t A[C::LC * 16];           // bf16, row t, 8-byte units over (j,re/im)
    alignas(16) uint16_t V[C::NW][C::LC * C::WCOLS];   // per wave: v^T tile, then y staging
    int ticket;
    unsigned epoch;
    unsigned flag;
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

template <class C, bool SEG>
__global__ void __launch_bounds__(C::THREADS)
prefill_chunk_kernel(PrefillArgs a, ScanPlan plan) {
    constexpr int LC = C::LC, M = C::M, P = C::P, WCOLS = C::WCOLS, NTW = C::NTW;
    constexpr int ROWS = 2 * M;          // state rows (mode, re/im) per value column
    __shared__ Smem<C> sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int col = lane & 15;

    // ---- work item ------------------------------------------------------------------
    int seq, seg;
    unsigned tag = 0;
    if (SEG) {
        // Tickets are taken in the order workgroups start, so every predecessor
        // of a segment (a smaller ticket) is already running or finished.
        // Eight ticket counters, one per residue of blockIdx mod 8 (the XCD the
        // hardware's round-robin dispatch sends the workgroup to), so that no
        // single address takes every workgroup's atomic.  Counter x hands out
        // the work items x, x + 8, x + 16, ... in start order.
        const int xq = (int)(blockIdx.x & 7u);
        if (tid == 0) {
            const unsigned t = __hip_atomic_fetch_add(&plan.hdr[SCAN_HDR_TICKET0 + SCAN_HDR_STRIDE * xq], 1u,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sm.ticket = (int)(t * 8u + (unsigned)xq);
            sm.epoch = ld_agent_u(&plan.hdr[SCAN_HDR_EPOCH]);
        }
        __syncthreads();
        const int ticket = sm.ticket;
        tag = ((sm.epoch + 1u) & 0x3FFFFFFFu) << 2;
        if (ticket >= plan.nblocks) {
            // Only possible with a workspace that was not zero-filled before first use.
            if (tid == 0) __hip_atomic_fetch_or(&plan.hdr[SCAN_HDR_ERROR], SCAN_ERR_TICKET, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        seg = ticket / plan.nseq;
        seq = ticket - seg * plan.nseq;
    } else {
        seq = remap_xcd(blockIdx.x, gridDim.x);
        seg = 0;
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

    // ---- pole tables: lambda^tau and c lambda^tau for tau = 0..LC ----------
    for (int idx = tid; idx < (LC + 1) * M; idx += C::THREADS) {
        const int tau = idx / M, j = idx - tau * M;
        const float r = a.rho[k * M + j];
        const float th = a.theta[k * M + j];
        const float mag = tau == 0 ? 1.f : exp2f((float)tau * log2f(r));
        // theta*tau reaches ~400 rad: form and reduce the angle in fp64.
        double ang = (double)th * (double)tau;
        ang -= 6.283185307179586476925 * rint(ang * 0.15915494309189533577);
        float sn, cs;
        sincosf((float)ang, &sn, &cs);
        const float pr = mag * cs, pi = mag * sn;
        sm.pw[tau][j] = make_float2(pr, pi);
        const float cr = a.c[(k * M + j) * 2], ci = a.c[(k * M + j) * 2 + 1];
        sm.cpw[tau][j] = make_float2(cr * pr - ci * pi, cr * pi + ci * pr);
    }
    __syncthreads();
    for (int tau = tid; tau < LC; tau += C::THREADS) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < M; ++j) s += sm.cpw[tau][j].x;
        sm.psi[tau] = s;
    }

    // ---- state in the accumulator layout ---------------------------------------------
    // st_in: state entering position 0 (segment 0 only), read once up front so that
    // an aliasing state_out written by the last segment cannot race with it.
    f32x4_t st_in[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int p = wave * WCOLS + nt * 16 + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * g + i, j = row >> 1, cmp = row & 1;
            float x = 0.f;
            if (seg == 0 && a.state_in && j < M) x = a.state_in[((((size_t)b * K + k) * M + j) * 2 + cmp) * P + p];
            st_in[nt][i] = x;
        }
    }

    // ---- chunk pipeline helpers ---------------------------------------------------------
    const int vrow_l = lane / C::LPR;          // row of this lane inside a wave load
    const int vunit = lane % C::LPR;           // 16-byte unit of this lane inside a row
    const size_t vcol0 = (size_t)wave * WCOLS + vunit * 8;
    uint16_t* Vw = sm.V[wave];

    uint4 vreg[C::NLD];
    float cd[C::CPL], cw[C::CPL], cr_[C::CPL];   // controls of the loaded chunk (wave 0 only)

    auto load_chunk = [&](int c) {
        const int t0 = c * LC;
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            const int t = t0 + i * C::RPI + vrow_l;
            if (t < L) {
                const size_t off = (((size_t)b * L + t) * K + k) * P + vcol0;
                vreg[i] = *reinterpret_cast<const uint4*>(vg + off);
            } else {
                vreg[i] = make_uint4(0, 0, 0, 0);
            }
        }
        if (wave == 0) {
#pragma unroll
            for (int u = 0; u < C::CPL; ++u) {
                const int r = lane * C::CPL + u;
                const int t = t0 + r;
                if (r < LC && t < L) {
                    const size_t row = ((size_t)b * L + t) * K + k;
                    cd[u] = a.delta[row];
                    cw[u] = bf16_to_f32(gwg[row]);
                    cr_[u] = bf16_to_f32(grg[row]);
                } else {
                    cd[u] = 0.f;
                    cw[u] = 0.f;
                    cr_[u] = 0.f;
                }
            }
        }
    };

    // v tile and controls of the loaded chunk -> LDS, the chunk-local clock sums
    // (wave 0 scans the controls it holds), then the loads of chunk `next`
    // (if >= 0) are issued so that they overlap this chunk's arithmetic.
    // v element (t, p') goes to ((t/8)*WCOLS + p'')*8 + t%8, where p'' permutes the
    // low 3 bits of p' by a key of (t/8, p'/8) so a wave's 2-byte stores spread over
    // all banks.  Ends with the shared tiles complete (barrier).
    auto stage_chunk = [&](int next) {
        __syncthreads();   // previous readers of the shared tiles are done
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            const int tr = i * C::RPI + vrow_l;
            const int blk = tr >> 3, tt = tr & 7;
            const uint32_t w4[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int pp = vunit * 8 + e;
                const int key = (blk * (WCOLS / 8) + (pp >> 3)) & 7;
                const int pph = (pp & ~7) | ((pp & 7) ^ key);
                const uint16_t val = (uint16_t)(w4[e >> 1] >> ((e & 1) * 16));
                Vw[(blk * WCOLS + pph) * 8 + tt] = val;
            }
        }
        if (wave == 0) {
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
                    const float q = excl + loc[u];
                    sm.q2[idx] = q * LOG2E;
                    sm.eq[idx] = expf(-q);
                    sm.gw[idx] = cw[u];
                    sm.gr[idx] = cr_[u];
                }
            }
        }
        if (next >= 0) load_chunk(next);
        __syncthreads();
    };

    // W[(j,re/im)][s] = {Re,Im}(lambda_j^{n-1-s}) e^{-(qh(n-1)-qh(s))} g_w(s), hi + lo bf16.
    auto build_W = [&](int n) {
        const float qe = sm.q2[n - 1];
        for (int idx = tid; idx < 16 * C::UNITS; idx += C::THREADS) {
            const int row = idx / C::UNITS, u = idx - row * C::UNITS;
            const int j = row >> 1, cmp = row & 1;
            uint16_t hh[8], hl[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = u * 8 + e;
                float val = 0.f;
                if (j < M && s < n) {
                    const float2 pw = sm.pw[n - 1 - s][j < M ? j : 0];
                    val = (cmp ? pw.y : pw.x) * exp2f(sm.q2[s] - qe) * sm.gw[s];
                }
                const uint16_t hb = f32_to_bf16(val);
                hh[e] = hb;
                hl[e] = f32_to_bf16(val - bf16_to_f32(hb));
            }
            const int off = row * LC + ((u ^ (row & C::GSWZ)) * 8);
            *reinterpret_cast<uint4*>(&sm.Whi[off]) =
                make_uint4(pack2(hh[0], hh[1]), pack2(hh[2], hh[3]), pack2(hh[4], hh[5]), pack2(hh[6], hh[7]));
            *reinterpret_cast<uint4*>(&sm.Wlo[off]) =
                make_uint4(pack2(hl[0], hl[1]), pack2(hl[2], hl[3]), pack2(hl[4], hl[5]), pack2(hl[6], hl[7]));
        }
    };

    // G[t][s] = e^{-(qh(t)-qh(s))} g_w(s) psi(t-s) for s <= t, bf16.  Only the
    // 32-wide k blocks the MFMA loop reads are built.
    auto build_G = [&]() {
        for (int idx = tid; idx < LC * C::UNITS; idx += C::THREADS) {
            const int r = idx / C::UNITS, u = idx - r * C::UNITS;
            const int nks = ((r & ~15) + 15) / 32 + 1;
            if (u >= 4 * nks) continue;
            const float qr = sm.q2[r];
            uint16_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = u * 8 + e;
                float val = 0.f;
                if (s <= r) val = exp2f(sm.q2[s] - qr) * sm.gw[s] * sm.psi[r - s];
                h[e] = f32_to_bf16(val);
            }
            uint4 pk = make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
            *reinterpret_cast<uint4*>(&sm.G[r * LC + ((u ^ (r & C::GSWZ)) * 8)]) = pk;
        }
    };

    // A[t][(j,re/im)] = e^{-qh(t)} {Re, -Im}(c_j lambda_j^{t+1}), bf16, 8-byte units swizzled by t.
    auto build_A = [&]() {
        for (int idx = tid; idx < LC * 4; idx += C::THREADS) {
            const int r = idx >> 2, q = idx & 3;
            const float e = sm.eq[r];
            uint16_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = 4 * q + i, j = kk >> 1, cmp = kk & 1;
                float val = 0.f;
                if (j < M) {
                    const float2 cp = sm.cpw[r + 1][j < M ? j : 0];
                    val = e * (cmp ? -cp.y : cp.x);
                }
                h[i] = f32_to_bf16(val);
            }
            *reinterpret_cast<uint2*>(&sm.A[r * 16 + ((q ^ ((r >> 2) & 3)) * 4)]) =
                make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]));
        }
    };

    // v fragments: lane (g, col) holds v(s = 32ks + 8g .. +7, p = 16nt + col)
    auto load_vf = [&](bf16x8_t (&vf)[C::KS][NTW]) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const int blk = 4 * ks + g;
                const int pp = nt * 16 + col;
                const int key = (blk * (WCOLS / 8) + (pp >> 3)) & 7;
                const int pph = (pp & ~7) | ((pp & 7) ^ key);
                vf[ks][nt] = *reinterpret_cast<const bf16x8_t*>(&Vw[(blk * WCOLS + pph) * 8]);
            }
        }
    };

    // h <- Lambda h + W_hi V + W_lo V, with Lambda_j = lambda_j^n e^{-qh(n-1)}.
    // Also folds Lambda into the running segment transfer (tr: modes 2g, 2g+1).
    auto state_update = [&](f32x4_t (&st)[NTW], const bf16x8_t (&vf)[C::KS][NTW], int n, float (&tr)[4]) {
        float lam[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int j = 2 * g + h;
            float lr = 0.f, li = 0.f;
            if (j < M) {
                const float2 pw = sm.pw[n][j < M ? j : 0];
                const float e = sm.eq[n - 1];
                lr = pw.x * e;
                li = pw.y * e;
            }
            lam[2 * h] = lr;
            lam[2 * h + 1] = li;
            const float ar = tr[2 * h], ai = tr[2 * h + 1];
            tr[2 * h] = ar * lr - ai * li;
            tr[2 * h + 1] = ar * li + ai * lr;
        }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            f32x4_t d;
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float lr = lam[i], li = lam[i + 1];
                const float hr = st[nt][i], hi = st[nt][i + 1];
                d[i] = lr * hr - li * hi;
                d[i + 1] = li * hr + lr * hi;
            }
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const int off = col * LC + (((4 * ks + g) ^ (col & C::GSWZ)) * 8);
                const bf16x8_t wh = *reinterpret_cast<const bf16x8_t*>(&sm.Whi[off]);
                const bf16x8_t wl = *reinterpret_cast<const bf16x8_t*>(&sm.Wlo[off]);
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, vf[ks][nt], d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wl, vf[ks][nt], d, 0, 0, 0);
            }
            st[nt] = d;
        }
    };

    // y^T tiles: carry term then the intra-chunk product; staged into Vw (bf16).
    auto output = [&](const f32x4_t (&st)[NTW], const bf16x8_t (&vf)[C::KS][NTW]) {
        // State fragments as the A operand of the carry product.  The K axis
        // holds (state row, hi/lo half) pairs: lane (g, col) supplies the bf16
        // hi parts of its state rows 4g..4g+3 in elements 0..3 and the lo parts
        // in elements 4..7; the B operand repeats the matching carry-matrix
        // entries in both halves.
        bf16x8_t sf[NTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            u16x8_t raw;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = st[nt][i];
                const uint16_t hb = f32_to_bf16(x);
                raw[i] = hb;
                raw[4 + i] = f32_to_bf16(x - bf16_to_f32(hb));
            }
            sf[nt] = __builtin_bit_cast(bf16x8_t, raw);
        }
        constexpr int qu = C::QU;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
            const int tr = mt * 16 + col;          // position (row of G, A) owned by this lane
            const u16x4_t a4 = *reinterpret_cast<const u16x4_t*>(&sm.A[tr * 16 + ((g ^ ((tr >> 2) & 3)) * 4)]);
            const bf16x8_t af =
                __builtin_bit_cast(bf16x8_t, u16x8_t{a4[0], a4[1], a4[2], a4[3], a4[0], a4[1], a4[2], a4[3]});
            f32x4_t acc[NTW];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[nt], af, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            const int nks = mt / 2 + 1;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                if (ks < nks) {
                    const bf16x8_t gf = *reinterpret_cast<const bf16x8_t*>(
                        &sm.G[tr * LC + (((4 * ks + g) ^ (tr & C::GSWZ)) * 8)]);
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt)
                        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[ks][nt], gf, acc[nt], 0, 0, 0);
                }
            }
            // lane holds y(t = tr, p = 16nt + 4g + i), i = 0..3
            const float grv = sm.gr[tr];
            const int yswz = (tr / C::YROWS128) & (qu - 1);
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const uint16_t h0 = f32_to_bf16(acc[nt][0] * grv);
                const uint16_t h1 = f32_to_bf16(acc[nt][1] * grv);
                const uint16_t h2 = f32_to_bf16(acc[nt][2] * grv);
                const uint16_t h3 = f32_to_bf16(acc[nt][3] * grv);
                const int q = (nt * 4 + g) ^ yswz;
                *reinterpret_cast<uint2*>(&Vw[tr * WCOLS + q * 4]) = make_uint2(pack2(h0, h1), pack2(h2, h3));
            }
        }
    };

    // staged y -> global, 16 bytes per lane (undo the 8-byte unit swizzle)
    auto store_y = [&](int t0, int n) {
        constexpr int qu = C::QU;
#pragma unroll
        for (int i = 0; i < C::NLD; ++i) {
            const int tr = i * C::RPI + vrow_l;
            const int t = t0 + tr;
            const int yswz = (tr / C::YROWS128) & (qu - 1);
            const int q0 = (2 * vunit) ^ yswz;          // physical 8-byte unit of the first half
            const uint4 raw = *reinterpret_cast<const uint4*>(&Vw[tr * WCOLS + (q0 & ~1) * 4]);
            uint4 outv = raw;
            if (q0 & 1) outv = make_uint4(raw.z, raw.w, raw.x, raw.y);
            if (tr < n) {
                const size_t off = (((size_t)b * L + t) * K + k) * P + vcol0;
                *reinterpret_cast<uint4*>(yg + off) = outv;
            }
        }
    };

    // Look-back message rows: rows (j, re/im) of this lane's value columns.
    auto publish = [&](float* dst, const f32x4_t (&s)[NTW], unsigned kind, const float (&trn)[4]) {
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
    // until an inclusive state is found (segment 0 always publishes one).
    auto lookback = [&](f32x4_t (&e)[NTW]) {
        float cf[4] = {1.f, 0.f, 1.f, 0.f};   // accumulated transfer of modes 2g, 2g+1
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) e[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int pred = seg - 1; pred >= 0; --pred) {
            if (tid == 0) {
                unsigned f = 0;
                int it = 0;
                for (; it < SPIN_LIMIT; ++it) {
                    f = ld_agent_u(&plan.flags[slot + pred]);
                    if ((f & ~3u) == tag && (f & 3u) != 0) break;
                    __builtin_amdgcn_s_sleep(2);
                }
                if (it == SPIN_LIMIT) {
                    __hip_atomic_fetch_or(&plan.hdr[SCAN_HDR_ERROR], SCAN_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                    f = tag | FLAG_INCL;   // give up: treat the (unwritten) state as final
                }
                sm.flag = f;
            }
            __syncthreads();
            const unsigned f = sm.flag;
            __syncthreads();   // sm.flag may be rewritten by the next poll
            const bool incl = (f & 3u) == FLAG_INCL;
            const float* src = (incl ? plan.incl : plan.agg) + (slot + pred) * (size_t)ROWS * P;
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const int p = wave * WCOLS + nt * 16 + col;
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const int row = 4 * g + i;
                    if (row < ROWS) {
                        const float sr = ld_agent(&src[(size_t)row * P + p]);
                        const float si = ld_agent(&src[(size_t)(row + 1) * P + p]);
                        e[nt][i] += cf[i] * sr - cf[i + 1] * si;
                        e[nt][i + 1] += cf[i] * si + cf[i + 1] * sr;
                    }
                }
            }
            if (incl) break;
            // compose with the predecessor's transfer: cf <- cf * Lambda_pred
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const int row = 4 * g + i;
                float lr = 0.f, li = 0.f;
                if (row < ROWS) {
                    lr = ld_agent(&plan.lam[(slot + pred) * ROWS + row]);
                    li = ld_agent(&plan.lam[(slot + pred) * ROWS + row + 1]);
                }
                const float ar = cf[i], ai = cf[i + 1];
                cf[i] = ar * lr - ai * li;
                cf[i + 1] = ar * li + ai * lr;
            }
        }
    };

    // ---- sweep 1 (segmented scan only): aggregate of this segment ----------------------
    f32x4_t st[NTW];
    const bool has_succ = SEG && seg + 1 < nseg;
    if (c_begin < c_end) load_chunk(c_begin);
    if (has_succ) {
        float tr[4] = {1.f, 0.f, 1.f, 0.f};
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) st[nt] = st_in[nt];   // segment 0: its inclusive state directly
        for (int c = c_begin; c < c_end; ++c) {
            const int n = min(LC, L - c * LC);
            // prefetch: next chunk of this sweep, else the first chunk of sweep 2
            stage_chunk(c + 1 < c_end ? c + 1 : c_begin);
            build_W(n);
            __syncthreads();
            bf16x8_t vf[C::KS][NTW];
            load_vf(vf);
            state_update(st, vf, n, tr);
        }
        if (seg == 0) {
            publish(plan.incl + (slot + seg) * (size_t)ROWS * P, st, FLAG_INCL, tr);
        } else {
            publish(plan.agg + (slot + seg) * (size_t)ROWS * P, st, FLAG_AGG, tr);
            f32x4_t e[NTW];
            lookback(e);
            // inclusive = Lambda_seg * entering + aggregate
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                f32x4_t inc;
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    inc[i] = tr[i] * e[nt][i] - tr[i + 1] * e[nt][i + 1] + st[nt][i];
                    inc[i + 1] = tr[i] * e[nt][i + 1] + tr[i + 1] * e[nt][i] + st[nt][i + 1];
                }
                st_in[nt] = e[nt];
                st[nt] = inc;
            }
            __syncthreads();
            publish(plan.incl + (slot + seg) * (size_t)ROWS * P, st, FLAG_INCL, tr);
        }
    } else if (SEG && seg > 0) {
        // last segment: no successor needs an aggregate; only the entering state
        f32x4_t e[NTW];
        lookback(e);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) st_in[nt] = e[nt];
    }

    // ---- sweep 2: outputs ------------------------------------------------------------------
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) st[nt] = st_in[nt];
    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * LC;
        const int n = min(LC, L - t0);
        stage_chunk(c + 1 < c_end ? c + 1 : -1);
        build_G();
        build_W(n);
        build_A();
        __syncthreads();
        bf16x8_t vf[C::KS][NTW];
        load_vf(vf);
        output(st, vf);
        float tr[4] = {1.f, 0.f, 1.f, 0.f};
        state_update(st, vf, n, tr);
        store_y(t0, n);
    }

    // ---- leaving state ----------------------------------------------------------------------
    if (seg + 1 >= nseg && a.state_out) {
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

    // ---- launch bookkeeping: the last workgroup to finish re-arms the workspace -----------
    if (SEG) {
        __syncthreads();
        if (tid == 0) {
            // per-counter completion first, then one count per finished counter
            const int xq = (int)(blockIdx.x & 7u);
            const unsigned cnt = (unsigned)((plan.nblocks - xq + 7) / 8);
            const unsigned done = __hip_atomic_fetch_add(&plan.hdr[SCAN_HDR_DONE0 + SCAN_HDR_STRIDE * xq], 1u,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (done + 1 == cnt) {
                const unsigned nq = (unsigned)(plan.nblocks < 8 ? plan.nblocks : 8);
                const unsigned xd = __hip_atomic_fetch_add(&plan.hdr[SCAN_HDR_XDONE], 1u, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                if (xd + 1 == nq) {   // every workgroup of this launch has finished: re-arm
                    for (int x = 0; x < 8; ++x) {
                        st_agent_u(&plan.hdr[SCAN_HDR_TICKET0 + SCAN_HDR_STRIDE * x], 0u);
                        st_agent_u(&plan.hdr[SCAN_HDR_DONE0 + SCAN_HDR_STRIDE * x], 0u);
                    }
                    st_agent_u(&plan.hdr[SCAN_HDR_XDONE], 0u);
                    st_agent_u(&plan.hdr[SCAN_HDR_EPOCH], sm.epoch + 1u);
                }
            }
        }
    }
}

template <int P, int M, int LC>
hipError_t launch_cfg(const PrefillArgs& a, const ScanPlan& plan, hipStream_t s) {
    using C = Cfg<P, M, LC>;
    if (plan.nblocks == 0) return hipSuccess;
    if (plan.nseg > 1)
        hipLaunchKernelGGL((prefill_chunk_kernel<C, true>), dim3((unsigned)plan.nblocks), dim3(C::THREADS), 0, s, a,
                           plan);
    else
        hipLaunchKernelGGL((prefill_chunk_kernel<C, false>), dim3((unsigned)plan.nblocks), dim3(C::THREADS), 0, s, a,
                           plan);
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
    return mok && pok && lok && io_dtype == ESSH_BF16 && !per_mode;
}

ScanPlan plan_chunked(int B, int L, int K_T, int m, int P, int Lc) {
    ScanPlan p{};
    p.nseq = B * K_T;
    p.nchunks = (L + Lc - 1) / Lc;
    if (p.nseq == 0 || p.nchunks == 0) return p;
    // Enough workgroups to fill 256 CUs several times over: sequences alone when
    // there are plenty of them, otherwise segments of at least two chunks.
    constexpr int TARGET_BLOCKS = 2048;
    int seg_chunks = p.nchunks;
    if (p.nseq < TARGET_BLOCKS) {
        const int want_seg = (TARGET_BLOCKS + p.nseq - 1) / p.nseq;
        seg_chunks = (p.nchunks + want_seg - 1) / want_seg;
        if (seg_chunks < 2) seg_chunks = 2;
        if (seg_chunks > p.nchunks) seg_chunks = p.nchunks;
    }
    p.seg_chunks = seg_chunks;
    p.nseg = (p.nchunks + seg_chunks - 1) / seg_chunks;
    p.nblocks = p.nseq * p.nseg;
    (void)P;
    (void)m;
    return p;
}

size_t chunked_workspace_bytes(int B, int L, int K_T, int m, int P, int Lc) {
    const ScanPlan p = plan_chunked(B, L, K_T, m, P, Lc);
    if (p.nseg <= 1) return 0;
    const size_t slots = (size_t)p.nseq * p.nseg;
    return align256(SCAN_HDR_WORDS * sizeof(unsigned)) + align256(slots * sizeof(unsigned)) +
           align256(slots * 2 * m * sizeof(float)) + 2 * align256(slots * 2 * (size_t)m * P * sizeof(float));
}

void bind_workspace(ScanPlan& p, void* ws, int m, int P) {
    if (p.nseg <= 1) return;
    const size_t slots = (size_t)p.nseq * p.nseg;
    char* base = static_cast<char*>(ws);
    p.hdr = reinterpret_cast<unsigned*>(base);
    base += align256(SCAN_HDR_WORDS * sizeof(unsigned));
    p.flags = reinterpret_cast<unsigned*>(base);
    base += align256(slots * sizeof(unsigned));
    p.lam = reinterpret_cast<float*>(base);
    base += align256(slots * 2 * m * sizeof(float));
    p.agg = reinterpret_cast<float*>(base);
    base += align256(slots * 2 * (size_t)m * P * sizeof(float));
    p.incl = reinterpret_cast<float*>(base);
}

hipError_t launch_prefill_chunked(const PrefillArgs& a, int m, int P, const ScanPlan& plan, hipStream_t s) {
    switch (P) {
        case 16: return launch_m<16>(a, m, plan, s);
        case 32: return launch_m<32>(a, m, plan, s);
        case 64: return launch_m<64>(a, m, plan, s);
        case 128: return launch_m<128>(a, m, plan, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace essh
