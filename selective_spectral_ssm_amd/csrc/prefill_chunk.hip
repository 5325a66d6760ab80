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
// (Sec. 4.1, "the channels remain independent"), so a workgroup owns one
// (batch row, channel) and walks the chunks of a segment in order, keeping
// the channel's mode state in registers.
//
// gfx950 mapping
//   * Each wave owns 16*NTW value columns for all positions: its share of the
//     state lives in VGPRs in the 16x16 MFMA accumulator layout (lane (g,col)
//     holds state rows 4g..4g+3 = (mode 2g, re/im), (mode 2g+1, re/im) of
//     column col), which is also the operand layout the carry product needs,
//     so the state never leaves registers.
//   * The intra-chunk product is computed transposed, Y^T = V^T G^T, with
//     v_mfma_f32_16x16x32_bf16: the V fragment a lane holds (8 consecutive
//     positions of one value column) is then the A operand of Y^T and the B
//     operand of the end-state product W V, and each output lane holds four
//     consecutive value columns of one position (one 8-byte LDS store).
//   * G and the carry matrix A are rounded once to bf16 (the output is bf16);
//     W, which feeds the fp32 state, is split into bf16 hi + lo, and the
//     state is split into hi + lo for the carry product, so the state path
//     keeps ~16 mantissa bits.
//   * v is streamed with 16-byte loads one chunk ahead of the arithmetic and
//     written to LDS transposed ([t/8][column][8]) with a bank swizzle; y is
//     staged through the same LDS region and written with 16-byte stores.
//   * Clocks, gates and pole tables are staged in LDS; G, W, A are built
//     cooperatively once per chunk and read by every wave.
//   * Workgroups are remapped so consecutive channels of the same batch row
//     run on the same XCD (the clock/gate rows they share stay in one L2).
#include "essh_internal.h"

namespace essh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float LOG2E = 1.4426950408889634f;

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
    static constexpr int CPT = (LC + THREADS - 1) / THREADS;   // control entries per thread
    static_assert(P % 16 == 0 && NT % NW == 0, "P must be 16, 32, 64 or 128");
    static_assert(LC % 32 == 0 && LC <= 128, "chunk length must be 32, 64 or 128");
    static_assert(M >= 1 && M <= 8, "1..8 modes");
    static_assert(LC % RPI == 0, "v tile loads must tile the chunk");
};

template <class C>
struct __align__(16) Smem {
    float dl[C::LC];                 // raw clock of the chunk
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
};

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Work-item order: channel fastest, then batch row, then segment.  When the
// grid is a multiple of 8 the hardware's round-robin XCD assignment is undone
// so that each XCD receives a contiguous range of work items.
__device__ __forceinline__ int remap_xcd(int bid, int nblocks) {
    if ((nblocks & 7) != 0) return bid;
    return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

template <class C>
__global__ void __launch_bounds__(C::THREADS)
prefill_chunk_kernel(PrefillArgs a, int seg_chunks) {
    constexpr int LC = C::LC, M = C::M, P = C::P, WCOLS = C::WCOLS, NTW = C::NTW;
    __shared__ Smem<C> sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int col = lane & 15;

    const int work = remap_xcd(blockIdx.x, gridDim.x);
    const int k = work % a.K_T;
    const int rest = work / a.K_T;
    const int b = rest % a.B;
    const int seg = rest / a.B;
    const int L = a.L, K = a.K;
    const int nchunks = (L + LC - 1) / LC;
    const int c_begin = seg * seg_chunks;
    const int c_end = min(nchunks, c_begin + seg_chunks);

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

    // ---- entering state, in the accumulator layout --------------------------
    f32x4_t st[NTW];
    {
        const float* src = (seg == 0) ? a.state_in : nullptr;
        const float* ws_in = nullptr;
        if (seg > 0) ws_in = static_cast<const float*>(a.workspace);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int p = wave * WCOLS + nt * 16 + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i, j = row >> 1, cmp = row & 1;
                float x = 0.f;
                if (j < M) {
                    if (src) {
                        x = src[((((size_t)b * K + k) * M + j) * 2 + cmp) * P + p];
                    } else if (ws_in) {
                        // entering states of segments: [seg][B][K_T][M][2][P]
                        const size_t e = (((((size_t)seg * a.B + b) * a.K_T + k) * M + j) * 2 + cmp) * P + p;
                        x = ws_in[e];
                    }
                }
                st[nt][i] = x;
            }
        }
    }

    // ---- chunk loop -----------------------------------------------------------
    const int vrow_l = lane / C::LPR;          // row of this lane inside a wave load
    const int vunit = lane % C::LPR;           // 16-byte unit of this lane inside a row
    const size_t vcol0 = (size_t)wave * WCOLS + vunit * 8;

    uint4 vreg[C::NLD];
    float cd[C::CPT], cw[C::CPT], cr_[C::CPT];

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
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) {
            const int r = tid + u * C::THREADS;
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
    };

    uint16_t* Vw = sm.V[wave];
    if (c_begin < c_end) load_chunk(c_begin);

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * LC;
        const int n = min(LC, L - t0);
        __syncthreads();   // previous chunk's readers of the shared tiles are done

        // v tile -> LDS, transposed: element (t, p') at ((t/8)*WCOLS + p'')*8 + t%8,
        // where p'' permutes the low 3 bits of p' by a key of (t/8, p'/8) so a
        // wave's 2-byte stores spread over all banks.
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
        // controls -> LDS
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) {
            const int r = tid + u * C::THREADS;
            if (r < LC) {
                sm.dl[r] = cd[u];
                sm.gw[r] = cw[u];
                sm.gr[r] = cr_[u];
            }
        }
        __syncthreads();

        // chunk-local inclusive clock sums (wave 0)
        if (wave == 0) {
            constexpr int PER = (LC + 63) / 64;
            float loc[PER];
            float run = 0.f;
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int idx = lane * PER + u;
                run += idx < LC ? sm.dl[idx] : 0.f;
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
            for (int u = 0; u < PER; ++u) {
                const int idx = lane * PER + u;
                if (idx < LC) {
                    const float q = excl + loc[u];
                    sm.q2[idx] = q * LOG2E;
                    sm.eq[idx] = expf(-q);
                }
            }
        }
        __syncthreads();

        // G[t][s] = e^{-(qh(t)-qh(s))} g_w(s) psi(t-s) for s <= t, bf16.
        // Only the 32-wide k blocks the MFMA loop reads are built.
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
        // W[(j,re/im)][s] = {Re,Im}(lambda_j^{n-1-s}) e^{-(qh(n-1)-qh(s))} g_w(s), hi + lo bf16.
        {
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
        }
        // A[t][(j,re/im)] = e^{-qh(t)} {Re, -Im}(c_j lambda_j^{t+1}), bf16, 8-byte units swizzled by t.
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
        __syncthreads();

        // prefetch the next chunk while this one is multiplied
        if (c + 1 < c_end) load_chunk(c + 1);

        // ---- MFMA phase (each wave: its WCOLS value columns) ----------------
        // v fragments: lane (g, col) holds v(s = 32ks + 8g .. +7, p = 16nt + col)
        bf16x8_t vf[C::KS][NTW];
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
        // State fragments as the A operand of the carry product.  The K axis
        // of one 16x16x32 product holds (state row, hi/lo half) pairs: lane
        // (g, col) supplies the bf16 hi parts of its state rows 4g..4g+3 in
        // elements 0..3 and the lo parts in elements 4..7; the B operand
        // repeats the matching carry-matrix entries in both halves.  Keeping
        // every product of the accumulation chain on the same MFMA shape
        // avoids a dependent 16x16x16 -> 16x16x32 accumulator hand-off.
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

        const int qu = C::QU;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
            const int tr = mt * 16 + col;          // position (row of G, A) owned by this lane
            // carry term first: y^T += H^T A^T over the (state row, hi/lo) axis
            const u16x4_t a4 = *reinterpret_cast<const u16x4_t*>(&sm.A[tr * 16 + ((g ^ ((tr >> 2) & 3)) * 4)]);
            const bf16x8_t af = __builtin_bit_cast(bf16x8_t, u16x8_t{a4[0], a4[1], a4[2], a4[3], a4[0], a4[1], a4[2], a4[3]});
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

        // end state: h <- Lambda h + W_hi V + W_lo V
        {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                f32x4_t d;
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const int j = 2 * g + (i >> 1);
                    float lr = 0.f, li = 0.f;
                    if (j < M) {
                        const float2 pw = sm.pw[n][j < M ? j : 0];
                        const float e = sm.eq[n - 1];
                        lr = pw.x * e;
                        li = pw.y * e;
                    }
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
        }

        // staged y -> global, 16 bytes per lane (undo the 8-byte unit swizzle)
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
    }

    // ---- leaving state ----------------------------------------------------------
    float* dst = nullptr;
    size_t dst_base = 0;
    if (seg_chunks * (seg + 1) >= nchunks) {
        dst = a.state_out;
        dst_base = ((size_t)b * K + k) * M;
    }
    if (dst) {
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int p = wave * WCOLS + nt * 16 + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i, j = row >> 1, cmp = row & 1;
                if (j < M) dst[((dst_base + j) * 2 + cmp) * P + p] = st[nt][i];
            }
        }
    }
}

template <int P, int M, int LC>
hipError_t launch_cfg(const PrefillArgs& a, hipStream_t s) {
    using C = Cfg<P, M, LC>;
    const int nchunks = (a.L + LC - 1) / LC;
    const int seg_chunks = nchunks;       // one segment per (b, k)
    const long long blocks = (long long)a.B * a.K_T;
    if (blocks == 0 || a.L == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_chunk_kernel<C>), dim3((unsigned)blocks), dim3(C::THREADS), 0, s, a, seg_chunks);
    return hipGetLastError();
}

template <int P, int M>
hipError_t launch_lc(const PrefillArgs& a, hipStream_t s) {
    switch (a.Lc) {
        case 32: return launch_cfg<P, M, 32>(a, s);
        case 64: return launch_cfg<P, M, 64>(a, s);
        case 128: return launch_cfg<P, M, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <int P>
hipError_t launch_m(const PrefillArgs& a, int m, hipStream_t s) {
    switch (m) {
        case 1: return launch_lc<P, 1>(a, s);
        case 2: return launch_lc<P, 2>(a, s);
        case 4: return launch_lc<P, 4>(a, s);
        case 8: return launch_lc<P, 8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool chunked_supported(int m, int P, int Lc, int io_dtype, int per_mode) {
    const bool mok = m == 1 || m == 2 || m == 4 || m == 8;
    const bool pok = P == 16 || P == 32 || P == 64 || P == 128;
    const bool lok = Lc == 32 || Lc == 64 || Lc == 128;
    return mok && pok && lok && io_dtype == ESSH_BF16 && !per_mode;
}

size_t chunked_workspace_bytes(int, int, int, int, int, int) { return 0; }

hipError_t launch_prefill_chunked(const PrefillArgs& a, int m, int P, hipStream_t s) {
    switch (P) {
        case 16: return launch_m<16>(a, m, s);
        case 32: return launch_m<32>(a, m, s);
        case 64: return launch_m<64>(a, m, s);
        case 128: return launch_m<128>(a, m, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace essh
