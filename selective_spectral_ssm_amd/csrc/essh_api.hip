// essh_api.hip -- the extern "C" entry points of libessh (declared in include/essh.h).
//
// Host-side validation and dispatch only; every arithmetic step runs in the
// HIP kernels of prefill_chunk.hip, prefill_seq.hip and decode.hip.
#include <stdint.h>

#include "backward.h"

using namespace essh;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int effective_lc(const essh_dims* d) { return d->Lc == 0 ? 64 : d->Lc; }

essh_status check_dims(const essh_dims* d, bool need_L) {
    if (!d) return ESSH_ERR_INVALID_ARG;
    if (d->B < 0 || (need_L && d->L < 0) || d->K < 1) return ESSH_ERR_INVALID_ARG;
    if (d->K_T < 1 || d->K_T > d->K) return ESSH_ERR_INVALID_ARG;
    if (d->ctrl_per_mode != 0 && d->ctrl_per_mode != 1) return ESSH_ERR_INVALID_ARG;
    if (d->io_dtype != ESSH_F32 && d->io_dtype != ESSH_BF16) return ESSH_ERR_UNSUPPORTED;
    if (!(d->m == 1 || d->m == 2 || d->m == 4 || d->m == 8)) return ESSH_ERR_UNSUPPORTED;
    if (!(d->P == 16 || d->P == 32 || d->P == 64 || d->P == 128)) return ESSH_ERR_UNSUPPORTED;
    if (need_L && !(d->Lc == 0 || d->Lc == 32 || d->Lc == 64 || d->Lc == 128)) return ESSH_ERR_UNSUPPORTED;
    // sizes must stay within 32-bit work-item counts used by the launchers
    const long long lanes = (long long)d->B * d->K * d->P;
    if (lanes > (1LL << 30)) return ESSH_ERR_UNSUPPORTED;
    return ESSH_OK;
}

essh_status from_hip(hipError_t e) { return e == hipSuccess ? ESSH_OK : ESSH_ERR_HIP; }

}  // namespace

extern "C" {

int32_t essh_abi_version(void) { return ESSH_ABI_VERSION; }

const char* essh_status_string(essh_status s) {
    switch (s) {
        case ESSH_OK: return "ESSH_OK";
        case ESSH_ERR_INVALID_ARG: return "ESSH_ERR_INVALID_ARG: null or misaligned pointer, or a size out of range";
        case ESSH_ERR_UNSUPPORTED: return "ESSH_ERR_UNSUPPORTED: m, P, Lc or dtype outside the compiled set";
        case ESSH_ERR_WORKSPACE: return "ESSH_ERR_WORKSPACE: workspace missing or too small";
        case ESSH_ERR_HIP: return "ESSH_ERR_HIP: a HIP launch failed";
        case ESSH_ERR_SCRATCH:
            return "ESSH_ERR_SCRATCH: the dims need more look-back space than the static scratch of "
                   "essh_mixer_prefill_noalloc (ESSH_NOALLOC_SCRATCH_BYTES); use essh_mixer_prefill";
        default: return "ESSH: unknown status";
    }
}

essh_status essh_state_init(float* state, int32_t n_layers, const essh_dims* d, hipStream_t stream) {
    essh_status st = check_dims(d, false);
    if (st != ESSH_OK) return st;
    if (n_layers < 1 || !state || !aligned(state, 16)) return ESSH_ERR_INVALID_ARG;
    const size_t n = (size_t)n_layers * d->B * d->K * d->m * 2 * d->P;
    return from_hip(launch_fill_zero(state, n, stream));
}

size_t essh_prefill_workspace_bytes(const essh_dims* d) {
    if (check_dims(d, true) != ESSH_OK) return 0;
    const int lc = effective_lc(d);
    if (!chunked_supported(d->m, d->P, lc, d->io_dtype, d->ctrl_per_mode)) return 0;
    return chunked_workspace_bytes(d->B, d->L, d->K_T, d->m, d->P, lc, d->ctrl_per_mode);
}

essh_status essh_mixer_prefill(const essh_dims* d,
                               const void* v, const float* delta, const void* g_w, const void* g_r,
                               const float* rho, const float* theta, const float* c, const float* zl,
                               const float* state_in, float* state_out, void* y,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    essh_status st = check_dims(d, true);
    if (st != ESSH_OK) return st;
    const size_t io = d->io_dtype == ESSH_BF16 ? 2 : 4;
    if (!v || !delta || !g_w || !g_r || !rho || !theta || !c || !y) return ESSH_ERR_INVALID_ARG;
    if (!aligned(v, 16) || !aligned(y, 16) || !aligned(delta, 4) || !aligned(g_w, io) || !aligned(g_r, io) ||
        !aligned(rho, 4) || !aligned(theta, 4) || !aligned(c, 4) || (zl && !aligned(zl, 4)))
        return ESSH_ERR_INVALID_ARG;
    if ((state_in && !aligned(state_in, 16)) || (state_out && !aligned(state_out, 16))) return ESSH_ERR_INVALID_ARG;
    if ((d->P * io) % 16 != 0) return ESSH_ERR_UNSUPPORTED;

    const int lc = effective_lc(d);
    const bool chunked = chunked_supported(d->m, d->P, lc, d->io_dtype, d->ctrl_per_mode);
    const size_t need = chunked ? chunked_workspace_bytes(d->B, d->L, d->K_T, d->m, d->P, lc, d->ctrl_per_mode) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return ESSH_ERR_WORKSPACE;

    if (d->B == 0) return ESSH_OK;
    if (d->L == 0) {
        // no positions: the state passes through unchanged
        if (state_out) return from_hip(launch_copy_state(state_in, state_out, d->B, d->K, d->K_T, d->m, d->P, stream));
        return ESSH_OK;
    }

    PrefillArgs a{};
    a.B = d->B;
    a.L = d->L;
    a.K = d->K;
    a.K_T = d->K_T;
    a.Lc = lc;
    a.per_mode = d->ctrl_per_mode;
    a.v = v;
    a.delta = delta;
    a.g_w = g_w;
    a.g_r = g_r;
    a.rho = rho;
    a.theta = theta;
    a.c = c;
    a.zl = zl;
    a.state_in = state_in;
    a.state_out = state_out;
    a.y = y;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    hipError_t e;
    if (chunked) {
        ScanPlan plan = plan_chunked(d->B, d->L, d->K_T, d->m, d->P, lc, d->ctrl_per_mode);
        bind_workspace(plan, workspace, d->m, d->P);
        e = launch_prefill_chunked(a, d->m, d->P, plan, stream);
    } else if (d->io_dtype == ESSH_F32 && !d->ctrl_per_mode) {
        e = launch_prefill_f32_chunked(a, d->m, d->P, stream);
    } else {
        e = launch_prefill_sequential(a, d->m, d->P, d->io_dtype, stream);
    }
    return from_hip(e);
}

essh_status essh_mixer_decode_step(int32_t n_layers, const essh_dims* d,
                                   const void* v, const float* delta, const void* g_w, const void* g_r,
                                   const float* rho, const float* theta, const float* c, const float* zl,
                                   float* state, void* y, hipStream_t stream) {
    essh_status st = check_dims(d, false);
    if (st != ESSH_OK) return st;
    if (n_layers < 1) return ESSH_ERR_INVALID_ARG;
    const size_t io = d->io_dtype == ESSH_BF16 ? 2 : 4;
    if (!v || !delta || !g_w || !g_r || !rho || !theta || !c || !state || !y) return ESSH_ERR_INVALID_ARG;
    if (!aligned(v, 16) || !aligned(y, 16) || !aligned(state, 16) || !aligned(delta, 4) || !aligned(g_w, io) ||
        !aligned(g_r, io) || !aligned(rho, 4) || !aligned(theta, 4) || !aligned(c, 4) || (zl && !aligned(zl, 4)))
        return ESSH_ERR_INVALID_ARG;
    if ((long long)n_layers * d->B * d->K * d->P > (1LL << 30)) return ESSH_ERR_UNSUPPORTED;
    if (d->B > 65535 || n_layers > 65535) return ESSH_ERR_UNSUPPORTED;   // grid y and z extents
    if (d->B == 0) return ESSH_OK;

    DecodeArgs a{};
    a.n_layers = n_layers;
    a.B = d->B;
    a.K = d->K;
    a.K_T = d->K_T;
    a.per_mode = d->ctrl_per_mode;
    a.v = v;
    a.delta = delta;
    a.g_w = g_w;
    a.g_r = g_r;
    a.rho = rho;
    a.theta = theta;
    a.c = c;
    a.zl = zl;
    a.state = state;
    a.y = y;
    return from_hip(launch_decode(a, d->m, d->P, d->io_dtype, stream));
}

essh_status essh_decode_fused_step(int32_t n_layers, const essh_dims* d, int32_t d_model, const void* u,
                                   const void* w_in, const float* beta, float eps_norm, const void* w_ctl,
                                   const float* b_ctl, const float* rho, const float* theta, const float* c,
                                   const float* zl, const void* w_out, float* state, float* z, float* y,
                                   hipStream_t stream) {
    essh_status st = check_dims(d, false);
    if (st != ESSH_OK) return st;
    if (n_layers < 1 || !(eps_norm > 0.f) || eps_norm > 3.0e38f) return ESSH_ERR_INVALID_ARG;
    const size_t io = d->io_dtype == ESSH_BF16 ? 2 : 4;
    if (!u || !w_in || !beta || !w_ctl || !b_ctl || !rho || !theta || !c || !w_out || !state || !z || !y)
        return ESSH_ERR_INVALID_ARG;
    if (!aligned(u, io) || !aligned(w_in, 16) || !aligned(w_ctl, 16) || !aligned(w_out, 16) || !aligned(beta, 4) ||
        !aligned(b_ctl, 4) || !aligned(rho, 4) || !aligned(theta, 4) || !aligned(c, 4) || (zl && !aligned(zl, 4)) ||
        !aligned(state, 4) || !aligned(z, 4) || !aligned(y, 4))
        return ESSH_ERR_INVALID_ARG;
    // u staged in LDS, 16-byte weight loads; the retained channel outputs staged in LDS
    if (d_model < 8 || d_model % 8 != 0 || d_model > 8192 || (long long)d->K_T * d->P > 8192)
        return ESSH_ERR_UNSUPPORTED;
    if (d->B > 65535 || n_layers > 65535 || d->K_T > 65535) return ESSH_ERR_UNSUPPORTED;   // grid extents
    if ((long long)n_layers * d->B * d->K * d->P > (1LL << 30) ||
        (long long)n_layers * d->K * d->P * d_model > (1LL << 40))
        return ESSH_ERR_UNSUPPORTED;
    if (d->B == 0) return ESSH_OK;

    FusedDecodeArgs a{};
    a.n_layers = n_layers;
    a.B = d->B;
    a.K = d->K;
    a.K_T = d->K_T;
    a.m = d->m;
    a.P = d->P;
    a.d_model = d_model;
    a.eps_norm = eps_norm;
    a.u = u;
    a.w_in = static_cast<const uint16_t*>(w_in);
    a.beta = beta;
    a.w_ctl = static_cast<const uint16_t*>(w_ctl);
    a.b_ctl = b_ctl;
    a.rho = rho;
    a.theta = theta;
    a.c = c;
    a.zl = zl;
    a.w_out = static_cast<const uint16_t*>(w_out);
    a.state = state;
    a.z = z;
    a.y = y;
    return from_hip(launch_decode_fused(a, d->io_dtype, stream));
}

size_t essh_prefill_backward_workspace_bytes(const essh_dims* d) {
    if (check_dims(d, true) != ESSH_OK || d->ctrl_per_mode) return 0;
    return backward_workspace_bytes(d->B, d->L, d->K, d->K_T, d->m, d->P);
}

essh_status essh_mixer_prefill_backward(const essh_dims* d,
                                        const void* v, const float* delta, const void* g_w, const void* g_r,
                                        const float* rho, const float* theta, const float* c, const float* zl,
                                        const float* state_in, const void* dy, const float* dstate_out,
                                        void* dv, float* ddelta, float* dg_w, float* dg_r,
                                        float* drho, float* dtheta, float* dc, float* dzl, float* dstate_in,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    essh_status st = check_dims(d, true);
    if (st != ESSH_OK) return st;
    if (d->ctrl_per_mode) return ESSH_ERR_UNSUPPORTED;
    if ((long long)d->B * d->K_T > 65535) return ESSH_ERR_UNSUPPORTED;   // grid z extent
    const size_t io = d->io_dtype == ESSH_BF16 ? 2 : 4;
    if (!v || !delta || !g_w || !g_r || !rho || !theta || !c || !dy || !dv || !ddelta || !dg_w || !dg_r || !drho ||
        !dtheta || !dc)
        return ESSH_ERR_INVALID_ARG;
    if (!aligned(v, 16) || !aligned(dy, 16) || !aligned(dv, 16) || !aligned(delta, 4) || !aligned(g_w, io) ||
        !aligned(g_r, io) || !aligned(rho, 4) || !aligned(theta, 4) || !aligned(c, 4) || (zl && !aligned(zl, 4)) ||
        (state_in && !aligned(state_in, 4)) || (dstate_out && !aligned(dstate_out, 4)) || !aligned(ddelta, 4) ||
        !aligned(dg_w, 4) || !aligned(dg_r, 4) || !aligned(drho, 4) || !aligned(dtheta, 4) || !aligned(dc, 4) ||
        (dzl && !aligned(dzl, 4)) || (dstate_in && !aligned(dstate_in, 4)))
        return ESSH_ERR_INVALID_ARG;
    if ((d->P * io) % 16 != 0) return ESSH_ERR_UNSUPPORTED;
    const size_t need = backward_workspace_bytes(d->B, d->L, d->K, d->K_T, d->m, d->P);
    if (d->B > 0 && d->L > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return ESSH_ERR_WORKSPACE;

    if (d->B == 0 || d->L == 0) {
        // no positions: the mode tables get zero gradient and the adjoint passes through
        const size_t km = (size_t)d->K_T * d->m;
        hipError_t e = launch_fill_zero(drho, km, stream);
        if (e == hipSuccess) e = launch_fill_zero(dtheta, km, stream);
        if (e == hipSuccess) e = launch_fill_zero(dc, 2 * km, stream);
        if (e == hipSuccess && dzl) e = launch_fill_zero(dzl, km, stream);
        if (e == hipSuccess && dstate_in)
            e = launch_copy_state(dstate_out, dstate_in, d->B, d->K, d->K_T, d->m, d->P, stream);
        return from_hip(e);
    }

    BackwardArgs a{};
    a.B = d->B;
    a.L = d->L;
    a.K = d->K;
    a.K_T = d->K_T;
    a.v = v;
    a.delta = delta;
    a.g_w = g_w;
    a.g_r = g_r;
    a.rho = rho;
    a.theta = theta;
    a.c = c;
    a.zl = zl;
    a.state_in = state_in;
    a.dy = dy;
    a.dstate_out = dstate_out;
    a.dv = dv;
    a.ddelta = ddelta;
    a.dg_w = dg_w;
    a.dg_r = dg_r;
    a.drho = drho;
    a.dtheta = dtheta;
    a.dc = dc;
    a.dzl = dzl;
    a.dstate_in = dstate_in;
    BwdPlan plan = plan_backward(d->B, d->L, d->K, d->K_T, d->m, d->P);
    bind_backward_workspace(plan, workspace, d->m);
    return from_hip(launch_prefill_backward(a, d->m, plan, d->io_dtype, stream));
}

}  // extern "C"
