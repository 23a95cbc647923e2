// mhc_api.cpp -- the exported C entry points: validation, planning, dispatch.
//
// No HIP header is included here: every check runs on the host before the first HIP
// call, so the whole file builds with a plain C++ compiler and its error paths can be
// exercised without a GPU. Kernel launches go through mhc::launch_* (mhc_kernels.hip).
#include <cstdint>
#include <cstring>

#include "../../include/mhc.h"
#include "mhc_bwd_plan.h"
#include "mhc_plan.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Attribute checks shared by every entry point (the aclnn guides reject unsupported
// hcMult / numIters / shapes with the invalid-parameter class). T is checked by callers
// that use it.
mhc_status check_params(const mhc_pre_params* p, mhc::Geometry* g)
{
    if (!p) return MHC_ERR_NULLPTR;
    if (p->x_dtype != MHC_DTYPE_BF16 && p->x_dtype != MHC_DTYPE_F16) return MHC_ERR_PARAM_INVALID;
    if (p->need_backward != 0 && p->need_backward != 1) return MHC_ERR_PARAM_INVALID;
    if (!(p->norm_eps > 0.0)) return MHC_ERR_PARAM_INVALID;      // also rejects NaN
    if (!(p->hc_eps >= 0.0)) return MHC_ERR_PARAM_INVALID;
    if (p->n_alpha == 3 && p->num_iters < 1) return MHC_ERR_PARAM_INVALID;
    if (p->num_iters < 0 || p->num_iters > 1000) return MHC_ERR_PARAM_INVALID;
    if (!mhc::make_geometry(p->n, p->D, p->n_alpha, g)) return MHC_ERR_PARAM_INVALID;
    g->x_f16 = p->x_dtype == MHC_DTYPE_F16;
    return MHC_OK;
}

}  // namespace

extern "C" {

int mhc_version(void) { return kVersion; }

const char* mhc_status_string(mhc_status s)
{
    switch (s) {
    case MHC_OK: return "MHC_OK: success";
    case MHC_ERR_NULLPTR: return "MHC_ERR_NULLPTR: a required pointer is NULL";
    case MHC_ERR_PARAM_INVALID:
        return "MHC_ERR_PARAM_INVALID: unsupported size/attribute, inconsistent outputs, "
               "misaligned pointer or buffer too small";
    case MHC_ERR_RUNTIME: return "MHC_ERR_RUNTIME: a HIP call failed";
    default: return "unknown mhc_status";
    }
}

mhc_status mhc_pre_packed_size(const mhc_pre_params* params, size_t* bytes)
{
    if (!params || !bytes) return MHC_ERR_NULLPTR;
    mhc::Geometry g;
    mhc_status st = check_params(params, &g);
    if (st != MHC_OK) return st;
    *bytes = g.packed_bytes;
    return MHC_OK;
}

mhc_status mhc_pre_workspace_size(const mhc_pre_params* params, size_t* bytes)
{
    if (!params || !bytes) return MHC_ERR_NULLPTR;
    mhc::Geometry g;
    mhc_status st = check_params(params, &g);
    if (st != MHC_OK) return st;
    if (params->T < 0) return MHC_ERR_PARAM_INVALID;
    *bytes = mhc::make_plan(g, params->T).ws_bytes;
    return MHC_OK;
}

mhc_status mhc_pre_forward_path(const mhc_pre_params* params, int32_t has_pre_mix, int32_t* path)
{
    if (!params || !path) return MHC_ERR_NULLPTR;
    mhc::Geometry g;
    mhc_status st = check_params(params, &g);
    if (st != MHC_OK) return st;
    if (params->T < 0) return MHC_ERR_PARAM_INVALID;
    *path = mhc::forward_path(mhc::make_plan(g, params->T), has_pre_mix != 0);
    return MHC_OK;
}

mhc_status mhc_pre_prepack(const mhc_pre_params* params, const float* phi, const float* gamma,
                           void* phi_packed, size_t packed_bytes, void* stream)
{
    if (!params || !phi || !phi_packed) return MHC_ERR_NULLPTR;
    mhc::Geometry g;
    mhc_status st = check_params(params, &g);
    if (st != MHC_OK) return st;
    if (packed_bytes < g.packed_bytes) return MHC_ERR_PARAM_INVALID;
    if (!aligned(phi_packed, 16) || !aligned(phi, 4) || (gamma && !aligned(gamma, 4)))
        return MHC_ERR_PARAM_INVALID;
    return mhc::launch_prepack(g, phi, gamma, phi_packed, stream) == 0 ? MHC_OK : MHC_ERR_RUNTIME;
}

}  // extern "C"

namespace {

// The forward; events is NULL or mhc::kStages + 1 validated, non-NULL hipEvent_t handles.
mhc_status forward_impl(const mhc_pre_params* params, const mhc_pre_tensors* t,
                        void* workspace, size_t workspace_bytes, void* stream,
                        void* const* events)
{
    // 1. required pointers
    if (!params || !t) return MHC_ERR_NULLPTR;
    if (!t->x || !t->alpha || !t->bias || !t->h_in || !t->h_post) return MHC_ERR_NULLPTR;
    if (!t->phi && !t->phi_packed) return MHC_ERR_NULLPTR;
    if (params->n_alpha == 3 && !t->h_res) return MHC_ERR_NULLPTR;
    if (!workspace) return MHC_ERR_NULLPTR;

    // 2. attributes and sizes
    mhc::Geometry g;
    mhc_status st = check_params(params, &g);
    if (st != MHC_OK) return st;
    if (params->T < 0) return MHC_ERR_PARAM_INVALID;

    // 3. output set: needBackward makes the intermediates mandatory; the Sinkhorn planes
    //    exist only with the res branch.
    const bool res_branch = params->n_alpha == 3;
    if (!res_branch && (t->sum_out || t->norm_out)) return MHC_ERR_PARAM_INVALID;
    if (params->need_backward) {
        if (!t->inv_rms || !t->h_mix || !t->h_pre) return MHC_ERR_PARAM_INVALID;
        if (res_branch && (!t->sum_out || !t->norm_out)) return MHC_ERR_PARAM_INVALID;
    }

    // 4. workspace
    const mhc::Plan plan = mhc::make_plan(g, params->T, t->pre_mix != nullptr);
    if (workspace_bytes < plan.ws_bytes) return MHC_ERR_PARAM_INVALID;

    // 5. alignment: 16-byte vector access to x and hIn, 256-byte workspace sections
    if (!aligned(t->x, 16) || !aligned(t->h_in, 16) || !aligned(workspace, 256))
        return MHC_ERR_PARAM_INVALID;
    if (t->phi_packed && !aligned(t->phi_packed, 16)) return MHC_ERR_PARAM_INVALID;
    const void* f32s[] = {t->phi, t->alpha, t->bias, t->gamma, t->pre_mix, t->h_post, t->h_res,
                          t->inv_rms, t->h_mix, t->h_pre, t->sum_out, t->norm_out};
    for (const void* q : f32s)
        if (q && !aligned(q, 4)) return MHC_ERR_PARAM_INVALID;

    if (params->T == 0) {   // empty input: success, no kernel launched
        for (int i = 0; events && i <= mhc::kStages; ++i)
            if (events[i] && mhc::record_event(events[i], stream) != 0) return MHC_ERR_RUNTIME;
        return MHC_OK;
    }

    char* ws = static_cast<char*>(workspace);

    mhc::ForwardArgs a;
    std::memset(&a, 0, sizeof a);
    a.x = t->x;
    a.packed = t->phi_packed;   // NULL: packed by the launch (in the kernel or by the pack kernel)
    a.phi = t->phi;
    a.gamma = t->gamma;
    a.packed_ws = ws + plan.off_packed;
    a.alpha = t->alpha;
    a.bias = t->bias;
    a.pre_mix = t->pre_mix;
    a.h_in = t->h_in;
    a.h_post = t->h_post;
    a.h_res = t->h_res;
    a.inv_rms = t->inv_rms;
    a.h_mix = t->h_mix;
    a.h_pre = t->h_pre;
    a.sum_out = res_branch ? t->sum_out : nullptr;
    a.norm_out = res_branch ? t->norm_out : nullptr;
    a.wts = reinterpret_cast<float*>(ws + plan.off_wts);
    a.rec = reinterpret_cast<float*>(ws + plan.off_rec);
    a.prx = plan.fused_geom ? reinterpret_cast<uint64_t*>(ws + plan.off_prx) : nullptr;
    a.hpx = plan.fused_geom ? reinterpret_cast<uint64_t*>(ws + plan.off_hpx) : nullptr;
    a.dpart = plan.decode_geom ? reinterpret_cast<uint64_t*>(ws + plan.off_dpart) : nullptr;
    a.dhp = plan.decode_geom ? reinterpret_cast<uint64_t*>(ws + plan.off_dhp) : nullptr;
    a.sync = reinterpret_cast<uint32_t*>(ws + plan.off_sync);
    a.num_iters = params->num_iters;
    a.norm_eps = params->norm_eps;
    a.hc_eps = params->hc_eps;
    return mhc::launch_forward(plan, a, stream, events) == 0 ? MHC_OK : MHC_ERR_RUNTIME;
}

}  // namespace

extern "C" {

mhc_status mhc_pre_forward(const mhc_pre_params* params, const mhc_pre_tensors* t,
                           void* workspace, size_t workspace_bytes, void* stream)
{
    return forward_impl(params, t, workspace, workspace_bytes, stream, nullptr);
}

mhc_status mhc_pre_forward_noalloc(const mhc_pre_params* params, const mhc_pre_tensors* t, void* stream)
{
    // the checks that need no device first, in the order mhc_pre_forward makes them; the
    // workspace comes from the library's per-GPU scratch array
    if (!params || !t) return MHC_ERR_NULLPTR;
    mhc::Geometry g;
    mhc_status st = check_params(params, &g);
    if (st != MHC_OK) return st;
    if (params->T < 0) return MHC_ERR_PARAM_INVALID;
    if (mhc::make_plan(g, params->T).ws_bytes > mhc::kScratchBytes) return MHC_ERR_PARAM_INVALID;
    void* ws = nullptr;
    if (mhc::scratch_for_current_device(&ws) != 0) return MHC_ERR_RUNTIME;
    return forward_impl(params, t, ws, mhc::kScratchBytes, stream, nullptr);
}

mhc_status mhc_pre_wait_status(void* workspace, size_t workspace_bytes, void* stream, int32_t* timed_out)
{
    if (!workspace || !timed_out) return MHC_ERR_NULLPTR;
    if (workspace_bytes < 256 || !aligned(workspace, 256)) return MHC_ERR_PARAM_INVALID;
    return mhc::read_and_clear_wait_flag(static_cast<uint32_t*>(workspace), timed_out, stream) == 0
               ? MHC_OK
               : MHC_ERR_RUNTIME;
}

static_assert(MHC_FORWARD_EVENTS == mhc::kStages + 1, "one event per kernel boundary");

mhc_status mhc_pre_forward_timed(const mhc_pre_params* params, const mhc_pre_tensors* t,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* events, int32_t num_events)
{
    if (!events) return MHC_ERR_NULLPTR;
    if (num_events != MHC_FORWARD_EVENTS) return MHC_ERR_PARAM_INVALID;
    return forward_impl(params, t, workspace, workspace_bytes, stream, events);
}

}  // extern "C"

namespace {

mhc_status check_bwd_params(const mhc_pre_bwd_params* p, mhc::bwd::Geometry* g)
{
    if (!p) return MHC_ERR_NULLPTR;
    if (p->x_f16 != 0 && p->x_f16 != 1) return MHC_ERR_PARAM_INVALID;
    if (p->num_iters < 0 || p->num_iters > 1000) return MHC_ERR_PARAM_INVALID;
    if (!(p->hc_eps >= 0.0)) return MHC_ERR_PARAM_INVALID;    // also rejects NaN
    if (p->T < 0) return MHC_ERR_PARAM_INVALID;
    if (!mhc::bwd::make_geometry(p->n, p->D, g, p->x_f16 == 1)) return MHC_ERR_PARAM_INVALID;
    return MHC_OK;
}

}  // namespace

extern "C" {

mhc_status mhc_pre_backward_workspace_size(const mhc_pre_bwd_params* params, size_t* bytes)
{
    if (!params || !bytes) return MHC_ERR_NULLPTR;
    mhc::bwd::Geometry g;
    mhc_status st = check_bwd_params(params, &g);
    if (st != MHC_OK) return st;
    *bytes = mhc::bwd::make_plan(g, params->T).ws_bytes;
    return MHC_OK;
}

mhc_status mhc_pre_backward(const mhc_pre_bwd_params* params, const mhc_pre_bwd_tensors* t,
                            void* workspace, size_t workspace_bytes, void* stream)
{
    if (!params || !t) return MHC_ERR_NULLPTR;
    mhc::bwd::Geometry g;
    mhc_status st = check_bwd_params(params, &g);
    if (st != MHC_OK) return st;
    // per-token tensors are empty (and may be NULL) when T == 0
    const bool tok = params->T > 0;
    if (!t->phi || !t->alpha || !t->grad_phi || !t->grad_alpha || !t->grad_bias || !workspace)
        return MHC_ERR_NULLPTR;
    if (tok && (!t->x || !t->grad_h_in || !t->grad_h_post || !t->grad_h_res || !t->inv_rms ||
                !t->h_mix || !t->h_pre || !t->h_post || !t->grad_x))
        return MHC_ERR_NULLPTR;
    if (tok && params->num_iters > 0 && (!t->sum_out || !t->norm_out)) return MHC_ERR_NULLPTR;
    if (t->gamma && !t->grad_gamma) return MHC_ERR_NULLPTR;
    const mhc::bwd::Plan plan = mhc::bwd::make_plan(g, params->T);
    if (workspace_bytes < plan.ws_bytes) return MHC_ERR_PARAM_INVALID;
    if (!aligned(t->x, 16) || !aligned(t->grad_h_in, 16) || !aligned(t->grad_x, 16) ||
        (t->grad_x_post && !aligned(t->grad_x_post, 16)) || !aligned(workspace, 256))
        return MHC_ERR_PARAM_INVALID;

    mhc::bwd::Args a;
    a.x = t->x;
    a.phi = t->phi;
    a.alpha = t->alpha;
    a.grad_h_in = t->grad_h_in;
    a.grad_h_post = t->grad_h_post;
    a.grad_h_res = t->grad_h_res;
    a.inv_rms = t->inv_rms;
    a.h_mix = t->h_mix;
    a.h_pre = t->h_pre;
    a.h_post = t->h_post;
    a.gamma = t->gamma;
    a.grad_x_post = t->grad_x_post;
    a.grad_x = t->grad_x;
    a.grad_phi = t->grad_phi;
    a.grad_alpha = t->grad_alpha;
    a.grad_bias = t->grad_bias;
    a.grad_gamma = t->gamma ? t->grad_gamma : nullptr;
    a.hc_eps = params->hc_eps;
    a.num_iters = params->num_iters;
    a.sum_out = params->num_iters > 0 ? t->sum_out : nullptr;
    a.norm_out = params->num_iters > 0 ? t->norm_out : nullptr;
    char* ws = static_cast<char*>(workspace);
    a.pack = ws + plan.off_pack;
    a.gmix = reinterpret_cast<uint16_t*>(ws + plan.off_gmix);
    a.c3 = reinterpret_cast<float*>(ws + plan.off_c3);
    a.terms = reinterpret_cast<double*>(ws + plan.off_terms);
    a.pphi = reinterpret_cast<float*>(ws + plan.off_pphi);
    a.pgam = reinterpret_cast<float*>(ws + plan.off_pgam);
    a.glog = reinterpret_cast<double*>(ws + plan.off_glog);
    return mhc::bwd::launch_backward(plan, a, stream) == 0 ? MHC_OK : MHC_ERR_RUNTIME;
}

}  // extern "C"

extern "C" {

mhc_status mhc_post(const mhc_post_params* params, const mhc_post_tensors* t, void* stream)
{
    if (!params || !t) return MHC_ERR_NULLPTR;
    if (params->T < 0 || (params->n != 4 && params->n != 6 && params->n != 8)) return MHC_ERR_PARAM_INVALID;
    if (params->D < 8 || params->D % 8 != 0 || params->D > mhc::kMaxD) return MHC_ERR_PARAM_INVALID;
    if (params->x_dtype != MHC_DTYPE_BF16 && params->x_dtype != MHC_DTYPE_F16) return MHC_ERR_PARAM_INVALID;
    if (params->reserved != 0) return MHC_ERR_PARAM_INVALID;
    if (params->T == 0) return MHC_OK;
    if (!t->x || !t->residual || !t->post || !t->comb || !t->out) return MHC_ERR_NULLPTR;
    if (!aligned(t->x, 16) || !aligned(t->residual, 16) || !aligned(t->out, 16) || !aligned(t->post, 4) ||
        !aligned(t->comb, 4))
        return MHC_ERR_PARAM_INVALID;
    return mhc::launch_post(params->T, params->n, params->D, t->x, t->residual, t->post, t->comb, t->out,
                            params->x_dtype == MHC_DTYPE_F16, stream) == 0
               ? MHC_OK
               : MHC_ERR_RUNTIME;
}

}  // extern "C"

extern "C" {

mhc_status mhc_pre_inv_rms(const mhc_pre_params* params, const uint16_t* x, float* inv_rms, void* stream)
{
    if (!params) return MHC_ERR_NULLPTR;
    mhc::Geometry g;
    mhc_status st = check_params(params, &g);
    if (st != MHC_OK) return st;
    if (params->T < 0) return MHC_ERR_PARAM_INVALID;
    if (params->T == 0) return MHC_OK;
    if (!x || !inv_rms) return MHC_ERR_NULLPTR;
    if (!aligned(x, 16) || !aligned(inv_rms, 4)) return MHC_ERR_PARAM_INVALID;
    return mhc::launch_inv_rms(params->T, params->n, params->D, params->norm_eps, x, inv_rms, g.x_f16, stream) == 0
               ? MHC_OK
               : MHC_ERR_RUNTIME;
}

mhc_status mhc_pre_sinkhorn(const mhc_pre_params* params, const mhc_pre_sinkhorn_tensors* t, void* stream)
{
    if (!params || !t) return MHC_ERR_NULLPTR;
    mhc::Geometry g;
    mhc_status st = check_params(params, &g);
    if (st != MHC_OK) return st;
    if (params->T < 0) return MHC_ERR_PARAM_INVALID;
    const bool res_branch = params->n_alpha == 3;
    if (!res_branch && (t->sum_out || t->norm_out)) return MHC_ERR_PARAM_INVALID;
    if (params->T == 0) return MHC_OK;
    if (!t->x || !t->h_mix || !t->inv_rms || !t->alpha || !t->bias || !t->h_in || !t->h_pre || !t->h_post)
        return MHC_ERR_NULLPTR;
    if (res_branch && !t->h_res) return MHC_ERR_NULLPTR;
    if (params->need_backward && res_branch && (!t->sum_out || !t->norm_out)) return MHC_ERR_PARAM_INVALID;
    if (!aligned(t->x, 16) || !aligned(t->h_in, 16)) return MHC_ERR_PARAM_INVALID;
    const void* f32s[] = {t->h_mix, t->inv_rms, t->alpha, t->bias, t->pre_mix, t->h_pre, t->h_post,
                          t->h_res, t->sum_out, t->norm_out};
    for (const void* q : f32s)
        if (q && !aligned(q, 4)) return MHC_ERR_PARAM_INVALID;

    mhc::ForwardArgs a;
    std::memset(&a, 0, sizeof a);
    a.x = t->x;
    a.alpha = t->alpha;
    a.bias = t->bias;
    a.pre_mix = t->pre_mix;
    a.h_in = t->h_in;
    a.h_pre = t->h_pre;
    a.h_post = t->h_post;
    a.h_res = t->h_res;
    a.sum_out = res_branch ? t->sum_out : nullptr;
    a.norm_out = res_branch ? t->norm_out : nullptr;
    a.num_iters = params->num_iters;
    a.norm_eps = params->norm_eps;
    a.hc_eps = params->hc_eps;
    return mhc::launch_pre_sinkhorn(params->T, params->n, params->D, params->n_alpha, g.x_f16, a, t->h_mix,
                                    t->inv_rms, stream) == 0
               ? MHC_OK
               : MHC_ERR_RUNTIME;
}

}  // extern "C"
