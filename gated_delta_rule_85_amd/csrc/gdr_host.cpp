// gdr_host.cpp -- the C ABI declared in include/gdr.h: argument validation
// (pure host code, no HIP call before it passes), workspace sizing and
// dispatch to the gfx950 kernels.
#include <stdio.h>
#include <stdarg.h>
#include <string.h>

#include <atomic>

#include "gdr.h"
#include "gdr_kernels.hpp"

// Workspace of gdr_forward_chunked_noalloc: one array per device, placed by
// the code object's loader, never allocated by a call.  Host code must not
// pass this name to a kernel or a copy (on the host it is a stand-in, not a
// device address); it uses the address hipGetSymbolAddress returns for the
// current device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_WORKSPACE_MAX];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch[kMaxScratchDevices];

// Device address of the current device's scratch array, looked up on the
// first call made with that device current and kept.  Threads that race on the
// first lookup store the same address.
hipError_t noalloc_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    void *ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (!ptr) {
        if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch[dev].store(ptr, std::memory_order_release);
    }
    *out = ptr;
    return hipSuccess;
}

thread_local char g_detail[512];

gdr_status fail(gdr_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return s;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// mode: 0 chunked forward, 1 decode step, 2 gradient of the chunked forward.
gdr_status check(const gdr_args *a, int mode) {
    const int for_decode = mode == 1;
    if (!a) return fail(GDR_ERR_INVALID_ARGUMENT, "args is NULL");
    if (a->variant < GDR_DELTANET || a->variant > GDR_KLA)
        return fail(GDR_ERR_INVALID_ARGUMENT, "unknown variant %d", a->variant);
    if (a->dtype != GDR_F32 && a->dtype != GDR_BF16)
        return fail(GDR_ERR_INVALID_ARGUMENT, "unknown dtype %d", a->dtype);
    if (a->flags & ~(GDR_FLAG_QK_L2NORM | GDR_FLAG_RAW_GATES))
        return fail(GDR_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", (unsigned)a->flags);
    if ((a->flags & GDR_FLAG_RAW_GATES) && a->variant != GDR_DELTANET) {
        if (!(a->decay_scale > 0.f && a->decay_scale <= 3.402823466e+38f))
            return fail(GDR_ERR_INVALID_ARGUMENT,
                        "decay_scale must be finite and > 0 with GDR_FLAG_RAW_GATES");
    } else if (a->decay_scale != 0.f) {
        return fail(GDR_ERR_INVALID_ARGUMENT,
                    "decay_scale is only used with GDR_FLAG_RAW_GATES and a decaying variant");
    }
    if (a->B < 1 || a->T < 1 || a->H < 1)
        return fail(GDR_ERR_INVALID_ARGUMENT, "B, T, H must be >= 1 (got %lld, %lld, %lld)",
                    (long long)a->B, (long long)a->T, (long long)a->H);
    if (a->dk < 1 || a->dv < 1)
        return fail(GDR_ERR_INVALID_ARGUMENT, "dk, dv must be >= 1");
    if ((a->dk != 64 && a->dk != 128) || (a->dv != 64 && a->dv != 128))
        return fail(GDR_ERR_UNSUPPORTED, "dk and dv must each be 64 or 128 (got %lld, %lld)",
                    (long long)a->dk, (long long)a->dv);
    if (a->B > 65535 || a->H > 65535 || a->B * a->H > (int64_t(1) << 24) ||
        a->T > (int64_t(1) << 31))
        return fail(GDR_ERR_UNSUPPORTED, "B, H or T beyond the supported range "
                    "(B, H <= 65535, B*H <= 2^24, T <= 2^31)");
    if (for_decode) {
        if (a->T != 1) return fail(GDR_ERR_INVALID_ARGUMENT, "decode needs T == 1 (got %lld)",
                                   (long long)a->T);
        if (!a->state_in || !a->state_out)
            return fail(GDR_ERR_INVALID_ARGUMENT, "decode needs state_in and state_out");
    } else {
        if (a->chunk != 0 && a->chunk != 64)
            return fail(GDR_ERR_UNSUPPORTED, "chunk must be 0 or 64 (got %d)", a->chunk);
    }
    if (mode == 2) {
        if (a->flags != 0)
            return fail(GDR_ERR_UNSUPPORTED, "the gradient takes stored inputs (flags must be 0)");
        if (a->B * a->H * ((a->T + 63) / 64) > (int64_t(1) << 31) - 1)
            return fail(GDR_ERR_UNSUPPORTED, "B * H * ceil(T / 64) must be below 2^31");
        if (!a->q || !a->k || !a->v)
            return fail(GDR_ERR_INVALID_ARGUMENT, "q, k and v are required");
    } else if (!a->q || !a->k || !a->v || !a->o) {
        return fail(GDR_ERR_INVALID_ARGUMENT, "q, k, v and o are required");
    }

    const int v = a->variant;
    const bool needs_alpha = v != GDR_DELTANET;
    const bool needs_beta = v != GDR_GDN2;
    const bool needs_gates = v == GDR_GDN2;
    if (needs_alpha != (a->alpha != nullptr))
        return fail(GDR_ERR_INVALID_ARGUMENT, needs_alpha ? "alpha is required for this variant"
                                                          : "alpha must be NULL for DeltaNet");
    if (needs_beta != (a->beta != nullptr))
        return fail(GDR_ERR_INVALID_ARGUMENT, needs_beta ? "beta (eta for KLA) is required"
                                                         : "beta must be NULL for GDN-2");
    if (needs_gates != (a->erase_b != nullptr) || needs_gates != (a->write_w != nullptr))
        return fail(GDR_ERR_INVALID_ARGUMENT, needs_gates
                        ? "erase_b and write_w are required for GDN-2"
                        : "erase_b and write_w are only used by GDN-2");
    if (v == GDR_KLA && !(a->eps >= 0.f))
        return fail(GDR_ERR_INVALID_ARGUMENT, "eps must be >= 0");

    const void *ptrs[] = {a->q, a->k, a->v, a->o, a->alpha, a->beta, a->erase_b,
                          a->write_w, a->state_in, a->state_out, a->v_route, a->delta_out};
    const char *names[] = {"q", "k", "v", "o", "alpha", "beta", "erase_b",
                           "write_w", "state_in", "state_out", "v_route", "delta_out"};
    for (int i = 0; i < 12; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(GDR_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
    if (mode == 2) {
        if (a->v_route)
            return fail(GDR_ERR_UNSUPPORTED, "the gradient takes v_route = NULL (pass v + v_route "
                                             "as v; the gradient w.r.t. v_route equals d_v)");
        return GDR_OK;
    }
    if (a->o == a->q || a->o == a->k || a->o == a->v || (a->v_route && a->o == a->v_route))
        return fail(GDR_ERR_INVALID_ARGUMENT, "o must not alias an input");
    if (a->delta_out) {
        const void *others[] = {a->q, a->k, a->v, a->o, a->alpha, a->beta, a->erase_b,
                                a->write_w, a->state_in, a->state_out, a->v_route};
        for (const void *x : others)
            if (x == a->delta_out)
                return fail(GDR_ERR_INVALID_ARGUMENT, "delta_out must not alias another argument");
    }
    return GDR_OK;
}

// The gradient outputs: present exactly for the inputs the variant takes,
// aligned, and distinct from every input and from each other.
gdr_status check_grads(const gdr_args *a, const gdr_grads *g) {
    if (!g) return fail(GDR_ERR_INVALID_ARGUMENT, "grads is NULL");
    const int v = a->variant;
    struct Out { float *p; bool need; const char *name; };
    const Out outs[] = {{g->d_q, true, "d_q"},
                        {g->d_k, true, "d_k"},
                        {g->d_v, true, "d_v"},
                        {g->d_alpha, v != GDR_DELTANET, "d_alpha"},
                        {g->d_beta, v != GDR_GDN2, "d_beta"},
                        {g->d_erase_b, v == GDR_GDN2, "d_erase_b"},
                        {g->d_write_w, v == GDR_GDN2, "d_write_w"}};
    for (const Out &o : outs)
        if (o.need != (o.p != nullptr))
            return fail(GDR_ERR_INVALID_ARGUMENT, o.need ? "%s is required for this variant"
                                                         : "%s must be NULL for this variant",
                        o.name);
    const void *ins[] = {a->q, a->k, a->v, a->alpha, a->beta, a->erase_b, a->write_w,
                         a->state_in, g->d_o, g->d_state_out};
    const void *outp[] = {g->d_q, g->d_k, g->d_v, g->d_alpha, g->d_beta, g->d_erase_b,
                          g->d_write_w, g->d_state_in};
    const char *onames[] = {"d_q", "d_k", "d_v", "d_alpha", "d_beta", "d_erase_b",
                            "d_write_w", "d_state_in"};
    for (int i = 0; i < 8; ++i) {
        if (!outp[i]) continue;
        if (!aligned16(outp[i]))
            return fail(GDR_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", onames[i]);
        for (const void *in : ins)
            if (in && in == outp[i])
                return fail(GDR_ERR_INVALID_ARGUMENT, "%s must not alias an input", onames[i]);
        for (int j = 0; j < i; ++j)
            if (outp[j] == outp[i])
                return fail(GDR_ERR_INVALID_ARGUMENT, "%s and %s are the same buffer",
                            onames[j], onames[i]);
    }
    if ((g->d_o && !aligned16(g->d_o)) || (g->d_state_out && !aligned16(g->d_state_out)))
        return fail(GDR_ERR_INVALID_ARGUMENT, "d_o and d_state_out must be 16-byte aligned");
    return GDR_OK;
}

// A caller's workspace of `need` bytes: present, 256-byte aligned, large enough.
gdr_status check_workspace(const void *workspace, size_t ws_bytes, size_t need) {
    if (!workspace) return fail(GDR_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(GDR_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (ws_bytes < need)
        return fail(GDR_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
    return GDR_OK;
}

gdr::Problem to_problem(const gdr_args *a) {
    gdr::Problem p;
    p.variant = a->variant;
    p.bf16 = a->dtype == GDR_BF16;
    p.B = a->B; p.T = a->T; p.H = a->H; p.dk = a->dk; p.dv = a->dv;
    p.chunk = a->chunk ? a->chunk : 64;
    p.q = a->q; p.k = a->k; p.v = a->v;
    p.alpha = a->alpha; p.beta = a->beta; p.erase_b = a->erase_b; p.write_w = a->write_w;
    p.eps = a->eps;
    p.flags = a->flags;
    p.decay_scale = a->decay_scale;
    p.state_in = a->state_in; p.state_out = a->state_out;
    p.o = a->o;
    p.v_route = a->v_route;
    p.delta_out = a->delta_out;
    return p;
}

}  // namespace

extern "C" {

gdr_status gdr_check_args(const gdr_args *a, int for_decode) { return check(a, for_decode); }

size_t gdr_forward_workspace_size(const gdr_args *a) {
    if (check(a, 0) != GDR_OK) return 0;
    return gdr::forward_workspace_bytes(to_problem(a));
}

gdr_status gdr_forward_chunked(const gdr_args *a, void *workspace, size_t ws_bytes,
                               void *hip_stream) {
    gdr_status s = check(a, 0);
    if (s != GDR_OK) return s;
    gdr::Problem p = to_problem(a);
    size_t need = gdr::forward_workspace_bytes(p);
    if (need > 0) {
        if (!workspace) return fail(GDR_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(GDR_ERR_WORKSPACE, "workspace is not 256-byte aligned");
        if (ws_bytes < need)
            return fail(GDR_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
    }
    hipError_t e = gdr::launch_forward(p, workspace, reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GDR_OK;
}

gdr_status gdr_forward_chunked_noalloc(const gdr_args *a, void *hip_stream) {
    gdr_status s = check(a, 0);
    if (s != GDR_OK) return s;
    gdr::Problem p = to_problem(a);
    p.ws_cap = GDR_NOALLOC_WORKSPACE_MAX;
    const size_t need = gdr::forward_workspace_bytes(p);
    if (need > GDR_NOALLOC_WORKSPACE_MAX)
        return fail(GDR_ERR_WORKSPACE,
                    "this call needs %zu bytes of workspace; the static workspace of "
                    "gdr_forward_chunked_noalloc holds %zu (use gdr_forward_chunked)",
                    need, (size_t)GDR_NOALLOC_WORKSPACE_MAX);
    void *ws = nullptr;
    hipError_t e = noalloc_scratch(&ws);
    if (e != hipSuccess)
        return fail(GDR_ERR_HIP, "static workspace lookup failed: %s", hipGetErrorString(e));
    e = gdr::launch_forward(p, ws, reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GDR_OK;
}

gdr_status gdr_decode_step(const gdr_args *a, void *hip_stream) {
    gdr_status s = check(a, 1);
    if (s != GDR_OK) return s;
    hipError_t e = gdr::launch_decode(to_problem(a), reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GDR_OK;
}

size_t gdr_backward_workspace_size(const gdr_args *a) {
    if (check(a, 2) != GDR_OK) return 0;
    return gdr::backward_workspace_bytes(to_problem(a));
}

gdr_status gdr_backward_chunked(const gdr_args *a, const gdr_grads *g, void *workspace,
                                size_t ws_bytes, void *hip_stream) {
    gdr_status s = check(a, 2);
    if (s != GDR_OK) return s;
    if ((s = check_grads(a, g)) != GDR_OK) return s;
    gdr::Problem p = to_problem(a);
    p.o = nullptr;
    p.state_out = nullptr;
    p.delta_out = nullptr;
    const size_t need = gdr::backward_workspace_bytes(p);
    if ((s = check_workspace(workspace, ws_bytes, need)) != GDR_OK) return s;
    const gdr::Grads gr{g->d_o, g->d_state_out, g->d_q, g->d_k, g->d_v, g->d_alpha,
                        g->d_beta, g->d_erase_b, g->d_write_w, g->d_state_in};
    hipError_t e =
        gdr::launch_backward(p, gr, workspace, false, reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GDR_OK;
}

gdr_status gdr_forward_chunked_save(const gdr_args *a, void *workspace, size_t ws_bytes,
                                    void *hip_stream) {
    gdr_status s = check(a, 0);
    if (s != GDR_OK) return s;
    // what the gradient takes, so that the kept records serve it
    if ((s = check(a, 2)) != GDR_OK) return s;
    if (a->delta_out)
        return fail(GDR_ERR_UNSUPPORTED, "gdr_forward_chunked_save takes delta_out = NULL");
    const gdr::Problem p = to_problem(a);
    const size_t need = gdr::backward_workspace_bytes(p);
    if ((s = check_workspace(workspace, ws_bytes, need)) != GDR_OK) return s;
    hipError_t e = gdr::launch_forward_save(p, workspace, reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GDR_OK;
}

gdr_status gdr_backward_chunked_saved(const gdr_args *a, const gdr_grads *g, void *workspace,
                                      size_t ws_bytes, void *hip_stream) {
    gdr_status s = check(a, 2);
    if (s != GDR_OK) return s;
    if ((s = check_grads(a, g)) != GDR_OK) return s;
    gdr::Problem p = to_problem(a);
    p.o = nullptr;
    p.state_out = nullptr;
    p.delta_out = nullptr;
    const size_t need = gdr::backward_workspace_bytes(p);
    if ((s = check_workspace(workspace, ws_bytes, need)) != GDR_OK) return s;
    const gdr::Grads gr{g->d_o, g->d_state_out, g->d_q, g->d_k, g->d_v, g->d_alpha,
                        g->d_beta, g->d_erase_b, g->d_write_w, g->d_state_in};
    hipError_t e =
        gdr::launch_backward(p, gr, workspace, true, reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GDR_OK;
}

const char *gdr_status_string(int status) {
    switch (status) {
    case GDR_OK: return "GDR_OK";
    case GDR_ERR_INVALID_ARGUMENT: return "GDR_ERR_INVALID_ARGUMENT";
    case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED";
    case GDR_ERR_WORKSPACE: return "GDR_ERR_WORKSPACE";
    case GDR_ERR_HIP: return "GDR_ERR_HIP";
    default: return "unknown gdr_status";
    }
}

const char *gdr_last_error_detail(void) { return g_detail; }

}  // extern "C"
