// gdr_kernels.hpp -- internal interface between the C-ABI host layer
// (gdr_host.cpp) and the kernel translation units.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

enum Variant { kDeltaNet = 0, kGatedDeltaNet = 1, kKDA = 2, kGDN2 = 3, kKLA = 4 };

// Compile-time facts of a variant.
template <int V> struct VariantTraits {
    static constexpr bool kHasDecay = V != kDeltaNet;
    static constexpr bool kChannelDecay = V == kKDA || V == kGDN2;
    static constexpr bool kScalarBeta = V != kGDN2;     // beta (or eta) per token
    static constexpr bool kKaczmarz = V == kKLA;        // beta = eta / (||k||^2 + eps)
    static constexpr bool kGates = V == kGDN2;          // erase b [dk], write w [dv]
};

// Input transforms applied on load (the values of the C ABI's gdr_flag).
constexpr int kQkL2Norm = 1, kRawGates = 2;
constexpr float kL2NormEps = 1e-6f;   // added to sum_i x_i^2 before the square root

// Everything a kernel needs about one call; pointers are device memory.
struct Problem {
    int variant;
    int bf16;            // 1: q, k, v, o are bfloat16; 0: float32
    int64_t B, T, H, dk, dv;
    int chunk;
    const void *q, *k, *v;
    const float *alpha, *beta, *erase_b, *write_w;
    float eps;
    int flags;           // kQkL2Norm | kRawGates
    float decay_scale;   // s in exp(-s softplus(alpha)) with kRawGates
    const float *state_in;
    float *state_out;
    void *o;
    const void *v_route;   // added to v as it is loaded (NULL = none)
    void *delta_out;       // per-token written residual delta_t (NULL = not written)
};

// Decode step (T == 1).  Returns the launch status.
hipError_t launch_decode(const Problem &p, hipStream_t stream);

// Chunked forward.
size_t forward_workspace_bytes(const Problem &p);
hipError_t launch_forward(const Problem &p, void *workspace, hipStream_t stream);

// The chunked forward's per-chunk factors (in the input dtype, fragment-major
// per chunk-head; chunk-head index = (b * H + h) * nbmax + c) for all
// nbmax = ceil(T / C) chunks of every head, as the gradient needs them.
struct ForwardStates {
    const void *W, *Ut, *Qt, *Kbt, *P;
    const float *gam;
    long nbmax;
};
size_t forward_states_bytes(const Problem &p);
ForwardStates forward_states_ptrs(const Problem &p, void *workspace);
// The gradient's states pass, one block of chunks [c0, c0 + nc) at a time:
// the factors of the block (prep), then the scan over it from s_in (NULL =
// zeros) to s_out (NULL = dropped), recording the state entering each chunk
// ([B*H][nbmax][dk][dv] in s_chunks) and each chunk's Delta = U~ - W S
// ([B*H][nbmax][C][dv] in d_chunks), both in the input dtype.  No outputs.
hipError_t launch_states_prep(const Problem &p, void *workspace, long c0, int nc, bool concurrent,
                              hipStream_t stream);
hipError_t launch_states_scan(const Problem &p, void *workspace, long c0, int nc,
                              const float *s_in, float *s_out, void *s_chunks, void *d_chunks,
                              hipStream_t stream);

// Gradient of the chunked forward: upstream gradients in, input gradients out.
struct Grads {
    const void *d_o;            // [B,T,H,dv] input dtype, or NULL
    const float *d_state_out;   // [B,H,dk,dv] or NULL
    float *d_q, *d_k, *d_v, *d_alpha, *d_beta, *d_erase_b, *d_write_w, *d_state_in;
};
size_t backward_workspace_bytes(const Problem &p);
hipError_t launch_backward(const Problem &p, const Grads &g, void *workspace, hipStream_t stream);

}  // namespace gdr
