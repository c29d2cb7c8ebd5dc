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
    // The largest forward workspace the caller holds (0 = any size): a plan
    // that would need more is not taken.
    size_t ws_cap = 0;
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
// The gradient's states pass: the factors of every chunk (prep), then the
// scan from s_in (NULL = zeros) to s_out (NULL = dropped), recording the state
// entering each chunk ([B*H][NC][dk][dv] in s_chunks) and each chunk's
// Delta = U~ - W S ([B*H][NC][C][dv] in d_chunks), both in the input dtype.
// with_o: the scan also writes p.o (the forward that keeps what its gradient
// needs); otherwise no outputs.  Long bf16 sequences run in blocks of 64
// chunks as the forward does, each launch running the scan of one block beside
// the prep of the next; that takes B*H*dk*dv*4 bytes (rounded up to 256) + 256
// bytes of scratch, free for the duration of the call, for the state carried
// between blocks and the prep's ticket counter (one pass without it).  Where
// the forward runs in segments (forward_segments), so does this pass, its
// segments' arrays in the scratch.
hipError_t launch_states_pass(const Problem &p, void *workspace, const float *s_in, float *s_out,
                              void *s_chunks, void *d_chunks, bool with_o, void *scratch,
                              size_t scratch_bytes, hipStream_t stream);

// The sequence segments the bf16 forward takes for p (few heads per device:
// the chain's column slices at most a quarter of the compute units), or 0:
// the number of segments, each of *L chunks but the last, shorter one.
long forward_segments(const Problem &p, long *L);
// The segments' serial combine: from s0 (NULL = zeros), S_{j+1} = M_j S_j + N_j
// for j = 0 .. nseg - 2, with M [nseg-1][B*H][dk][dk], N and Sst
// [nseg-1][B*H][dk][dv] (fp32); S_{j+1} is written to Sst[j].
hipError_t launch_segment_combine(const Problem &p, const float *s0, long nseg, const float *M,
                                  const float *N, float *Sst, hipStream_t stream);

// Gradient of the chunked forward: upstream gradients in, input gradients out.
struct Grads {
    const void *d_o;            // [B,T,H,dv] input dtype, or NULL
    const float *d_state_out;   // [B,H,dk,dv] or NULL
    float *d_q, *d_k, *d_v, *d_alpha, *d_beta, *d_erase_b, *d_write_w, *d_state_in;
};
size_t backward_workspace_bytes(const Problem &p);
// saved: the workspace already holds the factors and the per-chunk states of
// p (left by launch_forward_save), so the states pass is skipped.
hipError_t launch_backward(const Problem &p, const Grads &g, void *workspace, bool saved,
                           hipStream_t stream);
// The chunked forward as one pass that leaves in the gradient's workspace the
// factors of every chunk and the state and Delta entering each (the gradient's
// states pass, with the outputs written too).
hipError_t launch_forward_save(const Problem &p, void *workspace, hipStream_t stream);

}  // namespace gdr
