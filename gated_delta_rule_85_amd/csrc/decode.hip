// decode.hip -- single-token recurrent step of the gated delta rule on gfx950.
//
// Per (b, h) and token: S~ = D S; r = S~^T a; y = S~^T q; delta = u - r;
// S <- S~ + k delta^T; o = S^T q = y + (k . q) delta.  The fixed-size state is
// what makes decode memory constant ("Gated DeltaNet-2: Decoupling Erase and
// Write in Linear Attention", introduction), so the step is a streaming
// read-modify-write of S: 2 * dk * dv * 4 bytes per head against
// ~4 * dk * dv flops.  The kernel is HBM-bound and is built for that:
//
//   * one workgroup per (b, h, slice of COLS value columns); columns of S are
//     independent in this step, so slices need no communication;
//   * each thread owns a 4-column float4 strip of DK / rows-per-pass rows and
//     issues all its 16-byte loads before any arithmetic (deep memory-level
//     parallelism, every row segment read as whole 64-byte runs);
//   * the two column reductions r and y are fused into the single pass over
//     S held in registers, reduced across lanes with shuffles and across
//     waves through LDS;
//   * the updated state is written from the same registers, so S is read once
//     and written once.
#include "gdr_device.hpp"

namespace gdr {
namespace {

constexpr int kThreads = 256;

template <int V, typename TI, int DK, int COLS>
__global__ __launch_bounds__(kThreads) void decode_kernel(Problem p) {
    using VT = VariantTraits<V>;
    constexpr int TPR = COLS / 4;          // threads covering one row slice
    constexpr int RPP = kThreads / TPR;    // rows per pass
    constexpr int PASSES = DK / RPP;
    constexpr int NWAVE = kThreads / kWave;
    constexpr int LANES_PER_COLGROUP = kWave / TPR;  // lanes sharing a column group in a wave
    static_assert(DK % RPP == 0, "row tiling");

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int H = (int)p.H;
    const int dv = (int)p.dv;
    const int col0 = blockIdx.x * COLS;
    const long bh = (long)b * H + h;       // T == 1: token index == (b, h)

    const int cg = tid % TPR;              // column group: columns col0 + 4*cg .. +3
    const int r0 = tid / TPR;              // first row
    const float *Sin = p.state_in + bh * DK * (long)dv + col0 + 4 * cg;
    float *Sout = p.state_out + bh * DK * (long)dv + col0 + 4 * cg;

    // Issue every state load first.
    f32x4 s[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i)
        s[i] = *reinterpret_cast<const f32x4 *>(Sin + (long)(r0 + i * RPP) * dv);

    __shared__ float sh_q[DK], sh_k[DK], sh_a[DK], sh_dec[DK];
    __shared__ float sh_u[COLS], sh_delta[COLS];
    __shared__ float sh_red[2][NWAVE][COLS];
    __shared__ float sh_scal[2];

    const TI *q = reinterpret_cast<const TI *>(p.q) + bh * DK;
    const TI *k = reinterpret_cast<const TI *>(p.k) + bh * DK;
    const TI *v = reinterpret_cast<const TI *>(p.v) + bh * (long)dv + col0;
    float beta = 0.f;
    if constexpr (VT::kScalarBeta) beta = p.beta[bh];

    if (tid < DK) {
        float kk = to_f32(k[tid]);
        sh_q[tid] = to_f32(q[tid]);
        sh_k[tid] = kk;
        if constexpr (VT::kGates) sh_a[tid] = p.erase_b[bh * DK + tid] * kk;
        if constexpr (VT::kChannelDecay) sh_dec[tid] = p.alpha[bh * DK + tid];
    } else if (tid >= 128 && tid < 128 + COLS) {
        int j = tid - 128;
        float vv = to_f32(v[j]);
        if constexpr (VT::kGates)
            sh_u[j] = p.write_w[bh * (long)dv + col0 + j] * vv;
        else
            sh_u[j] = vv;  // scaled by beta below (KLA needs ||k|| first)
    }
    __syncthreads();

    // Wave 0: ||k||^2 and k . q over the key dimension.
    if (wave == 0) {
        float kn = 0.f, kq = 0.f;
#pragma unroll
        for (int i = lane; i < DK; i += kWave) {
            kn += sh_k[i] * sh_k[i];
            kq += sh_k[i] * sh_q[i];
        }
        kn = wave_sum(kn);
        kq = wave_sum(kq);
        if (lane == 0) {
            sh_scal[0] = kn;
            sh_scal[1] = kq;
        }
    }

    float sdec = 1.f;
    if constexpr (VT::kHasDecay && !VT::kChannelDecay) sdec = p.alpha[bh];

    // Decay in registers, then the fused column reductions.  For scalar-beta
    // variants r accumulates k . S~ and is scaled by beta afterwards.
    f32x4 r = zero4(), y = zero4();
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const int row = r0 + i * RPP;
        float d = 1.f;
        if constexpr (VT::kChannelDecay) d = sh_dec[row];
        else if constexpr (VT::kHasDecay) d = sdec;
        if constexpr (VT::kHasDecay) s[i] *= d;
        float ar;
        if constexpr (VT::kGates) ar = sh_a[row];
        else ar = sh_k[row];
        const float qr = sh_q[row];
        r += ar * s[i];
        y += qr * s[i];
    }
    // Lanes tid, tid + TPR, ... within a wave share a column group.
#pragma unroll
    for (int off = TPR; off < kWave; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            r[c] += __shfl_xor(r[c], off, kWave);
            y[c] += __shfl_xor(y[c], off, kWave);
        }
    }
    if (lane < TPR) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            sh_red[0][wave][4 * cg + c] = r[c];
            sh_red[1][wave][4 * cg + c] = y[c];
        }
    }
    __syncthreads();
    (void)LANES_PER_COLGROUP;

    if (tid < COLS) {
        float rr = 0.f, yy = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) {
            rr += sh_red[0][w][tid];
            yy += sh_red[1][w][tid];
        }
        float bt = beta;
        if constexpr (VT::kKaczmarz) bt = beta / (sh_scal[0] + p.eps);
        float delta;
        if constexpr (VT::kGates) delta = sh_u[tid] - rr;
        else delta = bt * (sh_u[tid] - rr);
        sh_delta[tid] = delta;
        const float o = yy + sh_scal[1] * delta;
        TI *op = reinterpret_cast<TI *>(p.o) + bh * (long)dv + col0 + tid;
        *op = from_f32<TI>(o);
    }
    __syncthreads();

    f32x4 dl;
#pragma unroll
    for (int c = 0; c < 4; ++c) dl[c] = sh_delta[4 * cg + c];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const int row = r0 + i * RPP;
        f32x4 out = s[i] + sh_k[row] * dl;
        *reinterpret_cast<f32x4 *>(Sout + (long)row * dv) = out;
    }
}

template <int V, typename TI, int DK>
hipError_t launch_dk(const Problem &p, hipStream_t stream) {
    constexpr int COLS = 64;
    dim3 grid((unsigned)(p.dv / COLS), (unsigned)p.H, (unsigned)p.B);
    hipLaunchKernelGGL((decode_kernel<V, TI, DK, COLS>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int V, typename TI>
hipError_t launch_t(const Problem &p, hipStream_t stream) {
    return p.dk == 128 ? launch_dk<V, TI, 128>(p, stream) : launch_dk<V, TI, 64>(p, stream);
}

template <int V>
hipError_t launch_v(const Problem &p, hipStream_t stream) {
    return p.bf16 ? launch_t<V, bf16>(p, stream) : launch_t<V, float>(p, stream);
}

}  // namespace

hipError_t launch_decode(const Problem &p, hipStream_t stream) {
    switch (p.variant) {
    case kDeltaNet: return launch_v<kDeltaNet>(p, stream);
    case kGatedDeltaNet: return launch_v<kGatedDeltaNet>(p, stream);
    case kKDA: return launch_v<kKDA>(p, stream);
    case kGDN2: return launch_v<kGDN2>(p, stream);
    case kKLA: return launch_v<kKLA>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdr
