// decode.hip -- single-token recurrent step of the gated delta rule on gfx950.
//
// Per (b, h) and token: S~ = D S; r = S~^T a; y = S~^T q; delta = u - r;
// S <- S~ + k delta^T; o = S^T q = y + (k . q) delta.  The fixed-size state is
// what makes decode memory constant ("Gated DeltaNet-2: Decoupling Erase and
// Write in Linear Attention", introduction), so the step is a streaming
// read-modify-write of S: 2 * dk * dv * 4 bytes per head against
// ~6 * dk * dv flops.  The kernels are HBM-bound and are built for that:
//
//   * columns of S are independent in this step, so the state is cut into
//     (b, h, 32-column) tiles and each tile belongs to one wave outright;
//   * all of a tile's 16-byte state loads are in flight before any
//     arithmetic, and the column reductions are fused into that single pass
//     and finished with lane butterflies;
//   * the per-token inputs (cold in the cache: a new token every step) are
//     requested before the state (which tends to stay in the last-level
//     cache between steps);
//   * the updated state is written from the same registers: S is read once
//     and written once.
#include "gdr_device.hpp"

namespace gdr {
namespace {

// One (b, h, CW-column) tile of the step, owned by one wave.  Lanes are laid
// out as LPR = CW / 4 lanes per row (one float4 each, so a row segment is one
// whole 128-byte line for CW = 32) and 64 / LPR rows per pass.  Every
// reduction over the key rows (r, y, ||k||^2, k . q) is a butterfly over the
// lanes that share a column group: no LDS, no barrier.  load() only issues
// loads and keeps raw values, so nothing waits on them until finish().
template <int V, typename TI, int DK, int CW> struct DecodeTile {
    using VT = VariantTraits<V>;
    static constexpr int LPR = CW / 4;          // lanes per row
    static constexpr int RPP = kWave / LPR;     // rows per pass
    static constexpr int PASSES = DK / RPP;
    f32x4 s[PASSES];
    TI kraw[PASSES], qraw[PASSES], vr[4];
    float ar[PASSES], dr[PASSES];
    float beta, sdec;
    f32x4 wr;

    __device__ __forceinline__ void load(const Problem &p, long tile, int lane) {
        const int dv = (int)p.dv, tph = dv / CW;
        const long bh = tile / tph;
        const int col0 = (int)(tile % tph) * CW;
        const int cg = lane % LPR, r0 = lane / LPR;
        const TI *q = reinterpret_cast<const TI *>(p.q) + bh * DK;
        const TI *k = reinterpret_cast<const TI *>(p.k) + bh * DK;
#pragma unroll
        for (int i = 0; i < PASSES; ++i) {
            const int row = r0 + i * RPP;
            kraw[i] = k[row];
            qraw[i] = q[row];
            if constexpr (VT::kGates) ar[i] = p.erase_b[bh * DK + row];
            if constexpr (VT::kChannelDecay) dr[i] = p.alpha[bh * DK + row];
        }
        beta = VT::kScalarBeta ? p.beta[bh] : 0.f;
        sdec = (VT::kHasDecay && !VT::kChannelDecay) ? p.alpha[bh] : 1.f;
        const TI *v = reinterpret_cast<const TI *>(p.v) + bh * (long)dv + col0 + 4 * cg;
#pragma unroll
        for (int c = 0; c < 4; ++c) vr[c] = v[c];
        if constexpr (VT::kGates)
            wr = *reinterpret_cast<const f32x4 *>(p.write_w + bh * (long)dv + col0 + 4 * cg);
        const float *Sin = p.state_in + bh * DK * (long)dv + col0 + 4 * cg;
#pragma unroll
        for (int i = 0; i < PASSES; ++i)
            s[i] = *reinterpret_cast<const f32x4 *>(Sin + (long)(r0 + i * RPP) * dv);
    }

    __device__ __forceinline__ void finish(const Problem &p, long tile, int lane) {
        const int dv = (int)p.dv, tph = dv / CW;
        const long bh = tile / tph;
        const int col0 = (int)(tile % tph) * CW;
        const int cg = lane % LPR, r0 = lane / LPR;
        f32x4 u;
#pragma unroll
        for (int c = 0; c < 4; ++c) u[c] = to_f32(vr[c]);
        if constexpr (VT::kGates) u *= wr;
        f32x4 r = zero4(), y = zero4();
        float kn = 0.f, kq = 0.f;
        float kr[PASSES];
#pragma unroll
        for (int i = 0; i < PASSES; ++i) {
            kr[i] = to_f32(kraw[i]);
            const float qq = to_f32(qraw[i]);
            if constexpr (VT::kChannelDecay) s[i] *= dr[i];
            else if constexpr (VT::kHasDecay) s[i] *= sdec;
            const float a = VT::kGates ? ar[i] * kr[i] : kr[i];
            r += a * s[i];
            y += qq * s[i];
            kn += kr[i] * kr[i];
            kq += kr[i] * qq;
        }
#pragma unroll
        for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                r[c] += __shfl_xor(r[c], off, kWave);
                y[c] += __shfl_xor(y[c], off, kWave);
            }
            kn += __shfl_xor(kn, off, kWave);
            kq += __shfl_xor(kq, off, kWave);
        }
        f32x4 dl;
        if constexpr (VT::kGates) {
            dl = u - r;
        } else {
            float bt = beta;
            if constexpr (VT::kKaczmarz) bt = beta / (kn + p.eps);
            dl = bt * (u - r);
        }
        if (r0 == 0) {
            const f32x4 o = y + kq * dl;
            TI *op = reinterpret_cast<TI *>(p.o) + bh * (long)dv + col0 + 4 * cg;
#pragma unroll
            for (int c = 0; c < 4; ++c) op[c] = from_f32<TI>(o[c]);
        }
        float *Sout = p.state_out + bh * DK * (long)dv + col0 + 4 * cg;
#pragma unroll
        for (int i = 0; i < PASSES; ++i)
            *reinterpret_cast<f32x4 *>(Sout + (long)(r0 + i * RPP) * dv) = s[i] + kr[i] * dl;
    }
};

template <int V, typename TI, int DK, int CW, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void decode_wave_kernel(Problem p) {
    using Tile = DecodeTile<V, TI, DK, CW>;
    const long tile = (long)blockIdx.x * WAVES + threadIdx.x / kWave;
    if (tile >= p.B * p.H * (p.dv / CW)) return;
    Tile t;
    t.load(p, tile, threadIdx.x & (kWave - 1));
    t.finish(p, tile, threadIdx.x & (kWave - 1));
}

template <int V, typename TI, int DK>
hipError_t launch_dk(const Problem &p, hipStream_t stream) {
    // 32-column tiles, four independent waves per workgroup.
    constexpr int CW = 32, WAVES = 4;
    const long tiles = p.B * p.H * (p.dv / CW);
    dim3 grid((unsigned)((tiles + WAVES - 1) / WAVES));
    hipLaunchKernelGGL((decode_wave_kernel<V, TI, DK, CW, WAVES>), grid, dim3(WAVES * kWave), 0,
                       stream, p);
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
