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
//     and written once;
//   * the tile's state is addressed through a buffer descriptor of its own
//     (wave-uniform base), one per-lane offset and a uniform offset per row
//     pass, instead of sixteen 64-bit addresses per lane: the kernel stays
//     within 128 registers, so four waves share a SIMD and a batch-64 step's
//     4096 tiles are all resident at once.
#include "gdr_device.hpp"

namespace gdr {
namespace {

// A length-dk vector of the token (k, q, a per-row gate) spread over the 64
// lanes of a wave in 4-byte words, so that it arrives in one or two fully
// coalesced loads, and read back per key row with a lane permute.  fp32:
// word j of lane L holds element L + 64 j.  bf16: lane L holds elements 2L and
// 2L + 1 (lanes beyond dk/2 repeat lower ones).
template <typename X, int DK> struct RowVec {
    static constexpr int NW = sizeof(X) == 4 ? (DK + 63) / 64 : 1;
    uint32_t w[NW];

    __device__ __forceinline__ void load(const X *row, int lane) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(row);
        if constexpr (sizeof(X) == 4) {
#pragma unroll
            for (int j = 0; j < NW; ++j) w[j] = p[(lane + 64 * j) % DK];
        } else {
            w[0] = p[lane % (DK / 2)];
        }
    }
    // Replace every element this lane holds by f(element) (fp32 vectors).
    template <typename F> __device__ __forceinline__ void map(F f) {
        static_assert(sizeof(X) == 4, "fp32 row vectors only");
#pragma unroll
        for (int j = 0; j < NW; ++j) w[j] = __float_as_uint(f(__uint_as_float(w[j])));
    }
    // Element r0 + 8 i, for a lane-dependent r0 in [0, 8) and a compile-time i.
    __device__ __forceinline__ float get(int r0, int i) const {
        if constexpr (sizeof(X) == 4) {
            const int j = i / 8;
            return __uint_as_float((uint32_t)__shfl((int)w[j], r0 + 8 * i - 64 * j, kWave));
        } else {
            const uint32_t x = (uint32_t)__shfl((int)w[0], (r0 >> 1) + 4 * i, kWave);
            return __uint_as_float((r0 & 1) ? (x & 0xffff0000u) : (x << 16));
        }
    }
};

// One (b, h, CW-column) tile of the step, owned by one wave.  Lanes are laid
// out as LPR = CW / 4 lanes per row (one float4 each, so a row segment is one
// whole 128-byte line for CW = 32) and RPP = 64 / LPR consecutive rows per
// pass: one load instruction of the workgroup's four waves covers a contiguous
// run of rows of one head.  Lane (r0, cg) owns rows r0 + RPP i.  Every
// reduction over the key rows (r, y, ||k||^2, k . q) is a butterfly over the
// lanes that share a column group: no LDS, no barrier.  load() only issues
// loads and keeps raw words, so nothing waits on them until finish().
// FL: kQkL2Norm | kRawGates, and kRouteIO when a routed value is added to v
// or the written residual is stored (each pointer may still be NULL).
constexpr int kRouteIO = 4;

template <int V, typename TI, int DK, int CW, int FL> struct DecodeTile {
    static constexpr bool NORM = FL & kQkL2Norm, RAWG = FL & kRawGates, ROUTE = FL & kRouteIO;
    using VT = VariantTraits<V>;
    static constexpr int LPR = CW / 4;          // lanes per row
    static constexpr int RPP = kWave / LPR;     // rows per pass
    static constexpr int PASSES = DK / RPP;
    static_assert(RPP == 8, "row vectors are permuted for eight rows per pass");
    f32x4 s[PASSES];
    RowVec<TI, DK> kv, qv;
    RowVec<float, DK> av, dv_;
    // The four value elements as raw 32-bit words (vx: the routed value).
    static constexpr int VW = (int)sizeof(TI);
    uint32_t vr[VW], vx[ROUTE ? VW : 1];
    float beta, sdec;
    f32x4 wr;

    // bh and col0 are wave-uniform.
    __device__ __forceinline__ void load(const Problem &p, long bh, int col0, int lane) {
        const int dv = (int)p.dv;
        const int cg = lane % LPR, r0 = lane / LPR;
        kv.load(static_cast<const TI *>(p.k) + bh * DK, lane);
        qv.load(static_cast<const TI *>(p.q) + bh * DK, lane);
        if constexpr (VT::kGates) av.load(p.erase_b + bh * DK, lane);
        if constexpr (VT::kChannelDecay) dv_.load(p.alpha + bh * DK, lane);
        beta = VT::kScalarBeta ? p.beta[bh] : 0.f;
        sdec = (VT::kHasDecay && !VT::kChannelDecay) ? p.alpha[bh] : 1.f;
        const TI *v = static_cast<const TI *>(p.v) + bh * (long)dv + col0 + 4 * cg;
#pragma unroll
        for (int w = 0; w < VW; ++w) vr[w] = reinterpret_cast<const uint32_t *>(v)[w];
        if constexpr (ROUTE) {
            const TI *x = p.v_route ? static_cast<const TI *>(p.v_route) + bh * (long)dv + col0 + 4 * cg
                                    : v;
#pragma unroll
            for (int w = 0; w < VW; ++w) vx[w] = reinterpret_cast<const uint32_t *>(x)[w];
        }
        if constexpr (VT::kGates)
            wr = *reinterpret_cast<const f32x4 *>(p.write_w + bh * (long)dv + col0 + 4 * cg);
        // The token's inputs (cold in the cache) are issued before the state:
        // the scheduler must not sink them past the state loads.
        __builtin_amdgcn_sched_barrier(0);
        const auto rs = make_rsrc(p.state_in + bh * DK * (long)dv + col0);
        const unsigned voff = (unsigned)(r0 * dv + 4 * cg) * 4u, pass = (unsigned)(RPP * dv) * 4u;
#pragma unroll
        for (int i = 0; i < PASSES; ++i) {
            typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, i * pass, 0);
            s[i] = __builtin_bit_cast(f32x4, w);
        }
    }

    __device__ __forceinline__ void finish(const Problem &p, long bh, int col0, int lane) {
        const int dv = (int)p.dv;
        const int cg = lane % LPR, r0 = lane / LPR;
        // On-load transforms: gates from pre-activations now; the q/k
        // normalisation, a per-token scalar each, after the reductions below.
        constexpr bool rawg = RAWG;
        const float ds = p.decay_scale;
        // The value words and the write gate are opaque until here, so that
        // their arithmetic (and the wait for them) cannot be hoisted above the
        // state loads.
#pragma unroll
        for (int w = 0; w < VW; ++w) asm volatile("" : "+v"(vr[w]));
        if constexpr (ROUTE)
#pragma unroll
            for (int w = 0; w < VW; ++w) asm volatile("" : "+v"(vx[w]));
        if constexpr (VT::kGates)
#pragma unroll
            for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(wr[c]));
        auto elem = [](const uint32_t *w, int c) {
            if constexpr (sizeof(TI) == 4) return __uint_as_float(w[c]);
            else return __uint_as_float((c & 1) ? (w[c / 2] & 0xffff0000u) : (w[c / 2] << 16));
        };
        f32x4 u;
#pragma unroll
        for (int c = 0; c < 4; ++c) u[c] = elem(vr, c);
        if constexpr (ROUTE)
            if (p.v_route)
#pragma unroll
                for (int c = 0; c < 4; ++c) u[c] += elem(vx, c);
        if constexpr (VT::kGates) {
            if constexpr (rawg)
#pragma unroll
                for (int c = 0; c < 4; ++c) wr[c] = sigmoid_f(wr[c]);
            u *= wr;
        }
        float bet = beta, sd = sdec;
        if constexpr (rawg) {
            if constexpr (VT::kScalarBeta) bet = sigmoid_f(beta);
            if constexpr (VT::kHasDecay && !VT::kChannelDecay) sd = __expf(-ds * softplus_f(sdec));
        }
        if constexpr (rawg) {
            // per-row gates: each lane activates the words it holds
            if constexpr (VT::kChannelDecay) dv_.map([&](float x) { return __expf(-ds * softplus_f(x)); });
            if constexpr (VT::kGates) av.map([](float x) { return sigmoid_f(x); });
        }
        f32x4 r = zero4(), y = zero4();
        float kn = 0.f, kq = 0.f, qn = 0.f;
        float kr[PASSES];
#pragma unroll
        for (int i = 0; i < PASSES; ++i) {
            kr[i] = kv.get(r0, i);
            const float qq = qv.get(r0, i);
            if constexpr (VT::kChannelDecay) s[i] *= dv_.get(r0, i);
            else if constexpr (VT::kHasDecay) s[i] *= sd;
            const float a = VT::kGates ? av.get(r0, i) * kr[i] : kr[i];
            r += a * s[i];
            y += qq * s[i];
            kn += kr[i] * kr[i];
            kq += kr[i] * qq;
            if constexpr (NORM) qn += qq * qq;
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
            if constexpr (NORM) qn += __shfl_xor(qn, off, kWave);
        }
        // k^ = rk k and q^ = rq q: every use of k and q above is linear in
        // each, so the scalars apply to the sums.
        float rk = 1.f;
        if constexpr (NORM) {
            rk = rsqrtf(kn + kL2NormEps);
            const float rq = rsqrtf(qn + kL2NormEps);
            r *= rk;
            y *= rq;
            kq *= rk * rq;
            kn *= rk * rk;
        }
        f32x4 dl;
        if constexpr (VT::kGates) {
            dl = u - r;
        } else {
            float bt = bet;
            if constexpr (VT::kKaczmarz) bt = bet / (kn + p.eps);
            dl = bt * (u - r);
        }
        if (r0 == 0) {
            const f32x4 o = y + kq * dl;
            TI *op = static_cast<TI *>(p.o) + bh * (long)dv + col0 + 4 * cg;
#pragma unroll
            for (int c = 0; c < 4; ++c) op[c] = from_f32<TI>(o[c]);
            if constexpr (ROUTE)
                if (p.delta_out) {
                    TI *dp = static_cast<TI *>(p.delta_out) + bh * (long)dv + col0 + 4 * cg;
#pragma unroll
                    for (int c = 0; c < 4; ++c) dp[c] = from_f32<TI>(dl[c]);
                }
        }
        const auto rs = make_rsrc(p.state_out + bh * DK * (long)dv + col0);
        const unsigned voff = (unsigned)(r0 * dv + 4 * cg) * 4u, pass = (unsigned)(RPP * dv) * 4u;
#pragma unroll
        for (int i = 0; i < PASSES; ++i) {
            typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
            const f32x4 x = s[i] + (kr[i] * rk) * dl;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs, voff, i * pass, 0);
        }
    }
};

// FL: the on-load transforms (kQkL2Norm | kRawGates), one instance each.
template <int V, typename TI, int DK, int CW, int WAVES, int FL>
__global__ __launch_bounds__(WAVES * 64)
void decode_wave_kernel(Problem p) {
    using Tile = DecodeTile<V, TI, DK, CW, FL>;
    // The tile index is wave-uniform; d_v is 64 or 128, so a head has 2 or 4
    // column tiles and the split is a shift.
    const long tile = (long)blockIdx.x * WAVES + __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    if (tile >= p.B * p.H * (p.dv / CW)) return;
    const int sh = p.dv == 128 ? 2 : 1;
    static_assert(CW == 32, "d_v / CW column tiles per head");
    const long bh = tile >> sh;
    const int col0 = (int)(tile & ((1 << sh) - 1)) * CW;
    Tile t;
    t.load(p, bh, col0, threadIdx.x & (kWave - 1));
    t.finish(p, bh, col0, threadIdx.x & (kWave - 1));
}

template <int V, typename TI, int DK>
hipError_t launch_dk(const Problem &p, hipStream_t stream) {
    // 32-column tiles, four independent waves per workgroup.
    constexpr int CW = 32, WAVES = 4;
    const long tiles = p.B * p.H * (p.dv / CW);
    dim3 grid((unsigned)((tiles + WAVES - 1) / WAVES));
    const int fl = (p.flags & (kQkL2Norm | kRawGates)) |
                   ((p.v_route || p.delta_out) ? kRouteIO : 0);
    switch (fl) {
    case kRouteIO:
        hipLaunchKernelGGL((decode_wave_kernel<V, TI, DK, CW, WAVES, kRouteIO>), grid,
                           dim3(WAVES * kWave), 0, stream, p);
        break;
    case kRouteIO | kQkL2Norm:
        hipLaunchKernelGGL((decode_wave_kernel<V, TI, DK, CW, WAVES, kRouteIO | kQkL2Norm>), grid,
                           dim3(WAVES * kWave), 0, stream, p);
        break;
    case kRouteIO | kRawGates:
        hipLaunchKernelGGL((decode_wave_kernel<V, TI, DK, CW, WAVES, kRouteIO | kRawGates>), grid,
                           dim3(WAVES * kWave), 0, stream, p);
        break;
    case kRouteIO | kQkL2Norm | kRawGates:
        hipLaunchKernelGGL(
            (decode_wave_kernel<V, TI, DK, CW, WAVES, kRouteIO | kQkL2Norm | kRawGates>), grid,
            dim3(WAVES * kWave), 0, stream, p);
        break;
    case 0:
        hipLaunchKernelGGL((decode_wave_kernel<V, TI, DK, CW, WAVES, 0>), grid, dim3(WAVES * kWave),
                           0, stream, p);
        break;
    case kQkL2Norm:
        hipLaunchKernelGGL((decode_wave_kernel<V, TI, DK, CW, WAVES, kQkL2Norm>), grid,
                           dim3(WAVES * kWave), 0, stream, p);
        break;
    case kRawGates:
        hipLaunchKernelGGL((decode_wave_kernel<V, TI, DK, CW, WAVES, kRawGates>), grid,
                           dim3(WAVES * kWave), 0, stream, p);
        break;
    default:
        hipLaunchKernelGGL((decode_wave_kernel<V, TI, DK, CW, WAVES, kQkL2Norm | kRawGates>), grid,
                           dim3(WAVES * kWave), 0, stream, p);
        break;
    }
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
