// backward.hip -- gradient of the chunked gated delta-rule forward on gfx950.
//
// With the chunk form of the forward (per chunk of C = 64 tokens, incoming
// state S, g_r = sum_{j<=r} log alpha_j per key channel, g_C its last row):
//     A = strict_lower(Gram(a, k)),  P = lower(Gram(q, k)),
//     Gram(X, Y)[r][s] = sum_i X[r][i] Y[s][i] e^{g_r[i] - g_s[i]},
//     T = (I + A)^{-1},  W = T (a (.) e^g),  U~ = T u,  Delta = U~ - W S,
//     O = (q (.) e^g) S + P Delta,  S' = Diag(e^{g_C}) S + (k (.) e^{g_C - g})^T Delta,
// the gradient of a loss with upstream dO and dS' runs backwards over the
// chunks (the only sequential part):
//     dDelta = P^T dO + Kbar dS',   dS = Qt^T dO + Diag(e^{g_C}) dS' - W^T dDelta,
// and then, for every chunk independently, through the chunk's factors:
//     dQt = dO S^T, dKbar = Delta dS'^T, dW = -dDelta S^T, dP = dO Delta^T,
//     dT = dW At^T + dDelta u^T, dAt = T^T dW, du = T^T dDelta,
//     dA = -strict_lower(T^T dT T^T), and the Gram products' own backward,
// ending in the element-wise chain rule to q, k, the erase/write vectors and
// the decay (a reverse cumulative sum of dg over the chunk, since g restarts
// in every chunk).  This is the chain rule through the same closed form the
// forward uses ("Gated DeltaNet-2", technical core: the chunkwise WY algorithm;
// "Kaczmarz Linear Attention", Implementation: only B = Diag(beta) changes per
// variant).  The derivation and the kernels are our own.
//
// Three launches after the forward's own factors and per-chunk states
// (launch_forward_states):
//   reverse_scan_kernel   one workgroup per (16 value columns, h, b): the
//                         sequential pass; records dS' and dDelta per chunk.
//   chunk_grad_kernel     persistent workgroups over chunk-heads: the rest, in
//                         fp32 on the matrix cores (16x16x4) with the chunk's
//                         intermediates in a per-workgroup global scratch slot.
#include "gdr_device.hpp"

namespace gdr {
namespace {

constexpr int C = kChunk;
constexpr int kXcds = 8;

template <typename T> __device__ __forceinline__ float f32(T x) { return to_f32(x); }

// acc += A B over one 16x16 tile at (m0, n0) on fp32 matrix cores; A(m, k) and
// B(k, n) return operand elements.  A lane supplies row l16 / K-element lg of
// A and K-element lg / column l16 of B, and holds rows 4 lg .. 4 lg + 3 of
// column l16 of the result.  All operand reads of four K-steps go out first.
template <int K, typename FA, typename FB>
__device__ __forceinline__ f32x4 mm_tile(FA A, FB B, int m0, int n0, int l16, int lg, f32x4 acc) {
    static_assert(K % 16 == 0, "K in steps of 16");
#pragma unroll 2
    for (int k0 = 0; k0 < K; k0 += 16) {
        float a[4], b[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            a[s] = A(m0 + l16, k0 + 4 * s + lg);
            b[s] = B(k0 + 4 * s + lg, n0 + l16);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    }
    return acc;
}

// ============================================================================
// reverse scan
// ============================================================================
constexpr int kRevThreads = 256;

template <typename TI, int DK, int DV>
__global__ __launch_bounds__(kRevThreads) void reverse_scan_kernel(Problem p, ForwardStates f,
                                                                   Grads g, float *dS_chunks,
                                                                   float *dDelta) {
    constexpr int NS = DV / 16;
    __shared__ float sdS[DK][17], sdO[C][17], sdD[C][17];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int H = (int)p.H;
    const long T = p.T, NC = f.nbmax;
    const long nwg = p.B * p.H * NS;
    const long per_xcd = (nwg + kXcds - 1) / kXcds;
    const long logical = (long)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= nwg) return;
    const long bh = logical / NS;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int col0 = (int)(logical % NS) * 16;
    const TI *W = static_cast<const TI *>(f.W), *Qt = static_cast<const TI *>(f.Qt);
    const TI *Kbt = static_cast<const TI *>(f.Kbt), *P = static_cast<const TI *>(f.P);
    const TI *dO = static_cast<const TI *>(g.d_o);

    for (int idx = tid; idx < DK * 16; idx += kRevThreads) {
        const int i = idx / 16, j = idx % 16;
        sdS[i][j] = g.d_state_out ? g.d_state_out[(bh * DK + i) * DV + col0 + j] : 0.f;
    }
    __syncthreads();
    for (long c = NC - 1; c >= 0; --c) {
        const long ch = bh * NC + c;
        // dO of this chunk's rows (zero past T and without upstream); record
        // the gradient with respect to the state leaving the chunk.
        for (int idx = tid; idx < C * 16; idx += kRevThreads) {
            const int r = idx / 16, j = idx % 16;
            const long t = c * C + r;
            sdO[r][j] = (dO && t < T) ? f32(dO[((b * T + t) * H + h) * DV + col0 + j]) : 0.f;
        }
        for (int idx = tid; idx < DK * 16; idx += kRevThreads) {
            const int i = idx / 16, j = idx % 16;
            dS_chunks[(ch * DK + i) * DV + col0 + j] = sdS[i][j];
        }
        __syncthreads();
        {   // dDelta = Kbar dS' + P^T dO: one 16-row tile per wave
            const int m0 = 16 * wave;
            f32x4 acc = zero4();
            acc = mm_tile<DK>([&](int r, int i) { return f32(Kbt[ch * DK * C + frag_off<TI>(i, r, C)]); },
                              [&](int i, int n) { return sdS[i][n]; }, m0, 0, l16, lg, acc);
            acc = mm_tile<C>([&](int r, int s) { return f32(P[ch * C * C + frag_off<TI>(s, r, C)]); },
                             [&](int s, int n) { return sdO[s][n]; }, m0, 0, l16, lg, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = m0 + 4 * lg + i;
                sdD[r][l16] = acc[i];
                dDelta[(ch * C + r) * DV + col0 + l16] = acc[i];
            }
        }
        __syncthreads();
        // dS = Diag(e^{g_C}) dS' + Qt^T dO - W^T dDelta
        constexpr int NU = DK / 64;
        f32x4 nd[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int m0 = 16 * (wave + 4 * u);
            f32x4 aq = zero4(), aw = zero4();
            aq = mm_tile<C>([&](int i, int s) { return f32(Qt[ch * C * DK + frag_off<TI>(s, i, DK)]); },
                            [&](int s, int n) { return sdO[s][n]; }, m0, 0, l16, lg, aq);
            aw = mm_tile<C>([&](int i, int r) { return f32(W[ch * C * DK + frag_off<TI>(r, i, DK)]); },
                            [&](int r, int n) { return sdD[r][n]; }, m0, 0, l16, lg, aw);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + 4 * lg + i;
                nd[u][i] = f.gam[ch * DK + row] * sdS[row][l16] + aq[i] - aw[i];
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) sdS[16 * (wave + 4 * u) + 4 * lg + i][l16] = nd[u][i];
        __syncthreads();
    }
    if (g.d_state_in)
        for (int idx = tid; idx < DK * 16; idx += kRevThreads) {
            const int i = idx / 16, j = idx % 16;
            g.d_state_in[(bh * DK + i) * DV + col0 + j] = sdS[i][j];
        }
}

// ============================================================================
// per-chunk gradient
// ============================================================================
constexpr int kGradThreads = 256;

// fp32 intermediates of one chunk-head, row-major, in one workgroup's slot.
template <int DK, int DV> struct GradSlot {
    enum { Xq, Xa, Xk, Qg, Ag, Kb, Wm, dQt, dKb, dWm, dAg, dXq, dXa, dXk, G, NCK };   // C x DK
    enum { Uu, Dl, dUu, NCV };                                                            // C x DV
    enum { Am, Pm, Tm, Dm, dTm, dPm, dAm, Ym, NCC };                                      // C x C
    static constexpr long kCK = (long)C * DK, kCV = (long)C * DV, kCC = (long)C * C;
    // vectors: per-row beta, per-row |k|^2, dgam (DK), row/column decay sums (2 C)
    static constexpr long kVec = 4 * C + DK;
    static constexpr long kFloats = NCK * kCK + NCV * kCV + NCC * kCC + kVec;
    float *base;
    __device__ float *ck(int which) const { return base + which * kCK; }
    __device__ float *cv(int which) const { return base + NCK * kCK + which * kCV; }
    __device__ float *cc(int which) const { return base + NCK * kCK + NCV * kCV + which * kCC; }
    __device__ float *vec() const { return base + NCK * kCK + NCV * kCV + NCC * kCC; }
};

template <int V, typename TI, int DK, int DV>
__global__ __launch_bounds__(kGradThreads) void chunk_grad_kernel(Problem p, Grads g,
                                                                 const float *S_chunks,
                                                                 const float *dS_chunks,
                                                                 const float *dDelta,
                                                                 float *scratch) {
    using VT = VariantTraits<V>;
    using Slot = GradSlot<DK, DV>;
    constexpr int NT = kGradThreads;
    constexpr bool kRowDecay = VT::kHasDecay && !VT::kChannelDecay;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int H = (int)p.H;
    const long T = p.T, NC = (p.T + C - 1) / C;
    const long nitems = NC * p.H * p.B;
    const Slot sl{scratch + (long)blockIdx.x * Slot::kFloats};
    const TI *q = static_cast<const TI *>(p.q), *k = static_cast<const TI *>(p.k);
    const TI *v = static_cast<const TI *>(p.v), *dO = static_cast<const TI *>(g.d_o);
    float *Xq = sl.ck(Slot::Xq), *Xa = sl.ck(Slot::Xa), *Xk = sl.ck(Slot::Xk);
    float *Qg = sl.ck(Slot::Qg), *Ag = sl.ck(Slot::Ag), *Kb = sl.ck(Slot::Kb), *Wm = sl.ck(Slot::Wm);
    float *dQt = sl.ck(Slot::dQt), *dKb = sl.ck(Slot::dKb), *dWm = sl.ck(Slot::dWm);
    float *dAg = sl.ck(Slot::dAg), *dXq = sl.ck(Slot::dXq), *dXa = sl.ck(Slot::dXa);
    float *dXk = sl.ck(Slot::dXk), *Gd = sl.ck(Slot::G);
    float *Uu = sl.cv(Slot::Uu), *Dl = sl.cv(Slot::Dl), *dUu = sl.cv(Slot::dUu);
    float *Am = sl.cc(Slot::Am), *Pm = sl.cc(Slot::Pm), *Tm = sl.cc(Slot::Tm), *Dm = sl.cc(Slot::Dm);
    float *dTm = sl.cc(Slot::dTm), *dPm = sl.cc(Slot::dPm), *dAm = sl.cc(Slot::dAm), *Ym = sl.cc(Slot::Ym);
    float *vbeta = sl.vec(), *vkn = vbeta + C, *vdgam = vkn + C, *vrow = vdgam + DK, *vcol = vrow + C;
    constexpr int GW = VT::kChannelDecay ? DK : 1;   // columns of g in use
    __shared__ float sA[C][C + 1], sT[C][C + 1];

    for (long item = blockIdx.x; item < nitems; item += gridDim.x) {
        const long c = item % NC, bh = item / NC;
        const int b = (int)(bh / H), h = (int)(bh % H);
        const long t0 = c * C;
        const int nvalid = (int)min((long)C, T - t0);
        const long ch = bh * NC + c;
        const float *S = S_chunks + ch * DK * DV;
        const float *dSp = dS_chunks + ch * DK * DV;
        const float *dD = dDelta + ch * C * DV;
        auto tok = [&](int r) -> long { return ((long)b * T + t0 + r) * H + h; };

        __syncthreads();   // the previous item is done with the slot
        // ---- E0: decay prefix sums, step sizes ------------------------------
        for (int i = tid; i < GW; i += NT) {
            float gg = 0.f;
            for (int r = 0; r < C; ++r) {
                if (VT::kHasDecay && r < nvalid)
                    gg += logf(VT::kChannelDecay ? p.alpha[tok(r) * DK + i] : p.alpha[tok(r)]);
                Gd[r * DK + i] = gg;
            }
        }
        for (int r = wave; r < C; r += NT / kWave) {
            float s2 = 0.f;
            if (r < nvalid)
                for (int i = lane; i < DK; i += kWave) {
                    const float x = f32(k[tok(r) * DK + i]);
                    s2 += x * x;
                }
            s2 = wave_sum(s2);
            if (lane == 0) {
                vkn[r] = s2;
                float bt = 0.f;
                if constexpr (VT::kScalarBeta) {
                    bt = r < nvalid ? p.beta[tok(r)] : 0.f;
                    if constexpr (VT::kKaczmarz) bt = bt / (s2 + p.eps);
                }
                vbeta[r] = bt;
            }
        }
        __syncthreads();
        // ---- E0b: element-wise operands ---------------------------------------
        for (int idx = tid; idx < C * DK; idx += NT) {
            const int r = idx / DK, i = idx % DK;
            const int gi = VT::kChannelDecay ? i : 0;
            const bool ok = r < nvalid;
            const float qq = ok ? f32(q[tok(r) * DK + i]) : 0.f;
            const float kk = ok ? f32(k[tok(r) * DK + i]) : 0.f;
            float aa;
            if constexpr (VT::kGates) aa = ok ? p.erase_b[tok(r) * DK + i] * kk : 0.f;
            else aa = vbeta[r] * kk;
            const float gr = Gd[r * DK + gi], gC = Gd[(C - 1) * DK + gi], gm = Gd[(C / 2 - 1) * DK + gi];
            if constexpr (VT::kChannelDecay) {
                Xq[idx] = qq * __expf(gr - gm);
                Xa[idx] = aa * __expf(gr - gm);
                Xk[idx] = kk * __expf(gm - gr);
            } else {
                Xq[idx] = qq;
                Xa[idx] = aa;
                Xk[idx] = kk;
            }
            const float eg = __expf(gr);
            Qg[idx] = qq * eg;
            Ag[idx] = aa * eg;
            Kb[idx] = kk * __expf(gC - gr);
        }
        for (int idx = tid; idx < C * DV; idx += NT) {
            const int r = idx / DV, j = idx % DV;
            const bool ok = r < nvalid;
            const float vv = ok ? f32(v[tok(r) * DV + j]) : 0.f;
            if constexpr (VT::kGates) Uu[idx] = ok ? p.write_w[tok(r) * DV + j] * vv : 0.f;
            else Uu[idx] = vbeta[r] * vv;
        }
        if constexpr (kRowDecay)
            for (int idx = tid; idx < C * C; idx += NT) {
                const int r = idx / C, s = idx % C;
                Dm[idx] = s <= r ? __expf(Gd[r * DK] - Gd[s * DK]) : 0.f;
            }
        __syncthreads();
        // ---- E1: A and P ------------------------------------------------------
        for (int t = wave; t < 32; t += NT / kWave) {
            const bool isP = t >= 16;
            const int tt = t & 15, m0 = 16 * (tt / 4), n0 = 16 * (tt % 4);
            const float *X = isP ? Xq : Xa;
            f32x4 acc = mm_tile<DK>([&](int m, int kk) { return X[m * DK + kk]; },
                                    [&](int kk, int n) { return Xk[n * DK + kk]; }, m0, n0, l16, lg,
                                    zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = m0 + 4 * lg + i, s = n0 + l16;
                float val = acc[i];
                if constexpr (kRowDecay) val *= Dm[r * C + s];
                val = isP ? (s <= r ? val : 0.f) : (s < r ? val : 0.f);
                (isP ? Pm : Am)[r * C + s] = val;
            }
        }
        __syncthreads();
        // ---- E2: T = (I + A)^{-1} by forward substitution in LDS, one column
        // per thread: T[r][c] = [r == c] - sum_{c <= s < r} A[r][s] T[s][c].
        for (int idx = tid; idx < C * C; idx += NT) sA[idx / C][idx % C] = Am[idx];
        __syncthreads();
        if (tid < C) {
            const int cc = tid;
            for (int r = 0; r < C; ++r) {
                float acc = r == cc ? 1.f : 0.f;
                for (int s = cc; s < r; ++s) acc -= sA[r][s] * sT[s][cc];
                sT[r][cc] = acc;
            }
        }
        __syncthreads();
        for (int idx = tid; idx < C * C; idx += NT) Tm[idx] = sT[idx / C][idx % C];
        __syncthreads();
        // ---- E3: W = T At, U~ = T u, then Delta = U~ - W S ----------------------
        for (int t = wave; t < 4 * (DK / 16) + 4 * (DV / 16); t += NT / kWave) {
            const bool isU = t >= 4 * (DK / 16);
            const int tt = isU ? t - 4 * (DK / 16) : t;
            const int ncol = isU ? DV / 16 : DK / 16;
            const int m0 = 16 * (tt / ncol), n0 = 16 * (tt % ncol);
            const float *Bsrc = isU ? Uu : Ag;
            const int ld = isU ? DV : DK;
            f32x4 acc = mm_tile<C>([&](int m, int s) { return Tm[m * C + s]; },
                                   [&](int s, int n) { return Bsrc[s * ld + n]; }, m0, n0, l16, lg,
                                   zero4());
            float *dst = isU ? Dl : Wm;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(m0 + 4 * lg + i) * ld + n0 + l16] = acc[i];
        }
        __syncthreads();
        for (int t = wave; t < 4 * (DV / 16); t += NT / kWave) {
            const int m0 = 16 * (t / (DV / 16)), n0 = 16 * (t % (DV / 16));
            f32x4 acc = mm_tile<DK>([&](int m, int i) { return Wm[m * DK + i]; },
                                    [&](int i, int n) { return S[i * DV + n]; }, m0, n0, l16, lg,
                                    zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) Dl[(m0 + 4 * lg + i) * DV + n0 + l16] -= acc[i];
        }
        __syncthreads();
        // ---- E4: contractions over the value channels ------------------------
        auto dOf = [&](int r, int j) -> float {
            return (dO && r < nvalid) ? f32(dO[tok(r) * DV + j]) : 0.f;
        };
        {
            constexpr int NCK = 4 * (DK / 16);   // tiles of a C x DK result
            for (int t = wave; t < 3 * NCK + 32; t += NT / kWave) {
                if (t < 3 * NCK) {
                    const int which = t / NCK, tt = t % NCK;
                    const int m0 = 16 * (tt / (DK / 16)), n0 = 16 * (tt % (DK / 16));
                    f32x4 acc;
                    if (which == 0)        // dQt = dO S^T
                        acc = mm_tile<DV>(dOf, [&](int j, int i) { return S[i * DV + j]; }, m0, n0,
                                          l16, lg, zero4());
                    else if (which == 1)   // dKbar = Delta dS'^T
                        acc = mm_tile<DV>([&](int r, int j) { return Dl[r * DV + j]; },
                                          [&](int j, int i) { return dSp[i * DV + j]; }, m0, n0, l16,
                                          lg, zero4());
                    else                   // dW = -dDelta S^T
                        acc = mm_tile<DV>([&](int r, int j) { return -dD[r * DV + j]; },
                                          [&](int j, int i) { return S[i * DV + j]; }, m0, n0, l16,
                                          lg, zero4());
                    float *dst = which == 0 ? dQt : which == 1 ? dKb : dWm;
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[(m0 + 4 * lg + i) * DK + n0 + l16] = acc[i];
                } else {
                    const int tt = t - 3 * NCK;
                    const bool isT = tt >= 16;
                    const int t16 = tt & 15, m0 = 16 * (t16 / 4), n0 = 16 * (t16 % 4);
                    f32x4 acc;
                    if (!isT)   // dP = lower(dO Delta^T)
                        acc = mm_tile<DV>(dOf, [&](int j, int s) { return Dl[s * DV + j]; }, m0, n0,
                                          l16, lg, zero4());
                    else        // dT (first part) = dDelta u^T
                        acc = mm_tile<DV>([&](int r, int j) { return dD[r * DV + j]; },
                                          [&](int j, int s) { return Uu[s * DV + j]; }, m0, n0, l16,
                                          lg, zero4());
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = m0 + 4 * lg + i, s = n0 + l16;
                        if (isT) dTm[r * C + s] = acc[i];
                        else dPm[r * C + s] = s <= r ? acc[i] : 0.f;
                    }
                }
            }
        }
        for (int i = tid; i < DK; i += NT) {   // d e^{g_C}: sum_j S dS'
            float acc = 0.f;
            for (int j = 0; j < DV; ++j) acc += S[i * DV + j] * dSp[i * DV + j];
            vdgam[i] = acc;
        }
        __syncthreads();
        // ---- E5: dT += dW At^T; dAt = T^T dW; du = T^T dDelta ---------------
        {
            constexpr int NCK = 4 * (DK / 16), NCV = 4 * (DV / 16);
            for (int t = wave; t < 16 + NCK + NCV; t += NT / kWave) {
                if (t < 16) {
                    const int m0 = 16 * (t / 4), n0 = 16 * (t % 4);
                    f32x4 acc = mm_tile<DK>([&](int r, int i) { return dWm[r * DK + i]; },
                                            [&](int i, int s) { return Ag[s * DK + i]; }, m0, n0,
                                            l16, lg, zero4());
#pragma unroll
                    for (int i = 0; i < 4; ++i) dTm[(m0 + 4 * lg + i) * C + n0 + l16] += acc[i];
                } else if (t < 16 + NCK) {
                    const int tt = t - 16, m0 = 16 * (tt / (DK / 16)), n0 = 16 * (tt % (DK / 16));
                    f32x4 acc = mm_tile<C>([&](int r, int s) { return Tm[s * C + r]; },
                                           [&](int s, int i) { return dWm[s * DK + i]; }, m0, n0, l16,
                                           lg, zero4());
#pragma unroll
                    for (int i = 0; i < 4; ++i) dAg[(m0 + 4 * lg + i) * DK + n0 + l16] = acc[i];
                } else {
                    const int tt = t - 16 - NCK, m0 = 16 * (tt / (DV / 16)), n0 = 16 * (tt % (DV / 16));
                    f32x4 acc = mm_tile<C>([&](int r, int s) { return Tm[s * C + r]; },
                                           [&](int s, int j) { return dD[s * DV + j]; }, m0, n0, l16,
                                           lg, zero4());
#pragma unroll
                    for (int i = 0; i < 4; ++i) dUu[(m0 + 4 * lg + i) * DV + n0 + l16] = acc[i];
                }
            }
        }
        __syncthreads();
        // ---- E6: dA = -strict_lower(T^T (dT T^T)) ------------------------------
        for (int t = wave; t < 16; t += NT / kWave) {
            const int m0 = 16 * (t / 4), n0 = 16 * (t % 4);
            f32x4 acc = mm_tile<C>([&](int r, int s) { return dTm[r * C + s]; },
                                   [&](int s, int n) { return Tm[n * C + s]; }, m0, n0, l16, lg, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) Ym[(m0 + 4 * lg + i) * C + n0 + l16] = acc[i];
        }
        __syncthreads();
        for (int t = wave; t < 16; t += NT / kWave) {
            const int m0 = 16 * (t / 4), n0 = 16 * (t % 4);
            f32x4 acc = mm_tile<C>([&](int r, int s) { return Tm[s * C + r]; },
                                   [&](int s, int n) { return Ym[s * C + n]; }, m0, n0, l16, lg, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = m0 + 4 * lg + i, s = n0 + l16;
                dAm[r * C + s] = s < r ? -acc[i] : 0.f;
            }
        }
        __syncthreads();
        // ---- E7: the Gram products' backward ------------------------------------
        if constexpr (kRowDecay) {
            // G = (X Y^T) (.) D with D = e^{g_r - g_s}: dg_r += sum_s dG G, dg_s -= sum_r dG G;
            // then the operands see dG (.) D.
            for (int r = tid; r < C; r += NT) {
                float rs = 0.f, cs = 0.f;
                for (int s = 0; s < C; ++s) {
                    rs += dAm[r * C + s] * Am[r * C + s] + dPm[r * C + s] * Pm[r * C + s];
                    cs += dAm[s * C + r] * Am[s * C + r] + dPm[s * C + r] * Pm[s * C + r];
                }
                vrow[r] = rs;
                vcol[r] = cs;
            }
            __syncthreads();
            for (int idx = tid; idx < C * C; idx += NT) {
                dAm[idx] *= Dm[idx];
                dPm[idx] *= Dm[idx];
            }
            __syncthreads();
        }
        {
            constexpr int NCK = 4 * (DK / 16);
            for (int t = wave; t < 3 * NCK; t += NT / kWave) {
                const int which = t / NCK, tt = t % NCK;
                const int m0 = 16 * (tt / (DK / 16)), n0 = 16 * (tt % (DK / 16));
                f32x4 acc;
                if (which == 0)        // dXa = dA Xk
                    acc = mm_tile<C>([&](int r, int s) { return dAm[r * C + s]; },
                                     [&](int s, int i) { return Xk[s * DK + i]; }, m0, n0, l16, lg, zero4());
                else if (which == 1)   // dXq = dP Xk
                    acc = mm_tile<C>([&](int r, int s) { return dPm[r * C + s]; },
                                     [&](int s, int i) { return Xk[s * DK + i]; }, m0, n0, l16, lg, zero4());
                else {                 // dXk = dA^T Xa + dP^T Xq
                    acc = mm_tile<C>([&](int s, int r) { return dAm[r * C + s]; },
                                     [&](int r, int i) { return Xa[r * DK + i]; }, m0, n0, l16, lg, zero4());
                    acc = mm_tile<C>([&](int s, int r) { return dPm[r * C + s]; },
                                     [&](int r, int i) { return Xq[r * DK + i]; }, m0, n0, l16, lg, acc);
                }
                float *dst = which == 0 ? dXa : which == 1 ? dXq : dXk;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(m0 + 4 * lg + i) * DK + n0 + l16] = acc[i];
            }
        }
        __syncthreads();
        // ---- E8: element-wise chain rule ----------------------------------------
        // dg (per channel, or summed over channels for a scalar decay) goes into
        // Xq's slot, the gradient with respect to a into Xa's, k into Xk's.
        for (int idx = tid; idx < C * DK; idx += NT) {
            const int r = idx / DK, i = idx % DK;
            const int gi = VT::kChannelDecay ? i : 0;
            const float gr = Gd[r * DK + gi], gC = Gd[(C - 1) * DK + gi], gm = Gd[(C / 2 - 1) * DK + gi];
            float dq = dXq[idx], da = dXa[idx], dk = dXk[idx], dg = 0.f;
            if constexpr (VT::kChannelDecay) {
                dg = Xa[idx] * da + Xq[idx] * dq - Xk[idx] * dk;
                dq *= __expf(gr - gm);
                da *= __expf(gr - gm);
                dk *= __expf(gm - gr);
            }
            const float eg = __expf(gr);
            dq += dQt[idx] * eg;
            da += dAg[idx] * eg;
            dk += dKb[idx] * __expf(gC - gr);
            dg += dQt[idx] * Qg[idx] + dAg[idx] * Ag[idx] - dKb[idx] * Kb[idx];
            Xq[idx] = dg;
            Xa[idx] = da;
            Xk[idx] = dk;
            dQt[idx] = dq;
        }
        __syncthreads();
        // dg of g_C (row C-1): sum over rows of dKbar (.) Kbar, and d e^{g_C} e^{g_C}
        for (int i = tid; i < DK; i += NT) {
            const int gi = VT::kChannelDecay ? i : 0;
            float acc = vdgam[i] * __expf(Gd[(C - 1) * DK + gi]);
            for (int r = 0; r < C; ++r) acc += dKb[r * DK + i] * Kb[r * DK + i];
            vdgam[i] = acc;
        }
        __syncthreads();
        // ---- E9: outputs -------------------------------------------------------------
        // per row: the step-size gradient needs sum_i da k and sum_j du v
        for (int r = wave; r < C; r += NT / kWave) {
            float sa = 0.f, su = 0.f;
            if (r < nvalid) {
                for (int i = lane; i < DK; i += kWave) sa += Xa[r * DK + i] * f32(k[tok(r) * DK + i]);
                for (int j = lane; j < DV; j += kWave) su += dUu[r * DV + j] * f32(v[tok(r) * DV + j]);
            }
            sa = wave_sum(sa);
            su = wave_sum(su);
            if (lane == 0 && VT::kScalarBeta) {
                const float dbeta = sa + su;
                if (r < nvalid) {
                    if constexpr (VT::kKaczmarz) {
                        // beta = eta / n, n = |k|^2 + eps: d eta = dbeta / n, and dk gets
                        // -2 beta dbeta k / n (added below through vkn)
                        const float n = vkn[r] + p.eps;
                        g.d_beta[tok(r)] = dbeta / n;
                        vkn[r] = -2.f * vbeta[r] * dbeta / n;
                    } else {
                        g.d_beta[tok(r)] = dbeta;
                    }
                }
            }
        }
        __syncthreads();
        for (int idx = tid; idx < C * DK; idx += NT) {
            const int r = idx / DK, i = idx % DK;
            if (r >= nvalid) continue;
            const long o = tok(r) * DK + i;
            const float kk = f32(k[o]);
            float dk = Xk[idx];
            const float da = Xa[idx];
            if constexpr (VT::kGates) {
                const float bg = p.erase_b[o];
                dk += bg * da;
                g.d_erase_b[o] = da * kk;
            } else {
                dk += vbeta[r] * da;
                if constexpr (VT::kKaczmarz) dk += vkn[r] * kk;
            }
            g.d_q[o] = dQt[idx];
            g.d_k[o] = dk;
        }
        for (int idx = tid; idx < C * DV; idx += NT) {
            const int r = idx / DV, j = idx % DV;
            if (r >= nvalid) continue;
            const long o = tok(r) * DV + j;
            const float du = dUu[idx];
            if constexpr (VT::kGates) {
                g.d_v[o] = p.write_w[o] * du;
                g.d_write_w[o] = du * f32(v[o]);
            } else {
                g.d_v[o] = vbeta[r] * du;
            }
        }
        // decay: dl_t = sum_{r >= t} dg_r (g restarts each chunk; row C-1 also
        // carries g_C's gradient), d alpha = dl / alpha
        if constexpr (VT::kHasDecay) {
            if constexpr (VT::kChannelDecay) {
                for (int i = tid; i < DK; i += NT) {
                    float acc = vdgam[i];
                    for (int r = C - 1; r >= 0; --r) {
                        acc += Xq[r * DK + i];
                        if (r < nvalid) {
                            const long o = tok(r) * DK + i;
                            g.d_alpha[o] = acc / p.alpha[o];
                        }
                    }
                }
            } else {
                // channel sums of the per-channel terms, plus the decay matrix's
                if (tid < C) {
                    float s = vrow[tid] - vcol[tid];
                    for (int i = 0; i < DK; ++i) s += Xq[tid * DK + i];
                    dAg[tid] = s;   // dAg is free now: per-row dg
                }
                __syncthreads();
                if (tid == 0) {
                    float acc = 0.f;
                    for (int i = 0; i < DK; ++i) acc += vdgam[i];
                    for (int r = C - 1; r >= 0; --r) {
                        acc += dAg[r];
                        if (r < nvalid) g.d_alpha[tok(r)] = acc / p.alpha[tok(r)];
                    }
                }
            }
        }
    }
}

template <int V, typename TI, int DK, int DV>
hipError_t backward_shape(const Problem &p, const Grads &g, void *ws, hipStream_t st) {
    char *base = static_cast<char *>(ws);
    const long NC = (p.T + C - 1) / C, nheads = p.B * p.H;
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    size_t off = al(forward_states_bytes(p));
    float *S_chunks = reinterpret_cast<float *>(base + off);
    off += al((size_t)nheads * NC * DK * DV * 4);
    float *dS_chunks = reinterpret_cast<float *>(base + off);
    off += al((size_t)nheads * NC * DK * DV * 4);
    float *dDelta = reinterpret_cast<float *>(base + off);
    off += al((size_t)nheads * NC * C * DV * 4);
    float *scratch = reinterpret_cast<float *>(base + off);

    ForwardStates f;
    hipError_t e = launch_forward_states(p, ws, S_chunks, &f, st);
    if (e != hipSuccess) return e;
    const long nwg = nheads * (DV / 16);
    hipLaunchKernelGGL((reverse_scan_kernel<TI, DK, DV>), dim3((unsigned)(kXcds * ((nwg + kXcds - 1) / kXcds))),
                       dim3(kRevThreads), 0, st, p, f, g, dS_chunks, dDelta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const long items = NC * nheads;
    const long slots = 256;
    hipLaunchKernelGGL((chunk_grad_kernel<V, TI, DK, DV>), dim3((unsigned)(items < slots ? items : slots)),
                       dim3(kGradThreads), 0, st, p, g, S_chunks, dS_chunks, dDelta, scratch);
    return hipGetLastError();
}

template <int V, typename TI>
hipError_t backward_t(const Problem &p, const Grads &g, void *ws, hipStream_t st) {
    if (p.dk == 128 && p.dv == 128) return backward_shape<V, TI, 128, 128>(p, g, ws, st);
    if (p.dk == 128 && p.dv == 64) return backward_shape<V, TI, 128, 64>(p, g, ws, st);
    if (p.dk == 64 && p.dv == 128) return backward_shape<V, TI, 64, 128>(p, g, ws, st);
    return backward_shape<V, TI, 64, 64>(p, g, ws, st);
}

template <int V>
hipError_t backward_v(const Problem &p, const Grads &g, void *ws, hipStream_t st) {
    return p.bf16 ? backward_t<V, bf16>(p, g, ws, st) : backward_t<V, float>(p, g, ws, st);
}

}  // namespace

size_t backward_workspace_bytes(const Problem &p) {
    const long NC = (p.T + C - 1) / C, nheads = p.B * p.H;
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t slot = (size_t)(15 * C * p.dk + 3 * C * p.dv + 8 * C * C + 4 * C + p.dk) * 4;
    return al(forward_states_bytes(p)) + 2 * al((size_t)nheads * NC * p.dk * p.dv * 4) +
           al((size_t)nheads * NC * C * p.dv * 4) + 256 * slot;
}

hipError_t launch_backward(const Problem &p, const Grads &g, void *workspace, hipStream_t stream) {
    switch (p.variant) {
    case kDeltaNet: return backward_v<kDeltaNet>(p, g, workspace, stream);
    case kGatedDeltaNet: return backward_v<kGatedDeltaNet>(p, g, workspace, stream);
    case kKDA: return backward_v<kKDA>(p, g, workspace, stream);
    case kGDN2: return backward_v<kGDN2>(p, g, workspace, stream);
    case kKLA: return backward_v<kKLA>(p, g, workspace, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdr
