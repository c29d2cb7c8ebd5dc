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
// Launches after the forward's own factors and per-chunk states and Deltas
// (launch_states_pass):
//   bw_prep_kernel        per chunk-head, parallel: P^T dO, Qt^T dO and the
//                         transposed factors the reverse chain reads.
//   reverse_chain_kernel  one workgroup per (16 value columns, h, b): the
//                         sequential pass; records dS' and dDelta per chunk.
//   chunk_grad_kernel     persistent workgroups over chunk-heads: the rest, on
//                         fp32 matrix cores (16x16x4) and, where both operands
//                         are stored in bf16, exact bf16 ones (16x16x32), with
//                         the chunk's 64 x 64 matrices in LDS.
#include <type_traits>

#include "gdr_device.hpp"

namespace gdr {
namespace {

constexpr int C = kChunk;
constexpr int kXcds = 8;

template <typename T> __device__ __forceinline__ float f32(T x) { return to_f32(x); }

// ============================================================================
// reverse pass over the chunks
// ============================================================================
// With dS' the gradient of the state leaving chunk c, the chunk's Delta and
// its incoming state receive
//     dDelta = X1 + Kbar dS',                       X1 = P^T dO,
//     dS     = Diag(e^{g_C}) dS' + X2 - W^T dDelta,  X2 = Qt^T dO.
// X1 and X2 do not depend on the chain: bw_prep computes them for every chunk
// in parallel, and rewrites Kbar and W^T fragment-major with their
// contraction index contiguous.  The sequential chain then has the shape of
// the forward's state chain (two matrix-core steps between two barriers per
// chunk), and copy waves move dS' and dDelta of each chunk from LDS to the
// workspace beside it.

// Chain operands of every chunk-head, in the input dtype.
struct RevFactors {
    void *Kb;   // [nch] C x DK   Kbar, fragment-major (rows r, contraction over i)
    void *Wt;   // [nch] DK x C   W^T, fragment-major (rows i, contraction over r)
    void *X1;   // [nch] C x DV   P^T dO, accumulator layout
    void *X2;   // [nch] DK x DV  Qt^T dO, accumulator layout
};

// (row, k) of the element at offset `off` of a rows x K fragment-major matrix
// (the inverse of frag_off).
template <typename TI> __device__ __forceinline__ void frag_pos(int off, int K, int &r, int &k) {
    using M = Mma<TI>;
    const int e = off % M::kPerLane, q = off / M::kPerLane;
    const int ln = q % kWave, tile = q / kWave, kt = K / M::kK;
    r = (tile / kt) * 16 + (ln & 15);
    k = (tile % kt) * M::kK + (ln >> 4) * M::kPerLane + e;
}

// Offset of element (row i, value column j) of a rows x DV matrix kept in
// accumulator layout: 16 x 16 tiles, value tile major; in a tile, lane
// (j % 16) + 16 ((i % 16) / 4) holds rows i .. i+3 of column j.
__device__ __forceinline__ long afrag_off(int j, int i, int rows) {
    return ((long)((j >> 4) * (rows / 16) + (i >> 4)) * kWave + (j & 15) + 16 * ((i & 15) >> 2)) * 4 +
           (i & 3);
}

template <typename TI> __device__ __forceinline__ void copy16(TI *dst, const TI *src, int n, int tid,
                                                              int nt) {
    constexpr int V = 16 / sizeof(TI);
    for (int o = tid * V; o < n; o += nt * V)
        *reinterpret_cast<f32x4 *>(dst + o) = *reinterpret_cast<const f32x4 *>(src + o);
}

constexpr int kBpThreads = 256;

template <typename TI, int DK, int DV>
__global__ __launch_bounds__(kBpThreads) void bw_prep_kernel(Problem p, ForwardStates f, Grads g,
                                                            RevFactors rf, long c0, int ncb) {
    using M = Mma<TI>;
    constexpr int NL = M::kPerLane;
    __shared__ __attribute__((aligned(16))) TI sm[C * C + C * DK + C * DV];
    TI *sP = sm, *sQ = sm + C * C, *sdO = sm + C * C + C * DK;   // first stage
    TI *sK = sm, *sW = sm + C * DK;                              // second stage
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int H = (int)p.H;
    const long T = p.T, NC = f.nbmax, nitems = (long)ncb * p.B * p.H;
    const TI *dO = static_cast<const TI *>(g.d_o);
    for (long item = blockIdx.x; item < nitems; item += gridDim.x) {
        // chunks c0 .. c0 + ncb - 1 of every head
        const long c = c0 + item % ncb, bh = item / ncb, ch = bh * NC + c;
        const int b = (int)(bh / H), h = (int)(bh % H);
        const long t0 = c * C;
        const int nvalid = (int)min((long)C, T - t0);
        __syncthreads();
        copy16(sP, static_cast<const TI *>(f.P) + ch * C * C, C * C, tid, kBpThreads);
        copy16(sQ, static_cast<const TI *>(f.Qt) + ch * C * DK, C * DK, tid, kBpThreads);
        for (int o = 4 * tid; o < C * DV; o += 4 * kBpThreads) {
            const int r = o / DV, j = o % DV;
            f32x4 x = zero4();
            if (dO && r < nvalid) x = load4(dO + (((long)b * T + t0 + r) * H + h) * DV + j);
            store4(sdO + o, x);
        }
        __syncthreads();
        // X1 = P^T dO and X2 = Qt^T dO on fp32 matrix cores
        constexpr int NX1 = (C / 16) * (DV / 16), NX = NX1 + (DK / 16) * (DV / 16);
        for (int t = wave; t < NX; t += kBpThreads / kWave) {
            const bool x1 = t < NX1;
            const int tt = x1 ? t : t - NX1;
            const int Rb = tt / (DV / 16), Jb = tt % (DV / 16);
            const int row = 16 * Rb + l16, col = 16 * Jb + l16;
            f32x4 acc = zero4();
            if constexpr (sizeof(TI) == 2) {
                // bf16 operands: their products are exact in fp32, so the bf16
                // matrix cores give the fp32 result up to summation order, with
                // an eighth of the matrix-core instructions.
#pragma unroll
                for (int s0 = 0; s0 < C; s0 += 32) {
                    bf16x8 a8, b8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int s = s0 + 8 * lg + e;
                        a8[e] = x1 ? sP[frag_off<TI>(s, row, C)] : sQ[frag_off<TI>(s, row, DK)];
                        b8[e] = sdO[s * DV + col];
                    }
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc, 0, 0, 0);
                }
            } else {
                for (int s0 = 0; s0 < C; s0 += 16) {
                    float av[4], bv[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int s = s0 + 4 * u + lg;
                        av[u] = to_f32(x1 ? sP[frag_off<TI>(s, row, C)] : sQ[frag_off<TI>(s, row, DK)]);
                        bv[u] = to_f32(sdO[s * DV + col]);
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], bv[u], acc, 0, 0, 0);
                }
            }
            TI *dst = static_cast<TI *>(x1 ? rf.X1 : rf.X2) + ch * (x1 ? C : DK) * DV;
            store4(dst + afrag_off(col, 16 * Rb + 4 * lg, x1 ? C : DK), acc);
        }
        __syncthreads();
        copy16(sK, static_cast<const TI *>(f.Kbt) + ch * DK * C, DK * C, tid, kBpThreads);
        copy16(sW, static_cast<const TI *>(f.W) + ch * C * DK, C * DK, tid, kBpThreads);
        __syncthreads();
        TI *kb = static_cast<TI *>(rf.Kb) + ch * C * DK, *wt = static_cast<TI *>(rf.Wt) + ch * DK * C;
        for (int qo = tid * NL; qo < C * DK; qo += kBpThreads * NL) {
            int r, i, i2, r2;
            frag_pos<TI>(qo, DK, r, i);    // Kbar element (r, i .. i+NL-1) = Kbar^T (i.., r)
            frag_pos<TI>(qo, C, i2, r2);   // W^T element (i2, r2 .. r2+NL-1) = W (r2.., i2)
            TI xk[NL], xw[NL];
#pragma unroll
            for (int e = 0; e < NL; ++e) {
                xk[e] = sK[frag_off<TI>(i + e, r, C)];
                xw[e] = sW[frag_off<TI>(r2 + e, i2, DK)];
            }
#pragma unroll
            for (int e = 0; e < NL; ++e) {
                kb[qo + e] = xk[e];
                wt[qo + e] = xw[e];
            }
        }
    }
}

// One chunk's chain operands, loaded through buffer descriptors (per-lane
// offsets fixed, per-chunk address arithmetic scalar).
template <typename TI, int DK> struct RevOps {
    using M = Mma<TI>;
    static constexpr int KS_D = DK / M::kK, KS_C = C / M::kK, NI = DK / 64;
    static constexpr int FB = kWave * M::kPerLane * (int)sizeof(TI);   // bytes per fragment tile
    typedef typename std::conditional<sizeof(TI) == 2, bf16x4, f32x4>::type raw4;
    typename M::frag Kf[KS_D], Wf[NI][KS_C];
    raw4 X1, X2[NI];
    f32x4 gam[NI];
    __device__ __forceinline__ void load(const RevFactors &rf, const float *gm, long ch, int DV,
                                         int col0, int w, int lane) {
        const unsigned loff = (unsigned)lane * (M::kPerLane * sizeof(TI));
        const auto rk = make_rsrc(static_cast<const char *>(rf.Kb) + (ch * C * DK) * (long)sizeof(TI) +
                                  w * KS_D * FB);
        const auto rw = make_rsrc(static_cast<const char *>(rf.Wt) + (ch * DK * C) * (long)sizeof(TI) +
                                  w * NI * KS_C * FB);
        const auto rg = make_rsrc(gm + ch * DK + 16 * NI * w);
        const auto r1 = make_rsrc(static_cast<const char *>(rf.X1) +
                                  (ch * C * DV + (long)((col0 / 16) * (C / 16) + w) * kWave * 4) *
                                      (long)sizeof(TI));
        const auto r2 = make_rsrc(static_cast<const char *>(rf.X2) +
                                  (ch * DK * DV + (long)((col0 / 16) * (DK / 16) + w * NI) * kWave * 4) *
                                      (long)sizeof(TI));
#pragma unroll
        for (int ks = 0; ks < KS_D; ++ks) Kf[ks] = buf_load<typename M::frag>(rk, loff + ks * FB);
#pragma unroll
        for (int a = 0; a < NI; ++a) {
#pragma unroll
            for (int ks = 0; ks < KS_C; ++ks)
                Wf[a][ks] = buf_load<typename M::frag>(rw, loff + (a * KS_C + ks) * FB);
            gam[a] = buf_load<f32x4>(rg, (unsigned)(lane >> 4) * 16u + 64u * a);
            X2[a] = buf_load<raw4>(r2, ((unsigned)lane + (unsigned)a * kWave) * 4u * sizeof(TI));
        }
        X1 = buf_load<raw4>(r1, (unsigned)lane * 4u * sizeof(TI));
    }
};

constexpr int kRevThreads = 512;

// One workgroup per (16 value columns, h, b): waves 0-3 carry dS (fp32, in
// matrix-core accumulators) backwards over the chunks; waves 4-7 copy each
// chunk's dS' and dDelta from LDS to the workspace.
// Chunks c0 + ncb - 1 down to c0; dS enters from ds_in (NULL = zeros) and
// leaves to ds_out (NULL = dropped).  Segmented (L > 0): blockIdx.y is a
// segment of L chunks (the last one shorter), entering from ds_in for the
// last segment and from dSend[nseg - 2 - s] for segment s (the combine's
// order), and only segment 0 writes ds_out.
template <typename TI, int DK, int DEPTH>
__global__ __launch_bounds__(kRevThreads, 4) void reverse_chain_kernel(
    Problem p, const float *gm, RevFactors rf, TI *dS_chunks, TI *dD_chunks, long NC, long c0,
    int ncb, const float *ds_in, float *ds_out, long L, const float *dSend) {
    if (L > 0) {
        const long sg = blockIdx.y, nseg = gridDim.y;
        c0 = sg * L;
        ncb = (int)(NC - c0 < L ? NC - c0 : L);
        if (sg != nseg - 1) ds_in = dSend + (nseg - 2 - sg) * p.B * p.H * DK * p.dv;
        if (sg != 0) ds_out = nullptr;
    }
    using M = Mma<TI>;
    using RO = RevOps<TI, DK>;
    constexpr int KS_D = RO::KS_D, KS_C = RO::KS_C, NI = RO::NI;
    constexpr int PT = 8;
    __shared__ __attribute__((aligned(16))) TI sSt[2][16][DK + PT];   // dS'^T, double-buffered
    __shared__ __attribute__((aligned(16))) TI sDt[2][16][C + PT];    // dDelta^T, double-buffered
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int DV = (int)p.dv;
    const int nslice = DV / 16;
    const long nwg = p.B * p.H * nslice;
    const long per_xcd = (nwg + kXcds - 1) / kXcds;
    const long logical = (long)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= nwg) return;
    const long bh = logical / nslice;
    const int col0 = (int)(logical % nslice) * 16;
    const long ch0 = bh * NC + c0;
    // the n-th chunk of the reverse pass, clamped for prefetches past the end
    auto chunk = [&](long n) { return ch0 + ncb - 1 - (n < ncb ? n : ncb - 1); };

    if (wave < 4) {
        const int w = wave;
        f32x4 S[NI];
#pragma unroll
        for (int a = 0; a < NI; ++a)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int i = 16 * (w * NI + a) + 4 * lg + m;
                S[a][m] = ds_in ? ds_in[(bh * DK + i) * DV + col0 + l16] : 0.f;
            }
        auto write_st = [&](int buf) {
#pragma unroll
            for (int a = 0; a < NI; ++a) store4(&sSt[buf][l16][16 * (w * NI + a) + 4 * lg], S[a]);
        };
        write_st(0);
        __syncthreads();
        auto step = [&](const RO &op, long n) __attribute__((always_inline)) {
            const int cur = (int)(n & 1);
            typename M::frag Sf[KS_D];
#pragma unroll
            for (int ks = 0; ks < KS_D; ++ks) Sf[ks] = M::load(&sSt[cur][l16][0], ks * M::kK, lane);
            f32x4 d0 = zero4(), d1 = zero4();
#pragma unroll
            for (int ks = 0; ks < KS_D; ks += 2) {
                d0 = M::mma(op.Kf[ks], Sf[ks], d0);
                if (ks + 1 < KS_D) d1 = M::mma(op.Kf[ks + 1], Sf[ks + 1], d1);
            }
            store4(&sDt[cur][l16][16 * w + 4 * lg], to_f32x4(op.X1) + (d0 + d1));
            __syncthreads();
            typename M::frag Df[KS_C];
#pragma unroll
            for (int ks = 0; ks < KS_C; ++ks) Df[ks] = M::load(&sDt[cur][l16][0], ks * M::kK, lane);
#pragma unroll
            for (int a = 0; a < NI; ++a) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < KS_C; ++ks) acc = M::mma(op.Wf[a][ks], Df[ks], acc);
                S[a] = S[a] * op.gam[a] + to_f32x4(op.X2[a]) - acc;
            }
            write_st(cur ^ 1);
            __syncthreads();
        };
        if constexpr (DEPTH == 2) {
            RO A, Bq;
            A.load(rf, gm, chunk(0), DV, col0, w, lane);
            for (long n = 0; n < ncb; n += 2) {
                Bq.load(rf, gm, chunk(n + 1), DV, col0, w, lane);
                __builtin_amdgcn_sched_barrier(0);   // issue the prefetch first
                step(A, n);
                if (n + 1 >= ncb) break;
                A.load(rf, gm, chunk(n + 2), DV, col0, w, lane);
                __builtin_amdgcn_sched_barrier(0);
                step(Bq, n + 1);
            }
        } else {
            RO cur;
            for (long n = 0; n < ncb; ++n) {
                cur.load(rf, gm, chunk(n), DV, col0, w, lane);
                step(cur, n);
            }
        }
        // the copy waves still move the last chunk
        __syncthreads();
        __syncthreads();
        if (ds_out) {
#pragma unroll
            for (int a = 0; a < NI; ++a)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int i = 16 * (w * NI + a) + 4 * lg + m;
                    ds_out[(bh * DK + i) * DV + col0 + l16] = S[a][m];
                }
        }
    } else {
        // Copy dS' and dDelta of the n-th chunk in the window where the chain
        // computes the next one; the same barriers as the chain.
        const int tt = tid - 4 * kWave;
        __syncthreads();
        __syncthreads();
        __syncthreads();
        for (long n = 0; n < ncb; ++n) {
            const int buf = (int)(n & 1);
            const long ch = ch0 + ncb - 1 - n;
            copy_transposed<TI, 16, DK + PT>(dS_chunks + ch * DK * DV + col0, DV, sSt[buf], DK, DK, tt,
                                             4 * kWave);
            copy_transposed<TI, 16, C + PT>(dD_chunks + ch * C * DV + col0, DV, sDt[buf], C, C, tt,
                                            4 * kWave);
            __syncthreads();
            __syncthreads();
        }
    }
}

// The segmented reverse pass's transitions: segment s = nseg - 1 - blockIdx.y
// of L chunks (the last one shorter), for one head and one 16-column tile per
// workgroup of four waves, its chunks in reverse order: either the chain from
// dS' = 0 over d_v's columns (N, the gradient entering the segment from its
// own chunks) or the chain over the identity's d_k columns with X1 and X2
// taken as zero (M, the product of the chunks' maps dS' -> (Diag(e^{g_C}) -
// W^T Kbar) dS').  The step is the reverse chain's.
template <int DK, int DV>
__global__ __launch_bounds__(4 * kWave) void rev_transition_kernel(Problem p, const float *gm,
                                                                  RevFactors rf, long NC, long L,
                                                                  long nseg, float *Mo, float *No) {
    using TI = bf16;
    using M = Mma<TI>;
    using RO = RevOps<TI, DK>;
    constexpr int KS_D = RO::KS_D, KS_C = RO::KS_C, NI = RO::NI;
    constexpr int PT = 8, NV = DV / 16, NK = DK / 16;
    __shared__ __attribute__((aligned(16))) TI sSt[2][16][DK + PT];   // dS'^T
    __shared__ __attribute__((aligned(16))) TI sDt[2][16][C + PT];    // dDelta^T
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const long BH = p.B * p.H;
    const long nwg = BH * (NV + NK);
    const long per_xcd = (nwg + kXcds - 1) / kXcds;
    const long logical = (long)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= nwg) return;
    const long bh = logical / (NV + NK);
    const int r = (int)(logical % (NV + NK));
    const bool mrole = r >= NV;                  // wave-uniform
    const int col0 = 16 * (mrole ? r - NV : r);
    const long j = blockIdx.y, sg = nseg - 1 - j;
    const long c0 = sg * L, nc = (NC - c0 < L ? NC - c0 : L);
    const long ch0 = bh * NC + c0;
    auto chunk = [&](long n) { return ch0 + nc - 1 - (n < nc ? n : nc - 1); };
    // X1 and X2 are read for the identity's columns too (value tile 0, in
    // bounds) and multiplied by zero there.
    const int xcol = mrole ? 0 : col0;
    const float xk = mrole ? 0.f : 1.f;
    f32x4 S[NI];
#pragma unroll
    for (int a = 0; a < NI; ++a)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int i = 16 * (w * NI + a) + 4 * lg + m;
            S[a][m] = (mrole && i == col0 + l16) ? 1.f : 0.f;
        }
    auto write_st = [&](int buf) {
#pragma unroll
        for (int a = 0; a < NI; ++a) store4(&sSt[buf][l16][16 * (w * NI + a) + 4 * lg], S[a]);
    };
    write_st(0);
    __syncthreads();
    auto step = [&](const RO &op, long n) __attribute__((always_inline)) {
        const int cur = (int)(n & 1);
        typename M::frag Sf[KS_D];
#pragma unroll
        for (int ks = 0; ks < KS_D; ++ks) Sf[ks] = M::load(&sSt[cur][l16][0], ks * M::kK, lane);
        f32x4 d0 = zero4(), d1 = zero4();
#pragma unroll
        for (int ks = 0; ks < KS_D; ks += 2) {
            d0 = M::mma(op.Kf[ks], Sf[ks], d0);
            if (ks + 1 < KS_D) d1 = M::mma(op.Kf[ks + 1], Sf[ks + 1], d1);
        }
        store4(&sDt[cur][l16][16 * w + 4 * lg], xk * to_f32x4(op.X1) + (d0 + d1));
        __syncthreads();
        typename M::frag Df[KS_C];
#pragma unroll
        for (int ks = 0; ks < KS_C; ++ks) Df[ks] = M::load(&sDt[cur][l16][0], ks * M::kK, lane);
#pragma unroll
        for (int a = 0; a < NI; ++a) {
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < KS_C; ++ks) acc = M::mma(op.Wf[a][ks], Df[ks], acc);
            S[a] = S[a] * op.gam[a] + xk * to_f32x4(op.X2[a]) - acc;
        }
        write_st(cur ^ 1);
        __syncthreads();
    };
    RO A, Bq;
    A.load(rf, gm, chunk(0), DV, xcol, w, lane);
    for (long n = 0; n < nc; n += 2) {
        Bq.load(rf, gm, chunk(n + 1), DV, xcol, w, lane);
        __builtin_amdgcn_sched_barrier(0);   // issue the prefetch first
        step(A, n);
        if (n + 1 >= nc) break;
        A.load(rf, gm, chunk(n + 2), DV, xcol, w, lane);
        __builtin_amdgcn_sched_barrier(0);
        step(Bq, n + 1);
    }
    const int pitch = mrole ? DK : DV;
    float *out = (mrole ? Mo + (j * BH + bh) * (long)DK * DK : No + (j * BH + bh) * (long)DK * DV) + col0;
#pragma unroll
    for (int a = 0; a < NI; ++a)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int i = 16 * (w * NI + a) + 4 * lg + m;
            out[(long)i * pitch + l16] = S[a][m];
        }
}

// ============================================================================
// per-chunk gradient
// ============================================================================
// Persistent workgroups of eight waves, each looping over chunk-heads.  The
// 64 x 64 matrices (T, A then Y, dP, dT then dA) live in LDS; the chunk's
// C x dk operands and intermediate gradients live in a per-workgroup fp32
// slot in global memory (rows contiguous, so every operand fetch is a 16-byte
// load per lane or a 64-byte row segment per 16 lanes).  Input gradients are
// written from the matrix-core accumulators.
constexpr int kGradThreads = 512;
constexpr int kGradWaves = kGradThreads / kWave;
constexpr int kGradSlots = 512;   // at most two workgroups per compute unit
constexpr int CP = C + 2;         // LDS row pitch of the C x C matrices

template <int DK> struct GradSlot {
    enum { Xq, Xa, Xk, Ag, G, dQt, dKb, dWm, dAg, dG, NCK };   // C x DK each
    enum { Am, Pm, NCC };                                    // C x C each
    static constexpr long kCK = (long)C * DK, kCC = (long)C * C;
    static constexpr long kFloats = NCK * kCK + NCC * kCC;
    float *base;
    __device__ float *ck(int which) const { return base + which * kCK; }
    __device__ float *cc(int which) const { return base + NCK * kCK + which * kCC; }
};

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 ld4(const bf16 *p) {
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// acc += X Y^T over K for two row-major, K-contiguous operands: x4(k) and
// y4(k) return this lane's row (m0 + l16 of X, n0 + l16 of Y) at columns
// k .. k+3.  Within each block of 16, lane group lg takes K indices 4 lg ..
// 4 lg + 3 across the four steps: the same permutation of K on both sides,
// so the sum is unchanged and each operand is one 4-wide load.
template <int K, typename FX, typename FY>
__device__ __forceinline__ f32x4 mm_rr(FX x4, FY y4, int lg, f32x4 acc) {
#pragma unroll 2
    for (int k0 = 0; k0 < K; k0 += 16) {
        const f32x4 a = x4(k0 + 4 * lg), b = y4(k0 + 4 * lg);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    }
    return acc;
}

// acc += A B over k in [k_begin, k_end) (multiples of 16): a(k) is this
// lane's A element at row m0 + l16, b(k) its B element at column n0 + l16.
template <typename FA, typename FB>
__device__ __forceinline__ f32x4 mm_kr(FA a, FB b, int k_begin, int k_end, int lg, f32x4 acc) {
    for (int k0 = k_begin; k0 < k_end; k0 += 16) {
        float av[4], bv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            av[s] = a(k0 + 4 * s + lg);
            bv[s] = b(k0 + 4 * s + lg);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], acc, 0, 0, 0);
    }
    return acc;
}

__device__ __forceinline__ bf16x8 ld8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// acc += X Y^T over K on bf16 matrix cores: x8(k) and y8(k) return this lane's
// row (m0 + l16 of X, n0 + l16 of Y) at columns k .. k+7.
template <int K, typename FX, typename FY>
__device__ __forceinline__ f32x4 mm_rr8(FX x8, FY y8, int lg, f32x4 acc) {
#pragma unroll 2
    for (int k0 = 0; k0 < K; k0 += 32)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x8(k0 + 8 * lg), y8(k0 + 8 * lg), acc, 0, 0, 0);
    return acc;
}

// acc += A B over all k in [0, K) (K a multiple of 16), unrolled so that every
// operand read is issued ahead of the products; operands outside a triangle
// must read as zero.
template <int K, typename FA, typename FB>
__device__ __forceinline__ f32x4 mm_kc(FA a, FB b, int lg, f32x4 acc) {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        float av[4], bv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            av[s] = a(k0 + 4 * s + lg);
            bv[s] = b(k0 + 4 * s + lg);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], acc, 0, 0, 0);
    }
    return acc;
}

// acc += A B over k in [K0, K1) (compile-time multiples of 16), unrolled.
template <int K0, int K1, typename FA, typename FB>
__device__ __forceinline__ f32x4 mm_kt(FA a, FB b, int lg, f32x4 acc) {
#pragma unroll
    for (int k0 = K0; k0 < K1; k0 += 16) {
        float av[4], bv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            av[s] = a(k0 + 4 * s + lg);
            bv[s] = b(k0 + 4 * s + lg);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], acc, 0, 0, 0);
    }
    return acc;
}

// Calls f(std::integral_constant<int, R>) for a wave-uniform block row R in
// 0 .. 3, so that triangular K ranges become compile-time constants.
template <typename F> __device__ __forceinline__ void with_block(int R, F f) {
    switch (R) {
    case 0: f(std::integral_constant<int, 0>{}); break;
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    default: f(std::integral_constant<int, 3>{}); break;
    }
}

// Strictly upper 16 x 16 block t of a 4 x 4 block grid, t = 0 .. 5.
__device__ __forceinline__ int up_r(int t) { return (t >= 3) + (t >= 5); }
__device__ __forceinline__ int up_s(int t) { return t + 1 - 2 * (t >= 3) - (t >= 5); }

// Sum over the 16 lanes that share lg (the columns of one accumulator row).
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Lower-triangular 16 x 16 block t of a 4 x 4 block grid, t = 0 .. 9.
__device__ __forceinline__ int tri_r(int t) { return (t >= 1) + (t >= 3) + (t >= 6); }
__device__ __forceinline__ int tri_s(int t) { const int r = tri_r(t); return t - r * (r + 1) / 2; }

template <int V, typename TI, int DK, int DV>
__global__ __launch_bounds__(kGradThreads, 4) void chunk_grad_kernel(
    Problem p, Grads g, const TI *S_chunks, const TI *D_chunks, const TI *dS_chunks,
    const TI *dD_chunks, float *scratch, long c0, int ncb) {
    using VT = VariantTraits<V>;
    using Slot = GradSlot<DK>;
    constexpr int NT = kGradThreads, NW = kGradWaves;
    constexpr bool kRowDecay = VT::kHasDecay && !VT::kChannelDecay;
    constexpr int NKB = DK / 16, NVB = DV / 16;
    constexpr bool kSlotX = VT::kChannelDecay;   // split Gram operands staged in the slot
    constexpr bool kMfma8 = sizeof(TI) == 2;     // bf16 inputs: bf16 products where exact
    static_assert(kSlotX || VT::kScalarBeta, "variants without channel decay take a scalar beta");
    __shared__ float sB[4][C][CP];   // 0: T; 1: A, then Y; 2: dP; 3: dT, then dA
    __shared__ float sG[C], sbeta[C], sn[C], ssa[C], ssu[C], sdg[C], svrow[C], svcol[C], scoef[C];
    __shared__ float sdgam[DK], sdgc[DK];
    // Channel decay: the split Gram operands are scaled relative to their own
    // 16-row block's reference m_R = (g_{16R} + g_{16R+15}) / 2; an
    // off-diagonal tile (R, S) multiplies its right operand by the middle
    // factor e^{m_R - m_S} <= 1, pair_of(R, S), and row 6 holds ones for the
    // diagonal tiles.
    __shared__ __attribute__((aligned(16))) float sMf[kSlotX ? 7 : 1][kSlotX ? DK : 4];
    float(*sT)[CP] = sB[0];
    float(*sA)[CP] = sB[1];
    float(*sY)[CP] = sB[1];
    float(*sdP)[CP] = sB[2];
    float(*sdT)[CP] = sB[3];
    float(*sdA)[CP] = sB[3];

    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int H = (int)p.H;
    const long T = p.T, NC = (p.T + C - 1) / C;
    const long nitems = (long)ncb * p.H * p.B;   // chunks c0 .. c0 + ncb - 1 of every head
    const Slot sl{scratch + (long)blockIdx.x * Slot::kFloats};
    const TI *q = static_cast<const TI *>(p.q), *k = static_cast<const TI *>(p.k);
    const TI *v = static_cast<const TI *>(p.v), *dO = static_cast<const TI *>(g.d_o);
    const bool hdo = dO != nullptr;
    float *Xq = sl.ck(Slot::Xq), *Xa = sl.ck(Slot::Xa), *Xk = sl.ck(Slot::Xk);
    float *Ag = sl.ck(Slot::Ag), *Gd = sl.ck(Slot::G), *dQt = sl.ck(Slot::dQt);
    float *dKb = sl.ck(Slot::dKb), *dWm = sl.ck(Slot::dWm), *dAg = sl.ck(Slot::dAg);
    float *dGd = sl.ck(Slot::dG), *Am = sl.cc(Slot::Am), *Pm = sl.cc(Slot::Pm);

    for (long item = blockIdx.x; item < nitems; item += gridDim.x) {
        // An opaque thread index per item keeps the compiler from hoisting
        // per-lane addresses out of the item loop (they would stay live
        // across it and spill).
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
        const long c = c0 + item % ncb, bh = item / ncb;
        const int b = (int)(bh / H), h = (int)(bh % H);
        const long t0 = c * C;
        const int nvalid = (int)min((long)C, T - t0);
        const long ch = bh * NC + c;
        const TI *S = S_chunks + ch * DK * DV, *Dl = D_chunks + ch * C * DV;
        const TI *dSp = dS_chunks + ch * DK * DV, *dD = dD_chunks + ch * C * DV;
        auto tok = [&](int r) -> long { return ((long)b * T + t0 + r) * H + h; };
        auto rowc = [&](int r) { return r < nvalid ? r : nvalid - 1; };   // clamped, in bounds
        // Operands of the Gram products and their backward: with a channel-wise
        // decay the split, scaled rows staged in the slot; otherwise q, k and
        // a = beta k read from the inputs (rows past T are zero).
        auto in4 = [&](const TI *x, int r, int kk) -> f32x4 {
            const f32x4 y = ld4(x + tok(rowc(r)) * DK + kk);
            return r < nvalid ? y : zero4();
        };
        auto in1 = [&](const TI *x, int r, int col) -> float {
            const float y = f32(x[tok(rowc(r)) * DK + col]);
            return r < nvalid ? y : 0.f;
        };
        auto ag4 = [&](int r, int kk) -> f32x4 {
            if constexpr (kSlotX) return ld4(Ag + r * DK + kk);
            else if constexpr (kRowDecay) return in4(k, r, kk) * (sbeta[r] * __expf(sG[r]));
            else return in4(k, r, kk) * sbeta[r];
        };
        auto xq1 = [&](int r, int col) -> float {
            if constexpr (kSlotX) return Xq[r * DK + col];
            else return in1(q, r, col);
        };
        auto xk1 = [&](int r, int col) -> float {
            if constexpr (kSlotX) return Xk[r * DK + col];
            else return in1(k, r, col);
        };
        auto xa1 = [&](int r, int col) -> float {
            if constexpr (kSlotX) return Xa[r * DK + col];
            else return in1(k, r, col) * sbeta[r];
        };

        __syncthreads();   // the previous item is done with LDS and the slot
        // ---- A: decay prefix sums, step sizes, element-wise operands -------------
        if constexpr (kRowDecay) {
            if (wave == 0) {
                float x = lane < nvalid ? logf(p.alpha[tok(lane)]) : 0.f;
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) {
                    const float y = __shfl_up(x, off, kWave);
                    if (lane >= off) x += y;
                }
                sG[lane] = x;
            }
        }
        if constexpr (VT::kChannelDecay) {
            if (tid < DK) {
                float gg = 0.f;
                for (int r = 0; r < C; ++r) {
                    if (r < nvalid) gg += fmaxf(logf(p.alpha[tok(r) * DK + tid]), kLogDecayFloor);
                    Gd[r * DK + tid] = gg;
                }
            }
        }
        if (tid < C) ssa[tid] = ssu[tid] = sdg[tid] = 0.f;
        if (tid < DK) sdgc[tid] = 0.f;
        if constexpr (VT::kKaczmarz) {
            // |k_r|^2: eight lanes per row, one pass of loads
            static_assert(NT == 8 * C, "eight threads per row");
            const int r = tid >> 3, part = tid & 7;
            const TI *kr = k + tok(rowc(r)) * DK + part * (DK / 8);
            float s2 = 0.f;
#pragma unroll
            for (int i = 0; i < DK / 8; i += 4) {
                const f32x4 x = ld4(kr + i);
                s2 += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
            }
            s2 += __shfl_xor(s2, 1, kWave);
            s2 += __shfl_xor(s2, 2, kWave);
            s2 += __shfl_xor(s2, 4, kWave);
            if (part == 0) {
                const float n = s2 + p.eps;
                sn[r] = n;
                sbeta[r] = r < nvalid ? p.beta[tok(r)] / n : 0.f;
            }
        } else if constexpr (VT::kScalarBeta) {
            if (tid < C) sbeta[tid] = tid < nvalid ? p.beta[tok(tid)] : 0.f;
        }
        __syncthreads();
        if constexpr (kSlotX) {
            for (int idx = tid; idx < C * DK; idx += NT) {
                const int r = idx / DK, i = idx % DK;
                const bool ok = r < nvalid;
                const long o = tok(rowc(r)) * DK + i;
                const float qq = ok ? f32(q[o]) : 0.f, kk = ok ? f32(k[o]) : 0.f;
                float aa;
                if constexpr (VT::kGates) aa = ok ? p.erase_b[o] * kk : 0.f;
                else aa = sbeta[r] * kk;
                const float gr = Gd[idx];
                const int rb = 16 * (r >> 4);
                const float mref = 0.5f * (Gd[rb * DK + i] + Gd[(rb + 15) * DK + i]);
                const float e = __expf(gr - mref);
                Xq[idx] = qq * e;
                Xa[idx] = aa * e;
                Xk[idx] = kk * __expf(mref - gr);
                Ag[idx] = aa * __expf(gr);
            }
            for (int idx = tid; idx < 7 * DK; idx += NT) {
                const int pr = idx / DK, i = idx % DK;
                float m = 1.f;
                if (pr < 6) {
                    const int R = pair_r(pr), S = pair_s(pr);
                    m = __expf(0.5f * (Gd[16 * R * DK + i] + Gd[(16 * R + 15) * DK + i]) -
                               0.5f * (Gd[16 * S * DK + i] + Gd[(16 * S + 15) * DK + i]));
                }
                sMf[pr][i] = m;
            }
            __syncthreads();
        }
        // ---- B: the Gram products A (and P for a scalar decay) ---------------------
        for (int t = wave; t < (kRowDecay ? 20 : 10); t += NW) {
            const bool isP = t >= 10;
            const int R = tri_r(t % 10), Sb = tri_s(t % 10);
            f32x4 acc;
            if constexpr (kSlotX) {
                const float *X = isP ? Xq : Xa;
                const float *mrow = sMf[Sb < R ? pair_of(R, Sb) : 6];
                acc = mm_rr<DK>([&](int kk) { return ld4(X + (16 * R + l16) * DK + kk); },
                                [&](int kk) { return ld4(Xk + (16 * Sb + l16) * DK + kk) * ld4(mrow + kk); },
                                lg, zero4());
            } else {
                // q k^T or k k^T (rows of A scaled by beta below): exact products of the inputs
                const TI *X = isP ? q : k;
                const int ra = 16 * R + l16, rb = 16 * Sb + l16;
                if constexpr (kMfma8) {
                    const bf16x8 z8 = {};
                    acc = mm_rr8<DK>(
                        [&](int kk) { const bf16x8 x = ld8(X + tok(rowc(ra)) * DK + kk); return ra < nvalid ? x : z8; },
                        [&](int kk) { const bf16x8 x = ld8(k + tok(rowc(rb)) * DK + kk); return rb < nvalid ? x : z8; },
                        lg, zero4());
                } else {
                    acc = mm_rr<DK>([&](int kk) { return in4(X, ra, kk); }, [&](int kk) { return in4(k, rb, kk); },
                                    lg, zero4());
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 16 * R + 4 * lg + m, s = 16 * Sb + l16;
                float val = acc[m];
                if constexpr (!kSlotX) val *= isP ? 1.f : sbeta[r];
                if constexpr (kRowDecay) val *= s <= r ? __expf(sG[r] - sG[s]) : 0.f;
                if (isP) {
                    Pm[r * C + s] = s <= r ? val : 0.f;
                } else {
                    val = s < r ? val : 0.f;
                    sA[r][s] = val;
                    if constexpr (kRowDecay) Am[r * C + s] = val;
                }
            }
        }
        __syncthreads();
        // ---- C: T = (I + A)^{-1}: diagonal blocks by substitution, then the
        // off-diagonal blocks by distance, T_ij = -T_ii sum_{j<=m<i} A_im T_mj.
        // The strictly upper blocks of T and of A/Y are read as zeros by the
        // full-K products below.
        for (int idx = tid; idx < 6 * 256; idx += NT) {
            const int t = idx >> 8, e = idx & 255;
            const int r = 16 * up_r(t) + (e >> 4), s = 16 * up_s(t) + (e & 15);
            sT[r][s] = 0.f;
            sA[r][s] = 0.f;
        }
        if (tid < C) {
            const int o = 16 * (tid >> 4), cc = tid & 15;
            for (int r = 0; r < 16; ++r) {
                float acc = r == cc ? 1.f : 0.f;
                for (int s = cc; s < r; ++s) acc -= sA[o + r][o + s] * sT[o + s][o + cc];
                sT[o + r][o + cc] = r < cc ? 0.f : acc;
            }
        }
        __syncthreads();
        for (int d = 1; d < 4; ++d) {
            if (wave < 4 - d) {
                const int I = wave + d, J = wave;
                float(*sX)[17] = reinterpret_cast<float(*)[17]>(&sdP[0][0] + wave * 16 * 17);
                f32x4 x = mm_kr([&](int m) { return sA[16 * I + l16][m]; },
                                [&](int m) { return sT[m][16 * J + l16]; }, 16 * J, 16 * I, lg, zero4());
#pragma unroll
                for (int m = 0; m < 4; ++m) sX[4 * lg + m][l16] = x[m];
                __builtin_amdgcn_wave_barrier();   // LDS is in order within a wave
                const f32x4 t = mm_kr([&](int m) { return sT[16 * I + l16][16 * I + m]; },
                                      [&](int m) { return sX[m][l16]; }, 0, 16, lg, zero4());
#pragma unroll
                for (int m = 0; m < 4; ++m) sT[16 * I + 4 * lg + m][16 * J + l16] = -t[m];
            }
            __syncthreads();
        }
        // ---- D: contractions over the value channels ---------------------------------
        //   dQt = dO S^T, dW = -dDelta S^T, dKbar = Delta dS'^T   (C x DK)
        //   dP = lower(dO Delta^T), dT_u = dDelta u^T              (C x C, lower blocks)
        auto ldo = [&](int r, int j) -> f32x4 {
            if (!hdo) return zero4();
            const f32x4 x = ld4(dO + tok(rowc(r)) * DV + j);
            return r < nvalid ? x : zero4();
        };
        auto ldu = [&](int r, int j) -> f32x4 {
            const long o = tok(rowc(r)) * DV + j;
            const f32x4 x = ld4(v + o);
            if constexpr (VT::kGates) return r < nvalid ? x * ld4(p.write_w + o) : zero4();
            else return x * sbeta[r];
        };
        auto ldo8 = [&](int r, int j) -> bf16x8 {
            const bf16x8 z8 = {};
            if constexpr (kMfma8) {
                if (!hdo) return z8;
                const bf16x8 x = ld8(reinterpret_cast<const bf16 *>(dO) + tok(rowc(r)) * DV + j);
                return r < nvalid ? x : z8;
            } else {
                return z8;
            }
        };
        auto tdv8 = [&](const TI *x, int r, int j) -> bf16x8 {
            if constexpr (kMfma8) return ld8(reinterpret_cast<const bf16 *>(x) + r * DV + j);
            else return bf16x8{};
        };
        for (int idx = tid; idx < 6 * 256; idx += NT) {
            const int t = idx >> 8, e = idx & 255;
            const int r = 16 * up_r(t) + (e >> 4), s = 16 * up_s(t) + (e & 15);
            sdP[r][s] = 0.f;
            sdT[r][s] = 0.f;
        }
        constexpr int NMAIN = 2 * NKB;   // C x DK tile groups: 16 columns, two block rows
        // bf16 with two tile groups per wave (t = wave and wave + NW): both
        // have the same two block rows, so one pass over the value channels
        // loads those rows' dO, dDelta and Delta once for both, and the wave
        // waits for its operands half as often.  Each accumulator sees the same
        // products in the same order as in the per-tile loop below.
        constexpr bool kPair = kMfma8 && NMAIN == 2 * NW;
        int t_first = wave;
        if constexpr (kPair) {
            const int R0 = 2 * (wave & 1);
            const int Nt[2] = {wave >> 1, (wave + NW) >> 1};
            f32x4 aq[2][2], aw[2][2], ak[2][2];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int u = 0; u < 2; ++u) aq[x][u] = aw[x][u] = ak[x][u] = zero4();
#pragma unroll 1
            for (int j0 = 0; j0 < DV; j0 += 32) {
                const int j = j0 + 8 * lg;
                bf16x8 bs[2], bd[2];
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    bs[x] = tdv8(S, 16 * Nt[x] + l16, j);
                    bd[x] = tdv8(dSp, 16 * Nt[x] + l16, j);
                }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int r = 16 * (R0 + u) + l16;
                    const bf16x8 xo = ldo8(r, j), xd = tdv8(dD, r, j), xl = tdv8(Dl, r, j);
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        aq[x][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xo, bs[x], aq[x][u], 0, 0, 0);
                        aw[x][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xd, bs[x], aw[x][u], 0, 0, 0);
                        ak[x][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, bd[x], ak[x][u], 0, 0, 0);
                    }
                }
            }
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int o = (16 * (R0 + u) + 4 * lg + m) * DK + 16 * Nt[x] + l16;
                        dQt[o] = aq[x][u][m];
                        dWm[o] = -aw[x][u][m];
                        dKb[o] = ak[x][u][m];
                    }
            t_first = NMAIN + wave;
        }
        for (int t = t_first; t < NMAIN + 10; t += NW) {
            if (t < NMAIN) {
                if constexpr (kMfma8) {
                    // bf16 inputs: every operand here is stored in bf16, so the
                    // bf16 products are exact and only the summation order differs
                    const int N = t >> 1, R0 = 2 * (t & 1);
                    f32x4 aq[2] = {zero4(), zero4()}, aw[2] = {zero4(), zero4()}, ak[2] = {zero4(), zero4()};
                    const int si = 16 * N + l16;
#pragma unroll 1
                    for (int j0 = 0; j0 < DV; j0 += 32) {
                        const int j = j0 + 8 * lg;
                        const bf16x8 bs = tdv8(S, si, j), bd = tdv8(dSp, si, j);
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int r = 16 * (R0 + u) + l16;
                            aq[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ldo8(r, j), bs, aq[u], 0, 0, 0);
                            aw[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tdv8(dD, r, j), bs, aw[u], 0, 0, 0);
                            ak[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tdv8(Dl, r, j), bd, ak[u], 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            const int o = (16 * (R0 + u) + 4 * lg + m) * DK + 16 * N + l16;
                            dQt[o] = aq[u][m];
                            dWm[o] = -aw[u][m];
                            dKb[o] = ak[u][m];
                        }
                } else {
                    const int N = t >> 1, R0 = 2 * (t & 1);
                    f32x4 aq[2] = {zero4(), zero4()}, aw[2] = {zero4(), zero4()}, ak[2] = {zero4(), zero4()};
                    const int si = 16 * N + l16;
#pragma unroll 1
                    for (int j0 = 0; j0 < DV; j0 += 16) {
                        const int j = j0 + 4 * lg;
                        const f32x4 bs = ld4(S + si * DV + j), bd = ld4(dSp + si * DV + j);
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int r = 16 * (R0 + u) + l16;
                            const f32x4 xo = ldo(r, j), xd = ld4(dD + r * DV + j), xl = ld4(Dl + r * DV + j);
#pragma unroll
                            for (int s4 = 0; s4 < 4; ++s4) {
                                aq[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(xo[s4], bs[s4], aq[u], 0, 0, 0);
                                aw[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(xd[s4], bs[s4], aw[u], 0, 0, 0);
                                ak[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(xl[s4], bd[s4], ak[u], 0, 0, 0);
                            }
                        }
                    }
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            const int o = (16 * (R0 + u) + 4 * lg + m) * DK + 16 * N + l16;
                            dQt[o] = aq[u][m];
                            dWm[o] = -aw[u][m];
                            dKb[o] = ak[u][m];
                        }
                }
            } else {
                const int R = tri_r(t - NMAIN), Sb = tri_s(t - NMAIN);
                const int r = 16 * R + l16, s = 16 * Sb + l16;
                f32x4 ap = zero4(), at = zero4();
                float cs = 1.f;   // column scale of dT_u
                if constexpr (kMfma8 && !VT::kGates) {
                    // dP = dO Delta^T and dT_u = dDelta (beta v)^T = (dDelta v^T) Diag(beta)
#pragma unroll
                    for (int j0 = 0; j0 < DV; j0 += 32) {
                        const int j = j0 + 8 * lg;
                        const bf16x8 vs = ld8(reinterpret_cast<const bf16 *>(v) + tok(rowc(s)) * DV + j);
                        ap = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ldo8(r, j), tdv8(Dl, s, j), ap, 0, 0, 0);
                        at = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tdv8(dD, r, j), vs, at, 0, 0, 0);
                    }
                    cs = sbeta[s];   // zero past T
                } else {
#pragma unroll 2
                    for (int j0 = 0; j0 < DV; j0 += 16) {
                        const int j = j0 + 4 * lg;
                        const f32x4 xo = ldo(r, j), xd = ld4(dD + r * DV + j);
                        const f32x4 yl = ld4(Dl + s * DV + j), yu = ldu(s, j);
#pragma unroll
                        for (int s4 = 0; s4 < 4; ++s4) {
                            ap = __builtin_amdgcn_mfma_f32_16x16x4f32(xo[s4], yl[s4], ap, 0, 0, 0);
                            at = __builtin_amdgcn_mfma_f32_16x16x4f32(xd[s4], yu[s4], at, 0, 0, 0);
                        }
                    }
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int rr = 16 * R + 4 * lg + m, ss = 16 * Sb + l16;
                    sdP[rr][ss] = ss <= rr ? ap[m] : 0.f;
                    sdT[rr][ss] = at[m] * cs;
                }
            }
        }
        // dL/d e^{g_C} per key channel: sum_j S dS'
        for (int idx = tid; idx < DK * 4; idx += NT) {
            const int i = idx >> 2, qd = idx & 3;
            float acc = 0.f;
#pragma unroll
            for (int j = qd * (DV / 4); j < (qd + 1) * (DV / 4); j += 4) {
                const f32x4 a = ld4(S + i * DV + j), bq = ld4(dSp + i * DV + j);
                acc += a[0] * bq[0] + a[1] * bq[1] + a[2] * bq[2] + a[3] * bq[3];
            }
            acc += __shfl_xor(acc, 1, kWave);
            acc += __shfl_xor(acc, 2, kWave);
            if (qd == 0) sdgam[i] = acc;
        }
        __syncthreads();
        // ---- E: dT += dW At^T (strictly lower); dAt = T^T dW; du = T^T dDelta -----
        // bf16: the chunk's dDelta is staged in LDS over the retired A tile,
        // transposed with a 66-element pitch, for the du products.
        constexpr bool kStageD = sizeof(TI) == 2;
        constexpr int QP = C + 2;
        static_assert(!kStageD || (DV * QP * 2 <= C * CP * 4 && DK * QP * 2 <= C * CP * 4),
                      "a staged tile fits a C x CP fp32 tile");
        bf16 (*sDd)[QP] = reinterpret_cast<bf16 (*)[QP]>(&sB[1][0][0]);
        if constexpr (kStageD) {
            for (int idx = tid; idx < C * DV / 8; idx += NT) {
                const int r = idx / (DV / 8), c8 = 8 * (idx % (DV / 8));
                const bf16x8 d8 = ld8(reinterpret_cast<const bf16 *>(dD) + r * DV + c8);
#pragma unroll
                for (int e = 0; e < 8; ++e) sDd[c8 + e][r] = d8[e];
            }
            __syncthreads();
        }
        for (int t = wave; t < 10 + 4 * NKB + 4 * NVB; t += NW) {
            if (t < 10) {
                const int R = tri_r(t), Sb = tri_s(t);
                f32x4 acc;
#pragma unroll
                for (int m = 0; m < 4; ++m) acc[m] = sdT[16 * R + 4 * lg + m][16 * Sb + l16];
                acc = mm_rr<DK>([&](int kk) { return ld4(dWm + (16 * R + l16) * DK + kk); },
                                [&](int kk) { return ag4(16 * Sb + l16, kk); }, lg, acc);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int r = 16 * R + 4 * lg + m, s = 16 * Sb + l16;
                    sdT[r][s] = s < r ? acc[m] : 0.f;
                }
            } else if (t < 10 + 4 * NKB) {
                // T^T is upper triangular: s from the tile's own block row on
                const int tt = t - 10, R = tt / NKB, N = tt % NKB;
                f32x4 acc = zero4();
                with_block(R, [&](auto Rc) {
                    constexpr int RB = decltype(Rc)::value;
                    acc = mm_kt<16 * RB, C>([&](int m) { return sT[m][16 * RB + l16]; },
                                            [&](int m) { return dWm[m * DK + 16 * N + l16]; }, lg, acc);
                });
#pragma unroll
                for (int m = 0; m < 4; ++m) dAg[(16 * R + 4 * lg + m) * DK + 16 * N + l16] = acc[m];
            } else {
                const int tt = t - 10 - 4 * NKB, R = tt / NVB, N = tt % NVB;
                f32x4 acc = zero4();
                with_block(R, [&](auto Rc) {
                    constexpr int RB = decltype(Rc)::value;
                    acc = mm_kt<16 * RB, C>([&](int m) { return sT[m][16 * RB + l16]; },
                                            [&](int m) {
                                                if constexpr (kStageD) return (float)sDd[16 * N + l16][m];
                                                else return f32(dD[m * DV + 16 * N + l16]);
                                            }, lg, acc);
                });
                const int j = 16 * N + l16;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int r = 16 * R + 4 * lg + m;
                    const long o = tok(rowc(r)) * DV + j;
                    const float vv = f32(v[o]), du = acc[m];
                    if constexpr (VT::kGates) {
                        if (r < nvalid) {
                            g.d_v[o] = p.write_w[o] * du;
                            g.d_write_w[o] = du * vv;
                        }
                    } else {
                        if (r < nvalid) g.d_v[o] = sbeta[r] * du;
                        const float su = row16_sum(r < nvalid ? du * vv : 0.f);
                        if (l16 == 0) atomicAdd(&ssu[r], su);
                    }
                }
            }
        }
        __syncthreads();
        // ---- F: dA = -strict_lower(T^T (dT T^T)) ------------------------------------
        for (int t = wave; t < 10; t += NW) {
            const int R = tri_r(t), Nb = tri_s(t);
            const f32x4 acc = mm_kc<C>([&](int m) { return sdT[16 * R + l16][m]; },
                                       [&](int m) { return sT[16 * Nb + l16][m]; }, lg, zero4());
#pragma unroll
            for (int m = 0; m < 4; ++m) sY[16 * R + 4 * lg + m][16 * Nb + l16] = acc[m];
        }
        __syncthreads();
        for (int t = wave; t < 10; t += NW) {
            const int R = tri_r(t), Nb = tri_s(t);
            const f32x4 acc = mm_kc<C>([&](int m) { return sT[m][16 * R + l16]; },
                                       [&](int m) { return sY[m][16 * Nb + l16]; }, lg, zero4());
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 16 * R + 4 * lg + m, n = 16 * Nb + l16;
                sdA[r][n] = n < r ? -acc[m] : 0.f;
            }
        }
        __syncthreads();
        // ---- G: a scalar decay inside the Gram products: G = (X Y^T) (.) D with
        // D = e^{g_r - g_s} gives dg_r += sum_s dG G and dg_s -= sum_r dG G, and
        // the operands then see dG (.) D.
        if constexpr (kRowDecay) {
            for (int r = wave; r < C; r += NW) {
                const float x = sdA[r][lane] * Am[r * C + lane] + sdP[r][lane] * Pm[r * C + lane];
                const float y = sdA[lane][r] * Am[lane * C + r] + sdP[lane][r] * Pm[lane * C + r];
                const float xs = wave_sum(lane <= r ? x : 0.f), ys = wave_sum(lane >= r ? y : 0.f);
                if (lane == 0) {
                    svrow[r] = xs;
                    svcol[r] = ys;
                }
            }
            __syncthreads();
            for (int idx = tid; idx < C * C; idx += NT) {
                const int r = idx / C, s = idx % C;
                const float d = s <= r ? __expf(sG[r] - sG[s]) : 0.f;
                sdA[r][s] *= d;
                sdP[r][s] *= d;
            }
            __syncthreads();
        }
        // ---- H: Gram backward, element-wise chain rule, outputs --------------------------
        //   dXa = dA Xk, dXq = dP Xk, dXk = dA^T Xa + dP^T Xq
        // bf16 inputs without a channel decay: the chunk's q and k are staged
        // in LDS over the retired T and Y tiles, transposed with a 66-element
        // pitch (a lane's column reads then fall in distinct banks), so the
        // operand reads below are LDS reads rather than one global load per
        // element.  Rows past T stage as zeros.
        constexpr bool kStageQK = !kSlotX && sizeof(TI) == 2;
        bf16 (*sQt)[QP] = reinterpret_cast<bf16 (*)[QP]>(&sB[0][0][0]);
        bf16 (*sKt)[QP] = reinterpret_cast<bf16 (*)[QP]>(&sB[1][0][0]);
        if constexpr (kStageQK) {
            for (int idx = tid; idx < C * DK / 8; idx += NT) {
                const int r = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
                const bool ok = r < nvalid;
                const long o = tok(rowc(r)) * DK + c8;
                const bf16x8 z8 = {};
                const bf16x8 qv = ok ? ld8(reinterpret_cast<const bf16 *>(q) + o) : z8;
                const bf16x8 kv = ok ? ld8(reinterpret_cast<const bf16 *>(k) + o) : z8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sQt[c8 + e][r] = qv[e];
                    sKt[c8 + e][r] = kv[e];
                }
            }
            __syncthreads();
        }
        auto hk = [&](int m, int cc) -> float {
            if constexpr (kStageQK) return (float)sKt[cc][m];
            else return xk1(m, cc);
        };
        // middle factor of tile (R, S) of the split Gram operands at channel cc
        // (1 on the diagonal and without a channel decay)
        auto mfac = [&](int R, int S, int cc) -> float {
            if constexpr (kSlotX) return sMf[S < R ? pair_of(R, S) : 6][cc];
            else return 1.f;
        };
        auto ha = [&](int m, int cc) -> float {
            if constexpr (kStageQK) return (float)sKt[cc][m] * sbeta[m];
            else return xa1(m, cc);
        };
        auto hq = [&](int m, int cc) -> float {
            if constexpr (kStageQK) return (float)sQt[cc][m];
            else return xq1(m, cc);
        };
        for (int t = wave; t < 4 * NKB; t += NW) {
            const int R = t / NKB, N = t % NKB, col = 16 * N + l16;
            // dA and dP are lower triangular: rows of this block row take
            // s < 16 (R + 1), columns take r >= 16 R
            f32x4 xa = zero4(), xq = zero4(), xk = zero4();
            with_block(R, [&](auto Rc) {
                constexpr int RB = decltype(Rc)::value;
                xa = mm_kt<0, 16 * (RB + 1)>([&](int m) { return sdA[16 * RB + l16][m]; },
                                             [&](int m) { return hk(m, col) * mfac(RB, m >> 4, col); },
                                             lg, xa);
                xq = mm_kt<0, 16 * (RB + 1)>([&](int m) { return sdP[16 * RB + l16][m]; },
                                             [&](int m) { return hk(m, col) * mfac(RB, m >> 4, col); },
                                             lg, xq);
                xk = mm_kt<16 * RB, C>([&](int m) { return sdA[m][16 * RB + l16]; },
                                       [&](int m) { return ha(m, col) * mfac(m >> 4, RB, col); }, lg, xk);
                xk = mm_kt<16 * RB, C>([&](int m) { return sdP[m][16 * RB + l16]; },
                                       [&](int m) { return hq(m, col) * mfac(m >> 4, RB, col); }, lg, xk);
            });
            float e_col = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 16 * R + 4 * lg + m, idx = r * DK + col;
                const long o = tok(rowc(r)) * DK + col;
                const bool ok = r < nvalid;
                float qq, kk;
                if constexpr (kStageQK) {
                    qq = (float)sQt[col][r];
                    kk = (float)sKt[col][r];
                } else {
                    qq = ok ? f32(q[o]) : 0.f;
                    kk = ok ? f32(k[o]) : 0.f;
                }
                float bg = 0.f;
                if constexpr (VT::kGates) bg = ok ? p.erase_b[o] : 0.f;
                const float aa = (VT::kGates ? bg : sbeta[r]) * kk;
                float dq = xq[m], da = xa[m], dk = xk[m], dg = 0.f;
                float gr = 0.f, gC = 0.f;
                if constexpr (VT::kChannelDecay) {
                    gr = Gd[idx];
                    gC = Gd[(C - 1) * DK + col];
                    const float mref = 0.5f * (Gd[16 * R * DK + col] + Gd[(16 * R + 15) * DK + col]);
                    const float e = __expf(gr - mref);
                    dg = Xa[idx] * da + Xq[idx] * dq - Xk[idx] * dk;
                    dq *= e;
                    da *= e;
                    dk *= __expf(mref - gr);
                } else if constexpr (kRowDecay) {
                    gr = sG[r];
                    gC = sG[C - 1];
                }
                const float eg = __expf(gr), ekc = __expf(gC - gr);
                const float dqt = dQt[idx], dag = dAg[idx], dkb = dKb[idx];
                dq += dqt * eg;
                da += dag * eg;
                dk += dkb * ekc;
                const float kb = kk * ekc;
                dg += (dqt * qq + dag * aa) * eg - dkb * kb;
                e_col += dkb * kb;
                float sa = 0.f;
                if (ok) {
                    g.d_q[o] = dq;
                    if constexpr (VT::kGates) {
                        g.d_k[o] = dk + bg * da;
                        g.d_erase_b[o] = da * kk;
                    } else if constexpr (VT::kKaczmarz) {
                        dQt[idx] = dk + sbeta[r] * da;   // completed once d eta is known
                        sa = da * kk;
                    } else {
                        g.d_k[o] = dk + sbeta[r] * da;
                        sa = da * kk;
                    }
                }
                if constexpr (VT::kScalarBeta) {
                    sa = row16_sum(sa);
                    if (l16 == 0) atomicAdd(&ssa[r], sa);
                }
                if constexpr (VT::kChannelDecay) dGd[idx] = dg;
                if constexpr (kRowDecay) {
                    dg = row16_sum(dg);
                    if (l16 == 0) atomicAdd(&sdg[r], dg);
                }
            }
            if constexpr (VT::kChannelDecay) atomicAdd(&sdgc[col], e_col);
            if constexpr (kRowDecay) {
                e_col = wave_sum(e_col);
                if (lane == 0) atomicAdd(&sdgc[0], e_col);
            }
        }
        __syncthreads();
        // ---- I: step sizes, decay (reverse cumulative sum of dg within the chunk) ----
        if constexpr (VT::kScalarBeta) {
            if (tid < nvalid) {
                const float db = ssa[tid] + ssu[tid];
                if constexpr (VT::kKaczmarz) {
                    // beta = eta / n with n = |k|^2 + eps
                    g.d_beta[tok(tid)] = db / sn[tid];
                    scoef[tid] = -2.f * sbeta[tid] * db / sn[tid];
                } else {
                    g.d_beta[tok(tid)] = db;
                }
            }
        }
        if constexpr (VT::kChannelDecay) {
            if (tid < DK) {
                const int i = tid;
                float acc = sdgam[i] * __expf(Gd[(C - 1) * DK + i]) + sdgc[i];
                for (int r = C - 1; r >= 0; --r) {
                    acc += dGd[r * DK + i];
                    if (r < nvalid) {
                        // d/d alpha of the chunk form, whose log decay is
                        // floored: taken at the applied decay max(alpha, e^F)
                        const long o = tok(r) * DK + i;
                        g.d_alpha[o] = acc / fmaxf(p.alpha[o], kDecayFloor);
                    }
                }
            }
        } else if constexpr (kRowDecay) {
            if (wave == NW - 1) {
                float gsum = 0.f;
                for (int i = lane; i < DK; i += kWave) gsum += sdgam[i];
                const float dgC = wave_sum(gsum) * __expf(sG[C - 1]) + sdgc[0];
                // suffix sums over the rows: x_t + x_{t+1} + ... + x_{C-1}
                float x = sdg[lane] + svrow[lane] - svcol[lane];
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) {
                    const float y = __shfl_down(x, off, kWave);
                    if (lane + off < kWave) x += y;
                }
                if (lane < nvalid) g.d_alpha[tok(lane)] = (x + dgC) / p.alpha[tok(lane)];
            }
        }
        if constexpr (VT::kKaczmarz) {
            __syncthreads();
            for (int idx = tid; idx < C * DK; idx += NT) {
                const int r = idx / DK, i = idx % DK;
                if (r < nvalid) {
                    const long o = tok(r) * DK + i;
                    float kk;
                    if constexpr (kStageQK) kk = (float)sKt[i][r];   // still staged
                    else kk = f32(k[o]);
                    g.d_k[o] = dQt[idx] + scoef[r] * kk;
                }
            }
        }
    }
}

// The gradient's workspace: the forward's per-chunk factors of every chunk,
// then the per-chunk records of the two sequential passes and the reverse
// factors, then the per-chunk gradient workers' scratch.
template <typename TI, int DK, int DV> struct BwLayout {
    TI *S_chunks, *D_chunks, *dS_chunks, *dD_chunks;
    // dS_chunks is written only by the reverse chain: until then (in the
    // states pass) it serves as that pass's scratch.
    size_t dS_bytes;
    RevFactors rf;
    float *scratch;
    BwLayout(const Problem &p, void *ws) {
        char *base = static_cast<char *>(ws);
        const long NC = (p.T + C - 1) / C, nch = p.B * p.H * NC;
        auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
        size_t off = al(forward_states_bytes(p));
        S_chunks = reinterpret_cast<TI *>(base + off);
        off += al((size_t)nch * DK * DV * sizeof(TI));
        D_chunks = reinterpret_cast<TI *>(base + off);
        off += al((size_t)nch * C * DV * sizeof(TI));
        dS_chunks = reinterpret_cast<TI *>(base + off);
        dS_bytes = (size_t)nch * DK * DV * sizeof(TI);
        off += al(dS_bytes);
        dD_chunks = reinterpret_cast<TI *>(base + off);
        off += al((size_t)nch * C * DV * sizeof(TI));
        rf.Kb = base + off;
        off += al((size_t)nch * C * DK * sizeof(TI));
        rf.Wt = base + off;
        off += al((size_t)nch * DK * C * sizeof(TI));
        rf.X1 = base + off;
        off += al((size_t)nch * C * DV * sizeof(TI));
        rf.X2 = base + off;
        off += al((size_t)nch * DK * DV * sizeof(TI));
        scratch = reinterpret_cast<float *>(base + off);
    }
};

// The forward that keeps what its gradient needs: the gradient's states pass
// (the factors of every chunk, then the scan recording the state and Delta
// entering each chunk) with the scan also writing o and state_out.
template <typename TI, int DK, int DV>
hipError_t forward_save_shape(const Problem &p, void *ws, hipStream_t st) {
    const BwLayout<TI, DK, DV> L(p, ws);
    return launch_states_pass(p, ws, p.state_in, p.state_out, L.S_chunks, L.D_chunks, true,
                              L.dS_chunks, L.dS_bytes, st);
}

template <int V, typename TI, int DK, int DV>
hipError_t backward_shape(const Problem &p, const Grads &g, void *ws, bool saved, hipStream_t st) {
    const BwLayout<TI, DK, DV> L(p, ws);
    const long NC = (p.T + C - 1) / C;
    TI *const S_chunks = L.S_chunks, *const D_chunks = L.D_chunks;
    TI *const dS_chunks = L.dS_chunks, *const dD_chunks = L.dD_chunks;
    const RevFactors rf = L.rf;
    float *const scratch = L.scratch;

    // The states pass (in blocks for long bf16 sequences, as the forward),
    // then one pass per kernel over all chunks, in order on `st`.
    // (Overlapping the sequential passes with the parallel ones on a second
    // stream measured slower: the two kinds of kernel slow each other down
    // more than they overlap.)  With `saved`, the states pass already ran as
    // the forward that kept its records in this workspace.
    const ForwardStates f = forward_states_ptrs(p, ws);
    hipError_t e = hipSuccess;
    if (!saved && (e = launch_states_pass(p, ws, p.state_in, nullptr, S_chunks, D_chunks, false,
                                          dS_chunks, L.dS_bytes, st)) != hipSuccess)
        return e;
    const long items = NC * p.B * p.H;
    hipLaunchKernelGGL((bw_prep_kernel<TI, DK, DV>), dim3((unsigned)(items < 16384 ? items : 16384)),
                       dim3(kBpThreads), 0, st, p, f, g, rf, 0L, (int)NC);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const long nwg = p.B * p.H * (DV / 16);
    const unsigned chain_grid = (unsigned)(kXcds * ((nwg + kXcds - 1) / kXcds));
    constexpr int DEPTH = sizeof(TI) == 2 ? 2 : 1;
    // Where the forward runs in segments (few heads), so does the reverse
    // pass: every segment's transitions side by side, the serial combine
    // from d_state_out backwards, then every segment's recording chain from
    // its end state; the segments' arrays in the per-chunk gradient's
    // scratch, which that kernel only uses later.
    long SL = 0;   // chunks per segment
    const long nseg = sizeof(TI) == 2 ? forward_segments(p, &SL) : 0;
    const long BH = p.B * p.H;
    const size_t seg_floats = nseg > 1 ? (size_t)(nseg - 1) * BH * DK * (DK + 2 * DV) : 0;
    const bool rseg = nseg > 1 && seg_floats <= (size_t)kGradSlots * GradSlot<DK>::kFloats;
    if constexpr (sizeof(TI) == 2) {
        if (rseg) {
            float *Mo = scratch, *No = Mo + (nseg - 1) * BH * DK * DK;
            float *Se = No + (nseg - 1) * BH * DK * DV;
            const long nwg1 = BH * (DV / 16 + DK / 16);
            hipLaunchKernelGGL((rev_transition_kernel<DK, DV>),
                               dim3((unsigned)(kXcds * ((nwg1 + kXcds - 1) / kXcds)), (unsigned)(nseg - 1)),
                               dim3(4 * kWave), 0, st, p, f.gam, rf, NC, SL, nseg, Mo, No);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if ((e = launch_segment_combine(p, g.d_state_out, nseg, Mo, No, Se, st)) != hipSuccess) return e;
            hipLaunchKernelGGL((reverse_chain_kernel<TI, DK, 2>), dim3(chain_grid, (unsigned)nseg),
                               dim3(kRevThreads), 0, st, p, f.gam, rf, dS_chunks, dD_chunks, NC, 0L, (int)NC,
                               g.d_state_out, g.d_state_in, SL, static_cast<const float *>(Se));
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    if (!rseg) {
        hipLaunchKernelGGL((reverse_chain_kernel<TI, DK, DEPTH>), dim3(chain_grid), dim3(kRevThreads), 0, st,
                           p, f.gam, rf, dS_chunks, dD_chunks, NC, 0L, (int)NC, g.d_state_out,
                           g.d_state_in, 0L, static_cast<const float *>(nullptr));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    int dev = 0, cus = 0, per_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
        return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
             &per_cu, reinterpret_cast<const void *>(chunk_grad_kernel<V, TI, DK, DV>), kGradThreads,
             0)) != hipSuccess)
        return e;
    long slots = (long)cus * (per_cu > 0 ? per_cu : 1);
    if (slots > kGradSlots) slots = kGradSlots;
    hipLaunchKernelGGL((chunk_grad_kernel<V, TI, DK, DV>), dim3((unsigned)(items < slots ? items : slots)),
                       dim3(kGradThreads), 0, st, p, g, S_chunks, D_chunks, dS_chunks, dD_chunks,
                       scratch, 0L, (int)NC);
    return hipGetLastError();
}

template <int V, typename TI>
hipError_t backward_t(const Problem &p, const Grads &g, void *ws, bool saved, hipStream_t st) {
    if (p.dk == 128 && p.dv == 128) return backward_shape<V, TI, 128, 128>(p, g, ws, saved, st);
    if (p.dk == 128 && p.dv == 64) return backward_shape<V, TI, 128, 64>(p, g, ws, saved, st);
    if (p.dk == 64 && p.dv == 128) return backward_shape<V, TI, 64, 128>(p, g, ws, saved, st);
    return backward_shape<V, TI, 64, 64>(p, g, ws, saved, st);
}

template <int V>
hipError_t backward_v(const Problem &p, const Grads &g, void *ws, bool saved, hipStream_t st) {
    return p.bf16 ? backward_t<V, bf16>(p, g, ws, saved, st)
                  : backward_t<V, float>(p, g, ws, saved, st);
}

template <typename TI> hipError_t forward_save_t(const Problem &p, void *ws, hipStream_t st) {
    if (p.dk == 128 && p.dv == 128) return forward_save_shape<TI, 128, 128>(p, ws, st);
    if (p.dk == 128 && p.dv == 64) return forward_save_shape<TI, 128, 64>(p, ws, st);
    if (p.dk == 64 && p.dv == 128) return forward_save_shape<TI, 64, 128>(p, ws, st);
    return forward_save_shape<TI, 64, 64>(p, ws, st);
}

}  // namespace

size_t backward_workspace_bytes(const Problem &p) {
    const long NC = (p.T + C - 1) / C, nch = p.B * p.H * NC;
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t es = p.bf16 ? 2 : 4;
    const size_t slot = (size_t)(10 * C * p.dk + 2 * C * C) * 4;
    return al(forward_states_bytes(p)) + 3 * al((size_t)nch * p.dk * p.dv * es) +
           3 * al((size_t)nch * C * p.dv * es) + 2 * al((size_t)nch * C * p.dk * es) +
           kGradSlots * slot;
}

hipError_t launch_backward(const Problem &p, const Grads &g, void *workspace, bool saved,
                           hipStream_t stream) {
    switch (p.variant) {
    case kDeltaNet: return backward_v<kDeltaNet>(p, g, workspace, saved, stream);
    case kGatedDeltaNet: return backward_v<kGatedDeltaNet>(p, g, workspace, saved, stream);
    case kKDA: return backward_v<kKDA>(p, g, workspace, saved, stream);
    case kGDN2: return backward_v<kGDN2>(p, g, workspace, saved, stream);
    case kKLA: return backward_v<kKLA>(p, g, workspace, saved, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_forward_save(const Problem &p, void *workspace, hipStream_t stream) {
    if (p.variant < kDeltaNet || p.variant > kKLA) return hipErrorInvalidValue;
    return p.bf16 ? forward_save_t<bf16>(p, workspace, stream)
                  : forward_save_t<float>(p, workspace, stream);
}

}  // namespace gdr
