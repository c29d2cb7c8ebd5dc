// forward.hip -- chunkwise-parallel prefill of the gated delta rule on gfx950.
//
// The sequence of every (b, h) is cut into chunks of C = 64 tokens.  Inside a
// chunk, with g_r = sum_{j<=r} log alpha_j (inclusive, per key channel i for
// channel-wise decay) and the chunk's incoming state S, the recurrence
//     S_t = (I - k_t a_t^T) D_t S_{t-1} + k_t u_t^T,   o_t = S_t^T q_t
// unrolls to the closed form (an algebraic identity, not an approximation):
//     A[r][s] = sum_i a_r[i] k_s[i] e^{g_r[i] - g_s[i]}      (s <  r)
//     P[r][s] = sum_i q_r[i] k_s[i] e^{g_r[i] - g_s[i]}      (s <= r)
//     T = (I + A)^{-1}              (unit lower triangular)
//     W = T (a (.) e^{g}),   U~ = T U
//     Delta = U~ - W S
//     O = (q (.) e^{g}) S + P Delta
//     S' = Diag(e^{g_C}) S + (k (.) e^{g_C - g})^T Delta
// This is the chunk-wise parallel form that the pages keep for every variant
// ("Kaczmarz Linear Attention", Implementation section: only the per-chunk
// diagonal coefficient matrix Diag(beta_1..beta_C) changes; "Gated
// DeltaNet-2", technical core: a chunkwise WY algorithm in which the
// channel-wise decay is absorbed into an asymmetric erase factor -- here the
// left factor a (.) e^{g} differs from the right factor k (.) e^{-g}).  The
// derivation and the kernel design are our own.
//
// Two kernels:
//   chunk_prep  fully parallel over (chunk, h, b): persistent workgroups that
//               loop over chunk-heads (bf16; one workgroup per chunk-head for
//               fp32).  Gate prefix sums, the two 64x64 Gram products A and P
//               on bf16 matrix cores (fp32 accumulate), the unit-lower-
//               triangular inverse T in LDS (fp32; 16x16 diagonal blocks by
//               substitution, off-diagonal blocks by a 2 x 2 block recursion),
//               then W and U~ on matrix cores.  It writes per-chunk factors W,
//               U~^T, q(.)e^{g}, K-bar^T, P and e^{g_C} to the workspace.
//   chunk_scan  one workgroup per (slice of 16*NJ value columns, h, b): the
//               sequential pass over chunks.  Columns of S evolve independently
//               given the chunk factors, so the state is split by value
//               columns; each wave keeps its rows of S in fp32 MFMA
//               accumulators for the whole sequence and a bf16 copy of S^T in
//               LDS feeds the products.  The next chunk's factors are loaded
//               while the current one is computed.
// A long bf16 sequence runs as blocks of 64 chunks, the prep of block i + 1
// beside the scan of block i (see launch_shape).
//
// All products are written as D = A * B^T over a K-contiguous pair of
// operands, so every fragment is one 16-byte load; operand order is chosen so
// that each lane's four accumulator values are four consecutive elements of
// the destination.  The chunk factors are stored fragment-major, so the scan
// reads each operand tile as one contiguous 1 KB block.
#include <atomic>
#include <type_traits>

#include "gdr_device.hpp"

namespace gdr {
namespace {

constexpr int C = kChunk;          // chunk length
constexpr int kPrepThreads = 256;
constexpr int kXcds = 8;           // accelerator complex dies per MI355X

// Per chunk-head factors, each block contiguous; the operand factors are
// stored fragment-major (frag_off / ufrag_off below).
template <typename TI> struct WsPtrs {
    TI *W;     // [nch] C x DK    T (a (.) e^{g})
    TI *Ut;    // [nch] DV x C    (T U)^T, accumulator layout
    TI *Qt;    // [nch] C x DK    q (.) e^{g}
    TI *Kbt;   // [nch] DK x C    (k (.) e^{g_C - g})^T
    TI *P;     // [nch] C x C     decayed q k^T, lower triangle incl. diagonal
    float *gam;// [nch][DK]       e^{g_C}
};

// A block of consecutive chunks processed by one prep launch and one scan
// launch.  The workspace holds the factors of `nbmax` chunks per head; the
// state enters from s_in (NULL = zeros) and leaves to s_out (NULL = dropped).
struct Block {
    long c0;             // first chunk of the block
    int nc;              // chunks in the block
    int nbmax;           // chunk stride of the workspace slot
    const float *s_in;
    float *s_out;
    void *s_chunks;      // states-only scans: the state entering each chunk, [B*H][nbmax][dk][dv]
    void *d_chunks;      //   and each chunk's Delta, [B*H][nbmax][C][dv], both in the input dtype
    // bf16 prep beside a concurrent scan: after its first item, a workgroup
    // takes its next one from a shared ticket counter (NULL = every
    // gridDim.x-th item).  Every item processed draws one ticket, so a launch
    // advances the counter by exactly its item count; ticket_base is the
    // counter's value when the launch starts.  ticket_clear (if not NULL) is
    // set to zero by the launch, for the launches after it.
    unsigned *ticket;
    unsigned ticket_base;
    unsigned *ticket_clear;
    // Scan: write o with streaming (non-temporal) stores (a separate kernel
    // instance).  A 16-column slice writes 32 of each token row's bytes; in
    // the pipelined forward, keeping these partial lines out of the caches
    // leaves them to the next block's factors.
    bool nt_out;
    // Scan with s_chunks: also write o (and s_out), i.e. the forward that
    // keeps what its gradient needs; otherwise the states alone.
    bool with_o = false;
};

struct WsLayout {
    size_t W, Ut, Qt, Kbt, P, gam, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Layout of one workspace slot holding `nbmax` chunks for every head.
WsLayout ws_layout(const Problem &p, long nbmax) {
    const size_t es = p.bf16 ? 2 : 4;
    const size_t nch = (size_t)p.B * p.H * nbmax;
    WsLayout L;
    size_t o = 0;
    L.W = o;   o = align256(o + nch * C * p.dk * es);
    L.Ut = o;  o = align256(o + nch * C * p.dv * es);
    L.Qt = o;  o = align256(o + nch * C * p.dk * es);
    L.Kbt = o; o = align256(o + nch * C * p.dk * es);
    L.P = o;   o = align256(o + nch * C * C * es);
    L.gam = o; o = align256(o + nch * p.dk * 4);
    L.total = o;
    return L;
}

template <typename TI> WsPtrs<TI> ws_ptrs(const Problem &p, long nbmax, void *base) {
    WsLayout L = ws_layout(p, nbmax);
    char *b = static_cast<char *>(base);
    return WsPtrs<TI>{reinterpret_cast<TI *>(b + L.W), reinterpret_cast<TI *>(b + L.Ut),
                      reinterpret_cast<TI *>(b + L.Qt), reinterpret_cast<TI *>(b + L.Kbt),
                      reinterpret_cast<TI *>(b + L.P), reinterpret_cast<float *>(b + L.gam)};
}

// Execution plan of one forward: the sequence is cut into blocks of `nb`
// chunks.  With more than one block, two workspace slots alternate and an fp32
// state carrier passes the state from block to block.
struct Plan {
    long NC, nb, nblk;
    size_t slot, carrier, ticket, total;
};

constexpr long kBlockChunks = 64;
constexpr long kPipelineChunks = 512;          // pipeline from this many chunks on
constexpr size_t kSinglePassBytes = 1ull << 30;  // or when one pass's factors exceed this

hipError_t device_cus(long *out);   // compute units of the current device

Plan make_plan(const Problem &p) {
    Plan q;
    q.NC = (p.T + C - 1) / C;
    // Long bf16 sequences are pipelined in blocks of 64 chunks: the scan then
    // reads factors the prep has just written, still in the caches.  Below
    // that the prep and the scan run as one pass each, which measured faster:
    // with few blocks there is little to overlap, and the two kernels slow
    // each other down.  A channel decay's heavier prep gains from the overlap
    // from half that length, and so does a scalar decay's when its scan
    // (16-column slices) takes more than a quarter and at most half of the
    // compute units: fewer leave each block's prep too little to do, more
    // leave it too few units.  The single pass's workspace is capped.
    const bool channel = p.variant == kKDA || p.variant == kGDN2;
    long cus = 0;
    const long slices = p.B * p.H * (p.dv / 16);
    const bool half =
        device_cus(&cus) == hipSuccess && slices > cus / 4 && slices <= cus / 2;
    const long from = (channel || half) ? kPipelineChunks / 2 : kPipelineChunks;
    const bool pipe = p.bf16 && q.NC > kBlockChunks &&
                      (q.NC >= from || ws_layout(p, q.NC).total > kSinglePassBytes);
    q.nb = pipe ? kBlockChunks : q.NC;
    q.nblk = (q.NC + q.nb - 1) / q.nb;
    q.slot = ws_layout(p, q.nb).total;
    q.carrier = q.nblk > 1 ? align256((size_t)p.B * p.H * p.dk * p.dv * 4) : 0;
    q.ticket = q.nblk > 1 ? 256 : 0;   // the prep's ticket counter
    q.total = (q.nblk > 1 ? 2 : 1) * q.slot + q.carrier + q.ticket;
    return q;
}

// Sequence-parallel plan.  When the chain's column slices would occupy at
// most a quarter of the compute units (few heads: B * H * d_v / 16 small),
// the sequence is cut into segments of L chunks whose chains run side by
// side: the prep over every chunk; each segment but the last from S = 0 (its
// local end state N_s) and from the identity with U~ = 0 (its transition M_s,
// the product of the chunks' maps S -> (Diag(e^{g_C}) - Kbar^T W) S); a short
// serial combine S_{s+1} = M_s S_s + N_s from the initial state; then every
// segment's scan from its start state, writing o.  The state update of a chunk
// is affine in S, so this is the same recurrence.
struct SegPlan {
    long nseg = 0;                     // segments (0: the plan is not used)
    long L = 0;                        // chunks per segment, the last one shorter
    size_t M = 0, N = 0, S = 0;        // byte offsets: M_s, N_s, start states
    size_t total = 0;
};
constexpr long kSegMinChunks = 16;     // chunks per segment at least
constexpr long kSegMinTotal = 64;      // chunks of the sequence at least
constexpr long kSegMax = 16;           // segments at most

SegPlan seg_plan(const Problem &p) {
    SegPlan s;
    long cus = 0;
    if (!p.bf16 || device_cus(&cus) != hipSuccess) return s;
    const long NC = (p.T + C - 1) / C, BH = p.B * p.H;
    const long slices = BH * (p.dv / 16);
    if (4 * slices > cus || NC < kSegMinTotal) return s;
    long nseg = cus / slices;
    if (nseg > NC / kSegMinChunks) nseg = NC / kSegMinChunks;
    if (nseg > kSegMax) nseg = kSegMax;
    if (nseg < 2) return s;
    const long L = (NC + nseg - 1) / nseg;
    nseg = (NC + L - 1) / L;
    if (nseg < 2) return s;
    size_t o = ws_layout(p, NC).total;
    s.M = o; o = align256(o + (size_t)(nseg - 1) * BH * p.dk * p.dk * 4);
    s.N = o; o = align256(o + (size_t)(nseg - 1) * BH * p.dk * p.dv * 4);
    s.S = o; o = align256(o + (size_t)(nseg - 1) * BH * p.dk * p.dv * 4);
    if (o > kSinglePassBytes || (p.ws_cap && o > p.ws_cap)) return s;
    s.nseg = nseg;
    s.L = L;
    s.total = o;
    return s;
}

// ---- small vector stores ------------------------------------------------------

__device__ __forceinline__ void store8(bf16 *dst, const float *x) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
    *reinterpret_cast<bf16x8 *>(dst) = v;
}
__device__ __forceinline__ void store8(float *dst, const float *x) {
    *reinterpret_cast<f32x4 *>(dst) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
// kPerLane consecutive input elements as floats (8 for bf16, 1 for fp32).
__device__ __forceinline__ void load_lane(const bf16 *src, float *x) {
    bf16x8 v = *reinterpret_cast<const bf16x8 *>(src);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void load_lane(const float *src, float *x) { x[0] = *src; }


// Four (bf16: one 8-byte store) or eight (one 16-byte store) consecutive k.
__device__ __forceinline__ void store_frag4(bf16 *base, int r, int k, int K, f32x4 x) {
    store4(base + frag_off<bf16>(r, k, K), x);
}
__device__ __forceinline__ void store_frag4(float *base, int r, int k, int K, f32x4 x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) base[frag_off<float>(r, k + e, K)] = x[e];
}
__device__ __forceinline__ void store_frag8(bf16 *base, int r, int k, int K, const float *x) {
    store8(base + frag_off<bf16>(r, k, K), x);
}
__device__ __forceinline__ void store_frag8(float *base, int r, int k, int K, const float *x) {
#pragma unroll
    for (int e = 0; e < 8; ++e) base[frag_off<float>(r, k + e, K)] = x[e];
}
// The ten lower-triangular 16x16 tiles (R >= S) of a 64x64 matrix in row
// order, and the six strictly upper ones, as arithmetic on the tile number
// (no table: a table read is a memory load, and its wait would also wait for
// every load issued before it).
__device__ __forceinline__ int lower_r(int t) { return (t >= 1) + (t >= 3) + (t >= 6); }
__device__ __forceinline__ int lower_s(int t) {
    const int r = lower_r(t);
    return t - r * (r + 1) / 2;
}
__device__ __forceinline__ int upper_r(int t) { return (t >= 3) + (t >= 5); }
__device__ __forceinline__ int upper_s(int t) { return t + 1 - 2 * (t >= 3) - (t >= 5); }

// ============================================================================
// chunk_prep
// ============================================================================
template <int V, typename TI, int DK, int DV>
__global__ __launch_bounds__(kPrepThreads) void chunk_prep_kernel(Problem p, WsPtrs<TI> ws, Block blk) {
    using VT = VariantTraits<V>;
    using M = Mma<TI>;
    constexpr int PT = 8;                                  // pad (elements) of TI tiles
    constexpr int PF = 4;                                  // pad of fp32 tiles
    constexpr int GW = VT::kChannelDecay ? DK : 1;         // width of a g row
    constexpr int NL = M::kPerLane;

    __shared__ __attribute__((aligned(16))) float sG[C][GW];
    __shared__ float sBeta[C];
    __shared__ __attribute__((aligned(16))) TI sAt[DK][C + PT];   // (a (.) e^{g})^T
    __shared__ __attribute__((aligned(16))) TI sUt[DV][C + PT];   // U^T
    __shared__ __attribute__((aligned(16))) float sAm[C][C + PF]; // A (strictly lower)
    __shared__ __attribute__((aligned(16))) float sT[C][C + PF];  // T = (I + A)^{-1}
    __shared__ float sX[3][16][17];
    __shared__ float sRk[C], sRq[C];   // 1/|k_r|, 1/|q_r| with the q/k normalisation, else 1

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool l2 = p.flags & kQkL2Norm, rawg = p.flags & kRawGates;
    const float ds = p.decay_scale;
    const int l16 = lane & 15, lg = lane >> 4;
    const long c = blk.c0 + blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    const long T = p.T;
    const int H = (int)p.H;
    const long t0 = c * C;
    const int nvalid = (int)min((long)C, T - t0);
    const long ch = ((long)b * H + h) * blk.nbmax + blockIdx.x;   // slot-local chunk-head
    const TI *q = static_cast<const TI *>(p.q);
    const TI *k = static_cast<const TI *>(p.k);
    const TI *v = static_cast<const TI *>(p.v);
    auto tok = [&](int r) -> long { return ((long)b * T + t0 + r) * H + h; };

    // ---- phase 0: row norms, decay prefix sums, per-token write strength -----
    // |k_r|^2 and |q_r|^2 over the key channels, one wave per row: each wave
    // issues the loads of all its rows before the first reduction, so that
    // they wait once instead of once per row.
    constexpr int kNW = kPrepThreads / kWave, kRPW = C / kNW, kEPL = (DK + kWave - 1) / kWave;
    float kx[kRPW][kEPL], qx[kRPW][kEPL];
#pragma unroll
    for (int n = 0; n < kRPW; ++n) {
        const int r = wave + kNW * n;
#pragma unroll
        for (int e = 0; e < kEPL; ++e) {
            const int i = lane + kWave * e;
            const bool ok = r < nvalid && i < DK;
            kx[n][e] = ok ? to_f32(k[tok(r) * DK + i]) : 0.f;
            qx[n][e] = ok ? to_f32(q[tok(r) * DK + i]) : 0.f;
        }
    }
#pragma unroll
    for (int n = 0; n < kRPW; ++n) {
        const int r = wave + kNW * n;
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int e = 0; e < kEPL; ++e) {
            sk += kx[n][e] * kx[n][e];
            sq += qx[n][e] * qx[n][e];
        }
        sk = wave_sum(sk);
        sq = wave_sum(sq);
        if (lane == 0) {
            const float rk = l2 ? rsqrtf(sk + kL2NormEps) : 1.f;
            sRk[r] = rk;
            sRq[r] = l2 ? rsqrtf(sq + kL2NormEps) : 1.f;
            // beta_r = eta_r / (|k_r|^2 + eps) for KLA, |k_r| of the key in use.
            if constexpr (VT::kKaczmarz) {
                const float eta = r < nvalid ? p.beta[tok(r)] : 0.f;
                sBeta[r] = r < nvalid ? (rawg ? sigmoid_f(eta) : eta) / (sk * rk * rk + p.eps) : 0.f;
            }
        }
    }
    if constexpr (VT::kChannelDecay) {
        if (tid < DK) {
            float g = 0.f;
            for (int r = 0; r < C; ++r) {
                if (r < nvalid) g += fmaxf(log_decay(p.alpha[tok(r) * DK + tid], rawg, ds), kLogDecayFloor);
                sG[r][tid] = g;
            }
        }
    } else if constexpr (VT::kHasDecay) {
        if (wave == 0) {
            float g = lane < nvalid ? log_decay(p.alpha[tok(lane)], rawg, ds) : 0.f;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                float y = __shfl_up(g, off, kWave);
                if (lane >= off) g += y;
            }
            sG[lane][0] = g;
        }
    } else {
        if (tid < C) sG[tid][0] = 0.f;
    }
    if constexpr (VT::kScalarBeta && !VT::kKaczmarz) {
        if (tid < C) {
            const float bt = tid < nvalid ? p.beta[tok(tid)] : 0.f;
            sBeta[tid] = tid < nvalid ? (rawg ? sigmoid_f(bt) : bt) : 0.f;
        }
    }
    __syncthreads();

    // ---- phase 1: element-wise factors ------------------------------------
    // Thread -> key channel i and groups of 8 consecutive rows, so that the
    // transposed tiles get 16-byte writes and the global reads of a row are
    // coalesced across lanes.
    {
        const int i = tid % DK;
        const float gC = sG[C - 1][VT::kChannelDecay ? i : 0];
        if (tid < DK) ws.gam[ch * DK + i] = VT::kHasDecay ? __expf(gC) : 1.f;
        for (int r0 = 8 * (tid / DK); r0 < C; r0 += 8 * (kPrepThreads / DK)) {
            float at[8], kb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = r0 + e;
                float kk = 0.f, qq = 0.f, a = 0.f;
                if (r < nvalid) {
                    kk = to_f32(k[tok(r) * DK + i]) * sRk[r];
                    qq = to_f32(q[tok(r) * DK + i]) * sRq[r];
                    if constexpr (VT::kGates) {
                        const float bg = p.erase_b[tok(r) * DK + i];
                        a = (rawg ? sigmoid_f(bg) : bg) * kk;
                    } else {
                        a = sBeta[r] * kk;
                    }
                }
                float eg = 1.f, egc = 1.f;
                if constexpr (VT::kHasDecay) {
                    const float g = sG[r][VT::kChannelDecay ? i : 0];
                    eg = __expf(g);
                    egc = __expf(gC - g);
                }
                at[e] = a * eg;
                kb[e] = kk * egc;
                ws.Qt[ch * C * DK + frag_off<TI>(r, i, DK)] = from_f32<TI>(qq * eg);
            }
            store8(&sAt[i][r0], at);
            store_frag8(ws.Kbt + ch * DK * C, i, r0, C, kb);
        }
        const int j = tid % DV;
        for (int r0 = 8 * (tid / DV); r0 < C; r0 += 8 * (kPrepThreads / DV)) {
            float u[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = r0 + e;
                float uu = 0.f;
                if (r < nvalid) {
                    float vv = to_f32(v[tok(r) * DV + j]);
                    if (p.v_route) vv += to_f32(static_cast<const TI *>(p.v_route)[tok(r) * DV + j]);
                    if constexpr (VT::kGates) {
                        const float wg = p.write_w[tok(r) * DV + j];
                        uu = (rawg ? sigmoid_f(wg) : wg) * vv;
                    } else {
                        uu = sBeta[r] * vv;
                    }
                }
                u[e] = uu;
            }
            store8(&sUt[j][r0], u);
        }
    }

    // ---- phase 2: A and P on matrix cores -----------------------------------
    // Computed transposed, D'(s, r) = sum_i Kr[s][i] L[r][i], so a lane holds
    // four consecutive s of one row r.  Channel-wise decay is split between
    // the operands around the reference m_R = (g_{16R} + g_{16R+15}) / 2 of the
    // tile's row block R: the left factor e^{g_r - m_R} and the right factor
    // e^{m_R - g_s} each stay within e^{+-7.5 F} (F the log-decay floor), and
    // off the diagonal (s in an earlier block) the right one is at most 1.
    // Scalar decay is applied to the product as e^{g_r - g_s} <= 1.
    for (int tl = wave; tl < 10; tl += kPrepThreads / kWave) {
        const int R = lower_r(tl), S = lower_s(tl);
        const int rs = 16 * S + l16;   // row supplying the K_R operand
        const int rr = 16 * R + l16;   // row supplying the A_L / Q_L operands
        f32x4 accA = zero4(), accP = zero4();
        float br = 0.f;
        if constexpr (VT::kScalarBeta) br = sBeta[rr];
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += M::kK) {
            const int kb = k0 + NL * lg;   // first key channel of this lane's slice
            float kr[NL], ar[NL], qr[NL];
            if (rs < nvalid) load_lane(&k[tok(rs) * DK + kb], kr);
            else {
#pragma unroll
                for (int e = 0; e < NL; ++e) kr[e] = 0.f;
            }
            if (rr < nvalid) {
                load_lane(&k[tok(rr) * DK + kb], ar);
                load_lane(&q[tok(rr) * DK + kb], qr);
            } else {
#pragma unroll
                for (int e = 0; e < NL; ++e) ar[e] = qr[e] = 0.f;
            }
            const float rks = sRk[rs], rkr = sRk[rr], rqr = sRq[rr];
#pragma unroll
            for (int e = 0; e < NL; ++e) {
                kr[e] *= rks;
                ar[e] *= rkr;
                qr[e] *= rqr;
                float a;
                if constexpr (VT::kGates) {
                    float bg = rr < nvalid ? p.erase_b[tok(rr) * DK + kb + e] : 0.f;
                    if (rawg) bg = sigmoid_f(bg);
                    a = rr < nvalid ? bg * ar[e] : 0.f;
                } else {
                    a = br * ar[e];
                }
                if constexpr (VT::kChannelDecay) {
                    const float gref = 0.5f * (sG[16 * R][kb + e] + sG[16 * R + 15][kb + e]);
                    const float fl = __expf(sG[rr][kb + e] - gref);
                    kr[e] *= __expf(gref - sG[rs][kb + e]);
                    a *= fl;
                    qr[e] *= fl;
                }
                ar[e] = a;
            }
            const typename M::frag fk = M::from_f32x8(kr);
            accA = M::mma(fk, M::from_f32x8(ar), accA);
            accP = M::mma(fk, M::from_f32x8(qr), accP);
        }
        // lane: row r = rr, columns s = 16 S + 4 lg + m
        const int r = rr;
        f32x4 Av, Pv;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int s = 16 * S + 4 * lg + m;
            float f = 1.f;
            if constexpr (VT::kHasDecay && !VT::kChannelDecay)
                f = s <= r ? __expf(sG[r][0] - sG[s][0]) : 0.f;
            Av[m] = s < r ? accA[m] * f : 0.f;
            Pv[m] = s <= r ? accP[m] * f : 0.f;
        }
        *reinterpret_cast<f32x4 *>(&sAm[r][16 * S + 4 * lg]) = Av;
        store_frag4(ws.P + ch * C * C, r, 16 * S + 4 * lg, C, Pv);
    }
    for (int idx = tid; idx < 6 * 16 * 4; idx += kPrepThreads) {
        // zero the strictly upper tiles of P (4 values per thread-step)
        const int t6 = idx / 64, e = idx % 64;
        const int r = 16 * upper_r(t6) + e / 4;
        const int s = 16 * upper_s(t6) + 4 * (e % 4);
        store_frag4(ws.P + ch * C * C, r, s, C, zero4());
    }
    __syncthreads();

    // ---- phase 3: T = (I + A)^{-1} ------------------------------------------
    if (wave == 0) {
        // Diagonal blocks by forward substitution; lane = (block, column).
        const int R = lg, cc = l16;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < r; ++j) acc += sAm[16 * R + r][16 * R + j] * x[j];
            x[r] = r == cc ? 1.f : (r < cc ? 0.f : -acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[16 * R + r][16 * R + cc] = x[r];
    } else {
        for (int idx = tid - kWave; idx < 6 * 256; idx += kPrepThreads - kWave) {
            const int t6 = idx >> 8, e = idx & 255;
            sT[16 * upper_r(t6) + (e >> 4)][16 * upper_s(t6) + (e & 15)] = 0.f;
        }
    }
    __syncthreads();
    // Off-diagonal blocks by distance d = R - S:
    //   T_RS = -T_RR * sum_{J=S}^{R-1} A_RJ T_JS
    for (int d = 1; d < 4; ++d) {
        const int nb = 4 - d;
        for (int idx = tid; idx < nb * 256; idx += kPrepThreads) {
            const int blk = idx >> 8, e = idx & 255;
            const int R = d + blk, S = R - d, r = e >> 4, cc = e & 15;
            float acc = 0.f;
            for (int J = S; J < R; ++J)
#pragma unroll
                for (int jj = 0; jj < 16; ++jj)
                    acc += sAm[16 * R + r][16 * J + jj] * sT[16 * J + jj][16 * S + cc];
            sX[blk][r][cc] = acc;
        }
        __syncthreads();
        for (int idx = tid; idx < nb * 256; idx += kPrepThreads) {
            const int blk = idx >> 8, e = idx & 255;
            const int R = d + blk, S = R - d, r = e >> 4, cc = e & 15;
            float acc = 0.f;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj)
                acc += sT[16 * R + r][16 * R + jj] * sX[blk][jj][cc];
            sT[16 * R + r][16 * S + cc] = -acc;
        }
        __syncthreads();
    }

    // ---- phase 4: W = T (a (.) e^{g}) and U~ = T U on matrix cores -----------
    {
        const int R = wave;                                   // row tile of T
        const int nK = (16 * (R + 1) + M::kK - 1) / M::kK;    // K-steps covering s <= r
        typename M::frag Tf[C / M::kK];
#pragma unroll
        for (int ks = 0; ks < C / M::kK; ++ks) {
            if (ks < nK) {
                float tmp[8];
#pragma unroll
                for (int e = 0; e < NL; ++e) tmp[e] = sT[16 * R + l16][ks * M::kK + NL * lg + e];
                Tf[ks] = M::from_f32x8(tmp);
            }
        }
        // W'(i, r) = sum_s At[i][s] T[r][s]: lane holds W[r][i .. i+3].
#pragma unroll 2
        for (int mi = 0; mi < DK / 16; ++mi) {
            f32x4 acc = zero4();
            const TI *arow = &sAt[16 * mi + l16][0];
#pragma unroll
            for (int ks = 0; ks < C / M::kK; ++ks)
                if (ks < nK) acc = M::mma(M::load(arow, ks * M::kK, lane), Tf[ks], acc);
            store_frag4(ws.W + ch * C * DK, 16 * R + l16, 16 * mi + 4 * lg, DK, acc);
        }
        // U~(r, j) = sum_s T[r][s] Ut[j][s]: lane holds U~^T[j][r .. r+3].
#pragma unroll 2
        for (int nj = 0; nj < DV / 16; ++nj) {
            f32x4 acc = zero4();
            const TI *urow = &sUt[16 * nj + l16][0];
#pragma unroll
            for (int ks = 0; ks < C / M::kK; ++ks)
                if (ks < nK) acc = M::mma(Tf[ks], M::load(urow, ks * M::kK, lane), acc);
            store4(ws.Ut + ch * DV * C + ufrag_off(16 * nj + l16, 16 * R + 4 * lg), acc);
        }
    }
}

// ============================================================================
// chunk_prep, bf16 inputs: the same factors as chunk_prep_kernel, restructured
// for memory-level parallelism and occupancy.  All global reads of the chunk
// are issued at once before any arithmetic; eight waves share the work; LDS
// tiles are unpadded with an XOR swizzle of their 16-byte chunks and are
// reused as the phases retire them, so that for scalar-decay variants two
// workgroups fit on a CU and one's loads overlap the other's arithmetic.  q is
// kept in registers rather than LDS.
// ============================================================================
constexpr int kPrep2Threads = 512;

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (bf16)0.f;
    return z;
}

// Element offset in an unpadded tile with CPR 16-byte chunks per row whose
// chunk index is XORed with the row: sixteen lanes reading one column chunk of
// sixteen consecutive rows touch distinct banks.  EPC = elements per chunk.
template <int CPR, int EPC> __device__ __forceinline__ int swz(int r, int col) {
    return (r * CPR + ((col / EPC) ^ (r & (CPR - 1)))) * EPC + col % EPC;
}

// Raw global inputs of one chunk-head, held in registers from the issue of
// their loads (during the previous chunk-head's arithmetic) to their use.  The
// loads are unconditional (rows past T read the last valid row) so that the
// compiler's waits for them stay exact; staging masks those rows.  q is held
// here only with a channel decay; otherwise each wave loads its own q rows in
// the matrix-core fragment layout (the kernel's qf).
template <int V, int DK, int DV, bool RT> struct PrepRaw {
    using VT = VariantTraits<V>;
    static constexpr int NT = kPrep2Threads;
    static constexpr int KC = DK / 8, VC = DV / 8;            // 16-byte chunks per row
    static constexpr int NQ = C * KC / NT;                     // q / k chunks per thread
    static constexpr int NV = C * VC / NT;                     // v chunks per thread
    static constexpr int NA = VT::kChannelDecay ? C * DK / 4 / NT : 1;
    static_assert(C * KC % NT == 0 && C * VC % NT == 0 && C * DK / 4 % NT == 0, "whole passes");
    static constexpr int NQR = VT::kChannelDecay ? NQ : 1;   // q chunks held here
    bf16x8 k[NQ], q[NQR], v[NV], vr[RT ? NV : 1];   // vr: the routed value
    f32x4 eb[VT::kGates ? 2 * NQ : 1], ww[VT::kGates ? 2 * NV : 1];   // erase / write gates
    f32x4 al[NA];                                              // channel-wise alpha
    float a1, be;                                              // scalar alpha, beta / eta

    __device__ __forceinline__ void issue(const Problem &p, long c, int h, int b, int tid) {
        const long T = p.T, t0 = c * C;
        const int H = (int)p.H;
        const int last = (int)min((long)C, T - t0) - 1;
        auto tok = [&](int r) -> long { return ((long)b * T + t0 + (r < last ? r : last)) * H + h; };
        const bf16 *qp = static_cast<const bf16 *>(p.q);
        const bf16 *kp = static_cast<const bf16 *>(p.k);
        const bf16 *vp = static_cast<const bf16 *>(p.v);
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int idx = tid + n * NT;
            const int r = idx / KC, pc = idx % KC;
            k[n] = *reinterpret_cast<const bf16x8 *>(&kp[tok(r) * DK + 8 * pc]);
            if constexpr (VT::kChannelDecay)
                q[n] = *reinterpret_cast<const bf16x8 *>(&qp[tok(r) * DK + 8 * pc]);
            if constexpr (VT::kGates) {
                eb[2 * n] = *reinterpret_cast<const f32x4 *>(&p.erase_b[tok(r) * DK + 8 * pc]);
                eb[2 * n + 1] = *reinterpret_cast<const f32x4 *>(&p.erase_b[tok(r) * DK + 8 * pc + 4]);
            }
        }
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            const int idx = tid + n * NT;
            const int r = idx / VC, pc = idx % VC;
            v[n] = *reinterpret_cast<const bf16x8 *>(&vp[tok(r) * DV + 8 * pc]);
            if constexpr (RT)
                vr[n] = *reinterpret_cast<const bf16x8 *>(
                    &static_cast<const bf16 *>(p.v_route)[tok(r) * DV + 8 * pc]);
            if constexpr (VT::kGates) {
                ww[2 * n] = *reinterpret_cast<const f32x4 *>(&p.write_w[tok(r) * DV + 8 * pc]);
                ww[2 * n + 1] = *reinterpret_cast<const f32x4 *>(&p.write_w[tok(r) * DV + 8 * pc + 4]);
            }
        }
        if constexpr (VT::kChannelDecay) {
#pragma unroll
            for (int n = 0; n < NA; ++n) {
                const int idx = tid + n * NT;
                const int r = idx / (DK / 4), i4 = 4 * (idx % (DK / 4));
                al[n] = *reinterpret_cast<const f32x4 *>(&p.alpha[tok(r) * DK + i4]);
            }
        } else if constexpr (VT::kHasDecay) {
            a1 = p.alpha[tok(tid & (kWave - 1))];
        }
        if constexpr (VT::kScalarBeta) be = p.beta[tok(tid & (C - 1))];
    }
};

// The prep's LDS tiles (one workgroup's).
template <int V, int DK, int DV> struct PrepSmem {
    using VT = VariantTraits<V>;
    static constexpr int GW = VT::kChannelDecay ? DK : 1;
    static constexpr int R1 = C * DK * 2 > C * C * 4 ? C * DK * 2 : C * C * 4;   // k   -> T
    static constexpr int R3 = C * DV * 2 > C * C * 4 ? C * DV * 2 : C * C * 4;   // u   -> A
    static constexpr bool kRowDecay = VT::kHasDecay && !VT::kChannelDecay;
    static constexpr bool kSplit = VT::kChannelDecay;
    static constexpr int NS = VT::kGates ? 2 : 3;
    alignas(16) char smem1[R1];
    alignas(16) char smem3[R3];
    alignas(16) bf16 sAg[VT::kGates ? C * DK : 8];   // b (.) k
    alignas(16) float sG[C][GW];
    float sBeta[C];
    float sEg[kRowDecay ? C : 1], sEgc[kRowDecay ? C : 1];   // e^{g_r}, e^{g_C - g_r}
    alignas(16) bf16 sAt[DK * C];   // (a (.) e^{g})^T, [DK][C]
    alignas(16) bf16 sUt[DV * C];   // U^T, [DV][C]
    float sX[4][16][17];
    alignas(16) bf16 sSplit[kSplit ? NS : 1][kSplit ? C * DK : 8];   // see prep_body
    alignas(16) float sM[kSplit ? 6 : 1][kSplit ? DK : 4];
    unsigned sNext;   // the item after the current one
};

// The bf16 prep of one workgroup: wg0 is its index among the nwg workgroups
// of the prep (its first item).  RT: a routed value is added to v as it is
// staged.
template <int V, int DK, int DV, bool RT>
__device__ __forceinline__ void prep_body(const Problem &p, const WsPtrs<bf16> &ws, const Block &blk,
                                          const unsigned wg0, const unsigned nwg,
                                          PrepSmem<V, DK, DV> &sm) {
    using VT = VariantTraits<V>;
    using M = Mma<bf16>;
    using Raw = PrepRaw<V, DK, DV, RT>;
    constexpr int NT = kPrep2Threads, NW = NT / kWave;
    constexpr int GW = VT::kChannelDecay ? DK : 1;
    constexpr int KC = DK / 8, VC = DV / 8;   // 16-byte chunks per k row / v row
    constexpr int NQ = Raw::NQ, NV = Raw::NV;
    auto &smem1 = sm.smem1;
    auto &smem3 = sm.smem3;
    auto &sAg = sm.sAg;
    auto &sG = sm.sG;
    auto &sBeta = sm.sBeta;
    constexpr bool kRowDecay = VT::kHasDecay && !VT::kChannelDecay;
    auto &sEg = sm.sEg;
    auto &sEgc = sm.sEgc;
    auto &sAt = sm.sAt;
    auto &sUt = sm.sUt;
    auto &sX = sm.sX;
    // Channel decay: the Gram products' split operands, k e^{m - g} (right)
    // and a e^{g - m}, q e^{g - m} (left), with m = (g_{16R} + g_{16R+15}) / 2
    // the reference of the row's own 16-row block R, are formed once per item
    // in phase 1 instead of per tile in phase 2 (this prep runs one workgroup
    // per CU, so the LDS is there).  With gates, a = b (.) k is scaled in
    // place in its own tile.  A diagonal tile (R, R) multiplies them as they
    // are.  An off-diagonal tile (R, S), S < R, needs its right operand
    // relative to m_R instead of m_S: its k fragments are multiplied by the
    // middle factor e^{m_R - m_S} <= 1 from sM (both left and right factors of
    // such a tile then stay bounded, the right one by 1).
    constexpr bool kSplit = VT::kChannelDecay;
    constexpr int NS = VT::kGates ? 2 : 3;
    auto &sSplit = sm.sSplit;
    auto &sM = sm.sM;
    bf16 *const sKr = sSplit[0];
    bf16 *const sQl = sSplit[kSplit ? NS - 1 : 0];
    bf16 *const sAl = VT::kGates ? sAg : sSplit[kSplit && !VT::kGates ? 1 : 0];
    bf16 *sK = reinterpret_cast<bf16 *>(smem1);    // [C][DK]
    bf16 *sV = reinterpret_cast<bf16 *>(smem3);    // [C][DV]
    float *sT = reinterpret_cast<float *>(smem1);  // [C][C]
    float *sAm = reinterpret_cast<float *>(smem3); // [C][C]
    auto kx = [](int r, int col) { return swz<KC, 8>(r, col); };
    auto vx = [](int r, int col) { return swz<VC, 8>(r, col); };
    auto tx = [](int r, int col) { return swz<C / 8, 8>(r, col); };   // [D][C] bf16 tiles
    auto fx = [](int r, int col) { return swz<C / 4, 4>(r, col); };   // [C][C] fp32 tiles

    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const long T = p.T;
    const int H = (int)p.H;
    const bf16 *q = static_cast<const bf16 *>(p.q);
    // Work items are the block's chunk-heads, head fastest: the heads of one
    // chunk run together, so the 128-byte lines of the per-token gates (laid
    // out [B, T, H], two tokens of all sixteen heads per line at H = 16) are
    // fetched once for all of them, and the rows of q, k and v that the
    // workgroups in flight read are whole token rows of all heads.  A
    // workgroup takes item wg0 first, then every nwg-th item or
    // the next ticket (blk.ticket), and loads the next item's inputs while it
    // computes the current one.
    // Item indices fit in 32 bits (the host keeps B * H * ceil(T / 64) below
    // 2^31), so their split into (chunk, head, batch row) is 32-bit scalar
    // arithmetic.
    const unsigned nc = (unsigned)blk.nc, nitems = nc * (unsigned)(p.H * p.B);
    unsigned item = wg0;
    if (blk.ticket_clear && item == 0 && threadIdx.x == 0) *blk.ticket_clear = 0u;
    if (item >= nitems) return;
    unsigned &sNext = sm.sNext;
    auto chunk_of = [&](unsigned it) { return blk.c0 + (long)((it / (unsigned)H) % nc); };
    auto head_of = [&](unsigned it) { return (int)(it % (unsigned)H); };
    auto row_of = [&](unsigned it) { return (int)((it / (unsigned)H) / nc); };
    Raw raw;
    raw.issue(p, chunk_of(item), head_of(item), row_of(item), (int)threadIdx.x);
    // Gram tiles of this wave: row block gR, column blocks gS0 .. gS0+gN-1.
    // The ten lower-triangular 16x16 tiles are grouped so that a wave's tiles
    // share their q rows: (3,0-1) (3,2-3) (2,0-1) (2,2) (1,0-1) (0,0); waves
    // 6 and 7 have none.
    const int gR = wave < 2 ? 3 : (wave < 4 ? 2 : (wave == 4 ? 1 : 0));
    const int gS0 = (wave == 1 || wave == 3) ? 2 : 0;
    const int gN = wave < 6 ? ((wave == 3 || wave == 5) ? 1 : 2) : 0;
    // Without a channel decay, q is read once per item, as the fragments of
    // the q rows of block qR (lane: row 16 qR + l16, elements 32 ks + 8 lg ..
    // + 7).  For waves 0-5, qR = gR: the rows phase 2 multiplies.  Waves 6 and
    // 7, which have no Gram tile, take blocks 1 and 0, so that every row
    // block is held by two waves, and each wave writes half of its block's
    // q (.) e^g (fragments 2 qh and 2 qh + 1): the fragments are the only q
    // the item needs.  The next item's are loaded as soon as phase 2 is done
    // with the current ones.  Rows past T read the last valid row, whose
    // products only reach rows never stored.
    const int qR = wave == 6 ? 1 : (wave == 7 ? 0 : gR);
    const int qh = (wave == 1 || wave == 3 || wave == 6 || wave == 7) ? 1 : 0;
    bf16x8 qf[kSplit ? 1 : DK / 32];
    auto load_qf = [&](long c, int h, int b, int l16, int lg) {
        const long t0 = c * C;
        const int last = (int)min((long)C, T - t0) - 1;
        const int rr = min(16 * qR + l16, last);
        const long row = ((long)b * T + t0 + rr) * H + h;
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
            qf[ks] = *reinterpret_cast<const bf16x8 *>(&q[row * DK + 32 * ks + 8 * lg]);
    };
    if constexpr (!kSplit)
        load_qf(chunk_of(item), head_of(item), row_of(item), (int)threadIdx.x & 15,
                ((int)threadIdx.x & 63) >> 4);

    for (;;) {
    // The thread index is re-derived opaquely each item, so that the many
    // per-thread LDS and workspace offsets are recomputed where they are used
    // instead of being hoisted out of the loop and held in registers.
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int l16 = lane & 15, lg = lane >> 4;
    const int h = head_of(item), b = row_of(item);
    const long c = chunk_of(item);
    const long t0 = c * C;
    const int nvalid = (int)min((long)C, T - t0);
    const long ch = ((long)b * H + h) * blk.nbmax + (c - blk.c0);   // slot-local chunk-head

    __syncthreads();   // the previous item is done with every LDS tile
    // The next item: a ticket drawn now (its latency hides behind the staging,
    // after which it is published) or the static stride.
    unsigned tk = 0;
    if (blk.ticket && tid == 0) tk = atomicAdd(blk.ticket, 1u);
    // ---- stage: the raw inputs into LDS -------------------------------------
    // Rows past T were loaded from the last valid row; they stage as zero
    // (k, v, b (.) k, beta) and as no decay.  The on-load transforms happen
    // here: q and k rows are normalised in registers (a row's chunks sit in
    // KC consecutive lanes), gates are activated, and the decay is staged as
    // its log.
    const bool l2 = p.flags & kQkL2Norm, rawg = p.flags & kRawGates;
    const float ds = p.decay_scale;
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        const int idx = tid + n * NT;
        const int r = idx / KC, pc = idx % KC;
        bf16x8 kv = r < nvalid ? raw.k[n] : zero_bf16x8();
        if (l2) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sk += (float)kv[e] * (float)kv[e];
                if constexpr (kSplit) sq += (float)raw.q[n][e] * (float)raw.q[n][e];
            }
#pragma unroll
            for (int off = 1; off < KC; off <<= 1) {
                sk += __shfl_xor(sk, off, kWave);
                if constexpr (kSplit) sq += __shfl_xor(sq, off, kWave);
            }
            const float rk = rsqrtf(sk + kL2NormEps), rq = rsqrtf(sq + kL2NormEps);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kv[e] = (bf16)((float)kv[e] * rk);
                if constexpr (kSplit) raw.q[n][e] = (bf16)((float)raw.q[n][e] * rq);
            }
        }
        *reinterpret_cast<bf16x8 *>(&sK[kx(r, 8 * pc)]) = kv;
        if constexpr (VT::kGates) {
            bf16x8 av;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float b0 = raw.eb[2 * n][e], b1 = raw.eb[2 * n + 1][e];
                if (rawg) {
                    b0 = sigmoid_f(b0);
                    b1 = sigmoid_f(b1);
                }
                av[e] = (bf16)(b0 * (float)kv[e]);
                av[e + 4] = (bf16)(b1 * (float)kv[e + 4]);
            }
            *reinterpret_cast<bf16x8 *>(&sAg[kx(r, 8 * pc)]) = av;
        }
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        const int idx = tid + n * NT;
        const int r = idx / VC, pc = idx % VC;
        bf16x8 vv = r < nvalid ? raw.v[n] : zero_bf16x8();
        if constexpr (RT) {
            const bf16x8 vr = r < nvalid ? raw.vr[n] : zero_bf16x8();
#pragma unroll
            for (int e = 0; e < 8; ++e) vv[e] = (bf16)((float)vv[e] + (float)vr[e]);
        }
        if constexpr (VT::kGates) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float w0 = raw.ww[2 * n][e], w1 = raw.ww[2 * n + 1][e];
                if (rawg) {
                    w0 = sigmoid_f(w0);
                    w1 = sigmoid_f(w1);
                }
                vv[e] = (bf16)(w0 * (float)vv[e]);
                vv[e + 4] = (bf16)(w1 * (float)vv[e + 4]);
            }
        }
        *reinterpret_cast<bf16x8 *>(&sV[vx(r, 8 * pc)]) = vv;
    }
    if constexpr (!kSplit) {
        if (l2) {
            // a fragment row's elements sit in the four lanes l16 + 16 lg
            float sq = 0.f;
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) sq += (float)qf[ks][e] * (float)qf[ks][e];
            sq += __shfl_xor(sq, 16, kWave);
            sq += __shfl_xor(sq, 32, kWave);
            const float rq = rsqrtf(sq + kL2NormEps);
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)((float)qf[ks][e] * rq);
        }
    }
    if constexpr (VT::kChannelDecay) {
#pragma unroll
        for (int n = 0; n < Raw::NA; ++n) {
            const int idx = tid + n * NT;
            const int r = idx / (DK / 4), i4 = 4 * (idx % (DK / 4));
            f32x4 lg4 = zero4();
            if (r < nvalid)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    lg4[e] = fmaxf(log_decay(raw.al[n][e], rawg, ds), kLogDecayFloor);
            *reinterpret_cast<f32x4 *>(&sG[r][i4]) = lg4;
        }
    } else if constexpr (VT::kHasDecay) {
        if (wave == 0) sG[lane][0] = lane < nvalid ? log_decay(raw.a1, rawg, ds) : 0.f;
    } else {
        if (tid < C) sG[tid][0] = 0.f;
    }
    if constexpr (VT::kScalarBeta)
        if (tid < C) sBeta[tid] = tid < nvalid ? (rawg ? sigmoid_f(raw.be) : raw.be) : 0.f;
    if (tid == 0) sNext = blk.ticket ? nwg + (tk - blk.ticket_base) : item + nwg;
    __syncthreads();

    // ---- gates: decay prefix sums (of the staged logs); KLA step size --------
    if constexpr (VT::kChannelDecay) {
        if (tid < DK) {
            float g = 0.f;
            for (int r = 0; r < C; ++r) {
                g += sG[r][tid];
                sG[r][tid] = g;
            }
        }
    } else if constexpr (VT::kHasDecay) {
        if (wave == 0) {
            float g = sG[lane][0];
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const float y = __shfl_up(g, off, kWave);
                if (lane >= off) g += y;
            }
            sG[lane][0] = g;
            const float gC = __shfl(g, C - 1, kWave);
            sEg[lane] = __expf(g);
            sEgc[lane] = __expf(gC - g);
        }
    }
    if constexpr (VT::kKaczmarz) {
        // beta_r = eta_r / (||k_r||^2 + eps), from the stored keys: eight lanes
        // per row, all 64 rows at once.
        static_assert(NT == 8 * C, "eight lanes per row");
        const int r = tid >> 3, part = tid & 7;
        float s2 = 0.f;
#pragma unroll
        for (int i = 8 * part; i < DK; i += 64) {
            const bf16x8 kv = *reinterpret_cast<const bf16x8 *>(&sK[kx(r, i)]);
#pragma unroll
            for (int e = 0; e < 8; ++e) s2 += (float)kv[e] * (float)kv[e];
        }
        s2 += __shfl_xor(s2, 1, kWave);
        s2 += __shfl_xor(s2, 2, kWave);
        s2 += __shfl_xor(s2, 4, kWave);
        if (part == 0) sBeta[r] = r < nvalid ? sBeta[r] / (s2 + p.eps) : 0.f;
    }
    __syncthreads();

    // ---- phase 1: element-wise factors ------------------------------------
    // The workspace stores of this phase (q (.) e^g, Kbar^T, e^{g_C}) go out
    // at once: the Gram products load nothing from global memory, so no wait
    // for their operands can be held up by them.
    {
        // q (.) e^{g}, from registers: the row layout with a channel decay,
        // else half a row block per wave from its q fragments
        if constexpr (kSplit) {
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
                const int idx = tid + n * NT;
                const int r = idx / KC, pc = idx % KC;
                bf16x8 o;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    o[e] = (bf16)((float)raw.q[n][e] * __expf(sG[r][8 * pc + e]));
                *reinterpret_cast<bf16x8 *>(ws.Qt + ch * C * DK + frag_off<bf16>(r, 8 * pc, DK)) = o;
            }
        } else {
            const int r = 16 * qR + l16;
            const float egr = kRowDecay ? sEg[r] : 1.f;
            // Fragments NH qh .. NH qh + NH - 1 of the row block, selected by
            // the wave-uniform qh and stored unconditionally: written as
            // stores under a condition on the fragment index, the compiler
            // merged them into one store whose data and address it selected
            // by different tests on the wave index (wrong for d_k = 64).
            constexpr int NH = DK / 64;
#pragma unroll
            for (int j = 0; j < NH; ++j) {
                const int ks = qh * NH + j;
                const bf16x8 src = qh ? qf[NH + j] : qf[j];
                bf16x8 o;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)src[e] * egr);
                *reinterpret_cast<bf16x8 *>(ws.Qt + ch * C * DK + frag_off<bf16>(r, 32 * ks + 8 * lg, DK)) = o;
            }
        }
        // (a (.) e^{g})^T into LDS and (k (.) e^{g_C - g})^T to the workspace.
        // A thread transposes two columns of eight rows: its eight 4-byte
        // reads are all issued before any arithmetic, so they wait once.
        static_assert(DK / 2 * (C / 8) <= NT && DV / 2 * (C / 8) <= NT, "one pass");
        if (tid < DK / 2 * (C / 8)) {
            const int i0 = 2 * (tid % (DK / 2)), r0 = 8 * (tid / (DK / 2));
            uint32_t kw[8], aw[VT::kGates ? 8 : 1];
            float2 gw[VT::kChannelDecay ? 8 : 1];
            bf16x2 alw[VT::kGates ? 8 : 1];   // a e^{g - g_ref}, written back in place
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kw[e] = *reinterpret_cast<const uint32_t *>(&sK[kx(r0 + e, i0)]);
                if constexpr (VT::kGates)
                    aw[e] = *reinterpret_cast<const uint32_t *>(&sAg[kx(r0 + e, i0)]);
                if constexpr (VT::kChannelDecay)
                    gw[e] = *reinterpret_cast<const float2 *>(&sG[r0 + e][i0]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int i = i0 + cc;
                const float gC = sG[C - 1][VT::kChannelDecay ? i : 0];
                // the reference of the 16-row block holding rows r0 .. r0 + 7
                const int ib = VT::kChannelDecay ? i : 0;
                const float gref = 0.5f * (sG[16 * (r0 >> 4)][ib] + sG[16 * (r0 >> 4) + 15][ib]);
                // element cc of a word holding two bf16 (little-endian)
                auto half = [&](uint32_t w) {
                    return __uint_as_float(cc ? (w & 0xffff0000u) : (w << 16));
                };
                float at[8], kb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = r0 + e;
                    const float kk = half(kw[e]);
                    float a;
                    if constexpr (VT::kGates) a = half(aw[e]);
                    else a = sBeta[r] * kk;
                    float eg = 1.f, egc = 1.f;
                    if constexpr (VT::kChannelDecay) {
                        const float g = cc ? gw[e].y : gw[e].x;
                        eg = __expf(g);
                        egc = __expf(gC - g);
                        if constexpr (VT::kGates) alw[e][cc] = (bf16)(a * __expf(g - gref));
                    } else if constexpr (kRowDecay) {
                        eg = sEg[r];
                        egc = sEgc[r];
                    }
                    at[e] = a * eg;
                    kb[e] = kk * egc;
                }
                store8(&sAt[tx(i, r0)], at);
                bf16x8 kbo;
#pragma unroll
                for (int e = 0; e < 8; ++e) kbo[e] = (bf16)kb[e];
                *reinterpret_cast<bf16x8 *>(ws.Kbt + ch * DK * C + frag_off<bf16>(i, r0, C)) = kbo;
                if (r0 == 0) ws.gam[ch * DK + i] = VT::kHasDecay ? __expf(gC) : 1.f;
            }
            // the same elements this thread read, so no other thread races it
            if constexpr (VT::kGates) {
#pragma unroll
                for (int e = 0; e < 8; ++e) *reinterpret_cast<bf16x2 *>(&sAg[kx(r0 + e, i0)]) = alw[e];
            }
        }
        if constexpr (kSplit) {
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
                const int idx = tid + n * NT;
                const int r = idx / KC, pc = idx % KC;
                const bf16x8 k8 = *reinterpret_cast<const bf16x8 *>(&sK[kx(r, 8 * pc)]);
                const float br = VT::kScalarBeta ? sBeta[r] : 0.f;
                bf16x8 kr8, al8, ql8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int i = 8 * pc + e;
                    const float gref = 0.5f * (sG[16 * (r >> 4)][i] + sG[16 * (r >> 4) + 15][i]);
                    const float g = sG[r][i];
                    const float fl = __expf(g - gref);
                    kr8[e] = (bf16)((float)k8[e] * __expf(gref - g));
                    if constexpr (!VT::kGates) al8[e] = (bf16)(br * (float)k8[e] * fl);
                    ql8[e] = (bf16)((float)raw.q[n][e] * fl);
                }
                *reinterpret_cast<bf16x8 *>(&sKr[kx(r, 8 * pc)]) = kr8;
                if constexpr (!VT::kGates) *reinterpret_cast<bf16x8 *>(&sAl[kx(r, 8 * pc)]) = al8;
                *reinterpret_cast<bf16x8 *>(&sQl[kx(r, 8 * pc)]) = ql8;
            }
            // middle factors e^{m_R - m_S} of the six off-diagonal tiles
            for (int idx = tid; idx < 6 * DK; idx += NT) {
                const int pr = idx / DK, i = idx % DK;
                const int R = pair_r(pr), S = pair_s(pr);
                const float mR = 0.5f * (sG[16 * R][i] + sG[16 * R + 15][i]);
                const float mS = 0.5f * (sG[16 * S][i] + sG[16 * S + 15][i]);
                sM[pr][i] = __expf(mR - mS);
            }
        }
        // U^T into LDS, two columns of eight rows per thread in the same way
        if (tid < DV / 2 * (C / 8)) {
            const int j0 = 2 * (tid % (DV / 2)), r0 = 8 * (tid / (DV / 2));
            uint32_t vw[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) vw[e] = *reinterpret_cast<const uint32_t *>(&sV[vx(r0 + e, j0)]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                float u[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float vv = __uint_as_float(cc ? (vw[e] & 0xffff0000u) : (vw[e] << 16));
                    if constexpr (VT::kGates) u[e] = vv;
                    else u[e] = sBeta[r0 + e] * vv;
                }
                store8(&sUt[tx(j0 + cc, r0)], u);
            }
        }
    }
    // Every raw register is consumed: the next item's loads go out now and
    // arrive during phases 2-4.  After its last item a workgroup still issues
    // them, so that the issue is unconditional and the compiler's waits stay
    // exact; they then read item 0 of the launch, one region that every
    // workgroup's last prefetch shares and finds in L2 (the workgroup's own
    // last item has been evicted by then, and re-reading it cost ~18 MB per
    // 64-chunk block of a pipelined forward).
    const unsigned next_item = sNext;
    {
        const unsigned next = next_item < nitems ? next_item : 0u;
        raw.issue(p, chunk_of(next), head_of(next), row_of(next), tid);
    }
    __syncthreads();

    // ---- phase 2: A and P on matrix cores ---------------------------------------
    // Computed transposed, D'(s, r) = sum_i Kr[s][i] L[r][i]: a lane holds four
    // consecutive s of one row r.  Channel-wise decay is split between the
    // operands around each 16-row block's reference (see sSplit); scalar decay
    // multiplies the product by e^{g_r - g_s} <= 1.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (u >= gN) break;
        const int R = gR, S = gS0 + u;
        const int rs = 16 * S + l16;
        const int rr = 16 * R + l16;
        f32x4 accA = zero4(), accP = zero4();
        float br = 0.f;
        if constexpr (VT::kScalarBeta) br = sBeta[rr];
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
            const int kb = 32 * ks + 8 * lg;
            if constexpr (!kSplit) {
                // a_r = beta_r k_r and the decay are scalars per row: the stored
                // bf16 rows go to the matrix cores as they are and the scalars
                // multiply the product.
                const bf16x8 kr8 = *reinterpret_cast<const bf16x8 *>(&sK[kx(rs, kb)]);
                const bf16x8 kq8 = *reinterpret_cast<const bf16x8 *>(&sK[kx(rr, kb)]);
                accA = M::mma(kr8, kq8, accA);
                accP = M::mma(kr8, qf[ks], accP);
            } else {
                bf16x8 kq = *reinterpret_cast<const bf16x8 *>(&sKr[kx(rs, kb)]);
                if (S < R) {   // wave-uniform
                    const float *mf = &sM[kSplit ? pair_of(R, S) : 0][kSplit ? kb : 0];
                    const f32x4 m0 = *reinterpret_cast<const f32x4 *>(mf);
                    const f32x4 m1 = *reinterpret_cast<const f32x4 *>(mf + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kq[e] = (bf16)((float)kq[e] * m0[e]);
                        kq[e + 4] = (bf16)((float)kq[e + 4] * m1[e]);
                    }
                }
                accA = M::mma(kq, *reinterpret_cast<const bf16x8 *>(&sAl[kx(rr, kb)]), accA);
                accP = M::mma(kq, *reinterpret_cast<const bf16x8 *>(&sQl[kx(rr, kb)]), accP);
            }
        }
        const int r = rr;
        f32x4 Av, Pv;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int s2 = 16 * S + 4 * lg + m;
            float f = 1.f;
            if constexpr (kRowDecay) f = s2 <= r ? __expf(sG[r][0] - sG[s2][0]) : 0.f;
            float fa = f;
            if constexpr (!VT::kChannelDecay && !VT::kGates) fa = f * br;
            Av[m] = s2 < r ? accA[m] * fa : 0.f;
            Pv[m] = s2 <= r ? accP[m] * f : 0.f;
        }
        *reinterpret_cast<f32x4 *>(&sAm[fx(r, 16 * S + 4 * lg)]) = Av;
        store_frag4(ws.P + ch * C * C, r, 16 * S + 4 * lg, C, Pv);
    }
    if (tid < 6 * 16 * 4) {
        const int idx = tid;
        const int t6 = idx / 64, e = idx % 64;
        const int r = 16 * upper_r(t6) + e / 4;
        const int s2 = 16 * upper_s(t6) + 4 * (e % 4);
        // The zero is made here, opaque to the compiler: hoisted out of the
        // item loop it was spilled, and its reload (a scratch load) waited for
        // every load in flight, the next item's prefetch included.
        unsigned z = 0u;
        asm volatile("" : "+v"(z));
        *reinterpret_cast<uint2 *>(ws.P + ch * C * C + frag_off<bf16>(r, s2, C)) = make_uint2(z, z);
    }
    // the q fragments are free: the next item's go out now (item 0's after
    // the last item, as above)
    if constexpr (!kSplit) {
        const unsigned next = next_item < nitems ? next_item : 0u;
        load_qf(chunk_of(next), head_of(next), row_of(next), l16, lg);
    }
    __syncthreads();

    // ---- phase 3: T = (I + A)^{-1} ------------------------------------------
    if (wave == 0) {
        // Diagonal 16x16 blocks by forward substitution; lane = (block, column).
        const int R = lg, cc = l16;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < r; ++j) acc += sAm[fx(16 * R + r, 16 * R + j)] * x[j];
            x[r] = r == cc ? 1.f : (r < cc ? 0.f : -acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[fx(16 * R + r, 16 * R + cc)] = x[r];
    } else {
#pragma unroll
        for (int n = 0; n < (6 * 256 + NT - kWave - 1) / (NT - kWave); ++n) {
            const int idx = tid - kWave + n * (NT - kWave);
            if (idx >= 6 * 256) break;
            const int t6 = idx >> 8, e = idx & 255;
            sT[fx(16 * upper_r(t6) + (e >> 4), 16 * upper_s(t6) + (e & 15))] = 0.f;
        }
    }
    __syncthreads();
    // Off-diagonal blocks by 2 x 2 block recursion on fp32 matrix cores
    // (16x16x4, full fp32 products).  With L = [[L11, 0], [L21, L22]] unit
    // lower triangular, L^{-1} = [[T11, 0], [-T22 L21 T11, T22]]:
    //   16x16 level: T10 = -T11 (A10 T00), T32 = -T33 (A32 T22)   (waves 0, 1)
    //   32x32 level: Y = [A20 A21; A30 A31] [T00 0; T10 T11]      (waves 0-3)
    //                [T20 T21; T30 T31] = -[T22 0; T32 T33] Y
    // A lane feeds row l16 / K-element lg of the left factor and K-element lg /
    // column l16 of the right one, and receives rows 4 lg .. 4 lg + 3 of column
    // l16; intermediate tiles go through sX to become right-hand operands.
    using MF = Mma<float>;
    // acc += X(xr, xc) Y(yr, yc) for 16x16 blocks of two C x C fp32 LDS tiles
    auto mm16 = [&](f32x4 acc, const float *X, int xr, int xc, const float *Y, int yr, int yc) {
        float a[4], t[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            a[s4] = X[fx(16 * xr + l16, 16 * xc + 4 * s4 + lg)];
            t[s4] = Y[fx(16 * yr + 4 * s4 + lg, 16 * yc + l16)];
        }
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) acc = MF::mma(a[s4], t[s4], acc);
        return acc;
    };
    // acc += T(r, r') Z for a 16x16 intermediate Z held in sX[z]
    auto mm16x = [&](f32x4 acc, int r, int r2, int z) {
        float a[4], t[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            a[s4] = sT[fx(16 * r + l16, 16 * r2 + 4 * s4 + lg)];
            t[s4] = sX[z][4 * s4 + lg][l16];
        }
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) acc = MF::mma(a[s4], t[s4], acc);
        return acc;
    };
    if (wave < 2) {
        const int R = 1 + 2 * wave, S = R - 1;
        const f32x4 xv = mm16(zero4(), sAm, R, S, sT, S, S);
#pragma unroll
        for (int i = 0; i < 4; ++i) sX[wave][4 * lg + i][l16] = xv[i];
        // The wave reads back what it wrote: LDS keeps one wave's accesses in
        // order; the fence keeps the compiler from reordering them.
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const f32x4 tv = mm16x(zero4(), R, R, wave);
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[fx(16 * R + 4 * lg + i, 16 * S + l16)] = -tv[i];
    }
    __syncthreads();
    if (wave < 4) {
        const int R = 2 + (wave >> 1), S = wave & 1;
        f32x4 yv = mm16(zero4(), sAm, R, S, sT, S, S);
        if (S == 0) yv = mm16(yv, sAm, R, 1, sT, 1, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) sX[wave][4 * lg + i][l16] = yv[i];
    }
    __syncthreads();
    if (wave < 4) {
        const int R = 2 + (wave >> 1), S = wave & 1;
        f32x4 tv = mm16x(zero4(), R, R, wave);
        if (R == 3) tv = mm16x(tv, 3, 2, wave - 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[fx(16 * R + 4 * lg + i, 16 * S + l16)] = -tv[i];
    }
    __syncthreads();

    // ---- phase 4: W and U~ on matrix cores --------------------------------------
    {
        const int R = wave & 3, half = wave >> 2;
        const int nK = R / 2 + 1;                 // K-steps of 32 covering s <= r
        M::frag Tf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (ks < nK) {
                const int row = 16 * R + l16, col = 32 * ks + 8 * lg;
                const f32x4 t0v = *reinterpret_cast<const f32x4 *>(&sT[fx(row, col)]);
                const f32x4 t1v = *reinterpret_cast<const f32x4 *>(&sT[fx(row, col + 4)]);
                const float tmp[8] = {t0v[0], t0v[1], t0v[2], t0v[3], t1v[0], t1v[1], t1v[2], t1v[3]};
                Tf[ks] = M::from_f32x8(tmp);
            }
        }
#pragma unroll
        for (int mi = half * (DK / 32); mi < (half + 1) * (DK / 32); ++mi) {
            f32x4 acc = zero4();
            const int row = 16 * mi + l16;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (ks < nK)
                    acc = M::mma(*reinterpret_cast<const M::frag *>(&sAt[tx(row, 32 * ks + 8 * lg)]),
                                 Tf[ks], acc);
            store_frag4(ws.W + ch * C * DK, 16 * R + l16, 16 * mi + 4 * lg, DK, acc);
        }
#pragma unroll
        for (int nj = half * (DV / 32); nj < (half + 1) * (DV / 32); ++nj) {
            f32x4 acc = zero4();
            const int row = 16 * nj + l16;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (ks < nK)
                    acc = M::mma(Tf[ks],
                                 *reinterpret_cast<const M::frag *>(&sUt[tx(row, 32 * ks + 8 * lg)]),
                                 acc);
            store4(ws.Ut + ch * DV * C + ufrag_off(16 * nj + l16, 16 * R + 4 * lg), acc);
        }
    }
    item = next_item;
    if (item >= nitems) break;
    }   // items
}

template <int V, int DK, int DV, bool RT>
__global__ __launch_bounds__(kPrep2Threads, (V == kKDA || V == kGDN2) ? 2 : 4)
void chunk_prep_bf16_kernel(Problem p, WsPtrs<bf16> ws, Block blk) {
    __shared__ PrepSmem<V, DK, DV> sm;
    prep_body<V, DK, DV, RT>(p, ws, blk, blockIdx.x, gridDim.x, sm);
}

// ============================================================================
// chunk_scan, split roles: eight waves per workgroup, which owns NJ 16-column
// tiles of one head's state.  Waves 0-3 run only the state recurrence
// (Delta = U~ - W S, then S <- Gamma S + Kbar^T Delta) and load only W,
// Kbar^T, U~ and e^{g_C}; waves 4-7 produce the output of the previous chunk,
// O = Qt S + P Delta, from double-buffered copies of S^T and Delta^T in LDS,
// and load only Qt and P.  The state chain per chunk is then two short
// matrix-core steps between two barriers, and the output work runs beside it
// on the same SIMDs.  The chunk factors are shared by all column tiles of a
// head, so wider slices (larger NJ) read them fewer times in all.
// ============================================================================
// SG: the decay is a scalar per chunk (every entry of e^{g_C} is equal), so
// one 4-byte load per lane replaces the per-row vector loads.
template <typename TI, int DK, int NJ, bool SG> struct ChainOps {
    using M = Mma<TI>;
    static constexpr int KS_D = DK / M::kK, KS_C = C / M::kK, NI = DK / 64;
    static constexpr int FB = kWave * M::kPerLane * (int)sizeof(TI);   // bytes per fragment tile
    typedef typename std::conditional<sizeof(TI) == 2, bf16x4, f32x4>::type raw4;
    typename M::frag Wf[KS_D], Kf[NI][KS_C];
    raw4 U[NJ];
    f32x4 gam[NI];
    // The factors of the Delta step (W, U~) and of the state update (Kbar^T,
    // e^{g_C}) load separately, so that each half of a step can issue the
    // next chunk's share.
    __device__ __forceinline__ void load_w(const WsPtrs<TI> &ws, long ch, int DV, int col0, int w,
                                           int lane) {
        const unsigned loff = (unsigned)lane * (M::kPerLane * sizeof(TI));
        const auto rw = make_rsrc(reinterpret_cast<const char *>(ws.W + ch * C * DK) + w * KS_D * FB);
        const auto ru = make_rsrc(reinterpret_cast<const char *>(ws.Ut + ch * (long)DV * C) +
                                  ((col0 / 16) * (C / 16) + w) * (kWave * 4 * (int)sizeof(TI)));
#pragma unroll
        for (int ks = 0; ks < KS_D; ++ks) Wf[ks] = buf_load<typename M::frag>(rw, loff + ks * FB);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            U[j] = buf_load<raw4>(ru, ((unsigned)lane + (unsigned)(j * (C / 16) * kWave)) * 4u *
                                          sizeof(TI));
    }
    __device__ __forceinline__ void load_k(const WsPtrs<TI> &ws, long ch, int w, int lane) {
        const unsigned loff = (unsigned)lane * (M::kPerLane * sizeof(TI));
        const auto rk = make_rsrc(reinterpret_cast<const char *>(ws.Kbt + ch * DK * C) +
                                  w * NI * KS_C * FB);
        const auto rg = make_rsrc(ws.gam + ch * DK + 16 * NI * w);
#pragma unroll
        for (int a = 0; a < NI; ++a) {
#pragma unroll
            for (int ks = 0; ks < KS_C; ++ks)
                Kf[a][ks] = buf_load<typename M::frag>(rk, loff + (a * KS_C + ks) * FB);
            if constexpr (!SG) gam[a] = buf_load<f32x4>(rg, (unsigned)(lane >> 4) * 16u + 64u * a);
        }
        if constexpr (SG) {
            const float g = buf_load<float>(rg, 0u);
#pragma unroll
            for (int a = 0; a < NI; ++a) gam[a] = f32x4{g, g, g, g};
        }
    }
};

template <typename TI, int DK> struct OutOps {
    using M = Mma<TI>;
    static constexpr int KS_D = DK / M::kK, KS_C = C / M::kK;
    static constexpr int FB = kWave * M::kPerLane * (int)sizeof(TI);
    typename M::frag Qf[KS_D], Pf[KS_C];
    __device__ __forceinline__ void load_q(const WsPtrs<TI> &ws, long ch, int w, int lane) {
        const unsigned loff = (unsigned)lane * (M::kPerLane * sizeof(TI));
        const auto rq = make_rsrc(reinterpret_cast<const char *>(ws.Qt + ch * C * DK) + w * KS_D * FB);
#pragma unroll
        for (int ks = 0; ks < KS_D; ++ks) Qf[ks] = buf_load<typename M::frag>(rq, loff + ks * FB);
    }
    __device__ __forceinline__ void load_p(const WsPtrs<TI> &ws, long ch, int w, int lane) {
        const unsigned loff = (unsigned)lane * (M::kPerLane * sizeof(TI));
        const auto rp = make_rsrc(reinterpret_cast<const char *>(ws.P + ch * C * C) + w * KS_C * FB);
#pragma unroll
        for (int ks = 0; ks < KS_C; ++ks) Pf[ks] = buf_load<typename M::frag>(rp, loff + ks * FB);
    }
};

constexpr int kScan2Threads = 512;
// The output waves stage o in LDS and write it every kOutBurst chunks.  Loads
// and stores share one wait counter, and the compiler lets a store complete
// out of order, so a wait for the next chunk's prefetched factors also waits
// for any o store issued after those loads; staged, only one wait in
// kOutBurst does.
constexpr int kOutBurst = 8;

// STATES: instead of the outputs, record the state entering every chunk and
// its Delta (input dtype) in blk.s_chunks and blk.d_chunks; the output waves
// then only copy them.  SAVE: the outputs and that record both, the output
// waves copying S_c and Delta_c beside their O_c.
// A scalar decay's instances keep to 128 registers, so that a prep workgroup
// fits beside them; a channel decay's never share a unit with a prep.
// The scan's LDS tiles (one workgroup's).
template <typename TI, int DK, int NJ, bool STATES> struct ScanSmem {
    static constexpr int PT = 8;
    static constexpr int SW = 16 * NJ;   // value columns of the slice
    alignas(16) TI sSt[2][SW][DK + PT];   // S^T, double-buffered
    alignas(16) TI sDt[2][SW][C + PT];    // Delta^T, double-buffered
    // o of the last kOutBurst chunks, written to HBM in one burst (see below)
    alignas(16) TI sO[STATES ? 1 : kOutBurst][C][SW];
};

// The scan of one workgroup; wg is its index in the scan's grid.
template <typename TI, int DK, int DEPTH, int NJ, bool STATES, bool NTO, bool SG, bool SAVE>
__device__ __forceinline__ void scan_body(const Problem &p, const WsPtrs<TI> &ws, const Block &blk,
                                          const unsigned wg, ScanSmem<TI, DK, NJ, STATES> &sm) {
    using M = Mma<TI>;
    using CO = ChainOps<TI, DK, NJ, SG>;
    using OO = OutOps<TI, DK>;
    constexpr int KS_D = CO::KS_D, KS_C = CO::KS_C, NI = CO::NI;
    constexpr int PT = 8;
    constexpr int SW = 16 * NJ;   // value columns of the slice
    auto &sSt = sm.sSt;
    auto &sDt = sm.sDt;
    auto &sO = sm.sO;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int l16 = lane & 15, lg = lane >> 4;
    const int H = (int)p.H, DV = (int)p.dv;
    const long T = p.T;
    const long NC = blk.nc;                 // chunks of this block
    const int nslice = DV / SW;
    const long nwg = p.B * p.H * nslice;
    const long per_xcd = (nwg + kXcds - 1) / kXcds;
    const long logical = (long)(wg % kXcds) * per_xcd + wg / kXcds;
    if (logical >= nwg) return;
    // The scan is the sequential part: when the next block's prep shares the
    // compute unit, its waves are issued first.
    __builtin_amdgcn_s_setprio(3);
    const long bh = logical / nslice;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int col0 = (int)(logical % nslice) * SW;
    const long ch0 = bh * blk.nbmax;        // slot-local chunk-heads of this head
    const long last = NC - 1;
    auto chunk = [&](long c) { return ch0 + (c < 0 ? 0 : (c < last ? c : last)); };

    if (wave < 4) {
        // ---------------- state chain ----------------
        const int w = wave;
        f32x4 S[NJ][NI];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int a = 0; a < NI; ++a)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int i = 16 * (w * NI + a) + 4 * lg + m;
                    S[j][a][m] = blk.s_in ? blk.s_in[(bh * DK + i) * DV + col0 + 16 * j + l16] : 0.f;
                }
        auto write_st = [&](int buf) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int a = 0; a < NI; ++a)
                    store4(&sSt[buf][16 * j + l16][16 * (w * NI + a) + 4 * lg], S[j][a]);
        };
        write_st(0);
        __syncthreads();
        // Every step consumes its whole register set on every path: a loaded
        // value left unused on some path makes the compiler wait for all
        // loads in flight before it reuses any register.
        // pre_update issues the next chunk's state-update factors once this
        // step's Delta is in LDS.
        auto step = [&](const CO &op, long c, auto &&pre_update) __attribute__((always_inline)) {
            const int cur = (int)(c & 1);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                typename M::frag Sf[KS_D];
#pragma unroll
                for (int ks = 0; ks < KS_D; ++ks)
                    Sf[ks] = M::load(&sSt[cur][16 * j + l16][0], ks * M::kK, lane);
                f32x4 d0 = zero4(), d1 = zero4();
#pragma unroll
                for (int ks = 0; ks < KS_D; ks += 2) {
                    d0 = M::mma(op.Wf[ks], Sf[ks], d0);
                    if (ks + 1 < KS_D) d1 = M::mma(op.Wf[ks + 1], Sf[ks + 1], d1);
                }
                store4(&sDt[cur][16 * j + l16][16 * w + 4 * lg], to_f32x4(op.U[j]) - (d0 + d1));
            }
            pre_update();
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                typename M::frag Df[KS_C];
#pragma unroll
                for (int ks = 0; ks < KS_C; ++ks)
                    Df[ks] = M::load(&sDt[cur][16 * j + l16][0], ks * M::kK, lane);
#pragma unroll
                for (int a = 0; a < NI; ++a) {
                    f32x4 acc = S[j][a] * op.gam[a];
#pragma unroll
                    for (int ks = 0; ks < KS_C; ++ks) acc = M::mma(op.Kf[a][ks], Df[ks], acc);
                    S[j][a] = acc;
                }
            }
            write_st(cur ^ 1);
            __syncthreads();
        };
        if constexpr (DEPTH == 2) {
            CO A, Bq;
            A.load_w(ws, chunk(0), DV, col0, w, lane);
            A.load_k(ws, chunk(0), w, lane);
            for (long c = 0; c < NC; c += 2) {
                Bq.load_w(ws, chunk(c + 1), DV, col0, w, lane);
                __builtin_amdgcn_sched_barrier(0);   // issue the prefetch first
                step(A, c, [&] { Bq.load_k(ws, chunk(c + 1), w, lane); });
                if (c + 1 >= NC) break;
                A.load_w(ws, chunk(c + 2), DV, col0, w, lane);
                __builtin_amdgcn_sched_barrier(0);
                step(Bq, c + 1, [&] { A.load_k(ws, chunk(c + 2), w, lane); });
            }
        } else {
            CO cur;
            for (long c = 0; c < NC; ++c) {
                cur.load_w(ws, chunk(c), DV, col0, w, lane);
                cur.load_k(ws, chunk(c), w, lane);
                step(cur, c, [] {});
            }
        }
        // The output waves still finish the last chunk.
        __syncthreads();
        __syncthreads();
        if (blk.s_out) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int a = 0; a < NI; ++a)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int i = 16 * (w * NI + a) + 4 * lg + m;
                        blk.s_out[(bh * DK + i) * DV + col0 + 16 * j + l16] = S[j][a][m];
                    }
        }
    } else if constexpr (STATES) {
        // Copy S_c and Delta_c of chunk c from LDS to the workspace, in the
        // window where the output waves would compute O_c; same barriers.
        const int tt = tid - 4 * kWave;
        TI *sg = static_cast<TI *>(blk.s_chunks), *dg = static_cast<TI *>(blk.d_chunks);
        __syncthreads();
        __syncthreads();
        __syncthreads();
        for (long c = 0; c < NC; ++c) {
            const int buf = (int)(c & 1);
            copy_transposed<TI, SW, DK + PT>(sg + (ch0 + c) * (long)DK * DV + col0, DV, sSt[buf], DK,
                                             DK, tt, 4 * kWave);
            copy_transposed<TI, SW, C + PT>(dg + (ch0 + c) * (long)C * DV + col0, DV, sDt[buf], C, C,
                                            tt, 4 * kWave);
            __syncthreads();
            __syncthreads();
        }
    } else {
        // ---------------- outputs of the previous chunk ----------------
        const int w = wave - 4;
        __builtin_amdgcn_s_setprio(2);   // the chain waves' instructions go first
        TI *out = static_cast<TI *>(p.o);
        __syncthreads();          // S_0 in place
        __syncthreads();          // first chunk: no output yet
        __syncthreads();
        // Writes the staged o of chunks c - c % kOutBurst .. c: each wave its
        // own sixteen token rows, one 16-byte piece per lane and store.
        typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
        auto flush = [&](long c) {
            constexpr int EPP = 16 / (int)sizeof(TI);   // elements per piece
            constexpr int PPR = SW / EPP;               // pieces per token row
            const long first = c - c % kOutBurst;
            const int n = (int)(c - first + 1) * 16 * PPR;
            for (int idx = lane; idx < n; idx += kWave) {
                const int kk = idx / (16 * PPR), rem = idx % (16 * PPR);
                const int tl = 16 * w + rem / PPR, pc = rem % PPR;
                const long tt = (blk.c0 + first + kk) * C + tl;
                if (tt < T) {
                    const u32x4v x = *reinterpret_cast<const u32x4v *>(&sO[kk][tl][pc * EPP]);
                    u32x4v *dst = reinterpret_cast<u32x4v *>(
                        &out[((b * T + tt) * H + h) * (long)DV + col0 + pc * EPP]);
                    if constexpr (NTO) __builtin_nontemporal_store(x, dst);
                    else *dst = x;
                }
            }
        };
        // op holds the factors of chunk c; S_c and Delta_c are in LDS buffer c % 2.
        // The chain overwrites S_c's buffer in the second half of its next
        // step and Delta_c's only in the step after, so Qt S runs beside the
        // chain's Delta step and P Delta (and the stores) beside its state
        // update.
        // pre_pd issues the next chunk's P once Qt S is done.
        auto step = [&](const OO &op, long c, auto &&pre_pd) __attribute__((always_inline)) {
            const int buf = (int)(c & 1);
            f32x4 Ov[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                Ov[j] = zero4();
#pragma unroll
                for (int ks = 0; ks < KS_D; ++ks)
                    Ov[j] = M::mma(M::load(&sSt[buf][16 * j + l16][0], ks * M::kK, lane), op.Qf[ks],
                                   Ov[j]);
            }
            pre_pd();
            if constexpr (SAVE) {
                // S_c and Delta_c, from the buffers O_c reads, before the
                // barrier after which the chain overwrites S_c's; issued
                // after the next chunk's prefetch, so that a wait for those
                // loads does not wait for these stores.
                TI *sg = static_cast<TI *>(blk.s_chunks), *dg = static_cast<TI *>(blk.d_chunks);
                copy_transposed<TI, SW, DK + PT>(sg + (ch0 + c) * (long)DK * DV + col0, DV, sSt[buf],
                                                 DK, DK, tid - 4 * kWave, 4 * kWave);
                copy_transposed<TI, SW, C + PT>(dg + (ch0 + c) * (long)C * DV + col0, DV, sDt[buf], C,
                                                C, tid - 4 * kWave, 4 * kWave);
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                // P is zero above the diagonal, so all K-steps may run.
#pragma unroll
                for (int ks = 0; ks < KS_C; ++ks)
                    Ov[j] = M::mma(M::load(&sDt[buf][16 * j + l16][0], ks * M::kK, lane), op.Pf[ks],
                                   Ov[j]);
                store4(&sO[c % kOutBurst][16 * w + l16][16 * j + 4 * lg], Ov[j]);
            }
            if (c % kOutBurst == kOutBurst - 1 || c == NC - 1) flush(c);
            if (p.delta_out) {
                // each token's written residual: the chunk's Delta, rows past T dropped
                const long tc = (blk.c0 + c) * C;
                copy_transposed<TI, SW, C + PT>(
                    static_cast<TI *>(p.delta_out) + ((b * T + tc) * H + h) * (long)DV + col0,
                    (long)H * DV, sDt[buf], C, T - tc, tid - 4 * kWave, 4 * kWave);
            }
            __syncthreads();
        };
        if constexpr (DEPTH == 2) {
            OO A, Bq;
            A.load_q(ws, chunk(0), w, lane);
            A.load_p(ws, chunk(0), w, lane);
            for (long c = 0; c < NC; c += 2) {
                Bq.load_q(ws, chunk(c + 1), w, lane);
                __builtin_amdgcn_sched_barrier(0);
                step(A, c, [&] { Bq.load_p(ws, chunk(c + 1), w, lane); });
                if (c + 1 >= NC) break;
                A.load_q(ws, chunk(c + 2), w, lane);
                __builtin_amdgcn_sched_barrier(0);
                step(Bq, c + 1, [&] { A.load_p(ws, chunk(c + 2), w, lane); });
            }
        } else {
            OO cur;
            for (long c = 0; c < NC; ++c) {
                cur.load_q(ws, chunk(c), w, lane);
                cur.load_p(ws, chunk(c), w, lane);
                step(cur, c, [] {});
            }
        }
    }
}

template <typename TI, int DK, int DEPTH, int NJ, bool STATES, bool NTO, bool SG, bool SAVE = false>
__global__ __launch_bounds__(kScan2Threads, SG ? 4 : 2) void chunk_scan2_kernel(Problem p, WsPtrs<TI> ws,
                                                                   Block blk) {
    __shared__ ScanSmem<TI, DK, NJ, STATES> sm;
    scan_body<TI, DK, DEPTH, NJ, STATES, NTO, SG, SAVE>(p, ws, blk, blockIdx.x, sm);
}

// ============================================================================
// One launch of the pipelined forward: its first scan_grid workgroups run the
// scan of block i (o written with streaming stores), the rest the prep of
// block i + 1 into the other workspace slot.  The two share no data; the
// scan reads what the previous launch's prep wrote.  Issued in order on one
// stream, these launches keep every dependency of the pipeline (the prep
// before the scan of its block, a slot's scan before its next prep, the
// state carried from block to block), and a launch starts as soon as the one
// before it ends, where a wait on another stream's event took ~11 us per
// block.  Workgroups are dispatched in index order, so the scan's take their
// units first, one per unit; the LDS of the two roles overlays, so the launch
// asks for the prep's footprint and a prep workgroup still fits beside a
// scan workgroup.
// MODE: kPipeForward, the forward (o with streaming stores); kPipeStates, the
// gradient's states pass (the state and Delta entering each chunk, no o);
// kPipeSave, both (the forward that keeps its gradient's records).
static_assert(kScan2Threads == kPrep2Threads, "one workgroup size for both roles");
constexpr int kPipeForward = 0, kPipeStates = 1, kPipeSave = 2;
template <int V, int DK, int DV, int NJ, bool STATES> union PipeSmem {
    PrepSmem<V, DK, DV> prep;
    ScanSmem<bf16, DK, NJ, STATES> scan;
};
template <int V, int DK, int DV, bool RT, int NJ, int MODE>
__global__ __launch_bounds__(kPrep2Threads, (V == kKDA || V == kGDN2) ? 2 : 4)
void chunk_pipe_kernel(Problem p, WsPtrs<bf16> scan_ws, Block scan_blk, unsigned scan_grid,
                       WsPtrs<bf16> prep_ws, Block prep_blk) {
    constexpr bool SG = !VariantTraits<V>::kChannelDecay;
    constexpr bool STATES = MODE == kPipeStates, SAVE = MODE == kPipeSave, NTO = MODE == kPipeForward;
    __shared__ PipeSmem<V, DK, DV, NJ, STATES> sm;
    if (blockIdx.x < scan_grid)
        scan_body<bf16, DK, 2, NJ, STATES, NTO, SG, SAVE>(p, scan_ws, scan_blk, blockIdx.x, sm.scan);
    else
        prep_body<V, DK, DV, RT>(p, prep_ws, prep_blk, blockIdx.x - scan_grid, gridDim.x - scan_grid,
                                 sm.prep);
}

// ---- sequence-parallel state pass -------------------------------------------
// The transitions: segment blockIdx.y of L chunks, for one head and one
// 16-column tile per workgroup of four waves, either the chain from S = 0 over
// d_v's columns (N_s) or the chain over the identity's d_k columns with U~
// taken as zero (M_s).  The chain step is the scan's: Delta = U~ - W S into
// LDS, then S <- Diag(e^{g_C}) S + Kbar^T Delta, S in fp32 accumulators and a
// bf16 copy of S^T in LDS as the operand; the next chunk's factors are loaded
// while the current one is stepped.
template <int DK, int DV, bool SG>
__global__ __launch_bounds__(4 * kWave) void seg_transition_kernel(Problem p, WsPtrs<bf16> ws, long NC,
                                                                  long L, float *Mo, float *No) {
    using TI = bf16;
    using M = Mma<TI>;
    using CO = ChainOps<TI, DK, 1, SG>;
    constexpr int KS_D = CO::KS_D, KS_C = CO::KS_C, NI = CO::NI;
    constexpr int PT = 8, NV = DV / 16, NK = DK / 16;
    __shared__ __attribute__((aligned(16))) TI sSt[2][16][DK + PT];   // S^T
    __shared__ __attribute__((aligned(16))) TI sDt[2][16][C + PT];    // Delta^T
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
    const long seg = blockIdx.y;
    const long c0 = seg * L, nc = (NC - c0 < L ? NC - c0 : L);
    const long ch0 = bh * NC + c0, last = nc - 1;
    auto chunk = [&](long c) { return ch0 + (c < last ? c : last); };
    // U~ is read for the identity's columns too (from value tile 0, in
    // bounds) and multiplied by zero there.
    const int ucol = mrole ? 0 : col0;
    const float uk = mrole ? 0.f : 1.f;
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
    auto step = [&](const CO &op, long c, auto &&pre_update) __attribute__((always_inline)) {
        const int cur = (int)(c & 1);
        typename M::frag Sf[KS_D];
#pragma unroll
        for (int ks = 0; ks < KS_D; ++ks) Sf[ks] = M::load(&sSt[cur][l16][0], ks * M::kK, lane);
        f32x4 d0 = zero4(), d1 = zero4();
#pragma unroll
        for (int ks = 0; ks < KS_D; ks += 2) {
            d0 = M::mma(op.Wf[ks], Sf[ks], d0);
            if (ks + 1 < KS_D) d1 = M::mma(op.Wf[ks + 1], Sf[ks + 1], d1);
        }
        store4(&sDt[cur][l16][16 * w + 4 * lg], uk * to_f32x4(op.U[0]) - (d0 + d1));
        pre_update();
        __syncthreads();
        typename M::frag Df[KS_C];
#pragma unroll
        for (int ks = 0; ks < KS_C; ++ks) Df[ks] = M::load(&sDt[cur][l16][0], ks * M::kK, lane);
#pragma unroll
        for (int a = 0; a < NI; ++a) {
            f32x4 acc = S[a] * op.gam[a];
#pragma unroll
            for (int ks = 0; ks < KS_C; ++ks) acc = M::mma(op.Kf[a][ks], Df[ks], acc);
            S[a] = acc;
        }
        write_st(cur ^ 1);
        __syncthreads();
    };
    CO A, Bq;
    A.load_w(ws, chunk(0), DV, ucol, w, lane);
    A.load_k(ws, chunk(0), w, lane);
    for (long c = 0; c < nc; c += 2) {
        Bq.load_w(ws, chunk(c + 1), DV, ucol, w, lane);
        __builtin_amdgcn_sched_barrier(0);   // issue the prefetch first
        step(A, c, [&] { Bq.load_k(ws, chunk(c + 1), w, lane); });
        if (c + 1 >= nc) break;
        A.load_w(ws, chunk(c + 2), DV, ucol, w, lane);
        __builtin_amdgcn_sched_barrier(0);
        step(Bq, c + 1, [&] { A.load_k(ws, chunk(c + 2), w, lane); });
    }
    const int pitch = mrole ? DK : DV;
    float *out = (mrole ? Mo + (seg * BH + bh) * (long)DK * DK : No + (seg * BH + bh) * (long)DK * DV) + col0;
#pragma unroll
    for (int a = 0; a < NI; ++a)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int i = 16 * (w * NI + a) + 4 * lg + m;
            out[(long)i * pitch + l16] = S[a][m];
        }
}

// The combine: for one head and 16 value columns per workgroup, from the
// initial state (zeros when state_in is NULL), S_{s+1} = M_s S_s + N_s for
// s = 0 .. nseg - 2, each start state written for its segment's scan.  One
// wave per 16 rows of S, on fp32 matrix cores (16x16x4: full fp32 products)
// with M_s and S in LDS; M_{s+1} is loaded into registers while M_s is used.
template <int DK, int DV>
__global__ __launch_bounds__(4 * DK) void seg_combine_kernel(Problem p, const float *s0, long nseg,
                                                             const float *Mi, const float *Ni, float *Sst) {
    using MF = Mma<float>;
    constexpr int NT = 4 * DK;              // DK / 16 waves
    constexpr int MP = DK + 4, SP = 16 + 4; // LDS row pitches (fewer bank conflicts)
    constexpr int NL = DK / 16;             // 16-byte pieces of M per thread
    __shared__ __attribute__((aligned(16))) float sM[DK][MP];
    __shared__ float sS[DK][SP];
    const int tid = threadIdx.x, lane = tid & 63;
    const int R = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave's 16 rows
    const int l16 = lane & 15, lg = lane >> 4;
    const long BH = p.B * p.H;
    const long bh = blockIdx.x / (DV / 16);
    const int col0 = 16 * (int)(blockIdx.x % (DV / 16));
    for (int idx = tid; idx < DK * 16; idx += NT) {
        const int i = idx / 16, c = idx % 16;
        sS[i][c] = s0 ? s0[(bh * DK + i) * DV + col0 + c] : 0.f;
    }
    f32x4 mr[NL];
    auto load_m = [&](long s) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(Mi + (s * BH + bh) * (long)DK * DK);
#pragma unroll
        for (int n = 0; n < NL; ++n) mr[n] = src[tid + n * NT];
    };
    auto store_m = [&]() {
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            const int e = 4 * (tid + n * NT);
            *reinterpret_cast<f32x4 *>(&sM[e / DK][e % DK]) = mr[n];
        }
    };
    load_m(0);
    store_m();
    __syncthreads();
    for (long s = 0; s + 1 < nseg; ++s) {
        const bool next = s + 2 < nseg;   // M_{s+1} is needed
        if (next) load_m(s + 1);
        const float *Nt = Ni + (s * BH + bh) * (long)DK * DV + col0;
        f32x4 acc;
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = Nt[(16 * R + 4 * lg + m) * DV + l16];
#pragma unroll 8
        for (int k0 = 0; k0 < DK; k0 += 4)
            acc = MF::mma(sM[16 * R + l16][k0 + lg], sS[k0 + lg][l16], acc);
        __syncthreads();   // every wave is done reading M_s and S_s
        float *St = Sst + (s * BH + bh) * (long)DK * DV + col0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 16 * R + 4 * lg + m;
            sS[r][l16] = acc[m];
            St[r * DV + l16] = acc[m];
        }
        if (next) store_m();
        __syncthreads();
    }
}

// The outputs: segment blockIdx.y's scan (the forward's scan kernel body,
// 16-column slices) from its start state; only the last segment writes the
// final state.  blk describes the whole sequence.  STATES / SAVE: the
// gradient's records instead of o, or both (see scan_body); the record
// pointers of blk are moved by the segment's first chunk like the factors.
template <int DK, bool SG, bool STATES = false, bool SAVE = false>
__global__ __launch_bounds__(kScan2Threads, SG ? 4 : 2) void seg_scan_kernel(Problem p, WsPtrs<bf16> ws,
                                                                            Block blk, long L,
                                                                            const float *Sst) {
    __shared__ ScanSmem<bf16, DK, 1, STATES> sm;
    const long seg = blockIdx.y, nseg = gridDim.y, NC = blk.nc;
    Block b = blk;
    b.c0 = seg * L;
    b.nc = (int)(NC - b.c0 < L ? NC - b.c0 : L);
    b.s_in = seg == 0 ? blk.s_in : Sst + (seg - 1) * p.B * p.H * DK * p.dv;
    b.s_out = seg == nseg - 1 ? blk.s_out : nullptr;
    // the factors of the segment's chunks: every pointer moved by c0 chunks
    WsPtrs<bf16> w = ws;
    w.W += b.c0 * C * DK;
    w.Ut += b.c0 * C * p.dv;
    w.Qt += b.c0 * C * DK;
    w.Kbt += b.c0 * C * DK;
    w.P += b.c0 * C * C;
    w.gam += b.c0 * DK;
    if constexpr (STATES || SAVE) {
        b.s_chunks = static_cast<bf16 *>(blk.s_chunks) + b.c0 * DK * p.dv;
        b.d_chunks = static_cast<bf16 *>(blk.d_chunks) + b.c0 * C * p.dv;
    }
    scan_body<bf16, DK, 2, 1, STATES, false, SG, SAVE>(p, w, b, blockIdx.x, sm);
}

// ---- dispatch -----------------------------------------------------------------


constexpr int kMaxDevices = 64;

// Compute units of the current device, queried once per device.  Threads
// that race on the first query each store the same value; the atomics make
// that well defined.
hipError_t device_cus(long *out) {
    static std::atomic<long> ncu[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    long n = ncu[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        int cus = 0;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
            return e;
        n = cus > 0 ? cus : 1;
        ncu[dev].store(n, std::memory_order_relaxed);
    }
    *out = n;
    return hipSuccess;
}

// Whether the scan takes 32-column slices (see launch_scan), and its number of
// workgroups.  concurrent: a prep runs beside it.
bool scan_wide(const Problem &p, bool scalar_decay, bool concurrent, long cus) {
    if (!p.bf16 || p.dv % 32 != 0) return false;
    return scalar_decay ? p.B * p.H * (p.dv / 16) > cus : concurrent;
}
long scan_workgroups(const Problem &p, bool scalar_decay, bool concurrent, long cus) {
    return p.B * p.H * (p.dv / (scan_wide(p, scalar_decay, concurrent, cus) ? 32 : 16));
}

// Workgroups of the bf16 prep kernel that the device holds at once (resident
// slots) and its compute units, queried once per device and kernel instance.
// The unit count is stored before the slot count (release) and read after it
// (acquire), so a thread that sees the slots also sees the units.
template <int V, int DK, int DV, bool RT> hipError_t prep_slots(long *slots_out, long *cus_out) {
    static std::atomic<long> slots[kMaxDevices] = {}, ncu[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    long sl = slots[dev].load(std::memory_order_acquire), nc = 0;
    if (sl == 0) {
        int per_cu = 0, cus = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(&chunk_prep_bf16_kernel<V, DK, DV, RT>),
            kPrep2Threads, 0);
        if (e != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) !=
            hipSuccess)
            return e;
        nc = cus > 0 ? cus : 1;
        sl = (long)(per_cu > 0 ? per_cu : 1) * nc;
        ncu[dev].store(nc, std::memory_order_relaxed);
        slots[dev].store(sl, std::memory_order_release);
    } else {
        nc = ncu[dev].load(std::memory_order_relaxed);
    }
    *slots_out = sl;
    *cus_out = nc;
    return hipSuccess;
}

// Workgroups of a bf16 prep over the items of blk.  Persistent workgroups,
// each looping over chunk-heads with the next one's inputs in flight.  Alone,
// the grid fills every resident slot; beside a concurrent scan, one workgroup
// per compute unit, so that a scan workgroup still fits on every unit, plus a
// second one for each unit the scan leaves free: in whichever order the two
// grids are placed, every scan workgroup still finds a unit with room.
template <int V, int DK, int DV>
hipError_t prep_grid(const Problem &p, const Block &blk, bool concurrent, long *grid) {
    long slots = 0, cus = 0;
    hipError_t e = p.v_route ? prep_slots<V, DK, DV, true>(&slots, &cus)
                             : prep_slots<V, DK, DV, false>(&slots, &cus);
    if (e != hipSuccess) return e;
    const long items = (long)blk.nc * p.H * p.B;
    const long free_cus = cus - scan_workgroups(p, !VariantTraits<V>::kChannelDecay, concurrent, cus);
    const long extra = free_cus > 0 ? (free_cus < slots - cus ? free_cus : slots - cus) : 0;
    // A channel-decay prep (one workgroup per unit) never shares a unit with
    // the scan: beside one it takes just the units the scan leaves free, so
    // that no workgroup of its static split starts late.
    long want = slots;
    if (concurrent)
        want = VariantTraits<V>::kChannelDecay ? (free_cus > 0 ? free_cus : cus) : cus + extra;
    *grid = items < want ? items : want;
    return hipSuccess;
}

template <int V, typename TI, int DK, int DV>
hipError_t launch_prep(const Problem &p, const WsPtrs<TI> &w, const Block &blk, bool concurrent,
                       hipStream_t st) {
    if constexpr (sizeof(TI) == 2) {
        long grid = 0;
        hipError_t e = prep_grid<V, DK, DV>(p, blk, concurrent, &grid);
        if (e != hipSuccess) return e;
        const bool rt = p.v_route != nullptr;
        if (rt)
            hipLaunchKernelGGL((chunk_prep_bf16_kernel<V, DK, DV, true>), dim3((unsigned)grid),
                               dim3(kPrep2Threads), 0, st, p, w, blk);
        else
            hipLaunchKernelGGL((chunk_prep_bf16_kernel<V, DK, DV, false>), dim3((unsigned)grid),
                               dim3(kPrep2Threads), 0, st, p, w, blk);
    } else {
        const dim3 pgrid((unsigned)blk.nc, (unsigned)p.H, (unsigned)p.B);
        hipLaunchKernelGGL((chunk_prep_kernel<V, TI, DK, DV>), pgrid, dim3(kPrepThreads), 0, st,
                           p, w, blk);
    }
    return hipGetLastError();
}


template <typename TI, int DK, int DV>
hipError_t launch_scan(const Problem &p, const WsPtrs<TI> &w, const Block &blk, bool scalar_decay,
                       bool concurrent, hipStream_t st) {
    constexpr int DEPTH = sizeof(TI) == 2 ? 2 : 1;
    // Value columns per workgroup: 16, so that every head's chain is cut into
    // as many short, independent column slices as possible.  When 16-column
    // slices would need more workgroups than there are compute units, 32
    // (scalar decay, bf16: the instance that fits the register budget beside
    // a prep workgroup) halves the factor loads per column instead; below
    // that, the longer per-chunk chain of a wide slice costs more than it saves.
    // A channel-decay scan beside its prep takes 32 columns too: that prep
    // cannot share a unit with it, and the units a wide scan frees speed the
    // prep up more than the longer chain slows the scan.
    long cus = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    const bool wide = scan_wide(p, scalar_decay, concurrent, cus);
    auto go = [&](auto sg, auto nj) {
        constexpr bool SG = decltype(sg)::value;
        constexpr int NJ = decltype(nj)::value;
        const long nwg = p.B * p.H * (DV / (16 * NJ));
        const long grid = kXcds * ((nwg + kXcds - 1) / kXcds);
        if (blk.s_chunks && blk.with_o)
            hipLaunchKernelGGL((chunk_scan2_kernel<TI, DK, DEPTH, NJ, false, false, SG, true>),
                               dim3((unsigned)grid), dim3(kScan2Threads), 0, st, p, w, blk);
        else if (blk.s_chunks)
            hipLaunchKernelGGL((chunk_scan2_kernel<TI, DK, DEPTH, NJ, true, false, SG>),
                               dim3((unsigned)grid), dim3(kScan2Threads), 0, st, p, w, blk);
        else if (blk.nt_out)
            hipLaunchKernelGGL((chunk_scan2_kernel<TI, DK, DEPTH, NJ, false, true, SG>),
                               dim3((unsigned)grid), dim3(kScan2Threads), 0, st, p, w, blk);
        else
            hipLaunchKernelGGL((chunk_scan2_kernel<TI, DK, DEPTH, NJ, false, false, SG>),
                               dim3((unsigned)grid), dim3(kScan2Threads), 0, st, p, w, blk);
    };
    using One = std::integral_constant<int, 1>;
    using Two = std::integral_constant<int, sizeof(TI) == 2 && DV % 32 == 0 ? 2 : 1>;
    if (!scalar_decay) {
        if (wide) go(std::false_type{}, Two{});
        else go(std::false_type{}, One{});
    }
    else if (wide) go(std::true_type{}, Two{});
    else go(std::true_type{}, One{});
    return hipGetLastError();
}

// The scan of block sb and the prep of block pb in one launch
// (chunk_pipe_kernel), with the grids each would take beside the other.  The
// states and saving scans take no routed value.
template <int V, int DK, int DV, int MODE>
hipError_t launch_pipe(const Problem &p, const WsPtrs<bf16> &sw, const Block &sb,
                       const WsPtrs<bf16> &pw, const Block &pb, hipStream_t st) {
    long cus = 0, pgrid = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    if ((e = prep_grid<V, DK, DV>(p, pb, true, &pgrid)) != hipSuccess) return e;
    const bool wide = scan_wide(p, !VariantTraits<V>::kChannelDecay, true, cus);
    const long nwg = p.B * p.H * (DV / (wide ? 32 : 16));
    const long sgrid = kXcds * ((nwg + kXcds - 1) / kXcds);
    const dim3 grid((unsigned)(sgrid + pgrid));
    auto go = [&](auto nj) {
        constexpr int NJ = decltype(nj)::value;
        if constexpr (MODE == kPipeForward) {
            if (p.v_route) {
                hipLaunchKernelGGL((chunk_pipe_kernel<V, DK, DV, true, NJ, MODE>), grid,
                                   dim3(kPrep2Threads), 0, st, p, sw, sb, (unsigned)sgrid, pw, pb);
                return;
            }
        }
        hipLaunchKernelGGL((chunk_pipe_kernel<V, DK, DV, false, NJ, MODE>), grid, dim3(kPrep2Threads),
                           0, st, p, sw, sb, (unsigned)sgrid, pw, pb);
    };
    if (wide) go(std::integral_constant<int, DV % 32 == 0 ? 2 : 1>{});
    else go(std::integral_constant<int, 1>{});
    return hipGetLastError();
}

// The sequence-parallel forward (see SegPlan), all on the caller's stream.
// `fac` holds the factors of every chunk (ws_layout of all chunks); `seg`
// the segments' transitions, local end states and start states at the
// plan's offsets relative to the end of the factors.  MODE: kPipeForward
// (o), kPipeStates (the gradient's records from s_in, no o), kPipeSave (both).
template <int V, int DK, int DV, int MODE = kPipeForward>
hipError_t launch_segments(const Problem &p, const SegPlan &s, void *fac, void *seg, const float *s_in,
                           float *s_out, void *s_chunks, void *d_chunks, hipStream_t st) {
    constexpr bool SG = !VariantTraits<V>::kChannelDecay;
    const long NC = (p.T + C - 1) / C, BH = p.B * p.H;
    const WsPtrs<bf16> w = ws_ptrs<bf16>(p, NC, fac);
    const Block all{0, (int)NC, (int)NC, s_in, s_out, s_chunks, d_chunks, nullptr, 0u, nullptr,
                    false, MODE == kPipeSave};
    hipError_t e = launch_prep<V, bf16, DK, DV>(p, w, all, false, st);
    if (e != hipSuccess) return e;
    const size_t base = ws_layout(p, NC).total;
    char *sb = static_cast<char *>(seg);
    float *Mo = reinterpret_cast<float *>(sb + (s.M - base)), *No = reinterpret_cast<float *>(sb + (s.N - base));
    float *Sst = reinterpret_cast<float *>(sb + (s.S - base));
    const long nwg1 = BH * (DV / 16 + DK / 16);
    hipLaunchKernelGGL((seg_transition_kernel<DK, DV, SG>),
                       dim3((unsigned)(kXcds * ((nwg1 + kXcds - 1) / kXcds)), (unsigned)(s.nseg - 1)),
                       dim3(4 * kWave), 0, st, p, w, NC, s.L, Mo, No);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((seg_combine_kernel<DK, DV>), dim3((unsigned)(BH * (DV / 16))), dim3(4 * DK), 0, st, p,
                       s_in, s.nseg, static_cast<const float *>(Mo), static_cast<const float *>(No), Sst);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const long nwg3 = BH * (DV / 16);
    const dim3 grid3((unsigned)(kXcds * ((nwg3 + kXcds - 1) / kXcds)), (unsigned)s.nseg);
    const float *Sc = Sst;
    if constexpr (MODE == kPipeStates)
        hipLaunchKernelGGL((seg_scan_kernel<DK, SG, true, false>), grid3, dim3(kScan2Threads), 0, st, p, w,
                           all, s.L, Sc);
    else if constexpr (MODE == kPipeSave)
        hipLaunchKernelGGL((seg_scan_kernel<DK, SG, false, true>), grid3, dim3(kScan2Threads), 0, st, p, w,
                           all, s.L, Sc);
    else
        hipLaunchKernelGGL((seg_scan_kernel<DK, SG>), grid3, dim3(kScan2Threads), 0, st, p, w, all, s.L, Sc);
    return hipGetLastError();
}

template <int V, typename TI, int DK, int DV>
hipError_t launch_shape(const Problem &p, void *ws, hipStream_t stream) {
    if constexpr (sizeof(TI) == 2) {
        const SegPlan s = seg_plan(p);
        if (s.nseg > 1) {
            char *fac = static_cast<char *>(ws);
            return launch_segments<V, DK, DV>(p, s, fac, fac + ws_layout(p, (p.T + C - 1) / C).total,
                                              p.state_in, p.state_out, nullptr, nullptr, stream);
        }
    }
    const Plan q = make_plan(p);
    char *base = static_cast<char *>(ws);
    if (q.nblk == 1) {
        const WsPtrs<TI> w = ws_ptrs<TI>(p, q.nb, base);
        const Block blk{0, (int)q.NC, (int)q.nb, p.state_in, p.state_out, nullptr, nullptr,
                        nullptr, 0u, nullptr, false};
        hipError_t e = launch_prep<V, TI, DK, DV>(p, w, blk, false, stream);
        if (e != hipSuccess) return e;
        return launch_scan<TI, DK, DV>(p, w, blk, !VariantTraits<V>::kChannelDecay, false, stream);
    }
    // Pipelined, on the caller's stream: the prep of block 0 alone (every
    // resident slot, a fixed stride; it clears the ticket counter that the
    // later scalar-decay preps draw from, so that the units without a scan
    // take more items), then one launch per block running the scan of block i
    // beside the prep of block i + 1 (chunk_pipe_kernel), then the last scan.
    // Two workspace slots alternate.  A channel-decay prep fills a unit's
    // registers and never shares one; it runs on the units the scan leaves
    // free, with a static split, which measured faster.
    hipError_t e = hipSuccess;
    float *carrier = reinterpret_cast<float *>(base + 2 * q.slot);
    unsigned *ticket = reinterpret_cast<unsigned *>(base + 2 * q.slot + q.carrier);
    unsigned ticket_base = 0;
    auto block = [&](long i) {
        const long c0 = i * q.nb;
        const bool tickets = i > 0 && !VariantTraits<V>::kChannelDecay;
        return Block{c0, (int)min(q.nb, q.NC - c0), (int)q.nb,
                     i == 0 ? p.state_in : carrier, i == q.nblk - 1 ? p.state_out : carrier,
                     nullptr, nullptr, tickets ? ticket : nullptr, ticket_base,
                     i == 0 ? ticket : nullptr, true};
    };
    auto slot = [&](long i) { return ws_ptrs<TI>(p, q.nb, base + (i & 1) * q.slot); };
    if ((e = launch_prep<V, TI, DK, DV>(p, slot(0), block(0), false, stream)) != hipSuccess) return e;
    for (long i = 0; i < q.nblk; ++i) {
        const Block sb = block(i);
        if (i + 1 == q.nblk)
            return launch_scan<TI, DK, DV>(p, slot(i), sb, !VariantTraits<V>::kChannelDecay, true, stream);
        const Block pb = block(i + 1);
        if (pb.ticket) ticket_base += (unsigned)(pb.nc * p.H * p.B);
        if constexpr (sizeof(TI) == 2)
            e = launch_pipe<V, DK, DV, kPipeForward>(p, slot(i), sb, slot(i + 1), pb, stream);
        else
            e = hipErrorInvalidValue;   // only bf16 inputs are pipelined
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---- the gradient's states pass ----------------------------------------------
// The workspace holds the factors of all chunks at their own positions: the
// pointers of a block are shifted by its first chunk, so the kernels' block-
// local chunk index lands on the global one.
template <typename TI> WsPtrs<TI> shifted(WsPtrs<TI> w, const Problem &p, long c0) {
    w.W += c0 * C * p.dk;
    w.Ut += c0 * C * p.dv;
    w.Qt += c0 * C * p.dk;
    w.Kbt += c0 * C * p.dk;
    w.P += c0 * C * C;
    w.gam += c0 * p.dk;
    return w;
}

template <typename T> struct type_tag { using type = T; };

// Calls f(variant, dtype tag, DK, DV) with compile-time constants for p.
template <typename F> hipError_t dispatch_shape(const Problem &p, F &&f) {
    auto with_type = [&](auto v) {
        auto with_dims = [&](auto ti) {
            using I = std::integral_constant<int, 128>;
            using J = std::integral_constant<int, 64>;
            if (p.dk == 128 && p.dv == 128) return f(v, ti, I{}, I{});
            if (p.dk == 128 && p.dv == 64) return f(v, ti, I{}, J{});
            if (p.dk == 64 && p.dv == 128) return f(v, ti, J{}, I{});
            return f(v, ti, J{}, J{});
        };
        return p.bf16 ? with_dims(type_tag<bf16>{}) : with_dims(type_tag<float>{});
    };
    switch (p.variant) {
    case kDeltaNet: return with_type(std::integral_constant<int, kDeltaNet>{});
    case kGatedDeltaNet: return with_type(std::integral_constant<int, kGatedDeltaNet>{});
    case kKDA: return with_type(std::integral_constant<int, kKDA>{});
    case kGDN2: return with_type(std::integral_constant<int, kGDN2>{});
    case kKLA: return with_type(std::integral_constant<int, kKLA>{});
    default: return hipErrorInvalidValue;
    }
}

template <int V, typename TI>
hipError_t launch_t(const Problem &p, void *ws, hipStream_t stream) {
    if (p.dk == 128 && p.dv == 128) return launch_shape<V, TI, 128, 128>(p, ws, stream);
    if (p.dk == 128 && p.dv == 64) return launch_shape<V, TI, 128, 64>(p, ws, stream);
    if (p.dk == 64 && p.dv == 128) return launch_shape<V, TI, 64, 128>(p, ws, stream);
    return launch_shape<V, TI, 64, 64>(p, ws, stream);
}

template <int V>
hipError_t launch_v(const Problem &p, void *ws, hipStream_t stream) {
    return p.bf16 ? launch_t<V, bf16>(p, ws, stream) : launch_t<V, float>(p, ws, stream);
}

}  // namespace

size_t forward_workspace_bytes(const Problem &p) {
    const SegPlan s = seg_plan(p);
    return s.nseg > 1 ? s.total : make_plan(p).total;
}

size_t forward_states_bytes(const Problem &p) { return ws_layout(p, (p.T + C - 1) / C).total; }

ForwardStates forward_states_ptrs(const Problem &p, void *workspace) {
    const long NC = (p.T + C - 1) / C;
    const WsLayout L = ws_layout(p, NC);
    char *b = static_cast<char *>(workspace);
    return ForwardStates{b + L.W, b + L.Ut, b + L.Qt, b + L.Kbt, b + L.P,
                         reinterpret_cast<const float *>(b + L.gam), NC};
}

hipError_t launch_states_pass(const Problem &p, void *workspace, const float *s_in, float *s_out,
                              void *s_chunks, void *d_chunks, bool with_o, void *scratch,
                              size_t scratch_bytes, hipStream_t stream) {
    return dispatch_shape(p, [&](auto v, auto ti, auto dk, auto dv) -> hipError_t {
        using TI = typename decltype(ti)::type;
        constexpr int V = decltype(v)::value, DK = decltype(dk)::value, DV = decltype(dv)::value;
        constexpr bool kScalar = !VariantTraits<V>::kChannelDecay;
        const long NC = (p.T + C - 1) / C;
        const WsPtrs<TI> full = ws_ptrs<TI>(p, NC, workspace);
        // Every chunk keeps its own factors and records: a block of chunks
        // [c0, c0 + nc) gets the factor pointers (shifted) and the record
        // pointers moved by c0, so that the kernels' block-local chunk index
        // lands on the global one.
        auto block = [&](long c0, int nc, const float *si, float *so, unsigned *tk, unsigned tb,
                         unsigned *tclear) {
            return Block{c0, nc, (int)NC, si, so,
                         static_cast<TI *>(s_chunks) + c0 * DK * (long)DV,
                         static_cast<TI *>(d_chunks) + c0 * C * (long)DV, tk, tb, tclear, false,
                         with_o};
        };
        // The forward's choice of segments, of when to pipeline, and its
        // blocks.  Segmented, the segments' arrays go to the scratch.
        if constexpr (sizeof(TI) == 2) {
            const SegPlan sp = seg_plan(p);
            if (sp.nseg > 1 && scratch && scratch_bytes >= sp.total - ws_layout(p, NC).total) {
                return with_o ? launch_segments<V, DK, DV, kPipeSave>(p, sp, workspace, scratch, s_in,
                                                                      s_out, s_chunks, d_chunks, stream)
                              : launch_segments<V, DK, DV, kPipeStates>(p, sp, workspace, scratch, s_in,
                                                                        s_out, s_chunks, d_chunks, stream);
            }
        }
        const Plan q = make_plan(p);
        const size_t carrier_bytes = align256((size_t)p.B * p.H * DK * DV * 4);
        if constexpr (sizeof(TI) == 2) {
            if (q.nblk > 1 && scratch && scratch_bytes >= carrier_bytes + 256) {
                // As the pipelined forward: the prep of block 0 alone (it
                // clears the ticket counter), then one launch per block with
                // the scan of block i beside the prep of block i + 1, then the
                // last scan, all on `stream`; the state is carried between
                // blocks in fp32 in the scratch.
                float *carrier = static_cast<float *>(scratch);
                unsigned *ticket =
                    reinterpret_cast<unsigned *>(static_cast<char *>(scratch) + carrier_bytes);
                unsigned ticket_base = 0;
                auto blk_i = [&](long i) {
                    const long c0 = i * q.nb;
                    const bool tickets = i > 0 && kScalar;
                    return block(c0, (int)min(q.nb, q.NC - c0), i == 0 ? s_in : carrier,
                                 i == q.nblk - 1 ? s_out : carrier, tickets ? ticket : nullptr,
                                 ticket_base, i == 0 ? ticket : nullptr);
                };
                hipError_t e = launch_prep<V, TI, DK, DV>(p, full, blk_i(0), false, stream);
                if (e != hipSuccess) return e;
                for (long i = 0; i < q.nblk; ++i) {
                    const Block sb = blk_i(i);
                    const WsPtrs<TI> w = shifted(full, p, sb.c0);
                    if (i + 1 == q.nblk) return launch_scan<TI, DK, DV>(p, w, sb, kScalar, true, stream);
                    const Block pb = blk_i(i + 1);
                    if (pb.ticket) ticket_base += (unsigned)(pb.nc * p.H * p.B);
                    const WsPtrs<TI> wn = shifted(full, p, pb.c0);
                    e = with_o ? launch_pipe<V, DK, DV, kPipeSave>(p, w, sb, wn, pb, stream)
                               : launch_pipe<V, DK, DV, kPipeStates>(p, w, sb, wn, pb, stream);
                    if (e != hipSuccess) return e;
                }
                return hipSuccess;
            }
        }
        hipError_t e = launch_prep<V, TI, DK, DV>(
            p, full, block(0, (int)NC, nullptr, nullptr, nullptr, 0u, nullptr), false, stream);
        if (e != hipSuccess) return e;
        return launch_scan<TI, DK, DV>(p, full, block(0, (int)NC, s_in, s_out, nullptr, 0u, nullptr),
                                       kScalar, false, stream);
    });
}

long forward_segments(const Problem &p, long *L) {
    const SegPlan s = seg_plan(p);
    if (L) *L = s.L;
    return s.nseg > 1 ? s.nseg : 0;
}

hipError_t launch_segment_combine(const Problem &p, const float *s0, long nseg, const float *M,
                                  const float *N, float *Sst, hipStream_t stream) {
    auto go = [&](auto dk, auto dv) {
        constexpr int DK = decltype(dk)::value, DV = decltype(dv)::value;
        hipLaunchKernelGGL((seg_combine_kernel<DK, DV>), dim3((unsigned)(p.B * p.H * (DV / 16))),
                           dim3(4 * DK), 0, stream, p, s0, nseg, M, N, Sst);
        return hipGetLastError();
    };
    using I = std::integral_constant<int, 128>;
    using J = std::integral_constant<int, 64>;
    if (p.dk == 128 && p.dv == 128) return go(I{}, I{});
    if (p.dk == 128 && p.dv == 64) return go(I{}, J{});
    if (p.dk == 64 && p.dv == 128) return go(J{}, I{});
    return go(J{}, J{});
}

hipError_t launch_forward(const Problem &p, void *workspace, hipStream_t stream) {
    switch (p.variant) {
    case kDeltaNet: return launch_v<kDeltaNet>(p, workspace, stream);
    case kGatedDeltaNet: return launch_v<kGatedDeltaNet>(p, workspace, stream);
    case kKDA: return launch_v<kKDA>(p, workspace, stream);
    case kGDN2: return launch_v<kGDN2>(p, workspace, stream);
    case kKLA: return launch_v<kKLA>(p, workspace, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdr
