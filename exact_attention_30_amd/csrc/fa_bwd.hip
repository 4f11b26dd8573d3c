// Backward kernels ("L'attention fusionnée", «La passe arrière»).
//
// P is never stored: every kernel rebuilds it tile by tile from the scores and
// the saved row log-sum-exp, P = exp(S * scale - L) (computed as
// exp2(S * scale*log2(e) - L*log2(e))).  The softmax Jacobian term of each query
// row is replaced by Delta_i = sum_d dO_id O_id, produced by a row-reduction
// kernel before the other two.  Gradients:
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - Delta),
//     dQ = dS K * scale,   dK = dS^T Q * scale.
// As on that page, the gradients come from two kernels and no atomic
// additions: one walks query tiles for a fixed key tile (dK, dV), the other
// walks key tiles for a fixed query tile (dQ), so results do not depend on the
// order in which workgroups run.  With grouped-query attention the dK/dV
// kernel also loops over the query heads that share the kv head, which keeps
// the group sum inside one workgroup.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

// ---------------------------------------------------------------------------
// Delta_i = sum_d dO_id * O_id.  HBM-bound: each row is read once, 16 bytes per
// lane, and reduced over the lanes of the row in a fixed order.
// ---------------------------------------------------------------------------
// lanes per row of the preprocess: 16 bytes each, rounded up to a power of
// two so the row reduction is a butterfly
template <class E, int D>
__host__ __device__ constexpr int pre_lanes()
{
    int n = D / (16 / (int)sizeof(E)), p = 1;
    while (p < n) p *= 2;
    return p;
}

// E: element type of dO (and of O); EO: element type of O, float32 with
// bf16 dO when O was stored unrounded.  A lane takes the 16 bytes of dO that
// hold its CH columns and the O of those columns, so with EO = float and
// E = bf16 the fma chain runs over the same columns in the same order as with
// a bf16 O: an O holding bf16 values gives the same bits.
template <class E, int D, class EO = E>
__global__ __launch_bounds__(256) void bwd_pre_kernel(PreArgs a)
{
    constexpr int CH = 16 / (int)sizeof(E);
    constexpr int LPR = pre_lanes<E, D>();  // lanes per row (a power of two)
    constexpr int RPB = 256 / LPR;          // rows per workgroup
    const int tid = threadIdx.x;
    const long row = (long)blockIdx.x * RPB + tid / LPR;
    const int col = (tid % LPR) * CH;
    float acc = 0.f;
    if (row < a.rows && col < D) {  // lanes past the end of a row add nothing
        const EO* o = static_cast<const EO*>(a.o) + row * D + col;
        const E* d = static_cast<const E*>(a.dout) + row * D + col;
        if constexpr (sizeof(E) == 2 && sizeof(EO) == 2) {
            const bf16x8 x = *reinterpret_cast<const bf16x8*>(o);
            const bf16x8 y = *reinterpret_cast<const bf16x8*>(d);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
        } else if constexpr (sizeof(E) == 2) {
            const f32x4 x0 = reinterpret_cast<const f32x4*>(o)[0];
            const f32x4 x1 = reinterpret_cast<const f32x4*>(o)[1];
            const bf16x8 y = *reinterpret_cast<const bf16x8*>(d);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = fmaf(x0[e], (float)y[e], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = fmaf(x1[e], (float)y[4 + e], acc);
        } else {
            const f32x4 x = *reinterpret_cast<const f32x4*>(o);
            const f32x4 y = *reinterpret_cast<const f32x4*>(d);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = fmaf(x[e], y[e], acc);
        }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (row < a.rows && (tid % LPR) == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV.  One workgroup per (batch, kv head, key tile of NW*32 keys); wave w
// owns keys key0 + 32w .. +31.  K of those keys stays in registers (B operand
// of S = Q K^T); V of the workgroup's keys is loaded once into LDS and read as
// the B operand of dP = dO V^T, which keeps the kernel within the register
// budget of two waves per SIMD.  Query tiles of BQ rows (of every query head
// of the group) stream into LDS in natural layout (asynchronous loads,
// double-buffered); they are read row-wise as A operands of S and dP, and
// transposed (ds_read_b64_tr_b16) as A operands of dK^T += Q^T dS and
// dV^T += dO^T P.  S, dP, P and dS share one accumulator layout (rows =
// queries, columns = keys), so P and dS feed those products from registers.
// ---------------------------------------------------------------------------
template <class E, int D, int NW, int BQ>
struct DkdvCfg {
    static constexpr int NT = NW * 64;
    static constexpr int BK = NW * 32;
    using QTile = DmaTile<E, D, BQ, NT>;
    using VTile = DmaTile<E, D, BK, NT>;
    static constexpr int STATS = 2 * BQ * 4;  // L*log2(e) and Delta rows (floats)
    static constexpr int BUF = 2 * QTile::BYTES + STATS;
    static constexpr size_t SMEM = (size_t)VTile::BYTES + 2 * (size_t)BUF;
};

template <class E, int D, int NW, int BQ, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, sizeof(E) == 2 ? 8 / NW : 1) void bwd_dkdv_kernel(BwdArgs a)
{
    using Cfg = DkdvCfg<E, D, NW, BQ>;
    using QT = typename Cfg::QTile;
    using VT = typename Cfg::VTile;
    constexpr int BK = Cfg::BK;
    constexpr int NQB = BQ / 32;
    constexpr int NDB = D / 32;
    constexpr int NKS = D / 16;
    static_assert(2 * BQ <= Cfg::NT, "one thread per L / Delta row");

    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* Vs = smem;
    unsigned char* qbuf = smem + VT::BYTES;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int c = lane & 31;
    const int G = a.Hq / a.Hkv;

    const int nkt = (a.Tk + BK - 1) / BK;
    // causal: the first key tiles see the most query rows
    const TileId id = map_tile(blockIdx.x, a.B, a.Hq, a.Hkv, 1, nkt, false);
    const int b = id.b, hk = id.h;
    const int key0 = id.tile * BK;
    const int krow = key0 + w * 32 + c;  // the key this lane owns

    const size_t kvoff = (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const E* kh = static_cast<const E*>(a.k) + kvoff;
    const E* vh = static_cast<const E*>(a.v) + kvoff;

    // query tiles that see this key tile (query row i sees keys j <= i + off
    // when causal), for each of the G query heads
    const int nq = (a.Tq + BQ - 1) / BQ;
    const int i0 = CAUSAL ? max(key0 - a.off, 0) / BQ : 0;
    const int niq = max(nq - i0, 0);
    const int nit = G * niq;

    QT qdma;
    qdma.init(tid);
    // issue the loads of flattened iteration `it` (query head, query tile);
    // the L / Delta row of this thread (if any) goes to a register
    auto issue = [&](int it, unsigned char* buf, float& stat) {
        const int hq = hk * G + it / niq, i = i0 + it % niq;
        const size_t qoff = (size_t)(b * a.Hq + hq) * a.Tq * D;
        qdma.load(buf, static_cast<const E*>(a.q) + qoff, i * BQ, a.Tq, w);
        qdma.load(buf + QT::BYTES, static_cast<const E*>(a.dout) + qoff, i * BQ, a.Tq, w);
        if (tid < 2 * BQ) {
            const int qi = min(i * BQ + (tid % BQ), a.Tq - 1);
            const size_t off = (size_t)(b * a.Hq + hq) * a.Tq + qi;
            stat = tid < BQ ? a.lse[off] * kLog2e : a.delta[off];
        }
    };

    {
        VT vdma;
        vdma.init(tid);
        vdma.load(Vs, vh, key0, a.Tk, w);
    }
    float stat = 0.f;
    if (nit > 0) issue(0, qbuf, stat);  // no query row may see this key block

    Frag<E> kf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kf[ks] = global_frag<E>(kh, krow, a.Tk, D, 16 * ks + 8 * g);

    // Q and dO rows (A of S, dP); the V tile has the same row format, so the
    // same offsets read V rows w*32 + c (B of dP)
    RowReader<QT, E, D> qrd;
    qrd.init(c, g);
    static_assert(QT::ROWBYTES == VT::ROWBYTES, "Q and V tiles share a row format");
    TrReader<QT, E, D> trd;   // Q^T and dO^T (A of dK^T, dV^T)
    trd.init(lane);

    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = f32x16{};

    if (tid < 2 * BQ) reinterpret_cast<float*>(qbuf + 2 * QT::BYTES)[tid] = stat;
    wait_global_loads();
    __syncthreads();

    for (int it = 0; it < nit; ++it) {
        const int BI = it & 1;
        const unsigned char* Qs = qbuf + BI * Cfg::BUF;
        const unsigned char* dOs = Qs + QT::BYTES;
        const float* Ls = reinterpret_cast<const float*>(dOs + QT::BYTES);
        const float* Ds = Ls + BQ;
        unsigned char* nb = qbuf + (1 - BI) * Cfg::BUF;
        const bool more = it + 1 < nit;
        if (more) issue(it + 1, nb, stat);

        const int qbase = (i0 + it % niq) * BQ;
        const bool need_mask = (CAUSAL && qbase + a.off < key0 + BK - 1) || (qbase + BQ > a.Tq);

#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) mma(s, qrd.frag(Qs, qb * 32, ks), kf[ks]);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) mma(dp, qrd.frag(dOs, qb * 32, ks), qrd.frag(Vs, w * 32, ks));
            // rows of this lane's registers: queries qb*32 + 8*(r/4) + 4g + r%4
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int q = qb * 32 + 8 * rg + 4 * g;
                const f32x4 L4 = *reinterpret_cast<const f32x4*>(Ls + q);
                const f32x4 D4 = *reinterpret_cast<const f32x4*>(Ds + q);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * rg + e;
                    float p = fast_exp2(fmaf(s[r], a.c, -L4[e]));
                    if (need_mask) {
                        const int qi = qbase + q + e;
                        const bool vis = (qi < a.Tq) && (!CAUSAL || krow <= qi + a.off);
                        if (!vis) p = 0.f;
                    }
                    s[r] = p;                     // P
                    dp[r] = p * (dp[r] - D4[e]);  // dS
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const Frag<E> pf = acc_frag<E>(s, t);
                const Frag<E> sf = acc_frag<E>(dp, t);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    mma(dv[db], trd.frag(dOs, qb * 32 + 16 * t, db), pf);
                    mma(dk[db], trd.frag(Qs, qb * 32 + 16 * t, db), sf);
                }
            }
        }

        if (more && tid < 2 * BQ) reinterpret_cast<float*>(nb + 2 * QT::BYTES)[tid] = stat;
        wait_global_loads();
        __syncthreads();
    }

    // this lane: key krow, columns 32db + 8rg + 4g + e
    if (krow < a.Tk) {
        E* dkh = static_cast<E*>(a.dk) + kvoff + (size_t)krow * D;
        E* dvh = static_cast<E*>(a.dv) + kvoff + (size_t)krow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int col = db * 32 + 8 * rg + 4 * g;
                if constexpr (sizeof(E) == 2) {
                    bf16x4 x, y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] = (bf16)(dk[db][4 * rg + e] * a.scale);
                        y[e] = (bf16)dv[db][4 * rg + e];
                    }
                    *reinterpret_cast<bf16x4*>(dkh + col) = x;
                    *reinterpret_cast<bf16x4*>(dvh + col) = y;
                } else {
                    f32x4 x, y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] = dk[db][4 * rg + e] * a.scale;
                        y[e] = dv[db][4 * rg + e];
                    }
                    *reinterpret_cast<f32x4*>(dkh + col) = x;
                    *reinterpret_cast<f32x4*>(dvh + col) = y;
                }
            }
    }
}

// ---------------------------------------------------------------------------
// dQ.  One workgroup per (batch, query head, query tile of NW*32 rows); wave w
// owns 32 queries, keeps Q and dO of them in registers and walks key tiles in
// the forward's order.  S^T = K Q^T and dP^T = V dO^T are formed with keys as
// rows, so dS^T feeds dQ^T += K^T dS^T from registers; the K^T operand is read
// transposed from the natural K tile.
// ---------------------------------------------------------------------------
template <class E, int D, int NW, int BC>
struct DqCfg {
    static constexpr int NT = NW * 64;
    static constexpr int BR = NW * 32;
    using Tile = DmaTile<E, D, BC, NT>;
    static constexpr int BUF = 2 * Tile::BYTES;
    static constexpr size_t SMEM = 2 * (size_t)BUF;
};

template <class E, int D, int NW, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, sizeof(E) == 2 ? 8 / NW : 1) void bwd_dq_kernel(BwdArgs a)
{
    using Cfg = DqCfg<E, D, NW, BC>;
    using Tile = typename Cfg::Tile;
    constexpr int BR = Cfg::BR;
    constexpr int NKB = BC / 32;
    constexpr int NDB = D / 32;
    constexpr int NKS = D / 16;

    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int c = lane & 31;

    const int nqt = (a.Tq + BR - 1) / BR;
    const TileId id = map_tile(blockIdx.x, a.B, a.Hq, a.Hkv, a.Hq / a.Hkv, nqt, CAUSAL);
    const int b = id.b, hq = id.h;
    const int hk = hq / (a.Hq / a.Hkv);
    const int q0 = id.tile * BR;
    const int qrow = q0 + w * 32 + c;

    const size_t qoff = (size_t)(b * a.Hq + hq) * a.Tq * D;
    const size_t kvoff = (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const E* kh = static_cast<const E*>(a.k) + kvoff;
    const E* vh = static_cast<const E*>(a.v) + kvoff;

    // key tiles visited (query row i sees keys j <= i + off when causal)
    const int kend = CAUSAL ? min(q0 + BR + a.off, a.Tk) : a.Tk;
    const int nkv = (kend + BC - 1) / BC;
    const int nfull = CAUSAL ? min((q0 + a.off + 1) / BC, a.Tk / BC) : a.Tk / BC;

    Tile dma;
    dma.init(tid);
    dma.load(smem, kh, 0, a.Tk, w);
    dma.load(smem + Tile::BYTES, vh, 0, a.Tk, w);

    RowReader<Tile, E, D> rrd;  // K and V rows (A of S^T, dP^T)
    rrd.init(c, g);
    TrReader<Tile, E, D> trd;   // K^T (A of dQ^T)
    trd.init(lane);

    Frag<E> qf[NKS], of[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        qf[ks] = global_frag<E>(static_cast<const E*>(a.q) + qoff, qrow, a.Tq, D, 16 * ks + 8 * g);
        of[ks] = global_frag<E>(static_cast<const E*>(a.dout) + qoff, qrow, a.Tq, D, 16 * ks + 8 * g);
    }
    float L2 = 0.f, Dl = 0.f;
    if (qrow < a.Tq) {
        const size_t r = (size_t)(b * a.Hq + hq) * a.Tq + qrow;
        L2 = a.lse[r] * kLog2e;
        Dl = a.delta[r];
    }

    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};

    wait_global_loads();
    __syncthreads();

    auto step = [&](auto bufi, int j) {
        constexpr int BI = decltype(bufi)::value;
        const unsigned char* Ks = smem + BI * Cfg::BUF;
        const unsigned char* Vs = Ks + Tile::BYTES;
        if (j + 1 < nkv) {
            unsigned char* nb = smem + (1 - BI) * Cfg::BUF;
            dma.load(nb, kh, (j + 1) * BC, a.Tk, w);
            dma.load(nb + Tile::BYTES, vh, (j + 1) * BC, a.Tk, w);
        }
        const bool need_mask = j >= nfull;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) mma(s, rrd.frag(Ks, kb * 32, ks), qf[ks]);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) mma(dp, rrd.frag(Vs, kb * 32, ks), of[ks]);
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], a.c, -L2));  // P^T
            if (need_mask) {
                // a real branch (the empty asm keeps the compiler from turning
                // it into selects executed on every tile)
                asm volatile("");
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kj = j * BC + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    const bool vis = kj < a.Tk && (!CAUSAL || kj <= qrow + a.off);
                    s[r] = vis ? s[r] : 0.f;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[r] = s[r] * (dp[r] - Dl);  // dS^T
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const Frag<E> sf = acc_frag<E>(dp, t);
#pragma unroll
                for (int db = 0; db < NDB; ++db) mma(dq[db], trd.frag(Ks, kb * 32 + 16 * t, db), sf);
            }
        }

        wait_global_loads();
        __syncthreads();
    };

    for (int j = 0; j < nkv; j += 2) {
        step(std::integral_constant<int, 0>{}, j);
        if (j + 1 < nkv) step(std::integral_constant<int, 1>{}, j + 1);
    }

    if (qrow < a.Tq) {
        E* dqh = static_cast<E*>(a.dq) + qoff + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int col = db * 32 + 8 * rg + 4 * g;
                if constexpr (sizeof(E) == 2) {
                    bf16x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (bf16)(dq[db][4 * rg + e] * a.scale);
                    *reinterpret_cast<bf16x4*>(dqh + col) = x;
                } else {
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = dq[db][4 * rg + e] * a.scale;
                    *reinterpret_cast<f32x4*>(dqh + col) = x;
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <class E, int D, class EO = E>
static hipError_t launch_pre_t(const PreArgs& a, hipStream_t stream)
{
    constexpr int LPR = pre_lanes<E, D>();
    constexpr int RPB = 256 / LPR;
    const long grid = (a.rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((bwd_pre_kernel<E, D, EO>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// dtype 0: bf16 O and dO; 1: float32 O and dO; 2: float32 O, bf16 dO
hipError_t launch_bwd_pre(const PreArgs& a, int D, int dtype, hipStream_t stream)
{
    if (dtype == 2) {
        if (D == 96) return launch_pre_t<bf16, 96, float>(a, stream);
        return D == 64 ? launch_pre_t<bf16, 64, float>(a, stream) : launch_pre_t<bf16, 128, float>(a, stream);
    }
    if (dtype == 0) {
        if (D == 96) return launch_pre_t<bf16, 96>(a, stream);
        return D == 64 ? launch_pre_t<bf16, 64>(a, stream) : launch_pre_t<bf16, 128>(a, stream);
    }
    return D == 64 ? launch_pre_t<float, 64>(a, stream) : launch_pre_t<float, 128>(a, stream);
}

// Tile shapes of the backward: dK/dV workgroups own NW*32 keys and stream BQ
// query rows per step; dQ workgroups own NW*32 queries and stream BC keys.
constexpr int kDkdvNW = 4, kDkdvBQ = 32;
constexpr int kDqNW = 4, kDqBC = 64;

template <class E, int D, bool CAUSAL>
static hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t stream)
{
    constexpr int NW = kDkdvNW, BQ = kDkdvBQ;
    using Cfg = DkdvCfg<E, D, NW, BQ>;
    static_assert(Cfg::SMEM <= 160 * 1024, "LDS budget");
    auto kern = bwd_dkdv_kernel<E, D, NW, BQ, CAUSAL>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::SMEM);
    if (attr != hipSuccess) return attr;
    const int nkt = (a.Tk + Cfg::BK - 1) / Cfg::BK;
    const long grid = (long)nkt * a.B * a.Hkv;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::SMEM, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int D, int dtype, bool causal, hipStream_t stream)
{
    if (dtype == 0) return launch_bwd_dkdv_bf16(a, D, causal, stream);
    if (D == 64) return causal ? launch_dkdv_t<float, 64, true>(a, stream) : launch_dkdv_t<float, 64, false>(a, stream);
    return causal ? launch_dkdv_t<float, 128, true>(a, stream) : launch_dkdv_t<float, 128, false>(a, stream);
}

template <class E, int D, bool CAUSAL>
static hipError_t launch_dq_t(const BwdArgs& a, hipStream_t stream)
{
    constexpr int NW = kDqNW, BC = kDqBC;
    using Cfg = DqCfg<E, D, NW, BC>;
    static_assert(Cfg::SMEM <= 160 * 1024, "LDS budget");
    auto kern = bwd_dq_kernel<E, D, NW, BC, CAUSAL>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::SMEM);
    if (attr != hipSuccess) return attr;
    const int nqt = (a.Tq + Cfg::BR - 1) / Cfg::BR;
    const long grid = (long)nqt * a.B * a.Hq;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::SMEM, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int D, int dtype, bool causal, hipStream_t stream)
{
    if (dtype == 0) return launch_bwd_dq_bf16(a, D, causal, stream);
    if (D == 64) return causal ? launch_dq_t<float, 64, true>(a, stream) : launch_dq_t<float, 64, false>(a, stream);
    return causal ? launch_dq_t<float, 128, true>(a, stream) : launch_dq_t<float, 128, false>(a, stream);
}

// Every kernel variant is instantiated explicitly: referencing a kernel
// template only from a launcher has left some instantiations without their
// host-side handle.
template __global__ void bwd_pre_kernel<bf16, 64>(PreArgs);
template __global__ void bwd_pre_kernel<bf16, 96>(PreArgs);
template __global__ void bwd_pre_kernel<bf16, 128>(PreArgs);
template __global__ void bwd_pre_kernel<float, 64>(PreArgs);
template __global__ void bwd_pre_kernel<float, 128>(PreArgs);
template __global__ void bwd_pre_kernel<bf16, 64, float>(PreArgs);
template __global__ void bwd_pre_kernel<bf16, 96, float>(PreArgs);
template __global__ void bwd_pre_kernel<bf16, 128, float>(PreArgs);
template __global__ void bwd_dq_kernel<float, 64, kDqNW, kDqBC, true>(BwdArgs);
template __global__ void bwd_dq_kernel<float, 64, kDqNW, kDqBC, false>(BwdArgs);
template __global__ void bwd_dq_kernel<float, 128, kDqNW, kDqBC, true>(BwdArgs);
template __global__ void bwd_dq_kernel<float, 128, kDqNW, kDqBC, false>(BwdArgs);
template __global__ void bwd_dkdv_kernel<float, 64, kDkdvNW, kDkdvBQ, true>(BwdArgs);
template __global__ void bwd_dkdv_kernel<float, 64, kDkdvNW, kDkdvBQ, false>(BwdArgs);
template __global__ void bwd_dkdv_kernel<float, 128, kDkdvNW, kDkdvBQ, true>(BwdArgs);
template __global__ void bwd_dkdv_kernel<float, 128, kDkdvNW, kDkdvBQ, false>(BwdArgs);

}  // namespace fa
