// bf16 backward kernels ("L'attention fusionnée", «La passe arrière»).
//
// P is rebuilt tile by tile from the scores and the saved row log-sum-exp,
// P = exp2(S * scale*log2(e) - L*log2(e)), and the softmax Jacobian term of a
// query row is the precomputed Delta_i = sum_d dO_id O_id:
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - Delta),   dK = dS^T Q * scale.
//
// dK/dV kernel.  One workgroup of four waves per (batch, kv head, block of
// 128 keys), one wave per SIMD; wave w owns 32 keys.  K and V of those keys
// stay in registers (B operands of S = Q K^T and dP = dO V^T); the dK^T and
// dV^T accumulators (the MFMA accumulators of dK^T += Q^T dS, dV^T += dO^T P)
// never leave the matrix-core register file.  Query tiles of 32 rows, of every
// query head of the kv group, stream through LDS; the group sum of dK and dV
// therefore stays inside the workgroup and no atomics are needed (the result
// is bitwise reproducible).
//
// Software pipeline.  Per query tile t a wave runs
//     A(t): S = Q_t K^T, dP = dO_t V^T          (16 MFMAs, row reads of Q_t, dO_t)
//     B(t): P, mask, dS, bf16 operands          (vector ALU)
//     C(t): dV^T += dO_t^T P, dK^T += Q_t^T dS  (16 MFMAs, transposed reads)
// and iteration i issues C(i-1) and A(i+1) on the matrix core interleaved
// with the vector work of B(i), all three independent, so one wave per SIMD
// keeps both units busy.  Tiles arrive by LDS DMA four iterations ahead into
// six stage buffers; the loop is unrolled over the stages so every LDS offset
// is an immediate.  Causal masking uses, per accumulator register, a
// workgroup-uniform lane mask: with 32-row query tiles and 32-key waves a tile
// is wholly visible, wholly invisible or exactly the lower triangle.
#include <type_traits>
#include <utility>

#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_pipe.hpp"

namespace fa {

template <int D>
struct DkdvBf16Cfg {
    static constexpr int NW = 4;
    static constexpr int NT = 64 * NW;
    static constexpr int BK = 32 * NW;  // keys per workgroup
    static constexpr int BQ = 32;       // query rows per tile
    static constexpr int NSTAGE = 6;    // LDS stage buffers (even: register sets alternate)
    static constexpr int AHEAD = 4;     // tiles in flight ahead of the one entering B
    using QT = SwzTile<D, BQ, NT>;      // Q and dO tiles
    using Fmt = DmaTile<bf16, D, BQ, NT>;
    static constexpr int STATS = 512;   // L*log2(e) (64 floats) and Delta (64 floats)
    static constexpr int STAGE = 2 * QT::BYTES + STATS;
    static constexpr int SMEM = NSTAGE * STAGE;
    static_assert(AHEAD + 2 <= NSTAGE, "stages in use: t-1, t, t+1 and AHEAD - 1 in flight");
};

// Lane mask of accumulator register r (rows = queries 8(r/4) + 4g + r%4,
// columns = keys c) for a query tile that starts at the wave's first key:
// query row >= key.
__host__ __device__ constexpr uint64_t tri_mask(int r)
{
    const int q0 = 8 * (r / 4) + r % 4;  // row of lane group g = 0
    const int q1 = q0 + 4;               // row of lane group g = 1
    const uint64_t lo = (q0 + 1 >= 32) ? 0xffffffffull : ((1ull << (q0 + 1)) - 1);
    const uint64_t hi = (q1 + 1 >= 32) ? 0xffffffffull : ((1ull << (q1 + 1)) - 1);
    return lo | (hi << 32);
}

// f(stage, i + K) for K = 0 .. N-1, with the stage as a compile-time constant
template <class F, int... K>
__device__ __forceinline__ void unroll_stages(F& f, int i, std::integer_sequence<int, K...>)
{
    (f(std::integral_constant<int, K>{}, i + K), ...);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void dkdv_bf16_kernel(BwdArgs a)
{
    using Cfg = DkdvBf16Cfg<D>;
    using QT = typename Cfg::QT;
    using Fmt = typename Cfg::Fmt;
    constexpr int BK = Cfg::BK, BQ = Cfg::BQ, NSTAGE = Cfg::NSTAGE, STAGE = Cfg::STAGE;
    constexpr int AHEAD = Cfg::AHEAD;
    constexpr int NDB = D / 32;
    constexpr int NKS = D / 16;

    extern __shared__ __align__(1024) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int c = lane & 31;
    const int G = a.Hq / a.Hkv;

    const int nkt = (a.T + BK - 1) / BK;
    // causal: the first key tiles see the most query rows
    const TileId id = map_tile(blockIdx.x, a.B, a.Hq, a.Hkv, 1, nkt, false);
    const int b = id.b, hk = id.h;
    const int key0 = id.tile * BK;
    const int kw = key0 + 32 * w;  // first key of this wave
    const int krow = kw + c;       // the key this lane owns

    const size_t kvoff = (size_t)(b * a.Hkv + hk) * a.T * D;
    const bf16* kh = static_cast<const bf16*>(a.k) + kvoff;
    const bf16* vh = static_cast<const bf16*>(a.v) + kvoff;

    // flattened sequence of (query head, query tile) seeing this key block
    const int nq = (a.T + BQ - 1) / BQ;
    const int i0 = CAUSAL ? key0 / BQ : 0;
    const int niq = nq - i0;
    const int n = G * niq;
    const int npad = (n + NSTAGE - 1) / NSTAGE * NSTAGE;  // padded tiles: all masked

    QT qt;
    qt.init(tid);
    const uint32_t lds0 = lds_addr(smem);
    // DMA instructions per tile of this wave: Q and dO, plus L (wave 0) or
    // Delta (wave 1)
    const int vpt = 2 * QT::NI + (w < 2 ? 1 : 0);
    // DMA cursor: (query head, query tile) of the next tile to issue; the
    // flattened order runs over the query tiles i0 .. nq-1 of each head
    int dhq = hk * G, dti = i0;
    auto issue = [&](int st) {
        const size_t qoff = (size_t)(b * a.Hq + dhq) * a.T * D;
        const uint32_t base = lds0 + (uint32_t)(st * STAGE);
        qt.load(base, static_cast<const bf16*>(a.q) + qoff, dti * BQ, a.T, w);
        qt.load(base + QT::BYTES, static_cast<const bf16*>(a.dout) + qoff, dti * BQ, a.T, w);
        if (w < 2) {
            const float* src = (w == 0 ? a.lse : a.delta) + (size_t)(b * a.Hq + dhq) * a.T + dti * BQ;
            const i32x4 r = buffer_rsrc(src, (a.T - dti * BQ) * 4);
            dma_b32(base + 2 * QT::BYTES + 256 * w, r, (uint32_t)(lane * 4));
        }
        if (++dti == nq) {
            dti = i0;
            ++dhq;
        }
    };
    // wait until tile t has landed, given that tiles t+1 .. t+2 may be in flight
    auto wait_tile = [&](int t) {
        const int after = (t + 1 < n) + (t + 2 < n);  // tiles issued after t
        if (vpt == 2 * QT::NI + 1) {
            if (after == 2) vm_wait<2 * (2 * QT::NI + 1)>();
            else if (after == 1) vm_wait<2 * QT::NI + 1>();
            else vm_wait<0>();
        } else {
            if (after == 2) vm_wait<2 * (2 * QT::NI)>();
            else if (after == 1) vm_wait<2 * QT::NI>();
            else vm_wait<0>();
        }
    };

    // Zero every stage first: the first C step and the padded tiles at the end
    // compute on stages no tile has filled, with all-zero (masked) weights, and
    // 0 * (uninitialised LDS) could be NaN.
    for (int off = tid * 16; off < Cfg::SMEM; off += Cfg::NT * 16)
        *reinterpret_cast<u32x4*>(smem + off) = u32x4{0, 0, 0, 0};
    sync_lds();
    for (int t = 0; t < AHEAD && t < n; ++t) issue(t);  // stage t

    // B operands of S = Q K^T and dP = dO V^T: this lane's key row, 8 columns
    // per 16-deep step
    Frag<bf16> kf[NKS], vf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        kf[ks] = global_frag<bf16>(kh, krow, a.T, D, 16 * ks + 8 * g);
        vf[ks] = global_frag<bf16>(vh, krow, a.T, D, 16 * ks + 8 * g);
    }

    RowReader<Fmt, bf16, D> qrd;  // Q and dO rows (A of S, dP)
    qrd.init(c, g);
    TrReader<Fmt, bf16, D> trd;   // Q^T and dO^T (A of dK^T, dV^T)
    trd.init(lane);

    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = f32x16{};
    f32x16 S[2], DP[2];        // scores and dP of tiles of parity 0 / 1
    // bf16 P and dS of tiles of parity 0 / 1, as B operands of C: 16-deep
    // step t, packed pairs of elements 2e, 2e + 1
    uint32_t PW[2][2][4], SW[2][2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) PW[1][t][e] = SW[1][t][e] = 0u;
    auto frag_of = [](const uint32_t (&wv)[4]) {
        Frag<bf16> f;
        f.v = __builtin_bit_cast(bf16x8, u32x4{wv[0], wv[1], wv[2], wv[3]});
        return f;
    };

    // L of tile t (natural log) -> L * log2(e), in place, by wave 0
    auto convert_l = [&](int t) {
        if (w == 0 && lane < BQ) {
            float* Ls = reinterpret_cast<float*>(smem + (t % NSTAGE) * STAGE + 2 * QT::BYTES);
            Ls[lane] *= kLog2e;
        }
    };

    wait_tile(1 < n ? 1 : 0);  // tiles 0 and 1
    sync_lds();
    convert_l(0);
    sync_lds();

    int bti = i0;  // query tile of the tile entering B
    auto tile_q = [&](int st) { return smem + st * STAGE; };
    auto tile_do = [&](int st) { return smem + st * STAGE + QT::BYTES; };

    // A(t): S = Q_t K^T and dP = dO_t V^T into register set P1
    auto step_a = [&](auto st_tag, auto par_tag) {
        constexpr int ST = decltype(st_tag)::value, P1 = decltype(par_tag)::value;
        S[P1] = f32x16{};
        DP[P1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            mma(S[P1], qrd.frag(tile_q(ST), 0, ks), kf[ks]);
            mma(DP[P1], qrd.frag(tile_do(ST), 0, ks), vf[ks]);
        }
    };
    // C(t): dV^T += dO_t^T P, dK^T += Q_t^T dS from register set P0
    auto step_c = [&](auto st_tag, auto par_tag) {
        constexpr int ST = decltype(st_tag)::value, P0 = decltype(par_tag)::value;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                mma(dv[db], trd.frag(tile_do(ST), 16 * t, db), frag_of(PW[P0][t]));
                mma(dk[db], trd.frag(tile_q(ST), 16 * t, db), frag_of(SW[P0][t]));
            }
    };

    // one iteration: tile i enters B; stage ST = i % NSTAGE (compile time)
    auto body = [&](auto st_tag, int i) {
        constexpr int ST = decltype(st_tag)::value;
        constexpr int PB = ST & 1, PO = PB ^ 1;
        constexpr int SPREV = (ST + NSTAGE - 1) % NSTAGE, SNEXT = (ST + 1) % NSTAGE;
        if (i + AHEAD < n) issue((ST + AHEAD) % NSTAGE);
        convert_l(i + 1);

        // Tiles wholly visible to this wave take no mask code.  The others
        // (causal: the diagonal tile, query rows 0..31 against keys 0..31 of
        // the wave, and tiles wholly in the past of the wave's keys; the
        // padding past the last tile) set the invisible scores to -inf in a
        // branch, so that P = 0 there.
        const bool pad = i >= n;
        const int qb = bti * BQ;  // first query row of tile i
        if (pad || (CAUSAL && qb <= kw)) {
            asm volatile("");  // keep this a branch
            const bool tri = !pad && qb == kw;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint64_t m = tri ? tri_mask(r) : 0ull;
                S[PB][r] = __builtin_amdgcn_inverse_ballot_w64(m) ? S[PB][r] : -INFINITY;
            }
        }
        if (++bti == nq) bti = i0;

        // L*log2(e) and Delta of this lane's 16 rows of tile i
        const float* Ls = reinterpret_cast<const float*>(smem + ST * STAGE + 2 * QT::BYTES);
        const float* Ds = Ls + 64;
        f32x4 L4[4], D4[4];
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            L4[rg] = *reinterpret_cast<const f32x4*>(Ls + 8 * rg + 4 * g);
            D4[rg] = *reinterpret_cast<const f32x4*>(Ds + 8 * rg + 4 * g);
        }

        // Matrix products of this iteration, in slot order k = 0 .. N-1:
        //   k < NC : C(i-1), (t, db, which) -> dV^T (which 0) or dK^T (which 1)
        //   k >= NC: A(i+1), (ks, which)    -> S (which 0) or dP (which 1)
        constexpr int NC = 2 * 2 * NDB, NA = 2 * NKS, N = NC + NA;
        constexpr int NCHUNK = 32, CPS = (NCHUNK + N - 1) / N;  // B chunks per slot
        constexpr int AHD = 4;                                   // reads run AHD products ahead
        auto frag_for = [&](int k) -> Frag<bf16> {
            if (k < NC) {
                const int which = k & 1, db = (k >> 1) % NDB, t = (k >> 1) / NDB;
                return trd.frag(which ? tile_q(SPREV) : tile_do(SPREV), 16 * t, db);
            }
            const int kk = k - NC, which = kk & 1, ks = kk >> 1;
            return qrd.frag(which ? tile_do(SNEXT) : tile_q(SNEXT), 0, ks);
        };
        auto mfma_at = [&](int k, const Frag<bf16>& f) {
            if (k < NC) {
                const int which = k & 1, db = (k >> 1) % NDB, t = (k >> 1) / NDB;
                if (which)
                    mma(dk[db], f, frag_of(SW[PO][t]));
                else
                    mma(dv[db], f, frag_of(PW[PO][t]));
            } else {
                const int kk = k - NC, which = kk & 1, ks = kk >> 1;
                if (which)
                    mma(DP[PO], f, vf[ks]);
                else
                    mma(S[PO], f, kf[ks]);
            }
        };
        // B(i) in 32 chunks, each pinned to its slot by passing its inputs
        // and outputs through empty asm statements (ordered among themselves
        // and with the slot barriers): even chunk 2r forms P of register r, odd chunk 2r + 1 its dS and, for odd r, rounds the pair
        // (r - 1, r) of P and dS into the bf16 operands of C(i).
        float pv[16], dsv[16];
        auto b_chunk = [&](int j) {
            const int r = j >> 1;
            if (!(j & 1)) {
                float x = S[PB][r];
                pin(x);
                pv[r] = fast_exp2(fmaf(x, a.c, -L4[r >> 2][r & 3]));
                pin(pv[r]);
            } else {
                float y = DP[PB][r];
                pin(y);
                dsv[r] = pv[r] * (y - D4[r >> 2][r & 3]);
                pin(dsv[r]);
                if (r & 1) {
                    const int t = (r - 1) >> 3, e = (r - 1) & 7;
                    uint32_t pp = pack_bf16(pv[r - 1], pv[r]);
                    uint32_t ss = pack_bf16(dsv[r - 1], dsv[r]);
                    pin(pp);
                    pin(ss);
                    PW[PB][t][e >> 1] = pp;
                    SW[PB][t][e >> 1] = ss;
                }
            }
        };

        S[PO] = f32x16{};
        DP[PO] = f32x16{};
        Frag<bf16> ring[AHD + 1];
#pragma unroll
        for (int k = 0; k < AHD; ++k) ring[k] = frag_for(k);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < N; ++k) {
#pragma unroll
            for (int j = k * CPS; j < (k + 1) * CPS && j < NCHUNK; ++j) b_chunk(j);
            if (k + AHD < N) ring[(k + AHD) % (AHD + 1)] = frag_for(k + AHD);
            mfma_at(k, ring[k % (AHD + 1)]);
            __builtin_amdgcn_sched_barrier(0);
        }

        wait_tile(i + 2);
        sync_lds();
    };

    step_a(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    for (int i = 0; i < npad; i += NSTAGE)
        unroll_stages(body, i, std::make_integer_sequence<int, NSTAGE>{});
    step_c(std::integral_constant<int, NSTAGE - 1>{}, std::integral_constant<int, 1>{});

    // this lane: key krow, columns 32db + 8rg + 4g + e
    if (krow < a.T) {
        bf16* dkh = static_cast<bf16*>(a.dk) + kvoff + (size_t)krow * D;
        bf16* dvh = static_cast<bf16*>(a.dv) + kvoff + (size_t)krow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int col = db * 32 + 8 * rg + 4 * g;
                bf16x4 x, y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = (bf16)(dk[db][4 * rg + e] * a.scale);
                    y[e] = (bf16)dv[db][4 * rg + e];
                }
                *reinterpret_cast<bf16x4*>(dkh + col) = x;
                *reinterpret_cast<bf16x4*>(dvh + col) = y;
            }
    }
}

template <int D, bool CAUSAL>
static hipError_t launch_dkdv(const BwdArgs& a, hipStream_t stream)
{
    using Cfg = DkdvBf16Cfg<D>;
    static_assert(Cfg::SMEM <= 160 * 1024, "LDS budget");
    auto kern = dkdv_bf16_kernel<D, CAUSAL>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::SMEM);
    if (attr != hipSuccess) return attr;
    const int nkt = (a.T + Cfg::BK - 1) / Cfg::BK;
    const long grid = (long)nkt * a.B * a.Hkv;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::SMEM, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, int D, bool causal, hipStream_t stream)
{
    if (D == 64) return causal ? launch_dkdv<64, true>(a, stream) : launch_dkdv<64, false>(a, stream);
    return causal ? launch_dkdv<128, true>(a, stream) : launch_dkdv<128, false>(a, stream);
}

// Every kernel variant is instantiated explicitly: referencing a kernel
// template only from a launcher has left some instantiations without their
// host-side handle.
template __global__ void dkdv_bf16_kernel<64, true>(BwdArgs);
template __global__ void dkdv_bf16_kernel<64, false>(BwdArgs);
template __global__ void dkdv_bf16_kernel<128, true>(BwdArgs);
template __global__ void dkdv_bf16_kernel<128, false>(BwdArgs);

}  // namespace fa
