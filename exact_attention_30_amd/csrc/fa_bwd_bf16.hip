// bf16 backward kernels ("L'attention fusionnée", «La passe arrière»).
//
// P is rebuilt tile by tile from the scores and the saved row log-sum-exp,
// P = exp2(S * scale*log2(e) - L*log2(e)), and the softmax Jacobian term of a
// query row is the precomputed Delta_i = sum_d dO_id O_id:
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - Delta),   dK = dS^T Q * scale.
//
// dK/dV kernel.  One workgroup of eight waves per (batch, kv head, block of
// 256 keys): two waves per SIMD, so the matrix work of one overlaps the
// vector work of the other.  Wave w owns 32 keys: K of those keys stays in
// registers (B operand of S = Q K^T) and the dK^T, dV^T accumulators never
// leave the register file; V of the wave's keys is loaded once into LDS in
// read order (B operand of dP = dO V^T), which keeps a wave within its 256
// registers.
// Query tiles of 32 rows, of every query head of the kv group, stream through
// LDS, shared by the eight waves; the group sum of dK and dV therefore stays
// inside the workgroup and no atomics are needed (the result is bitwise
// reproducible).  Per query tile a wave runs
//     S = Q_t K^T                    (8 MFMAs, row reads of Q_t), then the mask
//     dP = dO_t V^T  beside  P        (8 MFMAs, row reads of dO_t and V)
//     dV^T += dO_t^T P  beside  dS    (8 MFMAs, transposed reads)
//     dK^T += Q_t^T dS                (8 MFMAs, transposed reads)
// (MFMA counts for head size 128), the vector work of P and dS placed
// between the products that do not depend on it.
// The tiles arrive by explicitly scheduled LDS DMA in four stage buffers at
// the bottom of LDS, computed in pairs with one barrier per pair (each tile
// loads the tile two ahead into a stage of the previous pair, its Q between
// the score products); the loop is unrolled over the
// stages and the per-lane read addresses carry the LDS base, so every read is
// one address register plus an immediate offset, with no address arithmetic
// in the loop.
// Tiles wholly visible to a wave carry no mask code; the few that straddle the
// diagonal j = i + off of the causal mask take a per-element mask in a rarely
// taken branch, and a wave skips the products of the tiles none of its keys
// sees (and of the padding tiles that round the loop up to whole stages).
#include <type_traits>
#include <utility>

#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_pipe.hpp"

namespace fa {

// ADQ: the variant that also accumulates dQ with atomic adds (below)
template <int D, int NWV, bool ADQ = false>  // head size in memory; waves per workgroup
struct DkdvBf16Cfg {
    static constexpr int DT = tile_dim(D);  // head size of the tiles and products
    static constexpr int NW = NWV;          // 8: two per SIMD; 4: one, several workgroups per CU
    static constexpr int NT = 64 * NW;
    static constexpr int BK = 32 * NW;  // keys per workgroup
    static constexpr int BQ = 32;       // query rows per tile
    // LDS stage buffers: tiles are computed in pairs with one barrier per
    // pair, and the next pair's two tiles load into the previous pair's
    // stages (each while the tile two before it is computed)
    static constexpr int NSTAGE = 4;
    // Q and dO tiles: 32 rows; D = 64 needs only four waves to move them
    static constexpr int QNT = (BQ * DT / 8 >= NT) ? NT : BQ * DT / 8;
    using QT = SwzTile<DT, BQ, QNT, D>;
    using Fmt = DmaTile<bf16, DT, BQ, QNT>;
    using VW = RowFragTile<DT, 32, D>;  // V rows of one wave, in read order
    static constexpr int STATS = 512;  // L*log2(e) (64 floats) and Delta (64 floats)
    static constexpr int STAGE = 2 * QT::BYTES + STATS;
    // ADQ: per wave a 32 x 32 bf16 tile of dS (row query, column key) and a
    // 32 x D fp32 tile of its part of dQ
    static constexpr int DSW = 32 * 32 * 2;
    static constexpr int RED = 32 * D * 4;
    static constexpr int SMEM = NSTAGE * STAGE + NW * VW::BYTES + (ADQ ? NW * (DSW + RED) : 0);
    // every read offset of a stage fits the 16-bit immediate of a DS read
    static_assert((NSTAGE - 1) * STAGE + QT::BYTES + 16 * Fmt::ROWBYTES < 65536, "LDS immediates");
    static_assert(NSTAGE == 4, "two pairs of stages");
    static_assert(QT::NI == 1, "one Q and one dO instruction per loading wave");
    // a workgroup may take a pair of key blocks (kpair)
    static constexpr bool PAIRABLE = D != 64;
};

// f(stage, i + K) for K = 0 .. N-1, with the stage as a compile-time constant
template <class F, int... K>
__device__ __forceinline__ void unroll_stages(F& f, int i, std::integer_sequence<int, K...>)
{
    (f(std::integral_constant<int, K>{}, i + K), ...);
}

template <int D, bool CAUSAL, int NWV, bool ADQ = false>
__global__ __launch_bounds__(64 * NWV, 8 / NWV) void dkdv_bf16_kernel(BwdArgs a)
{
    using Cfg = DkdvBf16Cfg<D, NWV, ADQ>;
    static_assert(!ADQ || (D == 64 && NWV == 8 && Cfg::NT * 4 == 32 * D),
                  "the atomic dQ variant: D = 64, eight waves, four dQ elements per thread");
    using QT = typename Cfg::QT;
    using Fmt = typename Cfg::Fmt;
    using VW = typename Cfg::VW;
    constexpr int BK = Cfg::BK, BQ = Cfg::BQ, NSTAGE = Cfg::NSTAGE, STAGE = Cfg::STAGE;
    // Products run over the D columns of the tensors; the LDS tiles are
    // Cfg::DT wide (D = 96: 128, the last 32 columns zeros that no product reads)
    constexpr int NDB = D / 32;  // 32-column blocks
    constexpr int NKS = D / 16;  // 16-deep steps over the head dimension
    constexpr int QW = Cfg::QNT / 64;  // waves that move Q and dO tiles

    extern __shared__ __align__(1024) unsigned char smem[];
    unsigned char* stages = smem;
    unsigned char* Vs = smem + NSTAGE * STAGE;  // V rows of wave w at Vs + w * VW::BYTES
    // ADQ: this wave's dS tile, and the waves' dQ parts [w][32][D]
    [[maybe_unused]] unsigned char* dsw = Vs + Cfg::NW * VW::BYTES + (ADQ ? (threadIdx.x >> 6) * Cfg::DSW : 0);
    [[maybe_unused]] float* red = reinterpret_cast<float*>(Vs + Cfg::NW * VW::BYTES + (ADQ ? Cfg::NW * Cfg::DSW : 0));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int c = lane & 31;
    const int G = a.Hq / a.Hkv;

    const int nkt = (a.Tk + BK - 1) / BK;
    // causal: the first key blocks see the most query rows; the nsplit chunks
    // of one key block are neighbours (and share an XCD where possible)
    const int S = a.nsplit;
    // Key-block pairs are compiled only where they pay: at D = 64 the loop
    // over two blocks costs registers (occupancy 3 -> 2) and measured 1.7-1.9 %
    // slower at C2 and C3, which do not use it.
    constexpr bool PAIRABLE = DkdvBf16Cfg<D, NWV, ADQ>::PAIRABLE;
    // kpair: workgroup m takes key blocks m and nkt - 1 - m (one block for
    // the middle one when nkt is odd), which together see the same number of
    // query tiles whatever m is
    const TileId id = map_tile(blockIdx.x, a.B, a.Hq, a.Hkv, S, PAIRABLE && a.kpair ? (nkt + 1) / 2 : nkt, false);
    const int b = id.b, hk = id.h / S, split = id.h % S;
    const int npass = PAIRABLE && a.kpair && nkt - 1 - id.tile != id.tile ? 2 : 1;
    // With kpair a key block in the upper half of the 256-key blocks walks
    // its query tiles upward, the others downward.  The workgroups of a kv
    // head then read the same Q and dO tile at the same time: all start
    // their first block at the last tile, and each starts its second one at
    // the tile where those that switched before it have arrived.  The rule
    // depends on the keys alone, so 128- and 256-key blocks add the same
    // terms in the same order.
    const int nkt256 = (a.Tk + 255) / 256;
    // the work of one key block (first key key0), its query tiles walked
    // down (dir < 0) or up
    auto run_block = [&](const int key0, const int dir) __attribute__((always_inline)) {
    // first key of this wave.  With eight waves, w and w + 4 share a SIMD;
    // pairing key blocks r and 7 - r there gives every SIMD the same number
    // of causal tiles that one of its waves skips (below).  With four, each
    // wave has a SIMD of the workgroup to itself.
    const int kw = Cfg::NW == 4 ? key0 + 32 * w : key0 + 32 * (w < 4 ? w : 11 - w);
    const int krow = kw + c;       // the key this lane owns

    const size_t kvoff = (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const bf16* kh = static_cast<const bf16*>(a.k) + kvoff;
    const bf16* vh = static_cast<const bf16*>(a.v) + kvoff;

    // the (query head, query tile) pairs that see this key block (query row i
    // sees keys j <= i + off when causal), in visiting order; this workgroup
    // takes the contiguous chunk [p0, p0 + n) of them
    const int nq = (a.Tq + BQ - 1) / BQ;
    const int i0 = CAUSAL ? max(key0 - a.off, 0) / BQ : 0;
    const int niq = max(nq - i0, 0);
    const long npair = (long)G * niq;
    const int p0 = (int)(npair * split / S);
    const int n = (int)(npair * (split + 1) / S) - p0;
    const int npad = (n + NSTAGE - 1) / NSTAGE * NSTAGE;  // padded tiles: skipped

    const uint32_t lds0 = lds_addr(stages);
    QT qt;
    if (w < QW) qt.init(tid);
    // DMA instructions per tile of this wave: Q and dO, and L (wave 0) or
    // Delta (wave 1)
    const int vpt = (w < QW ? 2 : 0) + (w < 2 ? 1 : 0);
    // Tiles are visited from the last query tile down to i0, the G query
    // heads of the kv group interleaved per tile: every workgroup of the kv
    // head then reads the same tile at about the same time, so the tiles are
    // fetched from memory once per L2 rather than once per workgroup.
    // DMA cursor: (query head, query tile) of the next tile to issue
    int dhq = hk * G + p0 % G, dti = dir < 0 ? nq - 1 - p0 / G : i0 + p0 / G;
    auto issue = [&](int st) {
        const uint32_t base = lds0 + (uint32_t)(st * STAGE);
        if (w < QW) {
            const size_t qoff = (size_t)(b * a.Hq + dhq) * a.Tq * D;
            qt.load(base, static_cast<const bf16*>(a.q) + qoff, dti * BQ, a.Tq, w);
            qt.load(base + QT::BYTES, static_cast<const bf16*>(a.dout) + qoff, dti * BQ, a.Tq, w);
        }
        if (w < 2) {
            const float* src = (w == 0 ? a.lse : a.delta) + (size_t)(b * a.Hq + dhq) * a.Tq + dti * BQ;
            const i32x4 r = buffer_rsrc(src, (a.Tq - dti * BQ) * 4);
            dma_b32(base + 2 * QT::BYTES + 256 * w, r, (uint32_t)(lane * 4));
        }
        if (++dhq == (hk + 1) * G) {
            dhq = hk * G;
            dti += dir;
        }
    };
    {  // this wave's 32 V rows (rows past T read as zeros)
        const int left = a.Tk - kw;
        const i32x4 r = buffer_rsrc(vh + (size_t)kw * D, left > 0 ? left * D * 2 : 0);
        const uint32_t vb = lds_addr(Vs) + (uint32_t)(w * VW::BYTES);
#pragma unroll
        for (int f = 0; f < VW::NDMA; ++f) dma_b128(vb + (uint32_t)(f * 1024), r, VW::dma_off(f, lane));
    }
    for (int t = 0; t < 2 && t < n; ++t) issue(t);  // the first pair, stages 0 and 1 (then per tile, below)

    // B operand of S = Q K^T: this lane's key row, 8 columns per 16-deep step
    Frag<bf16> kf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kf[ks] = global_frag<bf16>(kh, krow, a.Tk, D, 16 * ks + 8 * g);
    // ADQ: the B operand of dQ = dS K over this wave's 32 keys: for step t
    // (keys 16t .. 16t + 15) and column block db, lane (g, c) holds
    // K[kw + 16t + 8g + e][32db + c], e = 0..7 (zero past Tk)
    [[maybe_unused]] bf16x8 ktf[ADQ ? 2 : 1][ADQ ? NDB : 1];
    if constexpr (ADQ) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int key = kw + 16 * t + 8 * g + e;
                    ktf[t][db][e] = key < a.Tk ? kh[(size_t)key * D + 32 * db + c] : (bf16)0.f;
                }
    }

    // Q, dO rows (A of S, dP) and Q^T, dO^T (A of dK^T, dV^T) in the
    // stages; V rows 32w + c (B of dP) in read order
    SwzRowFrags<Fmt, Cfg::DT> qrd;
    qrd.init(lds_addr(stages), c, g);
    SwzTrFrags<Fmt, Cfg::DT> trd;
    trd.init(lds_addr(stages), lane);
    uint32_t vrd = lds_addr(Vs) + (uint32_t)(w * VW::BYTES + 16 * lane);
    asm volatile("" : "+v"(vrd));
    auto frag = [](bf16x8 v) {
        Frag<bf16> f;
        f.v = v;
        return f;
    };

    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = f32x16{};

    // The stats of the tile in stage st, in place, by the wave whose own DMA
    // moved them: L (natural log) -> -L*log2(e)/c (wave 0) and Delta ->
    // -Delta (wave 1), the initial values of the S and dP accumulators.
    auto convert_l = [&](int st) {
        if (w < 2 && lane < BQ) {
            float* x = reinterpret_cast<float*>(stages + st * STAGE + 2 * QT::BYTES + 256 * w);
            x[lane] = w == 0 ? -(x[lane] * kLog2e) / a.c : -x[lane];
        }
    };

    vm_wait<0>();  // V and the first tiles
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) settle(kf[ks].v);
    convert_l(0);
    convert_l(1);
    sync_lds();
    int bti = dir < 0 ? nq - 1 - p0 / G : i0 + p0 / G, bh = p0 % G;  // query tile and head being computed

    auto body = [&](auto st_tag, int i) {
        constexpr int ST = decltype(st_tag)::value;
        const unsigned char* Qs = stages + ST * STAGE;
        const unsigned char* dOs = Qs + QT::BYTES;
        const float* Ls = reinterpret_cast<const float*>(dOs + QT::BYTES);
        const float* Ds = Ls + 64;
        // Tile i + 2 goes into stage ST + 2, which no wave reads after the
        // barrier that ended the previous pair.  Its Q tile is issued between
        // this tile's score products rather than with the rest at the top:
        // loads issued together reach LDS in one burst that stalls every
        // wave's fragment reads.  (Spreading dO too makes the compiler spill.)
        // A tile past the chunk gets resources of no records: its DMAs read
        // nothing and fill a stage that no tile reads.
        const bool ld = i + 2 < n;
        const int lhq = dhq, lti = dti;  // the cursor's tile, then the cursor moves on
        {
            const bool wrap = dhq + 1 == (hk + 1) * G;
            dhq = ld ? (wrap ? hk * G : dhq + 1) : dhq;
            dti = (ld && wrap) ? dti + dir : dti;
        }
        const uint32_t lbase = lds0 + (uint32_t)(((ST + 2) % NSTAGE) * STAGE);
        if (w < 2) {  // L (wave 0) or Delta (wave 1)
            const float* src = (w == 0 ? a.lse : a.delta) + (size_t)(b * a.Hq + lhq) * a.Tq + lti * BQ;
            const i32x4 r = buffer_rsrc(src, ld ? (a.Tq - lti * BQ) * 4 : 0);
            dma_b32(lbase + 2 * QT::BYTES + 256 * w, r, (uint32_t)(lane * 4));
        }
        i32x4 rq, ro;
        {
            const int row0 = lti * BQ;
            const size_t off = ((size_t)(b * a.Hq + lhq) * a.Tq + row0) * D;
            const int bytes = ld ? (a.Tq - row0) * D * 2 : 0;
            rq = buffer_rsrc(static_cast<const bf16*>(a.q) + off, bytes);
            ro = buffer_rsrc(static_cast<const bf16*>(a.dout) + off, bytes);
        }
        auto part = [&](int k) __attribute__((always_inline)) {  // 0: Q, 1: dO
            if (QW < Cfg::NW && w >= QW) return;  // (uniform per wave)
            dma_b128_nofence(lbase + (uint32_t)(k * QT::BYTES + w * 1024), k == 0 ? rq : ro, qt.voff[0]);
        };

        constexpr uint32_t QI = ST * STAGE, OI = QI + QT::BYTES;  // Q_t, dO_t in the stage
        const bool pad = i >= n;
        const int qb = bti * BQ;
        const int hq_t = hk * G + bh;  // this tile's query head
        (void)hq_t;
        if (++bh == G) {
            bh = 0;
            bti += dir;
        }
        // A tile that no key of this wave sees (or a padding tile) adds
        // nothing: the wave skips its products (the other wave of its SIMD
        // has the matrix pipe to itself meanwhile) but not the barrier below.
        const bool work = !(pad || (CAUSAL && qb + BQ - 1 + a.off < kw));
        part(1);
        if (!work) part(0);
        if (work) {
            // S starts at -L*log2(e)/c and dP at -Delta of their query rows
            // (rows 8*(r/4) + 4g + r%4 of this lane's registers; waves 0 and 1
            // prepared them in the stage): after the products c*s is the
            // exponent of P and dp is dP - Delta.  Every operand fragment is
            // read ahead of its product (S: two products ahead, the others
            // one), into registers the other phases do not use.
            f32x16 s, dp;
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + 8 * rg + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[4 * rg + e] = l4[e];
            }
            {
                constexpr int SAH = 2;
                bf16x8 qr[SAH + 1];
#pragma unroll
                for (int ks = 0; ks < SAH; ++ks) qr[ks] = qrd.read(ks, QI);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    if (ks + SAH < NKS) qr[(ks + SAH) % (SAH + 1)] = qrd.read(ks + SAH, QI);
                    if (ks == NKS / 2) {
#pragma unroll
                        for (int rg = 0; rg < 4; ++rg) {
                            const f32x4 d4 = *reinterpret_cast<const f32x4*>(Ds + 8 * rg + 4 * g);
#pragma unroll
                            for (int e = 0; e < 4; ++e) dp[4 * rg + e] = d4[e];
                        }
                    }
                    mma(s, frag(qr[ks % (SAH + 1)]), kf[ks]);
                    if (ks == 1) part(0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // Tiles wholly visible to this wave take no mask code; the others set
            // the invisible scores to -inf, so that P = 0 there.  Lane c's key
            // kw + c is visible to query qb + row iff c <= qb + off - kw + row.
            if (CAUSAL && qb + a.off < kw + 31) {
                asm volatile("");  // keep this a branch
                const int dlt = max(qb + a.off - kw, -64);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 8 * (r >> 2) + 4 * g + (r & 3);
                    s[r] = c <= dlt + row ? s[r] : -INFINITY;
                }
            }
            __builtin_amdgcn_sched_barrier(0);

            // The vector work runs between the products that do not need it, in
            // this wave's own instruction stream: P between the dP products (from
            // the third on, once S has left the pipe), dS between the dV products.
            // Each group is fenced and each result pinned where it is formed.
            Frag<bf16> pf0, pf1;
            {
                constexpr int PAH = 1;
                bf16x8 ro[PAH + 1], rv[PAH + 1];  // dO and V fragments, PAH products ahead
#pragma unroll
                for (int j = 0; j < PAH; ++j) {
                    ro[j] = qrd.read(j, OI);
                    rv[j] = lds_b128(vrd + (uint32_t)VW::frag_off(0, j));
                }
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    if (ks + PAH < NKS) {
                        ro[(ks + PAH) % (PAH + 1)] = qrd.read(ks + PAH, OI);
                        rv[(ks + PAH) % (PAH + 1)] = lds_b128(vrd + (uint32_t)VW::frag_off(0, ks + PAH));
                    }
                    mma(dp, frag(ro[ks % (PAH + 1)]), frag(rv[ks % (PAH + 1)]));
                    if (ks >= 2) {
                        constexpr int per = (16 + NKS - 3) / (NKS - 2);
#pragma unroll
                        for (int r = per * (ks - 2); r < per * (ks - 1) && r < 16; ++r) {
                            float x = fast_exp2(s[r] * a.c);  // P
                            pin(x);
                            s[r] = x;
                        }
                        if (ks == NKS - 1) {
                            pf0 = acc_frag<bf16>(s, 0);
                            pf1 = acc_frag<bf16>(s, 1);
                            pin(pf0.v);
                            pin(pf1.v);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // dV and dK products: transposed fragments of dO (dV) and Q (dK),
            // one product ahead
            Frag<bf16> sf0, sf1;
            constexpr int NU = 2 * NDB;                    // dV products
            constexpr int U0 = NU >= 8 ? 2 : 1;            // first one with dS work beside it
            constexpr int PER = NU >= 8 ? 4 : (16 + NU - U0 - 1) / (NU - U0);
            auto tr_read = [&](int u) -> bf16x8 {         // fragment of dV (u < NU) or dK product
                const int v = u % NU, t = v / NDB, db = v % NDB;
                return trd.read(db, (u < NU ? OI : QI) + 16 * t * Fmt::ROWBYTES);
            };
            constexpr int TAH = 2;
            bf16x8 rt[TAH + 1];
#pragma unroll
            for (int j = 0; j < TAH; ++j) rt[j] = tr_read(j);
#pragma unroll
            for (int u = 0; u < 2 * NU; ++u) {
                if (u + TAH < 2 * NU) rt[(u + TAH) % (TAH + 1)] = tr_read(u + TAH);
                const int t = (u % NU) / NDB, db = (u % NU) % NDB;
                if (u < NU) {
                    mma(dv[db], frag(rt[u % (TAH + 1)]), t ? pf1 : pf0);
                    if (u >= U0) {
                        const int r0 = PER * (u - U0), r1 = min(16, PER * (u - U0 + 1));
#pragma unroll
                        for (int r = r0; r < r1; ++r) {
                            float x = s[r] * dp[r];  // dS = P (dP - Delta)
                            pin(x);
                            dp[r] = x;
                        }
                        if (r0 <= 7 && r1 > 7) {
                            sf0 = acc_frag<bf16>(dp, 0);
                            pin(sf0.v);
                        }
                        if (r0 < 16 && r1 >= 16) {
                            sf1 = acc_frag<bf16>(dp, 1);
                            pin(sf1.v);
                        }
                    }
                } else {
                    mma(dk[db], frag(rt[u % (TAH + 1)]), t ? sf1 : sf0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (ADQ) {
                // dS, rounded to bf16 as the dK product uses it, into this
                // wave's tile (row query 8(r/4) + 4g + r%4, column key c),
                // read back as the A operand of dQ = dS K (row query c, keys
                // 16t + 8g .. + 7), then this wave's part of the tile's dQ
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    reinterpret_cast<bf16*>(dsw)[(8 * (r >> 2) + 4 * g + (r & 3)) * 32 + c] = (bf16)dp[r];
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                f32x16 dqa[NDB];
#pragma unroll
                for (int db = 0; db < NDB; ++db) dqa[db] = f32x16{};
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const bf16x8 af = *reinterpret_cast<const bf16x8*>(dsw + (c * 32 + 16 * t + 8 * g) * 2);
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, ktf[t][db], dqa[db], 0, 0, 0);
                }
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        red[((tid >> 6) * 32 + 8 * (r >> 2) + 4 * g + (r & 3)) * D + 32 * db + c] = dqa[db][r];
            }
        }
        if constexpr (ADQ) {
            // The tile's dQ: the waves' parts summed in wave order (a wave
            // that skipped the tile adds zeros) and added to the fp32 dQ of
            // its rows with atomic adds (a.part: [B][Hq][Tq][D], zeroed
            // before the launch; dK/dV workgroups of other keys add theirs)
            if (!pad) {
                if (!work) {
#pragma unroll
                    for (int r = 0; r < 32 * D / 64; ++r) red[((tid >> 6) * 32) * D + r * 64 + lane] = 0.f;
                }
                sync_lds();
                const int e0 = 4 * tid;  // 32 x D = 2048 elements, four per thread
                const int qr = e0 / D, d = e0 % D;
                f32x4 sum = {};
#pragma unroll
                for (int ww = 0; ww < Cfg::NW; ++ww) sum += *reinterpret_cast<const f32x4*>(red + (ww * 32 + qr) * D + d);
                if (qb + qr < a.Tq) {
                    float* dst = a.part + ((size_t)(b * a.Hq + hq_t) * a.Tq + qb + qr) * D + d;
#pragma unroll
                    for (int e = 0; e < 4; ++e) unsafeAtomicAdd(dst + e, sum[e]);
                }
                sync_lds();
            }
        }
        // One barrier per pair (measured 1.4 % faster than one per tile: the
        // waves of a SIMD drift out of phase within the pair).  The next
        // pair's tiles must have landed before it; wave 0, which moved their
        // L, converts them first.
        if constexpr (ST % 2 == 1) {
            vm_wait<0>();
            convert_l((ST + 1) % NSTAGE);
            convert_l((ST + 2) % NSTAGE);
            sync_lds();
        }
    };

    for (int i = 0; i < npad; i += NSTAGE)
        unroll_stages(body, i, std::make_integer_sequence<int, NSTAGE>{});

    // this lane: key krow, columns 32db + 8rg + 4g + e
    if (krow < a.Tk) {
        if (S == 1 && a.gf32) {  // float32 gradients: the same values, not rounded
            float* dkh = static_cast<float*>(a.dk) + kvoff + (size_t)krow * D;
            float* dvh = static_cast<float*>(a.dv) + kvoff + (size_t)krow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int col = db * 32 + 8 * rg + 4 * g;
                    f32x4 x, y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] = dk[db][4 * rg + e] * a.scale;
                        y[e] = dv[db][4 * rg + e];
                    }
                    *reinterpret_cast<f32x4*>(dkh + col) = x;
                    *reinterpret_cast<f32x4*>(dvh + col) = y;
                }
        } else if (S == 1) {
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
        } else {
            // fp32 partial sums of this chunk (dK unscaled)
            const size_t plane = (size_t)a.B * a.Hkv * a.Tk * D;
            float* pk = a.part + (size_t)split * plane + kvoff + (size_t)krow * D;
            float* pv = pk + (size_t)S * plane;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int col = db * 32 + 8 * rg + 4 * g;
                    f32x4 x, y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] = dk[db][4 * rg + e];
                        y[e] = dv[db][4 * rg + e];
                    }
                    *reinterpret_cast<f32x4*>(pk + col) = x;
                    *reinterpret_cast<f32x4*>(pv + col) = y;
                }
        }
    }
    };
    if constexpr (PAIRABLE) {
        for (int pass = 0; pass < npass; ++pass) {
            const int key0 = (pass == 0 ? id.tile : nkt - 1 - id.tile) * BK;
            run_block(key0, a.kpair && key0 / 256 >= (nkt256 + 1) / 2 ? 1 : -1);
        }
    } else {
        run_block(id.tile * BK, -1);
    }
}

// out = scale * (sum of the S fp32 partials part[s * plane + .]), added in
// chunk order (so the result does not depend on scheduling), rounded to
// bf16, or stored as float32 with f32 set.  One thread per 8 consecutive
// elements; n8 = plane / 8.
__global__ __launch_bounds__(256) void sum_partials_kernel(const float* part, void* out0, void* out1,
                                                           long n8, long plane, int S, float scale0,
                                                           float scale1, int f32)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    // blockIdx.y: the first tensor's S planes, or the second's after them
    const bool second = blockIdx.y == 1;
    const float* base = part + (second ? (size_t)S * plane : 0);
    const float scale = second ? scale1 : scale0;
    f32x4 lo = {}, hi = {};
    for (int s = 0; s < S; ++s) {
        const f32x4* p = reinterpret_cast<const f32x4*>(base + (size_t)s * plane) + 2 * i;
        lo += p[0];
        hi += p[1];
    }
    void* out = second ? out1 : out0;
    if (f32) {
        f32x4* op = static_cast<f32x4*>(out) + 2 * i;
        op[0] = lo * scale;
        op[1] = hi * scale;
        return;
    }
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = (bf16)(lo[e] * scale);
        x[4 + e] = (bf16)(hi[e] * scale);
    }
    static_cast<bf16x8*>(out)[i] = x;
}

// out0 (and out1, when given: dK and dV in one launch) = scale * the sum, in
// chunk order, of the S fp32 partial planes of each (out1's follow out0's)
static hipError_t sum_partials(const float* part, void* out0, void* out1, long plane, int S,
                               float scale0, float scale1, int f32, hipStream_t stream)
{
    const long n8 = plane / 8;
    hipLaunchKernelGGL(sum_partials_kernel, dim3((unsigned)((n8 + 255) / 256), out1 ? 2 : 1), dim3(256),
                       0, stream, part, out0, out1, n8, plane, S, scale0, scale1, f32);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dQ kernel.  One workgroup of eight waves per (batch, query head, block of
// 256 query rows), two waves per SIMD; wave w owns 32 queries and keeps Q and
// dO of them in registers.  Key tiles of 64 rows walk past in the forward's
// order, K and V by LDS DMA two tiles ahead into four stage buffers (K
// swizzled, read row-wise and transposed; V in read order; every read one
// address register plus an immediate offset).  Per
// 32-key block a wave forms S^T = K Q^T and dP^T = V dO^T with keys as rows,
// P^T = exp2(S^T c - L), dS^T = P^T (dP^T - Delta), and accumulates
// dQ^T += K^T dS^T with dS^T straight from registers; K^T is read transposed
// from the K tile.  A block's dQ products run beside the next block's vector
// work, the tile's last block's at its end.  No atomics: each dQ row is owned
// by one wave.
// ---------------------------------------------------------------------------
template <int D, int NWV>  // head size of the tensors in memory; waves per workgroup
struct DqBf16Cfg {
    static constexpr int DT = tile_dim(D);  // head size of the tiles and products
    static constexpr int NW = NWV;          // 8: two per SIMD; 4: one, two workgroups per CU
    static constexpr int NT = 64 * NW;
    static constexpr int BR = 32 * NW;  // query rows per workgroup
    static constexpr int BC = 64;       // keys per tile
    // four stages, the tile two ahead loading into the stage of tile t - 2
    // (one barrier per tile) or, with pairs, the next pair into the previous
    // pair's stages
    static constexpr int NSTAGE = 4;
    static constexpr int AHEAD = 2;
    using KT = SwzTile<DT, BC, NT, D>;  // K: read row-wise and transposed
    using Fmt = DmaTile<bf16, DT, BC, NT>;
    using VT = RowFragTile<DT, BC, D>;  // V: read row-wise, stored in read order
    static constexpr int VI = VT::NDMA / NW;  // V DMA instructions per wave and tile
    static_assert(VT::NDMA % NW == 0, "V DMA split");
    // K tiles of all stages first, then the V tiles: every read offset fits
    // the 16-bit immediate of a DS read
    static constexpr int VBASE = NSTAGE * KT::BYTES;
    static constexpr int SMEM = VBASE + NSTAGE * VT::BYTES;
    // (the last 16-byte read of a region starts 16 bytes before its end)
    static_assert((NSTAGE - 1) * KT::BYTES + BC * Fmt::ROWBYTES - 16 < 65536, "LDS immediates");
    static_assert((NSTAGE - 1) * VT::BYTES + VT::BYTES - 16 < 65536, "LDS immediates");
    static_assert(AHEAD + 1 <= NSTAGE, "a stage is refilled only after the barrier that ends its tile");
    // Barriers: one per pair of tiles at D = 64 (the next pair loads into
    // the previous pair's stages), one per tile otherwise.  Measured in one
    // process: pairs 1.4 % (C3) and 3.6 % (C2) faster than one per tile at
    // D = 64, 3.9 % slower at D = 128 and 4.1 % at D = 96, bitwise the same.
    static constexpr bool PAIRS = D == 64;
};

template <int D, bool CAUSAL, int NWV>
__global__ __launch_bounds__(64 * NWV, 8 / NWV) void dq_bf16_kernel(BwdArgs a)
{
    using Cfg = DqBf16Cfg<D, NWV>;
    using KT = typename Cfg::KT;
    using Fmt = typename Cfg::Fmt;
    using VT = typename Cfg::VT;
    constexpr int BR = Cfg::BR, BC = Cfg::BC, NSTAGE = Cfg::NSTAGE, NWAVE = Cfg::NW;
    constexpr int AHEAD = Cfg::AHEAD;
    constexpr int NKB = BC / 32;
    // Products run over the D columns of the tensors; the LDS tiles are
    // Cfg::DT wide (D = 96: 128, the last 32 columns zeros that no product reads)
    constexpr int NDB = D / 32;  // 32-column blocks
    constexpr int NKS = D / 16;  // 16-deep steps over the head dimension
    constexpr int VPT = KT::NI + Cfg::VI;  // DMA instructions per tile and wave

    extern __shared__ __align__(1024) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int c = lane & 31;

    const int nqt = (a.Tq + BR - 1) / BR;
    // the nsplit chunks of one query block are neighbours
    const int S = a.nsplit;
    const TileId id = map_tile(blockIdx.x, a.B, a.Hq, a.Hkv, (a.Hq / a.Hkv) * S, nqt, CAUSAL);
    const int b = id.b, hq = id.h / S, split = id.h % S;
    const int hk = hq / (a.Hq / a.Hkv);
    const int q0 = id.tile * BR;
    // first query of this wave.  With eight waves, w and w + 4 share a SIMD;
    // pairing row blocks r and 7 - r there evens out the causal tiles their
    // waves skip.  With four, each wave has a SIMD of the workgroup to itself.
    const int qw = NWAVE == 4 ? q0 + 32 * w : q0 + 32 * (w < 4 ? w : 11 - w);
    const int qrow = qw + c;  // the query this lane owns

    const size_t qoff = (size_t)(b * a.Hq + hq) * a.Tq * D;
    const size_t kvoff = (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const bf16* kh = static_cast<const bf16*>(a.k) + kvoff;
    const bf16* vh = static_cast<const bf16*>(a.v) + kvoff;

    // key tiles visited by the workgroup (query row i sees keys j <= i + off
    // when causal), of which this workgroup takes the chunk [j0, j0 + nkv);
    // tiles below nfull are wholly visible to this wave
    const int kend = CAUSAL ? min(q0 + BR + a.off, a.Tk) : a.Tk;
    const int nall = (kend + BC - 1) / BC;
    const int j0 = nall * split / S;
    const int nkv = nall * (split + 1) / S - j0;
    const int npad = (nkv + NSTAGE - 1) / NSTAGE * NSTAGE;  // loop bound (tiles past nkv are skipped)
    const int nfull = CAUSAL ? min((qw + a.off + 1) / BC, a.Tk / BC) : a.Tk / BC;
    // the first nkw tiles of the chunk are those some row of this wave sees;
    // past them the wave only issues its share of the loads and crosses the
    // barriers
    const int nkw = CAUSAL ? min(nkv, max(0, (qw + 32 + a.off + BC - 1) / BC - j0)) : nkv;

    const uint32_t lds0 = lds_addr(smem);
    KT kt;
    kt.init(tid);
    uint32_t vdma[Cfg::VI];
#pragma unroll
    for (int i = 0; i < Cfg::VI; ++i) vdma[i] = VT::dma_off(w + NWAVE * i, lane);
    auto issue = [&](int t, int st) {  // tile j0 + t into stage st
        const int j = j0 + t;
        kt.load(lds0 + (uint32_t)(st * KT::BYTES), kh, j * BC, a.Tk, w);
        const int left = a.Tk - j * BC;
        const i32x4 r = buffer_rsrc(vh + (size_t)j * BC * D, left > 0 ? left * D * 2 : 0);
        const uint32_t vb = lds0 + (uint32_t)(Cfg::VBASE + st * VT::BYTES);
#pragma unroll
        for (int i = 0; i < Cfg::VI; ++i) dma_b128(vb + (uint32_t)((w + NWAVE * i) * 1024), r, vdma[i]);
    };
    // wait until chunk tile t has landed while tiles t + 1 .. t + AHEAD - 1
    // (those that exist) stay in flight
    auto wait_tile = [&](int t) {
        const int after = nkv - 1 - t;
        if (after >= 1)
            vm_wait<VPT>();
        else
            vm_wait<0>();
        static_assert(AHEAD == 2, "wait counts assume one tile in flight after the awaited one");
    };

    // O of this lane's row, when the kernel forms Delta (loads issued first,
    // so their latency passes under the set-up below)
    Frag<bf16> orow[NKS];
    if (a.delta_out) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            orow[ks] = global_frag<bf16>(static_cast<const bf16*>(a.o) + qoff, qrow, a.Tq, D, 16 * ks + 8 * g);
    }
    for (int t = 0; t < AHEAD && t < nkv; ++t) issue(t, t);

    // B operands of S^T = K Q^T and dP^T = V dO^T: this lane's query row
    Frag<bf16> qf[NKS], of[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        qf[ks] = global_frag<bf16>(static_cast<const bf16*>(a.q) + qoff, qrow, a.Tq, D, 16 * ks + 8 * g);
        of[ks] = global_frag<bf16>(static_cast<const bf16*>(a.dout) + qoff, qrow, a.Tq, D, 16 * ks + 8 * g);
    }
    float L2 = 0.f, Dl = 0.f;
    const size_t rix = (size_t)(b * a.Hq + hq) * a.Tq + qrow;  // this lane's row of lse, Delta
    if (qrow < a.Tq) {
        L2 = a.lse[rix] * kLog2e;
        if (!a.delta_out) Dl = a.delta[rix];
    }
    if (a.delta_out) {
        // Delta = sum_d dO O of this lane's row, formed here and written for
        // the dK/dV kernel, in the order of the preprocess kernel, so the
        // bits are the same: an fma chain over each 8 columns (the lane's
        // chunks 2ks + g), then chunk pairs from the highest bit of the chunk
        // index down; g, the lowest, is added last across the lane pair.
        // The pairs run over the tile width's chunks (a power of two), the
        // padding chunks (D = 96) adding +0, as the preprocess kernel's lanes
        // past D do.
        constexpr int NKT = Cfg::DT / 16;
        static_assert((NKT & (NKT - 1)) == 0, "the chunk pairs assume a power of two");
        float vs[NKT];
#pragma unroll
        for (int ks = 0; ks < NKT; ++ks) {
            float acc = 0.f;
            if (ks < NKS) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf((float)orow[ks].v[e], (float)of[ks].v[e], acc);
            }
            vs[ks] = acc;
        }
#pragma unroll
        for (int bit = NKT / 2; bit >= 1; bit /= 2)
#pragma unroll
            for (int ks = 0; ks < bit; ++ks) vs[ks] += vs[ks + bit];
        Dl = pair_sum(vs[0]);
        if (qrow < a.Tq && g == 0 && split == 0) a.delta_out[rix] = Dl;
    }

    SwzRowFrags<Fmt, Cfg::DT> krd;  // K rows (A of S^T)
    krd.init(lds0, c, g);
    SwzTrFrags<Fmt, Cfg::DT> ktr;   // K^T (A of dQ^T)
    ktr.init(lds0, lane);
    uint32_t vrd = lds0 + (uint32_t)(Cfg::VBASE + 16 * lane);  // V rows (A of dP^T)
    asm volatile("" : "+v"(vrd));
    auto frag = [](bf16x8 v) {
        Frag<bf16> f;
        f.v = v;
        return f;
    };

    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};

    vm_wait<0>();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        settle(qf[ks].v);
        settle(of[ks].v);
    }
    settle(L2);
    settle(Dl);
    sync_lds();

    // dS^T of the previous 32-key block of the tile, the B operands of its
    // dQ products, which run interleaved with the next block's vector work
    Frag<bf16> sp[2];
    // product m of dQ^T += K^T dS^T for the block whose K^T starts at LDS
    // offset koff: its K^T fragment, and the product with that fragment
    auto kt_frag = [&](int m, uint32_t koff) __attribute__((always_inline)) {
        return ktr.read(m % NDB, koff + 16 * (m / NDB) * Fmt::ROWBYTES);
    };
    auto dq_product = [&](int m, const bf16x8& kf) __attribute__((always_inline)) {
        mma(dq[m % NDB], frag(kf), sp[m / NDB]);
    };

    auto body = [&](auto st_tag, int t) {  // chunk tile t = key tile j0 + t
        if (t >= nkv) return;  // (uniform) past the chunk
        constexpr int ST = decltype(st_tag)::value;
        constexpr uint32_t KI = ST * KT::BYTES, VIM = ST * VT::BYTES;  // this stage's tiles
        if constexpr (Cfg::PAIRS) {
            if constexpr (ST % 2 == 0) {
                // tiles t and t + 1 (issued together) have landed, and every
                // wave has left tiles t - 2 and t - 1, whose stages take
                // t + 2 and t + 3
                vm_wait<0>();
                sync_lds();
                if (t + 2 < nkv) issue(t + 2, (ST + 2) % NSTAGE);
                if (t + 3 < nkv) issue(t + 3, (ST + 3) % NSTAGE);
            }
        } else if (t + AHEAD < nkv) {
            issue(t + AHEAD, (ST + AHEAD) % NSTAGE);
        }
        const int j = j0 + t;
        const bool masked = j >= nfull;  // diagonal or future tile
        if (t < nkw) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                f32x16 s = f32x16{}, dp = f32x16{};
                {
                    // K and V fragments, one step ahead of their products
                    auto kread = [&](int ks) { return krd.read(ks, KI + kb * 32 * Fmt::ROWBYTES); };
                    auto vread = [&](int ks) {
                        return lds_b128(vrd + VIM + (uint32_t)VT::frag_off(kb, ks));
                    };
                    bf16x8 rk[3], rv[3];
                    rk[0] = kread(0);
                    rv[0] = vread(0);
                    rk[1] = kread(1);
                    rv[1] = vread(1);
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        if (ks + 2 < NKS) {
                            rk[(ks + 2) % 3] = kread(ks + 2);
                            rv[(ks + 2) % 3] = vread(ks + 2);
                        }
                        mma(s, frag(rk[ks % 3]), qf[ks]);
                        mma(dp, frag(rv[ks % 3]), of[ks]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                if (masked) {
                    asm volatile("");  // keep this a branch
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kj = j * BC + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                        const bool vis = kj < a.Tk && (!CAUSAL || kj <= qrow + a.off);
                        s[r] = vis ? s[r] : -INFINITY;
                    }
                }
                // P and dS of this block beside the dQ products of the block
                // before it (none for the first block of the tile)
                const uint32_t KP = KI + (kb > 0 ? kb - 1 : 0) * 32 * Fmt::ROWBYTES;
                constexpr int NPROD = 2 * NDB;  // dQ products of one block
                bf16x8 kr[3];                   // K^T fragments, read two products ahead
                if (kb > 0) {
                    kr[0] = kt_frag(0, KP);
                    kr[1] = kt_frag(1, KP);
                }
#pragma unroll
                for (int m = 0; m < NPROD; ++m) {
                    if (kb > 0 && m + 2 < NPROD) kr[(m + 2) % 3] = kt_frag(m + 2, KP);
                    if (kb > 0) dq_product(m, kr[m % 3]);
#pragma unroll
                    for (int r = m * 16 / NPROD; r < (m + 1) * 16 / NPROD; ++r) {
                        const float p = fast_exp2(fmaf(s[r], a.c, -L2));  // P^T
                        dp[r] = p * (dp[r] - Dl);                         // dS^T
                        // formed in this group (pure arithmetic would otherwise be
                        // placed ahead of all the products)
                        asm volatile("" : "+v"(dp[r]));
                    }
                    // fenced every two products (measured: every product, or no
                    // fence, ran 2-3 % slower)
                    if (m % 2 == 1) __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2) sp[t2] = acc_frag<bf16>(dp, t2);
            }
            // the tile's last block
            constexpr uint32_t KL = KI + (NKB - 1) * 32 * Fmt::ROWBYTES;
            {
                bf16x8 kr[3];
                kr[0] = kt_frag(0, KL);
                kr[1] = kt_frag(1, KL);
#pragma unroll
                for (int m = 0; m < 2 * NDB; ++m) {
                    if (m + 2 < 2 * NDB) kr[(m + 2) % 3] = kt_frag(m + 2, KL);
                    dq_product(m, kr[m % 3]);
                }
            }
        }
        if constexpr (!Cfg::PAIRS) {
            wait_tile(t + 1);
            sync_lds();
        }
    };

    for (int t = 0; t < npad; t += NSTAGE)
        unroll_stages(body, t, std::make_integer_sequence<int, NSTAGE>{});

    if (qrow < a.Tq) {
        if (S == 1 && a.gf32) {  // float32 dQ: the same values, not rounded
            float* dqh = static_cast<float*>(a.dq) + qoff + (size_t)qrow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = dq[db][4 * rg + e] * a.scale;
                    *reinterpret_cast<f32x4*>(dqh + db * 32 + 8 * rg + 4 * g) = x;
                }
        } else if (S == 1) {
            bf16* dqh = static_cast<bf16*>(a.dq) + qoff + (size_t)qrow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    bf16x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (bf16)(dq[db][4 * rg + e] * a.scale);
                    *reinterpret_cast<bf16x4*>(dqh + db * 32 + 8 * rg + 4 * g) = x;
                }
        } else {  // fp32 partial sums of this chunk (unscaled)
            float* ph = a.part + (size_t)split * a.B * a.Hq * a.Tq * D + qoff + (size_t)qrow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = dq[db][4 * rg + e];
                    *reinterpret_cast<f32x4*>(ph + db * 32 + 8 * rg + 4 * g) = x;
                }
        }
    }
}

template <int D, bool CAUSAL, int NWV>
static hipError_t launch_dq(const BwdArgs& a, hipStream_t stream)
{
    using Cfg = DqBf16Cfg<D, NWV>;
    static_assert(Cfg::SMEM * (8 / NWV) <= 160 * 1024, "LDS budget");
    auto kern = dq_bf16_kernel<D, CAUSAL, NWV>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::SMEM);
    if (attr != hipSuccess) return attr;
    const int nqt = (a.Tq + Cfg::BR - 1) / Cfg::BR;
    const long grid = (long)nqt * a.B * a.Hq * a.nsplit;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::SMEM, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    return sum_partials(a.part, a.dq, nullptr, (long)a.B * a.Hq * a.Tq * D, a.nsplit, a.scale, 0.f,
                        a.gf32, stream);
}

hipError_t launch_bwd_dq_bf16(const BwdArgs& a, int D, bool causal, hipStream_t stream)
{
    if (D == 64) {
        if (dq_rows(a.B, a.Hq, a.Tq, D) == 128)
            return causal ? launch_dq<64, true, 4>(a, stream) : launch_dq<64, false, 4>(a, stream);
        return causal ? launch_dq<64, true, 8>(a, stream) : launch_dq<64, false, 8>(a, stream);
    }
    if (D == 96) return causal ? launch_dq<96, true, 8>(a, stream) : launch_dq<96, false, 8>(a, stream);
    return causal ? launch_dq<128, true, 8>(a, stream) : launch_dq<128, false, 8>(a, stream);
}

template <int D, bool CAUSAL, int NWV, bool ADQ = false>
static hipError_t launch_dkdv(const BwdArgs& a, hipStream_t stream)
{
    using Cfg = DkdvBf16Cfg<D, NWV, ADQ>;
    static_assert(Cfg::SMEM * (8 / NWV) <= 160 * 1024, "LDS budget");
    auto kern = dkdv_bf16_kernel<D, CAUSAL, NWV, ADQ>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::SMEM);
    if (attr != hipSuccess) return attr;
    const int nkt = (a.Tk + Cfg::BK - 1) / Cfg::BK;
    BwdArgs p = a;
    // pairs of key blocks balance causal work only when every block's query
    // range ends at the last tile (no offset) and the blocks are not split
    p.kpair = Cfg::PAIRABLE && CAUSAL && a.nsplit == 1 && a.off == 0 && a.Tq == a.Tk;
    const long grid = (long)(p.kpair ? (nkt + 1) / 2 : nkt) * a.B * a.Hkv * a.nsplit;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::SMEM, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    const long plane = (long)a.B * a.Hkv * a.Tk * D;
    return sum_partials(a.part, a.dk, a.dv, plane, a.nsplit, a.scale, 1.f, a.gf32, stream);
}

// The dK/dV kernel's tile table: keys per workgroup.  At D = 64 a workgroup
// of four waves (128 keys) needs about 50 KiB of LDS, so several share a
// compute unit; used where the 256-key blocks number fewer than kDkdvSmall.
constexpr long kDkdvSmall = 256;
int dkdv_keys(int B, int Hkv, int Tk, int D)
{
    const long blocks256 = (long)((Tk + 255) / 256) * B * Hkv;
    return (D == 64 && blocks256 < kDkdvSmall) ? 128 : 256;
}

// Chunks per key block for the bf16 dK/dV kernel: enough workgroups for about
// two per compute unit when the key blocks alone are too few (few kv heads,
// short keys), at most 8, and at least 8 (query head, query tile) pairs per
// chunk.  Independent of the query offset, so a caller can size the
// workspace from the shapes alone.
int dkdv_nsplit(int B, int Hq, int Hkv, int Tq, int Tk, int D)
{
    constexpr long kTarget = 512;
    const int bk = dkdv_keys(B, Hkv, Tk, D);
    const long wgs = (long)((Tk + bk - 1) / bk) * B * Hkv;
    if (wgs <= 0 || wgs >= kTarget) return 1;
    long s = (kTarget + wgs - 1) / wgs;
    s = s < 8 ? s : 8;
    const long pairs = (long)(Hq / Hkv) * ((Tq + 31) / 32);
    const long cap = pairs / 8 > 1 ? pairs / 8 : 1;
    return (int)(s < cap ? s : cap);
}

// The dQ kernel's tile table: query rows per workgroup.  At D = 64 its
// stages take 64 KiB, so two workgroups of four waves (128 rows) share a
// compute unit.  Measured against 256-row blocks split in two (one process):
// causal B=2 Hq=8 T=512 18.1 -> 14.7 us, but T=4096 (256 blocks of 256
// rows) 83.0 -> 84.7 us; so 128 rows where the 256-row blocks number fewer
// than the 256 compute units.
int dq_rows(int B, int Hq, int Tq, int D)
{
    const long blocks256 = (long)((Tq + 255) / 256) * B * Hq;
    return (D == 64 && blocks256 < 256) ? 128 : 256;
}

// Chunks of the key range per query block for the bf16 dQ kernel: about two
// workgroups per compute unit when the query blocks alone are too few, at
// most 8, and at least 4 key tiles per chunk (8 with 128-row blocks).
int dq_nsplit(int B, int Hq, int Hkv, int Tq, int Tk, int D)
{
    (void)Hkv;
    constexpr long kTarget = 512;
    const int br = dq_rows(B, Hq, Tq, D);
    const long wgs = (long)((Tq + br - 1) / br) * B * Hq;
    if (wgs <= 0 || wgs >= kTarget) return 1;
    long s = (kTarget + wgs - 1) / wgs;
    s = s < 8 ? s : 8;
    const long tiles = (Tk + 63) / 64;
    const long per = br == 128 ? 8 : 4;
    const long cap = tiles / per > 1 ? tiles / per : 1;
    return (int)(s < cap ? s : cap);
}

hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, int D, bool causal, hipStream_t stream)
{
    if (D == 64) {
        if (dkdv_keys(a.B, a.Hkv, a.Tk, D) == 128)
            return causal ? launch_dkdv<64, true, 4>(a, stream) : launch_dkdv<64, false, 4>(a, stream);
        return causal ? launch_dkdv<64, true, 8>(a, stream) : launch_dkdv<64, false, 8>(a, stream);
    }
    if (D == 96) return causal ? launch_dkdv<96, true, 8>(a, stream) : launch_dkdv<96, false, 8>(a, stream);
    return causal ? launch_dkdv<128, true, 8>(a, stream) : launch_dkdv<128, false, 8>(a, stream);
}

// The single-kernel backward of the pages' FA2 description ("L'attention
// fusionnée", «La passe arrière»: dK and dV in registers, dQ accumulated with
// atomic adds), at D = 64: the fp32 dQ accumulator in a.part ([B][Hq][Tq][D])
// is zeroed, the dK/dV kernel adds every tile's dQ to it, and a last kernel
// scales and rounds it into a.dq.  The order of the atomic adds varies from
// run to run, so dQ is not bitwise reproducible (dK, dV are).
__global__ __launch_bounds__(256) void zero_f32_kernel(float* p, long n4)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n4) reinterpret_cast<f32x4*>(p)[i] = f32x4{};
}

__global__ __launch_bounds__(256) void dq_from_acc_kernel(const float* acc, bf16* dq, long n8, float scale)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const f32x4* p = reinterpret_cast<const f32x4*>(acc) + 2 * i;
    const f32x4 lo = p[0], hi = p[1];
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = (bf16)(lo[e] * scale);
        x[4 + e] = (bf16)(hi[e] * scale);
    }
    reinterpret_cast<bf16x8*>(dq)[i] = x;
}

hipError_t launch_bwd_atomic_bf16(const BwdArgs& a0, bool causal, hipStream_t stream)
{
    BwdArgs a = a0;
    a.nsplit = 1;
    const long n = (long)a.B * a.Hq * a.Tq * 64;
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, stream,
                       a.part, n / 4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = causal ? launch_dkdv<64, true, 8, true>(a, stream) : launch_dkdv<64, false, 8, true>(a, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dq_from_acc_kernel, dim3((unsigned)((n / 8 + 255) / 256)), dim3(256), 0, stream,
                       a.part, static_cast<bf16*>(a.dq), n / 8, a.scale);
    return hipGetLastError();
}

// Every kernel variant is instantiated explicitly: referencing a kernel
// template only from a launcher has left some instantiations without their
// host-side handle.
template __global__ void dkdv_bf16_kernel<64, true, 8>(BwdArgs);
template __global__ void dkdv_bf16_kernel<64, false, 8>(BwdArgs);
template __global__ void dkdv_bf16_kernel<64, true, 4>(BwdArgs);
template __global__ void dkdv_bf16_kernel<64, false, 4>(BwdArgs);
template __global__ void dkdv_bf16_kernel<96, true, 8>(BwdArgs);
template __global__ void dkdv_bf16_kernel<96, false, 8>(BwdArgs);
template __global__ void dkdv_bf16_kernel<128, true, 8>(BwdArgs);
template __global__ void dkdv_bf16_kernel<128, false, 8>(BwdArgs);
template __global__ void dkdv_bf16_kernel<64, true, 8, true>(BwdArgs);
template __global__ void dkdv_bf16_kernel<64, false, 8, true>(BwdArgs);
template __global__ void dq_bf16_kernel<64, true, 8>(BwdArgs);
template __global__ void dq_bf16_kernel<64, false, 8>(BwdArgs);
template __global__ void dq_bf16_kernel<64, true, 4>(BwdArgs);
template __global__ void dq_bf16_kernel<64, false, 4>(BwdArgs);
template __global__ void dq_bf16_kernel<96, true, 8>(BwdArgs);
template __global__ void dq_bf16_kernel<96, false, 8>(BwdArgs);
template __global__ void dq_bf16_kernel<128, true, 8>(BwdArgs);
template __global__ void dq_bf16_kernel<128, false, 8>(BwdArgs);

}  // namespace fa
