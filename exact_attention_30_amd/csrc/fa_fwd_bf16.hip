// bf16 forward kernel: O = softmax(Q K^T * scale [+ causal mask]) V and the
// row log-sum-exp, without ever writing the T x T scores.
//
// Algorithm ("L'attention fusionnée", «Le softmax en ligne»; "FlashAttention:
// l'attenzione che non spreca memoria", «L'idea: lavorare a tessere»): a
// workgroup keeps a block of query rows in registers and streams key/value
// tiles through LDS; per tile it updates a running max m, a running sum l and
// the output numerator o, rescaling both by exp(m - m') when the max rises;
// o is divided by l once at the end and L = m + ln l is saved.
//
// MI355X mapping.
//   * Eight waves of 32 query rows, two per SIMD, each running on its own
//     (one barrier per two tiles for the shared LDS stages); at D = 64 on
//     small grids four waves, two workgroups per compute unit (the tile
//     table, fwd_rows).  A wave computes
//     S^T = K Q^T with the 32x32x16 bf16 MFMA, so a lane owns one query
//     column and its row reductions are in-lane plus one exchange with lane
//     c ^ 32.  The weights are formed from the S^T registers and fed back as
//     the B operand of O^T += V^T P^T: P never touches LDS.
//   * Software pipeline per wave: iteration i issues the products S_i and
//     P_{i-2} V_{i-2}, which do not depend on each other or on the softmax,
//     interleaved one by one with the vector work of tile i - 1 (exp2 of the
//     scores, row sums, bf16 packing).  On gfx950 vector instructions cost
//     MFMA time unless each wave slots them between its own independent
//     MFMAs (measured: about 90 % MFMA occupancy interleaved, 69 % when one
//     wave of a SIMD does the MFMAs and the other the vector work).
//   * K and V tiles move from HBM to LDS by LDS DMA in read order (no bank
//     conflicts, one address register per operand) into four stage buffers:
//     stage t = {K_t, V_{t-2}}, all that iteration t reads.  Stages move
//     in pairs: at every even iteration a wave waits for the two stages it
//     is about to read and crosses one barrier; the buffers the previous
//     pair used then take the next two, whose DMA instructions the even
//     iteration and the odd one after it spread over their products.
//   * Lazy rescale: the reference max of a row only moves when the row max
//     exceeds it by more than 8 (log2 units), so most tiles skip rescaling O
//     and l; the weights stay below 2^8, and o and l share the reference.
//     The weights are first formed with the current reference and the row
//     max is taken only when some lane's share of the tile sum exceeds 2^8
//     (implied whenever a weight does), so most tiles skip the max as well.
//   * Causal: query row i sees key j iff j <= i + off, where off places the
//     query rows among the keys (0 when both are the same sequence; the
//     cuTile kernel's input_pos, «Parte 1»).  Key tiles past the workgroup's
//     last visible key are not visited, and a wave skips the products of
//     those past its own last row's diagonal; tiles wholly visible to a wave run
//     without mask code; the others take the per-element mask derived from the
//     lane's query index and the key index ("Optimización de Flash Attention
//     ...", «Atención causal» and the K-loop split of «La pila de
//     optimización»).
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_pipe.hpp"

namespace fa {

template <int D, int NW>  // head size of the tensors in memory; waves per workgroup
struct FwdBf16Cfg {
    // head size of the tiles and products: D itself (the read-order tiles take
    // any multiple of 32 columns, so D = 96 needs no padding here)
    static constexpr int DT = D;
    static constexpr int NWAVE = NW;         // 8: two per SIMD; 4: one, two workgroups per CU
    static constexpr int NT = 64 * NWAVE;
    static constexpr int BR = 32 * NWAVE;    // query rows per workgroup
    static constexpr int BC = 64;            // keys per tile
    static constexpr int NSTAGE = 4;         // two pairs: one read, one in flight
    // fragment reads in flight ahead of their MFMA (measured in one process:
    // at D = 64 two ahead 1.1-1.3 % faster than three at C3 and C4; at
    // D = 96 and 128 two, three and four the same within 0.2 %, five spills)
    static constexpr int AHD = D == 64 ? 2 : 3;
    using KT = RowFragTile<DT, BC, D>;
    using VT = TrFragTile<DT, BC, D>;
    static constexpr int STAGE = KT::BYTES + VT::BYTES;
    static constexpr int SMEM = NSTAGE * STAGE;
    // DMA instructions per wave per tile, at most: 1 KiB block f goes to wave
    // f % NWAVE (D = 96: 12 blocks over 8 waves, two for waves 0-3, one for 4-7)
    static constexpr int KI = (KT::NDMA + NWAVE - 1) / NWAVE;
    static constexpr int VI = (VT::NDMA + NWAVE - 1) / NWAVE;
    static_assert(DT % 32 == 0, "32-column blocks");
    static_assert(NSTAGE == 4, "stages move in pairs");
};

// The reference max of a row moves only when a weight 2^(s c - mref) of the
// tile would exceed 2^8.
constexpr float kRescaleThresholdBf16 = 8.0f;
constexpr float kMaxWeightBf16 = 256.0f;  // 2^kRescaleThresholdBf16

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_bf16_kernel(FwdArgs a)
{
    using Cfg = FwdBf16Cfg<D, NW>;
    using KT = typename Cfg::KT;
    using VT = typename Cfg::VT;
    constexpr int BR = Cfg::BR, BC = Cfg::BC, NWAVE = Cfg::NWAVE;
    constexpr int KI = Cfg::KI, VI = Cfg::VI;
    constexpr int DT = Cfg::DT;   // tile head size (= D)
    constexpr int NKB = BC / 32;  // 32-key blocks per tile
    constexpr int NDB = DT / 32;  // 32-column blocks of the head dimension
    constexpr int NKS = DT / 16;  // 16-deep steps over the head dimension
    constexpr int AHD = Cfg::AHD, RING = AHD + 1;

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
    const int qrow = qw + c;      // the query this lane owns

    const bf16* qh = static_cast<const bf16*>(a.q) + (size_t)(b * a.Hq + hq) * a.Tq * D;
    const bf16* kh = static_cast<const bf16*>(a.k) + (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const bf16* vh = static_cast<const bf16*>(a.v) + (size_t)(b * a.Hkv + hk) * a.Tk * D;

    // key tiles visited by the workgroup (query row i sees keys j <= i + off
    // when causal), of which this workgroup takes the chunk [j0, j0 + nkv);
    // per wave, the tiles it sees completely (no mask)
    const int kend = CAUSAL ? min(q0 + BR + a.off, a.Tk) : a.Tk;
    const int nall = (kend + BC - 1) / BC;
    const int j0 = nall * split / S;
    const int nkv = nall * (split + 1) / S - j0;
    const int nfull = CAUSAL ? min((qw + a.off + 1) / BC, a.Tk / BC) : a.Tk / BC;
    const size_t rowidx = (size_t)(b * a.Hq + hq) * a.Tq + qrow;  // this lane's query row
    if (nkv == 0) {  // an empty chunk (uniform over the workgroup): nothing seen
        if (qrow < a.Tq && g == 0) {
            const size_t plane = (size_t)a.B * a.Hq * a.Tq;
            float* op = a.opart + ((size_t)split * plane + rowidx) * D;
            for (int d = 0; d < D; ++d) op[d] = 0.f;
            a.ml[2 * ((size_t)split * plane + rowidx)] = -INFINITY;
            a.ml[2 * ((size_t)split * plane + rowidx) + 1] = 0.f;
        }
        return;
    }

    // this thread's DMA source offsets (same for every tile)
    uint32_t koff[KI], voff[VI];
    // (past the last block, D = 96: a valid offset that no DMA uses)
#pragma unroll
    for (int i = 0; i < KI; ++i)
        koff[i] = KT::dma_off(KT::NDMA % NWAVE == 0 ? w + NWAVE * i : min(w + NWAVE * i, KT::NDMA - 1), lane);
#pragma unroll
    for (int i = 0; i < VI; ++i)
        voff[i] = VT::dma_off(VT::NDMA % NWAVE == 0 ? w + NWAVE * i : min(w + NWAVE * i, VT::NDMA - 1), lane);

    // Stage t = {K_t (t < nkv), V_{t-2} (2 <= t <= nkv + 1)} in buffer
    // t % NSTAGE: everything iteration t reads from LDS.
    const uint32_t lds0 = lds_addr(smem);
    // One buffer resource per head for K and one for V (reads past Tk return
    // zeros); a tile's rows enter through the lane offset, so the loads of a
    // tile need no per-tile resource.
    const i32x4 krs = buffer_rsrc(kh, a.Tk * D * 2), vrs = buffer_rsrc(vh, a.Tk * D * 2);
    auto tile_off = [&](int jl) { return (uint32_t)((j0 + jl) * BC * D * 2); };  // chunk tile jl
    auto load_stage = [&](int t) {
        const uint32_t base = lds0 + (uint32_t)((t % Cfg::NSTAGE) * Cfg::STAGE);
        if (t < nkv) {
            const uint32_t ro = tile_off(t);
#pragma unroll
            for (int i = 0; i < KI; ++i)
                if (KT::NDMA % NWAVE == 0 || w + NWAVE * i < KT::NDMA)  // (uniform per wave)
                    dma_b128(base + (uint32_t)((w + NWAVE * i) * 1024), krs, koff[i] + ro);
        }
        if (t >= 2 && t <= nkv + 1) {
            const uint32_t ro = tile_off(t - 2);
#pragma unroll
            for (int i = 0; i < VI; ++i)
                if (VT::NDMA % NWAVE == 0 || w + NWAVE * i < VT::NDMA)
                    dma_b128(base + (uint32_t)(KT::BYTES + (w + NWAVE * i) * 1024), vrs, voff[i] + ro);
        }
    };
    // One DMA instruction of stage t, without a branch (it is issued between
    // the products of an iteration, where a branch would cut the scheduled
    // block): part j < KI is K block w + NWAVE j, the others V blocks.  A
    // part of the stage that holds no tile (K_t with t >= nkv) gets an offset
    // past the resource's records: it reads nothing and writes zeros to a
    // region that no iteration reads.
    auto dma_part = [&](int t, int j) __attribute__((always_inline)) {
        const uint32_t base = lds0 + (uint32_t)((t % Cfg::NSTAGE) * Cfg::STAGE);
        if (j < KI) {
            if (!(KT::NDMA % NWAVE == 0 || w + NWAVE * j < KT::NDMA)) return;  // (uniform per wave)
            const uint32_t ro = t < nkv ? tile_off(t) : kPastEnd;
            dma_b128_nofence(base + (uint32_t)((w + NWAVE * j) * 1024), krs, koff[j] + ro);
        } else {
            const int jv = j - KI;
            if (!(VT::NDMA % NWAVE == 0 || w + NWAVE * jv < VT::NDMA)) return;
            const uint32_t ro = (t >= 2 && t <= nkv + 1) ? tile_off(t - 2) : kPastEnd;
            dma_b128_nofence(base + (uint32_t)(KT::BYTES + (w + NWAVE * jv) * 1024), vrs, voff[jv] + ro);
        }
    };
    load_stage(0);
    load_stage(1);

    // B operand of S^T = K Q^T: this lane's query row, 8 columns per step
    Frag<bf16> qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = global_frag<bf16>(qh, qrow, a.Tq, D, 16 * ks + 8 * g);

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    f32x16 s[2][NKB];          // S^T of tile i (being computed) and of tile i - 1
    u32x4 pf[2][NKB][2];       // P of tile i - 1 (being formed) and of tile i - 2 (B of P V),
                               // bf16 pairs
    float mref = -INFINITY;    // reference max, log2 units
    // the exponent's offset: mref, or 0 while the row has no reference;
    // noref: some row of the wave has none yet (both change with mref only)
    float msub = 0.f;
    bool noref = true;
    float l = 0.f;             // this lane's share of the row sum

    // fragment k of iteration t: score products first, then P V products
    auto frag_read = [&](int t, int k, auto ns) -> bf16x8 {
        constexpr int NS = decltype(ns)::value;
        const unsigned char* st = smem + (t % Cfg::NSTAGE) * Cfg::STAGE;
        if (k < NS) {
            const int kb = k % NKB, ks = k / NKB;
            return KT::read(st + 16 * lane, kb, ks);
        }
        const int m = k - NS, db = m % NDB, u = (m / NDB) % 2, kb = m / (2 * NDB);
        return VT::read(st + KT::BYTES + 8 * lane, 2 * kb + u, db);
    };

    // Mask of tile jl (chunk-local index) for this lane's query: keys past Tk
    // and, when causal, past qrow + off get -inf.
    auto mask_tile = [&](f32x16 (&st)[NKB], int jl) __attribute__((always_inline)) {
        const int j = j0 + jl;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kj = j * BC + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                const bool vis = kj < a.Tk && (!CAUSAL || kj <= qrow + a.off);
                if (!vis) st[kb][r] = -INFINITY;
            }
    };

    // Weights P = 2^(S c - mref) of one tile into bf16 B fragments; returns
    // this lane's share of their sum.
    auto weights = [&](const f32x16 (&st)[NKB], u32x4 (&pt)[NKB][2], float msub)
        __attribute__((always_inline)) -> float {
        float sum[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(st[kb][r], a.c, -msub));
            sum[kb] = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[kb] += p[r];
#pragma unroll
            for (int r = 0; r < 16; r += 2) pt[kb][r / 8][(r % 8) / 2] = pack_bf16(p[r], p[r + 1]);
        }
        float t = sum[0];
#pragma unroll
        for (int kb = 1; kb < NKB; ++kb) t += sum[kb];
        return t;
    };

    // Iteration i (parity P of i): S_i = Q K_i^T into s[P] (HS: i < nkw),
    // O^T += V_{i-2}^T P_{i-2}^T from pf[P] (HPV: i >= 2), and the weights of
    // tile i - 1 from s[P ^ 1] into pf[P ^ 1] (HW: 1 <= i <= nkw), the three
    // interleaved in one instruction stream.  The weights use the current
    // reference; when some weight of a lane may exceed 2^8 (its share of the
    // tile sum does), or a row has no reference yet, the tile takes the
    // reference update of the online softmax («Le softmax en ligne»): row max,
    // a new reference where it rose by more than 8, O and l rescaled, weights
    // recomputed.  O then includes P_{i-2} V_{i-2}, formed with the old
    // reference, so the rescale applies to it too.
    //
    // Stage loads (ISSUE): the buffers of stages i + 2 and i + 3 are free
    // from the barrier of an even i on.  Issued all at once there, the two
    // stages' DMA writes reach LDS in one burst that stalls every wave's
    // fragment reads; instead an even iteration spreads stage i + 2's
    // instructions over its products (kIssueEven) and the odd iteration after
    // it stage i + 3's (kIssueOdd).  Iterations whose parity is known only at
    // run time issue at the top (kIssueTop: an even one both stages after its
    // barrier, an odd one its stage i + 2, the even one before it having
    // spread its own); kIssueBarrier is the plain form, both stages at an
    // even barrier, nothing at an odd i.
    auto iteration = [&](int i, auto par, auto hs, auto hw, auto hpv, auto issue) __attribute__((always_inline)) {
        constexpr int ISSUE = decltype(issue)::value;
        constexpr bool SPREAD = ISSUE == kIssueEven || ISSUE == kIssueOdd;
        constexpr int P = decltype(par)::value;
        constexpr bool HS = decltype(hs)::value, HW = decltype(hw)::value, HPV = decltype(hpv)::value;
        constexpr int NS = HS ? NKS * NKB : 0;         // score products
        constexpr int NPV = HPV ? NKB * 2 * NDB : 0;   // P V products
        constexpr int N = NS + NPV;

        // Stages move in pairs, one barrier per pair: at an even i, stages i
        // and i + 1 have landed (this wave's DMA and, after the barrier,
        // every wave's) and every wave has left iterations i - 2 and i - 1,
        // whose buffers take stages i + 2 and i + 3.
        if ((i & 1) == 0) {
            vm_wait<0>();
            sync_lds();
            if constexpr (!SPREAD) {
                load_stage(i + 2);
                load_stage(i + 3);
            }
        } else if constexpr (ISSUE == kIssueTop) {
            load_stage(i + 2);
        }

        if constexpr (HW) {
            if (j0 + i - 1 >= nfull) {
                asm volatile("");  // keep this a branch
                mask_tile(s[P ^ 1], i - 1);
            }
        }

        // One group per product: the MFMA, the fragment read of the product
        // AHD later, and a share of the weights, which move through four
        // steps per element e (fma at step e, exp2 at e + 1, sum at e + 2,
        // bf16 pair at e + 3) so few temporaries are live; groups are fenced
        // so the compiler keeps this order.  The score products come first
        // (ks outer, kb inner: the two of one accumulator are two products
        // apart), then the P V products (db inner: one P operand for NDB
        // products in a row); alternating the two kinds measured 0.5-0.7 %
        // slower at D = 128 (no change at 64 and 96).
        constexpr int NE = HW ? 16 * NKB : 0;  // weight elements of this lane
        constexpr int NSTEP = HW ? NE + 3 : 0;
        auto product = [](int k) { return k; };  // k-th product: score index, or NS + P V index
        bf16x8 ring[RING];
        using NSc = std::integral_constant<int, NS>;
#pragma unroll
        for (int k = 0; k < AHD && k < N; ++k) ring[k] = frag_read(i, product(k), NSc{});
        const f32x16(&sw)[NKB] = s[P ^ 1];
        u32x4(&pw)[NKB][2] = pf[P ^ 1];
        float fx[NE > 0 ? NE : 1], px[NE > 0 ? NE : 1];
        float lt = 0.f;
        auto step = [&](int t) __attribute__((always_inline)) {
            if (t < NE) fx[t] = fmaf(sw[t / 16][t % 16], a.c, -msub);
            if (t >= 1 && t - 1 < NE) px[t - 1] = fast_exp2(fx[t - 1]);
            if (t >= 2 && t - 2 < NE) lt += px[t - 2];
            if (t >= 3 && (t - 3) % 2 == 0 && t - 2 < NE) {
                // the pair is formed here (the empty asm keeps the compiler
                // from sinking it, with both weights live, to the end)
                const int e = t - 3, kb = e / 16, r = e % 16;
                uint32_t pr = pack_bf16(px[e], px[e + 1]);
                asm volatile("" : "+v"(pr));
                pw[kb][r / 8][(r % 8) / 2] = pr;
            }
        };
        if constexpr (N == 0) {
            static_assert(!SPREAD, "no products to spread the loads over");
#pragma unroll
            for (int t = 0; t < NSTEP; ++t) step(t);
        }
        // stage i + 2's DMA parts go with products 0, STR, 2 STR, ...
        constexpr int NPART = KI + VI;
        constexpr int STR = N >= 4 * NPART ? 4 : N / (NPART > 0 ? NPART : 1);
        static_assert(!SPREAD || STR >= 1, "a product for every DMA part");
#pragma unroll
        for (int k = 0; k < N; ++k) {
            if (k + AHD < N) ring[(k + AHD) % RING] = frag_read(i, product(k + AHD), NSc{});
            Frag<bf16> af;
            af.v = ring[k % RING];
            const int pk = product(k);
            if (pk < NS) {
                const int kb = pk % NKB, ks = pk / NKB;
                if (ks == 0)
                    s[P][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af.v, qf[0].v, f32x16{}, 0, 0, 0);
                else
                    mma(s[P][kb], af, qf[ks]);
            } else {
                const int m = pk - NS, db = m % NDB, u = (m / NDB) % 2, kb = m / (2 * NDB);
                Frag<bf16> bf;
                bf.v = __builtin_bit_cast(bf16x8, pf[P][kb][u]);
                mma(o[db], af, bf);
            }
#pragma unroll
            for (int t = k * NSTEP / (N > 0 ? N : 1); t < (k + 1) * NSTEP / (N > 0 ? N : 1); ++t) step(t);
            if constexpr (SPREAD)
                if (k % STR == 0 && k / STR < NPART) dma_part(i + 2, k / STR);
            __builtin_amdgcn_sched_barrier(0);
        }

        if constexpr (HW) {
            if (noref || __builtin_amdgcn_ballot_w64(lt > kMaxWeightBf16)) {
                float mt = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; r += 2) mt = fmaxf(mt, fmaxf(s[P ^ 1][kb][r], s[P ^ 1][kb][r + 1]));
                mt = pair_max(mt) * a.c;
                const bool need = mt > mref + kRescaleThresholdBf16;
                if (__builtin_amdgcn_ballot_w64(need)) {
                    const float mnew = need ? mt : mref;
                    // 0 on a row's first visible key; 1 for rows that keep
                    // their reference (also those that have seen no key yet)
                    const float alpha = need ? fast_exp2(mref - mnew) : 1.f;
                    l *= alpha;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) o[db] *= alpha;
                    mref = mnew;
                    msub = (mref == -INFINITY) ? 0.f : mref;
                    noref = __builtin_amdgcn_ballot_w64(mref == -INFINITY) != 0;
                    lt = weights(s[P ^ 1], pf[P ^ 1], msub);
                }
            }
            l += lt;
        }
    };

    using F = std::false_type;
    using T = std::true_type;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // The wave computes the first nkw tiles of the chunk, those that some of
    // its rows see (causal: the tiles past its last row's diagonal are
    // skipped; the other wave of its SIMD has the matrix pipe meanwhile), and
    // then only keeps issuing its share of the workgroup's loads and crossing
    // the barriers: every wave runs i = 0 .. nkv + 1 in order, each even i
    // with one barrier.  nkw = 0 only for a chunk none of its rows sees, which
    // leaves o = 0, l = 0 and no reference, as masking every score would.
    const int nkw = CAUSAL ? min(nkv, max(0, (qw + 32 + a.off + BC - 1) / BC - j0)) : nkv;
    if (nkw > 0) {
        // Iterations 0 and 1 are the same for every nkw (with nkw = 1, the
        // product S_1 of iteration 1 is never used): no register state then
        // lives across the branch below.
        using IE = std::integral_constant<int, kIssueEven>;
        using IO = std::integral_constant<int, kIssueOdd>;
        using IT = std::integral_constant<int, kIssueTop>;
        using IB = std::integral_constant<int, kIssueBarrier>;
        iteration(0, P0{}, T{}, F{}, F{}, IE{});
        iteration(1, P1{}, T{}, T{}, F{}, IO{});
        if (nkw == 1) {
            iteration(2, P0{}, F{}, F{}, T{}, IB{});
        } else {
            int i = 2;
            for (; i + 1 < nkw; i += 2) {
                iteration(i, P0{}, T{}, T{}, T{}, IE{});
                iteration(i + 1, P1{}, T{}, T{}, T{}, IO{});
            }
            if (i < nkw) iteration(i++, P0{}, T{}, T{}, T{}, IE{});
            // i == nkw.  The last two iterations exist in one parity only:
            // with nkw odd, S_{nkw-1} and P_{nkw-2} move to the registers that
            // parity expects (a copy once per wave instead of a second version
            // of the code, across which the compiler spills).
            if (nkw & 1) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    s[1][kb] = s[0][kb];
#pragma unroll
                    for (int u = 0; u < 2; ++u) pf[0][kb][u] = pf[1][kb][u];
                }
            }
            // (nkw odd: iteration nkw - 1 was even and spread its stage)
            iteration(nkw, P0{}, F{}, T{}, T{}, IT{});
            iteration(nkw + 1, P1{}, F{}, F{}, T{}, IB{});
        }
    }
    for (int i = nkw > 0 ? nkw + 2 : 0; i <= nkv + 1; ++i)
        if ((i & 1) == 0) {
            vm_wait<0>();
            sync_lds();
            load_stage(i + 2);
            load_stage(i + 3);
        }

    // epilogue: divide by l, store O (this lane: query qrow, columns
    // 32db + 8rg + 4g + i) and lse
    const float lt = pair_sum(l);
    if (S > 1) {  // this chunk's unnormalised numerator, reference max and sum
        if (qrow < a.Tq) {
            const size_t plane = (size_t)a.B * a.Hq * a.Tq;
            float* op = a.opart + ((size_t)split * plane + rowidx) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = o[db][4 * rg + e];
                    *reinterpret_cast<f32x4*>(op + db * 32 + 8 * rg + 4 * g) = x;
                }
            if (g == 0) {
                a.ml[2 * ((size_t)split * plane + rowidx)] = mref;
                a.ml[2 * ((size_t)split * plane + rowidx) + 1] = lt;
            }
        }
        return;
    }
    const float inv = 1.f / lt;
    if (qrow < a.Tq) {
        const size_t orow = ((size_t)(b * a.Hq + hq) * a.Tq + qrow) * D;
        if (a.of32) {  // O as float32: the same values, not rounded to bf16
            float* oh = static_cast<float*>(a.o) + orow;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = o[db][4 * rg + e] * inv;
                    *reinterpret_cast<f32x4*>(oh + db * 32 + 8 * rg + 4 * g) = x;
                }
        } else {
            bf16* oh = static_cast<bf16*>(a.o) + orow;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    bf16x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (bf16)(o[db][4 * rg + e] * inv);
                    *reinterpret_cast<bf16x4*>(oh + db * 32 + 8 * rg + 4 * g) = x;
                }
        }
        if (g == 0) a.lse[(size_t)(b * a.Hq + hq) * a.Tq + qrow] = (mref + __log2f(lt)) * kLn2;
    }
}

// Merge of the key-range chunks of every query row, the rule by which block
// results combine ("FlashAttention" note, «Blockergebnisse…»; "L'attention
// fusionnée", «Le softmax en ligne»): with chunk s holding the numerator o_s
// and sum l_s relative to its reference max m_s (base 2),
//     M = max_s m_s,  w_s = 2^(m_s - M),  O = sum_s w_s o_s / sum_s w_s l_s,
//     lse = ln 2 * (M + log2 sum_s w_s l_s).
// A chunk that saw no key has m_s = -inf and weight 0; chunk 0 always holds
// key 0, which every row sees, so M is finite.  One thread per 8 consecutive
// elements of a row.  O is written as bf16, or as float32 with of32 set.
template <int D>
__global__ __launch_bounds__(256) void merge_chunks_kernel(const float* opart, const float* ml,
                                                           void* o, float* lse, long rows, int S,
                                                           int of32)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * (D / 8)) return;
    const long row = i / (D / 8);
    const int c8 = (int)(i % (D / 8)) * 8;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * (s * rows + row)]);
    float L = 0.f;
    f32x4 lo = {}, hi = {};
    for (int s = 0; s < S; ++s) {
        const float m = ml[2 * (s * rows + row)];
        const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
        L += w * ml[2 * (s * rows + row) + 1];
        const f32x4* p = reinterpret_cast<const f32x4*>(opart + ((size_t)s * rows + row) * D + c8);
        lo += w * p[0];
        hi += w * p[1];
    }
    const float inv = 1.f / L;
    if (of32) {
        f32x4* op = reinterpret_cast<f32x4*>(static_cast<float*>(o) + row * D + c8);
        op[0] = lo * inv;
        op[1] = hi * inv;
    } else {
        bf16x8 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = (bf16)(lo[e] * inv);
            x[4 + e] = (bf16)(hi[e] * inv);
        }
        *reinterpret_cast<bf16x8*>(static_cast<bf16*>(o) + row * D + c8) = x;
    }
    if (c8 == 0) lse[row] = (M + log2f(L)) * kLn2;
}

template <int D, bool CAUSAL, int NW>
static hipError_t launch_t(const FwdArgs& a, hipStream_t stream)
{
    using Cfg = FwdBf16Cfg<D, NW>;
    static_assert(Cfg::SMEM * (8 / NW) <= 160 * 1024, "LDS budget");
    auto kern = fwd_bf16_kernel<D, CAUSAL, NW>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::SMEM);
    if (attr != hipSuccess) return attr;
    const int nqt = (a.Tq + Cfg::BR - 1) / Cfg::BR;
    const long grid = (long)nqt * a.B * a.Hq * a.nsplit;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::SMEM, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    const long rows = (long)a.B * a.Hq * a.Tq;
    const long n8 = rows * (D / 8);
    hipLaunchKernelGGL(merge_chunks_kernel<D>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                       stream, a.opart, a.ml, a.o, a.lse, rows, a.nsplit, a.of32);
    return hipGetLastError();
}

// The forward's static tile table: query rows per workgroup, from the
// shapes.  At D = 64 a workgroup's four stage buffers take 64 KiB, so two
// workgroups of four waves (128 rows) share a compute unit, and they run
// independently (no barrier couples their waves).  Where the 256-row blocks
// alone are fewer than two per compute unit, 128-row blocks are faster
// (measured, unsplit 128 against the best 256-row split: causal B=2 Hq=8
// T=4096 68.6 -> 61.8 us; T=512 19.2 -> 16.1 us); on larger grids they were
// 5-8 % slower.  Everywhere else: 256 rows, eight waves.
int fwd_rows(int B, int Hq, int Tq, int D)
{
    const long blocks256 = (long)((Tq + 255) / 256) * B * Hq;
    return (D == 64 && blocks256 < 512) ? 128 : 256;
}

// Chunks of the key range per query block: about two workgroups per compute
// unit when the query blocks alone are too few, at most 8, and at least 4 key
// tiles per chunk (8 with 128-row blocks, whose short chunks measured slower
// than one: T=512 16.1 us unsplit, 17.6 in two chunks).
int fwd_nsplit(int B, int Hq, int Hkv, int Tq, int Tk, int D)
{
    (void)Hkv;
    constexpr long kTarget = 512;
    const int br = fwd_rows(B, Hq, Tq, D);
    const long wgs = (long)((Tq + br - 1) / br) * B * Hq;
    if (wgs <= 0 || wgs >= kTarget) return 1;
    long s = (kTarget + wgs - 1) / wgs;
    s = s < 8 ? s : 8;
    const long tiles = (Tk + 63) / 64;
    const long per = br == 128 ? 8 : 4;
    const long cap = tiles / per > 1 ? tiles / per : 1;
    return (int)(s < cap ? s : cap);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int D, bool causal, hipStream_t stream)
{
    if (D == 64) {
        if (fwd_rows(a.B, a.Hq, a.Tq, D) == 128)
            return causal ? launch_t<64, true, 4>(a, stream) : launch_t<64, false, 4>(a, stream);
        return causal ? launch_t<64, true, 8>(a, stream) : launch_t<64, false, 8>(a, stream);
    }
    if (D == 96) return causal ? launch_t<96, true, 8>(a, stream) : launch_t<96, false, 8>(a, stream);
    return causal ? launch_t<128, true, 8>(a, stream) : launch_t<128, false, 8>(a, stream);
}

// Every kernel variant is instantiated explicitly: referencing a kernel
// template only from a launcher has left some instantiations without their
// host-side handle.
template __global__ void fwd_bf16_kernel<64, true, 8>(FwdArgs);
template __global__ void fwd_bf16_kernel<64, false, 8>(FwdArgs);
template __global__ void fwd_bf16_kernel<64, true, 4>(FwdArgs);
template __global__ void fwd_bf16_kernel<64, false, 4>(FwdArgs);
template __global__ void fwd_bf16_kernel<96, true, 8>(FwdArgs);
template __global__ void fwd_bf16_kernel<96, false, 8>(FwdArgs);
template __global__ void fwd_bf16_kernel<128, true, 8>(FwdArgs);
template __global__ void fwd_bf16_kernel<128, false, 8>(FwdArgs);

}  // namespace fa
