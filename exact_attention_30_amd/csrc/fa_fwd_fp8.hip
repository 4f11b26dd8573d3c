// FP8 (e4m3) forward: Q, K and V in e4m3 with one descale factor each (the
// real value is the code times its descale), O in bf16 and the row
// log-sum-exp in fp32, in the units of the scaled scores.
//
// The narrower format is the pages' lever for the tensor cores
// ("FlashAttention: l'attenzione che non spreca memoria", «La frontiera»);
// they give no scaling convention, so the plainest is taken: one fp32
// descale per tensor, applied where it is exact to do so.  The descales of Q
// and K multiply the score scale (folded into the exp2 constant), the one of V
// multiplies O in the epilogue.
//
// Algorithm as in the bf16 forward ("L'attention fusionnée", «Le softmax en
// ligne»): a workgroup keeps 256 query rows in registers and streams 64-key
// tiles; a running (lazy) reference max, running sum l and numerator o per
// row; O = o / l at the end.
//
// MI355X mapping (gfx950, v_mfma_f32_32x32x64_f8f6f4: twice the bf16 rate).
//   * S^T = K Q^T: A = K rows (32 keys x 64 head columns per product), B =
//     Q^T, a lane's query in registers.  The 64 columns of one product are
//     split over the lane halves g and the 32 bytes of a lane's operand in
//     the same way for K and Q (column 64ks + 32h + 16g + i for byte 16h + i),
//     which is all the product needs: the order of a contraction index is
//     free as long as both operands share it (checked on the GPU with an
//     in-bounds probe of the instruction's operand layout).
//   * O^T += V^T P^T: B = P^T straight from the S^T registers, rounded to e4m3
//     (one v_cvt_pk_fp8_f32 per two weights): byte j = 16kb + r of a lane's
//     operand is the weight of score register r of key block kb, key
//     32kb + 8(r/4) + 4g + r%4.  A = V^T, whose byte j of lane (c, g) must be
//     V[that key][column c]: a pre-pass writes V transposed, tile by tile,
//     with each 64-byte row in that key order, so the product reads it as
//     plain row fragments.
//   * Per tile and wave: 4 score and 4 P V products (D = 128) instead of 16 +
//     16 in bf16; the same software pipeline as the bf16 forward (products
//     S_i, P_{i-2} V_{i-2} interleaved with the weights of tile i - 1), the
//     same lazy reference (moved only when a weight could exceed 2^8, so every
//     weight fits e4m3, whose largest value is 448), masks and causal offset,
//     stages moving in pairs through four buffers with one barrier per pair,
//     and causal waves computing only the tiles their rows see.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_pipe.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Byte q (0..63) of a transposed 64-key tile row holds key vt_key(q).  Lane
// half g reads row byte q = 32(j/16) + 16g + j%16 as byte j of its V^T
// operand, which must meet byte j of its P operand, the weight of key
// 32(j/16) + 8((j%16)/4) + 4g + j%4; written in q, that key is vt_key(q).
__host__ __device__ constexpr int vt_key(int q)
{
    return 32 * (q / 32) + 8 * ((q % 16) / 4) + 4 * ((q / 16) % 2) + (q % 4);
}

template <int D>
struct FwdFp8Cfg {
    static constexpr int NWAVE = 8;  // two per SIMD
    static constexpr int NT = 64 * NWAVE;
    static constexpr int BR = 32 * NWAVE;  // query rows per workgroup
    static constexpr int BC = 64;          // keys per tile
    static constexpr int NSTAGE = 4;
    static constexpr int AHD = 2;  // products whose fragments are read ahead
    // K tile: 64 key rows of D bytes, as row fragments (a byte pair counted
    // as one two-byte column); V^T tile: D rows of 64 bytes
    using KT = RowFragTile<D / 2, BC>;
    using VT = RowFragTile<32, D>;
    static constexpr int STAGE = KT::BYTES + VT::BYTES;
    static constexpr int SMEM = NSTAGE * STAGE;
};

constexpr float kFp8RescaleThreshold = 8.0f;
constexpr float kFp8MaxWeight = 256.0f;  // 2^kFp8RescaleThreshold <= 448

__device__ __forceinline__ void mma8(f32x16& acc, const i32x8& a, const i32x8& b)
{
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 join(const bf16x8& lo, const bf16x8& hi)
{
    const u32x4 l = __builtin_bit_cast(u32x4, lo), h = __builtin_bit_cast(u32x4, hi);
    return i32x8{(int)l[0], (int)l[1], (int)l[2], (int)l[3], (int)h[0], (int)h[1], (int)h[2], (int)h[3]};
}

// V^T pre-pass: vt[b][hk][t][d][q] = V[b][hk][64t + vt_key(q)][d] (zero past
// Tk).  One workgroup per 64-key tile, through LDS.
template <int D>
__global__ __launch_bounds__(256) void fp8_vt_kernel(const unsigned char* v, unsigned char* vt, int Tk,
                                                     int ntk)
{
    __shared__ __align__(16) unsigned char tile[64][D + 16];
    const long bh = blockIdx.x / ntk;
    const int t = blockIdx.x % ntk;
    const unsigned char* src = v + (size_t)bh * Tk * D + (size_t)t * 64 * D;
    for (int ch = threadIdx.x; ch < 64 * D / 16; ch += 256) {
        const int row = ch / (D / 16), c16 = ch % (D / 16);
        u32x4 x = {0, 0, 0, 0};
        if (t * 64 + row < Tk) x = *reinterpret_cast<const u32x4*>(src + (size_t)row * D + 16 * c16);
        *reinterpret_cast<u32x4*>(&tile[row][16 * c16]) = x;
    }
    __syncthreads();
    unsigned char* dst = vt + ((size_t)bh * ntk + t) * D * 64;
    for (int ch = threadIdx.x; ch < D * 4; ch += 256) {
        const int d = ch / 4, h = ch % 4;
        u32x4 x;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) word |= (uint32_t)tile[vt_key(16 * h + 4 * w4 + i)][d] << (8 * i);
            x[w4] = word;
        }
        *reinterpret_cast<u32x4*>(dst + d * 64 + 16 * h) = x;
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fwd_fp8_kernel(FwdArgs a)
{
    using Cfg = FwdFp8Cfg<D>;
    using KT = typename Cfg::KT;
    using VT = typename Cfg::VT;
    constexpr int BR = Cfg::BR, BC = Cfg::BC, NWAVE = Cfg::NWAVE;
    constexpr int NKB = BC / 32;  // 32-key blocks per tile
    constexpr int NDB = D / 32;   // 32-column blocks of the head dimension
    constexpr int NKS = D / 64;   // 64-deep steps over the head dimension
    constexpr int AHD = Cfg::AHD, RING = AHD + 1;

    extern __shared__ __align__(1024) unsigned char smem[];

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
    // first query of this wave (row blocks r and 7 - r on one SIMD, as in the
    // bf16 forward)
    const int qw = q0 + 32 * (w < 4 ? w : 11 - w);
    const int qrow = qw + c;     // the query this lane owns
    const int ntk = (a.Tk + BC - 1) / BC;

    const unsigned char* qh = static_cast<const unsigned char*>(a.q) + (size_t)(b * a.Hq + hq) * a.Tq * D;
    const unsigned char* kh = static_cast<const unsigned char*>(a.k) + (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const unsigned char* vth = static_cast<const unsigned char*>(a.v) + (size_t)(b * a.Hkv + hk) * ntk * D * 64;

    // key tiles visited (query row i sees keys j <= i + off when causal); per
    // wave, the tiles it sees completely (no mask)
    const int kend = CAUSAL ? min(q0 + BR + a.off, a.Tk) : a.Tk;
    const int nkv = (kend + BC - 1) / BC;  // >= 1
    const int nfull = CAUSAL ? min((qw + a.off + 1) / BC, a.Tk / BC) : a.Tk / BC;

    // DMA blocks (1 KiB) of a tile are spread over the waves: block f is
    // issued by wave f % NWAVE
    constexpr int KB = KT::NDMA, VB = VT::NDMA;

    // Stage t = {K_t (t < nkv), V^T_{t-2} (2 <= t <= nkv + 1)} in buffer
    // t % NSTAGE: everything iteration t reads from LDS.
    const uint32_t lds0 = lds_addr(smem);
    auto load_stage = [&](int t) {
        const uint32_t base = lds0 + (uint32_t)((t % Cfg::NSTAGE) * Cfg::STAGE);
        if (t < nkv) {
            const int row0 = t * BC;
            const i32x4 r = buffer_rsrc(kh + (size_t)row0 * D, (a.Tk - row0) * D);
            for (int f = w; f < KB; f += NWAVE) dma_b128(base + (uint32_t)(f * 1024), r, KT::dma_off(f, lane));
        }
        if (t >= 2 && t <= nkv + 1) {
            const i32x4 r = buffer_rsrc(vth + (size_t)(t - 2) * D * 64, D * 64);
            for (int f = w; f < VB; f += NWAVE)
                dma_b128(base + (uint32_t)(KT::BYTES + f * 1024), r, VT::dma_off(f, lane));
        }
    };
    // One DMA instruction of stage t without a branch, for iterations that
    // spread their loads over the products (as the bf16 forward does): part
    // 0 is this wave's K block, part 1 its V^T block; a part of a stage that
    // holds no tile gets a resource of no records (reads nothing, fills a
    // region that no iteration reads).
    static_assert(KB <= NWAVE && VB <= NWAVE, "at most one block of each tile per wave");
    auto dma_part = [&](int t, int j) __attribute__((always_inline)) {
        const uint32_t base = lds0 + (uint32_t)((t % Cfg::NSTAGE) * Cfg::STAGE);
        if (j == 0) {
            if (KB < NWAVE && w >= KB) return;  // (uniform per wave)
            const int row0 = t * BC;
            const i32x4 r = buffer_rsrc(kh + (size_t)row0 * D, t < nkv ? (a.Tk - row0) * D : 0);
            dma_b128_nofence(base + (uint32_t)(w * 1024), r, KT::dma_off(w, lane));
        } else {
            if (VB < NWAVE && w >= VB) return;
            const i32x4 r = buffer_rsrc(vth + (size_t)(t - 2) * D * 64, (t >= 2 && t <= nkv + 1) ? D * 64 : 0);
            dma_b128_nofence(base + (uint32_t)(KT::BYTES + w * 1024), r, VT::dma_off(w, lane));
        }
    };
    load_stage(0);
    load_stage(1);

    // B operand of S^T = K Q^T: this lane's query row, columns 64ks + 32h +
    // 16g + i in byte 16h + i (zeros past Tq)
    i32x8 qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        bf16x8 lo = {}, hi = {};
        if (qrow < a.Tq) {
            const unsigned char* r = qh + (size_t)qrow * D + 64 * ks + 16 * g;
            lo = *reinterpret_cast<const bf16x8*>(r);
            hi = *reinterpret_cast<const bf16x8*>(r + 32);
        }
        qf[ks] = join(lo, hi);
    }

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    f32x16 s[2][NKB];  // S^T of tile i (being computed) and of tile i - 1
    i32x8 pf[2];       // P of tile i - 1 (being formed) and of tile i - 2, e4m3
    float mref = -INFINITY;  // reference max, log2 units
    // the exponent's offset: mref, or 0 while the row has no reference;
    // noref: some row of the wave has none yet (both change with mref only)
    float msub = 0.f;
    bool noref = true;
    float l = 0.f;           // this lane's share of the row sum

    // A fragment of product k of iteration t: score products first (K rows),
    // then P V products (V^T rows)
    auto frag_read = [&](int t, int k, auto ns) -> i32x8 {
        constexpr int NS = decltype(ns)::value;
        const unsigned char* st = smem + (t % Cfg::NSTAGE) * Cfg::STAGE;
        if (k < NS) {
            const int kb = k % NKB, ks = k / NKB;
            return join(KT::read(st + 16 * lane, kb, 2 * ks), KT::read(st + 16 * lane, kb, 2 * ks + 1));
        }
        const int db = k - NS;
        return join(VT::read(st + KT::BYTES + 16 * lane, db, 0), VT::read(st + KT::BYTES + 16 * lane, db, 1));
    };

    // keys past Tk and, when causal, past qrow + off get -inf
    auto mask_tile = [&](f32x16 (&st)[NKB], int j) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kj = j * BC + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                const bool vis = kj < a.Tk && (!CAUSAL || kj <= qrow + a.off);
                if (!vis) st[kb][r] = -INFINITY;
            }
    };

    // e4m3 code of the weights 2^(S c - msub) of one tile (byte 16kb + r of
    // the operand: register r of block kb); returns this lane's share of
    // their fp32 sum
    auto weights = [&](const f32x16 (&st)[NKB], i32x8& pt, float msub) __attribute__((always_inline)) -> float {
        float sum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p[e] = fast_exp2(fmaf(st[kb][r + e], a.c, -msub));
                    sum += p[e];
                }
                // the low half first (the high half it keeps is overwritten next)
                int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pt[(16 * kb + r) / 4], false);
                wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
                pt[(16 * kb + r) / 4] = wd;
            }
        return sum;
    };

    // Iteration i (parity P of i): S_i = Q K_i^T into s[P] (HS), O^T +=
    // V_{i-2}^T P_{i-2}^T from pf[P] (HPV), and the weights of tile i - 1
    // from s[P ^ 1] into pf[P ^ 1] (HW), interleaved in one instruction
    // stream; then the reference update when some weight may exceed 2^8 or a
    // row has no reference yet (as in the bf16 forward).
    // ISSUE: where the iteration issues stage loads (kIssue* of the bf16
    // forward: an even iteration spreads stage i + 2 over its products, the
    // odd one after it stage i + 3)
    auto iteration = [&](int i, auto par, auto hs, auto hw, auto hpv, auto issue) __attribute__((always_inline)) {
        constexpr int ISSUE = decltype(issue)::value;
        constexpr bool SPREAD = ISSUE == kIssueEven || ISSUE == kIssueOdd;
        constexpr int P = decltype(par)::value;
        constexpr bool HS = decltype(hs)::value, HW = decltype(hw)::value, HPV = decltype(hpv)::value;
        constexpr int NS = HS ? NKS * NKB : 0;
        constexpr int NPV = HPV ? NDB : 0;
        constexpr int N = NS + NPV;

        // stages move in pairs, one barrier per pair (as in the bf16 forward)
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
            if (i - 1 >= nfull) {
                asm volatile("");  // keep this a branch
                mask_tile(s[P ^ 1], i - 1);
            }
        }

        // weight element e (register e % 16 of block e / 16) moves through
        // four steps: fma at step e, exp2 at e + 1, sum at e + 2, e4m3 pair
        // at e + 3; the steps are spread over the products
        constexpr int NE = HW ? 16 * NKB : 0;
        constexpr int NSTEP = HW ? NE + 3 : 0;
        // products in order: the score products (ks outer, kb inner), then
        // the P V products, whose operand P is the same for all four (an
        // order that alternates the two kinds measured about 1 % slower)
        auto product = [](int k) { return k; };
        using NSc = std::integral_constant<int, NS>;
        i32x8 ring[RING];
#pragma unroll
        for (int k = 0; k < AHD && k < N; ++k) ring[k] = frag_read(i, product(k), NSc{});
        const f32x16(&sw)[NKB] = s[P ^ 1];
        i32x8& pw = pf[P ^ 1];
        float fx[NE > 0 ? NE : 1], px[NE > 0 ? NE : 1];
        float lt = 0.f;
        auto step = [&](int t) __attribute__((always_inline)) {
            if (t < NE) fx[t] = fmaf(sw[t / 16][t % 16], a.c, -msub);
            if (t >= 1 && t - 1 < NE) px[t - 1] = fast_exp2(fx[t - 1]);
            if (t >= 2 && t - 2 < NE) lt += px[t - 2];
            if (t >= 3 && (t - 3) % 2 == 0 && t - 2 < NE) {
                const int e = t - 3;  // bytes e, e + 1 of the operand
                if (e % 4 == 0) {
                    // the low half; the high half it keeps (tile i - 3's
                    // weights, already used) is overwritten two steps later
                    pw[e / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(px[e], px[e + 1], pw[e / 4], false);
                } else {
                    int wd = __builtin_amdgcn_cvt_pk_fp8_f32(px[e], px[e + 1], pw[e / 4], true);
                    // formed here, not sunk with its weights live to the end
                    asm volatile("" : "+v"(wd));
                    pw[e / 4] = wd;
                }
            }
        };
        if constexpr (N == 0) {
            static_assert(!SPREAD, "no products to spread the loads over");
#pragma unroll
            for (int t = 0; t < NSTEP; ++t) step(t);
        }
        // stage i + 2's two DMA parts go with products 0 and STR
        constexpr int STR = N >= 8 ? 4 : N / 2;
        static_assert(!SPREAD || STR >= 1, "a product for every DMA part");
#pragma unroll
        for (int k = 0; k < N; ++k) {
            if (k + AHD < N) ring[(k + AHD) % RING] = frag_read(i, product(k + AHD), NSc{});
            const i32x8 af = ring[k % RING];
            const int pk = product(k);
            if (pk < NS) {
                const int kb = pk % NKB, ks = pk / NKB;
                if (ks == 0)
                    s[P][kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, qf[0], f32x16{}, 0, 0, 0, 0, 0, 0);
                else
                    mma8(s[P][kb], af, qf[ks]);
            } else {
                mma8(o[pk - NS], af, pf[P]);
            }
#pragma unroll
            for (int t = k * NSTEP / (N > 0 ? N : 1); t < (k + 1) * NSTEP / (N > 0 ? N : 1); ++t) step(t);
            if constexpr (SPREAD)
                if (k % STR == 0 && k / STR < 2) dma_part(i + 2, k / STR);
            __builtin_amdgcn_sched_barrier(0);
        }

        if constexpr (HW) {
            if (noref || __builtin_amdgcn_ballot_w64(lt > kFp8MaxWeight)) {
                float mt = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; r += 2) mt = fmaxf(mt, fmaxf(s[P ^ 1][kb][r], s[P ^ 1][kb][r + 1]));
                mt = pair_max(mt) * a.c;
                const bool need = mt > mref + kFp8RescaleThreshold;
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
    // The wave computes the tiles some of its rows see (nkw >= 1: every row
    // sees key 0), then only issues its share of the loads and crosses the
    // barriers; every wave runs i = 0 .. nkv + 1 in order (as in the bf16
    // forward).  Iterations 0 and 1 are the same for every nkw (with nkw = 1
    // the product S_1 is never used).
    const int nkw = CAUSAL ? min(nkv, (qw + 32 + a.off + BC - 1) / BC) : nkv;
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
        // one parity for the last two iterations (see the bf16 forward)
        if (nkw & 1) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[1][kb] = s[0][kb];
            pf[0] = pf[1];
        }
        iteration(nkw, P0{}, F{}, T{}, T{}, IT{});
        iteration(nkw + 1, P1{}, F{}, F{}, T{}, IB{});
    }
    for (int i = nkw + 2; i <= nkv + 1; ++i)
        if ((i & 1) == 0) {
            vm_wait<0>();
            sync_lds();
            load_stage(i + 2);
            load_stage(i + 3);
        }

    // epilogue: O = vscale * o / l (bf16; this lane: query qrow, columns
    // 32db + 8rg + 4g + e), lse = ln 2 (mref + log2 l)
    const float lt = pair_sum(l);
    const float f = a.vscale / lt;
    if (qrow < a.Tq) {
        bf16* oh = static_cast<bf16*>(a.o) + ((size_t)(b * a.Hq + hq) * a.Tq + qrow) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                bf16x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (bf16)(o[db][4 * rg + e] * f);
                *reinterpret_cast<bf16x4*>(oh + db * 32 + 8 * rg + 4 * g) = x;
            }
        if (g == 0) a.lse[(size_t)(b * a.Hq + hq) * a.Tq + qrow] = (mref + __log2f(lt)) * kLn2;
    }
}

template <int D>
static hipError_t launch_vt_t(const void* v, void* vt, int B, int Hkv, int Tk, hipStream_t stream)
{
    const int ntk = (Tk + 63) / 64;
    const long grid = (long)B * Hkv * ntk;
    hipLaunchKernelGGL(fp8_vt_kernel<D>, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const unsigned char*>(v), static_cast<unsigned char*>(vt), Tk, ntk);
    return hipGetLastError();
}

hipError_t launch_fp8_vt(const void* v, void* vt, int B, int Hkv, int Tk, int D, hipStream_t stream)
{
    return D == 64 ? launch_vt_t<64>(v, vt, B, Hkv, Tk, stream) : launch_vt_t<128>(v, vt, B, Hkv, Tk, stream);
}

template <int D, bool CAUSAL>
static hipError_t launch_t(const FwdArgs& a, hipStream_t stream)
{
    using Cfg = FwdFp8Cfg<D>;
    static_assert(Cfg::SMEM <= 160 * 1024, "LDS budget");
    auto kern = fwd_fp8_kernel<D, CAUSAL>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::SMEM);
    if (attr != hipSuccess) return attr;
    const int nqt = (a.Tq + Cfg::BR - 1) / Cfg::BR;
    const long grid = (long)nqt * a.B * a.Hq;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::SMEM, stream, a);
    return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdArgs& a, int D, bool causal, hipStream_t stream)
{
    if (D == 64) return causal ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
    return causal ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
}

// every kernel variant is instantiated explicitly (see the bf16 forward)
template __global__ void fp8_vt_kernel<64>(const unsigned char*, unsigned char*, int, int);
template __global__ void fp8_vt_kernel<128>(const unsigned char*, unsigned char*, int, int);
template __global__ void fwd_fp8_kernel<64, true>(FwdArgs);
template __global__ void fwd_fp8_kernel<64, false>(FwdArgs);
template __global__ void fwd_fp8_kernel<128, true>(FwdArgs);
template __global__ void fwd_fp8_kernel<128, false>(FwdArgs);

}  // namespace fa
