// Forward kernel: O = softmax(Q K^T * scale [+ causal mask]) V and the row
// log-sum-exp, without ever writing the T x T scores.
//
// Algorithm ("L'attention fusionnée", «Le softmax en ligne»; "FlashAttention:
// l'attenzione che non spreca memoria", «L'idea: lavorare a tessere»): a
// workgroup keeps a block of BR query rows in registers and streams key/value
// tiles of BC rows through LDS.  For every tile it updates a running max m, a
// running sum l and the output numerator o, rescaling both by exp(m - m') when
// the max rises; o is divided by l once at the end, and L = m + ln l is saved.
//
// MI355X mapping:
//   * NW waves, each owning 32 query rows; one wave computes S^T = K Q^T with
//     the 32x32 MFMA so that a lane owns one query column: its row max/sum is
//     an in-lane reduction plus one exchange with lane c ^ 32.
//   * The S^T accumulator is exponentiated in place (exp2 with scale*log2(e)
//     folded in: the cuTile page's INV_LOG_2 trick) and fed straight back as
//     the B operand of O^T += V^T P^T, so P never touches LDS.
//   * K and V tiles move from HBM to LDS with asynchronous global_load_lds
//     (no register staging), double-buffered: the next tile streams in while
//     the current one is used.  V^T fragments come from the natural V tile
//     through the transposing LDS read (ds_read_b64_tr_b16).
//   * The reference max of a row is only moved when the row max rises by more
//     than 8 in log2 units, so most tiles skip rescaling O and l; the weights
//     then stay below 2^8 and the result is unchanged (o and l share the
//     reference).
//   * Causal: tiles wholly in the future are never visited; tiles wholly in
//     the past run without mask code; only diagonal (and, non-causal, the
//     ragged last) tiles take the per-element mask, derived from the lane's
//     query index and the key index ("Optimización de Flash Attention ...",
//     «Atención causal» and the K-loop split of «La pila de optimización»).
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

template <class E, int D, int NW, int BC>
struct FwdCfg {
    static constexpr int NT = NW * 64;
    static constexpr int BR = NW * 32;
    using Tile = DmaTile<E, D, BC, NT>;  // K (read row-wise) and V (read transposed)
    static constexpr int BUF = 2 * Tile::BYTES;
    static constexpr size_t SMEM = 2 * (size_t)BUF;
};

// Threshold (log2 units) by which a row max must exceed the reference max
// before the accumulators are rescaled.
constexpr float kRescaleThreshold = 8.0f;

template <class E, int D, int NW, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, sizeof(E) == 2 ? 8 / NW : 1) void fwd_kernel(FwdArgs a)
{
    using Cfg = FwdCfg<E, D, NW, BC>;
    using Tile = typename Cfg::Tile;
    constexpr int BR = Cfg::BR;
    constexpr int NKB = BC / 32;  // 32-key blocks per tile
    constexpr int NDB = D / 32;   // 32-column blocks of the head dimension
    constexpr int NKS = D / 16;   // 16-deep steps over the head dimension

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
    const int qrow = q0 + w * 32 + c;  // the query this lane owns

    const E* qh = static_cast<const E*>(a.q) + (size_t)(b * a.Hq + hq) * a.Tq * D;
    const E* kh = static_cast<const E*>(a.k) + (size_t)(b * a.Hkv + hk) * a.Tk * D;
    const E* vh = static_cast<const E*>(a.v) + (size_t)(b * a.Hkv + hk) * a.Tk * D;

    // key tiles to visit (query row i sees keys j <= i + off when causal), and
    // how many of them need no mask
    const int kend = CAUSAL ? min(q0 + BR + a.off, a.Tk) : a.Tk;
    const int nkv = (kend + BC - 1) / BC;
    const int nfull = CAUSAL ? min((q0 + a.off + 1) / BC, a.Tk / BC) : a.Tk / BC;

    Tile dma;
    dma.init(tid);
    dma.load(smem, kh, 0, a.Tk, w);
    dma.load(smem + Tile::BYTES, vh, 0, a.Tk, w);

    RowReader<Tile, E, D> krd;
    krd.init(c, g);
    TrReader<Tile, E, D> vrd;
    vrd.init(lane);

    // B operand of S^T = K Q^T: this lane's query row, 8 columns per step
    Frag<E> qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = global_frag<E>(qh, qrow, a.Tq, D, 16 * ks + 8 * g);

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    float mref = -INFINITY;  // reference max, log2 units (scores * scale * log2 e)
    float l = 0.f;           // this lane's share of the row sum

    wait_global_loads();
    __syncthreads();

    // one key tile; BI (0 or 1) is the LDS buffer it sits in
    auto step = [&](auto bufi, int j) {
        constexpr int BI = decltype(bufi)::value;
        const unsigned char* Ks = smem + BI * Cfg::BUF;
        const unsigned char* Vs = Ks + Tile::BYTES;
        if (j + 1 < nkv) {
            unsigned char* nb = smem + (1 - BI) * Cfg::BUF;
            dma.load(nb, kh, (j + 1) * BC, a.Tk, w);
            dma.load(nb + Tile::BYTES, vh, (j + 1) * BC, a.Tk, w);
        }

        // S^T block kb: rows = keys 32kb.., columns = this wave's 32 queries
        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) mma(s[kb], krd.frag(Ks, kb * 32, ks), qf[ks]);
        }

        if (j >= nfull) {  // diagonal or ragged tile: mask from indices
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kj = j * BC + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    const bool vis = kj < a.Tk && (!CAUSAL || kj <= qrow + a.off);
                    if (!vis) s[kb][r] = -INFINITY;
                }
        }

        // row max of this tile (raw scores), then the lazy reference update
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mt = fmaxf(mt, fmaxf(s[kb][r], s[kb][r + 1]));
        mt = pair_max(mt) * a.c;
        const bool need = mt > mref + kRescaleThreshold;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float mnew = need ? mt : mref;
            // 0 on a row's first visible key; 1 for rows that keep their reference
            const float alpha = need ? fast_exp2(mref - mnew) : 1.f;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= alpha;
            mref = mnew;
        }
        const float msub = (mref == -INFINITY) ? 0.f : mref;

        // P = exp2(S c - mref): fp32 row sums (lse keeps full precision), then
        // rounded for the P V product
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[kb][r] = fast_exp2(fmaf(s[kb][r], a.c, -msub));
                l += s[kb][r];
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const Frag<E> pf = acc_frag<E>(s[kb], t);
#pragma unroll
                for (int db = 0; db < NDB; ++db) mma(o[db], vrd.frag(Vs, kb * 32 + 16 * t, db), pf);
            }
        }

        wait_global_loads();
        __syncthreads();
    };

    for (int j = 0; j < nkv; j += 2) {
        step(std::integral_constant<int, 0>{}, j);
        if (j + 1 < nkv) step(std::integral_constant<int, 1>{}, j + 1);
    }

    // epilogue: divide by l, store O (this lane: query qrow, columns
    // 32db + 8rg + 4g + i) and lse
    const float lt = pair_sum(l);
    const float inv = 1.f / lt;
    if (qrow < a.Tq) {
        E* oh = static_cast<E*>(a.o) + ((size_t)(b * a.Hq + hq) * a.Tq + qrow) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                E* p = oh + db * 32 + 8 * rg + 4 * g;
                if constexpr (sizeof(E) == 2) {
                    bf16x4 x;
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = (bf16)(o[db][4 * rg + i] * inv);
                    *reinterpret_cast<bf16x4*>(p) = x;
                } else {
                    f32x4 x;
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = o[db][4 * rg + i] * inv;
                    *reinterpret_cast<f32x4*>(p) = x;
                }
            }
        if (g == 0)
            a.lse[(size_t)(b * a.Hq + hq) * a.Tq + qrow] = (mref + __log2f(lt)) * kLn2;
    }
}

// Tile shape of the forward: NW waves of 32 query rows, BC keys per tile.
constexpr int kFwdNW = 4, kFwdBC = 64;

template <class E, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream)
{
    constexpr int NW = kFwdNW, BC = kFwdBC;
    using Cfg = FwdCfg<E, D, NW, BC>;
    static_assert(Cfg::SMEM <= 160 * 1024, "LDS budget");
    auto kern = fwd_kernel<E, D, NW, BC, CAUSAL>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::SMEM);
    if (attr != hipSuccess) return attr;
    const int nqt = (a.Tq + Cfg::BR - 1) / Cfg::BR;
    const long grid = (long)nqt * a.B * a.Hq;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::SMEM, stream, a);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int D, int dtype, bool causal, hipStream_t stream)
{
    if (dtype == 0) return launch_fwd_bf16(a, D, causal, stream);
    if (D == 64) return causal ? launch_fwd_t<float, 64, true>(a, stream) : launch_fwd_t<float, 64, false>(a, stream);
    return causal ? launch_fwd_t<float, 128, true>(a, stream) : launch_fwd_t<float, 128, false>(a, stream);
}

// Every kernel variant is instantiated explicitly: referencing a kernel
// template only from a launcher has left some instantiations without their
// host-side handle.
#define FA_FWD_INST(E, D, C) template __global__ void fwd_kernel<E, D, kFwdNW, kFwdBC, C>(FwdArgs);
FA_FWD_INST(float, 64, true)
FA_FWD_INST(float, 64, false)
FA_FWD_INST(float, 128, true)
FA_FWD_INST(float, 128, false)
#undef FA_FWD_INST

}  // namespace fa
