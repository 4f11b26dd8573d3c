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
//   * Eight waves of 32 query rows.  A wave computes S^T = K Q^T with the
//     32x32x16 bf16 MFMA, so a lane owns one query column: its row max and sum
//     are in-lane reductions plus one exchange with lane c ^ 32.  The S^T
//     accumulator is exponentiated in place (exp2, scale*log2 e folded in) and
//     fed back as the B operand of O^T += V^T P^T: P never touches LDS.
//   * Two waves per SIMD (eight per workgroup) in two groups of four that
//     run in lock step, one phase apart: in every phase one wave of each SIMD
//     issues MFMAs while its partner does vector work.  The matrix step of
//     tile j also issues the P V product of tile j - 1: M(j) = { O += P_{j-1}
//     V_{j-1}; S_j = Q K_j^T } (MFMAs, LDS reads), then V(j) = { mask; max;
//     rescale; P_j = exp2(...) } (vector ALU), which also reads the first
//     operand fragments of M(j + 1).
//   * K and V tiles move from HBM to LDS by LDS DMA in read order (no bank
//     conflicts, one address register per operand) into four stage buffers:
//     stage j = {K_j, V_{j-1}} is the LDS data of step M(j), issued six
//     phases before the first read of it.
//   * Lazy rescale: the reference max of a row only moves when the row max
//     exceeds it by more than 8 (log2 units), so most tiles skip rescaling O
//     and l; the weights stay below 2^8, and o and l share the reference.
//   * Causal: query row i sees key j iff j <= i + off, where off places the
//     query rows among the keys (0 when both are the same sequence; the
//     cuTile kernel's input_pos, «Parte 1»).  Key tiles past the workgroup's
//     last visible key are not visited; tiles wholly visible to a wave run
//     without mask code; the others take the per-element mask derived from the
//     lane's query index and the key index ("Optimización de Flash Attention
//     ...", «Atención causal» and the K-loop split of «La pila de
//     optimización»).
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_pipe.hpp"

namespace fa {

template <int D>  // head size of the tensors in memory
struct FwdBf16Cfg {
    static constexpr int DT = tile_dim(D);   // head size of the tiles and products
    static constexpr int NW = 4;             // waves per group
    static constexpr int NWAVE = 2 * NW;     // waves per workgroup (two per SIMD)
    static constexpr int NT = 64 * NWAVE;
    static constexpr int BR = 32 * NWAVE;    // query rows per workgroup
    static constexpr int BC = 64;            // keys per tile
    static constexpr int NSTAGE = 4;
    static constexpr int AHD = 6;            // fragment reads in flight ahead of their MFMA
    using KT = RowFragTile<DT, BC, D>;
    using VT = TrFragTile<DT, BC, D>;
    static constexpr int STAGE = KT::BYTES + VT::BYTES;
    static constexpr int SMEM = NSTAGE * STAGE;
    static constexpr int KI = KT::NDMA / NWAVE;  // DMA instructions per wave per tile
    static constexpr int VI = VT::NDMA / NWAVE;
    static_assert(KT::NDMA % NWAVE == 0 && VT::NDMA % NWAVE == 0, "DMA split");
};

constexpr float kRescaleThresholdBf16 = 8.0f;

// Scheduling pins for a run of N MFMAs whose A fragments come from LDS, AHD
// fragments ahead (the first AHD already in registers): each MFMA is followed
// by the reads of the fragment AHD products later.  The S products (first)
// use row fragments (one LDS read), the PV products transposed fragments
// (two).
template <int N, int AHD, class TPV, class TS, int... I>
__device__ __forceinline__ void pin_mfma_ds_interleave(std::integer_sequence<int, I...>, TPV, TS)
{
    constexpr int kDsRead = 0x100, kMfma = 0x008;
    constexpr int NS = TS::value ? (N - (TPV::value ? N / 2 : 0)) : 0;
    (
        [] {
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
            if constexpr (I + AHD < N)
                __builtin_amdgcn_sched_group_barrier(kDsRead, (I + AHD < NS) ? 1 : 2, 0);
        }(),
        ...);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fwd_bf16_kernel(FwdArgs a)
{
    using Cfg = FwdBf16Cfg<D>;
    using KT = typename Cfg::KT;
    using VT = typename Cfg::VT;
    constexpr int BR = Cfg::BR, BC = Cfg::BC, NWAVE = Cfg::NWAVE;
    constexpr int KI = Cfg::KI, VI = Cfg::VI;
    constexpr int DT = Cfg::DT;   // tile head size (D in memory; padding columns are zeros)
    constexpr int NKB = BC / 32;  // 32-key blocks per tile
    constexpr int NDB = DT / 32;  // 32-column blocks of the head dimension
    constexpr int NKS = DT / 16;  // 16-deep steps over the head dimension

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
    const int qw = q0 + 32 * w;   // first query of this wave
    const int qrow = qw + c;      // the query this lane owns
    const int grp = w / Cfg::NW;  // 0 or 1: phase offset of the ping-pong

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
#pragma unroll
    for (int i = 0; i < KI; ++i) koff[i] = KT::dma_off(w + NWAVE * i, lane);
#pragma unroll
    for (int i = 0; i < VI; ++i) voff[i] = VT::dma_off(w + NWAVE * i, lane);

    const uint32_t lds0 = lds_addr(smem);
    // stage s = {K_s (s < nkv), V_{s-1} (s >= 1)} in buffer s % NSTAGE
    auto load_stage = [&](int s) {
        const uint32_t base = lds0 + (uint32_t)((s % Cfg::NSTAGE) * Cfg::STAGE);
        if (s < nkv) {
            const int row0 = (j0 + s) * BC;
            const i32x4 r = buffer_rsrc(kh + (size_t)row0 * D, (a.Tk - row0) * D * 2);
#pragma unroll
            for (int i = 0; i < KI; ++i) dma_b128(base + (uint32_t)((w + NWAVE * i) * 1024), r, koff[i]);
        }
        if (s >= 1) {
            const int row0 = (j0 + s - 1) * BC;
            const i32x4 r = buffer_rsrc(vh + (size_t)row0 * D, (a.Tk - row0) * D * 2);
#pragma unroll
            for (int i = 0; i < VI; ++i)
                dma_b128(base + (uint32_t)(KT::BYTES + (w + NWAVE * i) * 1024), r, voff[i]);
        }
    };

    load_stage(0);
    load_stage(1);  // nkv >= 1, so stage 1 holds at least V_0
    if (nkv >= 2) load_stage(2);

    // B operand of S^T = K Q^T: this lane's query row, 8 columns per step
    Frag<bf16> qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = global_frag<bf16>(qh, qrow, a.Tq, D, 16 * ks + 8 * g);

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    f32x16 s[NKB];                 // S^T of the current tile (rows = keys)
    Frag<bf16> pf[NKB][2];         // P of the previous tile (B operands of P V)
    float mref = -INFINITY;        // reference max, log2 units
    float l = 0.f;                 // this lane's share of the row sum

    vm_wait<0>();
    sync_lds();

    // Matrix step M(j): S_j^T = K_j Q^T (S, j < nkv) and O^T += V_{j-1}^T
    // P_{j-1}^T (PV, j >= 1), all operands from stage j.  Product i reads its
    // A fragment AHD products ahead into a ring of registers; the first AHD
    // reads are issued by the preceding vector step of the same wave (its LDS
    // port is otherwise idle), so the matrix step starts without waiting.
    constexpr int AHD = Cfg::AHD, RING = AHD + 1;
    bf16x8 ring[RING];
    auto frag_read = [&](int j, int i, auto with_pv, auto with_s) -> bf16x8 {
        constexpr bool PV = decltype(with_pv)::value, SS = decltype(with_s)::value;
        constexpr int NS = SS ? NKS * NKB : 0;
        const unsigned char* st = smem + (j % Cfg::NSTAGE) * Cfg::STAGE;
        if (i < NS) {
            const int kb = i % NKB, ks = i / NKB;
            return KT::read(st + 16 * lane, kb, ks);
        }
        (void)PV;
        const int k = i - NS, db = k % NDB, t = (k / NDB) % 2, kb = k / (2 * NDB);
        return VT::read(st + KT::BYTES + 8 * lane, 2 * kb + t, db);
    };
    auto prefetch = [&](int j, auto with_pv, auto with_s) {
#pragma unroll
        for (int i = 0; i < AHD; ++i) ring[i] = frag_read(j, i, with_pv, with_s);
    };
    auto matrix_step = [&](int j, auto with_pv, auto with_s) {
        constexpr bool PV = decltype(with_pv)::value, SS = decltype(with_s)::value;
        constexpr int NPV = PV ? NKB * 2 * NDB : 0;   // PV products
        constexpr int NS = SS ? NKS * NKB : 0;        // S products
        constexpr int N = NPV + NS;
        static_assert(N > AHD, "prefetch depth");
        if constexpr (SS) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
        }
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if (i + AHD < N) ring[(i + AHD) % RING] = frag_read(j, i + AHD, with_pv, with_s);
            Frag<bf16> af;
            af.v = ring[i % RING];
            if (i < NS) {
                const int kb = i % NKB, ks = i / NKB;
                mma(s[kb], af, qf[ks]);
            } else {
                const int k = i - NS, db = k % NDB, t = (k / NDB) % 2, kb = k / (2 * NDB);
                mma(o[db], af, pf[kb][t]);
            }
        }
        pin_mfma_ds_interleave<N, AHD>(std::make_integer_sequence<int, N>{}, with_pv, with_s);
    };

    // Vector step V(j): mask, lazy reference update (rescaling O and l when it
    // moves), P_j = exp2(S_j c - mref) with fp32 row sums, rounded for P V.
    auto vector_step = [&](int jl) {
        const int j = j0 + jl;  // key tile
        if (j >= nfull) {
            asm volatile("");  // keep this a branch
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kj = j * BC + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    const bool vis = kj < a.Tk && (!CAUSAL || kj <= qrow + a.off);
                    if (!vis) s[kb][r] = -INFINITY;
                }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mt = fmaxf(mt, fmaxf(s[kb][r], s[kb][r + 1]));
        mt = pair_max(mt) * a.c;
        const bool need = mt > mref + kRescaleThresholdBf16;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float mnew = need ? mt : mref;
            // 0 on a row's first visible key; 1 for rows that keep their
            // reference (also those that have seen no key yet: -inf - -inf)
            const float alpha = need ? fast_exp2(mref - mnew) : 1.f;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= alpha;
            mref = mnew;
        }
        const float msub = (mref == -INFINITY) ? 0.f : mref;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[kb][r] = fast_exp2(fmaf(s[kb][r], a.c, -msub));
                l += s[kb][r];
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) pf[kb][t] = acc_frag<bf16>(s[kb], t);
        }
    };

    // Lock-step phases (ping-pong).  Group 0 runs the sequence M(0) V(0) M(1)
    // V(1) ... V(nkv-1) M(nkv), one step per phase; group 1 runs it one phase
    // later, so in every phase one wave of each SIMD issues MFMAs while its
    // partner does vector work (one MFMA stream per SIMD at a time runs faster
    // than two interleaved ones).  V(j) also issues the first fragment reads
    // of M(j + 1) from stage j + 1.  Stage s is issued at the start of phase
    // 2s - 6 (stages 0..2 before the loop) into the buffer of stage s - 4,
    // whose last reader ended with phase 2s - 7; stage j + 1 is waited for at
    // the end of phase 2j, before the first vector step that prefetches from
    // it (group 0's V(j), phase 2j + 1).
    auto issue_ahead = [&](int j) {  // phase 2j
        if (j + 3 <= nkv) load_stage(j + 3);
    };
    auto wait_after_even = [&](int j) {  // end of phase 2j: stage j + 1 must land
        if (j + 3 < nkv)
            vm_wait<2 * (KI + VI)>();
        else if (j + 3 == nkv)
            vm_wait<(KI + VI) + VI>();
        else if (j + 2 == nkv)
            vm_wait<VI>();
        else
            vm_wait<0>();
        sync_lds();
    };
    using T0 = std::integral_constant<bool, false>;
    using T1 = std::integral_constant<bool, true>;
    prefetch(0, T0{}, T1{});
    if (grp == 0) {
        issue_ahead(0);
        matrix_step(0, T0{}, T1{});
        wait_after_even(0);
        for (int j = 0; j + 1 < nkv; ++j) {
            vector_step(j);
            prefetch(j + 1, T1{}, T1{});
            sync_lds();
            issue_ahead(j + 1);
            matrix_step(j + 1, T1{}, T1{});
            wait_after_even(j + 1);
        }
        vector_step(nkv - 1);
        prefetch(nkv, T1{}, T0{});
        sync_lds();
        issue_ahead(nkv);
        matrix_step(nkv, T1{}, T0{});
        wait_after_even(nkv);
        sync_lds();
    } else {
        issue_ahead(0);
        wait_after_even(0);
        matrix_step(0, T0{}, T1{});
        sync_lds();
        for (int j = 0; j + 1 < nkv; ++j) {
            issue_ahead(j + 1);
            vector_step(j);
            prefetch(j + 1, T1{}, T1{});
            wait_after_even(j + 1);
            matrix_step(j + 1, T1{}, T1{});
            sync_lds();
        }
        issue_ahead(nkv);
        vector_step(nkv - 1);
        prefetch(nkv, T1{}, T0{});
        wait_after_even(nkv);
        matrix_step(nkv, T1{}, T0{});
        sync_lds();
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
                    if (db * 32 + 8 * rg + 4 * g >= D) continue;  // padding columns
                    f32x4 x;
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = o[db][4 * rg + i];
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
        bf16* oh = static_cast<bf16*>(a.o) + ((size_t)(b * a.Hq + hq) * a.Tq + qrow) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                if (db * 32 + 8 * rg + 4 * g >= D) continue;  // padding columns
                bf16x4 x;
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = (bf16)(o[db][4 * rg + i] * inv);
                *reinterpret_cast<bf16x4*>(oh + db * 32 + 8 * rg + 4 * g) = x;
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
// elements of a row.
template <int D>
__global__ __launch_bounds__(256) void merge_chunks_kernel(const float* opart, const float* ml,
                                                           bf16* o, float* lse, long rows, int S)
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
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = (bf16)(lo[e] * inv);
        x[4 + e] = (bf16)(hi[e] * inv);
    }
    *reinterpret_cast<bf16x8*>(o + row * D + c8) = x;
    if (c8 == 0) lse[row] = (M + log2f(L)) * kLn2;
}

template <int D, bool CAUSAL>
static hipError_t launch_t(const FwdArgs& a, hipStream_t stream)
{
    using Cfg = FwdBf16Cfg<D>;
    static_assert(Cfg::SMEM <= 160 * 1024, "LDS budget");
    auto kern = fwd_bf16_kernel<D, CAUSAL>;
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
                       stream, a.opart, a.ml, static_cast<bf16*>(a.o), a.lse, rows, a.nsplit);
    return hipGetLastError();
}

// Chunks of the key range per query block: about two workgroups per compute
// unit when the query blocks alone are too few, at most 8, and at least 4 key
// tiles per chunk.
int fwd_nsplit(int B, int Hq, int Hkv, int Tq, int Tk, int D)
{
    (void)Hkv;
    (void)D;
    constexpr long kTarget = 512;
    const long wgs = (long)((Tq + 255) / 256) * B * Hq;
    if (wgs <= 0 || wgs >= kTarget) return 1;
    long s = (kTarget + wgs - 1) / wgs;
    s = s < 8 ? s : 8;
    const long tiles = (Tk + 63) / 64;
    const long cap = tiles / 4 > 1 ? tiles / 4 : 1;
    return (int)(s < cap ? s : cap);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int D, bool causal, hipStream_t stream)
{
    if (D == 64) return causal ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
    if (D == 96) return causal ? launch_t<96, true>(a, stream) : launch_t<96, false>(a, stream);
    return causal ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
}

// Every kernel variant is instantiated explicitly: referencing a kernel
// template only from a launcher has left some instantiations without their
// host-side handle.
template __global__ void fwd_bf16_kernel<64, true>(FwdArgs);
template __global__ void fwd_bf16_kernel<64, false>(FwdArgs);
template __global__ void fwd_bf16_kernel<96, true>(FwdArgs);
template __global__ void fwd_bf16_kernel<96, false>(FwdArgs);
template __global__ void fwd_bf16_kernel<128, true>(FwdArgs);
template __global__ void fwd_bf16_kernel<128, false>(FwdArgs);

}  // namespace fa
