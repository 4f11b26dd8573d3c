// Device building blocks shared by the attention kernels (gfx950 / CDNA4).
//
// Matrix products use the 32x32 MFMA shape with fp32 accumulators:
//   bf16: v_mfma_f32_32x32x16_bf16 (one instruction per 16-deep step)
//   fp32: v_mfma_f32_32x32x2_f32   (eight instructions per 16-deep step)
// Register layouts of a 64-lane wave (lane = 32*g + c, g in {0,1}, c in 0..31):
//   A operand (32 x K):  lane holds A[c][8g .. 8g+7] of each 16-deep step
//   B operand (K x 32):  lane holds B[8g .. 8g+7][c]
//   accumulator (32x32): register r holds C[8*(r/4) + 4g + r%4][c]
// A "fragment" below is the 8 contraction elements one lane feeds to one
// 16-deep step.  Because the contraction index of a product may be permuted
// freely (as long as both operands use the same permutation), the
// accumulator of one product can feed the B operand of the next product
// without leaving registers: register r = 8t + e of a 32-row accumulator block
// becomes element e of the fragment for step t, which stands for contraction
// row 16t + 8*(e/4) + 4g + e%4.  The partner operand is then read from a
// tile stored with rows permuted by `perm16` (swap bits 2 and 3), so that the
// same 8 elements are contiguous in LDS.
//
// This is the MFMA form of the register-resident weights that "L'attention
// fusionnée" describes for mma.sync in «Sur les Tensor Cores».
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
// Word 3 of a raw buffer resource on gfx9-family chips (no swizzle, dword
// data format); with a zero stride, reads at or past num_records return 0.
constexpr int kBufferFlags = 0x00020000;
constexpr float kLn2 = 0.6931471805599453f;

template <class E>
struct Frag;
template <>
struct Frag<bf16> {
    bf16x8 v;
};
template <>
struct Frag<float> {
    f32x8 v;
};

// acc += A_frag x B_frag over one 16-deep contraction step.
__device__ __forceinline__ void mma(f32x16& acc, const Frag<bf16>& a, const Frag<bf16>& b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& acc, const Frag<float>& a, const Frag<float>& b)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// 8 contiguous elements of row `row` of a [nrows][D] global array, or zeros
// when the row is past the end.
template <class E>
__device__ __forceinline__ Frag<E> global_frag(const E* base, int row, int nrows, int D, int col)
{
    Frag<E> f;
    if (row < nrows && col < D) {  // rows past nrows and padding columns read as zeros
        const E* p = base + (size_t)row * D + col;
        if constexpr (sizeof(E) == 2) {
            f.v = *reinterpret_cast<const bf16x8*>(p);
        } else {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
            f.v = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    } else {
        if constexpr (sizeof(E) == 2) {
            f.v = bf16x8{};
        } else {
            f.v = f32x8{};
        }
    }
    return f;
}

// Registers 8t .. 8t+7 of an accumulator block as a B-operand fragment
// (rounded to nearest even for bf16).
template <class E>
__device__ __forceinline__ Frag<E> acc_frag(const f32x16& s, int t);
template <>
__device__ __forceinline__ Frag<bf16> acc_frag<bf16>(const f32x16& s, int t)
{
    Frag<bf16> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = (bf16)s[8 * t + e];
    return f;
}
template <>
__device__ __forceinline__ Frag<float> acc_frag<float>(const f32x16& s, int t)
{
    Frag<float> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = s[8 * t + e];
    return f;
}

// acc + the sum of a fragment's 8 elements (bf16: four v_dot2 with ones, so
// the sum is of the rounded values).
__device__ __forceinline__ float frag_sum(const Frag<bf16>& f, float acc)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {f.v[e], f.v[e + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, acc, false);
    }
    return acc;
}
__device__ __forceinline__ float frag_sum(const Frag<float>& f, float acc)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += f.v[e];
    return acc;
}

// Row permutation of transposed tiles inside each group of 16: swap bits 2, 3.
__device__ __forceinline__ constexpr int perm16(int r)
{
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Combine a value of lane c with the value of lane c ^ 32 (the two lanes of a
// wave that hold the same accumulator column).  v_permlane32_swap exchanges
// the upper half of its first operand with the lower half of its second; with
// both operands equal to x, element 0 of the result holds x of lane c - 32 in
// the upper lanes (x itself below) and element 1 holds x of lane c + 32 in the
// lower lanes (x itself above).  The lower lane's value always comes first,
// so both lanes compute bit-identical sums.
__device__ __forceinline__ float pair_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Tiles loaded straight from global memory into LDS (global_load_lds_dwordx4:
// each lane of a wave moves one 16-byte chunk; lane L of an instruction lands
// at byte 16*L of a 1 KiB LDS block whose base the instruction names).  No
// registers are involved, so the next tile streams in while the current one
// is used.  A tile is ROWS rows of D elements kept in natural [row][col]
// order; the 16-byte chunks of each row are XOR-swizzled so that the reads
// below hit distinct LDS banks.  Rows past the end of the sequence are loaded
// as copies of the last row: finite values that the masks then exclude.
// ---------------------------------------------------------------------------
template <class E, int D>
struct RowFmt {
    static constexpr int CH = 16 / (int)sizeof(E);  // elements per chunk
    static constexpr int CPR = D / CH;              // chunks per row
    static_assert(CPR >= 8, "rows must hold at least 8 chunks");
};

// Chunk swizzle of tile rows.  Two read patterns must both spread over the
// LDS banks, whether a cycle serves 128 or 256 bytes:
//   * fragment reads: consecutive rows, one chunk each (ds_read_b128);
//   * transposed reads: 4 aligned consecutive rows, 2 or 4 adjacent chunks
//     (an aligned block) per 16 or 32 lanes (ds_read_b64_tr_b16).
// With i = r % 4, f(r) = 4i + 2(((i/2) ^ (r/8)) % 2) + (r/4) % 2 is distinct
// over 16 consecutive rows (and over 8 modulo 8), while over 4 aligned rows
// both f/2 % 4 and f/4 % 4 are distinct.  Rows of 8 chunks use it modulo 8.
template <int CPR>
__device__ __forceinline__ constexpr int swz(int row)
{
    const int i = row & 3;
    return (4 * i + 2 * (((i >> 1) ^ (row >> 3)) & 1) + ((row >> 2) & 1)) & (CPR - 1);
}

template <class E, int D, int ROWS, int NT>
struct DmaTile {
    using F = RowFmt<E, D>;
    static constexpr int CPR = F::CPR;
    static constexpr int NCH = ROWS * CPR;  // chunks per tile
    static_assert(NCH % NT == 0, "tile chunks must divide over the threads");
    static_assert(ROWS % 16 == 0, "tiles hold whole swizzle periods");
    static constexpr int NI = NCH / NT;     // instructions per thread
    static constexpr int BYTES = ROWS * D * (int)sizeof(E);
    static constexpr int ROWBYTES = CPR * 16;

    // Byte offset in the tile of element (row, col).
    __device__ __forceinline__ static constexpr int offset(int row, int col)
    {
        const int ch = col / F::CH;
        return (row * CPR + (ch ^ fa::swz<CPR>(row))) * 16 + (col % F::CH) * (int)sizeof(E);
    }

    // Per-thread byte offsets (into the global rows of a tile) of the chunks
    // this thread moves; the same for every tile.
    uint32_t voff[NI];

    __device__ __forceinline__ void init(int tid)
    {
        const int lane = tid & 63, w = tid >> 6;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int p = (i * (NT / 64) + w) * 64 + lane;  // chunk position in the tile
            const int row = p / CPR;
            const int ch = (p % CPR) ^ fa::swz<CPR>(row);   // global chunk stored there
            voff[i] = (uint32_t)((row * D + ch * F::CH) * (int)sizeof(E));
        }
    }

    // Issue the loads of rows row0 .. row0+ROWS-1 of a [nrows][D] array; rows
    // past nrows read as zeros (buffer range check).  w: this wave's index
    // (wave-uniform).
    __device__ __forceinline__ void load(unsigned char* lds_tile, const E* head, int row0,
                                         int nrows, int w) const
    {
        const int left = nrows - row0;
        const int bytes = left > 0 ? left * D * (int)sizeof(E) : 0;
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(head + (size_t)row0 * D), (short)0, bytes, kBufferFlags);
#pragma unroll
        for (int i = 0; i < NI; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)(lds_tile + (i * (NT / 64) + w) * 1024),
                16, voff[i], 0, 0, 0);
    }
};

// Wait for this thread's outstanding global loads (including LDS-bound ones).
__device__ __forceinline__ void wait_global_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Row-wise fragment reads from a DMA tile: lane (g, c) reads the 8 elements
// at columns 16ks + 8g .. +7 of row rowbase + rowlane (rowbase a multiple of
// 16).  The per-lane byte offsets are computed once; in the loop a read is one
// LDS instruction with a constant offset.
template <class Tile, class E, int D>
struct RowReader {
    static constexpr int NKS = D / 16;
    static constexpr int NC = 8 * (int)sizeof(E) / 16;  // 16-byte chunks per fragment
    uint32_t off[NKS][NC];

    __device__ __forceinline__ void init(int rowlane, int g)
    {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int h = 0; h < NC; ++h)
                off[ks][h] = (uint32_t)Tile::offset(rowlane, 16 * ks + 8 * g + 8 * h / NC);
    }

    __device__ __forceinline__ Frag<E> frag(const unsigned char* tile, int rowbase, int ks) const
    {
        const unsigned char* t = tile + rowbase * Tile::ROWBYTES;
        Frag<E> f;
        if constexpr (sizeof(E) == 2) {
            f.v = *reinterpret_cast<const bf16x8*>(t + off[ks][0]);
        } else {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(t + off[ks][0]);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(t + off[ks][1]);
            f.v = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        return f;
    }
};

// A-operand fragment of a transposed product, read from a natural tile:
// lane (g, c) receives element (rows k(e), column 32db + c) for the 8
// contraction rows k(e) = rowbase + 8*(e/4) + 4g + e%4, the row order of the
// accumulator-to-operand reuse described at the top of this file (rowbase a
// multiple of 16).
//
// bf16: two ds_read_b64_tr_b16.  Within each group of 16 lanes that
// instruction hands lane i element (i % 4) of the 8 bytes addressed by lane
// 4e + i/4 of the group, for e = 0..3.  Lane 16m + j therefore addresses row
// rowbase + 8h + 4(m/2) + j/4 at column 32db + 16(m%2) + 4(j%4), and the 16
// lanes of the group receive 4 rows at 16 consecutive columns.
// fp32: eight single-element reads.
template <class Tile, class E, int D>
struct TrReader {
    static constexpr int NDB = D / 32;
    static constexpr int NO = sizeof(E) == 2 ? 2 : 8;
    uint32_t off[NDB][NO];

    __device__ __forceinline__ void init(int lane)
    {
        if constexpr (sizeof(E) == 2) {
            const int m = lane >> 4, j = lane & 15;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    off[db][h] = (uint32_t)Tile::offset(8 * h + 4 * (m >> 1) + (j >> 2),
                                                        db * 32 + 16 * (m & 1) + 4 * (j & 3));
        } else {
            const int g = lane >> 5, c = lane & 31;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    off[db][e] = (uint32_t)Tile::offset(8 * (e >> 2) + 4 * g + (e & 3), db * 32 + c);
        }
    }

    __device__ __forceinline__ Frag<E> frag(const unsigned char* tile, int rowbase, int db) const
    {
        const unsigned char* t = tile + rowbase * Tile::ROWBYTES;
        Frag<E> f;
        if constexpr (sizeof(E) == 2) {
            // (whole-vector results only: extracting single elements of the
            // transposed load's result has been miscompiled)
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(t + off[db][0]));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(t + off[db][1]));
            f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) f.v[e] = *reinterpret_cast<const float*>(t + off[db][e]);
        }
        return f;
    }
};

// ---------------------------------------------------------------------------
// Work mapping.  Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup id w runs on XCD w % 8).  When the number of kv groups
// (B * Hkv) is a multiple of 8, every XCD gets whole kv groups, so the query
// heads that share K/V also share that XCD's L2; inside an XCD, tiles are
// handed out heaviest first (for causal attention the last query tiles see the
// most keys).  Otherwise tiles are handed out heaviest first over all heads.
// `ntile` = tiles per head; `heavy_first_desc` says whether the heaviest tile
// has the largest index.
// ---------------------------------------------------------------------------
struct TileId {
    int b, h, tile;  // h: query head (per-query-tile kernels) or kv head
};

__device__ __forceinline__ TileId map_tile(int wg, int B, int Hq, int Hkv, int heads_per_group,
                                           int ntile, bool heavy_last_index)
{
    // heads_per_group: how many work heads share one kv head (Hq/Hkv for
    // query-tile kernels, 1 for key-tile kernels); total heads = Hkv * hpg.
    const int ngroups = B * Hkv;
    TileId id;
    int rank, grp, sub;
    if ((ngroups & 7) == 0) {
        const int x = wg & 7, s = wg >> 3;
        const int per = (ngroups >> 3) * heads_per_group;  // items per tile rank on one XCD
        rank = s / per;
        const int rem = s % per;
        grp = (rem / heads_per_group) * 8 + x;
        sub = rem % heads_per_group;
    } else {
        const int per = ngroups * heads_per_group;
        rank = wg / per;
        const int rem = wg % per;
        grp = rem / heads_per_group;
        sub = rem % heads_per_group;
    }
    id.b = grp / Hkv;
    id.h = (grp % Hkv) * heads_per_group + sub;
    id.tile = heavy_last_index ? (ntile - 1 - rank) : rank;
    (void)Hq;
    return id;
}

}  // namespace fa
