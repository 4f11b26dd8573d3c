// Read-order LDS tiles and explicitly scheduled LDS DMA (gfx950 / CDNA4).
//
// A read-order tile stores a block of K or V rows in exactly the order the
// MFMA operand reads consume it: every read is 64 lanes x 16 bytes (row-wise
// fragments, ds_read_b128) or 64 lanes x 8 bytes (transposed fragments,
// ds_read_b64_tr_b16) of contiguous LDS.  Contiguous lane addresses cannot
// collide on LDS banks, and each read of a tile is one per-lane base register
// plus a compile-time offset, so the hot loops carry no per-fragment address
// registers.  The tiles are filled straight from global memory by
// buffer_load_dwordx4 ... lds: lane L of one such instruction writes bytes
// 16L .. 16L+15 of a 1 KiB LDS block, so the block order fixes, for every
// lane, which 16 global bytes it fetches.
//
// The DMA is issued through inline assembly.  The compiler then does not
// treat these loads as LDS stores that every later LDS read might alias (which
// would make it wait for all outstanding DMA before any LDS read and so stall
// the prefetch of the next tiles); instead the kernels wait explicitly, with
// `vm_wait<N>`, for exactly the loads whose data they are about to read, and
// order LDS accesses around workgroup barriers with `sync_lds`.  Loads return
// in issue order, so waiting until at most N loads are outstanding completes
// every load issued before the last N.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"

namespace fa {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at `base` (wave-uniform): reads at
// offsets at or past `bytes` return zeros.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int bytes)
{
    const uint64_t addr = (uint64_t)(uintptr_t)base;
    // the words must sit in scalar registers; readfirstlane states that they
    // are uniform where the compiler cannot prove it
    return i32x4{__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)addr),
                 __builtin_amdgcn_readfirstlane((int32_t)((addr >> 32) & 0xffff)),
                 __builtin_amdgcn_readfirstlane(bytes), kBufferFlags};
}

// LDS tile width of the backward kernels, whose swizzled tiles need a
// power-of-two number of 16-byte chunks per row: D = 96 is stored 128 wide,
// columns D .. tile_dim(D) - 1 zeros that no product reads and no store
// writes.  (The forward's read-order tiles take D itself.)
__host__ __device__ constexpr int tile_dim(int D) { return D == 96 ? 128 : D; }

// Byte offset fetched for element (row, col) of a [rows][DS] bf16 array: a
// padding column (col >= DS) gets an offset past any buffer range, so the
// buffer load returns zeros there.
constexpr uint32_t kPastEnd = 0x80000000u;
__device__ __forceinline__ constexpr uint32_t elem_off(int row, int col, int ds)
{
    return col < ds ? (uint32_t)((row * ds + col) * 2) : kPastEnd;
}

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One LDS DMA instruction: this lane's 16 bytes at byte `voff` of the buffer
// land at LDS byte lds + 16 * lane.  `lds` must be wave-uniform.
__device__ __forceinline__ void dma_b128(uint32_t lds, const i32x4& rsrc, uint32_t voff)
{
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds)
                 : "memory");
}

// The same DMA without the memory clobber, for loads issued between the
// products of an iteration: the compiler may then keep LDS reads of other
// buffers where they are scheduled.  The destination must not be read before
// a later `vm_wait` and `sync_lds`, whose clobbers order it.
__device__ __forceinline__ void dma_b128_nofence(uint32_t lds, const i32x4& rsrc, uint32_t voff)
{
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds));
}

// Where an iteration of a forward kernel (two stages per barrier) issues
// its stage loads: kIssueBarrier, both stages of the next pair at an even
// iteration's barrier; kIssueEven / kIssueOdd, stage i + 2 spread over the
// products of an even / odd iteration; kIssueTop, at the top of an iteration
// whose parity is known only at run time.
enum { kIssueBarrier = 0, kIssueEven = 1, kIssueOdd = 2, kIssueTop = 3 };

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that also retires this wave's LDS reads (so no read of a
// buffer is in flight when another wave overwrites it after the barrier) but
// does not wait for outstanding global loads.  The asm statements are
// compiler barriers for memory accesses.
__device__ __forceinline__ void sync_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// Row-wise fragments of a ROWS x D bf16 block (A operand of S^T = K Q^T):
// fragment (kb, ks) gives lane (g, c) row 32kb + c, columns 16ks + 8g .. +7.
// ---------------------------------------------------------------------------
template <int D, int ROWS, int DS = D>
struct RowFragTile {
    static constexpr int NKS = D / 16;
    static constexpr int NKB = ROWS / 32;
    static constexpr int NDMA = NKB * NKS;  // 1 KiB blocks = DMA instructions
    static constexpr int BYTES = NDMA * 1024;

    __device__ __forceinline__ static constexpr int frag_off(int kb, int ks) { return (kb * NKS + ks) * 1024; }

    // global byte offset (within the block's first row) fetched by `lane` for
    // DMA instruction f
    __device__ __forceinline__ static uint32_t dma_off(int f, int lane)
    {
        const int kb = f / NKS, ks = f % NKS;
        const int row = 32 * kb + (lane & 31), col = 16 * ks + 8 * (lane >> 5);
        return elem_off(row, col, DS);
    }

    // lane's fragment (kb, ks) of the tile at `tile` (lane offset included by
    // the caller: tile + 16 * lane)
    __device__ __forceinline__ static bf16x8 read(const unsigned char* tile_lane, int kb, int ks)
    {
        return *reinterpret_cast<const bf16x8*>(tile_lane + frag_off(kb, ks));
    }
};

// ---------------------------------------------------------------------------
// Transposed fragments of a ROWS x D bf16 block (A operand of O^T += V^T P^T):
// for the 16-row step ts and column block db, lane (g, c) receives elements
// e = 0..7 = V[16ts + 8(e/4) + 4g + e%4][32db + c], the row order in which the
// S^T accumulator registers are reused as the B operand.  Each step is two
// ds_read_b64_tr_b16 (h = e/4), each reading a 512-byte block.  Within 16
// lanes that instruction gives lane i element i%4 of the 8 bytes addressed by
// lane 4e + i/4 (e = 0..3); so in block (ts, db, h), lane 16m + a holds the 8
// bytes V[16ts + 8h + 4(m/2) + a/4][32db + 16(m%2) + 4(a%4) .. +3].
// ---------------------------------------------------------------------------
template <int D, int ROWS, int DS = D>
struct TrFragTile {
    static constexpr int NTS = ROWS / 16;
    static constexpr int NDB = D / 32;
    static constexpr int NDMA = NTS * NDB;  // one 1 KiB block = both halves
    static constexpr int BYTES = NDMA * 1024;

    __device__ __forceinline__ static constexpr int block_off(int ts, int db, int h)
    {
        return ((ts * NDB + db) * 2 + h) * 512;
    }

    // DMA instruction f = ts * NDB + db: lane L fills bytes 16(L%32) .. +15 of
    // half h = L/32, i.e. the words of reading lanes 2s and 2s + 1 (s = L%32):
    // 8 consecutive elements of one row.
    __device__ __forceinline__ static uint32_t dma_off(int f, int lane)
    {
        const int ts = f / NDB, db = f % NDB;
        const int h = lane >> 5, s = lane & 31;
        const int row = 16 * ts + 8 * h + 4 * (s >> 4) + ((s & 7) >> 1);
        const int col = 32 * db + 16 * ((s >> 3) & 1) + 8 * (s & 1);
        return elem_off(row, col, DS);
    }

    // lane's fragment for step ts, column block db (tile_lane = tile + 8 * lane)
    __device__ __forceinline__ static bf16x8 read(const unsigned char* tile_lane, int ts, int db)
    {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(tile_lane + block_off(ts, db, 0)));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(tile_lane + block_off(ts, db, 1)));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

}  // namespace fa

namespace fa {

// One LDS DMA instruction of 4 bytes per lane: this lane's dword at byte
// `voff` of the buffer lands at LDS byte lds + 4 * lane.
__device__ __forceinline__ void dma_b32(uint32_t lds, const i32x4& rsrc, uint32_t voff)
{
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds)
                 : "memory");
}

// A ROWS x D bf16 block in natural [row][col] order with the chunk swizzle of
// DmaTile (row-wise and transposed reads both conflict-free), filled by the
// explicitly scheduled DMA above; NT threads share the instructions.  The
// rows come from a [nrows][DS] array (DS <= D; columns DS .. D-1 are zeros).
template <int D, int ROWS, int NT, int DS = D>
struct SwzTile {
    using Base = DmaTile<bf16, D, ROWS, NT>;
    static constexpr int NI = Base::NI;
    static constexpr int BYTES = Base::BYTES;
    static constexpr int CPR = Base::CPR;  // 16-byte chunks per tile row
    uint32_t voff[NI];

    // the chunk stored at each of this thread's DMA positions (the swizzle of
    // DmaTile) and the global bytes it comes from
    __device__ __forceinline__ void init(int tid)
    {
        const int lane = tid & 63, w = tid >> 6;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int p = (i * (NT / 64) + w) * 64 + lane;  // chunk position in the tile
            const int row = p / CPR;
            const int ch = (p % CPR) ^ fa::swz<CPR>(row);
            voff[i] = elem_off(row, ch * 8, DS);
        }
    }

    // rows row0 .. row0 + ROWS - 1 of a [nrows][DS] array into the tile at LDS
    // byte address `lds`; rows past nrows read as zeros.  w: this wave's index.
    __device__ __forceinline__ void load(uint32_t lds, const bf16* head, int row0, int nrows, int w) const
    {
        const int left = nrows - row0;
        const i32x4 r = buffer_rsrc(head + (size_t)row0 * DS, left > 0 ? left * DS * 2 : 0);
#pragma unroll
        for (int i = 0; i < NI; ++i) dma_b128(lds + (uint32_t)((i * (NT / 64) + w) * 1024), r, voff[i]);
    }
};

}  // namespace fa

namespace fa {

// Empty asm through which a value passes: the computation of an input or
// output cannot move across it, and such statements keep their order among
// themselves and with scheduling barriers.  Used to place vector work between
// matrix instructions in a fixed order.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(bf16x8& x) { asm volatile("" : "+v"(x)); }

// Empty asm that reads a register value loaded from global memory: the
// compiler's wait for that load is placed before this point.  Called once
// before a loop, it keeps the compiler from waiting at the value's first use
// inside the loop, where its s_waitcnt vmcnt(0) would also drain the
// explicitly issued LDS DMA of the tiles ahead on every pass.
__device__ __forceinline__ void settle(const bf16x8& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void settle(float x) { asm volatile("" ::"v"(x)); }

// Two floats rounded to nearest even bf16, packed (first in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(bf16)lo, (bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

}  // namespace fa

namespace fa {

// Reads at a 32-bit LDS byte address.  A compile-time constant added to the
// address becomes the instruction's 16-bit immediate offset.
__device__ __forceinline__ bf16x8 lds_b128(uint32_t addr)
{
    return *(const __attribute__((address_space(3))) bf16x8*)addr;
}
__device__ __forceinline__ bf16x4 lds_tr_b64(uint32_t addr)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)addr);
}

// Operand fragments of bf16 blocks stored in the swizzled row format `Tile`
// (DmaTile) inside one LDS region.  The region's address is folded into the
// per-lane addresses once, and an empty asm hides where they came from, so
// the compiler cannot re-derive them from the LDS symbol at every read (it
// would add the base again per read); each read is then one address register
// plus an immediate (block, stage and row offsets, below 64 KiB).
//
// SwzRowFrags: fragment ks of rows rowbase + c, columns 16ks + 8g .. +7
// (A or B operand, one ds_read_b128).
template <class Tile, int D>
struct SwzRowFrags {
    static constexpr int NKS = D / 16;
    uint32_t addr[NKS];

    __device__ __forceinline__ void init(uint32_t region, int c, int g)
    {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            addr[ks] = region + (uint32_t)Tile::offset(c, 16 * ks + 8 * g);
            asm volatile("" : "+v"(addr[ks]));
        }
    }
    // imm: byte offset of the block in the region + rowbase * ROWBYTES
    // (rowbase a multiple of 16, so the swizzle of row c applies)
    __device__ __forceinline__ bf16x8 read(int ks, uint32_t imm) const { return lds_b128(addr[ks] + imm); }
};

// SwzTrFrags: transposed fragment (A operand of a product that contracts over
// rows): lane (g, c) receives the elements (rowbase + 8(e/4) + 4g + e%4,
// 32db + c), e = 0..7, as two ds_read_b64_tr_b16 (see TrReader).
template <class Tile, int D>
struct SwzTrFrags {
    static constexpr int NDB = D / 32;
    uint32_t addr[NDB][2];

    __device__ __forceinline__ void init(uint32_t region, int lane)
    {
        const int m = lane >> 4, j = lane & 15;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                addr[db][h] = region + (uint32_t)Tile::offset(8 * h + 4 * (m >> 1) + (j >> 2),
                                                              db * 32 + 16 * (m & 1) + 4 * (j & 3));
                asm volatile("" : "+v"(addr[db][h]));
            }
    }
    // imm: byte offset of the block in the region + rowbase * ROWBYTES
    // (rowbase a multiple of 16)
    __device__ __forceinline__ bf16x8 read(int db, uint32_t imm) const
    {
        const bf16x4 lo = lds_tr_b64(addr[db][0] + imm);
        const bf16x4 hi = lds_tr_b64(addr[db][1] + imm);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

}  // namespace fa
