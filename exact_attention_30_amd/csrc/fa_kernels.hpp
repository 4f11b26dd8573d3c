// Kernel argument blocks and launcher declarations (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv;
    int Tq, Tk;   // query rows, key rows
    int off;      // causal: query row i sees key j iff j <= i + off (off >= 0)
    float c;      // scale * log2(e): scores are exponentiated in base 2
    float scale;  // for the natural-log lse
    // Split key range: with nsplit > 1, chunk s of a query block's key tiles
    // writes its unnormalised numerator o (fp32, opart[s][B][Hq][Tq][D]) and
    // its reference max and sum (ml[s][B][Hq][Tq][2], base-2 units), and a
    // merge kernel combines the chunks
    float* opart;
    float* ml;
    int nsplit;
    // fp8 forward: descale of V, applied to O (1 for the other element types)
    float vscale;
    // bf16 forward: O (and the merge's O) stored as float32, not rounded to bf16
    int of32 = 0;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse;
    const float* delta;
    void* dq;
    void* dk;
    void* dv;
    int B, Hq, Hkv;
    int Tq, Tk;  // query rows, key rows
    int off;     // causal: query row i sees key j iff j <= i + off (off >= 0)
    float c;     // scale * log2(e)
    float scale;
    // Split work: with nsplit > 1, chunk s of a key block (dK/dV kernel:
    // dK unscaled at part[s][B][Hkv][Tk][D], dV after all of them) or of a
    // query block's key range (dQ kernel: dQ unscaled at part[s][B][Hq][Tq][D])
    // writes fp32 partial sums, and a reduction adds them
    float* part;
    int nsplit;
    // dQ kernel (bf16) only: with delta_out set, it forms Delta of its rows
    // from o and dout itself, reads no delta and writes Delta to delta_out
    const void* o;
    float* delta_out;
    // dK/dV kernel (bf16) only: with kpair set, workgroup m takes key blocks
    // m and nkt - 1 - m (set by its launcher)
    int kpair = 0;
    // bf16 kernels: dQ, dK, dV (and the partial-sum reductions' results)
    // stored as float32, not rounded to bf16
    int gf32 = 0;
};

struct PreArgs {
    const void* o;
    const void* dout;
    float* delta;
    long rows;
};

// Each launcher enqueues one kernel on `stream` and returns the launch status.
// dtype: 0 = bf16, 1 = fp32.  Shapes have been validated by the caller.
hipError_t launch_fwd(const FwdArgs& a, int D, int dtype, bool causal, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdArgs& a, int D, bool causal, hipStream_t stream);
hipError_t launch_bwd_pre(const PreArgs& a, int D, int dtype, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int D, int dtype, bool causal, hipStream_t stream);
// chunks the bf16 dK/dV kernel splits each key block into, and the bf16 dQ
// kernel the key range of each query block into (1: no split)
int dkdv_nsplit(int B, int Hq, int Hkv, int Tq, int Tk, int D);
int dq_nsplit(int B, int Hq, int Hkv, int Tq, int Tk, int D);
// chunks the bf16 forward splits each query block's key range into
int fwd_nsplit(int B, int Hq, int Hkv, int Tq, int Tk, int D);
int fwd_rows(int B, int Hq, int Tq, int D);  // query rows per workgroup, bf16 forward
int dq_rows(int B, int Hq, int Tq, int D);   // query rows per workgroup, bf16 dQ
int dkdv_keys(int B, int Hkv, int Tk, int D);  // keys per workgroup, bf16 dK/dV
hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, int D, bool causal, hipStream_t stream);
// dK/dV with dQ accumulated by atomic adds (bf16, D = 64); a.part: the fp32
// dQ accumulator [B][Hq][Tq][64]
hipError_t launch_bwd_atomic_bf16(const BwdArgs& a, bool causal, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int D, int dtype, bool causal, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const BwdArgs& a, int D, bool causal, hipStream_t stream);
// fp8 (e4m3) forward: a.v is the transposed V that launch_fp8_vt writes
// (tile-major, [B][Hkv][ceil(Tk/64)][D][64 bytes]); D is 64 or 128
hipError_t launch_fp8_vt(const void* v, void* vt, int B, int Hkv, int Tk, int D, hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdArgs& a, int D, bool causal, hipStream_t stream);

}  // namespace fa
