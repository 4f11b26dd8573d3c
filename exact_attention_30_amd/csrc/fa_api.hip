// C ABI of the library: argument checks on the host, then kernel launches on
// the caller's stream.  No device memory is allocated here and no host
// synchronisation is done.  The contract is stated in include/fa.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_kernels.hpp"

// Workspace of fa_bwd_noalloc: one copy on every GPU the library runs on.  In
// host code this name is only a handle for hipGetSymbolAddress; kernels get
// the device address it returns.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape and option checks shared by every entry point; `D`/`dt` may be
// ignored by passing D = 64, dt = FA_BF16.  Tq query rows against Tk key rows;
// `off` (causal only) places query row i at key position i + off.
// bf16 inputs: the bf16 kernels, whose results are rounded to bf16 (FA_BF16)
// or stored as float32 (FA_BF16_F32OUT)
bool bf16_in(fa_dtype dt) { return dt == FA_BF16 || dt == FA_BF16_F32OUT; }

fa_status check_kv(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt, bool causal, int off)
{
    if (B < 0 || Tq < 0 || Tk < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FA_ERR_SHAPE;
    // query rows need at least one key
    if ((long long)B * Tq > 0 && Tk == 0) return FA_ERR_SHAPE;
    // every row sees key 0, and every key index a kernel forms fits an int
    if (causal && (off < 0 || (long long)off + Tq > 0x7fffffffLL - 4096)) return FA_ERR_SHAPE;
    // every tensor index must fit the 64-bit offsets and every grid the
    // 32-bit workgroup count: B*H*ceil(T/32) workgroups at most
    const long long qrows = (long long)B * Hq * (((long long)Tq + 31) / 32);
    const long long krows = (long long)B * Hkv * (((long long)Tk + 31) / 32);
    if (qrows > 0x7fffffffLL || krows > 0x7fffffffLL) return FA_ERR_SHAPE;
    if (dt != FA_BF16 && dt != FA_FP32 && dt != FA_BF16_F32OUT) return FA_ERR_UNSUPPORTED;
    // 64 and 128 in both types; 96 in bf16 (the forward on 96-column tiles,
    // the backward on 128-column LDS tiles whose last 32 columns read as zero)
    if (D != 64 && D != 128 && !(D == 96 && bf16_in(dt))) return FA_ERR_UNSUPPORTED;
    // one head of one tensor is addressed through a buffer resource whose
    // byte range is a signed 32-bit count (the float32 outputs of
    // FA_BF16_F32OUT held to the same bound)
    const long long esz = dt == FA_BF16 ? 2 : 4;
    if ((long long)Tq * D * esz > 0x7fffffffLL || (long long)Tk * D * esz > 0x7fffffffLL)
        return FA_ERR_SHAPE;
    return FA_OK;
}

fa_status check_scale(float scale)
{
    return (isfinite(scale) && scale > 0.f) ? FA_OK : FA_ERR_UNSUPPORTED;
}

fa_status from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// kernel family: 0 the bf16 kernels, 1 the fp32 kernels
int dtype_code(fa_dtype dt) { return bf16_in(dt) ? 0 : 1; }

void fill_bwd(fa::BwdArgs& a, const void* q, const void* k, const void* v, const void* dout,
              const float* lse, const float* delta, int B, int Hq, int Hkv, int Tq, int Tk,
              int off, float scale)
{
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.lse = lse;
    a.delta = delta;
    a.dq = a.dk = a.dv = nullptr;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Tq = Tq;
    a.Tk = Tk;
    a.off = off;
    a.c = scale * kLog2e;
    a.scale = scale;
    a.part = nullptr;
    a.nsplit = 1;
    a.o = nullptr;
    a.delta_out = nullptr;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// bytes of fp32 partial sums the split dK/dV stage uses (0: no split)
size_t split_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt)
{
    if (!bf16_in(dt) || (long long)B * Tk == 0) return 0;
    const int S = fa::dkdv_nsplit(B, Hq, Hkv, Tq, Tk, D);
    if (S <= 1) return 0;
    return align256((size_t)2 * S * (size_t)B * Hkv * (size_t)Tk * D * sizeof(float));
}

// bytes of fp32 partial sums the split dQ stage uses (0: no split)
size_t dq_split_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt)
{
    if (!bf16_in(dt) || (long long)B * Tq == 0) return 0;
    const int S = fa::dq_nsplit(B, Hq, Hkv, Tq, Tk, D);
    if (S <= 1) return 0;
    return align256((size_t)S * (size_t)B * Hq * (size_t)Tq * D * sizeof(float));
}

// the split stages of one backward run one after the other: they share one
// partial-sum region of the larger size
size_t shared_split_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt)
{
    const size_t a = split_bytes(B, Hq, Hkv, Tq, Tk, D, dt);
    const size_t b = dq_split_bytes(B, Hq, Hkv, Tq, Tk, D, dt);
    return a > b ? a : b;
}

}  // namespace

namespace {

// Device address of `scratch` on each device, looked up once per device with
// that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices] = {};

fa_status scratch_address(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_version(void) { return "0.3.0"; }

const char* fa_status_string(fa_status s)
{
    switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer";
    case FA_ERR_SHAPE: return "invalid shape";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or scale";
    case FA_ERR_ALIGN: return "misaligned pointer";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_SCRATCH: return "workspace larger than the static scratch of fa_bwd_noalloc";
    }
    return "unknown status";
}

// bytes of the forward's chunk partials: numerators, then (max, sum) pairs
size_t fwd_split_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt)
{
    if (!bf16_in(dt) || (long long)B * Tq == 0) return 0;
    const int S = fa::fwd_nsplit(B, Hq, Hkv, Tq, Tk, D);
    if (S <= 1) return 0;
    const size_t rows = (size_t)S * B * Hq * Tq;
    return align256(rows * D * sizeof(float)) + align256(rows * 2 * sizeof(float));
}

fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                       void* partial, int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale,
                       int causal, int q_offset, fa_dtype dt, void* stream)
{
    const int off = causal ? q_offset : 0;
    fa_status st = check_kv(B, Hq, Hkv, Tq, Tk, D, dt, causal != 0, off);
    if (st != FA_OK) return st;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if ((long long)B * Tq == 0) return FA_OK;
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
        !aligned(partial, 16))
        return FA_ERR_ALIGN;
    fa::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Tq = Tq;
    a.Tk = Tk;
    a.off = off;
    a.c = scale * kLog2e;
    a.scale = scale;
    a.opart = a.ml = nullptr;
    a.nsplit = 1;
    a.vscale = 1.f;
    a.of32 = dt == FA_BF16_F32OUT;
    if (partial && fwd_split_bytes(B, Hq, Hkv, Tq, Tk, D, dt) > 0) {
        a.nsplit = fa::fwd_nsplit(B, Hq, Hkv, Tq, Tk, D);
        const size_t rows = (size_t)a.nsplit * B * Hq * Tq;
        a.opart = static_cast<float*>(partial);
        a.ml = reinterpret_cast<float*>(static_cast<char*>(partial) + align256(rows * D * sizeof(float)));
    }
    return from_hip(fa::launch_fwd(a, D, dtype_code(dt), causal != 0, static_cast<hipStream_t>(stream)));
}

size_t fa_fwd_split_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt)
{
    if (check_kv(B, Hq, Hkv, Tq, Tk, D, dt, false, 0) != FA_OK) return 0;
    return fwd_split_bytes(B, Hq, Hkv, Tq, Tk, D, dt);
}

int fa_block_rows(fa_stage stage, int B, int H, int T, int D, fa_dtype dt)
{
    if (check_kv(B, H, H, T, T, D, dt, false, 0) != FA_OK) return 0;
    switch (stage) {
    case FA_STAGE_FWD: return bf16_in(dt) ? fa::fwd_rows(B, H, T, D) : 128;
    case FA_STAGE_DQ: return bf16_in(dt) ? fa::dq_rows(B, H, T, D) : 128;
    case FA_STAGE_DKDV: return bf16_in(dt) ? fa::dkdv_keys(B, H, T, D) : 128;
    }
    return 0;
}

fa_status fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                    int Hkv, int Tq, int Tk, int D, float scale, int causal, int q_offset,
                    fa_dtype dt, void* stream)
{
    return fa_fwd_split(q, k, v, o, lse, nullptr, B, Hq, Hkv, Tq, Tk, D, scale, causal, q_offset,
                        dt, stream);
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                 int Hkv, int T, int D, float scale, int causal, fa_dtype dt, void* stream)
{
    return fa_fwd_kv(q, k, v, o, lse, B, Hq, Hkv, T, T, D, scale, causal, 0, dt, stream);
}

// ---------------------------------------------------------------------------
// FP8 (e4m3) forward

size_t fa_fwd_fp8_workspace_bytes(int B, int Hkv, int Tk, int D)
{
    if (B < 0 || Hkv < 1 || Tk < 0 || (D != 64 && D != 128)) return 0;
    return (size_t)B * (size_t)Hkv * (size_t)((Tk + 63) / 64) * 64 * (size_t)D;
}

fa_status fa_fp8_transpose_v(const void* v, void* vt, int B, int Hkv, int Tk, int D, void* stream)
{
    if (B < 0 || Hkv < 1 || Tk < 0) return FA_ERR_SHAPE;
    if ((long long)B * Hkv * ((Tk + 63) / 64) > 0x7fffffffLL || (long long)Tk * D > 0x7fffffffLL)
        return FA_ERR_SHAPE;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * Tk == 0) return FA_OK;
    if (!v || !vt) return FA_ERR_NULL;
    if (!aligned(v, 16) || !aligned(vt, 16)) return FA_ERR_ALIGN;
    return from_hip(fa::launch_fp8_vt(v, vt, B, Hkv, Tk, D, static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_fp8_vt(const void* q, const void* k, const void* vt, float q_descale,
                        float k_descale, float v_descale, void* o, float* lse, int B, int Hq,
                        int Hkv, int Tq, int Tk, int D, float scale, int causal, int q_offset,
                        void* stream)
{
    const int off = causal ? q_offset : 0;
    // shape rules of the bf16 forward (a bf16 head bounds an fp8 head too)
    fa_status st = check_kv(B, Hq, Hkv, Tq, Tk, D, FA_BF16, causal != 0, off);
    if (st != FA_OK) return st;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((st = check_scale(scale)) != FA_OK || (st = check_scale(q_descale)) != FA_OK ||
        (st = check_scale(k_descale)) != FA_OK || (st = check_scale(v_descale)) != FA_OK)
        return st;
    if ((long long)B * Tq == 0) return FA_OK;
    if (!q || !k || !vt || !o || !lse) return FA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(vt, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    fa::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = vt;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Tq = Tq;
    a.Tk = Tk;
    a.off = off;
    a.c = scale * q_descale * k_descale * kLog2e;
    a.scale = scale * q_descale * k_descale;
    a.opart = a.ml = nullptr;
    a.nsplit = 1;
    a.vscale = v_descale;
    return from_hip(fa::launch_fwd_fp8(a, D, causal != 0, static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, float q_descale, float k_descale,
                     float v_descale, void* o, float* lse, void* workspace, int B, int Hq, int Hkv,
                     int Tq, int Tk, int D, float scale, int causal, int q_offset, void* stream)
{
    const int off = causal ? q_offset : 0;
    fa_status st = check_kv(B, Hq, Hkv, Tq, Tk, D, FA_BF16, causal != 0, off);
    if (st != FA_OK) return st;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if ((st = check_scale(scale)) != FA_OK || (st = check_scale(q_descale)) != FA_OK ||
        (st = check_scale(k_descale)) != FA_OK || (st = check_scale(v_descale)) != FA_OK)
        return st;
    if ((long long)B * Tq == 0) return FA_OK;
    if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
        !aligned(workspace, 16))
        return FA_ERR_ALIGN;
    if ((st = fa_fp8_transpose_v(v, workspace, B, Hkv, Tk, D, stream)) != FA_OK) return st;
    return fa_fwd_fp8_vt(q, k, workspace, q_descale, k_descale, v_descale, o, lse, B, Hq, Hkv, Tq, Tk,
                         D, scale, causal, q_offset, stream);
}

size_t fa_bwd_kv_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt)
{
    if (check_kv(B, Hq, Hkv, Tq, Tk, D, dt, false, 0) != FA_OK) return 0;
    return align256((size_t)B * (size_t)Hq * (size_t)Tq * sizeof(float)) +
           shared_split_bytes(B, Hq, Hkv, Tq, Tk, D, dt);
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int T, int D, fa_dtype dt)
{
    return fa_bwd_kv_workspace_bytes(B, Hq, Hkv, T, T, D, dt);
}

size_t fa_bwd_dkdv_split_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt)
{
    if (check_kv(B, Hq, Hkv, Tq, Tk, D, dt, false, 0) != FA_OK) return 0;
    return split_bytes(B, Hq, Hkv, Tq, Tk, D, dt);
}

size_t fa_bwd_dq_split_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt)
{
    if (check_kv(B, Hq, Hkv, Tq, Tk, D, dt, false, 0) != FA_OK) return 0;
    return dq_split_bytes(B, Hq, Hkv, Tq, Tk, D, dt);
}

fa_status fa_bwd_preprocess(const void* o, const void* dout, float* delta, int B, int Hq, int T,
                            int D, fa_dtype dt, void* stream)
{
    fa_status st = check_kv(B, Hq, 1, T, T, D, dt, false, 0);
    if (st != FA_OK) return st;
    if ((long long)B * T == 0) return FA_OK;
    if (!o || !dout || !delta) return FA_ERR_NULL;
    if (!aligned(o, 16) || !aligned(dout, 16) || !aligned(delta, 4)) return FA_ERR_ALIGN;
    fa::PreArgs a;
    a.o = o;
    a.dout = dout;
    a.delta = delta;
    a.rows = (long)B * Hq * T;
    // kernel instance: 0 bf16 O and dO, 1 float32 both, 2 float32 O with bf16 dO
    const int code = dt == FA_BF16_F32OUT ? 2 : dtype_code(dt);
    return from_hip(fa::launch_bwd_pre(a, D, code, static_cast<hipStream_t>(stream)));
}

// Checks shared by the two backward kernels' entry points.  `skip` is set
// when there is nothing to enqueue.
static fa_status bwd_check(const void* q, const void* k, const void* v, const void* dout,
                           const float* lse, const float* delta, int B, int Hq, int Hkv, int Tq,
                           int Tk, int D, float scale, int causal, int off, fa_dtype dt, bool& skip)
{
    fa_status st = check_kv(B, Hq, Hkv, Tq, Tk, D, dt, causal != 0, off);
    if (st != FA_OK) return st;
    if ((st = check_scale(scale)) != FA_OK) return st;
    skip = (long long)B * Tk == 0;
    if (skip) return FA_OK;
    // with no query row the key-side gradients are zero: only pointers to
    // them (and k, v) are needed
    if (Tq > 0) {
        if (!q || !dout || !lse || !delta) return FA_ERR_NULL;
        if (!aligned(q, 16) || !aligned(dout, 16) || !aligned(lse, 4) || !aligned(delta, 4))
            return FA_ERR_ALIGN;
    }
    if (!k || !v) return FA_ERR_NULL;
    if (!aligned(k, 16) || !aligned(v, 16)) return FA_ERR_ALIGN;
    return FA_OK;
}

fa_status fa_bwd_dkdv_split(const void* q, const void* k, const void* v, const void* dout,
                            const float* lse, const float* delta, void* dk, void* dv, void* partial,
                            int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
                            int q_offset, fa_dtype dt, void* stream)
{
    const int off = causal ? q_offset : 0;
    bool skip = false;
    fa_status st = bwd_check(q, k, v, dout, lse, delta, B, Hq, Hkv, Tq, Tk, D, scale, causal, off,
                             dt, skip);
    if (st != FA_OK || skip) return st;
    if (!dk || !dv) return FA_ERR_NULL;
    if (!aligned(dk, 16) || !aligned(dv, 16) || !aligned(partial, 16)) return FA_ERR_ALIGN;
    fa::BwdArgs a;
    fill_bwd(a, q, k, v, dout, lse, delta, B, Hq, Hkv, Tq, Tk, off, scale);
    a.dk = dk;
    a.dv = dv;
    a.gf32 = dt == FA_BF16_F32OUT;
    if (partial && split_bytes(B, Hq, Hkv, Tq, Tk, D, dt) > 0) {
        a.part = static_cast<float*>(partial);
        a.nsplit = fa::dkdv_nsplit(B, Hq, Hkv, Tq, Tk, D);
    }
    return from_hip(fa::launch_bwd_dkdv(a, D, dtype_code(dt), causal != 0, static_cast<hipStream_t>(stream)));
}

fa_status fa_bwd_dkdv_kv(const void* q, const void* k, const void* v, const void* dout,
                         const float* lse, const float* delta, void* dk, void* dv, int B, int Hq,
                         int Hkv, int Tq, int Tk, int D, float scale, int causal, int q_offset,
                         fa_dtype dt, void* stream)
{
    return fa_bwd_dkdv_split(q, k, v, dout, lse, delta, dk, dv, nullptr, B, Hq, Hkv, Tq, Tk, D,
                             scale, causal, q_offset, dt, stream);
}

// The dQ stage; with o set (bf16), the kernel forms Delta itself and writes
// it to `delta` instead of reading it.
static fa_status dq_enqueue(const void* q, const void* k, const void* v, const void* dout,
                            const float* lse, float* delta, const void* o, void* dq, void* partial,
                            int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
                            int q_offset, fa_dtype dt, void* stream);

fa_status fa_bwd_dq_split(const void* q, const void* k, const void* v, const void* dout,
                          const float* lse, const float* delta, void* dq, void* partial, int B,
                          int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
                          int q_offset, fa_dtype dt, void* stream)
{
    return dq_enqueue(q, k, v, dout, lse, const_cast<float*>(delta), nullptr, dq, partial, B, Hq,
                      Hkv, Tq, Tk, D, scale, causal, q_offset, dt, stream);
}

static fa_status dq_enqueue(const void* q, const void* k, const void* v, const void* dout,
                            const float* lse, float* delta, const void* o, void* dq, void* partial,
                            int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
                            int q_offset, fa_dtype dt, void* stream)
{
    const int off = causal ? q_offset : 0;
    bool skip = false;
    fa_status st = bwd_check(q, k, v, dout, lse, delta, B, Hq, Hkv, Tq, Tk, D, scale, causal, off,
                             dt, skip);
    if (st != FA_OK || skip || Tq == 0) return st;
    if (!dq) return FA_ERR_NULL;
    if (!aligned(dq, 16) || !aligned(partial, 16)) return FA_ERR_ALIGN;
    fa::BwdArgs a;
    fill_bwd(a, q, k, v, dout, lse, delta, B, Hq, Hkv, Tq, Tk, off, scale);
    a.dq = dq;
    a.gf32 = dt == FA_BF16_F32OUT;
    if (o) {
        a.o = o;
        a.delta_out = delta;
    }
    if (partial && dq_split_bytes(B, Hq, Hkv, Tq, Tk, D, dt) > 0) {
        a.part = static_cast<float*>(partial);
        a.nsplit = fa::dq_nsplit(B, Hq, Hkv, Tq, Tk, D);
    }
    return from_hip(fa::launch_bwd_dq(a, D, dtype_code(dt), causal != 0, static_cast<hipStream_t>(stream)));
}

fa_status fa_bwd_dq_delta(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, float* delta, void* dq, void* partial,
                          int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
                          int q_offset, fa_dtype dt, void* stream)
{
    fa_status st = check_kv(B, Hq, Hkv, Tq, Tk, D, dt, causal != 0, causal ? q_offset : 0);
    if (st != FA_OK) return st;
    if (!bf16_in(dt)) return FA_ERR_UNSUPPORTED;
    if ((long long)B * Tq * Tk > 0) {
        if (!o) return FA_ERR_NULL;
        if (!aligned(o, 16)) return FA_ERR_ALIGN;
    }
    if (dt == FA_BF16_F32OUT) {
        // float32 O: Delta from the preprocess kernel (the same bits as the
        // dQ kernel's own for an O of bf16 values), then the dQ kernel
        bool skip = false;
        const int off = causal ? q_offset : 0;
        st = bwd_check(q, k, v, dout, lse, delta, B, Hq, Hkv, Tq, Tk, D, scale, causal, off, dt, skip);
        if (st != FA_OK || skip || Tq == 0) return st;
        if (!dq) return FA_ERR_NULL;
        if (!aligned(dq, 16) || !aligned(partial, 16)) return FA_ERR_ALIGN;
        if ((st = fa_bwd_preprocess(o, dout, delta, B, Hq, Tq, D, dt, stream)) != FA_OK) return st;
        return fa_bwd_dq_split(q, k, v, dout, lse, delta, dq, partial, B, Hq, Hkv, Tq, Tk, D, scale,
                               causal, q_offset, dt, stream);
    }
    return dq_enqueue(q, k, v, dout, lse, delta, o, dq, partial, B, Hq, Hkv, Tq, Tk, D, scale,
                      causal, q_offset, dt, stream);
}

fa_status fa_bwd_dq_kv(const void* q, const void* k, const void* v, const void* dout,
                       const float* lse, const float* delta, void* dq, int B, int Hq, int Hkv,
                       int Tq, int Tk, int D, float scale, int causal, int q_offset, fa_dtype dt,
                       void* stream)
{
    return fa_bwd_dq_split(q, k, v, dout, lse, delta, dq, nullptr, B, Hq, Hkv, Tq, Tk, D, scale,
                           causal, q_offset, dt, stream);
}

fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, const float* delta, void* dk, void* dv, int B, int Hq,
                      int Hkv, int T, int D, float scale, int causal, fa_dtype dt, void* stream)
{
    return fa_bwd_dkdv_kv(q, k, v, dout, lse, delta, dk, dv, B, Hq, Hkv, T, T, D, scale, causal, 0,
                          dt, stream);
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                    const float* lse, const float* delta, void* dq, int B, int Hq, int Hkv, int T,
                    int D, float scale, int causal, fa_dtype dt, void* stream)
{
    return fa_bwd_dq_kv(q, k, v, dout, lse, delta, dq, B, Hq, Hkv, T, T, D, scale, causal, 0, dt,
                        stream);
}

fa_status fa_bwd_kv(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, void* workspace, int B, int Hq,
                    int Hkv, int Tq, int Tk, int D, float scale, int causal, int q_offset,
                    fa_dtype dt, void* stream)
{
    // validate everything before enqueuing anything
    const int off = causal ? q_offset : 0;
    fa_status st = check_kv(B, Hq, Hkv, Tq, Tk, D, dt, causal != 0, off);
    if (st != FA_OK) return st;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if ((long long)B * Tk == 0) return FA_OK;
    const bool rows = Tq > 0;
    if (!k || !v || !dk || !dv) return FA_ERR_NULL;
    if (rows && (!q || !o || !dout || !lse || !dq || !workspace)) return FA_ERR_NULL;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) || !aligned(dv, 16)) return FA_ERR_ALIGN;
    if (rows && (!aligned(q, 16) || !aligned(o, 16) || !aligned(dout, 16) || !aligned(lse, 4) ||
                 !aligned(dq, 16) || !aligned(workspace, 16)))
        return FA_ERR_ALIGN;
    // workspace: Delta, then the partial sums of the split stages (when the
    // shapes split; the dK/dV and dQ stages take turns with one region)
    float* delta = static_cast<float*>(workspace);
    void* partial = shared_split_bytes(B, Hq, Hkv, Tq, Tk, D, dt) > 0
                        ? static_cast<char*>(workspace) +
                              align256((size_t)B * (size_t)Hq * (size_t)Tq * sizeof(float))
                        : nullptr;
    if (!workspace) partial = nullptr;
    if (dt == FA_BF16) {
        // dQ first: its kernel holds dO of its rows and forms Delta as the
        // preprocess kernel would (the same bits), for dK/dV to read
        if (rows && (st = fa_bwd_dq_delta(q, k, v, o, dout, lse, delta, dq, partial, B, Hq, Hkv,
                                          Tq, Tk, D, scale, causal, q_offset, dt, stream)) != FA_OK)
            return st;
        return fa_bwd_dkdv_split(q, k, v, dout, lse, delta, dk, dv, partial, B, Hq, Hkv, Tq, Tk, D,
                                 scale, causal, q_offset, dt, stream);
    }
    if (rows && (st = fa_bwd_preprocess(o, dout, delta, B, Hq, Tq, D, dt, stream)) != FA_OK) return st;
    if ((st = fa_bwd_dkdv_split(q, k, v, dout, lse, delta, dk, dv, partial, B, Hq, Hkv, Tq, Tk, D,
                                scale, causal, q_offset, dt, stream)) != FA_OK)
        return st;
    return fa_bwd_dq_split(q, k, v, dout, lse, delta, dq, partial, B, Hq, Hkv, Tq, Tk, D, scale,
                           causal, q_offset, dt, stream);
}

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
                         int q_offset, fa_dtype dt, void* stream)
{
    fa_status st = check_kv(B, Hq, Hkv, Tq, Tk, D, dt, causal != 0, causal ? q_offset : 0);
    if (st != FA_OK) return st;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if (fa_bwd_kv_workspace_bytes(B, Hq, Hkv, Tq, Tk, D, dt) > FA_NOALLOC_SCRATCH_BYTES)
        return FA_ERR_SCRATCH;
    void* ws = nullptr;
    if ((long long)B * Tq * Tk > 0 && (st = scratch_address(&ws)) != FA_OK) return st;
    return fa_bwd_kv(q, k, v, o, dout, lse, dq, dk, dv, ws, B, Hq, Hkv, Tq, Tk, D, scale, causal,
                     q_offset, dt, stream);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace, int B, int Hq,
                 int Hkv, int T, int D, float scale, int causal, fa_dtype dt, void* stream)
{
    return fa_bwd_kv(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, Hq, Hkv, T, T, D, scale,
                     causal, 0, dt, stream);
}

size_t fa_bwd_atomic_workspace_bytes(int B, int Hq, int T, int D, fa_dtype dt)
{
    if (check_kv(B, Hq, Hq, T, T, D, dt, false, 0) != FA_OK || dt != FA_BF16 || D != 64) return 0;
    const size_t rows = (size_t)B * (size_t)Hq * (size_t)T;
    return align256(rows * sizeof(float)) + rows * (size_t)D * sizeof(float);
}

fa_status fa_bwd_atomic(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, int B, int Hq, int Hkv, int T, int D, float scale,
                        int causal, fa_dtype dt, void* stream)
{
    fa_status st = check_kv(B, Hq, Hkv, T, T, D, dt, causal != 0, 0);
    if (st != FA_OK) return st;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if (dt != FA_BF16 || D != 64) return FA_ERR_UNSUPPORTED;
    if ((long long)B * T == 0) return FA_OK;
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(dout, 16) || !aligned(lse, 4) || !aligned(dq, 16) || !aligned(dk, 16) ||
        !aligned(dv, 16) || !aligned(workspace, 16))
        return FA_ERR_ALIGN;
    // workspace: Delta, then the fp32 dQ accumulator
    float* delta = static_cast<float*>(workspace);
    float* acc = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          align256((size_t)B * (size_t)Hq * (size_t)T * sizeof(float)));
    if ((st = fa_bwd_preprocess(o, dout, delta, B, Hq, T, D, dt, stream)) != FA_OK) return st;
    fa::BwdArgs a;
    fill_bwd(a, q, k, v, dout, lse, delta, B, Hq, Hkv, T, T, 0, scale);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.part = acc;
    return from_hip(fa::launch_bwd_atomic_bf16(a, causal != 0, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
