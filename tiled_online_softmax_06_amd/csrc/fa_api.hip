// fa_api.hip — the C ABI of include/fa.h: host-side argument checks and
// dispatch to the gfx950 kernels.  No allocation, copy or synchronisation.
#include <math.h>
#include <stdint.h>
#include <mutex>
#include <hip/hip_runtime.h>

#include "fa_internal.h"
#include "../../include/fa.h"

namespace {

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

bool mul_ok(int64_t x, int64_t y, int64_t* out) {
    if (x != 0 && y > INT64_MAX / x) return false;
    *out = x * y;
    return true;
}

// Argument checks shared by the forward entry points.  Returns FA_OK with
// *empty set when B*H*N == 0 (nothing to launch).
struct FwdSizes { int64_t bh, rows, bytes, kvbytes, lbytes; bool empty; };

int check_forward(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                  int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d, float scale, int dtype,
                  FwdSizes* sz) {
    if (B < 0 || H < 0 || N < 0 || d < 0 || Hkv < 0) return FA_ERR_BAD_SHAPE;
    if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    float c = 0.f;
    if (!isfinite(scale) || !fa::exp2_factor(scale, &c)) return FA_ERR_BAD_SCALE;

    const int64_t esize = dtype == FA_DTYPE_FP32 ? 4 : 2;
    int64_t bh = 0, rows = 0, elems = 0, bytes = 0, bkv = 0, kvrows = 0, kvelems = 0, kvbytes = 0;
    if (!mul_ok(B, H, &bh) || !mul_ok(bh, N, &rows) || !mul_ok(rows, d, &elems) ||
        !mul_ok(elems, esize, &bytes) || !mul_ok(B, Hkv, &bkv) || !mul_ok(bkv, N, &kvrows) ||
        !mul_ok(kvrows, d, &kvelems) || !mul_ok(kvelems, esize, &kvbytes))
        return FA_ERR_BAD_SHAPE;
    *sz = FwdSizes{bh, rows, bytes, kvbytes, rows * 4, rows == 0};
    if (rows == 0) return FA_OK;
    // every query head needs a K/V head: Hkv >= 1 and divides H
    if (Hkv == 0 || H % Hkv != 0) return FA_ERR_BAD_SHAPE;
    // Kernel index limits: N and the workgroup count are 32-bit, and one
    // head's K / V rows are addressed with 32-bit buffer byte offsets.
    if (N > INT32_MAX || H > INT32_MAX || N * d * esize > INT32_MAX) return FA_ERR_BAD_SHAPE;
    const int64_t tiles = bh * ((N + fa::kMinRowsPerWorkgroup - 1) / fa::kMinRowsPerWorkgroup);
    if (tiles > INT32_MAX) return FA_ERR_BAD_SHAPE;

    if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL_POINTER;
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15u) return FA_ERR_MISALIGNED;
    if ((uintptr_t)LSE & 3u) return FA_ERR_MISALIGNED;
    const int64_t lbytes = rows * 4;
    if (overlaps(O, bytes, Q, bytes) || overlaps(O, bytes, K, kvbytes) || overlaps(O, bytes, V, kvbytes) ||
        overlaps(LSE, lbytes, Q, bytes) || overlaps(LSE, lbytes, K, kvbytes) ||
        overlaps(LSE, lbytes, V, kvbytes) || overlaps(LSE, lbytes, O, bytes))
        return FA_ERR_ALIAS;
    return FA_OK;
}

// Key ranges for a requested split count: `*ranges` ranges of `*kchunk`
// keys, kchunk a multiple of one 64-key tile, none empty (so at most one
// range per tile; fewer than asked when the tiles do not divide evenly).
void split_plan(int64_t N, int64_t splits, int64_t* ranges, int64_t* kchunk) {
    const int64_t tiles = (N + fa::kSplitAlign - 1) / fa::kSplitAlign;
    const int64_t s = splits < tiles ? splits : tiles;
    const int64_t per = s > 0 ? (tiles + s - 1) / s : 1;
    *kchunk = per * fa::kSplitAlign;
    *ranges = N > 0 ? (N + *kchunk - 1) / *kchunk : 1;
}

// Workspace bytes for `ranges` key ranges: fp32 partial O then partial LSE.
bool split_bytes(int64_t bh, int64_t N, int64_t d, int64_t ranges, int64_t* obytes, int64_t* lbytes) {
    int64_t prow = 0, pel = 0;
    if (!mul_ok(bh, ranges, &prow) || !mul_ok(prow, N, &prow) || !mul_ok(prow, d, &pel) ||
        !mul_ok(pel, 4, obytes) || !mul_ok(prow, 4, lbytes) || *obytes > INT64_MAX - *lbytes)
        return false;
    return true;
}

constexpr int64_t kComputeUnits = 256;   // MI355X

// Scratch for fa_forward_split_noalloc: the key split's float32 partial
// results in a fixed device array (one copy per GPU, held until the process
// ends).  Host code uses only the per-device address that
// hipGetSymbolAddress returns, never the array's name.
static __device__ __align__(256) char scratch[FA_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

}  // namespace

extern "C" int fa_forward_gqa(const void* Q, const void* K, const void* V, void* O, float* LSE,
                              int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                              float scale, int dtype, hipStream_t stream) {
    FwdSizes sz;
    const int st = check_forward(Q, K, V, O, LSE, B, H, Hkv, N, d, scale, dtype, &sz);
    if (st != FA_OK || sz.empty) return st;
    fa::FwdArgs a{Q, K, V, O, LSE, sz.bh, H, Hkv, N, (int)d, dtype, scale};
    return fa::launch_forward(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_forward(const void* Q, const void* K, const void* V, void* O, float* LSE,
                          int64_t B, int64_t H, int64_t N, int64_t d,
                          float scale, int dtype, hipStream_t stream) {
    return fa_forward_gqa(Q, K, V, O, LSE, B, H, H, N, d, scale, dtype, stream);
}

extern "C" int fa_forward_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE,
                              int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                              float scale, float q_descale, float k_descale, float v_descale,
                              int out_dtype, hipStream_t stream) {
    if (B < 0 || H < 0 || N < 0 || d < 0 || Hkv < 0) return FA_ERR_BAD_SHAPE;
    if (out_dtype != FA_DTYPE_FP32 && out_dtype != FA_DTYPE_FP16 && out_dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (!isfinite(scale) || !isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale))
        return FA_ERR_BAD_SCALE;
    // the kernel multiplies the scores of the codes by scale * q_descale *
    // k_descale (in log2 units); that factor must itself be a finite float
    float c = 0.f;
    if (!fa::exp2_factor((double)scale * (double)q_descale * (double)k_descale, &c)) return FA_ERR_BAD_SCALE;
    const int64_t oesize = out_dtype == FA_DTYPE_FP32 ? 4 : 2;
    int64_t bh = 0, rows = 0, bytes = 0, obytes = 0, bkv = 0, kvrows = 0, kvbytes = 0;
    if (!mul_ok(B, H, &bh) || !mul_ok(bh, N, &rows) || !mul_ok(rows, d, &bytes) || !mul_ok(bytes, oesize, &obytes) ||
        !mul_ok(B, Hkv, &bkv) || !mul_ok(bkv, N, &kvrows) || !mul_ok(kvrows, d, &kvbytes))
        return FA_ERR_BAD_SHAPE;
    if (rows == 0) return FA_OK;
    if (Hkv == 0 || H % Hkv != 0) return FA_ERR_BAD_SHAPE;
    if (N > INT32_MAX || H > INT32_MAX || N * d > INT32_MAX) return FA_ERR_BAD_SHAPE;
    const int64_t tiles = bh * ((N + fa::kMinRowsPerWorkgroup - 1) / fa::kMinRowsPerWorkgroup);
    if (tiles > INT32_MAX) return FA_ERR_BAD_SHAPE;
    if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL_POINTER;
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15u) return FA_ERR_MISALIGNED;
    if ((uintptr_t)LSE & 3u) return FA_ERR_MISALIGNED;
    const int64_t lbytes = rows * 4;
    if (overlaps(O, obytes, Q, bytes) || overlaps(O, obytes, K, kvbytes) || overlaps(O, obytes, V, kvbytes) ||
        overlaps(LSE, lbytes, Q, bytes) || overlaps(LSE, lbytes, K, kvbytes) ||
        overlaps(LSE, lbytes, V, kvbytes) || overlaps(LSE, lbytes, O, obytes))
        return FA_ERR_ALIAS;
    fa::Fp8Args a{Q, K, V, O, LSE, bh, H, Hkv, N, (int)d, out_dtype, scale, q_descale, k_descale, v_descale};
    return fa::launch_forward_fp8(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int64_t fa_split_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t splits) {
    if (B < 0 || H < 0 || N < 0 || d < 1 || splits < 1) return -1;
    int64_t bh = 0, ranges = 0, kchunk = 0, ob = 0, lb = 0;
    if (!mul_ok(B, H, &bh)) return -1;
    if (bh == 0 || N == 0) return 0;
    split_plan(N, splits, &ranges, &kchunk);
    if (ranges == 1) return 0;
    if (!split_bytes(bh, N, d, ranges, &ob, &lb)) return -1;
    return ob + lb;
}

extern "C" int64_t fa_split_suggest(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
    if (B < 0 || H < 0 || N < 0 || (d != 64 && d != 128)) return 1;
    int64_t bh = 0;
    if (!mul_ok(B, H, &bh) || bh == 0 || N == 0 || bh > ((int64_t)1 << 40) / N) return 1;
    const int64_t rows = fa::forward_rows_per_workgroup(dtype, (int)d);
    const int64_t slots = kComputeUnits * fa::forward_workgroups_per_cu(dtype, (int)d);
    const int64_t wg = bh * ((N + rows - 1) / rows);          // workgroups of one key range
    const int64_t tiles = (N + fa::kSplitAlign - 1) / fa::kSplitAlign;
    // Cost in 64-key tile steps of one workgroup: waves of workgroups times
    // (tiles per range + about 2 tiles of pipeline fill and epilogue), plus,
    // for S > 1, the merge's memory traffic (S partials read, O written) at
    // about 12.6 MB per tile step (7 TB/s for one 1.8 us step) and a fixed
    // 12 steps for the second launch and the partials' round trip (measured:
    // a 19 us unsplit launch ran 28 us split in two).  Each range keeps at
    // least 8 tiles (512 keys).
    int64_t most = tiles / 8;
    if (most > 64) most = 64;
    int64_t best = 1;
    double best_cost = 0.0;
    for (int64_t s = 1; s <= (most > 1 ? most : 1); ++s) {
        const int64_t waves = (wg * s + slots - 1) / slots;
        double cost = (double)waves * (double)((tiles + s - 1) / s + 2);
        if (s > 1) cost += 12.0 + (double)bh * (double)N * (double)d * (4.0 * s + 2.0) / 12.6e6;
        if (s == 1 || cost < best_cost) {
            best = s;
            best_cost = cost;
        }
    }
    return best;
}

extern "C" int fa_forward_split(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                                float scale, int dtype, int64_t splits, void* workspace,
                                int64_t workspace_bytes, hipStream_t stream) {
    if (splits < 1) return FA_ERR_BAD_SHAPE;
    FwdSizes sz;
    const int st = check_forward(Q, K, V, O, LSE, B, H, Hkv, N, d, scale, dtype, &sz);
    if (st != FA_OK || sz.empty) return st;
    int64_t ranges = 0, kchunk = 0, ob = 0, lb = 0;
    split_plan(N, splits, &ranges, &kchunk);
    if (ranges == 1) {
        fa::FwdArgs a{Q, K, V, O, LSE, sz.bh, H, Hkv, N, (int)d, dtype, scale};
        return fa::launch_forward(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
    }
    if (!split_bytes(sz.bh, N, d, ranges, &ob, &lb)) return FA_ERR_BAD_SHAPE;
    const int64_t wgs = sz.bh * ranges * ((N + fa::kMinRowsPerWorkgroup - 1) / fa::kMinRowsPerWorkgroup);
    if (wgs > INT32_MAX) return FA_ERR_BAD_SHAPE;
    if (!workspace || workspace_bytes < ob + lb) return FA_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 15u) return FA_ERR_MISALIGNED;
    if (overlaps(workspace, ob + lb, Q, sz.bytes) || overlaps(workspace, ob + lb, K, sz.kvbytes) ||
        overlaps(workspace, ob + lb, V, sz.kvbytes) || overlaps(workspace, ob + lb, O, sz.bytes) ||
        overlaps(workspace, ob + lb, LSE, sz.lbytes))
        return FA_ERR_ALIAS;
    float* o_part = (float*)workspace;
    float* lse_part = (float*)((char*)workspace + ob);
    fa::FwdArgs a{Q, K, V, O, LSE, sz.bh, H, Hkv, N, (int)d, dtype, scale};
    return fa::launch_forward_split(a, (int)ranges, (int)kchunk, o_part, lse_part, stream) == hipSuccess
               ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_forward_split_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                        int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                                        float scale, int dtype, int64_t splits, hipStream_t stream) {
    if (splits < 1) return FA_ERR_BAD_SHAPE;
    FwdSizes sz;
    const int st = check_forward(Q, K, V, O, LSE, B, H, Hkv, N, d, scale, dtype, &sz);
    if (st != FA_OK || sz.empty) return st;
    int64_t ranges = 0, kchunk = 0, ob = 0, lb = 0;
    split_plan(N, splits, &ranges, &kchunk);
    fa::FwdArgs a{Q, K, V, O, LSE, sz.bh, H, Hkv, N, (int)d, dtype, scale};
    if (ranges == 1) return fa::launch_forward(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
    if (!split_bytes(sz.bh, N, d, ranges, &ob, &lb)) return FA_ERR_BAD_SHAPE;
    const int64_t wgs = sz.bh * ranges * ((N + fa::kMinRowsPerWorkgroup - 1) / fa::kMinRowsPerWorkgroup);
    if (wgs > INT32_MAX) return FA_ERR_BAD_SHAPE;
    if (ob + lb > FA_SCRATCH_BYTES) return FA_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    const int sa = scratch_address(&ws);
    if (sa != FA_OK) return sa;
    // every partial element the merge reads is written by this call's
    // forward kernels first, so nothing needs clearing
    float* o_part = (float*)ws;
    float* lse_part = (float*)((char*)ws + ob);
    return fa::launch_forward_split(a, (int)ranges, (int)kchunk, o_part, lse_part, stream) == hipSuccess
               ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_merge(const float* O_parts, const float* LSE_parts, int64_t G, int64_t S, int64_t M,
                        int64_t d, void* O, float* LSE, int dtype, hipStream_t stream) {
    if (G < 0 || S < 0 || M < 0 || d < 0) return FA_ERR_BAD_SHAPE;
    if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    const int64_t esize = dtype == FA_DTYPE_FP32 ? 4 : 2;
    int64_t rows = 0, prows = 0, pel = 0, pbytes = 0, el = 0, obytes = 0;
    if (!mul_ok(G, M, &rows) || !mul_ok(rows, S, &prows) || !mul_ok(prows, d, &pel) ||
        !mul_ok(pel, 4, &pbytes) || !mul_ok(rows, d, &el) || !mul_ok(el, esize, &obytes) ||
        prows > INT64_MAX / 4)
        return FA_ERR_BAD_SHAPE;
    if (rows == 0) return FA_OK;
    if (S < 1 || S > INT32_MAX) return FA_ERR_BAD_SHAPE;
    if (!O_parts || !LSE_parts || !O || !LSE) return FA_ERR_NULL_POINTER;
    if (((uintptr_t)O_parts | (uintptr_t)O) & 15u) return FA_ERR_MISALIGNED;
    if (((uintptr_t)LSE_parts | (uintptr_t)LSE) & 3u) return FA_ERR_MISALIGNED;
    const int64_t lbytes = rows * 4, plbytes = prows * 4;
    if (overlaps(O, obytes, O_parts, pbytes) || overlaps(O, obytes, LSE_parts, plbytes) ||
        overlaps(LSE, lbytes, O_parts, pbytes) || overlaps(LSE, lbytes, LSE_parts, plbytes) ||
        overlaps(O, obytes, LSE, lbytes))
        return FA_ERR_ALIAS;
    return fa::launch_merge(O_parts, LSE_parts, G, S, M, (int)d, O, LSE, dtype, stream) == hipSuccess
               ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                           const float* LSE, float* Dws, void* dQ, void* dK, void* dV,
                           int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                           float scale, int dtype, hipStream_t stream) {
    if (B < 0 || H < 0 || N < 0 || d < 0 || Hkv < 0) return FA_ERR_BAD_SHAPE;
    if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    float c = 0.f;
    if (!isfinite(scale) || !fa::exp2_factor(scale, &c)) return FA_ERR_BAD_SCALE;

    const int64_t esize = 2;
    int64_t bh = 0, rows = 0, elems = 0, bytes = 0, bkv = 0, kvrows = 0, kvelems = 0, kvbytes = 0;
    if (!mul_ok(B, H, &bh) || !mul_ok(bh, N, &rows) || !mul_ok(rows, d, &elems) ||
        !mul_ok(elems, esize, &bytes) || !mul_ok(B, Hkv, &bkv) || !mul_ok(bkv, N, &kvrows) ||
        !mul_ok(kvrows, d, &kvelems) || !mul_ok(kvelems, esize, &kvbytes))
        return FA_ERR_BAD_SHAPE;
    if (rows == 0) return FA_OK;
    if (Hkv == 0 || H % Hkv != 0) return FA_ERR_BAD_SHAPE;
    if (N > INT32_MAX || H > INT32_MAX || N * d * esize > INT32_MAX) return FA_ERR_BAD_SHAPE;
    const int64_t tiles = bh * ((N + fa::kMinRowsPerWorkgroup - 1) / fa::kMinRowsPerWorkgroup);
    if (tiles > INT32_MAX) return FA_ERR_BAD_SHAPE;

    if (!Q || !K || !V || !O || !dO || !LSE || !Dws || !dQ || !dK || !dV) return FA_ERR_NULL_POINTER;
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O | (uintptr_t)dO | (uintptr_t)dQ |
         (uintptr_t)dK | (uintptr_t)dV) & 15u)
        return FA_ERR_MISALIGNED;
    if (((uintptr_t)LSE | (uintptr_t)Dws) & 3u) return FA_ERR_MISALIGNED;
    const int64_t lbytes = rows * 4;
    // outputs (dQ, dK, dV, Dws) must not overlap each other or any input
    struct Span { const void* p; int64_t n; };
    const Span ins[] = {{Q, bytes}, {K, kvbytes}, {V, kvbytes}, {O, bytes}, {dO, bytes}, {LSE, lbytes}};
    const Span outs[] = {{dQ, bytes}, {dK, kvbytes}, {dV, kvbytes}, {Dws, lbytes}};
    for (int i = 0; i < 4; ++i) {
        for (const Span& in : ins)
            if (overlaps(outs[i].p, outs[i].n, in.p, in.n)) return FA_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return FA_ERR_ALIAS;
    }

    fa::BwdArgs a{Q, K, V, O, dO, LSE, Dws, dQ, dK, dV, bh, H, Hkv, N, (int)d, dtype, scale};
    return fa::launch_backward(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL_POINTER: return "null pointer";
        case FA_ERR_BAD_SHAPE: return "bad shape";
        case FA_ERR_UNSUPPORTED_HEAD_DIM: return "unsupported head dimension (need 64 or 128)";
        case FA_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
        case FA_ERR_MISALIGNED: return "misaligned pointer";
        case FA_ERR_ALIAS: return "output overlaps an input or the other output";
        case FA_ERR_BAD_SCALE: return "scale is not finite";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_WORKSPACE: return "workspace missing or smaller than required";
        case FA_ERR_SCRATCH_LIMIT: return "partial results exceed the library's fixed scratch (FA_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

extern "C" const char* fa_version(void) {
    return fa::kernel_config_string();
}
