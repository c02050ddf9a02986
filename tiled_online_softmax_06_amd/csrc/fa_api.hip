// fa_api.hip — the C ABI of include/fa.h: host-side argument checks and
// dispatch to the gfx950 kernels.  No allocation, copy or synchronisation.
#include <math.h>
#include <stdint.h>
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

}  // namespace

extern "C" int fa_forward_gqa(const void* Q, const void* K, const void* V, void* O, float* LSE,
                              int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                              float scale, int dtype, hipStream_t stream) {
    if (B < 0 || H < 0 || N < 0 || d < 0 || Hkv < 0) return FA_ERR_BAD_SHAPE;
    if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (!isfinite(scale)) return FA_ERR_BAD_SCALE;

    const int64_t esize = dtype == FA_DTYPE_FP32 ? 4 : 2;
    int64_t bh = 0, rows = 0, elems = 0, bytes = 0, bkv = 0, kvrows = 0, kvelems = 0, kvbytes = 0;
    if (!mul_ok(B, H, &bh) || !mul_ok(bh, N, &rows) || !mul_ok(rows, d, &elems) ||
        !mul_ok(elems, esize, &bytes) || !mul_ok(B, Hkv, &bkv) || !mul_ok(bkv, N, &kvrows) ||
        !mul_ok(kvrows, d, &kvelems) || !mul_ok(kvelems, esize, &kvbytes))
        return FA_ERR_BAD_SHAPE;
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

    fa::FwdArgs a{Q, K, V, O, LSE, bh, H, Hkv, N, (int)d, dtype, scale};
    return fa::launch_forward(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_forward(const void* Q, const void* K, const void* V, void* O, float* LSE,
                          int64_t B, int64_t H, int64_t N, int64_t d,
                          float scale, int dtype, hipStream_t stream) {
    return fa_forward_gqa(Q, K, V, O, LSE, B, H, H, N, d, scale, dtype, stream);
}

extern "C" int fa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                           const float* LSE, float* Dws, void* dQ, void* dK, void* dV,
                           int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                           float scale, int dtype, hipStream_t stream) {
    if (B < 0 || H < 0 || N < 0 || d < 0 || Hkv < 0) return FA_ERR_BAD_SHAPE;
    if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (!isfinite(scale)) return FA_ERR_BAD_SCALE;

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
        default: return "unknown status";
    }
}

extern "C" const char* fa_version(void) {
    return fa::kernel_config_string();
}
