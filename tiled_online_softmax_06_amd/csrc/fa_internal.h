// Internal interface between the C-ABI layer (fa_api.hip) and the kernels
// (flash_fwd.hip, flash_fwd_fp8.hip, flash_bwd.hip).  Not installed; include/fa.h is the public header.
#pragma once

#include <float.h>
#include <math.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace fa {

// Factor c = |s| log2(e) that turns raw scores into base-2 exponents: the
// kernels take every weight as exp2(score * c - m).  Computed in double and
// rounded to float once.  Returns false when c is not a finite float (|s|
// above FLT_MAX / log2 e: the kernels would form 0 * inf = NaN); a c below
// FLT_MIN (s = 0 included) is raised to FLT_MIN, where every finite score
// times c is far below the rounding of exp2 near 0, so all weights are
// exactly 1 as for a zero factor, while a masked score -inf times c stays
// -inf (times 0 it would be NaN).
inline bool exp2_factor(double s, float* c) {
    const double x = fabs(s) * 1.4426950408889634;
    if (!(x <= (double)FLT_MAX)) return false;
    const float f = (float)x;
    if (!(f <= FLT_MAX)) return false;          // rounded up to infinity
    *c = f < FLT_MIN ? FLT_MIN : f;
    return true;
}

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int64_t bh;      // B * H (query heads are independent and contiguous)
    int64_t h;       // H, query heads per batch
    int64_t hkv;     // K/V heads per batch (divides H)
    int64_t n;       // sequence length
    int d;           // head dimension (64 or 128)
    int dtype;       // fa_dtype_t
    float scale;     // finite
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    float* dws;      // B * H * N floats: rowsum(dO * O)
    void* dq;
    void* dk;
    void* dv;
    int64_t bh;      // B * H
    int64_t h;       // H
    int64_t hkv;     // K/V heads (divides H)
    int64_t n;
    int d;
    int dtype;       // fp16 or bf16
    float scale;
};

struct Fp8Args {
    const void* q;   // e4m3 codes, (B, H, N, d)
    const void* k;   // e4m3 codes, (B, Hkv, N, d)
    const void* v;
    void* o;         // (B, H, N, d) of out_dtype
    float* lse;
    int64_t bh;
    int64_t h;
    int64_t hkv;
    int64_t n;
    int d;
    int out_dtype;   // fa_dtype_t of O
    float scale;
    float q_descale, k_descale, v_descale;
};

// Launches the FP8 forward kernel on `stream` (checked arguments).
hipError_t launch_forward_fp8(const Fp8Args& a, hipStream_t stream);

// Launches the backward kernels (row dots, dQ, dK/dV) on `stream`.
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);

// Launches the forward kernel matching (dtype, d) on `stream`.
// Preconditions (checked by the caller): shapes valid and non-empty,
// pointers non-null, aligned and non-overlapping outputs.
hipError_t launch_forward(const FwdArgs& a, hipStream_t stream);

// Key split (one kernel launch per call, then a merge): the keys of every
// head are cut into `splits` ranges of `kchunk` keys (kchunk a multiple of
// kSplitAlign; the last range may be shorter; none is empty).  The forward
// kernels write each range's normalised fp32 partial output to o_part,
// (B*H, splits, N, d), and its LSE to lse_part, (B*H, splits, N); the merge
// kernel then writes a.o and a.lse.
constexpr int kSplitAlign = 64;
hipError_t launch_forward_split(const FwdArgs& a, int splits, int kchunk, float* o_part, float* lse_part,
                                hipStream_t stream);

// Merges S normalised partial results per row: o_parts (G, S, M, d) and
// lse_parts (G, S, M) fp32 into o (G, M, d) of `dtype` and lse (G, M).
hipError_t launch_merge(const float* o_parts, const float* lse_parts, int64_t g, int64_t s, int64_t m, int d,
                        void* o, float* lse, int dtype, hipStream_t stream);

// Query rows per workgroup of the forward kernel chosen for (dtype, d), and
// how many of its workgroups one CU holds at once.
int forward_rows_per_workgroup(int dtype, int d);
int forward_workgroups_per_cu(int dtype, int d);

// Smallest number of rows handled by one workgroup over all configurations;
// used by the caller to bound the grid size.
constexpr int kMinRowsPerWorkgroup = 128;

// Describes the tile configurations compiled into the library.
const char* kernel_config_string();

}  // namespace fa
