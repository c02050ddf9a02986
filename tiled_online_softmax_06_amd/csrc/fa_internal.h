// Internal interface between the C-ABI layer (fa_api.hip) and the kernels
// (flash_fwd.hip).  Not installed; include/fa.h is the public header.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace fa {

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

// Launches the backward kernels (row dots, dQ, dK/dV) on `stream`.
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);

// Launches the forward kernel matching (dtype, d) on `stream`.
// Preconditions (checked by the caller): shapes valid and non-empty,
// pointers non-null, aligned and non-overlapping outputs.
hipError_t launch_forward(const FwdArgs& a, hipStream_t stream);

// Largest number of rows handled by one workgroup over all configurations;
// used by the caller to bound the grid size.
constexpr int kMinRowsPerWorkgroup = 128;

// Describes the tile configurations compiled into the library.
const char* kernel_config_string();

}  // namespace fa
