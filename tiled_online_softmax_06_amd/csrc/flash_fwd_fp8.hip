// flash_fwd_fp8.hip — attention forward with FP8 (OCP e4m3) inputs on gfx950.
//
// The unite.ai page "Atención Flash: Revolucionando la Eficiencia de los
// Modelos de Transformador", section "Atención Flash-3", names low-precision
// FP8 arithmetic for the attention products.  Reading: Q, K and V arrive as
// e4m3 codes with one float32 dequantisation factor per tensor (value =
// factor * code); the result is the forward definition applied to the
// dequantised values:
//
//     S = scale dq dk (Q8 K8^T),  O = dv softmax(S) V8,  LSE = ln sum_j exp(S_ij)
//
// Both products run on v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, float32
// accumulation; twice the bf16 rate).  The softmax is float32 as in the
// 16-bit kernels; the weights P are rounded to e4m3 for the second product,
// with the running reference kept 7 to 8.75 binades below the row maximum so
// that they use e4m3's range.
//
// Layouts (checked on the device with one-wave probes):
//   * The 32x32x64 MFMA pairs byte b of A lane (i, half) with byte b of B
//     lane (j, half), so any common assignment of the 64 contraction indices
//     to (half, byte) is consistent.  Q K^T uses dims 64 kc + 32 half + b.
//   * ds_read_b64_tr_b8: in each group of 16 lanes, lane 2e + s addresses row
//     e, bytes 8 s .. 8 s + 7 of an 8-row x 16-byte block; lane 8 s + c then
//     receives column 8 s + c of the block (byte e from row e).  V^T, the A
//     operand of O^T += V^T P^T, is read this way: read r (0..3) of lane
//     (dim, half) covers LDS rows 16 r + 8 half + 0..7 of the V tile.
//   * P leaves the score accumulator in runs of 4 keys (lane half h holds
//     keys 8 q + 4 h + 0..3) and is packed to e4m3 in that order; the V tile
//     is stored in LDS with bits 2 and 3 of the key index swapped, so that
//     the transpose reads return V rows in the same key order.
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"
#include "../../include/fa.h"

#include "fa_device.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2* lds_i32x2;

constexpr float kFp8Slack = 8.75f;
constexpr float kFp8Headroom = 7.0f;

// e4m3 MFMA, unscaled (the zero scale operands select the plain instruction).
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four floats to four e4m3 bytes (round to nearest even), byte e = x[e].
// The first conversion writes the low half of a register whose high half the
// second one overwrites, so it starts from whatever the register holds (an
// empty asm statement defines it) rather than from a zeroed register.
__device__ __forceinline__ int pack_fp8(float x0, float x1, float x2, float x3) {
    int any;
    asm volatile("" : "=v"(any));
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, any, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

// LDS swizzles for tiles of D-byte rows split into 16-byte chunks (chunk c
// of row r sits at position c ^ f(r)).
//  * K, row reads (ds_read_b128, 16 lanes = 16 consecutive rows, one chunk):
//    the 16 lanes must cover the 16 chunk slots of a 256-byte bank window.
//  * V, transpose reads (ds_read_b64_tr_b8, 32 lanes = 8 consecutive rows x
//    two adjacent chunks): the 16 (row, chunk) pairs must cover the 16 slots.
template <int D> __device__ __forceinline__ constexpr int swz8_k(int r) {
    return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
template <int D> __device__ __forceinline__ constexpr int swz8_v(int r) {
    return D == 128 ? (2 * ((r >> 1) & 3)) : (2 * ((r >> 2) & 1));
}

template <typename OutT> struct Store4;
template <> struct Store4<__bf16> {
    static __device__ __forceinline__ void run(__bf16* p, const float* v) { *(u32x2*)p = Mfma<__bf16>::pack4(v); }
};
template <> struct Store4<_Float16> {
    static __device__ __forceinline__ void run(_Float16* p, const float* v) { *(u32x2*)p = Mfma<_Float16>::pack4(v); }
};
template <> struct Store4<float> {
    static __device__ __forceinline__ void run(float* p, const float* v) {
        *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    }
};

// Workgroup: 4 waves x 32 query rows of one (b, h); K/V tiles of BC keys
// (a multiple of 64) DMA'd into double-buffered LDS; two workgroups per CU.
template <int D, int BC, typename OutT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
flash_fwd_fp8(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
              OutT* __restrict__ O, float* __restrict__ LSE,
              int n, int qtiles, int total, float c, int negate, float vscale, int nh, int grp)
{
    constexpr int NW = 4;
    constexpr int BR = 32 * NW;              // query rows per workgroup
    constexpr int ROWB = D;                  // bytes per K/V row
    constexpr int CPR = D / 16;              // 16-byte chunks per row
    constexpr int RPU = 64 / CPR;            // rows per 1 KB DMA unit
    constexpr int TILEB = BC * ROWB;         // bytes of one K (or V) tile
    constexpr int UNITS = TILEB / 1024;
    constexpr int UPW = UNITS / NW;          // DMA units per wave
    constexpr int KT = BC / 32;              // 32-key sub-tiles
    constexpr int DT = D / 32;               // 32-wide output column blocks
    constexpr int KC = D / 64;               // 64-dim contraction chunks of Q.K^T
    constexpr int G = BC / 64;               // 64-key groups (one P.V MFMA each)
    static_assert(UNITS % NW == 0 && BC % 64 == 0, "tile shape");

    __shared__ __attribute__((aligned(1024))) char ks0[TILEB];
    __shared__ __attribute__((aligned(1024))) char vs0[TILEB];
    __shared__ __attribute__((aligned(1024))) char ks1[TILEB];
    __shared__ __attribute__((aligned(1024))) char vs1[TILEB];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;

    const int tile = xcd_tile(blockIdx.x, total);
    const int bh = tile / qtiles;
    const int qt = tile - bh * qtiles;
    const int64_t base = (int64_t)bh * n * D;
    const int64_t kvbase = (int64_t)((bh / nh) * (nh / grp) + (bh % nh) / grp) * n * D;
    const int qrow = qt * BR + wave * 32 + col;

    // Q^T as the B operand: lane (col, half) holds Q[qrow][64 kc + 32 half +
    // 0..31]; rows past the end are clamped (computed, never stored).  A
    // negative scale flips the sign bits of Q (e4m3: bit 7), after the first
    // K/V tile's DMA has been issued (done here, the flip would make that DMA
    // wait for Q to arrive).
    i32x8 qf[KC];
    {
        const uint8_t* qp = Q + base + (int64_t)min(qrow, n - 1) * D + 32 * half;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const u32x4 lo = *(const u32x4*)(qp + 64 * kc);
            const u32x4 hi = *(const u32x4*)(qp + 64 * kc + 16);
            qf[kc] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    }
    auto negate_q = [&]() {
        if (negate) {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) qf[kc] ^= i32x8(0x80808080);
        }
    };

    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(K + kvbase), (short)0, n * ROWB, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(V + kvbase), (short)0, n * ROWB, 0x00020000);

    const int lrow = lane / CPR;
    const int lch = lane % CPR;
    // Per-lane DMA offsets within a tile: LDS row r of unit i is key r of
    // the K tile and key rv of the V tile (r with bits 2 and 3 swapped, the
    // order in which P leaves the score accumulators; see the P.V product),
    // at its swizzled chunk; the tile's byte offset is the scalar offset.
    int kdo[UPW], vdo[UPW];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
        const int r = (wave * UPW + i) * RPU + lrow;
        const int rv = (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
        kdo[i] = r * ROWB + 16 * (lch ^ swz8_k<D>(r));
        vdo[i] = rv * ROWB + 16 * (lch ^ swz8_v<D>(r));
    }
    // One DMA form for every tile: the fixed per-lane offsets plus a
    // wave-uniform tile offset.  The ragged last tile (j0 > 0) moves its
    // window back to end at the last key, n - BC (its rows below j0 are
    // masked, they belong to the previous tile); a sequence shorter than a
    // tile starts at 0 and its rows past the end read zeros (the per-lane
    // offset is bounds checked).
    auto tile_base = [&](int j0) { return min(j0, max(n - BC, 0)); };
    auto issue_loads = [&](int j0, auto stage) {
        constexpr int st = decltype(stage)::value;
        char* kdst = (st ? ks1 : ks0) + wave * UPW * 1024;
        char* vdst = (st ? vs1 : vs0) + wave * UPW * 1024;
        const int so = __builtin_amdgcn_readfirstlane(tile_base(j0) * ROWB);
#pragma unroll
        for (int i = 0; i < UPW; ++i) {
            dma16(krs, kdst + i * 1024, kdo[i], so);
            dma16(vrs, vdst + i * 1024, vdo[i], so);
        }
    };

    // K row reads: row col (+32 kt), chunks 4 kc + 2 half + {0, 1}.
    int kpos[KC][2];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int u = 0; u < 2; ++u) kpos[kc][u] = col * ROWB + 16 * ((4 * kc + 2 * half + u) ^ swz8_k<D>(col));
    // V transpose reads: lane 16 g + 2 e + s addresses row 8 half + e (+16 r),
    // chunk 2 dt + (g & 1), bytes 8 s ..; the swizzle depends on row bits
    // that come from e alone.
    const int tg = lane >> 4, te = (lane & 15) >> 1, ts = lane & 1;
    int voff[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        voff[dt] = (8 * half + te) * ROWB + 16 * ((2 * dt + (tg & 1)) ^ swz8_v<D>(te)) + 8 * ts;

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16(0.f);
    float mref = -INFINITY;   // reference max (log2 units of scaled scores)
    float lsum = 0.f;

    auto compute = [&](auto stage, int j0) {
        constexpr int st = decltype(stage)::value;
        const char* kb = st ? ks1 : ks0;
        const char* vb = st ? vs1 : vs0;

        // S^T = K Q^T (raw scores of the codes, fp32).
        f32x16 s[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            s[kt] = f32x16(0.f);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const char* kr = kb + 32 * kt * ROWB;
                const u32x4 lo = *(const u32x4*)(kr + kpos[kc][0]);
                const u32x4 hi = *(const u32x4*)(kr + kpos[kc][1]);
                const i32x8 a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                s[kt] = mfma_fp8(a, qf[kc], s[kt]);
            }
        }

        // Keys past the end of a ragged last tile get score -inf, hence weight
        // exp2(-inf) = 0 (c is never 0).  One limit per sub-tile is compared
        // with the registers' constant row offsets; the empty volatile asm
        // keeps the block a branch (otherwise it is turned into selects that
        // every tile executes).
        if (j0 + BC > n) {
            asm volatile("");
            // only LDS rows [lo, hi) of the ragged tile hold its keys
            const int kb0 = tile_base(j0);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int lo = j0 - kb0 - 32 * kt - 4 * half, hi = n - kb0 - 32 * kt - 4 * half;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 8 * (r >> 2) + (r & 3);
                    if (row < lo || row >= hi) s[kt][r] = -INFINITY;
                }
            }
        }

        // Tile max in four independent chains (one per group of 4 registers).
        float mp[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mp[r >> 2] = fmaxf(mp[r >> 2], s[kt][r]);
        const float mt = pair_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]))) * c;

        // The reference moves only when a tile max exceeds it by more than
        // kFp8Slack (log2 units; 2^8.75 < 448, e4m3's largest value), and
        // then to kFp8Headroom below that max: the row's largest weight stays
        // in [2^7, 2^8.75], so weights stay in e4m3's normal range (>= 2^-6)
        // down to 2^-13 of it, and rescales are rare.
        if (__ballot(mt > mref + kFp8Slack)) {
            const float mnew = fmaxf(mref, mt - kFp8Headroom);
            const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
            lsum *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
            mref = mnew;
        }

#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kt][r] = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -mref));
        float part[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = kt ? 0 : 4; r < 16; ++r) part[r & 3] += s[kt][r];
        lsum += (part[0] + part[1]) + (part[2] + part[3]);

        // P^T as the B operand, straight from the accumulators: dword
        // w = 4 kt + q of lane half h holds keys 32 kt + 8 q + 4 h + 0..3.
        // The transpose read r of lane half h returns LDS rows 16 r + 8 h +
        // 0..7 of its 64-key group as dwords 2 r, 2 r + 1, and the V tile
        // stores key 16 r + 8 s + 4 h + e at LDS row 16 r + 8 h + 4 s + e,
        // so both operands pair the same key in every byte.
        int pw[8 * G];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                pw[4 * kt + q] = pack_fp8(s[kt][4 * q + 0], s[kt][4 * q + 1], s[kt][4 * q + 2], s[kt][4 * q + 3]);
        // O^T += V^T P^T: per 64-key group, four transpose reads of 8 keys
        // per operand.
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int* w = pw + 8 * g;
            const i32x8 bp = {w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]};
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                i32x2 r4[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    r4[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (lds_i32x2)(vb + (64 * g + 16 * r) * ROWB + voff[dt]));
                const i32x8 a = {r4[0].x, r4[0].y, r4[1].x, r4[1].y, r4[2].x, r4[2].y, r4[3].x, r4[3].y};
                acc[dt] = mfma_fp8(a, bp, acc[dt]);
            }
        }
    };

    const int ntiles = (n + BC - 1) / BC;
    issue_loads(0, Int<0>{});
    negate_q();
    for (int t = 0;;) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA landed
        __syncthreads();                      // ... every wave's; stage 1 is free
        if (t + 1 < ntiles) issue_loads((t + 1) * BC, Int<1>{});
        compute(Int<0>{}, t * BC);
        if (++t == ntiles) break;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (t + 1 < ntiles) issue_loads((t + 1) * BC, Int<0>{});
        compute(Int<1>{}, t * BC);
        if (++t == ntiles) break;
    }

    const float ltot = pair_sum(lsum);
    if (qrow < n) {
        const float inv = vscale / ltot;
        OutT* orow = O + base + (int64_t)qrow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float ov[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = acc[dt][4 * g + e] * inv;
                Store4<OutT>::run(orow + 32 * dt + 8 * g + 4 * half, ov);
            }
        if (half == 0) LSE[(int64_t)bh * n + qrow] = (mref + log2f(ltot)) * kLn2;
    }
}

template <int D, int BC, typename OutT>
hipError_t launch_fp8_t(const Fp8Args& a, hipStream_t stream) {
    constexpr int BR = 128;
    const int n = (int)a.n;
    const int qtiles = (int)((a.n + BR - 1) / BR);
    const int total = (int)(a.bh * qtiles);
    // The scores of the codes carry scale * dq * dk (formed in double); c =
    // |that| log2(e) rounded once, a negative product negates Q, zero is
    // passed as FLT_MIN (exp2_factor: -inf masked scores stay -inf).  The
    // caller has checked that c is finite.
    const double sc = (double)a.scale * (double)a.q_descale * (double)a.k_descale;
    float c = FLT_MIN;
    exp2_factor(sc, &c);
    const int negate = sc < 0.0 ? 1 : 0;
    const float vscale = a.v_descale;
    const uint8_t* q = (const uint8_t*)a.q;
    const uint8_t* k = (const uint8_t*)a.k;
    const uint8_t* v = (const uint8_t*)a.v;
    OutT* o = (OutT*)a.o;
    float* lse = a.lse;
    const int nh = (int)a.h, grp = (int)(a.h / a.hkv);
    void* args[] = {&q, &k, &v, &o, &lse, (void*)&n, (void*)&qtiles, (void*)&total, (void*)&c, (void*)&negate,
                    (void*)&vscale, (void*)&nh, (void*)&grp};
    return hipLaunchKernel((const void*)&flash_fwd_fp8<D, BC, OutT>, dim3(total), dim3(256), args, 0, stream);
}

template <typename OutT>
hipError_t launch_fp8_out(const Fp8Args& a, hipStream_t stream) {
    return a.d == 128 ? launch_fp8_t<128, 64, OutT>(a, stream) : launch_fp8_t<64, 64, OutT>(a, stream);
}

}  // namespace

hipError_t launch_forward_fp8(const Fp8Args& a, hipStream_t stream) {
    switch (a.out_dtype) {
        case FA_DTYPE_BF16: return launch_fp8_out<__bf16>(a, stream);
        case FA_DTYPE_FP16: return launch_fp8_out<_Float16>(a, stream);
        case FA_DTYPE_FP32: return launch_fp8_out<float>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
