// flash_bwd.hip — attention backward kernels for gfx950 (CDNA4), fp16/bf16.
//
// The pages describe the backward pass only in outline: the unite.ai page
// "Atención Flash: Revolucionando la Eficiencia de los Modelos de
// Transformador" (section "Introducción a la Atención Flash", item 2:
// recompute the attention matrix in the backward pass instead of storing it;
// section "Atención Flash-2", item 2: a faster backward pass) and the nisoo.com
// page "Un'immersione approfondita nell'algoritmo FlashAttention – parte 3"
// (recomputation trades floating-point work for memory traffic).  What is
// computed is the gradient of the forward definition, per query head:
//
//     S = scale Q K^T,  P = exp(S - LSE) (LSE from the forward pass),  O = P V
//     D_i  = sum_e dO_ie O_ie
//     dV   = P^T dO
//     dP   = dO V^T,   dS = P * (dP - D)
//     dQ   = scale dS K,   dK = scale dS^T Q
//
// with S and P recomputed tile by tile from Q, K and the saved LSE, so no
// N x N matrix is stored.  Grouped K/V heads: dK and dV of a K/V head add up
// over the query heads that share it.
//
// Kernels:
//   flash_bwd_dot   D_i = <dO_i, O_i> in fp32 (one row per 16 lanes).
//   flash_bwd_dq    8 waves (d = 128) or 4 (d = 64) x 32 query rows; K/V
//                   tiles of 64 keys streamed through a three-stage (d = 128)
//                   or two-stage LDS ring:
//                   S^T = K Q^T, P^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
//   flash_bwd_dkdv_pp (d = 128) 8 waves x 32 keys in two groups one phase
//                   apart; flash_bwd_dkdv (d = 64) 4 waves x 32 keys; Q/dO
//                   tiles of 32 queries streamed through LDS: S = Q K^T, P,
//                   dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS.
// Every product runs on v_mfma_f32_32x32x16_{bf16,f16} with fp32
// accumulation; weights P and dS are rounded to the input type for the
// second products.  An accumulator (lane = column, registers = rows) feeds
// the B operand of the next product directly, its rows becoming the
// contraction index (chunk c2 of 16: registers 8 c2 .. 8 c2 + 7 hold rows
// 16 c2 + {0..3, 8..11} + 4 half); the A operand then supplies the same rows
// through the LDS transpose read ds_read_b64_tr_b16.
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"
#include "../../include/fa.h"

#include "fa_device.h"

namespace fa {
namespace {

// Swizzle for tiles read both ways: row reads (16 lanes, one chunk of 16
// consecutive rows) and transpose reads (4 consecutive rows x 4 consecutive
// chunks per 32 lanes).  For d = 128 (16 chunks per 256-byte row)
// f(r) = 4 (r mod 4) + (r / 4 mod 4) is a bijection on any 16 consecutive rows
// and maps rows 4m .. 4m+3 to 4t + (m mod 4), so chunk groups 4u.. land on
// 16 distinct positions; for d = 64 (two 128-byte rows per 256 bytes) the
// same two properties hold for rows of equal parity.
template <int D> __device__ __forceinline__ constexpr int swz_rt(int r) {
    return D == 128 ? (4 * (r & 3) + ((r >> 2) & 3)) : ((4 * ((r >> 1) & 1)) ^ ((r >> 2) & 3));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4;

// A operand from a transposed tile (swizzle swz_rt): lane (col, half) of
// column block dt receives, for contraction rows 16 c2 + {0..3, 8..11} +
// 4 half of a row-major tile (ROWB-byte rows), element 32 dt + col of each
// row.  The lane reads two 4-row halves.  With swz_rt, the offset of column
// block dt is the block-0 offset XOR 64 dt (the swizzle only permutes the
// chunk bits that dt does not touch), and the +8-row half sits at the
// 4-row offset XOR 32 (swz_rt(r + 8) = swz_rt(r) ^ 2) plus 8 rows; so one
// offset per lane, tr_offset0, serves every block and half.
template <int ROWB>
__device__ __forceinline__ u32x4 read_tr(const char* tile, int c2row0, int off0, int dt) {
    const char* t = tile + c2row0 * ROWB;
    const int lo = off0 ^ (64 * dt);
    const int hi = (lo ^ 32) + 8 * ROWB;
    const s16x4 l = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(t + lo));
    const s16x4 h = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(t + hi));
    const u32x2 l2 = __builtin_bit_cast(u32x2, l), h2 = __builtin_bit_cast(u32x2, h);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
}

// Block-0 offset: lane 4t+s of each 16-lane group addresses row t (+4 half)
// and the 4-element segment s of the group's 16 columns; rows are taken mod
// 16 for the swizzle (chunks c2 start at multiples of 16 rows).
template <int D>
__device__ __forceinline__ int tr_offset0(int lane) {
    constexpr int ROWB = 2 * D;
    const int half = lane >> 5;
    const int trt = (lane & 15) >> 2, trs = lane & 3, trg = (lane >> 4) & 1;
    const int r = 4 * half + trt;
    const int ch = 2 * trg + (trs >> 1);
    return r * ROWB + 16 * (ch ^ swz_rt<D>(r)) + 8 * (trs & 1);
}

// ---------------------------------------------------------------------------
// D_i = sum_e dO_ie O_ie, fp32.  16 lanes per row, 8 elements per lane.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256)
flash_bwd_dot(const T* __restrict__ O, const T* __restrict__ dO, float* __restrict__ Dr, int64_t rows)
{
    constexpr int LPR = D / 8;               // lanes per row
    // Grid-stride over rows; the stride is a multiple of LPR, so the LPR
    // lanes of a row stay together (and active together) on every pass.
    const int64_t stride = (int64_t)gridDim.x * (256 / LPR);
    const int part = threadIdx.x % LPR;
    for (int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR; row < rows; row += stride) {
        const u32x4 a = *(const u32x4*)(O + row * D + 8 * part);
        const u32x4 b = *(const u32x4*)(dO + row * D + 8 * part);
        typedef T t8 __attribute__((ext_vector_type(8)));
        const t8 x = __builtin_bit_cast(t8, a), y = __builtin_bit_cast(t8, b);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
        if (part == 0) Dr[row] = acc;
    }
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup: NW waves x 32 query rows of one (b, h); K/V tiles of 64
// keys.  d = 128: 8 waves (one workgroup per CU), so that each K/V tile
// brought into LDS serves 256 query rows, through a three-stage ring;
// d = 64: 4 waves, three workgroups per CU, two stages.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(D == 128 ? 512 : 256) __attribute__((amdgpu_waves_per_eu(2)))
flash_bwd_dq(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
             const T* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dr,
             T* __restrict__ dQ, int n, int qtiles, int total, float c, float scale, int nh, int grp)
{
    using M = Mfma<T>;
    constexpr int NW = D == 128 ? 8 : 4;
    constexpr int NST = D == 128 ? 3 : 2;    // LDS stages of the K/V ring
    constexpr int BC = 64;
    constexpr int BR = 32 * NW;
    constexpr int ROWB = D * 2;
    constexpr int CPR = D / 8;
    constexpr int RPU = 64 / CPR;
    constexpr int TILEB = BC * ROWB;
    constexpr int UNITS = TILEB / 1024;
    constexpr int UPW = UNITS / NW;
    constexpr int KT = BC / 32;
    constexpr int DT = D / 32;
    constexpr int KC = D / 16;
    constexpr int PC = BC / 16;
    static_assert(UNITS % NW == 0, "tile shape");

    __shared__ __attribute__((aligned(1024))) char ks0[TILEB];
    __shared__ __attribute__((aligned(1024))) char vs0[TILEB];
    __shared__ __attribute__((aligned(1024))) char ks1[TILEB];
    __shared__ __attribute__((aligned(1024))) char vs1[TILEB];
    __shared__ __attribute__((aligned(1024))) char ks2[NST > 2 ? TILEB : 16];
    __shared__ __attribute__((aligned(1024))) char vs2[NST > 2 ? TILEB : 16];
    auto kst = [&](auto stage) -> char* {
        constexpr int st = decltype(stage)::value;
        return st == 0 ? ks0 : st == 1 ? ks1 : ks2;
    };
    auto vst = [&](auto stage) -> char* {
        constexpr int st = decltype(stage)::value;
        return st == 0 ? vs0 : st == 1 ? vs1 : vs2;
    };

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
    const int qrc = min(qrow, n - 1);

    // Q^T and dO^T as B operands: lane (col, half) holds row qrow, elements
    // 16 kc + 8 half + 0..7.  Rows past the end are clamped (never stored).
    u32x4 qf[KC], of[KC];
    {
        const T* qp = Q + base + (int64_t)qrc * D + 8 * half;
        const T* op = dO + base + (int64_t)qrc * D + 8 * half;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            qf[kc] = *(const u32x4*)(qp + 16 * kc);
            of[kc] = *(const u32x4*)(op + 16 * kc);
        }
    }
    const float lse2 = LSE[(int64_t)bh * n + qrc] * 1.4426950408889634f;   // log2 units
    const float dval = Dr[(int64_t)bh * n + qrc];

    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(K + kvbase), (short)0, n * ROWB, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(V + kvbase), (short)0, n * ROWB, 0x00020000);

    // K is read row-wise (S^T) and transposed (dQ^T): swizzle swz_rt; V only
    // row-wise: swz_k.
    const int lrow = lane / CPR;
    const int lch = lane % CPR;
    // One DMA form for every key tile: per-lane offsets within the tile
    // plus a wave-uniform tile offset.  The ragged last tile's window ends at
    // the last key (its rows below the tile's first key are masked: they
    // belong to the previous tile); a sequence shorter than one tile reads
    // zeros past its end (the per-lane offset is bounds checked).
    auto tile_base = [&](int j0) { return min(j0, max(n - BC, 0)); };
    auto issue_loads = [&](int j0, auto stage) {
        char* kdst = kst(stage) + wave * UPW * 1024;
        char* vdst = vst(stage) + wave * UPW * 1024;
        const int so = __builtin_amdgcn_readfirstlane(tile_base(j0) * ROWB);
#pragma unroll
        for (int i = 0; i < UPW; ++i) {
            const int r = (wave * UPW + i) * RPU + lrow;
            dma16(krs, kdst + i * 1024, r * ROWB + 16 * (lch ^ swz_rt<D>(r)), so);
            dma16(vrs, vdst + i * 1024, r * ROWB + 16 * (lch ^ swz_k<D>(r)), so);
        }
    };

    // LDS read offsets (as in the dK/dV kernel): row reads of step (kt, kc)
    // at row 32 kt + col, chunk 2 kc + half under the row's swizzle, i.e. the
    // kc = 0 offset XOR 32 kc; transpose reads from tr_offset0.  Made opaque
    // once per tile so that the per-step offsets are not kept across the loop.
    const int koff = col * ROWB + 16 * (half ^ swz_rt<D>(col));
    const int voff = col * ROWB + 16 * (half ^ swz_k<D>(col));
    const int ktr = tr_offset0<D>(lane);

    f32x16 acc[DT];   // dQ^T (d x queries)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16(0.f);

    // One K/V tile as a fixed program (sched_barrier between steps):
    // S^T/dP^T steps (kt, kc) (two MFMAs each: K row x Q^T, V row x dO^T),
    // the P^T/dS^T vector work, then dQ^T steps (pc, dt) (one MFMA each, K
    // through the transpose read).  LDS operands run RQ steps ahead through
    // `qring` (1 step for S/dP, 2 for dQ: deeper rings spill at d = 128);
    // the first dQ^T operands are read before the vector work.
    constexpr int RQ = 1;
    u32x4 qring[2 * RQ];
    auto compute = [&](auto stage, int j0) {
        const char* kb = kst(stage);
        const char* vb = vst(stage);
        int ko = koff, vo = voff, to = ktr;
        asm volatile("" : "+v"(ko), "+v"(vo), "+v"(to));
        constexpr int N1 = KT * KC;
        auto read1 = [&](auto step) {
            constexpr int i = decltype(step)::value;
            constexpr int kt = i / KC, kc = i % KC;
            qring[2 * (i % RQ) + 0] = *(const u32x4*)(kb + 32 * kt * ROWB + (ko ^ (32 * kc)));
            qring[2 * (i % RQ) + 1] = *(const u32x4*)(vb + 32 * kt * ROWB + (vo ^ (32 * kc)));
        };
        // S^T = K Q^T and dP^T = V dO^T (keys x queries).
        f32x16 s[KT], dp[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) { s[kt] = f32x16(0.f); dp[kt] = f32x16(0.f); }
        static_for<0, RQ>([&](auto i) { read1(i); });
        // Matrix programs run at raised issue priority and the vector work at
        // the normal one: on a SIMD shared with another workgroup's wave, a
        // product whose operands are ready goes ahead of that wave's vector
        // instructions.
        __builtin_amdgcn_s_setprio(1);
        static_for<0, N1>([&](auto step) {
            constexpr int i = decltype(step)::value;
            constexpr int kt = i / KC, kc = i % KC;
            __builtin_amdgcn_sched_barrier(0);
            s[kt] = M::run(qring[2 * (i % RQ) + 0], qf[kc], s[kt]);
            dp[kt] = M::run(qring[2 * (i % RQ) + 1], of[kc], dp[kt]);
            if constexpr (i + RQ < N1) read1(Int<i + RQ>{});
        });
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        constexpr int N2 = PC * DT;
        auto read2 = [&](auto step) {
            constexpr int i = decltype(step)::value;
            constexpr int pc = i / DT, dt = i % DT;
            qring[i % (2 * RQ)] = read_tr<ROWB>(kb, 16 * pc, to, dt);
        };
        static_for<0, 2 * RQ>([&](auto i) { read2(i); });
        // P^T = exp2(S^T c - LSE log2 e); dS^T = P^T (dP^T - D).  Rows of a
        // ragged last tile that hold no key of it (below its first key, or
        // zeros past the end) get dS = 0, in a branch taken by that tile only:
        // two limits per sub-tile against the registers' constant row offsets,
        // and the empty volatile asm keeps the compiler from turning it into
        // selects that every tile executes.
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -lse2));
                s[kt][r] = pr * (dp[kt][r] - dval);
            }
        if (j0 + BC > n) {
            asm volatile("");
            const int kb = tile_base(j0);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int lo = j0 - kb - 32 * kt - 4 * half, hi = n - kb - 32 * kt - 4 * half;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 8 * (r >> 2) + (r & 3);
                    if (row < lo || row >= hi) s[kt][r] = 0.f;
                }
            }
        }
        u32x4 bsv[PC];
#pragma unroll
        for (int pc = 0; pc < PC; ++pc) {
            float w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = s[pc >> 1][8 * (pc & 1) + e];
            bsv[pc] = M::pack(w);
        }
        // dQ^T += K^T dS^T.
        __builtin_amdgcn_s_setprio(1);
        static_for<0, N2>([&](auto step) {
            constexpr int i = decltype(step)::value;
            constexpr int pc = i / DT, dt = i % DT;
            __builtin_amdgcn_sched_barrier(0);
            acc[dt] = M::run(qring[i % (2 * RQ)], bsv[pc], acc[dt]);
            if constexpr (i + 2 * RQ < N2) read2(Int<i + 2 * RQ>{});
        });
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    };

    const int ntiles = (n + BC - 1) / BC;
    if constexpr (NST == 2) {
        issue_loads(0, Int<0>{});
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
    } else {
        // Three stages: tile t in stage t mod 3; the DMA of tile t + 2 goes
        // out at the top of step t into the stage of tile t - 1, which every
        // wave finished reading in step t - 1.  Each wave waits only for tile
        // t's DMA (tile t + 1's, 2 UPW instructions, may still be in flight)
        // before a barrier without a fence (a fence waits for every load).
        // Tiles past the end are loaded too (never read), and the loop has
        // one exit, so the compiler's tracking of the loads stays exact.
        issue_loads(0, Int<0>{});
        issue_loads(BC, Int<1>{});
        static_assert(2 * UPW <= 15, "wait count below");
        auto stepk = [&](int t, auto stage) __attribute__((always_inline)) {
            constexpr int S = decltype(stage)::value;
            __builtin_amdgcn_s_waitcnt(0x0070 | (2 * UPW));   // vmcnt(2 UPW) lgkmcnt(0)
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            issue_loads((t + 2) * BC, Int<(S + 2) % 3>{});
            compute(stage, t * BC);
        };
        stepk(0, Int<0>{});
        int t = 1;
        for (; t + 3 <= ntiles; t += 3) {
            stepk(t, Int<1>{});
            stepk(t + 1, Int<2>{});
            stepk(t + 2, Int<0>{});
        }
        if (t < ntiles) stepk(t++, Int<1>{});
        if (t < ntiles) stepk(t++, Int<2>{});
        __builtin_amdgcn_s_waitcnt(0x0070);       // no DMA into LDS left in flight
    }

    if (qrow < n) {
        T* row = dQ + base + (int64_t)qrow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = acc[dt][4 * g + e] * scale;
                *(u32x2*)(row + 32 * dt + 8 * g + 4 * half) = M::pack4(v4);
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV.  Workgroup: 4 waves x 32 keys of one (b, K/V head); the queries of
// every query head sharing that K/V head stream through LDS, 32 at a time.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
flash_bwd_dkdv(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
               const T* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dr,
               T* __restrict__ dK, T* __restrict__ dV, int n, int ktiles, int total, float c, float scale,
               int nh, int grp)
{
    using M = Mfma<T>;
    constexpr int NW = 4;
    constexpr int BQ = 32;                   // queries per streamed tile
    constexpr int BK = 32 * NW;              // keys per workgroup
    constexpr int ROWB = D * 2;
    constexpr int CPR = D / 8;
    constexpr int RPU = 64 / CPR;
    constexpr int QTILEB = BQ * ROWB;
    constexpr int QUNITS = QTILEB / 1024;    // DMA units of a Q (or dO) tile
    constexpr int VTILEB = BK * ROWB;
    constexpr int VUNITS = VTILEB / 1024;
    constexpr int DT = D / 32;
    constexpr int KC = D / 16;
    static_assert(QUNITS <= NW * 2 && VUNITS % NW == 0 && 2 * BQ == 64, "tile shape");

    __shared__ __attribute__((aligned(1024))) char vs[VTILEB];
    __shared__ __attribute__((aligned(1024))) char qs0[QTILEB];
    __shared__ __attribute__((aligned(1024))) char os0[QTILEB];
    __shared__ __attribute__((aligned(1024))) char qs1[QTILEB];
    __shared__ __attribute__((aligned(1024))) char os1[QTILEB];
    __shared__ __attribute__((aligned(16))) float ls0[2 * BQ];   // LSE log2 e, then D
    __shared__ __attribute__((aligned(16))) float ls1[2 * BQ];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;

    const int tile = xcd_tile(blockIdx.x, total);
    const int bkv = tile / ktiles;           // b * Hkv + g
    const int kt0 = (tile - bkv * ktiles) * BK;
    const int nkv = nh / grp;
    const int b = bkv / nkv, g = bkv - b * nkv;
    const int64_t kvbase = (int64_t)bkv * n * D;
    const int key = kt0 + wave * 32 + col;   // this lane's key (column of S)
    const int keyc = min(key, n - 1);

    // K^T as the B operand of S = Q K^T: lane (col, half) holds K[key][16 kc +
    // 8 half + 0..7].
    u32x4 kf[KC];
    {
        const T* kp = K + kvbase + (int64_t)keyc * D + 8 * half;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) kf[kc] = *(const u32x4*)(kp + 16 * kc);
    }

    const int lrow = lane / CPR;
    const int lch = lane % CPR;
    // V tile of the workgroup's keys (rows past the end re-read the last row).
    {
        const __amdgpu_buffer_rsrc_t vrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(V + kvbase), (short)0, n * ROWB, 0x00020000);
#pragma unroll
        for (int i = 0; i < VUNITS / NW; ++i) {
            const int r = (wave * (VUNITS / NW) + i) * RPU + lrow;
            dma16(vrs, vs + (wave * (VUNITS / NW) + i) * 1024,
                  min(kt0 + r, n - 1) * ROWB + 16 * (lch ^ swz_k<D>(r)), 0);
        }
    }

    // One streamed tile: 32 query rows of Q and dO of query head h (swizzle
    // swz_rt: read row-wise and transposed), their LSE (log2 units) and D.
    // Units: wave w moves units w and w + 4 of the Q and dO tiles (QUNITS <= 8
    // each); wave 0 also stores LSE and D, loaded into a register one tile
    // earlier by load_lv (lanes 0..31: LSE, lanes 32..63: D).
    // First query row held by the LDS tile of the query tile at i0: i0 for
    // a full tile; the ragged last tile's window ends at the last query (its
    // rows below i0 are masked, they belong to the previous tile); a sequence
    // shorter than one tile starts at 0 and reads zeros past its end (the
    // per-lane offset is bounds checked).  So every Q/dO DMA has one form.
    auto qtile_base = [&](int i0) { return min(i0, max(n - BQ, 0)); };
    auto load_lv = [&](int h, int i0) {
        float lv = 0.f;
        if (wave == 0) {
            int ln;   // opaque lane copy: the per-lane address is not kept (and spilled) across the loop
            asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
            const int64_t rowi = ((int64_t)b * nh + h) * n + min(qtile_base(i0) + (ln & (BQ - 1)), n - 1);
            lv = (ln < BQ ? LSE : Dr)[rowi];
        }
        return lv;
    };
    auto issue_tile = [&](int h, int i0, auto stage, float lv) {
        constexpr int st = decltype(stage)::value;
        char* qd = st ? qs1 : qs0;
        char* od = st ? os1 : os0;
        float* ld = st ? ls1 : ls0;
        // Per-lane offsets are recomputed here from an opaque copy of the lane
        // index: hoisted out of the loop they would be spilled, and reloads
        // between the DMAs make each DMA wait for the one before it.
        int ln;
        asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
        const int lr = ln / CPR, lc = ln % CPR;
        // LSE / D first: a store after the DMAs would wait for them.
        if (wave == 0) ld[ln] = ln < BQ ? lv * 1.4426950408889634f : lv;   // 2 BQ == 64 lanes
        const int64_t qbase = ((int64_t)b * nh + h) * n * D;
        const __amdgpu_buffer_rsrc_t qrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(Q + qbase), (short)0, n * ROWB, 0x00020000);
        const __amdgpu_buffer_rsrc_t ors =
            __builtin_amdgcn_make_buffer_rsrc((void*)(dO + qbase), (short)0, n * ROWB, 0x00020000);
        const int so = __builtin_amdgcn_readfirstlane(qtile_base(i0) * ROWB);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int u = wave + NW * k;
            if (u < QUNITS) {
                const int r = u * RPU + lr;
                const int gofs = r * ROWB + 16 * (lc ^ swz_rt<D>(r));
                dma16(qrs, qd + u * 1024, gofs, so);
                dma16(ors, od + u * 1024, gofs, so);
            }
        }
    };

    // LDS read offsets.  Row reads of step kc: row col (Q, dO) or this lane's
    // key (V), chunk 2 kc + half under the row's swizzle; since rows are
    // ROWB >= 128 bytes, the offset is the kc = 0 offset XOR 32 kc.  Transpose
    // reads: tr_offset0 (see read_tr).  The three offsets are made opaque once
    // per tile (see compute): hoisted, the compiler keeps one register per
    // (step, operand) offset across the loop and spills at d = 128.
    const int qoff = col * ROWB + 16 * (half ^ swz_rt<D>(col));
    const int voff = (wave * 32 + col) * ROWB + 16 * (half ^ swz_k<D>(col));
    const int qtr = tr_offset0<D>(lane);

    f32x16 dka[DT], dva[DT];   // dK^T, dV^T (d x keys)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) { dka[dt] = f32x16(0.f); dva[dt] = f32x16(0.f); }

    // One streamed tile as a fixed program (sched_barrier between steps):
    // S/dP steps kc = 0..KC-1 (two MFMAs each: Q row x K, dO row x V), the
    // P/dS vector work, then dV/dK steps (c2, dt) (two MFMAs each, operands
    // from the transpose reads of dO and Q).  LDS operands run RB steps
    // ahead through `ring`: two at d = 128 (3-6 % faster than one, for a few
    // more spilled scalars; three spill inside the loop), one at d = 64 (two
    // are 24 % slower there); the first dV/dK operands are read before the
    // vector work.
    constexpr int RB = D == 128 ? 2 : 1;
    u32x4 ring[3 * RB];
    auto compute = [&](auto stage, int i0) {
        constexpr int st = decltype(stage)::value;
        const char* qb = st ? qs1 : qs0;
        const char* ob = st ? os1 : os0;
        const float* lb = st ? ls1 : ls0;
        int qo = qoff, vo = voff, to = qtr;
        asm volatile("" : "+v"(qo), "+v"(vo), "+v"(to));
        auto read1 = [&](auto step) {
            constexpr int kc = decltype(step)::value;
            ring[3 * (kc % RB) + 0] = *(const u32x4*)(qb + (qo ^ (32 * kc)));
            ring[3 * (kc % RB) + 1] = *(const u32x4*)(ob + (qo ^ (32 * kc)));
            ring[3 * (kc % RB) + 2] = *(const u32x4*)(vs + (vo ^ (32 * kc)));
        };
        // S = Q K^T and dP = dO V^T (queries x keys).
        f32x16 s = f32x16(0.f), dp = f32x16(0.f);
        static_for<0, RB>([&](auto i) { read1(i); });
        // Matrix programs run at raised issue priority and the vector work at
        // the normal one: on a SIMD shared with another workgroup's wave, a
        // product whose operands are ready goes ahead of that wave's vector
        // instructions.
        __builtin_amdgcn_s_setprio(1);
        static_for<0, KC>([&](auto step) {
            constexpr int kc = decltype(step)::value;
            __builtin_amdgcn_sched_barrier(0);
            s = M::run(ring[3 * (kc % RB) + 0], kf[kc], s);
            dp = M::run(ring[3 * (kc % RB) + 1], ring[3 * (kc % RB) + 2], dp);
            if constexpr (kc + RB < KC) read1(Int<kc + RB>{});
        });
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        // dV/dK step i = c2 * DT + dt: operands tr(dO) and tr(Q), rows 16 c2.
        auto read2 = [&](auto step) {
            constexpr int i = decltype(step)::value;
            constexpr int c2 = i / DT, dt = i % DT;
            ring[2 * (i % RB) + 0] = read_tr<ROWB>(ob, 16 * c2, to, dt);
            ring[2 * (i % RB) + 1] = read_tr<ROWB>(qb, 16 * c2, to, dt);
        };
        static_for<0, RB>([&](auto i) { read2(i); });
        // P = exp2(S c - LSE log2 e), dS = P (dP - D); register r holds query
        // row 8 (r / 4) + 4 half + r % 4: rows 8 q4 + 4 half .. +3 are four
        // consecutive floats.  Query rows past the end get P = dS = 0 (set,
        // not multiplied: their LSE and D slots need not be finite), in a
        // branch taken by a ragged last query block only (see the dQ kernel).
        float p[16], ds[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 l4 = *(const float4*)(lb + 8 * q4 + 4 * half);
            const float4 d4 = *(const float4*)(lb + BQ + 8 * q4 + 4 * half);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * q4 + e;
                const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lv[e]));
                p[r] = pr;
                ds[r] = pr * (dp[r] - dv[e]);
            }
        }
        if (i0 + BQ > n) {
            asm volatile("");
            // only rows [lo, hi) of a ragged query tile hold its queries
            const int qb = qtile_base(i0);
            const int lo = i0 - qb - 4 * half, hi = n - qb - 4 * half;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r >> 2) + (r & 3);
                if (row < lo || row >= hi) {
                    p[r] = 0.f;
                    ds[r] = 0.f;
                }
            }
        }
        const u32x4 bp[2] = {M::pack(&p[0]), M::pack(&p[8])};
        const u32x4 bs[2] = {M::pack(&ds[0]), M::pack(&ds[8])};
        // dV^T += dO^T P and dK^T += Q^T dS (contraction over the 32 queries).
        __builtin_amdgcn_s_setprio(1);
        static_for<0, 2 * DT>([&](auto step) {
            constexpr int i = decltype(step)::value;
            constexpr int c2 = i / DT, dt = i % DT;
            __builtin_amdgcn_sched_barrier(0);
            dva[dt] = M::run(ring[2 * (i % RB) + 0], bp[c2], dva[dt]);
            dka[dt] = M::run(ring[2 * (i % RB) + 1], bs[c2], dka[dt]);
            if constexpr (i + RB < 2 * DT) read2(Int<i + RB>{});
        });
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    };

    // Stream (query head, query tile) pairs: heads g grp .. g grp + grp - 1,
    // each over its query tiles.  Cursors (head, first row) of tiles t + 1 and
    // t + 2 advance by one tile per step (no divisions in the loop).
    const int steps = grp * ((n + BQ - 1) / BQ);
    auto advance = [&](int& h, int& r) {
        r += BQ;
        if (r >= n) { r = 0; ++h; }
    };
    int h1 = g * grp, r1 = 0;
    issue_tile(h1, r1, Int<0>{}, load_lv(h1, r1));
    advance(h1, r1);
    int h2 = h1, r2 = r1;
    float lv_next = steps > 1 ? load_lv(h2, r2) : 0.f;
    advance(h2, r2);
    int r0 = 0;
    // At the top of tile t (after the barrier, so every wave is done with
    // the other stage): the LSE/D store and Q/dO DMA of tile t + 1 into the
    // other stage (its LSE/D loaded one tile earlier), then the LSE/D load
    // of tile t + 2; all land while tile t computes.
    auto next = [&](int t, auto stage) {
        if (t + 1 < steps) {
            issue_tile(h1, r1, stage, lv_next);
            if (t + 2 < steps) lv_next = load_lv(h2, r2);
            h1 = h2; r1 = r2;
            advance(h2, r2);
        }
    };
    for (int t = 0;;) {
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): own loads and LDS stores done
        __syncthreads();
        next(t, Int<1>{});
        compute(Int<0>{}, r0);
        if (++t == steps) break;
        r0 = r0 + BQ >= n ? 0 : r0 + BQ;
        __builtin_amdgcn_s_waitcnt(0x0070);
        __syncthreads();
        next(t, Int<0>{});
        compute(Int<1>{}, r0);
        if (++t == steps) break;
        r0 = r0 + BQ >= n ? 0 : r0 + BQ;
    }

    if (key < n) {
        T* krow = dK + kvbase + (int64_t)key * D;
        T* vrow_out = dV + kvbase + (int64_t)key * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                float k4[4], v4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    k4[e] = dka[dt][4 * gq + e] * scale;
                    v4[e] = dva[dt][4 * gq + e];
                }
                *(u32x2*)(krow + 32 * dt + 8 * gq + 4 * half) = M::pack4(k4);
                *(u32x2*)(vrow_out + 32 * dt + 8 * gq + 4 * half) = M::pack4(v4);
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV at d = 128 with two wave groups in alternating phases.  Workgroup:
// 8 waves x 32 keys of one (b, K/V head), 256 keys; waves w and w + 4 share a
// SIMD.  The 32-query tiles of Q and dO (with their LSE and D) stream through
// a three-stage LDS ring.  Every wave runs MFMA phase j (S_j = Q_j K^T and
// dP_j = dO_j V^T, then dV^T += dO_{j-1}^T P_{j-1} and dK^T += Q_{j-1}^T
// dS_{j-1}), a workgroup barrier, vector phase j (P_j, dS_j), a barrier;
// group 1 runs one phase behind group 0, so on every SIMD one wave feeds the
// matrix core while the other computes exponentials.  Group 1 loads tile
// j + 2 at the start of its vector phase j, into the stage of tile j - 1
// (last read in its own MFMA phase j, one phase after group 0's), and waits
// for the loads before the barrier that ends the phase; group 0 first reads
// the tile two phases later.  No load is in flight during an MFMA phase.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
flash_bwd_dkdv_pp(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                  const T* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dr,
                  T* __restrict__ dK, T* __restrict__ dV, int n, int ktiles, int total, float c, float scale,
                  int nh, int grp)
{
    using M = Mfma<T>;
    constexpr int NW = 8;
    constexpr int BQ = 32;                   // queries per streamed tile
    constexpr int BK = 32 * NW;              // keys per workgroup
    constexpr int ROWB = D * 2;
    constexpr int CPR = D / 8;
    constexpr int RPU = 64 / CPR;
    constexpr int QTILEB = BQ * ROWB;
    constexpr int QUNITS = QTILEB / 1024;    // DMA units of a Q (or dO) tile
    constexpr int VTILEB = BK * ROWB;
    constexpr int VUNITS = VTILEB / 1024;
    constexpr int DT = D / 32;
    constexpr int KC = D / 16;
    constexpr int RB = 2;                    // LDS operand read-ahead (steps)
    static_assert(D == 128 && QUNITS == 8 && VUNITS % NW == 0 && 2 * BQ == 64, "tile shape");

    // Stage s of the Q and dO tiles at s * QTILEB, of their LSE (log2 units)
    // and D at s * 2 BQ; then the workgroup's V rows.
    __shared__ __attribute__((aligned(1024))) char qs[3 * QTILEB];
    __shared__ __attribute__((aligned(1024))) char os[3 * QTILEB];
    __shared__ __attribute__((aligned(16))) float ls[3 * 2 * BQ];
    __shared__ __attribute__((aligned(1024))) char vs[VTILEB];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int group = wave >> 2;
    const int gw = wave & 3;
    const int col = lane & 31;
    const int half = lane >> 5;

    const int tile = xcd_tile(blockIdx.x, total);
    const int bkv = tile / ktiles;           // b * Hkv + g
    const int kt0 = (tile - bkv * ktiles) * BK;
    const int nkv = nh / grp;
    const int b = bkv / nkv, g = bkv - b * nkv;
    const int64_t kvbase = (int64_t)bkv * n * D;
    const int key = kt0 + wave * 32 + col;   // this lane's key (column of S)
    const int keyc = min(key, n - 1);

    // K^T as the B operand of S = Q K^T: lane (col, half) holds K[key][16 kc +
    // 8 half + 0..7].
    u32x4 kf[KC];
    {
        const T* kp = K + kvbase + (int64_t)keyc * D + 8 * half;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) kf[kc] = *(const u32x4*)(kp + 16 * kc);
    }

    const int lrow = lane / CPR;
    const int lch = lane % CPR;
    // V rows of the workgroup's keys (rows past the end re-read the last row).
    {
        const __amdgpu_buffer_rsrc_t vrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(V + kvbase), (short)0, n * ROWB, 0x00020000);
#pragma unroll
        for (int i = 0; i < VUNITS / NW; ++i) {
            const int u = wave * (VUNITS / NW) + i;
            const int r = u * RPU + lrow;
            dma16(vrs, vs + u * 1024, min(kt0 + r, n - 1) * ROWB + 16 * (lch ^ swz_k<D>(r)), 0);
        }
    }

    // Loads of group 1.  load_lv: wave 4 reads a tile's LSE (lanes 0..31) and
    // D (lanes 32..63) into a register; issue_tile: its LSE / D into LDS
    // (first: a store after the DMAs would wait for them), then the Q and dO
    // units gw and gw + 4 of the tile.  Per-lane offsets come from an opaque
    // copy of the lane index, so that they are not kept across the loop.
    // First query row held by the LDS tile of the query tile at i0: i0 for
    // a full tile; the ragged last tile's window ends at the last query (its
    // rows below i0 are masked, they belong to the previous tile); a sequence
    // shorter than one tile starts at 0 and reads zeros past its end (the
    // per-lane offset is bounds checked).  So every Q/dO DMA has one form.
    auto qtile_base = [&](int i0) { return min(i0, max(n - BQ, 0)); };
    auto load_lv = [&](int h, int i0) {
        float lv = 0.f;
        if (wave == 4) {
            int ln;
            asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
            const int64_t rowi = ((int64_t)b * nh + h) * n + min(qtile_base(i0) + (ln & (BQ - 1)), n - 1);
            lv = (ln < BQ ? LSE : Dr)[rowi];
        }
        return lv;
    };
    auto issue_tile = [&](int h, int i0, int st, float lv) {
        int ln;
        asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
        const int lr = ln / CPR, lc = ln % CPR;
        if (wave == 4) ls[st * 2 * BQ + ln] = ln < BQ ? lv * 1.4426950408889634f : lv;
        const int64_t qbase = ((int64_t)b * nh + h) * n * D;
        const __amdgpu_buffer_rsrc_t qrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(Q + qbase), (short)0, n * ROWB, 0x00020000);
        const __amdgpu_buffer_rsrc_t ors =
            __builtin_amdgcn_make_buffer_rsrc((void*)(dO + qbase), (short)0, n * ROWB, 0x00020000);
        const int so = __builtin_amdgcn_readfirstlane(qtile_base(i0) * ROWB);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int u = gw + 4 * k;
            const int r = u * RPU + lr;
            const int gofs = r * ROWB + 16 * (lc ^ swz_rt<D>(r));
            dma16(qrs, qs + st * QTILEB + u * 1024, gofs, so);
            dma16(ors, os + st * QTILEB + u * 1024, gofs, so);
        }
    };

    // LDS read offsets (as in flash_bwd_dkdv); the stage offsets are
    // multiples of 8 KiB, which the XOR forms leave untouched.
    const int qoff = col * ROWB + 16 * (half ^ swz_rt<D>(col));
    const int voff = (wave * 32 + col) * ROWB + 16 * (half ^ swz_k<D>(col));
    const int qtr = tr_offset0<D>(lane);

    f32x16 dka[DT], dva[DT];   // dK^T, dV^T (d x keys)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) { dka[dt] = f32x16(0.f); dva[dt] = f32x16(0.f); }
    f32x16 s = f32x16(0.f), dp = f32x16(0.f);   // S and dP of the current tile
    u32x4 bp[2], bs[2];                         // P and dS of the previous tile (B operands)
    u32x4 ring[3 * RB];

    // MFMA phase as a fixed program: S/dP steps kc (Q row x K, dO row x V),
    // then dV/dK steps (c2, dt) (transposed dO and Q of the previous tile).
    auto mphase = [&](int stc, int stp, auto has_sdp, auto has_dvdk) {
        constexpr int N1 = decltype(has_sdp)::value ? KC : 0;
        constexpr int N2 = decltype(has_dvdk)::value ? 2 * DT : 0;
        constexpr int NS = N1 + N2;
        int qo = qoff + stc * QTILEB, vo = voff, to = qtr + stp * QTILEB;
        asm volatile("" : "+v"(qo), "+v"(vo), "+v"(to));
        auto read = [&](auto step) {
            constexpr int i = decltype(step)::value;
            if constexpr (i < N1) {
                ring[3 * (i % RB) + 0] = *(const u32x4*)(qs + (qo ^ (32 * i)));
                ring[3 * (i % RB) + 1] = *(const u32x4*)(os + (qo ^ (32 * i)));
                ring[3 * (i % RB) + 2] = *(const u32x4*)(vs + (vo ^ (32 * i)));
            } else {
                constexpr int k = i - N1, c2 = k / DT, dt = k % DT;
                ring[3 * (i % RB) + 0] = read_tr<ROWB>(os, 16 * c2, to, dt);
                ring[3 * (i % RB) + 1] = read_tr<ROWB>(qs, 16 * c2, to, dt);
            }
        };
        auto mma = [&](auto step) {
            constexpr int i = decltype(step)::value;
            if constexpr (i < N1) {
                s = M::run(ring[3 * (i % RB) + 0], kf[i], i == 0 ? f32x16(0.f) : s);
                dp = M::run(ring[3 * (i % RB) + 1], ring[3 * (i % RB) + 2], i == 0 ? f32x16(0.f) : dp);
            } else {
                constexpr int k = i - N1, c2 = k / DT, dt = k % DT;
                dva[dt] = M::run(ring[3 * (i % RB) + 0], bp[c2], dva[dt]);
                dka[dt] = M::run(ring[3 * (i % RB) + 1], bs[c2], dka[dt]);
            }
        };
        __builtin_amdgcn_s_setprio(1);
        static_for<0, (RB < NS ? RB : NS)>([&](auto i) { read(i); });
        static_for<0, NS>([&](auto step) {
            constexpr int i = decltype(step)::value;
            __builtin_amdgcn_sched_barrier(0);
            mma(step);
            if constexpr (i + RB < NS) read(Int<i + RB>{});
        });
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Vector phase: P = exp2(S c - LSE log2 e), dS = P (dP - D), packed as the
    // next MFMA phase's B operands.  Register r holds query row 8 (r / 4) +
    // 4 half + r % 4; rows past the end get P = dS = 0 (set, not multiplied:
    // their LSE and D slots need not be finite), in a branch taken by a
    // ragged last query tile only.
    auto vphase = [&](int st, int i0) {
        const float* lb = ls + st * 2 * BQ;
        float p[16], ds[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 l4 = *(const float4*)(lb + 8 * q4 + 4 * half);
            const float4 d4 = *(const float4*)(lb + BQ + 8 * q4 + 4 * half);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * q4 + e;
                const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lv[e]));
                p[r] = pr;
                ds[r] = pr * (dp[r] - dv[e]);
            }
        }
        if (i0 + BQ > n) {
            asm volatile("");
            // only rows [lo, hi) of a ragged query tile hold its queries
            const int qb = qtile_base(i0);
            const int lo = i0 - qb - 4 * half, hi = n - qb - 4 * half;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r >> 2) + (r & 3);
                if (row < lo || row >= hi) {
                    p[r] = 0.f;
                    ds[r] = 0.f;
                }
            }
        }
        bp[0] = M::pack(&p[0]);
        bp[1] = M::pack(&p[8]);
        bs[0] = M::pack(&ds[0]);
        bs[1] = M::pack(&ds[8]);
        // keep the vector work inside its phase
        asm volatile("" : "+v"(bp[0]), "+v"(bp[1]), "+v"(bs[0]), "+v"(bs[1]));
    };

    auto phase_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // Stream (query head, query tile) pairs: heads g grp .. g grp + grp - 1,
    // each over its query tiles; cursors advance one tile per step.
    const int steps = grp * ((n + BQ - 1) / BQ);
    auto advance = [&](int& h, int& r) {
        r += BQ;
        if (r >= n) { r = 0; ++h; }
    };
    int hn = g * grp, rn = 0;                // next tile to load (group 1)
    float lv_next = 0.f;                     // its LSE / D (wave 4)
    if (group == 1) {
        issue_tile(hn, rn, 0, load_lv(hn, rn));
        advance(hn, rn);
        if (steps > 1) {
            issue_tile(hn, rn, 1, load_lv(hn, rn));
            advance(hn, rn);
        }
        if (steps > 2) lv_next = load_lv(hn, rn);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): K, V, tiles 0 and 1 landed
    phase_barrier();
    if (group == 1) phase_barrier();     // group 1 runs one phase behind

    int rv = 0;                              // first row of the vector phase's tile
    // Vector phase j: group 1 first issues the loads of tile j + 2 (into
    // stage st2) and of the LSE / D of tile j + 3, then both groups take P
    // and dS; each wave waits for all its loads before the phase-ending
    // barrier, so no load is in flight during the next MFMA phase.
    auto vtail = [&](int j, int stc, int st2, auto has_sdp) {
        if (group == 1 && j + 2 < steps) {
            issue_tile(hn, rn, st2, lv_next);
            advance(hn, rn);
            if (j + 3 < steps) lv_next = load_lv(hn, rn);
        }
        if constexpr (decltype(has_sdp)::value) {
            vphase(stc, rv);
            rv = rv + BQ >= n ? 0 : rv + BQ;
        }
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
        phase_barrier();
    };

    using F = Int<0>;
    using Tr = Int<1>;
    // tile j lives in stage j mod 3; tile j + 2 goes into the stage of j - 1
    mphase(0, 0, Tr{}, F{});
    phase_barrier();
    vtail(0, 0, 2, Tr{});
    int stc = 1, stp = 0;
    for (int j = 1; j < steps; ++j) {
        mphase(stc, stp, Tr{}, Tr{});
        phase_barrier();
        vtail(j, stc, stp, Tr{});
        stp = stc;
        stc = stc == 2 ? 0 : stc + 1;
    }
    mphase(0, stp, F{}, Tr{});
    phase_barrier();
    vtail(steps, 0, 0, F{});
    if (group == 0) phase_barrier();

    // Lane (col, half) holds elements 8 gq + 4 half + 0..3 of each 32-wide
    // chunk dt of its key's row.  A swap between lanes col and col + 32 gives
    // half 0 all 8 elements of gq = 2 m and half 1 those of gq = 2 m + 1, so
    // each lane stores 16 contiguous bytes and each instruction fills whole
    // 32-byte segments of the rows.
    // The row address comes from an opaque copy of the lane index, so that
    // nothing of it is kept in registers across the tile loop.
    int ln;
    asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
    const int skey = kt0 + wave * 32 + (ln & 31);
    const int64_t srow = kvbase + (int64_t)min(skey, n - 1) * D + 8 * (ln >> 5);
    auto store_row = [&](T* row, const f32x16* acc, float f) __attribute__((always_inline)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                float lo[4], hi[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo[e] = acc[dt][8 * m + e] * f;
                    hi[e] = acc[dt][8 * m + 4 + e] * f;
                }
                const u32x2 a = M::pack4(lo), bb = M::pack4(hi);
                const auto s0 = __builtin_amdgcn_permlane32_swap(a.x, bb.x, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(a.y, bb.y, false, false);
                u32x4 out;
                out.x = s0[0];
                out.y = s1[0];
                out.z = s0[1];
                out.w = s1[1];
                if (skey < n) *(u32x4*)(row + 32 * dt + 16 * m) = out;
            }
    };
    store_row(dK + srow, dka, scale);
    store_row(dV + srow, dva, 1.f);
}

template <typename T, int D>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
    const int n = (int)a.n;
    const int nh = (int)a.h, grp = (int)(a.h / a.hkv);
    // scale log2(e), signed (no masking through -inf here); the caller has
    // checked that it is a finite float
    float c = FLT_MIN;
    exp2_factor(a.scale, &c);
    if (a.scale < 0.f) c = -c;
    const float scale = a.scale;
    const T* q = (const T*)a.q;
    const T* k = (const T*)a.k;
    const T* v = (const T*)a.v;
    const T* o = (const T*)a.o;
    const T* dout = (const T*)a.dout;
    const float* lse = a.lse;
    float* dr = a.dws;
    T* dq = (T*)a.dq;
    T* dk = (T*)a.dk;
    T* dv = (T*)a.dv;

    // 1. D = rowsum(dO * O)
    {
        const int64_t rows = a.bh * a.n;
        const int64_t need = (rows + 256 / (D / 8) - 1) / (256 / (D / 8));
        const int blocks = (int)(need < 8192 ? need : 8192);
        hipLaunchKernelGGL((flash_bwd_dot<T, D>), dim3(blocks), dim3(256), 0, stream, o, dout, dr, rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // 2. dQ
    {
        constexpr int nwq = D == 128 ? 8 : 4;   // waves (32 query rows each) per workgroup
        const int qtiles = (int)((a.n + 32 * nwq - 1) / (32 * nwq));
        const int total = (int)(a.bh * qtiles);
        void* args[] = {&q, &k, &v, &dout, &lse, &dr, &dq, (void*)&n, (void*)&qtiles, (void*)&total,
                        (void*)&c, (void*)&scale, (void*)&nh, (void*)&grp};
        hipError_t e = hipLaunchKernel((const void*)&flash_bwd_dq<T, D>, dim3(total), dim3(64 * nwq), args, 0,
                                       stream);
        if (e != hipSuccess) return e;
    }
    // 3. dK, dV: at d = 128 the two-group kernel (256 keys per workgroup),
    // at d = 64 the four-wave one (128 keys per workgroup)
    {
        const int bk = D == 128 ? 256 : 128;
        const int ktiles = (int)((a.n + bk - 1) / bk);
        const int total = (int)((a.bh / grp) * ktiles);
        void* args[] = {&q, &k, &v, &dout, &lse, &dr, &dk, &dv, (void*)&n, (void*)&ktiles, (void*)&total,
                        (void*)&c, (void*)&scale, (void*)&nh, (void*)&grp};
        if constexpr (D == 128)
            return hipLaunchKernel((const void*)&flash_bwd_dkdv_pp<T, D>, dim3(total), dim3(512), args, 0, stream);
        else
            return hipLaunchKernel((const void*)&flash_bwd_dkdv<T, D>, dim3(total), dim3(256), args, 0, stream);
    }
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
    switch (a.dtype) {
        case FA_DTYPE_BF16:
            return a.d == 128 ? launch_bwd_t<__bf16, 128>(a, stream) : launch_bwd_t<__bf16, 64>(a, stream);
        case FA_DTYPE_FP16:
            return a.d == 128 ? launch_bwd_t<_Float16, 128>(a, stream) : launch_bwd_t<_Float16, 64>(a, stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace fa
