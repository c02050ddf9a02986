// flash_fwd.hip — attention forward kernels for gfx950 (CDNA4).
//
// Method: the unite.ai page "Atención Flash: Revolucionando la Eficiencia de
// los Modelos de Transformador" (section "La Matemática detrás de la Atención
// Flash", formulas 1-2: safe softmax and the merge of partial softmaxes;
// section "Detalles de Implementación": query blocks outside, key/value blocks
// inside, running max M and sum L) and the nisoo.com page "Un'immersione
// approfondita nell'algoritmo FlashAttention – parte 3" (sections "Concetto di
// Divisione in Blocchi", "Softmax Sicura", "SafeSoftmax con Calcolo
// Normalizzatore Online").
//
// Every kernel: a workgroup owns a tile of query rows of one (b, h) head; each
// wave owns 32 rows (one query per lane pair) for the whole sweep over the
// keys, so the running state (max, sum, output) never leaves registers.  Per
// key/value tile:
//   1. K and V tiles are DMA'd from global memory straight into LDS (16 bytes
//      per lane, XOR-swizzled so the operand reads below are conflict free).
//   2. S^T = K Q^T on MFMA (32x32 outputs, fp32 accumulation).  Computing the
//      transpose puts one query per lane, so the row max and row sum are
//      in-lane reductions plus one cross-half swap.
//   3. Keys >= N in a ragged last tile are masked.
//   4. p = exp2(s * c - m) with c = scale * log2(e): one FMA and one v_exp_f32
//      per score, against the running reference max m.
//   5. m is raised to the tile's row max (the accumulators rescaled by
//      exp2(m_old - m_new), the weights taken again) only when it has to be:
//      fp16/bf16 kernels, when a lane's sum of the tile's weights exceeds
//      2^12 (and on the first tile); fp32 kernel, when the tile max exceeds
//      m by more than 2^8 in weight.  So the rescale, and in the 16-bit
//      kernels the tile max itself, are rare after the first tiles.
//   6. O^T += V^T P^T on MFMA; P goes straight from the accumulator registers
//      into the B operand (rounded to the input type for fp16/bf16), V^T is
//      read with the LDS transpose read ds_read_b64_tr_b16.
// Epilogue: O = O~ / l, LSE = (m + log2 l) ln 2.
//
// Kernels:
//   flash_fwd_pp  fp16/bf16, d = 128: 8 waves in two groups that alternate
//                 between the MFMA work and the softmax work of a tile, one
//                 group per phase, so each SIMD overlaps the two (below).
//   flash_fwd_16  fp16/bf16, d = 64: 4 waves, two workgroups per CU that the
//                 hardware interleaves.
//   flash_fwd_32  fp32 inputs on v_mfma_f32_32x32x2_f32.
//
// MFMA register layouts used (v_mfma_f32_32x32x16_{bf16,f16}, 32x32x2_f32):
//   A (32 x K): lane l supplies row l%32; B (K x 32): lane l supplies column
//   l%32; the K positions a lane supplies depend on l/32 identically for A and
//   B, so any pairing of the two is consistent.  D (32 x 32): lane l holds
//   column l%32, register r holds row 8*(r/4) + 4*(l/32) + r%4.
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"
#include "../../include/fa.h"

#include "fa_device.h"

namespace fa {
namespace {

// KS = 2 (few workgroups): 2 NW waves; waves w and w + NW hold the same
// query rows, group g = w / NW takes the key tiles g, g + 2, g + 4, ... into
// LDS stages of its own, and at the end group 1 hands its running state
// (m, l, O~) to group 0 through LDS, which merges the two by the merge of two
// partial softmaxes (R1) and writes the rows.  Twice the waves per SIMD, each
// with half the key sweep.
template <typename T, int D, int BC, int NW, int KS, bool PART>
__global__ void __launch_bounds__(NW * KS * 64) __attribute__((amdgpu_waves_per_eu(2)))
flash_fwd_16(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
             void* __restrict__ Out, float* __restrict__ LSE,
             int n, int qtiles, int total, float c, int negate, int nh, int grp, int splits, int kchunk)
{
    using M = Mfma<T>;
    constexpr int BR = 32 * NW;
    constexpr int ROWB = D * 2;              // bytes per K/V row
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int RPU = 64 / CPR;            // rows per 1 KB DMA unit
    constexpr int TILEB = BC * ROWB;         // bytes of one K (or V) tile
    constexpr int UNITS = TILEB / 1024;      // DMA units per tile
    constexpr int UPW = UNITS / NW;          // DMA units per wave
    constexpr int KT = BC / 32;              // 32-key sub-tiles
    constexpr int DT = D / 32;               // 32-wide output column blocks
    constexpr int KC = D / 16;               // contraction chunks of Q.K^T
    static_assert(UNITS % NW == 0 && BC % 32 == 0, "tile shape");

    static_assert(KS == 1 || KS == 2, "key groups");
    constexpr int TILEB3 = KS > 1 ? TILEB : 16;

    // Separate objects per stage, operand and key group, so the compiler can
    // see that the DMA into one stage never aliases the reads of another.
    __shared__ __attribute__((aligned(1024))) char ks0[TILEB];
    __shared__ __attribute__((aligned(1024))) char vs0[TILEB];
    __shared__ __attribute__((aligned(1024))) char ks1[TILEB];
    __shared__ __attribute__((aligned(1024))) char vs1[TILEB];
    __shared__ __attribute__((aligned(1024))) char ks2[TILEB];
    __shared__ __attribute__((aligned(1024))) char vs2[TILEB];
    __shared__ __attribute__((aligned(1024))) char ks3[TILEB3];
    __shared__ __attribute__((aligned(1024))) char vs3[TILEB3];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) % NW);   // row block
    const int kgrp = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) / NW);   // key group
    const int col = lane & 31;
    const int half = lane >> 5;

    const int tile = xcd_tile(blockIdx.x, total);
    const int hs = tile / qtiles;            // (b H + h) splits + key range
    const int qt = tile - hs * qtiles;
    const int bh = hs / splits;
    const int kbeg = (hs - bh * splits) * kchunk;
    const int nk = min(n - kbeg, kchunk);    // keys of this range (>= 1)
    const int64_t base = (int64_t)bh * n * D;
    // K/V head of this query head: query heads h of a batch share K/V head
    // h / grp (grp = 1: one K/V head per query head); the range starts at
    // key kbeg.
    const int64_t kvbase = (int64_t)((bh / nh) * (nh / grp) + (bh % nh) / grp) * n * D + (int64_t)kbeg * D;
    const int qrow = qt * BR + wave * 32 + col;

    // Q^T as the B operand: lane (col, half) holds Q[qrow][16*kc + 8*half + 0..7]
    // (rows past the end are clamped: computed, never stored).  A negative
    // scale flips the sign bits of Q, after the first K/V tile's DMA has been
    // issued (done here, the flip would make that DMA wait for Q to arrive).
    u32x4 qf[KC];
    {
        const T* qp = Q + base + (int64_t)min(qrow, n - 1) * D + 8 * half;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) qf[kc] = *(const u32x4*)(qp + 16 * kc);
    }
    auto negate_q = [&]() {
        if (negate) {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) qf[kc] ^= u32x4(0x80008000u);
        }
    };

    // Per-head buffer resources: any offset past the head reads zero instead
    // of faulting (the tail below also clamps, so this is a safety net).
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(K + kvbase), (short)0, nk * ROWB, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(V + kvbase), (short)0, nk * ROWB, 0x00020000);

    // DMA source offsets of this lane for the wave's units (within a tile).
    const int lrow = lane / CPR;             // row inside a unit
    const int lch = lane % CPR;              // LDS chunk position inside the row
    int kvo[UPW], vvo[UPW];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
        const int r = (wave * UPW + i) * RPU + lrow;
        kvo[i] = r * ROWB + 16 * (lch ^ swz_k<D>(r));
        vvo[i] = r * ROWB + 16 * (lch ^ swz_v<D>(r));
    }

    // LDS stages of key group G (compile time): KS = 1, stages 0 / 1 / 2 in
    // ks0..2 (vs0..2); KS = 2, group 0 in ks0 / ks1 and group 1 in ks2 / ks3.
    auto kst = [&](auto G, auto stage) -> char* {
        constexpr int g = decltype(G)::value, st = decltype(stage)::value;
        return g ? (st ? ks3 : ks2) : (st == 0 ? ks0 : st == 1 ? ks1 : ks2);
    };
    auto vst = [&](auto G, auto stage) -> char* {
        constexpr int g = decltype(G)::value, st = decltype(stage)::value;
        return g ? (st ? vs3 : vs2) : (st == 0 ? vs0 : st == 1 ? vs1 : vs2);
    };
    // First key held by the LDS tile of the tile at key j0: j0 itself for a
    // full tile; for the ragged last tile (j0 > 0) the window is moved back
    // to end at the last key, nk - BC, and its rows below j0 are masked (they
    // belong to the previous tile); a range shorter than one tile starts at
    // 0 and its rows past the end read zeros (the per-lane offset is bounds
    // checked).  Tiles past the end load the last window again (never read).
    // So every DMA has one form: per-lane offsets fixed for the kernel plus a
    // wave-uniform tile offset, with nothing to branch on.
    auto tile_base = [&](int j0) { return min(j0, max(nk - BC, 0)); };
    auto issue_loads = [&](int j0, auto G, auto stage) {
        char* kdst = kst(G, stage) + wave * UPW * 1024;
        char* vdst = vst(G, stage) + wave * UPW * 1024;
        const int so = tile_base(j0) * ROWB;
#pragma unroll
        for (int i = 0; i < UPW; ++i) {
            dma16(krs, kdst + i * 1024, kvo[i], so);
            dma16(vrs, vdst + i * 1024, vvo[i], so);
        }
    };

    // LDS read offsets of this lane (within a stage).
    // K, A operand of S^T: row col (+32 kt), logical chunk 2 kc + half.
    const int kx = half ^ swz_k<D>(col);
    // V, transpose read: lane 4t+s of each 16-lane group addresses row t
    // (+4 half) and the 4-element segment s of the group's 16 dims.
    const int trt = (lane & 15) >> 2, trs = lane & 3, trg = (lane >> 4) & 1;
    int voff[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const int r = 4 * half + trt;
        const int ch = 4 * dt + 2 * trg + (trs >> 1);
        voff[dt] = r * ROWB + 16 * (ch ^ swz_v<D>(r)) + 8 * (trs & 1);
    }

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16(0.f);
    float mref = -INFINITY;   // reference max (log2 units of scaled scores)
    float lsum = 0.f;         // this lane's part of the row sum

    // One tile as a fixed program (sched_barrier between steps): the S^T
    // steps (kt, kc), one K read each, then the softmax, then the P.V steps
    // (kt, c2, dt), two V transpose reads each.  LDS operands run R16 steps
    // ahead through `ring`; the first P.V operands are read before the
    // softmax so that they arrive while it runs.
    constexpr int R16 = 4;
    u32x4 ring[R16];
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4* lds_s16x4;
    auto compute = [&](auto G, auto stage, int j0, bool first) {
        const char* kb = kst(G, stage);
        const char* vb = vst(G, stage);
        constexpr int N1 = KT * KC;
        constexpr int N2 = KT * 2 * DT;
        auto read1 = [&](auto step) {
            constexpr int i = decltype(step)::value;
            constexpr int kt = i / KC, kc = i % KC;
            ring[i % R16] = *(const u32x4*)(kb + (32 * kt + col) * ROWB + 16 * ((2 * kc) ^ kx));
        };
        auto read2 = [&](auto step) {
            constexpr int i = decltype(step)::value;
            constexpr int kt = i / (2 * DT), c2 = (i / DT) % 2, dt = i % DT;
            const char* vrow = vb + (32 * kt + 16 * c2) * ROWB;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(vrow + voff[dt]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(vrow + 8 * ROWB + voff[dt]));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            ring[i % R16] = u32x4{l2.x, l2.y, h2.x, h2.y};
        };

        // S^T = K Q^T (raw scores, fp32).
        f32x16 s[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) s[kt] = f32x16(0.f);
        static_for<0, (R16 < N1 ? R16 : N1)>([&](auto i) { read1(i); });
        static_for<0, N1>([&](auto step) {
            constexpr int i = decltype(step)::value;
            constexpr int kt = i / KC, kc = i % KC;
            __builtin_amdgcn_sched_barrier(0);
            s[kt] = M::run(ring[i % R16], qf[kc], s[kt]);
            if constexpr (i + R16 < N1) read1(Int<i + R16>{});
        });
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, (R16 < N2 ? R16 : N2)>([&](auto i) { read2(i); });

        // ragged last tile: only LDS rows [lo, hi) hold keys of this tile
        // (register r of lane half h holds row 32 kt + 8 (r >> 2) + (r & 3) + 4 h)
        if (j0 + BC > nk) {
            const int kb = tile_base(j0);
            const int lo = j0 - kb - 4 * half, hi = nk - kb - 4 * half;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * kt + 8 * (r >> 2) + (r & 3);
                    if (row < lo || row >= hi) s[kt][r] = -INFINITY;
                }
        }

        // Weights against the current reference max first; the tile max, the
        // rescale of the output and sum by exp2(m_old - m_new) and a second
        // pass only when a lane's sum of them exceeds kTileSumLimit (and on
        // the first tile, where the reference is still -inf).
        auto raise = [&](bool first) {
            float mt = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kt][r]);
            const float mnew = fmaxf(mref, pair_max(mt) * c);
            if (!first) {
                const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
                lsum *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
            }
            mref = mnew;
        };
        // O^T += V^T P^T.  B operand: the lane's 8 weights of registers
        // 8*c2 .. 8*c2+7 (keys 16*c2 + {0..3, 8..11} + 4*half of the sub-tile).
        // Returns the lane's sum of the unrounded weights (four chains).
        u32x4 pb[KT * 2];
        auto weights = [&]() {
            float part[4];
#pragma unroll
            for (int j = 0; j < KT * 2; ++j) {
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pv[e] = __builtin_amdgcn_exp2f(fmaf(s[j >> 1][8 * (j & 1) + e], c, -mref));
                    part[e & 3] = (j == 0 && e < 4) ? pv[e] : part[e & 3] + pv[e];
                }
                pb[j] = M::pack(pv);
            }
            return (part[0] + part[1]) + (part[2] + part[3]);
        };
        if (first) raise(true);
        float t = weights();
        if (__ballot(t > kTileSumLimit)) {
            raise(false);
            t = weights();
        }
        lsum += t;
        static_for<0, N2>([&](auto step) {
            constexpr int i = decltype(step)::value;
            constexpr int j = i / DT, dt = i % DT;
            __builtin_amdgcn_sched_barrier(0);
            acc[dt] = M::run(ring[i % R16], pb[j], acc[dt]);
            if constexpr (i + R16 < N2) read2(Int<i + R16>{});
        });
        __builtin_amdgcn_sched_barrier(0);
    };

    // Two LDS stages per key group: while one is computed on, the DMA fills
    // the other.  Key group g visits tiles g, g + KS, ...; both groups run the
    // same number of steps (one barrier each), group 1 idling in the last
    // step when the tile count is odd.
    const int ntiles = (nk + BC - 1) / BC;
    const int nsteps = (ntiles + KS - 1) / KS;
    auto sweep = [&](auto G) {
        constexpr int g = decltype(G)::value;
        auto has = [&](int i) { return KS * i + g < ntiles; };
        if (has(0)) issue_loads(g * BC, G, Int<0>{});
        negate_q();
        for (int i = 0;;) {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA landed
            __syncthreads();                      // ... every wave's; stage 1 is free
            if (has(i + 1)) issue_loads((KS * (i + 1) + g) * BC, G, Int<1>{});
            if (has(i)) compute(G, Int<0>{}, (KS * i + g) * BC, i == 0);
            if (++i == nsteps) break;
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            if (has(i + 1)) issue_loads((KS * (i + 1) + g) * BC, G, Int<0>{});
            if (has(i)) compute(G, Int<1>{}, (KS * i + g) * BC, false);
            if (++i == nsteps) break;
        }
    };
    // KS = 1 (several workgroups per CU): three stages, the DMA of tile t + 2
    // issued at the top of step t into the stage of tile t - 1, which every
    // wave finished reading in step t - 1; each wave waits only for tile t's
    // DMA (tile t + 1's may still be in flight) before the barrier, which
    // carries no fence (a fence would wait for every load).  Tiles past the
    // end are loaded too (never read), so every step has the same loads in
    // flight; with one DMA form and one loop exit the compiler's tracking of
    // them stays exact and adds no waits of its own.
    auto sweep3 = [&]() {
        issue_loads(0, Int<0>{}, Int<0>{});
        issue_loads(BC, Int<0>{}, Int<1>{});
        negate_q();
        static_assert(2 * UPW == 4, "wait count below");
        auto stepk = [&](int t, auto stage) __attribute__((always_inline)) {
            constexpr int S = decltype(stage)::value;
            __builtin_amdgcn_s_waitcnt(0x0074);   // vmcnt(4) lgkmcnt(0): tile t landed
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            issue_loads((t + 2) * BC, Int<0>{}, Int<(S + 2) % 3>{});
            compute(Int<0>{}, Int<S>{}, t * BC, t == 0);
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
    };
    if constexpr (KS == 1) {
        sweep3();
    } else {
        // Group 1's waves run at raised issue priority: with equal priority
        // the older waves of group 0 go first on every SIMD, group 1 falls
        // behind within each step and group 0 waits for it at the barrier.
        if (kgrp == 0) {
            sweep(Int<0>{});
        } else {
            __builtin_amdgcn_s_setprio(1);
            sweep(Int<1>{});
            __builtin_amdgcn_s_setprio(0);
        }
    }

    if constexpr (KS > 1) {
        // Group 1 leaves (m, l, O~) in LDS (lane-major, conflict free); group 0
        // merges: m = max(m0, m1), l = a0 l0 + a1 l1, O~ = a0 O~0 + a1 O~1 with
        // a_g = exp2(m_g - m) (a group without keys has m = -inf, a = 0).
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();                          // every wave is done with the tiles
        char* accb = wave == 0 ? ks0 : wave == 1 ? vs0 : wave == 2 ? ks1 : vs1;
        float* ml = (float*)(ks2 + wave * 512);
        if (kgrp == 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *(float4*)(accb + ((dt * 4 + q) * 64 + lane) * 16) =
                        make_float4(acc[dt][4 * q], acc[dt][4 * q + 1], acc[dt][4 * q + 2], acc[dt][4 * q + 3]);
            ml[lane] = mref;
            ml[64 + lane] = lsum;
        }
        __syncthreads();
        if (kgrp == 1) return;
        const float m1 = ml[lane], l1 = ml[64 + lane];
        const float mm = fmaxf(mref, m1);
        const float a0 = __builtin_amdgcn_exp2f(mref - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
        lsum = a0 * lsum + a1 * l1;
        mref = mm;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 o1 = *(const float4*)(accb + ((dt * 4 + q) * 64 + lane) * 16);
                acc[dt][4 * q + 0] = a0 * acc[dt][4 * q + 0] + a1 * o1.x;
                acc[dt][4 * q + 1] = a0 * acc[dt][4 * q + 1] + a1 * o1.y;
                acc[dt][4 * q + 2] = a0 * acc[dt][4 * q + 2] + a1 * o1.z;
                acc[dt][4 * q + 3] = a0 * acc[dt][4 * q + 3] + a1 * o1.w;
            }
    }

    const float ltot = pair_sum(lsum);
    if (qrow < n) {
        const float inv = 1.0f / ltot;
        // Row hs n + qrow: the output row (one range: hs = bh), or the fp32
        // partial row of key range hs % splits.
        const int64_t orow0 = ((int64_t)hs * n + qrow) * D;
        if constexpr (PART) {
            float* orow = (float*)Out + orow0;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float4 ov;
                    ov.x = acc[dt][4 * g + 0] * inv;
                    ov.y = acc[dt][4 * g + 1] * inv;
                    ov.z = acc[dt][4 * g + 2] * inv;
                    ov.w = acc[dt][4 * g + 3] * inv;
                    *(float4*)(orow + 32 * dt + 8 * g + 4 * half) = ov;
                }
        } else {
            T* orow = (T*)Out + orow0;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float ov[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[e] = acc[dt][4 * g + e] * inv;
                    *(u32x2*)(orow + 32 * dt + 8 * g + 4 * half) = M::pack4(ov);
                }
        }
        if (half == 0) LSE[(int64_t)hs * n + qrow] = (mref + log2f(ltot)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Ping-pong kernel (fp16 / bf16): 8 waves = two groups of 4; waves w and w+4
// share a SIMD.  Each wave owns 32 query rows; key/value tiles of 64 keys.
// Every wave runs MFMA phase j (S_j = Q K_j^T, then O += P_{j-1} V_{j-1}),
// a workgroup barrier, softmax phase j (tile j's scores into weights), a
// barrier; group B runs one phase behind group A, so on every SIMD one wave
// feeds the matrix core while the other computes exponentials.
//
// LDS holds two stages of K and of V (64 KiB at d = 128, all under the
// 64 KiB immediate-offset range).  Group A loads V_j during its softmax phase
// j (phase 2j+1; the stage held V_{j-2}, last read in phase 2j-1); group B
// loads K_{j+2} during its softmax phase j (phase 2j+2; the stage held K_j,
// last read in phase 2j+1).  Each wave waits for its own loads before the
// barrier that ends the phase, so every tile is complete one phase before its
// first reader.  The first K operands of the next MFMA phase are read into
// registers at the end of each softmax phase.
// ---------------------------------------------------------------------------
template <typename T, int D, bool PART>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
flash_fwd_pp(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
             void* __restrict__ Out, float* __restrict__ LSE,
             int n, int qtiles, int total, float c, int negate, int nh, int grp, int splits, int kchunk)
{
    using M = Mfma<T>;
    constexpr int NW = 8;
    constexpr int BC = 64;                   // keys per tile
    constexpr int BR = 32 * NW;              // query rows per workgroup
    constexpr int ROWB = D * 2;              // bytes per K/V row
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int RPU = 64 / CPR;            // rows per 1 KB DMA unit
    constexpr int TILEB = BC * ROWB;         // bytes of one K (or V) tile
    constexpr int UNITS = TILEB / 1024;      // DMA units per tile
    constexpr int UPW = UNITS / 4;           // units per wave of the loading group
    constexpr int KT = BC / 32;              // 32-key sub-tiles
    constexpr int DT = D / 32;               // 32-wide output column blocks
    constexpr int KC = D / 16;               // contraction chunks of Q.K^T
    constexpr int PC = BC / 16;              // 16-key contraction chunks of P.V
    constexpr int R = 4;                     // LDS operand reads in flight
    static_assert(UNITS % 4 == 0 && 4 * TILEB <= 65536, "tile shape");

    __shared__ __attribute__((aligned(1024))) char ks0[TILEB];
    __shared__ __attribute__((aligned(1024))) char ks1[TILEB];
    __shared__ __attribute__((aligned(1024))) char vs0[TILEB];
    __shared__ __attribute__((aligned(1024))) char vs1[TILEB];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int group = wave >> 2;
    const int gw = wave & 3;                 // wave index inside its group
    const int col = lane & 31;
    const int half = lane >> 5;

    const int tile = xcd_tile(blockIdx.x, total);
    const int hs = tile / qtiles;            // (b H + h) splits + key range
    const int qt = tile - hs * qtiles;
    const int bh = hs / splits;
    const int kbeg = (hs - bh * splits) * kchunk;
    const int nk = min(n - kbeg, kchunk);    // keys of this range (>= 1)
    const int64_t base = (int64_t)bh * n * D;
    // K/V head of this query head: query heads h of a batch share K/V head
    // h / grp (grp = 1: one K/V head per query head); the range starts at
    // key kbeg.
    const int64_t kvbase = (int64_t)((bh / nh) * (nh / grp) + (bh % nh) / grp) * n * D + (int64_t)kbeg * D;
    const int qrow = qt * BR + wave * 32 + col;

    // Q^T as the B operand: lane (col, half) holds Q[qrow][16 kc + 8 half + 0..7];
    // rows past the end are clamped (computed, never stored).
    u32x4 qf[KC];
    {
        const T* qp = Q + base + (int64_t)min(qrow, n - 1) * D + 8 * half;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            qf[kc] = *(const u32x4*)(qp + 16 * kc);
            if (negate) qf[kc] ^= u32x4(0x80008000u);
        }
    }

    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(K + kvbase), (short)0, nk * ROWB, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(V + kvbase), (short)0, nk * ROWB, 0x00020000);

    // DMA: this wave moves units gw*UPW .. of a tile; K and V use their own
    // swizzles (chosen by the global chunk each lane fetches).
    const int lrow = lane / CPR;
    const int lch = lane % CPR;
    // One DMA form for every tile: fixed per-lane offsets plus a wave-uniform
    // tile offset.  The ragged last tile's LDS window ends at the last key
    // (its rows below the tile's first key are masked in the softmax); a
    // range shorter than one tile reads zeros past its end (the per-lane
    // offset is bounds checked).
    auto tile_base = [&](int j0) { return min(j0, max(nk - BC, 0)); };
    auto issue = [&](__amdgpu_buffer_rsrc_t rs, char* stage, int j0, auto isk) {
        constexpr bool IK = decltype(isk)::value;
        char* dst = stage + gw * UPW * 1024;
        const int so = tile_base(j0) * ROWB;
#pragma unroll
        for (int i = 0; i < UPW; ++i) {
            const int r = (gw * UPW + i) * RPU + lrow;
            const int sw = IK ? swz_k<D>(r) : swz_v<D>(r);
            dma16(rs, dst + i * 1024, r * ROWB + 16 * (lch ^ sw), so);
        }
    };

    // LDS read offsets.  K, A operand of S^T: row col (+32 kt), logical chunk
    // 2 kc + half.  V, transpose read: lane 4t+s of each 16-lane group
    // addresses row t (+4 half) and the 4-element segment s of the group's 16
    // dims.
    const int kx = half ^ swz_k<D>(col);
    const int trt = (lane & 15) >> 2, trs = lane & 3, trg = (lane >> 4) & 1;
    int voff[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const int r = 4 * half + trt;
        const int ch = 4 * dt + 2 * trg + (trs >> 1);
        voff[dt] = r * ROWB + 16 * (ch ^ swz_v<D>(r)) + 8 * (trs & 1);
    }

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16(0.f);
    float mref = -INFINITY;   // reference max (log2 units of scaled scores)
    float lsum = 0.f;         // this lane's part of the row sum
    f32x16 s[KT];             // raw scores of the current tile
    u32x4 p[PC];              // its packed weights (B operands of P.V)
    u32x4 ring[R];            // A operands in flight

    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4* lds_s16x4;

    // The MFMA phase as a fixed program: QK steps (kc, kt) first, one K read
    // each; then PV steps (pc, dt), two V transpose reads each.  Reads run R
    // steps ahead through `ring`; sched_barrier pins the order.
    auto mphase = [&](const char* kb, const char* vb, auto has_qk, auto has_pv, auto filled) {
        constexpr int NQK = decltype(has_qk)::value ? KC * KT : 0;
        constexpr int NPV = decltype(has_pv)::value ? PC * DT : 0;
        constexpr int NS = NQK + NPV;
        auto read = [&](auto step) {
            constexpr int i = decltype(step)::value;
            if constexpr (i < NQK) {
                constexpr int kc = i / KT, kt = i % KT;
                ring[i % R] = *(const u32x4*)(kb + (32 * kt + col) * ROWB + 16 * ((2 * kc) ^ kx));
            } else {
                constexpr int pc = (i - NQK) / DT, dt = (i - NQK) % DT;
                const char* vrow = vb + 16 * pc * ROWB;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(vrow + voff[dt]));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(vrow + 8 * ROWB + voff[dt]));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                ring[i % R] = u32x4{l2.x, l2.y, h2.x, h2.y};
            }
        };
        auto mma = [&](auto step) {
            constexpr int i = decltype(step)::value;
            if constexpr (i < NQK) {
                constexpr int kc = i / KT, kt = i % KT;
                s[kt] = M::run(ring[i % R], qf[kc], kc == 0 ? f32x16(0.f) : s[kt]);
            } else {
                constexpr int pc = (i - NQK) / DT, dt = (i - NQK) % DT;
                acc[dt] = M::run(ring[i % R], p[pc], acc[dt]);
            }
        };
        // The wave in its MFMA phase takes issue priority over the softmax-phase
        // wave on the same SIMD, so a product whose operands are ready is not
        // held behind the other wave's vector instructions.
        __builtin_amdgcn_s_setprio(1);
        if constexpr (!decltype(filled)::value) static_for<0, (R < NS ? R : NS)>([&](auto i) { read(i); });
        static_for<0, NS>([&](auto i) {
            constexpr int k = decltype(i)::value;
            __builtin_amdgcn_sched_barrier(0);
            mma(i);
            if constexpr (k + R < NS) read(Int<k + R>{});
            // With both kinds of products in the phase, the tile's exponent
            // arguments x = s c - m (the same m as the coming softmax phase)
            // are formed here, two or three per P.V product from the third
            // on, by the MFMA-phase wave, whose vector issue is otherwise idle.
            if constexpr (NQK > 0 && NPV > 0 && k >= NQK + 2) {
                constexpr int kk = k - NQK - 2;
                constexpr int f0 = (KT * 16) * kk / (NPV - 2), f1 = (KT * 16) * (kk + 1) / (NPV - 2);
                static_for<f0, f1>([&](auto ff) {
                    constexpr int q = decltype(ff)::value;
                    s[q >> 4][q & 15] = fmaf(s[q >> 4][q & 15], c, -mref);
                });
            }
        });
        if constexpr (NQK > 0 && NPV > 0) {
            // keep the exponent arguments in this phase
            asm volatile("" : "+v"(s[0]), "+v"(s[1]));
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // First R K operands of an MFMA phase, read ahead at the end of the
    // preceding softmax phase.
    auto prefetch = [&](const char* kb) {
        static_for<0, R>([&](auto step) {
            constexpr int i = decltype(step)::value;
            constexpr int kc = i / KT, kt = i % KT;
            ring[i] = *(const u32x4*)(kb + (32 * kt + col) * ROWB + 16 * ((2 * kc) ^ kx));
        });
    };

    // Online softmax of one tile (scores in s, weights packed into p).  Keys
    // past the end of a ragged last tile get score -inf, hence weight 0 (the
    // host never passes c = 0, so -inf * c stays -inf).
    // The weights are first taken against the current reference max, without
    // this tile's max: only when some lane's sum of them exceeds
    // kTileSumLimit is the reference raised to the tile max (the output and
    // sum rescaled) and the weights taken again.  The first tile always
    // raises it.  So every weight stays <= kTileSumLimit, and the tile max
    // (about 20 vector instructions per tile) is computed only on the rare
    // tiles that need it.
    auto softmax = [&](int j0, auto first) {
        // ragged last tile: only LDS rows [lo, hi) hold keys of this tile
        if (j0 + BC > nk) {
            const int kb = tile_base(j0);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int lo = j0 - kb - 32 * kt - 4 * half, hi = nk - kb - 32 * kt - 4 * half;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 8 * (r >> 2) + (r & 3);
                    if (row < lo || row >= hi) s[kt][r] = -INFINITY;
                }
            }
        }
        // Raise the reference max to this tile's max (both lanes of a query
        // pair agree) and rescale the running sum and output by
        // exp2(m_old - m_new).
        // first: s holds raw scores; otherwise x = s c - m from the MFMA phase
        constexpr bool XF = !decltype(first)::value;
        auto raise = [&](auto first) {
            float mp[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) mp[q] = fmaxf(s[q >> 1][8 * (q & 1)], s[q >> 1][8 * (q & 1) + 1]);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 2; r < 16; ++r) {
                    const int q = 2 * kt + (r >> 3);
                    if ((r & 7) >= 2) mp[q] = fmaxf(mp[q], s[kt][r]);
                }
            const float mx = pair_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])));
            const float mt = XF ? mx + mref : mx * c;
            const float mnew = fmaxf(mref, mt);
            if constexpr (!decltype(first)::value) {
                const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
                lsum *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
            }
            if constexpr (XF) {
                const float dm = mref - mnew;
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kt][r] += dm;
            }
            mref = mnew;
        };
        // Weights exp2(s c - m) packed into p; returns this lane's sum of the
        // unrounded weights (four chains, each started by its first weight).
        auto weights = [&]() {
            float part[4];
#pragma unroll
            for (int pc = 0; pc < PC; ++pc) {
                float w[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    w[e] = XF ? __builtin_amdgcn_exp2f(s[pc >> 1][8 * (pc & 1) + e])
                              : __builtin_amdgcn_exp2f(fmaf(s[pc >> 1][8 * (pc & 1) + e], c, -mref));
                    part[e & 3] = (pc == 0 && e < 4) ? w[e] : part[e & 3] + w[e];
                }
                p[pc] = M::pack(w);
            }
            return (part[0] + part[1]) + (part[2] + part[3]);
        };
        if constexpr (decltype(first)::value) raise(Int<1>{});
        float t = weights();
        if (__ballot(t > kTileSumLimit)) {
            raise(Int<0>{});
            t = weights();
        }
        lsum += t;
        // keep the whole softmax inside its phase
#pragma unroll
        for (int pc = 0; pc < PC; ++pc) asm volatile("" : "+v"(p[pc]));
        asm volatile("" : "+v"(lsum), "+v"(mref));
    };

    auto phase_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    const int ntiles = (nk + BC - 1) / BC;
    // Phase pair j (P = j & 1 selects the LDS stages at compile time):
    // MFMA phase j reads K_j from ks[P] and V_{j-1} from vs[1-P].
    auto pair = [&](int j, auto par, auto has_qk, auto has_pv, auto pf) {
        constexpr int P = decltype(par)::value;
        char* kcur = P ? ks1 : ks0;
        char* knxt = P ? ks0 : ks1;
        char* vprv = P ? vs0 : vs1;
        char* vcur = P ? vs1 : vs0;
        mphase(kcur, vprv, has_qk, has_pv, has_qk);
        phase_barrier();
        if (group == 0) {
            if (j < ntiles) issue(vrs, vcur, j * BC, Int<0>{});
        } else {
            if (j + 2 < ntiles) issue(krs, kcur, (j + 2) * BC, Int<1>{});
        }
        // tile 0's phase pair is the only one with Q.K^T and no P.V products
        if constexpr (decltype(has_qk)::value) softmax(j * BC, Int<!decltype(has_pv)::value>{});
        if constexpr (decltype(pf)::value) prefetch(knxt);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads landed
        phase_barrier();
    };

    using F = Int<0>;
    using Tr = Int<1>;
    if (group == 1) {
        issue(krs, ks0, 0, Int<1>{});
        if (ntiles > 1) issue(krs, ks1, BC, Int<1>{});
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    phase_barrier();
    prefetch(ks0);
    if (group == 1) phase_barrier();     // group B runs one phase behind
    // The last full pair of the loop may prefetch K operands of a tile that
    // does not exist (stale LDS, never used: the phase after it has no Q.K^T
    // products); this keeps one tail per tile-count parity.
    pair(0, Int<0>{}, Tr{}, F{}, Tr{});
    int j = 1;
    for (; j + 1 < ntiles; j += 2) {
        pair(j, Int<1>{}, Tr{}, Tr{}, Tr{});
        pair(j + 1, Int<0>{}, Tr{}, Tr{}, Tr{});
    }
    if (j < ntiles) {
        pair(j, Int<1>{}, Tr{}, Tr{}, F{});
        pair(j + 1, Int<0>{}, F{}, Tr{}, F{});
    } else {
        pair(j, Int<1>{}, F{}, Tr{}, F{});
    }
    if (group == 0) phase_barrier();

    const float ltot = pair_sum(lsum);
    if (qrow < n) {
        const float inv = 1.0f / ltot;
        // Row hs n + qrow: the output row (one range: hs = bh), or the fp32
        // partial row of key range hs % splits.
        const int64_t orow0 = ((int64_t)hs * n + qrow) * D;
        if constexpr (PART) {
            float* orow = (float*)Out + orow0;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float4 ov;
                    ov.x = acc[dt][4 * g + 0] * inv;
                    ov.y = acc[dt][4 * g + 1] * inv;
                    ov.z = acc[dt][4 * g + 2] * inv;
                    ov.w = acc[dt][4 * g + 3] * inv;
                    *(float4*)(orow + 32 * dt + 8 * g + 4 * half) = ov;
                }
        } else {
            T* orow = (T*)Out + orow0;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float ov[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[e] = acc[dt][4 * g + e] * inv;
                    *(u32x2*)(orow + 32 * dt + 8 * g + 4 * half) = M::pack4(ov);
                }
        }
        if (half == 0) LSE[(int64_t)hs * n + qrow] = (mref + log2f(ltot)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel: same structure on v_mfma_f32_32x32x2_f32 (one contraction
// element per lane per instruction, so V needs no transpose in LDS).
// ---------------------------------------------------------------------------
template <int D, int BC, int NW, bool PART>
__global__ void __launch_bounds__(NW * 64)
flash_fwd_32(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
             void* __restrict__ Out, float* __restrict__ LSE,
             int n, int qtiles, int total, float c, int negate, int nh, int grp, int splits, int kchunk)
{
    constexpr int NT = NW * 64;
    constexpr int BR = 32 * NW;
    constexpr int STR = D + 4;       // row stride of K and V in LDS (floats)
    constexpr int KT = BC / 32;
    constexpr int DT = D / 32;
    constexpr int CHUNKS = BC * D / 4;           // 16-byte chunks of a K (or V) tile
    constexpr int PER = (CHUNKS + NT - 1) / NT;

    __shared__ __attribute__((aligned(16))) float ks[BC * STR];
    __shared__ __attribute__((aligned(16))) float vs[BC * STR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;

    const int tile = xcd_tile(blockIdx.x, total);
    const int hs = tile / qtiles;            // (b H + h) splits + key range
    const int qt = tile - hs * qtiles;
    const int bh = hs / splits;
    const int kbeg = (hs - bh * splits) * kchunk;
    const int nk = min(n - kbeg, kchunk);    // keys of this range (>= 1)
    const int64_t base = (int64_t)bh * n * D;
    // K/V head of this query head: query heads h of a batch share K/V head
    // h / grp (grp = 1: one K/V head per query head); the range starts at
    // key kbeg.
    const int64_t kvbase = (int64_t)((bh / nh) * (nh / grp) + (bh % nh) / grp) * n * D + (int64_t)kbeg * D;
    const float* __restrict__ Qh = Q + base;
    const float* __restrict__ Kh = K + kvbase;
    const float* __restrict__ Vh = V + kvbase;
    const int qrow = qt * BR + wave * 32 + col;

    // Q^T as the B operand: lane (col, half) holds Q[qrow][2*kc + half].
    float qf[D / 2];
#pragma unroll
    for (int kc = 0; kc < D / 2; ++kc) {
        const float x = qrow < n ? Qh[(int64_t)qrow * D + 2 * kc + half] : 0.f;
        qf[kc] = negate ? -x : x;
    }

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16(0.f);
    float mref = -INFINITY;
    float lsum = 0.f;

    u32x4 kreg[PER], vreg[PER];
    auto gload = [&](int j0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int ch = tid + i * NT;
            const int key = ch / (D / 4), part = ch % (D / 4);
            const bool ok = (CHUNKS % NT == 0 || ch < CHUNKS) && j0 + key < nk;
            kreg[i] = ok ? *(const u32x4*)(Kh + (int64_t)(j0 + key) * D + 4 * part) : u32x4(0u);
            vreg[i] = ok ? *(const u32x4*)(Vh + (int64_t)(j0 + key) * D + 4 * part) : u32x4(0u);
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int ch = tid + i * NT;
            if (CHUNKS % NT == 0 || ch < CHUNKS) {
                const int key = ch / (D / 4), part = ch % (D / 4);
                *(u32x4*)&ks[key * STR + 4 * part] = kreg[i];
                *(u32x4*)&vs[key * STR + 4 * part] = vreg[i];
            }
        }
    };

    const int ntiles = (nk + BC - 1) / BC;
    gload(0);
    for (int t = 0; t < ntiles; ++t) {
        const int j0 = t * BC;
        __syncthreads();
        lstore();
        __syncthreads();
        if (t + 1 < ntiles) gload(j0 + BC);

        f32x16 s[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            s[kt] = f32x16(0.f);
#pragma unroll
            for (int kc = 0; kc < D / 2; ++kc)
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[(32 * kt + col) * STR + 2 * kc + half],
                                                             qf[kc], s[kt], 0, 0, 0);
        }

        const bool tail = j0 + BC > nk;
        if (tail) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (j0 + 32 * kt + acc_row(r, half) >= nk) s[kt][r] = -INFINITY;
        }
        float mt = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kt][r]);
        mt = pair_max(mt) * c;
        if (__ballot(mt > mref + kRescaleSlack)) {
            const float mnew = fmaxf(mref, mt);
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
        if (tail) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (j0 + 32 * kt + acc_row(r, half) >= nk) s[kt][r] = 0.f;
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) lsum += s[kt][r];

        // O^T += V^T P^T, one key per lane half per instruction: register r
        // of this lane is key 32*kt + acc_row(r, half).
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float* vrow = &vs[(32 * kt + acc_row(r, half)) * STR + col];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * dt], s[kt][r], acc[dt], 0, 0, 0);
            }
    }

    const float ltot = pair_sum(lsum);
    if (qrow < n) {
        const float inv = 1.0f / ltot;
        // Row hs n + qrow: the output row (one range: hs = bh), or the
        // partial row of key range hs % splits (same type: fp32).
        float* orow = (float*)Out + ((int64_t)hs * n + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float4 ov;
                ov.x = acc[dt][4 * g + 0] * inv;
                ov.y = acc[dt][4 * g + 1] * inv;
                ov.z = acc[dt][4 * g + 2] * inv;
                ov.w = acc[dt][4 * g + 3] * inv;
                *(float4*)(orow + 32 * dt + 8 * g + 4 * half) = ov;
            }
        if (half == 0) LSE[(int64_t)hs * n + qrow] = (mref + log2f(ltot)) * kLn2;
    }
}

constexpr int64_t kComputeUnitsFwd = 256;   // MI355X

template <typename Kern, typename T>
hipError_t launch(Kern kern, int nw, int br, const FwdArgs& a, void* out, float* lse, int splits, int kchunk,
                  hipStream_t stream) {
    const int n = (int)a.n;
    const int qtiles = (int)((a.n + br - 1) / br);
    const int total = (int)(a.bh * splits * qtiles);
    // c = |scale| log2(e) (a negative scale negates Q instead); scale = 0 is
    // passed as the smallest normal float (exp2_factor).  The caller has
    // checked that c is finite.
    float c = FLT_MIN;
    exp2_factor(a.scale, &c);
    const int negate = a.scale < 0.f ? 1 : 0;
    const T* q = (const T*)a.q;
    const T* k = (const T*)a.k;
    const T* v = (const T*)a.v;
    const int nh = (int)a.h, grp = (int)(a.h / a.hkv);
    void* args[] = {&q, &k, &v, &out, &lse, (void*)&n, (void*)&qtiles, (void*)&total, (void*)&c, (void*)&negate,
                    (void*)&nh, (void*)&grp, (void*)&splits, (void*)&kchunk};
    return hipLaunchKernel((const void*)kern, dim3(total), dim3(nw * 64), args, 0, stream);
}

// d = 64, fp16/bf16: when the grid holds at most one workgroup per CU (the
// ragged workload: 256), the key-group variant doubles the waves per SIMD and
// halves each wave's key sweep.  With more (the GPT-2-shaped workload: 768)
// the plain kernel keeps three workgroups per CU, where the key-group one (8
// waves, one workgroup per CU) would need more rounds.
template <typename T, bool PART>
hipError_t launch_d64(const FwdArgs& a, void* out, float* lse, int splits, int kchunk, hipStream_t stream) {
    constexpr int NW = 4;
    constexpr int BR = 32 * NW;
    const int64_t wgs = a.bh * splits * ((a.n + BR - 1) / BR);
    const int64_t keys = splits > 1 ? kchunk : a.n;
    if (wgs <= kComputeUnitsFwd && keys > 64)
        return launch<decltype(&flash_fwd_16<T, 64, 64, NW, 2, PART>), T>(
            &flash_fwd_16<T, 64, 64, NW, 2, PART>, 2 * NW, BR, a, out, lse, splits, kchunk, stream);
    return launch<decltype(&flash_fwd_16<T, 64, 64, NW, 1, PART>), T>(
        &flash_fwd_16<T, 64, 64, NW, 1, PART>, NW, BR, a, out, lse, splits, kchunk, stream);
}

// One launch of the kernel for (dtype, d); PART: fp32 partial outputs.
template <bool PART>
hipError_t launch_kernel(const FwdArgs& a, void* out, float* lse, int splits, int kchunk, hipStream_t stream) {
    constexpr int NW = 4;
    constexpr int BR = 32 * NW;
    switch (a.dtype) {
        case FA_DTYPE_BF16:
            return a.d == 128 ? launch<decltype(&flash_fwd_pp<__bf16, 128, PART>), __bf16>(
                                    &flash_fwd_pp<__bf16, 128, PART>, 8, 256, a, out, lse, splits, kchunk, stream)
                              : launch_d64<__bf16, PART>(a, out, lse, splits, kchunk, stream);
        case FA_DTYPE_FP16:
            return a.d == 128 ? launch<decltype(&flash_fwd_pp<_Float16, 128, PART>), _Float16>(
                                    &flash_fwd_pp<_Float16, 128, PART>, 8, 256, a, out, lse, splits, kchunk, stream)
                              : launch_d64<_Float16, PART>(a, out, lse, splits, kchunk, stream);
        case FA_DTYPE_FP32:
            return a.d == 128 ? launch<decltype(&flash_fwd_32<128, 32, NW, PART>), float>(
                                    &flash_fwd_32<128, 32, NW, PART>, NW, BR, a, out, lse, splits, kchunk, stream)
                              : launch<decltype(&flash_fwd_32<64, 64, NW, PART>), float>(
                                    &flash_fwd_32<64, 64, NW, PART>, NW, BR, a, out, lse, splits, kchunk, stream);
        default:
            return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// Merge of normalised partial results (the merge rule of the unite.ai page,
// section "La Matemática detrás de la Atención Flash", formula 2, with its
// normalisers restored, in log-sum-exp form): per row, with parts
// (O_s, LSE_s), m = max_s LSE_s, w_s = exp(LSE_s - m):
//     O = sum_s w_s O_s / sum_s w_s,   LSE = m + ln sum_s w_s.
// A part with LSE_s = -inf weighs 0; a row whose parts are all -inf gets
// O = 0, LSE = -inf.  D/4 lanes per row, 4 floats each; grid-stride.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256)
fa_merge_rows(const float* __restrict__ Op, const float* __restrict__ Lp, T* __restrict__ O,
              float* __restrict__ LSE, int64_t G, int S, int64_t M)
{
    constexpr int LPR = D / 4;               // lanes per row
    constexpr int RPB = 256 / LPR;           // rows per block pass
    const int64_t rows = G * M;
    const int part = threadIdx.x % LPR;
    for (int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR; row < rows;
         row += (int64_t)gridDim.x * RPB) {
        const int64_t g = row / M;
        const int64_t p0 = g * S * M + (row - g * M);   // part s of this row: p0 + s M
        float m = -INFINITY;
        for (int s = 0; s < S; ++s) m = fmaxf(m, Lp[p0 + s * M]);
        const float ms = m == -INFINITY ? 0.f : m;
        float l = 0.f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s = 0; s < S; ++s) {
            const float w = __builtin_amdgcn_exp2f((Lp[p0 + s * M] - ms) * 1.4426950408889634f);
            const float4 o = *(const float4*)(Op + (p0 + s * M) * D + 4 * part);
            l += w;
            acc.x = fmaf(w, o.x, acc.x);
            acc.y = fmaf(w, o.y, acc.y);
            acc.z = fmaf(w, o.z, acc.z);
            acc.w = fmaf(w, o.w, acc.w);
        }
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        const float ov[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
        if constexpr (sizeof(T) == 4) {
            *(float4*)((float*)O + row * D + 4 * part) = make_float4(ov[0], ov[1], ov[2], ov[3]);
        } else {
            *(u32x2*)(O + row * D + 4 * part) = Mfma<T>::pack4(ov);
        }
        if (part == 0) LSE[row] = l > 0.f ? m + logf(l) : -INFINITY;
    }
}

template <typename T, int D>
hipError_t launch_merge_t(const float* op, const float* lp, int64_t g, int64_t s, int64_t m, void* o, float* lse,
                          hipStream_t stream) {
    constexpr int RPB = 256 / (D / 4);
    const int64_t need = (g * m + RPB - 1) / RPB;
    const int blocks = (int)(need < 8192 ? need : 8192);
    hipLaunchKernelGGL((fa_merge_rows<T, D>), dim3(blocks), dim3(256), 0, stream, op, lp, (T*)o, lse, g, (int)s, m);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const FwdArgs& a, hipStream_t stream) {
    return launch_kernel<false>(a, a.o, a.lse, 1, (int)a.n, stream);
}

hipError_t launch_forward_split(const FwdArgs& a, int splits, int kchunk, float* o_part, float* lse_part,
                                hipStream_t stream) {
    hipError_t e = launch_kernel<true>(a, o_part, lse_part, splits, kchunk, stream);
    if (e != hipSuccess) return e;
    return launch_merge(o_part, lse_part, a.bh, splits, a.n, a.d, a.o, a.lse, a.dtype, stream);
}

hipError_t launch_merge(const float* o_parts, const float* lse_parts, int64_t g, int64_t s, int64_t m, int d,
                        void* o, float* lse, int dtype, hipStream_t stream) {
    switch (dtype) {
        case FA_DTYPE_BF16:
            return d == 128 ? launch_merge_t<__bf16, 128>(o_parts, lse_parts, g, s, m, o, lse, stream)
                            : launch_merge_t<__bf16, 64>(o_parts, lse_parts, g, s, m, o, lse, stream);
        case FA_DTYPE_FP16:
            return d == 128 ? launch_merge_t<_Float16, 128>(o_parts, lse_parts, g, s, m, o, lse, stream)
                            : launch_merge_t<_Float16, 64>(o_parts, lse_parts, g, s, m, o, lse, stream);
        case FA_DTYPE_FP32:
            return d == 128 ? launch_merge_t<float, 128>(o_parts, lse_parts, g, s, m, o, lse, stream)
                            : launch_merge_t<float, 64>(o_parts, lse_parts, g, s, m, o, lse, stream);
        default:
            return hipErrorInvalidValue;
    }
}

int forward_rows_per_workgroup(int dtype, int d) {
    return (dtype != FA_DTYPE_FP32 && d == 128) ? 256 : 128;
}

int forward_workgroups_per_cu(int dtype, int d) {
    return (dtype != FA_DTYPE_FP32 && d == 128) ? 1 : 2;
}

const char* kernel_config_string() {
    return "flash_fwd gfx950: d128 fp16/bf16 ping-pong 8 waves x 32 query rows, 64-key tiles; "
           "key split into 64-key-aligned ranges + fp32 partial merge; "
           "d64 fp16/bf16 4 waves x 32 rows, 2 workgroups/CU; fp32 4 waves (key tile 64, d128: 32); "
           "MFMA 32x32x16 bf16/f16, 32x32x2 f32";
}

}  // namespace fa
