// Batched kernels (several tokens per call) of the routed int4 MoE layer,
// gfx950.
//
// The batch-union rule of the colibrì summary (fr.news.hada.io topic 31297,
// "Principales fonctionnalités implémentées": in prefill and in the batched
// verification forward, each distinct expert of the batch is read once and
// applied to every position routed to it) on one GPU:
//   1. router: partial logits of all tokens on the matrix cores (fp32) over
//      column splits, W_r read once per 16 tokens;
//   2. top-k: logits summed over the splits, sigmoid, bias, group-limited
//      top-k per token (one wave each); the tokens' activations are converted
//      to scaled fp16 in MFMA operand order;
//   3. dispatch: one workgroup sorts the T*K (token, slot) entries by
//      expert then token in LDS, and writes counts, offsets, the permutation
//      and its inverse, the distinct experts and the tile list (up to 16 or 32
//      entries of one expert per tile; the shared expert's T tokens last);
//   4. gate/up: grouped int4 GEMM per (tile, 128 rows) on the matrix cores
//      (tiles of up to 32 entries when a call averages 8 or more per expert:
//      two MFMA row blocks share each dequantised weight fragment, and a
//      workgroup of 16 waves covers 256 rows);
//   5. h prep: h per entry as scaled fp16 (hi + lo parts for the exact-
//      fragment codecs) in MFMA order;
//   6. down: grouped int4 GEMM per (tile, 256 output rows);
//   7. combine: y = sum_j w_j d_j + d_shared in slot order (no atomics).
//
// Grouped GEMM scheme.  v_mfma_f32_16x16x32_f16 with the 16 tokens of a tile
// as its A rows and 16 weight rows as its B columns; K = 32 is exactly one
// scale group.  Int4 weights are dequantised in registers to fp16(code x
// scale), one rounding of relative size at most 2^-11, and the MFMAs
// accumulate over K in fp32.  The other codecs keep exact fragments (codes
// as fp16 integers or E2M1 values) and scale each MFMA's 16x16 group result
// by its row's group scale in fp32.
// A lane of quarter q loads 16 contiguous code bytes (one group of one row);
// a 4x4 exchange of dwords between the four quarters (permlane32/16 swaps)
// turns the four loads of a quarter-row into the B fragments of four
// consecutive groups.  Codes become fp16 through the same mantissa-OR and
// exact subtraction as in the decode kernels, which orders the 8 values of a
// fragment as columns (0,4,1,5,2,6,3,7) of its k-block; the activations are
// stored in that order.  Tokens' activations for a stage of K are staged
// in LDS (double buffered, one barrier per stage) and read as A fragments.
// MXFP4 experts take the same kernels: an E2M1 code dword becomes the same
// fragment through v_cvt_scalef32_pk_f16_fp4 and byte permutes, and the
// E8M0 byte takes the fp16 scale's place.  Int2 experts (two rows to a
// stored nibble) give two fragments per code dword, the even and the odd
// row's, into accumulators of their own.  Int8 experts run every group
// step once per nibble plane: the high plane's codes become 16 (c - 8) and
// the low plane's c exactly in fp16, two MFMAs under the group's one scale.  With the adaptive top-p cut a
// dropped choice (id -1) gets no dispatch entry and the combine skips it.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_device.h"
#include "moe_kernels.h"
#include "moe_layout.h"

namespace moe {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_lo(unsigned d) { return __builtin_bit_cast(float, d << 16); }
__device__ __forceinline__ float bf16_hi(unsigned d) { return __builtin_bit_cast(float, d & 0xFFFF0000u); }

__device__ __forceinline__ unsigned pack_h2(_Float16 lo, _Float16 hi) {
    return (unsigned)__builtin_bit_cast(unsigned short, lo) | ((unsigned)__builtin_bit_cast(unsigned short, hi) << 16);
}

// 8 offset-binary codes of one dword (columns 8q..8q+7 of a group, column c
// at bits 4c) -> fp16 values in fragment order (columns 0,4,1,5,2,6,3,7).
// The two exponent patterns OR-ed into the masked codes, held in VGPRs (see
// magic_exponents) so that each mask-and-or is one v_and_or_b32: a VOP3
// instruction here can take one scalar or literal operand, not two.
struct MagicExp {
    unsigned e1024, e64;  // 0x6400 (1024.0) and 0x5400 (64.0) in both halves
};
__device__ __forceinline__ MagicExp magic_exponents() {
    MagicExp m{0x64006400u, 0x54005400u};
    asm volatile("" : "+v"(m.e1024), "+v"(m.e64));
    return m;
}

// OFF = 8: offset-binary codes c -> c - 8 (int4); OFF = 0: unsigned c (the
// low-nibble plane of int8 codes).
template <int OFF = 8>
__device__ __forceinline__ f16x8 codes_to_f16x8(unsigned w, const MagicExp& mg) {
    const f16x2 k_lo = {(_Float16)(1024.0f + OFF), (_Float16)(1024.0f + OFF)};
    const f16x2 k_hi = {(_Float16)(64.0f + OFF), (_Float16)(64.0f + OFF)};
    const unsigned w8 = w >> 8;
    const f16x2 q0 = as_h2((w & 0x000F000Fu) | mg.e1024) - k_lo;
    const f16x2 q1 = as_h2((w & 0x00F000F0u) | mg.e64) - k_hi;
    const f16x2 q2 = as_h2((w8 & 0x000F000Fu) | mg.e1024) - k_lo;
    const f16x2 q3 = as_h2((w8 & 0x00F000F0u) | mg.e64) - k_hi;
    const u32x4 v = {__builtin_bit_cast(unsigned, q0), __builtin_bit_cast(unsigned, q1),
                     __builtin_bit_cast(unsigned, q2), __builtin_bit_cast(unsigned, q3)};
    return __builtin_bit_cast(f16x8, v);
}

// MXFP4: the same fragment order from eight E2M1 codes (code byte j holds
// columns 2j and 2j + 1): v_cvt_scalef32_pk_f16_fp4 turns each byte into an
// exact fp16 pair (scale 1), and byte permutes pair columns c and c + 4.
__device__ __forceinline__ f16x8 fp4_to_f16x8(unsigned w) {
    const unsigned p0 = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0));
    const unsigned p1 = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1));
    const unsigned p2 = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2));
    const unsigned p3 = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3));
    const u32x4 v = {__builtin_amdgcn_perm(p2, p0, 0x05040100u), __builtin_amdgcn_perm(p2, p0, 0x07060302u),
                     __builtin_amdgcn_perm(p3, p1, 0x05040100u), __builtin_amdgcn_perm(p3, p1, 0x07060302u)};
    return __builtin_bit_cast(f16x8, v);
}
// High-nibble plane of int8 codes (offset binary c): 16 (c - 8) exactly.
// Every nibble is moved to bits 4-7 of its half, where under the exponent
// of 1024 (ulp 1) it reads 1024 + 16c.
__device__ __forceinline__ f16x8 hi_codes_to_f16x8(unsigned w, const MagicExp& mg) {
    const f16x2 k = {(_Float16)1152.0f, (_Float16)1152.0f};  // 1024 + 128
    const f16x2 q0 = as_h2(((w << 4) & 0x00F000F0u) | mg.e1024) - k;
    const f16x2 q1 = as_h2((w & 0x00F000F0u) | mg.e1024) - k;
    const f16x2 q2 = as_h2(((w >> 4) & 0x00F000F0u) | mg.e1024) - k;
    const f16x2 q3 = as_h2(((w >> 8) & 0x00F000F0u) | mg.e1024) - k;
    const u32x4 v = {__builtin_bit_cast(unsigned, q0), __builtin_bit_cast(unsigned, q1),
                     __builtin_bit_cast(unsigned, q2), __builtin_bit_cast(unsigned, q3)};
    return __builtin_bit_cast(f16x8, v);
}
// Int2 codes two rows to a nibble (row 2v in bits 0-1, row 2v + 1 in bits
// 2-3, each + 2): the fragment of the row in bits 0-1 of every nibble (the
// other row's is that of w >> 2).
__device__ __forceinline__ f16x8 codes2_to_f16x8(unsigned w, const MagicExp& mg) {
    const f16x2 k_lo = {(_Float16)1026.0f, (_Float16)1026.0f};  // 1024 + 2
    const f16x2 k_hi = {(_Float16)66.0f, (_Float16)66.0f};      // 64 + 2
    const unsigned w8 = w >> 8;
    const f16x2 q0 = as_h2((w & 0x00030003u) | mg.e1024) - k_lo;
    const f16x2 q1 = as_h2((w & 0x00300030u) | mg.e64) - k_hi;
    const f16x2 q2 = as_h2((w8 & 0x00030003u) | mg.e1024) - k_lo;
    const f16x2 q3 = as_h2((w8 & 0x00300030u) | mg.e64) - k_hi;
    const u32x4 v = {__builtin_bit_cast(unsigned, q0), __builtin_bit_cast(unsigned, q1),
                     __builtin_bit_cast(unsigned, q2), __builtin_bit_cast(unsigned, q3)};
    return __builtin_bit_cast(f16x8, v);
}
// B fragment of one code dword of nibble plane pl (int8: 0 high, 1 low; the
// two planes' products under one scale sum to the int8 code's product) and
// row parity h (int2: 0 the even row, 1 the odd row of the stored row).
template <int F>
__device__ __forceinline__ f16x8 dequant_f16x8(unsigned w, const MagicExp& mg, int pl = 0, int h = 0) {
    if constexpr (F == kCodecMxfp4)
        return fp4_to_f16x8(w);
    else if constexpr (F == kCodecInt8)
        return pl ? codes_to_f16x8<0>(w, mg) : hi_codes_to_f16x8(w, mg);
    else if constexpr (F == kCodecInt2)
        return codes2_to_f16x8(h ? w >> 2 : w, mg);
    else
        return codes_to_f16x8(w, mg);
}
// A scale held in 16 bits (fp16 bits for int4, the E8M0 byte for MXFP4).
template <int F>
__device__ __forceinline__ float scale16(unsigned v) {
    if constexpr (F == kCodecMxfp4)
        return e8m0_to_float(v & 0xFFu);
    else
        return half_bits_to_float(v & 0xFFFFu);
}

// Lane (i, q) = (lane & 15, lane >> 4) holds the 4 dwords T[q][0..3] of
// group g+q of row i; afterwards d[m] holds T[m][q], i.e. dword q (columns
// 8q..8q+7) of group g+m: the B fragment of group g+m.
__device__ __forceinline__ void transpose_quarters(u32x4& d) {
    const auto r02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
    const auto r13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
    const auto r01 = __builtin_amdgcn_permlane16_swap(r02[0], r13[0], false, false);
    const auto r23 = __builtin_amdgcn_permlane16_swap(r02[1], r13[1], false, false);
    d[0] = r01[0];
    d[1] = r01[1];
    d[2] = r23[0];
    d[3] = r23[1];
}

// The fp16 scale in the low 16 bits of v in all eight lanes of a fragment.
__device__ __forceinline__ f16x8 splat_h8(unsigned v) {
    const _Float16 s = __builtin_bit_cast(_Float16, (unsigned short)(v & 0xFFFFu));
    return f16x8{s, s, s, s, s, s, s, s};
}

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int pair_token(const BatchArgs& a, int p) {
    const int n = a.T * a.K;
    return p < n ? a.perm[p] / a.K : p - n;
}

// Column of position j of a fragment inside its 8-column k-block.
__device__ __forceinline__ constexpr int frag_col(int j) { return (j >> 1) + 4 * (j & 1); }

// ---------------------------------------------------------------- router
// Partial logits of a 64-token x 16 NEB-expert tile over one of
// router_splits column ranges, on the matrix cores (v_mfma_f32_16x16x4_f32:
// tokens as A rows, W_r rows as B columns, bf16 activations widened exactly
// to fp32).  Wave w of the workgroup takes tokens 16w..16w+15 of the tile
// over the whole range, NEB expert blocks sharing each activation load; a
// lane loads 4 consecutive columns of its token and of its experts and feeds
// them to 4 MFMAs, one column each, so every k-block of an MFMA covers the
// same columns in A and B.  The splits are summed in order by the top-k
// kernel (deterministic).  Grid (expert tiles, splits, token tiles): with 4
// expert tiles and 16 splits a workgroup's XCD (its linear index mod 8)
// depends on the expert tile and the split only, so each block of W_r is read
// into one XCD's L2 for all token tiles.
template <int NEB, int NS>
__global__ void __launch_bounds__(256) batch_router_kernel(BatchArgs a) {
    // steps of 16 columns in flight (8 x 18 registers with 4 expert blocks)
    constexpr int DMAX = NEB == 4 ? 8 : 12;
    constexpr int D = NS < DMAX ? NS : DMAX;
    const int lane = threadIdx.x & 63, wv = wave_in_block();
    const int m = lane & 15, q = lane >> 4;
    const int e0 = blockIdx.x * 16 * NEB, split = blockIdx.y, t0 = blockIdx.z * 64 + 16 * wv;
    if (t0 >= a.T) return;
    const int t = t0 + m;
    const bool tok = t < a.T;
    const int c0 = split * (16 * NS) + 4 * q;  // a split is NS steps of 16 columns
    const uint16_t* xr = a.x + (size_t)(tok ? t : 0) * a.H + c0;
    const float* wr = a.router_w + (size_t)(e0 + m) * a.H + c0;
    f32x4 acc[NEB];
#pragma unroll
    for (int b = 0; b < NEB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x2 xv[D];
    f32x4 w[D][NEB];
    auto load = [&](int k, int slot) {
        xv[slot] = tok ? *as_global<u32x2>(xr + 16 * k) : u32x2{0u, 0u};
#pragma unroll
        for (int b = 0; b < NEB; ++b) w[slot][b] = *as_global<f32x4>(wr + (size_t)16 * b * a.H + 16 * k);
    };
#pragma unroll
    for (int k = 0; k < D; ++k) load(k, k);
    // straight-line over the split: step k is computed from its slot, which
    // then takes step k + D
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        const int slot = k % D;
        const float x0 = bf16_lo(xv[slot][0]), x1 = bf16_hi(xv[slot][0]);
        const float x2 = bf16_lo(xv[slot][1]), x3 = bf16_hi(xv[slot][1]);
#pragma unroll
        for (int b = 0; b < NEB; ++b) {
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(x0, w[slot][b][0], acc[b], 0, 0, 0);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(x1, w[slot][b][1], acc[b], 0, 0, 0);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(x2, w[slot][b][2], acc[b], 0, 0, 0);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(x3, w[slot][b][3], acc[b], 0, 0, 0);
        }
        if (k + D < NS) load(k + D, slot);
    }
    // lane holds tokens t0 + 4q + j of experts e0 + 16b + m
    float* out = a.logit_part + (size_t)split * a.T * a.E;
#pragma unroll
    for (int b = 0; b < NEB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tt = t0 + 4 * q + j;
            if (tt < a.T) out[(size_t)tt * a.E + e0 + 16 * b + m] = acc[b][j];
        }
}

// ---------------------------------------------------------------- top-k
// Group-limited top-k of token t on one wave.
template <int EPL>
__device__ __forceinline__ void topk_token(const BatchArgs& a, int t, int lane) {
    // logits = in-order sum of the router's partial sums (all partials
    // loaded first, so the loads overlap); s = sigmoid, sb = s + bias
    constexpr int MAXSP = kMaxRouterSplits;
    float part[MAXSP][EPL];
#pragma unroll
    for (int sp = 0; sp < MAXSP; ++sp)
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane * EPL + i;
            part[sp][i] = sp < a.router_splits && e < a.E ? a.logit_part[((size_t)sp * a.T + t) * a.E + e] : 0.0f;
        }
    float sv[EPL], key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        sv[i] = 0.0f;
        key[i] = -__builtin_inff();
        if (e < a.E) {
            float l = 0.0f;
#pragma unroll
            for (int sp = 0; sp < MAXSP; ++sp)
                if (sp < a.router_splits) l += part[sp][i];
            sv[i] = 1.0f / (1.0f + expf(-l));
            key[i] = sv[i] + a.bias[e];
        }
    }
    int id;
    float wt;
    wave_group_topk_values<EPL>(sv, key, a.E, a.G, a.TG, a.K, a.rsf, a.top_p, lane, &id, &wt);
    if (lane < a.K) {
        a.ids[(size_t)t * a.K + lane] = id;
        a.w[(size_t)t * a.K + lane] = wt;
    }
}

// Token t's activations on one wave: fp16 scaled by 2^kx (max |x| into
// [2^13, 2^14)), stored per (group, quarter) as 8 values in fragment order.
template <int CPL>
__device__ __forceinline__ void convert_token(const BatchArgs& a, int t, int lane) {
    const int KG = a.H / 32;
    const uint16_t* xr = a.x + (size_t)t * a.H;
    u32x4 raw[CPL][4];
    unsigned mx = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int g = lane + kWave * c;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            raw[c][q] = g < KG ? *as_global<u32x4>(xr + 32 * g + 8 * q) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const unsigned d = raw[c][q][z];
                mx = umax(mx, umax(d & 0x7FFFu, (d >> 16) & 0x7FFFu));
            }
        }
    }
    const int k = range_exponent(wave_max_u32(mx) >> 7);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int g = lane + kWave * c;
        if (g >= KG) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            _Float16 hv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int col = frag_col(j);
                const unsigned d = raw[c][q][col >> 1];
                const float f = (col & 1) ? bf16_hi(d) : bf16_lo(d);
                hv[j] = (_Float16)ldexpf(f, k);
            }
            const u32x4 o = {pack_h2(hv[0], hv[1]), pack_h2(hv[2], hv[3]), pack_h2(hv[4], hv[5]),
                             pack_h2(hv[6], hv[7])};
            *reinterpret_cast<u32x4*>(a.xa + (size_t)t * a.H + (size_t)(g * 4 + q) * 8) = o;
        }
    }
    if (lane == 0) a.kx[t] = k;
}

// One wave per token: the top-k in workgroups with blockIdx.y = 0 and,
// when the launch has a second row (convert), the activations in those with
// blockIdx.y = 1 (the two do not depend on each other).
template <int EPL, int CPL>
__global__ void __launch_bounds__(256) batch_topk_kernel(BatchArgs a) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave_in_block();
    if (t >= a.T) return;
    if (blockIdx.y == 0)
        topk_token<EPL>(a, t, lane);
    else
        convert_token<CPL>(a, t, lane);
}

// ---------------------------------------------------------------- dispatch
__device__ __forceinline__ int wave_exclusive_scan(int v, int lane, int* total) {
    int x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    *total = __shfl(x, kWave - 1);
    return x - v;
}

// One workgroup of 16 waves; a stable counting placement (entries by
// expert, then token, then slot).  Wave w owns a consecutive range of
// entries and walks it 64 at a time: a lane finds the lanes holding the same
// expert with eight ballots over the id's bits, so its rank among the wave's
// entries of that expert so far is the wave's running count (LDS) plus the
// number of such lanes below it.  The counts per wave and expert are then
// turned into each wave's first place per expert (expert offset plus the
// counts of the waves before it), and every entry goes to that place plus
// its rank.
constexpr int kDispatchWaves = 16;
__global__ void __launch_bounds__(64 * kDispatchWaves) batch_dispatch_kernel(BatchArgs a) {
    __shared__ int whist[kDispatchWaves][256];  // per wave: entries per expert, then its first place per expert
    __shared__ int rank[kMaxDispatchEntries];   // an entry's rank among its wave's entries of its expert
    __shared__ int cnt[256], off[256], toff[256], dpos[256], spos[256];
    __shared__ int totals[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = a.T * a.K;
    // an id outside [0, E) takes no entry, as a choice the top-p cut dropped
    auto valid = [&](int i) { return i < n && a.ids[i] >= 0 && a.ids[i] < a.E; };
    for (int i = tid; i < kDispatchWaves * 256; i += 64 * kDispatchWaves) (&whist[0][0])[i] = 0;
    __syncthreads();
    const int per_wave = (n + 64 * kDispatchWaves - 1) / (64 * kDispatchWaves) * 64;
    const int first = wv * per_wave;
    for (int i = first + lane; i < first + per_wave; i += 64) {
        const bool v = valid(i);
        const int e = v ? a.ids[i] : 0;
        unsigned long long same = __ballot(v);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const unsigned long long ones = __ballot((e >> bit) & 1);
            same &= ((e >> bit) & 1) ? ones : ~ones;
        }
        const int below = __popcll(same & ((1ull << lane) - 1));
        const int prev = v ? whist[wv][e] : 0;
        if (v) rank[i] = prev + below;
        __builtin_amdgcn_wave_barrier();
        if (v && below == 0) whist[wv][e] = prev + __popcll(same);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    if (tid < 256) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kDispatchWaves; ++w) c += whist[w][tid];
        cnt[tid] = c;
    }
    __syncthreads();
    if (tid < kWave) {
        // per expert: entries, MFMA tiles (none for a single), distinct
        // flag, single flag (1 to single_max entries: the GEMV path)
        int c[4], nt[4], f[4], g[4];
        int sc = 0, stl = 0, sf = 0, sg = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = 4 * tid + r;
            c[r] = e < a.E ? cnt[e] : 0;
            g[r] = c[r] > 0 && c[r] <= a.single_max ? 1 : 0;
            nt[r] = g[r] ? 0 : (c[r] + a.tile_tokens - 1) / a.tile_tokens;
            f[r] = c[r] > 0 ? 1 : 0;
            sc += c[r];
            stl += nt[r];
            sf += f[r];
            sg += g[r];
        }
        int tc, tt, tf, tg;
        int bc = wave_exclusive_scan(sc, tid, &tc);
        int bt = wave_exclusive_scan(stl, tid, &tt);
        int bf = wave_exclusive_scan(sf, tid, &tf);
        int bg = wave_exclusive_scan(sg, tid, &tg);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = 4 * tid + r;
            if (e < a.E) {
                off[e] = bc;
                toff[e] = bt;
                dpos[e] = bf;
                spos[e] = g[r] ? bg : -1;
            }
            bc += c[r];
            bt += nt[r];
            bf += f[r];
            bg += g[r];
        }
        if (tid == 0) {
            totals[0] = tc;
            totals[1] = tt;
            totals[2] = tf;
            totals[3] = tg;
        }
    }
    __syncthreads();
    // each wave's first place per expert
    if (tid < a.E) {
        int p = off[tid];
#pragma unroll
        for (int w = 0; w < kDispatchWaves; ++w) {
            const int c = whist[w][tid];
            whist[w][tid] = p;
            p += c;
        }
    }
    __syncthreads();
    // kept entries fill pairs [0, totals[0]); the rest of perm is -1 and a
    // dropped choice's inv is -1
    const int n_kept = totals[0];
    for (int i = first + lane; i < first + per_wave && i < n; i += 64) {
        if (valid(i)) {
            const int p = whist[wv][a.ids[i]] + rank[i];
            a.perm[p] = i;
            a.inv[i] = p;
        } else {
            a.inv[i] = -1;
        }
    }
    for (int p = n_kept + tid; p < n; p += 64 * kDispatchWaves) a.perm[p] = -1;
    for (int e = tid; e < a.E; e += 64 * kDispatchWaves) {
        const int c = cnt[e];
        a.counts[e] = c;
        a.offsets[e] = off[e];
        if (c > 0) {
            a.distinct[dpos[e]] = e;
            if (spos[e] >= 0)
                a.singles[spos[e]] = Tile{e, off[e], c, 0};
            else
                for (int i = 0; i * a.tile_tokens < c; ++i)
                    a.tiles[toff[e] + i] =
                        Tile{e, off[e] + a.tile_tokens * i, min(a.tile_tokens, c - a.tile_tokens * i), 0};
        }
    }
    if (tid == 0) {
        a.offsets[a.E] = n_kept;
        a.n_distinct[0] = totals[2];
        int nt = totals[1];
        for (int s = 0; s < a.S; ++s)
            for (int t0 = 0; t0 < a.T; t0 += a.tile_tokens)
                a.tiles[nt++] = Tile{a.E, n + t0, min(a.tile_tokens, a.T - t0), 0};
        a.n_tiles[0] = nt;
        if (a.n_singles) a.n_singles[0] = totals[3];
    }
}

// ---------------------------------------------------------------- item order
// Item k of workgroup b in the grouped kernels.  A launch's workgroups are
// dealt to the chip's 8 XCDs round robin (workgroup b runs on XCD b % 8, each
// XCD with an L2 of its own), so with a grid that is a multiple of 8 the item
// range is cut into 8 consecutive parts and XCD x's workgroups walk part x in
// order: the row blocks of one tile, which stage the same activations, then
// run side by side on one XCD and read them through its L2 once, instead of
// once on every XCD.  Returns a value >= items past the workgroup's last item.
__device__ __forceinline__ int grouped_item(int b, int grid, int k, int items) {
    if (grid & 7) return b + k * grid;
    const int per = (items + 7) >> 3;
    const int i = (b >> 3) + k * (grid >> 3);
    return i < per ? (b & 7) * per + i : items;
}

// ---------------------------------------------------------------- gate/up
// Gate and up scales of row r for groups g..g+3 as dwords (gate | up << 16).
// (MXFP4: E8M0 bytes in the same 16-bit places.)
template <int KG, int F>
__device__ __forceinline__ u32x4 gateup_scales4(const uint8_t* gus, int r, int g) {
    if constexpr (F == kCodecMxfp4) {
        if constexpr (KG >= kWave) {
            const u32x2 b = *as_global<u32x2>(gus + gateup_scale_index(r, g, 0, KG, 1));
            return u32x4{(b[0] & 0xFFu) | ((b[0] >> 8 & 0xFFu) << 16), (b[0] >> 16 & 0xFFu) | ((b[0] >> 24) << 16),
                         (b[1] & 0xFFu) | ((b[1] >> 8 & 0xFFu) << 16), (b[1] >> 16 & 0xFFu) | ((b[1] >> 24) << 16)};
        } else {
            constexpr int p = gateup_rows(KG);
            u32x4 v;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                v[m] = (unsigned)*as_global<uint8_t>(gus + gateup_scale_index(r, g + m, 0, KG, p)) |
                       ((unsigned)*as_global<uint8_t>(gus + gateup_scale_index(r, g + m, 1, KG, p)) << 16);
            return v;
        }
    } else {
        const uint16_t* gus16 = reinterpret_cast<const uint16_t*>(gus);
        if constexpr (KG >= kWave) {
            return *as_global<u32x4>(gus16 + gateup_scale_index(r, g, 0, KG, 1));
        } else {
            constexpr int p = gateup_rows(KG);
            u32x4 v;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                v[m] = (unsigned)*as_global<uint16_t>(gus16 + gateup_scale_index(r, g + m, 0, KG, p)) |
                       ((unsigned)*as_global<uint16_t>(gus16 + gateup_scale_index(r, g + m, 1, KG, p)) << 16);
            return v;
        }
    }
}

// Workgroup = W waves over 16 W rows of gate and the same rows of up for
// the (up to) TT tokens of one tile; wave w owns rows 16w..16w+15.  Rows
// are stored rows: with int2 (two rows per stored row) a workgroup covers
// twice as many matrix rows, with the even and the odd rows in accumulators
// of their own.  W = 8 (two workgroups per CU), or 16 (one per CU) for
// 32-entry tiles: a prefill item then stages its tile's activations once per
// 256 rows instead of once per 128 (prefill gate/up 0.93 ms to 0.88 ms per
// 512-token call); calls with few entries per expert keep 8 waves, whose
// twice as many items balance better over the CUs.
template <int KG, int F, int TT, int W>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(4))) batch_gateup_kernel(BatchArgs a) {
    // groups per LDS stage (8 when a 32-entry tile's two MFMA row blocks or
    // a two-fragment codec need the staging registers, else 16)
    static_assert(TT == 16 || TT == 32, "tile entries");
    static_assert(W == 8 || W == 16, "waves per workgroup");
    constexpr int NT = 64 * W;              // threads
    constexpr int NB = TT / 16;             // MFMA row blocks (16 tokens each) per tile
    constexpr int CK = KG < 16 ? KG : (NB > 1 || code_planes(F) > 1 || row_pack(F) > 1 ? 8 : 16);
    constexpr int NST = KG / CK;
    constexpr int NX = CK * 64 * NB;        // 16-byte staging elements of a stage
    constexpr int PT = (NX + NT - 1) / NT;  // per thread
    static_assert(CK % 4 == 0 && KG % CK == 0, "gate/up stage shape");
    __shared__ u32x4 xs[2][CK * 64 * NB];   // [(g * 4 + q) * TT + token]
    __shared__ int s_kx[2][TT];             // the entries' activation exponents, by item parity
    const int tid = threadIdx.x, lane = tid & 63, wv = wave_in_block();
    const int i = lane & 15, q = lane >> 4;
    const int n_tiles = a.n_tiles[0];
    constexpr int RP = row_pack(F);
    const int rblocks = a.I / (16 * W * RP);
    const int items = n_tiles * rblocks;
    const BlobLayout L = blob_layout(a.H, a.I, F);
    const int row_bytes = a.H / 2;
    const MagicExp mg = magic_exponents();
    int gs = 0;  // stages so far: selects the LDS buffer
    for (int ik = 0, item = grouped_item(blockIdx.x, gridDim.x, 0, items); item < items;
         item = grouped_item(blockIdx.x, gridDim.x, ++ik, items)) {
        const int tile = item / rblocks, rb = item - tile * rblocks;
        const Tile td = a.tiles[tile];
        const uint8_t* blob = td.expert < a.E ? a.table[td.expert] : a.shared_blob;
        const int row = rb * 16 * W + wv * 16 + i;
        const uint8_t* gq = blob + L.gate_q + (size_t)row * row_bytes;
        const uint8_t* uq = blob + L.up_q + (size_t)row * row_bytes;
        const uint8_t* gql = blob + L.gate_lo + (size_t)row * row_bytes;  // int8 low planes
        const uint8_t* uql = blob + L.up_lo + (size_t)row * row_bytes;
        const uint8_t* gus = blob + L.gu_s;
        const uint8_t* gus2 = blob + L.gu_s2;  // int2 odd rows
        const int sm = tid & (TT - 1);
        const uint16_t* xsrc = sm < td.count ? a.xa + (size_t)pair_token(a, td.first_pair + sm) * a.H : nullptr;
        f32x4 accg[RP][NB], accu[RP][NB];
#pragma unroll
        for (int h = 0; h < RP; ++h)
#pragma unroll
            for (int z = 0; z < NB; ++z) accg[h][z] = accu[h][z] = f32x4{0.f, 0.f, 0.f, 0.f};
        // the activation scaling exponents of the tile's entries for the
        // stores after the last step: thread tt < TT fetches entry tt's token
        // now and its exponent a quarter into the item and writes it to LDS
        // half-way (before a stage barrier); every thread issues the loads
        // (an entry past the count takes the last entry's), so the code
        // loads' wait counts stay exact and the stores wait on no load
        // (int4; the other codecs' kernels have no register to spare and
        // load the exponents in the stores)
        const int ib = ik & 1;
        int kxr = 0;
        if constexpr (F == kCodecInt4) {
            const int n_pairs = a.T * a.K;
            const int p = td.first_pair + (sm < td.count ? sm : td.count - 1);
            const int v = a.perm[p < n_pairs ? p : n_pairs - 1];
            kxr = p < n_pairs ? v / a.K : p - n_pairs;
        }
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        constexpr int NS = KG / 4;  // steps of 4 groups
        constexpr int P = code_planes(F);
        constexpr int NSP = NS * P;  // (step, plane) code loads, plane fastest
        // codes of load k = (step s, plane pl): lane of quarter q reads group
        // 4s + q of plane pl
        auto load_step = [&](int k, u32x4& g, u32x4& u) {
            const int s = k / P, pl = k - s * P;
            g = *as_global<u32x4>((pl ? gql : gq) + (4 * s + q) * 16);
            u = *as_global<u32x4>((pl ? uql : uq) + (4 * s + q) * 16);
        };
        // scales, four steps at a time: for steps 4h .. 4h+3 lane (i, q)
        // fetches step 4h + q of row i (16 bytes, so a wave load covers 16
        // rows x 64 bytes); step s's scales come from lane (i, s % 4) by a
        // lane shuffle
        auto quad_scales = [&](int h, u32x4 (&v)[RP]) {
            const int s = 4 * h + q;
#pragma unroll
            for (int z = 0; z < RP; ++z)
                v[z] = s < NS ? gateup_scales4<KG, F>(z ? gus2 : gus, row, 4 * s) : u32x4{0u, 0u, 0u, 0u};
        };
        auto stage_load = [&](int st, u32x4 (&v)[PT]) {
#pragma unroll
            for (int r = 0; r < PT; ++r) {
                const int e = tid + NT * r;
                v[r] = xsrc && e < NX ? *as_global<u32x4>(xsrc + (size_t)((st * CK + e / (4 * TT)) * 4 +
                                                        (e / TT) % 4) * 8)
                            : u32x4{0u, 0u, 0u, 0u};
            }
        };
        // two steps of codes in flight ahead of the one being computed, and
        // the next stage's activations in flight during a stage
        u32x4 v[PT];
        stage_load(0, v);
        u32x4 scl[RP], scn[RP];
        quad_scales(0, scl);
#pragma unroll
        for (int z = 0; z < RP; ++z) scn[z] = scl[z];
        u32x4 cg0, cu0, cg1 = {0u, 0u, 0u, 0u}, cu1 = cg1;
        load_step(0, cg0, cu0);
        if (NSP > 1) load_step(1, cg1, cu1);
        // fully unrolled over the stages: a loop back-edge here would make
        // the compiler drain the prefetched loads (register rotation copies)
#pragma unroll
        for (int st = 0; st < NST; ++st, ++gs) {
            if constexpr (F == kCodecInt4) {
                if (st == NST / 4) kxr = a.kx[kxr];
                if (st == NST / 2 && tid < TT) s_kx[ib][tid] = kxr;
            }
            const int buf = gs & 1;
#pragma unroll
            for (int r = 0; r < PT; ++r)
                if (tid + NT * r < NX) xs[buf][tid + NT * r] = v[r];
            __syncthreads();
            if (st + 1 < NST) stage_load(st + 1, v);
#pragma unroll
            for (int c = 0; c < CK / 4; ++c) {
                const int sidx = st * (CK / 4) + c;
                // the next four steps' scales two steps before they are needed
                if ((sidx & 3) == 0 && sidx > 0) {
#pragma unroll
                    for (int z = 0; z < RP; ++z) scl[z] = scn[z];
                }
                if ((sidx & 3) == 2 && sidx + 2 < NS) quad_scales(sidx / 4 + 1, scn);
                u32x4 sc0[RP];
#pragma unroll
                for (int z = 0; z < RP; ++z) {
                    const int src = i + 16 * (sidx & 3);
                    const u32x4 h = scl[z];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const unsigned hv = h[d];  // element copied first (bit_cast of an element reads element 0)
                        sc0[z][d] = (unsigned)__shfl((int)hv, src);
                    }
                }
#pragma unroll
                for (int pl = 0; pl < P; ++pl) {
                    const int k = sidx * P + pl;
                    u32x4 cg2 = cg1, cu2 = cu1;
                    if (k + 2 < NSP) load_step(k + 2, cg2, cu2);
                    transpose_quarters(cg0);
                    transpose_quarters(cu0);
                    if constexpr (F == kCodecInt4) {
                        // int4: each weight enters the MFMA as fp16(code x
                        // scale), one rounding (relative 2^-11), and the
                        // products accumulate in the MFMA's fp32 accumulator
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            const unsigned sv = sc0[0][m];
                            const f16x8 bg = codes_to_f16x8(cg0[m], mg) * splat_h8(sv);
                            const f16x8 bu = codes_to_f16x8(cu0[m], mg) * splat_h8(sv >> 16);
#pragma unroll
                            for (int z = 0; z < NB; ++z) {
                                const f16x8 af =
                                    __builtin_bit_cast(f16x8, xs[buf][((4 * c + m) * 4 + q) * TT + 16 * z + i]);
                                accg[0][z] = mfma16(af, bg, accg[0][z]);
                                accu[0][z] = mfma16(af, bu, accu[0][z]);
                            }
                        }
                    } else {
                    // other codecs: exact fragments, each group's product
                    // scaled in fp32
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
#pragma unroll
                        for (int h = 0; h < RP; ++h) {
                            const f16x8 bg = dequant_f16x8<F>(cg0[m], mg, pl, h);
                            const f16x8 bu = dequant_f16x8<F>(cu0[m], mg, pl, h);
                            const float sg = scale16<F>(sc0[h][m]);
                            const float su = scale16<F>(sc0[h][m] >> 16);
#pragma unroll
                            for (int z = 0; z < NB; ++z) {
                                const f16x8 af = __builtin_bit_cast(
                                    f16x8, xs[buf][((4 * c + m) * 4 + q) * TT + 16 * z + i]);
                                const f32x4 dg = mfma16(af, bg, zero);
                                const f32x4 du = mfma16(af, bu, zero);
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    accg[h][z][j] = fmaf(sg, dg[j], accg[h][z][j]);
                                    accu[h][z][j] = fmaf(su, du[j], accu[h][z][j]);
                                }
                                // scale and accumulate now: one group's two
                                // products in flight at a time (otherwise the
                                // compiler sinks the FMAs to the end of the
                                // stage and spills every product)
                                asm volatile("" : "+v"(accg[h][z]), "+v"(accu[h][z]));
                                __builtin_amdgcn_sched_barrier(0);
                            }
                        }
                    }
                    }
                    cg0 = cg1;
                    cu0 = cu1;
                    cg1 = cg2;
                    cu1 = cu2;
                    // keep the prefetch depth, not the whole stage, in flight
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
#pragma unroll
        for (int z = 0; z < NB; ++z)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tt = 16 * z + 4 * q + j;
                if (tt < td.count) {
                    const int p = td.first_pair + tt;
                    const int kx = F == kCodecInt4 ? s_kx[ib][tt] : a.kx[pair_token(a, p)];
#pragma unroll
                    for (int h = 0; h < RP; ++h) {
                        const float g = ldexpf(accg[h][z][j], -kx), u = ldexpf(accu[h][z][j], -kx);
                        a.h[(size_t)p * a.I + RP * row + h] = g / (1.0f + expf(-g)) * u;
                    }
                }
            }
    }
}

// ---------------------------------------------------------------- h prep
// One workgroup per entry: h as scaled fp16 hi + lo (hi = fp16(h 2^kh),
// lo = fp16(h 2^kh - hi)), kh putting max |h| into [2^13, 2^14); int4
// calls write the hi part only.
template <int CPT>
__global__ void __launch_bounds__(256) batch_hprep_kernel(BatchArgs a) {
    __shared__ unsigned wmax[4];
    const int p = blockIdx.x, tid = threadIdx.x;
    if (p >= a.offsets[a.E] && p < a.T * a.K) return;  // a pair left empty by the top-p cut
    const int n_el = (a.I / 32) * 4;  // (group, quarter) elements of 8 values
    const float* hr = a.h + (size_t)p * a.I;
    f32x4 v[CPT][2];
    unsigned mx = 0;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int e = tid + 256 * c;
#pragma unroll
        for (int z = 0; z < 2; ++z) {
            v[c][z] = e < n_el ? *as_global<f32x4>(hr + 8 * e + 4 * z) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                const float f = v[c][z][y];  // bit_cast of a vector element expression would read element 0
                mx = umax(mx, __builtin_bit_cast(unsigned, f) & 0x7FFFFFFFu);
            }
        }
    }
    mx = wave_max_u32(mx);
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();
    mx = umax(umax(wmax[0], wmax[1]), umax(wmax[2], wmax[3]));
    const int k = range_exponent(mx >> 23);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int e = tid + 256 * c;
        if (e >= n_el) continue;
        _Float16 hi[8], lo[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = frag_col(j);
            const float f = ldexpf(v[c][col >> 2][col & 3], k);
            hi[j] = (_Float16)f;
            lo[j] = (_Float16)(f - (float)hi[j]);
        }
        const size_t o = (size_t)p * a.I + (size_t)e * 8;
        *reinterpret_cast<u32x4*>(a.ha_hi + o) = u32x4{pack_h2(hi[0], hi[1]), pack_h2(hi[2], hi[3]),
                                                       pack_h2(hi[4], hi[5]), pack_h2(hi[6], hi[7])};
        if (a.codec != kCodecInt4)  // the int4 down kernel reads the hi part only
            *reinterpret_cast<u32x4*>(a.ha_lo + o) = u32x4{pack_h2(lo[0], lo[1]), pack_h2(lo[2], lo[3]),
                                                           pack_h2(lo[4], lo[5]), pack_h2(lo[6], lo[7])};
    }
    if (tid == 0) a.kh[p] = k;
}

// ---------------------------------------------------------------- down
constexpr int kDownThreads = 1024;                   // 16 waves
constexpr int kDownBlockRows = kDownThreads / 4;     // 16 rows per wave
// Workgroup = 16 waves over 256 output rows for the (up to) 16 entries of
// one tile (one workgroup per CU: the staged h, as many bytes per item as
// 128 rows of codes, serves twice the rows).  Int4: one MFMA per group on h
// as fp16 (one rounding of at most 2^-11, the size of the weight fragments'
// own); the exact-fragment codecs: two MFMAs (hi and lo parts of h, ~22
// bits) into one result.  Rows are stored rows (int2: 512 output
// rows, even and odd accumulated apart, the two rows' scales of a group in
// one dword).
template <int KGI, int F, int TT>
__global__ void __launch_bounds__(kDownThreads) __attribute__((amdgpu_waves_per_eu(4))) batch_down_kernel(BatchArgs a) {
    static_assert(TT == 16 || TT == 32, "tile entries");
    constexpr int NB = TT / 16;              // MFMA row blocks per tile
    constexpr int CK = KGI < 16 ? KGI : (NB > 1 || code_planes(F) > 1 || row_pack(F) > 1 ? 8 : 16);
    constexpr int NST = KGI / CK;
    constexpr int PART = CK * 64 * NB;       // staging elements of one part
    // parts of h staged: int4 takes h as one fp16 value (the weight
    // fragments are fp16(code x scale) already); the exact-fragment codecs
    // take hi and lo
    constexpr int NPARTS = F == kCodecInt4 ? 1 : 2;
    constexpr int PT = (NPARTS * PART + kDownThreads - 1) / kDownThreads;  // per thread
    static_assert(CK % 4 == 0 && KGI % CK == 0 && PT >= 1, "down stage shape");
    __shared__ u32x4 hs[2][NPARTS * PART];   // [part * PART + (g * 4 + q) * TT + token]
    __shared__ int s_kh[2][TT];              // the entries' h exponents, by item parity
    const int tid = threadIdx.x, lane = tid & 63, wv = wave_in_block();
    const int i = lane & 15, q = lane >> 4;
    const int n_tiles = a.n_tiles[0];
    constexpr int RP = row_pack(F);
    const int rblocks = a.H / (kDownBlockRows * RP);
    const int items = n_tiles * rblocks;
    const BlobLayout L = blob_layout(a.H, a.I, F);
    const int row_bytes = a.I / 2;
    const MagicExp mg = magic_exponents();
    int gs = 0;
    for (int ik = 0, item = grouped_item(blockIdx.x, gridDim.x, 0, items); item < items;
         item = grouped_item(blockIdx.x, gridDim.x, ++ik, items)) {
        const int tile = item / rblocks, rb = item - tile * rblocks;
        const Tile td = a.tiles[tile];
        const uint8_t* blob = td.expert < a.E ? a.table[td.expert] : a.shared_blob;
        const int row = rb * kDownBlockRows + wv * 16 + i;
        const uint8_t* dq = blob + L.down_q + (size_t)row * row_bytes;
        const uint8_t* dql = blob + L.down_lo + (size_t)row * row_bytes;  // int8 low plane
        const uint8_t* dsc = blob + L.down_s;
        const uint8_t* dsc2 = blob + L.down_s2;  // int2 odd rows
        const int sm = tid & (TT - 1);
        const bool has = sm < td.count;
        const size_t src = (size_t)(td.first_pair + sm) * a.I;
        // the entries' h scaling exponents for the stores after the last
        // step: thread tt < TT loads entry tt's now (every thread loads; an
        // entry past the count takes the last entry's) and writes it to LDS
        // half-way through the item (before a stage barrier), so the stores
        // wait on no load
        const int ib = ik & 1;
        int khr = a.kh[td.first_pair + (sm < td.count ? sm : td.count - 1)];
        f32x4 acc[RP][NB];
#pragma unroll
        for (int h = 0; h < RP; ++h)
#pragma unroll
            for (int z = 0; z < NB; ++z) acc[h][z] = f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        constexpr int NS = KGI / 4;  // steps of 4 groups
        constexpr int P = code_planes(F);
        constexpr int NSP = NS * P;  // (step, plane) loads, plane fastest
        // codes of plane pl and the scales of step s for load k = (s, pl)
        // (both planes of a step share its scales)
        // (int4 keeps each lane's own group, 4s + q, and needs its scale only)
        const uint16_t* dsc_q = reinterpret_cast<const uint16_t*>(dsc) + scale_index(row, q, KGI, a.down_p);
        auto load_step = [&](int k, u32x4& c, u32x4& sc) {
            const int s = k / P, pl = k - s * P;
            c = *as_global<u32x4>((pl ? dql : dq) + (4 * s + q) * 16);
            if constexpr (F == kCodecInt4) {
                // within a row the scale of group g + 1 lies down_p halves
                // after that of group g
                sc[0] = *as_global<uint16_t>(dsc_q + (size_t)4 * s * a.down_p);
                return;
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const size_t si = scale_index(row, 4 * s + m, KGI, a.down_p);
                if constexpr (F == kCodecMxfp4)
                    sc[m] = *as_global<uint8_t>(dsc + si);
                else if constexpr (RP > 1)
                    sc[m] = (unsigned)*as_global<uint16_t>(reinterpret_cast<const uint16_t*>(dsc) + si) |
                            ((unsigned)*as_global<uint16_t>(reinterpret_cast<const uint16_t*>(dsc2) + si) << 16);
                else
                    sc[m] = *as_global<uint16_t>(reinterpret_cast<const uint16_t*>(dsc) + si);
            }
        };
        auto stage_load = [&](int st, u32x4 (&v)[PT]) {
#pragma unroll
            for (int r = 0; r < PT; ++r) {
                const int e = tid + kDownThreads * r;
                if (e >= NPARTS * PART) break;
                const int part = e / PART, rest = e - part * PART;
                const uint16_t* base = part ? a.ha_lo : a.ha_hi;
                v[r] = has ? *as_global<u32x4>(base + src + (size_t)((st * CK + rest / (4 * TT)) * 4 +
                                                                 (rest / TT) % 4) * 8)
                           : u32x4{0u, 0u, 0u, 0u};
            }
        };
        u32x4 v[PT];
        stage_load(0, v);
        u32x4 cd0, sc0, cd1 = {0u, 0u, 0u, 0u}, sc1 = cd1;
        load_step(0, cd0, sc0);
        if (NSP > 1) load_step(1, cd1, sc1);
#pragma unroll
        for (int st = 0; st < NST; ++st, ++gs) {
            if (st == NST / 2 && tid < TT) s_kh[ib][tid] = khr;
            const int buf = gs & 1;
#pragma unroll
            for (int r = 0; r < PT; ++r)
                if (tid + kDownThreads * r < NPARTS * PART) hs[buf][tid + kDownThreads * r] = v[r];
            __syncthreads();
            if (st + 1 < NST) stage_load(st + 1, v);
#pragma unroll
            for (int c = 0; c < CK / 4; ++c) {
                const int sidx = st * (CK / 4) + c;
#pragma unroll
                for (int pl = 0; pl < P; ++pl) {
                    const int k = sidx * P + pl;
                    u32x4 cd2 = cd1, sc2 = sc1;
                    if (k + 2 < NSP) load_step(k + 2, cd2, sc2);
                    if constexpr (F == kCodecInt4) {
                        // int4: fp16(code x scale) fragments, as in gate/up
                        // (lane (i, q) keeps group 4s + q, MFMA d takes its
                        // dword d), against h as one fp16 value
                        const unsigned sv = sc0[0];
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            const f16x8 bw = codes_to_f16x8(cd0[d], mg) * splat_h8(sv);
#pragma unroll
                            for (int z = 0; z < NB; ++z) {
                                const int slot = ((4 * c + q) * 4 + d) * TT + 16 * z + i;
                                const f16x8 ah = __builtin_bit_cast(f16x8, hs[buf][slot]);
                                acc[0][z] = mfma16(ah, bw, acc[0][z]);
                            }
                        }
                    } else {
                    transpose_quarters(cd0);
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
#pragma unroll
                        for (int h = 0; h < RP; ++h) {
                            const f16x8 bw = dequant_f16x8<F>(cd0[m], mg, pl, h);
                            const float s = scale16<F>(sc0[m] >> (16 * h));
#pragma unroll
                            for (int z = 0; z < NB; ++z) {
                                const int slot = ((4 * c + m) * 4 + q) * TT + 16 * z + i;
                                const f16x8 ah = __builtin_bit_cast(f16x8, hs[buf][slot]);
                                const f16x8 al = __builtin_bit_cast(f16x8, hs[buf][PART + slot]);
                                const f32x4 d = mfma16(al, bw, mfma16(ah, bw, zero));
#pragma unroll
                                for (int j = 0; j < 4; ++j) acc[h][z][j] = fmaf(s, d[j], acc[h][z][j]);
                                asm volatile("" : "+v"(acc[h][z]));
                                __builtin_amdgcn_sched_barrier(0);
                            }
                        }
                    }
                    }
                    cd0 = cd1;
                    sc0 = sc1;
                    cd1 = cd2;
                    sc1 = sc2;
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
#pragma unroll
        for (int z = 0; z < NB; ++z)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tt = 16 * z + 4 * q + j;
                if (tt < td.count) {
                    const int p = td.first_pair + tt;
#pragma unroll
                    for (int h = 0; h < RP; ++h)
                        a.d[(size_t)p * a.H + RP * row + h] = ldexpf(acc[h][z][j], -s_kh[ib][tt]);
                }
            }
    }
}

// ---------------------------------------------------------------- combine
__global__ void __launch_bounds__(256) batch_combine_kernel(BatchArgs a) {
    const int t = blockIdx.x;
    const int r = blockIdx.y * 1024 + threadIdx.x * 4;
    if (r >= a.H) return;
    float wj[8];
    const float* dj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int pr = j < a.K ? a.inv[(size_t)t * a.K + j] : -1;  // -1: dropped by top-p
        wj[j] = pr >= 0 ? a.w[(size_t)t * a.K + j] : 0.0f;
        dj[j] = pr >= 0 ? a.d + (size_t)pr * a.H : nullptr;
    }
    const float* dsh = a.S > 0 ? a.d + (size_t)(a.T * a.K + t) * a.H : nullptr;
    {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (dj[j]) {
                const f32x4 v = *as_global<f32x4>(dj[j] + r);
#pragma unroll
                for (int z = 0; z < 4; ++z) acc[z] = fmaf(wj[j], v[z], acc[z]);
            }
        }
        if (dsh) {
            const f32x4 v = *as_global<f32x4>(dsh + r);
#pragma unroll
            for (int z = 0; z < 4; ++z) acc[z] += v[z];
        }
        *reinterpret_cast<f32x4*>(a.y + (size_t)t * a.H + r) = acc;
    }
}

// ---------------------------------------------------------------- launchers
constexpr int kGroupedGrid = 512;  // 2 workgroups of 8 waves per CU

template <int EPL>
hipError_t launch_topk(const BatchArgs& a, bool convert, hipStream_t st) {
    const dim3 grid((a.T + 3) / 4, convert ? 2 : 1);
    switch ((a.H / 32 + kWave - 1) / kWave) {
        case 1: hipLaunchKernelGGL((batch_topk_kernel<EPL, 1>), grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL((batch_topk_kernel<EPL, 2>), grid, dim3(256), 0, st, a); break;
        case 3: hipLaunchKernelGGL((batch_topk_kernel<EPL, 3>), grid, dim3(256), 0, st, a); break;
        case 4: hipLaunchKernelGGL((batch_topk_kernel<EPL, 4>), grid, dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// With timing events the launch goes through hipExtLaunchKernelGGL, which
// stamps them with the kernel's own start and end.
template <typename K>
hipError_t launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t st, const LaunchTiming& tm, const BatchArgs& a) {
    if (tm.start)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, tm.start, tm.stop, 0, a);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, st, a);
    return hipGetLastError();
}

int grouped_grid(const BatchArgs& a, int rblocks) {
    const long items = (long)batch_max_tiles(a.T, a.K, a.E, a.S) * rblocks;
    return (int)(items < kGroupedGrid ? items : kGroupedGrid);
}

template <int KG, int TT>
hipError_t launch_gateup_t(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm) {
    if constexpr (TT == 32) {
        if (a.I % (16 * 16 * row_pack(a.codec)) == 0) {
            // 16 waves over 256 rows, one workgroup per CU
            const int g = grouped_grid(a, a.I / (16 * 16 * row_pack(a.codec)));
            const dim3 grid(g < kGroupedGrid / 2 ? g : kGroupedGrid / 2);
            if (a.codec == kCodecMxfp4)
                return launch_timed(batch_gateup_kernel<KG, kCodecMxfp4, TT, 16>, grid, dim3(1024), st, tm, a);
            if (a.codec == kCodecInt4)
                return launch_timed(batch_gateup_kernel<KG, kCodecInt4, TT, 16>, grid, dim3(1024), st, tm, a);
            return hipErrorInvalidValue;
        }
    }
    const dim3 grid(grouped_grid(a, a.I / (kBlockRows * row_pack(a.codec))));
    if (a.codec == kCodecMxfp4) return launch_timed(batch_gateup_kernel<KG, kCodecMxfp4, TT, 8>, grid, dim3(512), st, tm, a);
    if (a.codec == kCodecInt4) return launch_timed(batch_gateup_kernel<KG, kCodecInt4, TT, 8>, grid, dim3(512), st, tm, a);
    if (TT == 16 && a.codec == kCodecInt8)
        return launch_timed(batch_gateup_kernel<KG, kCodecInt8, 16, 8>, grid, dim3(512), st, tm, a);
    if (TT == 16 && a.codec == kCodecInt2)
        return launch_timed(batch_gateup_kernel<KG, kCodecInt2, 16, 8>, grid, dim3(512), st, tm, a);
    return hipErrorInvalidValue;
}

template <int KG>
hipError_t launch_gateup(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm) {
    if (a.tile_tokens == 32) return launch_gateup_t<KG, 32>(a, st, tm);
    if (a.tile_tokens == 16) return launch_gateup_t<KG, 16>(a, st, tm);
    return hipErrorInvalidValue;
}

template <int KGI, int TT>
hipError_t launch_down_t(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm) {
    const int g = grouped_grid(a, a.H / (kDownBlockRows * row_pack(a.codec)));
    const dim3 grid(g < kGroupedGrid / 2 ? g : kGroupedGrid / 2);  // one workgroup per CU
    const dim3 block(kDownThreads);
    if (a.codec == kCodecMxfp4) return launch_timed(batch_down_kernel<KGI, kCodecMxfp4, TT>, grid, block, st, tm, a);
    if (a.codec == kCodecInt4) return launch_timed(batch_down_kernel<KGI, kCodecInt4, TT>, grid, block, st, tm, a);
    if (TT == 16 && a.codec == kCodecInt8)
        return launch_timed(batch_down_kernel<KGI, kCodecInt8, 16>, grid, block, st, tm, a);
    if (TT == 16 && a.codec == kCodecInt2)
        return launch_timed(batch_down_kernel<KGI, kCodecInt2, 16>, grid, block, st, tm, a);
    return hipErrorInvalidValue;
}

template <int KGI>
hipError_t launch_down(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm) {
    if (a.tile_tokens == 32) return launch_down_t<KGI, 32>(a, st, tm);
    if (a.tile_tokens == 16) return launch_down_t<KGI, 16>(a, st, tm);
    return hipErrorInvalidValue;
}

}  // namespace

namespace {
template <int NS>
hipError_t launch_router_ns(const BatchArgs& a, int neb, hipStream_t st) {
    const dim3 grid(a.E / (16 * neb), a.router_splits, (a.T + 63) / 64);
    if (neb == 4) hipLaunchKernelGGL((batch_router_kernel<4, NS>), grid, dim3(256), 0, st, a);
    else if (neb == 2) hipLaunchKernelGGL((batch_router_kernel<2, NS>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((batch_router_kernel<1, NS>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}
}  // namespace

hipError_t batch_router(const BatchArgs& a, hipStream_t st) {
    if (a.E % 16 || a.router_splits < 1 || a.H % (64 * a.router_splits)) return hipErrorInvalidValue;
    // expert blocks of 16 per wave: 4 (64-expert tiles) where they divide E
    const int neb = a.E % 64 == 0 ? 4 : (a.E % 32 == 0 ? 2 : 1);
    switch (a.H / a.router_splits / 16) {
        case 4: return launch_router_ns<4>(a, neb, st);
        case 8: return launch_router_ns<8>(a, neb, st);
        case 16: return launch_router_ns<16>(a, neb, st);
        case 24: return launch_router_ns<24>(a, neb, st);
        case 32: return launch_router_ns<32>(a, neb, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t batch_topk(const BatchArgs& a, bool convert, hipStream_t st) {
    if (a.E <= 64) return launch_topk<1>(a, convert, st);
    if (a.E <= 128) return launch_topk<2>(a, convert, st);
    return launch_topk<4>(a, convert, st);
}

hipError_t batch_dispatch(const BatchArgs& a, hipStream_t st) {
    if (a.T * a.K > kMaxDispatchEntries || a.E > 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL(batch_dispatch_kernel, dim3(1), dim3(64 * kDispatchWaves), 0, st, a);
    return hipGetLastError();
}

hipError_t batch_gateup(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm) {
    switch (a.H / 32) {
        case 8: return launch_gateup<8>(a, st, tm);
        case 16: return launch_gateup<16>(a, st, tm);
        case 32: return launch_gateup<32>(a, st, tm);
        case 64: return launch_gateup<64>(a, st, tm);
        case 128: return launch_gateup<128>(a, st, tm);
        case 192: return launch_gateup<192>(a, st, tm);
        case 256: return launch_gateup<256>(a, st, tm);
        default: return hipErrorInvalidValue;
    }
}

hipError_t batch_hprep(const BatchArgs& a, hipStream_t st) {
    const int pairs = a.T * (a.K + a.S);
    if ((a.I / 32) * 4 <= 256)
        hipLaunchKernelGGL((batch_hprep_kernel<1>), dim3(pairs), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((batch_hprep_kernel<2>), dim3(pairs), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t batch_down(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm) {
    switch (a.I / 32) {
        case 4: return launch_down<4>(a, st, tm);
        case 8: return launch_down<8>(a, st, tm);
        case 16: return launch_down<16>(a, st, tm);
        case 32: return launch_down<32>(a, st, tm);
        case 64: return launch_down<64>(a, st, tm);
        case 128: return launch_down<128>(a, st, tm);
        default: return hipErrorInvalidValue;
    }
}

// The expert table of a launch sequence whose blobs sit in cache slots: the
// pointers travel as the kernel's argument (no host staging to keep alive).
__global__ void __launch_bounds__(256) batch_table_kernel(ExpertTable t, int n, const uint8_t** table) {
    const int i = threadIdx.x;
    if (i < n) table[i] = t.p[i];
}

hipError_t batch_set_table(const ExpertTable& t, int n, const uint8_t** table, hipStream_t st) {
    if (n < 0 || n > 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL(batch_table_kernel, dim3(1), dim3(256), 0, st, t, n, table);
    return hipGetLastError();
}

hipError_t batch_combine(const BatchArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(batch_combine_kernel, dim3(a.T, (a.H + 1023) / 1024), dim3(256), 0, st, a);
    return hipGetLastError();
}

bool batch_shape_supported(int hidden, int inter) {
    return hidden % 256 == 0 && inter % kBlockRows == 0 && hidden / 32 <= 256 && inter / 32 <= 128;
}

bool batch_codec_supported(int codec, int hidden, int inter) {
    const int rp = row_pack(codec);
    return batch_shape_supported(hidden, inter) && hidden % (kDownBlockRows * rp) == 0 &&
           inter % (kBlockRows * rp) == 0;
}

}  // namespace moe
