// Device helpers shared by the decode and the batched kernels: vector
// types, global-address-space loads, DPP / permlane wave reductions, the
// activation range exponent and the wave-level group-limited top-k.
// Everything sits in an unnamed namespace, so each kernel file gets its own
// inlined copy.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

__device__ __forceinline__ f16x2 as_h2(unsigned u) { return __builtin_bit_cast(f16x2, u); }

// Weight and scale pointers reach the kernels through integers (blob
// tables, lane reads), which loses their address space; casting them to the
// global address space keeps the loads global_load rather than flat_load.
// Flat loads count against both the vector-memory and the LDS counters, so
// the compiler must drain every outstanding load before using any of them,
// which would serialise load pipelining.
#define MOE_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const MOE_GLOBAL T* as_global(const void* p) {
    return (const MOE_GLOBAL T*)(p);
}

__device__ __forceinline__ u32x4 load_stream16(const uint8_t* p) {
    return __builtin_nontemporal_load(as_global<u32x4>(p));
}

// E8M0 byte b -> 2^(b - 127) (b = 0 is the subnormal 2^-127; the packer
// refuses 255).
__device__ __forceinline__ float e8m0_to_float(unsigned b) {
    return __builtin_bit_cast(float, b ? b << 23 : 0x00400000u);
}

__device__ __forceinline__ float half_bits_to_float(unsigned bits16) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)bits16);
}

// DPP lane permutations inside rows of 16 lanes.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within 16

template <int CTRL>
__device__ __forceinline__ unsigned dpp_u(unsigned v) {
    return (unsigned)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, dpp_u<CTRL>(__builtin_bit_cast(unsigned, v)));
}
__device__ __forceinline__ unsigned umax(unsigned a, unsigned b) { return a > b ? a : b; }
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Value of the partner lane (lane index with bit BIT flipped, or for bits
// below 4 the lane mirrored inside its group of 2^(BIT+1), which also flips
// BIT) taken from `send`: permlane swaps across the halves and 16-lane rows
// of the wave, DPP inside a row.  No LDS traffic.
template <int BIT>
__device__ __forceinline__ float partner_value(float send, int lane) {
    const unsigned u = __builtin_bit_cast(unsigned, send);
    if constexpr (BIT == 5) {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return __builtin_bit_cast(float, (lane & 32) ? r[0] : r[1]);
    } else if constexpr (BIT == 4) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return __builtin_bit_cast(float, (lane & 16) ? r[0] : r[1]);
    } else if constexpr (BIT == 3) {
        return dpp_f<kDppMirror>(send);
    } else if constexpr (BIT == 2) {
        return dpp_f<kDppHalfMirror>(send);
    } else if constexpr (BIT == 1) {
        return dpp_f<kDppXor2>(send);
    } else {
        return dpp_f<kDppXor1>(send);
    }
}

// Sum of NV per-lane values over the lanes that differ only in bits [0, B),
// scattered: on return the lane holds the total of value index
// vi = (lane >> (B - log2 NV)) & (NV - 1), identical in the 2^(B - log2 NV)
// lanes of its set.  Each scatter step halves the values a lane keeps (the
// half selected by the step's lane bit) and adds the partner's copy of
// them; the remaining bits are summed whole.  Fixed order: deterministic.
template <int NV, int B, int S = 0>
__device__ __forceinline__ void scatter_steps(float (&v)[NV], int lane) {
    if constexpr ((NV >> S) > 1) {
        constexpr int half = (NV >> S) / 2;
        constexpr int BIT = B - 1 - S;
        const bool upper = (lane >> BIT) & 1;
#pragma unroll
        for (int t = 0; t < half; ++t) {
            const float keep = upper ? v[half + t] : v[t];
            const float send = upper ? v[t] : v[half + t];
            v[t] = keep + partner_value<BIT>(send, lane);
        }
        scatter_steps<NV, B, S + 1>(v, lane);
    }
}
template <int BIT>
__device__ __forceinline__ float sum_bits_below(float r, int lane) {
    if constexpr (BIT >= 0) {
        r += partner_value<BIT>(r, lane);
        return sum_bits_below<BIT - 1>(r, lane);
    } else {
        return r;
    }
}
template <int NV, int B>
__device__ __forceinline__ float reduce_scatter(float (&v)[NV], int lane) {
    static_assert((NV & (NV - 1)) == 0 && ilog2(NV) <= B && B <= 6, "bad reduce shape");
    scatter_steps<NV, B>(v, lane);
    return sum_bits_below<B - 1 - ilog2(NV)>(v[0], lane);
}

// Maximum over the wave, returned uniform (DPP inside rows, then the four
// row results read as scalars).
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
    v = umax(v, dpp_u<kDppXor1>(v));
    v = umax(v, dpp_u<kDppXor2>(v));
    v = umax(v, dpp_u<kDppHalfMirror>(v));
    v = umax(v, dpp_u<kDppMirror>(v));
    const unsigned a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const unsigned c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return umax(umax(a, b), umax(c, d));
}

// DPP move whose result the compiler folds into the consuming VALU op.
template <int CTRL>
__device__ __forceinline__ unsigned dpp_mov(unsigned v) {
    return (unsigned)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Maximum over the wave, in every lane: within 16-lane rows by DPP, across
// rows by the permlane swaps (no scalar round trip).
__device__ __forceinline__ unsigned wave_max_all(unsigned v) {
    v = umax(v, dpp_mov<kDppXor1>(v));
    v = umax(v, dpp_mov<kDppXor2>(v));
    v = umax(v, dpp_mov<kDppHalfMirror>(v));
    v = umax(v, dpp_mov<kDppMirror>(v));
    const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = umax(r32[0], r32[1]);
    const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return umax(r16[0], r16[1]);
}

// Sum over the wave in a fixed order, returned uniform.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// Power-of-two exponent k such that max_abs * 2^k lies in [2^13, 2^14),
// from the biased binary exponent of max_abs (shared by fp32 and bf16).
// Zero, subnormal or non-finite maxima give k = 0.
__device__ __forceinline__ int range_exponent(unsigned biased_exp) {
    if (biased_exp == 0 || biased_exp >= 255) return 0;
    int k = 140 - (int)biased_exp;
    return k > 100 ? 100 : (k < -100 ? -100 : k);
}

// Index of the calling wave inside its workgroup, as a wave-uniform value
// (scalar register): item and slot arithmetic derived from it then stays on
// the scalar unit instead of occupying vector registers.
__device__ __forceinline__ int wave_in_block() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ const uint8_t* readlane_ptr(const uint8_t* p, int src) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const unsigned lo = __builtin_amdgcn_readlane((unsigned)v, src);
    const unsigned hi = __builtin_amdgcn_readlane((unsigned)(v >> 32), src);
    return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// Pointer held by lane src, per lane (src may differ between lanes).
__device__ __forceinline__ const uint8_t* shfl_ptr(const uint8_t* p, int src) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const unsigned lo = __shfl((unsigned)v, src);
    const unsigned hi = __shfl((unsigned)(v >> 32), src);
    return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// Per-lane copy of a 16-entry kernel-argument array without dynamic
// indexing: lane j < 16 receives p[j].
__device__ __forceinline__ const uint8_t* lane_pick(const uint8_t* const (&p)[16], int lane) {
    const uint8_t* r = nullptr;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (lane == j) r = p[j];
    return r;
}

// ---------------------------------------------------------------- top-k
// Merge of two (largest, second largest) pairs.
__device__ __forceinline__ void top2_merge(float& a1, float& a2, float b1, float b2) {
    const float n1 = fmaxf(a1, b1);
    const float n2 = a1 >= b1 ? fmaxf(a2, b1) : fmaxf(a1, b2);
    a1 = n1;
    a2 = n2;
}

// Group-limited top-k of one token on one wave (every lane must call it).
// Lane l holds experts l*EPL .. l*EPL+EPL-1.  On return lane j < K holds
// the j-th choice (sb descending, ties to the lower index) in *my_id and its
// weight rsf * s_j / sum_chosen s in *my_w.
template <int EPL>
__device__ void wave_group_topk_values(const float (&s)[EPL], const float (&key)[EPL], int E, int G, int TG, int K,
                                       float rsf, float top_p, int lane, int* my_id, float* my_w) {
    const float NEG = -__builtin_inff();
    // Group score: the two largest biased scores of the group.
    const int lpg = (E / G) / EPL;  // lanes per group (power of two)
    float a1 = NEG, a2 = NEG;
#pragma unroll
    for (int i = 0; i < EPL; ++i) top2_merge(a1, a2, key[i], NEG);
    if (lpg > 1) top2_merge(a1, a2, dpp_f<kDppXor1>(a1), dpp_f<kDppXor1>(a2));
    if (lpg > 2) top2_merge(a1, a2, dpp_f<kDppXor2>(a1), dpp_f<kDppXor2>(a2));
    if (lpg > 4) top2_merge(a1, a2, dpp_f<kDppHalfMirror>(a1), dpp_f<kDppHalfMirror>(a2));
    if (lpg > 8) top2_merge(a1, a2, dpp_f<kDppMirror>(a1), dpp_f<kDppMirror>(a2));
    for (int o = 16; o < lpg; o <<= 1) top2_merge(a1, a2, __shfl_xor(a1, o), __shfl_xor(a2, o));
    const float gscore = a1 + a2;
    const int my_group = lane / lpg;
    int rank = 0;
    for (int g = 0; g < G; ++g) {
        const float o = readlane_f(gscore, g * lpg);
        rank += (o > gscore || (o == gscore && g < my_group)) ? 1 : 0;
    }
    const bool eligible = rank < TG;
    // The lane's candidates as order-preserving unsigned keys (larger float
    // -> larger key; 0 = not eligible or taken), sorted descending with ties
    // to the lower expert index; each step takes the wave maximum of the
    // lanes' heads, the lowest lane holding it wins (lanes own increasing
    // index ranges), and the winner shifts its list.
    unsigned u[EPL];
    int ei[EPL];
    float sv[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        unsigned v = __builtin_bit_cast(unsigned, key[i]);
        v = (v & 0x80000000u) ? ~v : (v | 0x80000000u);
        u[i] = eligible && e < E ? v : 0u;
        ei[i] = e;
        sv[i] = s[i];
    }
    auto order = [&](int p, int q) {
        const bool swap = u[q] > u[p] || (u[q] == u[p] && ei[q] < ei[p]);
        const unsigned tu = u[p];
        const int te = ei[p];
        const float ts = sv[p];
        u[p] = swap ? u[q] : u[p];
        ei[p] = swap ? ei[q] : ei[p];
        sv[p] = swap ? sv[q] : sv[p];
        u[q] = swap ? tu : u[q];
        ei[q] = swap ? te : ei[q];
        sv[q] = swap ? ts : sv[q];
    };
    if constexpr (EPL == 2) {
        order(0, 1);
    } else if constexpr (EPL == 4) {
        order(0, 1);
        order(2, 3);
        order(0, 2);
        order(1, 3);
        order(1, 2);
    }
    static_assert(EPL == 1 || EPL == 2 || EPL == 4, "experts per lane");
    float sum_s = 0.0f, mine_s = 0.0f;
    int mine_e = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j < K) {
            const unsigned mx = wave_max_all(u[0]);
            const int wl = __ffsll((long long)__ballot(u[0] == mx)) - 1;
            const int we = __builtin_amdgcn_readlane(ei[0], wl);
            const float se = readlane_f(sv[0], wl);
            if (lane == wl) {
#pragma unroll
                for (int i = 0; i + 1 < EPL; ++i) {
                    u[i] = u[i + 1];
                    ei[i] = ei[i + 1];
                    sv[i] = sv[i + 1];
                }
                u[EPL - 1] = 0u;
            }
            if (lane == j) {
                mine_e = we;
                mine_s = se;
            }
            sum_s += se;
        }
    }
    float denom = sum_s;
    bool keep = true;
    if (top_p < 1.0f) {
        // Adaptive top-p over the chosen experts: a choice is kept when the
        // shares s / sum_s of the choices ranked above it (larger s, ties to
        // the lower index) add up to less than top_p, tested as
        // sum of those s < top_p * sum_s; the kept weights are renormalised
        // over the kept s and a dropped choice gets id -1.
        float before = 0.0f;
        bool first = true;  // the top-ranked choice is always kept
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < K) {
                const float sj = readlane_f(mine_s, j);
                const int ej = __builtin_amdgcn_readlane(mine_e, j);
                if (sj > mine_s || (sj == mine_s && ej < mine_e)) {
                    before += sj;
                    first = false;
                }
            }
        }
        keep = lane < K && (first || before < top_p * sum_s);
        const unsigned long long km = __ballot(keep);
        float kept_s = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < K && ((km >> j) & 1ull)) kept_s += readlane_f(mine_s, j);
        denom = kept_s;
    }
    *my_id = keep ? mine_e : -1;
    *my_w = keep ? rsf * mine_s / denom : 0.0f;
}

}  // namespace
}  // namespace moe
