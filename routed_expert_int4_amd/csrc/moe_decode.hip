// Decode (one token per call) kernels of the routed int4 MoE layer, gfx950.
//
// Three launches per token, each streaming its weights from HBM once:
//   1. router_shared: router logits (one fp32 row of W_r per wave) and, in
//      the same grid, the shared expert's gate/up + SwiGLU (it does not depend
//      on the routing).  The last router workgroup to finish (atomic ticket)
//      runs the group-limited top-k on one wave.
//   2. gateup: gate/up + SwiGLU of the top_k routed experts.
//   3. down_combine: down projection of every selected expert and of the
//      shared expert for a block of output rows, and the weighted combine in
//      a fixed order (no float atomics: repeated calls are bit-identical).
//
// Int4 GEMV scheme.  A lane owns one 32-input scale group of the reduction
// dimension (several when a row has more than 64 groups) and keeps the
// matching activations in registers as fp16 pairs; every wave load is 64
// lanes x 16 contiguous bytes.  A 16-byte chunk holds the 32 codes of one
// group; each code (stored q+8) is OR-ed into the mantissa of an fp16
// constant (1024+u or 64+u) and the constant minus 8 is subtracted, which
// yields q exactly as fp16; v_dot2_f32_f16 then accumulates q*x pairs in
// fp32.  The fp16 scale is applied once per chunk in fp32.  Partial sums of
// the rows a wave visited are reduced across lanes with a reduce-scatter.
// Activations are scaled by a power of two before the fp16 conversion so
// that any finite bf16 input keeps 11 significant bits; the intermediate h
// of the down projection is split into fp16 hi + lo parts (about 22 bits).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_kernels.h"
#include "moe_layout.h"

namespace moe {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

__device__ __forceinline__ f16x2 as_h2(unsigned u) { return __builtin_bit_cast(f16x2, u); }

__device__ __forceinline__ u32x4 load_stream16(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float half_bits_to_float(unsigned bits16) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)bits16);
}

// 32 offset-binary codes (public nibble order: column 8d+j at bits 4j of
// dword d) dotted with activations arranged per dword d as the pairs
// (x0,x4), (x1,x5), (x2,x6), (x3,x7) of columns 8d..8d+7.
__device__ __forceinline__ float dot_chunk(u32x4 c, const f16x2* xp, float acc) {
    const f16x2 k_lo = {(_Float16)1032.0f, (_Float16)1032.0f};  // 1024 + 8
    const f16x2 k_hi = {(_Float16)72.0f, (_Float16)72.0f};      // 64 + 8
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const unsigned w = c[d];
        const unsigned w8 = w >> 8;
        const f16x2 q0 = as_h2((w & 0x000F000Fu) | 0x64006400u) - k_lo;
        const f16x2 q1 = as_h2((w & 0x00F000F0u) | 0x54005400u) - k_hi;
        const f16x2 q2 = as_h2((w8 & 0x000F000Fu) | 0x64006400u) - k_lo;
        const f16x2 q3 = as_h2((w8 & 0x00F000F0u) | 0x54005400u) - k_hi;
        acc = __builtin_amdgcn_fdot2(q0, xp[4 * d + 0], acc, false);
        acc = __builtin_amdgcn_fdot2(q1, xp[4 * d + 1], acc, false);
        acc = __builtin_amdgcn_fdot2(q2, xp[4 * d + 2], acc, false);
        acc = __builtin_amdgcn_fdot2(q3, xp[4 * d + 3], acc, false);
    }
    return acc;
}

// As dot_chunk with the activation given as hi + lo fp16 parts.
__device__ __forceinline__ float dot_chunk_hilo(u32x4 c, const f16x2* hp, const f16x2* lp, float acc) {
    const f16x2 k_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
    const f16x2 k_hi = {(_Float16)72.0f, (_Float16)72.0f};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const unsigned w = c[d];
        const unsigned w8 = w >> 8;
        const f16x2 q0 = as_h2((w & 0x000F000Fu) | 0x64006400u) - k_lo;
        const f16x2 q1 = as_h2((w & 0x00F000F0u) | 0x54005400u) - k_hi;
        const f16x2 q2 = as_h2((w8 & 0x000F000Fu) | 0x64006400u) - k_lo;
        const f16x2 q3 = as_h2((w8 & 0x00F000F0u) | 0x54005400u) - k_hi;
        acc = __builtin_amdgcn_fdot2(q0, hp[4 * d + 0], acc, false);
        acc = __builtin_amdgcn_fdot2(q0, lp[4 * d + 0], acc, false);
        acc = __builtin_amdgcn_fdot2(q1, hp[4 * d + 1], acc, false);
        acc = __builtin_amdgcn_fdot2(q1, lp[4 * d + 1], acc, false);
        acc = __builtin_amdgcn_fdot2(q2, hp[4 * d + 2], acc, false);
        acc = __builtin_amdgcn_fdot2(q2, lp[4 * d + 2], acc, false);
        acc = __builtin_amdgcn_fdot2(q3, hp[4 * d + 3], acc, false);
        acc = __builtin_amdgcn_fdot2(q3, lp[4 * d + 3], acc, false);
    }
    return acc;
}

// Sum of NV per-lane values over the lanes that differ only in bits [0, B),
// scattered: on return the lane holds the total of value index
// vi = (lane >> (B - log2 NV)) & (NV - 1), identical in the 2^(B - log2 NV)
// lanes of its set.  Fixed order: deterministic.
template <int NV, int B>
__device__ __forceinline__ float reduce_scatter(float (&v)[NV], int lane) {
    static_assert((NV & (NV - 1)) == 0 && ilog2(NV) <= B, "bad reduce shape");
#pragma unroll
    for (int s = 0; (NV >> s) > 1; ++s) {
        const int m = NV >> s;
        const int half = m / 2;
        const int bit = B - 1 - s;
        const bool upper = (lane >> bit) & 1;
#pragma unroll
        for (int t = 0; t < half; ++t) {
            const float keep = upper ? v[half + t] : v[t];
            const float send = upper ? v[t] : v[half + t];
            v[t] = keep + __shfl_xor(send, 1 << bit);
        }
    }
    float r = v[0];
#pragma unroll
    for (int bit = B - 1 - ilog2(NV); bit >= 0; --bit) r += __shfl_xor(r, 1 << bit);
    return r;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const unsigned t = (unsigned)__shfl_xor((int)v, o);
        v = t > v ? t : v;
    }
    return v;
}

// Power-of-two exponent k such that max_abs * 2^k lies in [2^13, 2^14),
// from the biased binary exponent of max_abs (shared by fp32 and bf16).
// Zero, subnormal or non-finite maxima give k = 0.
__device__ __forceinline__ int range_exponent(unsigned biased_exp) {
    if (biased_exp == 0 || biased_exp >= 255) return 0;
    int k = 140 - (int)biased_exp;
    return k > 100 ? 100 : (k < -100 ? -100 : k);
}

// ---------------------------------------------------------------- top-k
// Group-limited top-k of one token on one wave.  Lane l holds experts
// l*EPL .. l*EPL+EPL-1.  Writes ids[k] (sb descending, ties to the lower
// index) and w[k] = rsf * s / sum s.
template <int EPL>
__device__ void wave_group_topk(const float* __restrict__ logits, const float* __restrict__ bias, int E, int G,
                                int TG, int K, float rsf, int32_t* __restrict__ ids_out,
                                float* __restrict__ w_out, int lane) {
    float s[EPL], key[EPL];
    const float NEG = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        if (e < E) {
            const float l = logits[e];
            s[i] = 1.0f / (1.0f + expf(-l));
            key[i] = s[i] + bias[e];
        } else {
            s[i] = 0.0f;
            key[i] = NEG;
        }
    }
    // Group score: sum of the two largest biased scores of the group.
    const int gsize = E / G;
    const int lpg = gsize / EPL;  // lanes per group (power of two)
    float a1 = NEG, a2 = NEG;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        if (key[i] > a1) {
            a2 = a1;
            a1 = key[i];
        } else if (key[i] > a2) {
            a2 = key[i];
        }
    }
    for (int o = 1; o < lpg; o <<= 1) {
        const float b1 = __shfl_xor(a1, o), b2 = __shfl_xor(a2, o);
        const float n1 = fmaxf(a1, b1);
        const float n2 = a1 >= b1 ? fmaxf(a2, b1) : fmaxf(a1, b2);
        a1 = n1;
        a2 = n2;
    }
    const float gscore = a1 + a2;
    const int my_group = lane / lpg;
    int rank = 0;
    for (int g = 0; g < G; ++g) {
        const float o = __shfl(gscore, g * lpg);
        rank += (o > gscore || (o == gscore && g < my_group)) ? 1 : 0;
    }
    const bool eligible = (lane * EPL < E) && rank < TG;
    bool live[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) live[i] = eligible && (lane * EPL + i < E);

    float sum_s = 0.0f;
    float chosen_s[16];
    int chosen_e[16];
    for (int j = 0; j < K; ++j) {
        // lane-local best (lowest index among equals)
        float lb = NEG;
        int li = -1;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if (live[i] && (li < 0 || key[i] > lb)) {
                lb = key[i];
                li = i;
            }
        }
        // wave maximum of the lane bests
        unsigned ob = __builtin_bit_cast(unsigned, lb);
        // order-preserving map of floats to unsigned (larger float -> larger key)
        ob = (ob & 0x80000000u) ? ~ob : (ob | 0x80000000u);
        if (li < 0) ob = 0u;
        const unsigned mx = wave_max_u32(ob);
        const unsigned long long hit = __ballot(li >= 0 && ob == mx);
        const int wl = __ffsll((long long)hit) - 1;  // lowest lane holding the maximum
        const int wi = __shfl(li, wl);
        const int e = wl * EPL + wi;
        const float se = __shfl(li >= 0 ? s[li < 0 ? 0 : li] : 0.0f, wl);
        if (lane == wl) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == wi) live[i] = false;
        }
        chosen_e[j] = e;
        chosen_s[j] = se;
        sum_s += se;
    }
    if (lane == 0) {
        for (int j = 0; j < K; ++j) {
            ids_out[j] = chosen_e[j];
            w_out[j] = rsf * chosen_s[j] / sum_s;
        }
    }
}

// ---------------------------------------------------------------- gate/up
// Work items of the gate/up stage: (slot, block of R rows).  Each wave keeps
// the token's activations in registers and loops over items with a stride
// of the number of waves in the grid.
template <int KG>
struct GateUpShape {
    static constexpr int CPL = chunks_per_lane(KG);
    static constexpr int RPL = rows_per_load(KG);
    static constexpr int R = gateup_rows(KG);
    static constexpr int NL = R / RPL;  // wave loads per matrix per chunk column
    static constexpr int B = KG >= kWave ? 6 : ilog2(KG);
    static constexpr int NV = 2 * NL;
};

// Loads this lane's activation groups (bf16) and converts them to scaled
// fp16 pairs; returns the scaling exponent kx (activations * 2^kx).
template <int KG>
__device__ __forceinline__ int load_activation_pairs(const uint16_t* __restrict__ x, int lane,
                                                     f16x2 (&xp)[GateUpShape<KG>::CPL][16]) {
    using S = GateUpShape<KG>;
    const int g0 = KG >= kWave ? lane : (lane & (KG - 1));
    u32x4 raw[S::CPL][4];
    unsigned mx = 0;
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        const uint16_t* xg = x + 32 * (g0 + kWave * c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            raw[c][q] = *reinterpret_cast<const u32x4*>(xg + 8 * q);
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const unsigned d = raw[c][q][z];
                const unsigned lo = d & 0x7FFFu, hi = (d >> 16) & 0x7FFFu;
                mx = lo > mx ? lo : mx;
                mx = hi > mx ? hi : mx;
            }
        }
    }
    mx = wave_max_u32(mx);
    const int kx = range_exponent((mx >> 7) & 0xFFu);
    const float sc = __builtin_ldexpf(1.0f, kx);
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        unsigned dw[16];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int z = 0; z < 4; ++z) dw[4 * q + z] = raw[c][q][z];
        // columns 8d..8d+7 live in dwords 4d..4d+3 (two bf16 each)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned da = dw[4 * d + j / 2], db = dw[4 * d + 2 + j / 2];
                const unsigned ba = (j & 1) ? (da & 0xFFFF0000u) : (da << 16);
                const unsigned bb = (j & 1) ? (db & 0xFFFF0000u) : (db << 16);
                const float fa = __builtin_bit_cast(float, ba) * sc;
                const float fb = __builtin_bit_cast(float, bb) * sc;
                xp[c][4 * d + j] = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(fa, fb));
            }
        }
    }
    return kx;
}

// One gate/up work item: rows [rb*R, rb*R+R) of gate and up of one expert;
// writes h = silu(g) * u (fp32) for those rows.
template <int KG>
__device__ __forceinline__ void gateup_item(const uint8_t* __restrict__ blob, const BlobLayout& L, int rb,
                                            int lane, const f16x2 (&xp)[GateUpShape<KG>::CPL][16], int kx,
                                            float* __restrict__ h_out) {
    using S = GateUpShape<KG>;
    const int g0 = KG >= kWave ? lane : (lane & (KG - 1));
    const int row_sub = KG >= kWave ? 0 : (lane / KG);
    u32x4 cg[S::NL][S::CPL], cu[S::NL][S::CPL];
#pragma unroll
    for (int n = 0; n < S::NL; ++n) {
        const size_t row = (size_t)rb * S::R + n * S::RPL + row_sub;
#pragma unroll
        for (int c = 0; c < S::CPL; ++c) {
            const size_t off = (row * KG + g0 + kWave * c) * 16;
            cg[n][c] = load_stream16(blob + L.gate_q + off);
            cu[n][c] = load_stream16(blob + L.up_q + off);
        }
    }
    // scales: NL consecutive fp16 per (lane, chunk column)
    float sg[S::CPL][S::NL], su[S::CPL][S::NL];
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        const size_t si = ((size_t)rb * KG + g0 + kWave * c) * S::R + (size_t)row_sub * S::NL;
        const uint16_t* pg = reinterpret_cast<const uint16_t*>(blob + L.gate_s) + si;
        const uint16_t* pu = reinterpret_cast<const uint16_t*>(blob + L.up_s) + si;
        if constexpr (S::NL == 4) {
            const u32x2 a = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(pg));
            const u32x2 b = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(pu));
            sg[c][0] = half_bits_to_float(a[0] & 0xFFFFu);
            sg[c][1] = half_bits_to_float(a[0] >> 16);
            sg[c][2] = half_bits_to_float(a[1] & 0xFFFFu);
            sg[c][3] = half_bits_to_float(a[1] >> 16);
            su[c][0] = half_bits_to_float(b[0] & 0xFFFFu);
            su[c][1] = half_bits_to_float(b[0] >> 16);
            su[c][2] = half_bits_to_float(b[1] & 0xFFFFu);
            su[c][3] = half_bits_to_float(b[1] >> 16);
        } else {
#pragma unroll
            for (int n = 0; n < S::NL; ++n) {
                sg[c][n] = half_bits_to_float(pg[n]);
                su[c][n] = half_bits_to_float(pu[n]);
            }
        }
    }
    float v[S::NV];
#pragma unroll
    for (int n = 0; n < S::NL; ++n) {
        float ag = 0.0f, au = 0.0f;
#pragma unroll
        for (int c = 0; c < S::CPL; ++c) {
            ag = fmaf(sg[c][n], dot_chunk(cg[n][c], xp[c], 0.0f), ag);
            au = fmaf(su[c][n], dot_chunk(cu[n][c], xp[c], 0.0f), au);
        }
        v[n] = ag;
        v[S::NL + n] = au;
    }
    const float r = reduce_scatter<S::NV, S::B>(v, lane);
    // value index: top bit = matrix (0 gate, 1 up), low bits = row step n
    const float other = __shfl_xor(r, 1 << (S::B - 1));
    const int low_bits = S::B - ilog2(S::NV);
    const int vi = (lane >> low_bits) & (S::NV - 1);
    if (vi < S::NL && (lane & ((1 << low_bits) - 1)) == 0) {
        const float g = __builtin_ldexpf(r, -kx);
        const float u = __builtin_ldexpf(other, -kx);
        const float h = g / (1.0f + expf(-g)) * u;
        h_out[(size_t)rb * S::R + vi * S::RPL + row_sub] = h;
    }
}

// Blob of a slot: routed slots 0..K-1 follow the routing, shared ones follow.
__device__ __forceinline__ const uint8_t* slot_blob(const DecodeArgs& a, int slot) {
    if (slot >= a.K) return a.shared_blob;
    return a.direct ? a.blobs[slot] : a.table[a.ids[slot]];
}

// Slots [slot_begin, slot_end), or the launch's slot list when it has one.
template <int KG>
__device__ __forceinline__ void gateup_loop(const DecodeArgs& a, int slot_begin, int slot_end, bool use_list,
                                            int wave_id, int n_waves, int lane) {
    using S = GateUpShape<KG>;
    f16x2 xp[S::CPL][16];
    const int kx = load_activation_pairs<KG>(a.x, lane, xp);
    const BlobLayout L = blob_layout(a.H, a.I);
    const int per_slot = a.I / S::R;
    const int n_slots = use_list ? a.n_slot_list : slot_end - slot_begin;
    const int n_items = n_slots * per_slot;
    for (int item = wave_id; item < n_items; item += n_waves) {
        const int k = item / per_slot;
        const int slot = use_list ? a.slot_list[k] : slot_begin + k;
        const int rb = item % per_slot;
        gateup_item<KG>(slot_blob(a, slot), L, rb, lane, xp, kx, a.h + (size_t)slot * a.I);
    }
}

// ---------------------------------------------------------------- kernel 1
template <int KG, int EPL>
__global__ void __launch_bounds__(256) router_shared_kernel(DecodeArgs a, int n_router_wg, int n_shared_wg) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if ((int)blockIdx.x >= n_router_wg) {
        // shared expert gate/up
        const int wg = blockIdx.x - n_router_wg;
        gateup_loop<KG>(a, a.K, a.K + a.S, false, wg * 4 + wave, n_shared_wg * 4, lane);
        return;
    }
    // Router: logits[e] = sum_h W_r[e][h] x[h] in fp32.  Lane l covers
    // floats [4l + 256c, 4l + 256c + 4) of a row.
    constexpr int CR = KG / 8;  // H / 256
    float xr[CR][4];
#pragma unroll
    for (int c = 0; c < CR; ++c) {
        const u32x2 xb = *reinterpret_cast<const u32x2*>(a.x + 4 * lane + 256 * c);
        xr[c][0] = __builtin_bit_cast(float, xb[0] << 16);
        xr[c][1] = __builtin_bit_cast(float, xb[0] & 0xFFFF0000u);
        xr[c][2] = __builtin_bit_cast(float, xb[1] << 16);
        xr[c][3] = __builtin_bit_cast(float, xb[1] & 0xFFFF0000u);
    }
    const int n_router_waves = n_router_wg * 4;
    for (int e = blockIdx.x * 4 + wave; e < a.E; e += n_router_waves) {
        const float* row = a.router_w + (size_t)e * a.H;
        f32x4 wv[CR];
#pragma unroll
        for (int c = 0; c < CR; ++c)
            wv[c] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + 4 * lane + 256 * c));
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < CR; ++c) {
            acc = fmaf(wv[c][0], xr[c][0], acc);
            acc = fmaf(wv[c][1], xr[c][1], acc);
            acc = fmaf(wv[c][2], xr[c][2], acc);
            acc = fmaf(wv[c][3], xr[c][3], acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) a.logits[e] = acc;
    }
    // The last router workgroup to arrive runs the top-k.
    __threadfence();
    __syncthreads();
    __shared__ int s_last;
    if (threadIdx.x == 0) s_last = atomicAdd(a.ticket, 1u) == (unsigned)(n_router_wg - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (wave == 0) {
        wave_group_topk<EPL>(a.logits, a.bias, a.E, a.G, a.TG, a.K, a.rsf, a.ids, a.w, lane);
        if (lane == 0) atomicExch(a.ticket, 0u);
    }
}

// ---------------------------------------------------------------- kernel 2
template <int KG>
__global__ void __launch_bounds__(256) gateup_kernel(DecodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    gateup_loop<KG>(a, 0, a.K, a.n_slot_list > 0, blockIdx.x * 4 + wave, gridDim.x * 4, lane);
}

// ---------------------------------------------------------------- kernel 3
template <int KG>
struct DownShape {
    static constexpr int CPL = chunks_per_lane(KG);
    static constexpr int RPL = rows_per_load(KG);
    static constexpr int R = down_rows(KG);
    static constexpr int NL = R / RPL;
    static constexpr int B = KG >= kWave ? 6 : ilog2(KG);
};

// One workgroup = one wave per slot (routed experts, then shared ones) and a
// block of R output rows.  Each wave computes its expert's R outputs; the
// first R threads combine them in slot order.
template <int KG, int MAXW>
__global__ void __launch_bounds__(MAXW * 64) down_combine_kernel(DecodeArgs a) {
    using S = DownShape<KG>;
    const int lane = threadIdx.x & 63;
    const int slot = threadIdx.x >> 6;
    const int g0 = KG >= kWave ? lane : (lane & (KG - 1));
    const int row_sub = KG >= kWave ? 0 : (lane / KG);
    const int rb = blockIdx.x;
    const uint8_t* blob = slot_blob(a, slot);
    const BlobLayout L = blob_layout(a.H, a.I);

    u32x4 code[S::NL][S::CPL];
#pragma unroll
    for (int n = 0; n < S::NL; ++n) {
        const size_t row = (size_t)rb * S::R + n * S::RPL + row_sub;
#pragma unroll
        for (int c = 0; c < S::CPL; ++c) code[n][c] = load_stream16(blob + L.down_q + (row * KG + g0 + kWave * c) * 16);
    }
    float sc[S::CPL][S::NL];
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        const size_t si = ((size_t)rb * KG + g0 + kWave * c) * S::R + (size_t)row_sub * S::NL;
        const uint16_t* ps = reinterpret_cast<const uint16_t*>(blob + L.down_s) + si;
        if constexpr (S::NL % 8 == 0) {
#pragma unroll
            for (int n8 = 0; n8 < S::NL / 8; ++n8) {
                const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ps + 8 * n8));
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    sc[c][8 * n8 + 2 * z] = half_bits_to_float(q[z] & 0xFFFFu);
                    sc[c][8 * n8 + 2 * z + 1] = half_bits_to_float(q[z] >> 16);
                }
            }
        } else {
#pragma unroll
            for (int n = 0; n < S::NL; ++n) sc[c][n] = half_bits_to_float(ps[n]);
        }
    }
    // h of this slot, this lane's groups: scaled per group to [2^13, 2^14),
    // split into fp16 hi + lo pairs in the chunk's column order.
    f16x2 hp[S::CPL][16], lp[S::CPL][16];
    float hscale[S::CPL];
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        const float* hg = a.h + (size_t)slot * a.I + 32 * (g0 + kWave * c);
        float hv[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(hg + 4 * q);
            hv[4 * q + 0] = t[0];
            hv[4 * q + 1] = t[1];
            hv[4 * q + 2] = t[2];
            hv[4 * q + 3] = t[3];
        }
        unsigned mx = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const unsigned b = __builtin_bit_cast(unsigned, hv[i]) & 0x7FFFFFFFu;
            mx = b > mx ? b : mx;
        }
        const int kh = range_exponent(mx >> 23);
        hscale[c] = __builtin_ldexpf(1.0f, -kh);
        const float up = __builtin_ldexpf(1.0f, kh);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float fa = hv[8 * d + j] * up, fb = hv[8 * d + j + 4] * up;
                const f16x2 hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(fa, fb));
                const float ra = fa - (float)hi[0], rb2 = fb - (float)hi[1];
                hp[c][4 * d + j] = hi;
                lp[c][4 * d + j] = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(ra, rb2));
            }
        }
    }
    float v[S::NL];
#pragma unroll
    for (int n = 0; n < S::NL; ++n) {
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < S::CPL; ++c)
            acc = fmaf(sc[c][n] * hscale[c], dot_chunk_hilo(code[n][c], hp[c], lp[c], 0.0f), acc);
        v[n] = acc;
    }
    const float r = reduce_scatter<S::NL, S::B>(v, lane);
    __shared__ float part[MAXW][S::R];
    const int low_bits = S::B - ilog2(S::NL);
    if ((lane & ((1 << low_bits) - 1)) == 0) {
        const int vi = (lane >> low_bits) & (S::NL - 1);
        part[slot][vi * S::RPL + row_sub] = r;
    }
    __syncthreads();
    if ((int)threadIdx.x < S::R) {
        const int t = threadIdx.x;
        float y = 0.0f;
        for (int j = 0; j < a.K; ++j) y = fmaf(a.w[j], part[j][t], y);
        for (int j = a.K; j < a.K + a.S; ++j) y += part[j][t];
        a.y[(size_t)rb * S::R + t] = y;
    }
}

// ---------------------------------------------------------------- launchers
template <int KG, int EPL>
hipError_t launch_router_shared(const DecodeArgs& a, hipStream_t st) {
    const int n_router_wg = (a.E + 3) / 4;
    const int shared_items = a.S * (a.I / GateUpShape<KG>::R);
    const int shared_waves = shared_items < 512 ? shared_items : 512;
    const int n_shared_wg = a.S > 0 ? (shared_waves + 3) / 4 : 0;
    hipLaunchKernelGGL((router_shared_kernel<KG, EPL>), dim3(n_router_wg + n_shared_wg), dim3(256), 0, st, a,
                       n_router_wg, n_shared_wg);
    return hipGetLastError();
}

template <int KG>
hipError_t launch_gateup(const DecodeArgs& a, hipStream_t st) {
    const int n_slots = a.n_slot_list > 0 ? a.n_slot_list : a.K;
    const int items = n_slots * (a.I / GateUpShape<KG>::R);
    const int waves = items < 2048 ? items : 2048;
    hipLaunchKernelGGL((gateup_kernel<KG>), dim3((waves + 3) / 4), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int KG>
hipError_t launch_down(const DecodeArgs& a, hipStream_t st) {
    const int nw = a.K + a.S;
    const int grid = a.H / DownShape<KG>::R;
    if (nw <= 9)
        hipLaunchKernelGGL((down_combine_kernel<KG, 9>), dim3(grid), dim3(nw * 64), 0, st, a);
    else
        hipLaunchKernelGGL((down_combine_kernel<KG, 16>), dim3(grid), dim3(nw * 64), 0, st, a);
    return hipGetLastError();
}

template <int KG>
hipError_t router_dispatch_epl(const DecodeArgs& a, hipStream_t st) {
    if (a.E <= 64) return launch_router_shared<KG, 1>(a, st);
    if (a.E <= 128) return launch_router_shared<KG, 2>(a, st);
    return launch_router_shared<KG, 4>(a, st);
}

}  // namespace

// Kernels are instantiated for H/32 in {8,16,32,64,128,192,256} and
// I/32 in {4,8,16,32,64,128}.
hipError_t decode_router_and_shared(const DecodeArgs& a, hipStream_t st) {
    switch (a.H / 32) {
        case 8: return router_dispatch_epl<8>(a, st);
        case 16: return router_dispatch_epl<16>(a, st);
        case 32: return router_dispatch_epl<32>(a, st);
        case 64: return router_dispatch_epl<64>(a, st);
        case 128: return router_dispatch_epl<128>(a, st);
        case 192: return router_dispatch_epl<192>(a, st);
        case 256: return router_dispatch_epl<256>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t decode_routed_gateup(const DecodeArgs& a, hipStream_t st) {
    switch (a.H / 32) {
        case 8: return launch_gateup<8>(a, st);
        case 16: return launch_gateup<16>(a, st);
        case 32: return launch_gateup<32>(a, st);
        case 64: return launch_gateup<64>(a, st);
        case 128: return launch_gateup<128>(a, st);
        case 192: return launch_gateup<192>(a, st);
        case 256: return launch_gateup<256>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t decode_down_combine(const DecodeArgs& a, hipStream_t st) {
    switch (a.I / 32) {
        case 4: return launch_down<4>(a, st);
        case 8: return launch_down<8>(a, st);
        case 16: return launch_down<16>(a, st);
        case 32: return launch_down<32>(a, st);
        case 64: return launch_down<64>(a, st);
        case 128: return launch_down<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

bool decode_shape_supported(int hidden, int inter) {
    const int kh = hidden / 32, ki = inter / 32;
    const bool h_ok = kh == 8 || kh == 16 || kh == 32 || kh == 64 || kh == 128 || kh == 192 || kh == 256;
    const bool i_ok = ki == 4 || ki == 8 || ki == 16 || ki == 32 || ki == 64 || ki == 128;
    return h_ok && i_ok && hidden % 32 == 0 && inter % 32 == 0 && hidden % down_rows(ki) == 0 &&
           inter % gateup_rows(kh) == 0;
}

}  // namespace moe
