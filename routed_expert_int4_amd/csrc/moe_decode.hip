// Decode (one token per call) kernels of the routed int4 MoE layer, gfx950.
//
// Per token:
//   1. router: router logits, one fp32 row of W_r per wave, turned
//      into s = sigmoid(logit) and sb = s + bias; the last router block to
//      finish (device-scope counter) derives the group-limited top-k with DPP
//      reductions and writes ids, weights and the routed slots' blobs; in
//      the same launch other workgroups run the shared expert's gate/up +
//      SwiGLU (no routing dependency) and convert the token's activations
//      once into the integer operands of the routed experts' kernel.
//   2. gateup: gate/up + SwiGLU of the routed experts; the next items' loads
//      are in flight while the current ones are computed.
//   3. down_combine: one wave per slot (routed and shared) over a block of
//      output rows, row loads pipelined; the block is combined in slot order
//      (no float atomics: repeated calls are bit-identical).
//
// Int4 GEMV scheme.  A lane owns one 32-input scale group of the reduction
// dimension (several when a row has more than 64 groups) and keeps the
// matching activations in registers; every wave load is 64 lanes x 16
// contiguous bytes.  A 16-byte chunk holds the 32 codes of one group (stored
// q+8); masking the even and the odd nibbles gives two dwords of 8-bit codes
// per code dword, which v_dot4_i32_i8 multiplies with the activations held
// as exact 8-bit hi and lo parts of a 16-bit fixed-point form of the group
// (power-of-two scale per group).  The dot is exact in int32; the offset 8 is
// removed with a per-group correction, and the fp16 weight scale and the
// group's power of two are applied once per chunk in fp32.  Partial sums of
// the rows a wave visited are reduced across lanes with a reduce-scatter.
//
// The kernels are templated on the weight codec; the lane mapping, loads and
// pipelines stay those of int4.  MXFP4: E2M1 code bytes become exact fp16
// pairs (v_cvt_scalef32_pk_f16_fp4) dotted with fp16 activation pairs
// (v_dot2c_f32_f16), E8M0 scale bytes.  Int8: two int4-shaped nibble planes
// per matrix (q = 16 hi + lo), both dotted with the same 8-bit operands.
// Int2: int4-shaped planes of half the rows, a nibble holding the codes of
// two adjacent rows, one chunk dot yielding both rows.  With the adaptive
// top-p cut the router also writes the kept slots, gate/up covers only
// those and down skips the dropped slots' waves.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_device.h"
#include "moe_kernels.h"
#include "moe_layout.h"

namespace moe {
namespace {

// One 32-value group of an activation vector (x for gate/up, h for down) as
// 8-bit dot operands: the group scaled by a power of two to 16-bit integers
// a = round(v 2^k) (group maximum in [2^14, 2^15)), split exactly into
// a = 256 hi + lo with hi signed (v_dot4_i32_i8) and lo unsigned in [0, 255]
// (v_dot4_u32_u8).  Byte j of dword d pairs with nibble 2j (he, le) or 2j + 1
// (ho, lo) of code dword d, i.e. with columns 8d + 2j and 8d + 2j + 1 of the
// group.  The codes hold q + 8, so corr = 8 sum(a) is taken off the integer
// dot; |sum q a| < 2^23, so the int32 result converts to fp32 exactly.
struct HI8 {
    u32x4 he, ho, le, lo;
    int corr;
};

template <int CPL>
__device__ __forceinline__ void to_i8(const float (&hin)[CPL][32], HI8 (&ha)[CPL], float (&hscale)[CPL]) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const float (&hv)[32] = hin[c];
        unsigned mx = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) mx = umax(mx, __builtin_bit_cast(unsigned, hv[i]) & 0x7FFFFFFFu);
        const int kh = range_exponent(mx >> 23) + 1;  // max |v| 2^kh in [2^14, 2^15)
        hscale[c] = __builtin_ldexpf(1.0f, -kh);
        const float up = __builtin_ldexpf(1.0f, kh);
        int sum = 0;
        unsigned vhe[4], vho[4], vle[4], vlo[4];
        auto fix16 = [&](float v) {
            const float r = __builtin_rintf(v * up);
            return (int)(r > 32767.0f ? 32767.0f : (r < -32768.0f ? -32768.0f : r));
        };
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            unsigned he = 0, ho = 0, le = 0, lo = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ae = fix16(hv[8 * d + 2 * j]);
                const int ao = fix16(hv[8 * d + 2 * j + 1]);
                // a = 256 hi + lo with hi = floor(a / 256) signed, lo = a mod 256 unsigned
                he |= ((unsigned)(ae >> 8) & 0xFFu) << (8 * j);
                ho |= ((unsigned)(ao >> 8) & 0xFFu) << (8 * j);
                le |= ((unsigned)ae & 0xFFu) << (8 * j);
                lo |= ((unsigned)ao & 0xFFu) << (8 * j);
                sum += ae + ao;
            }
            vhe[d] = he;
            vho[d] = ho;
            vle[d] = le;
            vlo[d] = lo;
        }
        ha[c].he = u32x4{vhe[0], vhe[1], vhe[2], vhe[3]};
        ha[c].ho = u32x4{vho[0], vho[1], vho[2], vho[3]};
        ha[c].le = u32x4{vle[0], vle[1], vle[2], vle[3]};
        ha[c].lo = u32x4{vlo[0], vlo[1], vlo[2], vlo[3]};
        ha[c].corr = 8 * sum;
    }
}

// Exact integer dot of one 16-byte code chunk (32 columns of a group) with
// h in the HI8 form: sum_k q_k a_k, returned as float (|value| < 2^23).
__device__ __forceinline__ float dot_chunk_i8(u32x4 c, const HI8& a) {
    int hi = 0, lo = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const unsigned w = c[d], he = a.he[d], ho = a.ho[d], le = a.le[d], lo_ = a.lo[d];
        const int e = (int)(w & 0x0F0F0F0Fu), o = (int)((w >> 4) & 0x0F0F0F0Fu);
        hi = __builtin_amdgcn_sdot4(e, (int)he, hi, false);
        hi = __builtin_amdgcn_sdot4(o, (int)ho, hi, false);
        lo = (int)__builtin_amdgcn_udot4((unsigned)e, le, (unsigned)lo, false);
        lo = (int)__builtin_amdgcn_udot4((unsigned)o, lo_, (unsigned)lo, false);
    }
    return (float)(hi * 256 + lo - a.corr);
}

// MXFP4 scheme: the activation group as fp16 pairs in natural column order,
// scaled by a power of two so that its maximum lies in [2^14, 2^15) (exact
// for bf16 x; round to nearest for h), held in the HI8 container: dword j of
// he, ho, le, lo (code dword d = 0, 1, 2, 3) pairs with byte j of code dword
// d, i.e. columns 8d + 2j (low nibble) and 8d + 2j + 1 (high nibble).
template <int CPL>
__device__ __forceinline__ void to_f16(const float (&hin)[CPL][32], HI8 (&ha)[CPL], float (&hscale)[CPL]) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const float (&hv)[32] = hin[c];
        unsigned mx = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) mx = umax(mx, __builtin_bit_cast(unsigned, hv[i]) & 0x7FFFFFFFu);
        const int kh = range_exponent(mx >> 23) + 1;  // max |v| 2^kh in [2^14, 2^15)
        hscale[c] = __builtin_ldexpf(1.0f, -kh);
        const float up = __builtin_ldexpf(1.0f, kh);
        unsigned p[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const f16x2 pair = {(_Float16)(hv[2 * k] * up), (_Float16)(hv[2 * k + 1] * up)};
            p[k] = __builtin_bit_cast(unsigned, pair);
        }
        ha[c].he = u32x4{p[0], p[1], p[2], p[3]};
        ha[c].ho = u32x4{p[4], p[5], p[6], p[7]};
        ha[c].le = u32x4{p[8], p[9], p[10], p[11]};
        ha[c].lo = u32x4{p[12], p[13], p[14], p[15]};
        ha[c].corr = 0;
    }
}

// Dot of one 16-byte chunk of E2M1 codes with the fp16 pairs: each code byte
// becomes an fp16 pair with v_cvt_scalef32_pk_f16_fp4 (scale 1, so the pair
// holds the E2M1 values exactly), multiplied and summed in fp32 by
// v_dot2c_f32_f16.
__device__ __forceinline__ float dot_chunk_fp4(u32x4 c, const HI8& a) {
    float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const unsigned w = c[d];
        const u32x4 x = d == 0 ? a.he : d == 1 ? a.ho : d == 2 ? a.le : a.lo;
        acc0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0), as_h2(x[0]), acc0, false);
        acc1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1), as_h2(x[1]), acc1, false);
        acc0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2), as_h2(x[2]), acc0, false);
        acc1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3), as_h2(x[3]), acc1, false);
    }
    return acc0 + acc1;
}

// Int8 codes split into two nibble planes, q = 16 hi + lo (hi stored + 8,
// lo unsigned): both planes take the int4 dot with the same HI8 operands,
// 16 sum(q a) = 16 (sum((hi + 8) a) - corr) + sum(lo a), exact in int32
// (|value| < 2^28; the conversion to fp32 rounds once).
__device__ __forceinline__ float dot_chunk_int8(u32x4 chi, u32x4 clo, const HI8& a) {
    int h1 = 0, l1 = 0, h2 = 0, l2 = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const unsigned he = a.he[d], ho = a.ho[d], le = a.le[d], lo_ = a.lo[d];
        const unsigned w = chi[d], v = clo[d];
        const int e = (int)(w & 0x0F0F0F0Fu), o = (int)((w >> 4) & 0x0F0F0F0Fu);
        const int e2 = (int)(v & 0x0F0F0F0Fu), o2 = (int)((v >> 4) & 0x0F0F0F0Fu);
        h1 = __builtin_amdgcn_sdot4(e, (int)he, h1, false);
        h1 = __builtin_amdgcn_sdot4(o, (int)ho, h1, false);
        l1 = (int)__builtin_amdgcn_udot4((unsigned)e, le, (unsigned)l1, false);
        l1 = (int)__builtin_amdgcn_udot4((unsigned)o, lo_, (unsigned)l1, false);
        h2 = __builtin_amdgcn_sdot4(e2, (int)he, h2, false);
        h2 = __builtin_amdgcn_sdot4(o2, (int)ho, h2, false);
        l2 = (int)__builtin_amdgcn_udot4((unsigned)e2, le, (unsigned)l2, false);
        l2 = (int)__builtin_amdgcn_udot4((unsigned)o2, lo_, (unsigned)l2, false);
    }
    return (float)(16 * (h1 * 256 + l1 - a.corr) + h2 * 256 + l2);
}

// Int2 chunk: every nibble holds the codes of two rows (bits 0-1: the even
// row, bits 2-3: the odd row), each + 2; both rows take the int4 dot with the
// same HI8 operands and the offset correction 2 sum(a) = corr / 4.
__device__ __forceinline__ void dot_chunk_int2(u32x4 c, const HI8& a, float& r0, float& r1) {
    int h0 = 0, l0 = 0, h1 = 0, l1 = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const unsigned he = a.he[d], ho = a.ho[d], le = a.le[d], lo_ = a.lo[d];
        const unsigned w = c[d];
        const unsigned e = w & 0x0F0F0F0Fu, o = (w >> 4) & 0x0F0F0F0Fu;
        const int e0 = (int)(e & 0x03030303u), o0 = (int)(o & 0x03030303u);
        const int e1 = (int)((e >> 2) & 0x03030303u), o1 = (int)((o >> 2) & 0x03030303u);
        h0 = __builtin_amdgcn_sdot4(e0, (int)he, h0, false);
        h0 = __builtin_amdgcn_sdot4(o0, (int)ho, h0, false);
        l0 = (int)__builtin_amdgcn_udot4((unsigned)e0, le, (unsigned)l0, false);
        l0 = (int)__builtin_amdgcn_udot4((unsigned)o0, lo_, (unsigned)l0, false);
        h1 = __builtin_amdgcn_sdot4(e1, (int)he, h1, false);
        h1 = __builtin_amdgcn_sdot4(o1, (int)ho, h1, false);
        l1 = (int)__builtin_amdgcn_udot4((unsigned)e1, le, (unsigned)l1, false);
        l1 = (int)__builtin_amdgcn_udot4((unsigned)o1, lo_, (unsigned)l1, false);
    }
    const int corr = a.corr >> 2;
    r0 = (float)(h0 * 256 + l0 - corr);
    r1 = (float)(h1 * 256 + l1 - corr);
}

// Codec dispatch of the operand form and the chunk dot.
template <int F, int CPL>
__device__ __forceinline__ void to_operands(const float (&hin)[CPL][32], HI8 (&ha)[CPL], float (&hscale)[CPL]) {
    if constexpr (F == kCodecMxfp4)
        to_f16<CPL>(hin, ha, hscale);
    else
        to_i8<CPL>(hin, ha, hscale);
}
template <int F>
__device__ __forceinline__ float dot_chunk(u32x4 c, const HI8& a) {
    if constexpr (F == kCodecMxfp4)
        return dot_chunk_fp4(c, a);
    else
        return dot_chunk_i8(c, a);
}
// Chunk dot over the codec's planes: c[0] (and c[1] for int8).
template <int F, int P>
__device__ __forceinline__ float dot_planes(const u32x4 (&c)[P], const HI8& a) {
    if constexpr (F == kCodecInt8)
        return dot_chunk_int8(c[0], c[1], a);
    else
        return dot_chunk<F>(c[0], a);
}

// ---------------------------------------------------------------- gate/up
constexpr int kGateUpItemsPerRound = 2;   // routed gate/up kernel
constexpr int kSharedItemsPerRound = 3;   // shared expert's gate/up in the router launch
constexpr int kRouterWavesPerRow = 1;     // waves per router row (1, 2 or 4)
__host__ __device__ constexpr int router_blocks(int n_experts) {
    return (n_experts + 4 / kRouterWavesPerRow - 1) / (4 / kRouterWavesPerRow);
}
// Work items of the gate/up stage: (slot, block of R rows of gate and up).
template <int KG>
struct GateUpShape {
    static constexpr int CPL = chunks_per_lane(KG);
    static constexpr int RPL = rows_per_load(KG);
    static constexpr int R = gateup_rows(KG);
    static constexpr int NL = R / RPL;  // wave loads per matrix per chunk column
    static constexpr int B = KG >= kWave ? 6 : ilog2(KG);
    static constexpr int NV = 2 * NL;
    static_assert(RPL == 1 || NL == 1, "gate/up scale runs");
};

// NL consecutive fp16 scales (NL*2-byte aligned) -> (NL+1)/2 dwords.
template <int NL>
__device__ __forceinline__ void load_scales(const uint16_t* p, unsigned (&d)[(NL + 1) / 2]) {
    if constexpr (NL == 1) {
        d[0] = __builtin_nontemporal_load(as_global<uint16_t>(p));
    } else if constexpr (NL == 2) {
        d[0] = __builtin_nontemporal_load(as_global<unsigned>(p));
    } else if constexpr (NL == 4) {
        const u32x2 v = __builtin_nontemporal_load(as_global<u32x2>(p));
        d[0] = v[0];
        d[1] = v[1];
    } else if constexpr (NL % 8 != 0) {
        static_assert(NL % 4 == 0, "scale pack");
#pragma unroll
        for (int q = 0; q < NL / 4; ++q) {
            const u32x2 v = __builtin_nontemporal_load(as_global<u32x2>(p) + q);
            d[2 * q + 0] = v[0];
            d[2 * q + 1] = v[1];
        }
    } else {
#pragma unroll
        for (int q = 0; q < NL / 8; ++q) {
            const u32x4 v = __builtin_nontemporal_load(as_global<u32x4>(p) + q);
            d[4 * q + 0] = v[0];
            d[4 * q + 1] = v[1];
            d[4 * q + 2] = v[2];
            d[4 * q + 3] = v[3];
        }
    }
}
// NL consecutive E8M0 bytes (NL-byte aligned, up to 4 per dword).
template <int NL, int M>
__device__ __forceinline__ void load_scale_bytes(const uint8_t* p, unsigned (&d)[M]) {
    static_assert(M * 4 >= NL, "scale pack");
    if constexpr (NL == 1) {
        d[0] = __builtin_nontemporal_load(as_global<uint8_t>(p));
    } else if constexpr (NL == 2) {
        d[0] = __builtin_nontemporal_load(as_global<uint16_t>(p));
    } else if constexpr (NL == 4) {
        d[0] = __builtin_nontemporal_load(as_global<unsigned>(p));
    } else if constexpr (NL % 8 != 0) {
        static_assert(NL % 4 == 0, "scale pack");
#pragma unroll
        for (int q = 0; q < NL / 4; ++q) d[q] = __builtin_nontemporal_load(as_global<unsigned>(p) + q);
    } else if constexpr (NL % 16 != 0) {
#pragma unroll
        for (int q = 0; q < NL / 8; ++q) {
            const u32x2 v = __builtin_nontemporal_load(as_global<u32x2>(p) + q);
            d[2 * q + 0] = v[0];
            d[2 * q + 1] = v[1];
        }
    } else {
#pragma unroll
        for (int q = 0; q < NL / 16; ++q) {
            const u32x4 v = __builtin_nontemporal_load(as_global<u32x4>(p) + q);
            d[4 * q + 0] = v[0];
            d[4 * q + 1] = v[1];
            d[4 * q + 2] = v[2];
            d[4 * q + 3] = v[3];
        }
    }
}

// NL consecutive scales of codec F starting at byte pointer p.
template <int F, int NL, int M>
__device__ __forceinline__ void load_scales_c(const uint8_t* p, unsigned (&d)[M]) {
    if constexpr (F == kCodecMxfp4) {
        load_scale_bytes<NL>(p, d);
    } else {
        static_assert(M == (NL + 1) / 2, "scale pack");
        load_scales<NL>(reinterpret_cast<const uint16_t*>(p), d);
    }
}

// Scale n of a run loaded by load_scales_c.
template <int F, int N>
__device__ __forceinline__ float scale_at(const unsigned (&d)[N], int n) {
    if constexpr (F == kCodecMxfp4)
        return e8m0_to_float((d[n / 4] >> (8 * (n % 4))) & 0xFFu);
    else
        return half_bits_to_float((n & 1) ? (d[n / 2] >> 16) : (d[n / 2] & 0xFFFFu));
}

// This lane's activation groups (bf16, natural column order) in the HI8
// form, with the per-group factor that undoes the integer scaling.
template <int KG, int F>
__device__ __forceinline__ void convert_activations(const uint16_t* __restrict__ x, int lane,
                                                    HI8 (&xa)[GateUpShape<KG>::CPL], float (&xs)[GateUpShape<KG>::CPL]) {
    using S = GateUpShape<KG>;
    const int g0 = KG >= kWave ? lane : (lane & (KG - 1));
    float xv[S::CPL][32];
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        const uint16_t* xg = x + 32 * (g0 + kWave * c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 raw = *reinterpret_cast<const u32x4*>(xg + 8 * q);
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const unsigned d = raw[z];
                xv[c][8 * q + 2 * z] = __builtin_bit_cast(float, d << 16);
                xv[c][8 * q + 2 * z + 1] = __builtin_bit_cast(float, d & 0xFFFF0000u);
            }
        }
    }
    to_operands<F, S::CPL>(xv, xa, xs);
}

// The same conversion one chunk column at a time (32 floats live instead of
// 32 per column), for kernels that keep many other registers.
template <int KG, int F>
__device__ __forceinline__ void convert_activations_by_column(const uint16_t* __restrict__ x, int lane,
                                                              HI8 (&xa)[GateUpShape<KG>::CPL],
                                                              float (&xs)[GateUpShape<KG>::CPL]) {
    using S = GateUpShape<KG>;
    const int g0 = KG >= kWave ? lane : (lane & (KG - 1));
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        float xv[1][32];
        const uint16_t* xg = x + 32 * (g0 + kWave * c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 raw = *reinterpret_cast<const u32x4*>(xg + 8 * q);
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const unsigned d = raw[z];
                xv[0][8 * q + 2 * z] = __builtin_bit_cast(float, d << 16);
                xv[0][8 * q + 2 * z + 1] = __builtin_bit_cast(float, d & 0xFFFF0000u);
            }
        }
        HI8 a1[1];
        float s1[1];
        to_operands<F, 1>(xv, a1, s1);
        xa[c] = a1[0];
        xs[c] = s1[0];
    }
}

// Converted activations in the workspace: lane l, chunk column c holds the
// 16 byte dwords at [(c*64 + l)*16, +16) and (corr, factor) at
// meta + (c*64 + l)*2, meta = 16*64*CPL dwords on.
template <int KG>
__device__ __forceinline__ void store_activations(unsigned* __restrict__ xq, int lane,
                                                  const HI8 (&xa)[GateUpShape<KG>::CPL],
                                                  const float (&xs)[GateUpShape<KG>::CPL]) {
    using S = GateUpShape<KG>;
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        u32x4* p = reinterpret_cast<u32x4*>(xq + ((size_t)c * kWave + lane) * 16);
        p[0] = xa[c].he;
        p[1] = xa[c].ho;
        p[2] = xa[c].le;
        p[3] = xa[c].lo;
        u32x2* m = reinterpret_cast<u32x2*>(xq + (size_t)16 * kWave * S::CPL + ((size_t)c * kWave + lane) * 2);
        *m = u32x2{(unsigned)xa[c].corr, __builtin_bit_cast(unsigned, xs[c])};
    }
}
template <int KG>
__device__ __forceinline__ void load_activations(const unsigned* __restrict__ xq, int lane,
                                                 HI8 (&xa)[GateUpShape<KG>::CPL], float (&xs)[GateUpShape<KG>::CPL]) {
    using S = GateUpShape<KG>;
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        const u32x4* p = reinterpret_cast<const u32x4*>(xq + ((size_t)c * kWave + lane) * 16);
        xa[c].he = p[0];
        xa[c].ho = p[1];
        xa[c].le = p[2];
        xa[c].lo = p[3];
        const u32x2 m = *reinterpret_cast<const u32x2*>(xq + (size_t)16 * kWave * S::CPL + ((size_t)c * kWave + lane) * 2);
        const unsigned m0 = m[0], m1 = m[1];
        xa[c].corr = (int)m0;
        xs[c] = __builtin_bit_cast(float, m1);
    }
}

template <int KG, int F>
struct GateUpBuf {
    using S = GateUpShape<KG>;
    static constexpr int P = code_planes(F), RP = row_pack(F);
    u32x4 cg[S::NL][S::CPL][P], cu[S::NL][S::CPL][P];  // P code planes (int8: 2)
    unsigned sgu[RP][S::CPL][S::NL];  // per row parity (int2): 0..NL-1 gate, NL..2NL-1 up
};

template <int KG, int F>
__device__ __forceinline__ void gateup_issue(const uint8_t* __restrict__ blob, const BlobLayout& L, int rb, int lane,
                                             GateUpBuf<KG, F>& b) {
    using S = GateUpShape<KG>;
    constexpr int P = code_planes(F);
    const int g0 = KG >= kWave ? lane : (lane & (KG - 1));
    const int row_sub = KG >= kWave ? 0 : (lane / KG);
#pragma unroll
    for (int n = 0; n < S::NL; ++n) {
        const size_t row = (size_t)rb * S::R + n * S::RPL + row_sub;
#pragma unroll
        for (int c = 0; c < S::CPL; ++c) {
            const size_t off = (row * KG + g0 + kWave * c) * 16;
#pragma unroll
            for (int p = 0; p < P; ++p) {
                b.cg[n][c][p] = load_stream16(blob + (p ? L.gate_lo : L.gate_q) + off);
                b.cu[n][c][p] = load_stream16(blob + (p ? L.up_lo : L.up_q) + off);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < row_pack(F); ++h)
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        const uint8_t* p =
            blob + (h ? L.gu_s2 : L.gu_s) + ((size_t)rb * KG + g0 + kWave * c) * 2 * S::R * scale_bytes(F);
        if constexpr (S::RPL == 1) {
            load_scales_c<F, 2 * S::NL>(p, b.sgu[h][c]);
        } else if constexpr (F == kCodecMxfp4) {
            const unsigned g = __builtin_nontemporal_load(as_global<uint8_t>(p + row_sub));
            const unsigned u = __builtin_nontemporal_load(as_global<uint8_t>(p + S::R + row_sub));
            b.sgu[h][c][0] = g | (u << 8);
        } else {
            const uint16_t* p16 = reinterpret_cast<const uint16_t*>(p);
            const unsigned g = __builtin_nontemporal_load(as_global<uint16_t>(p16 + row_sub));
            const unsigned u = __builtin_nontemporal_load(as_global<uint16_t>(p16 + S::R + row_sub));
            b.sgu[h][c][0] = g | (u << 16);
        }
    }
}

// Position of h[i] (i < inter) in a slot's h buffer: the order in which the
// down kernel's lanes read it with contiguous 16-byte loads.  Lane g (group
// g of a chunk column c, groups of 32 values) reads values 4q..4q+3 of its
// group with load q of column c, so those 4 values sit at
// ((c * 8 + q) * G + g) * 4 with G = min(inter / 32, 64).
__device__ __forceinline__ size_t h_index(int i, int kgi) {
    const int g = i >> 5, e = i & 31;
    const int G = kgi < kWave ? kgi : kWave;
    const int c = g / kWave, gi = g % kWave;
    return ((size_t)(c * 8 + (e >> 2)) * G + gi) * 4 + (e & 3);
}

// Computes one item from its loaded buffer: h = silu(g) * u for rows
// [rb*R, rb*R + R), written as fp32 at their h_index positions.
// With SC the h values are stored with device-scope atomic stores, so that
// workgroups of the same launch on other XCDs can read them (the fused
// decode kernel); otherwise with plain stores, read after the launch ends.
// The activation operands come from xsrc(c, operands, factor) for chunk
// column c (registers, or LDS in the fused kernel).
template <int KG, int F, bool SC = false, typename XSrc>
__device__ __forceinline__ void gateup_compute_src(const GateUpBuf<KG, F>& b, int rb, int lane, const XSrc& xsrc,
                                                   float* __restrict__ h_out, int kgi, bool store) {
    using S = GateUpShape<KG>;
    constexpr int RP = row_pack(F);
    constexpr int NV = S::NV * RP;  // gate then up; inside each, row parity then step
    const int row_sub = KG >= kWave ? 0 : (lane / KG);
    float v[NV];
#pragma unroll
    for (int n = 0; n < S::NL; ++n) {
        if constexpr (F == kCodecInt2) {
            float ag0 = 0.0f, ag1 = 0.0f, au0 = 0.0f, au1 = 0.0f;
#pragma unroll
            for (int c = 0; c < S::CPL; ++c) {
                HI8 xc;
                float xsc;
                xsrc(c, xc, xsc);
                float g0, g1, u0, u1;
                dot_chunk_int2(b.cg[n][c][0], xc, g0, g1);
                dot_chunk_int2(b.cu[n][c][0], xc, u0, u1);
                ag0 = fmaf(scale_at<F>(b.sgu[0][c], n) * xsc, g0, ag0);
                ag1 = fmaf(scale_at<F>(b.sgu[RP - 1][c], n) * xsc, g1, ag1);
                au0 = fmaf(scale_at<F>(b.sgu[0][c], S::NL + n) * xsc, u0, au0);
                au1 = fmaf(scale_at<F>(b.sgu[RP - 1][c], S::NL + n) * xsc, u1, au1);
            }
            v[n] = ag0;
            v[S::NL + n] = ag1;
            v[2 * S::NL + n] = au0;
            v[3 * S::NL + n] = au1;
        } else {
            float ag = 0.0f, au = 0.0f;
#pragma unroll
            for (int c = 0; c < S::CPL; ++c) {
                HI8 xc;
                float xsc;
                xsrc(c, xc, xsc);
                ag = fmaf(scale_at<F>(b.sgu[0][c], n) * xsc, dot_planes<F>(b.cg[n][c], xc), ag);
                au = fmaf(scale_at<F>(b.sgu[0][c], S::NL + n) * xsc, dot_planes<F>(b.cu[n][c], xc), au);
            }
            v[n] = ag;
            v[S::NL + n] = au;
        }
    }
    const float r = reduce_scatter<NV, S::B>(v, lane);
    // value index: top bit = matrix (0 gate, 1 up), then row parity, then step
    // n.  partner_value may be a DPP mirror, which also flips the lower lane
    // bits: harmless with one value per matrix, but with two row parities the
    // up partner must be the exact lane xor.
    const float other =
        RP > 1 ? __shfl_xor(r, 1 << (S::B - 1)) : partner_value<S::B - 1>(r, lane);
    const int low_bits = S::B - ilog2(NV);
    const int vi = (lane >> low_bits) & (NV - 1);
    if (store && vi < RP * S::NL && (lane & ((1 << low_bits) - 1)) == 0) {
        const float g = r, u = other;
        const float h = g / (1.0f + expf(-g)) * u;
        const int n = vi % S::NL, parity = vi / S::NL;
        float* dst = h_out + h_index(RP * (rb * S::R + n * S::RPL + row_sub) + parity, kgi);
        if constexpr (SC)
            __hip_atomic_store(dst, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            *dst = h;
    }
}

// Operands held in registers.
template <int KG, int F, bool SC = false>
__device__ __forceinline__ void gateup_compute(const GateUpBuf<KG, F>& b, int rb, int lane,
                                               const HI8 (&xa)[GateUpShape<KG>::CPL],
                                               const float (&xs)[GateUpShape<KG>::CPL], float* __restrict__ h_out,
                                               int kgi, bool store) {
    gateup_compute_src<KG, F, SC>(
        b, rb, lane,
        [&](int c, HI8& o, float& f) {
            o = xa[c];
            f = xs[c];
        },
        h_out, kgi, store);
}

// Group-limited top-k of the token from s and sb (written by the router
// blocks with device-scope atomic stores, read back the same way), on one
// wave: lane j < K receives the j-th choice, its weight and
// its blob from the table (null without a table, and in lanes >= K).  The
// table entries of the lane's own experts are fetched beside its scores, so
// resolving the blobs costs no dependent load.
// The top-k of route_token from the lane's scores and table entries
// (experts lane * EPL .. lane * EPL + EPL - 1).
template <int EPL>
__device__ __forceinline__ void route_values(const DecodeArgs& a, int lane, const float (&sv)[EPL],
                                             const float (&key)[EPL], const uint8_t* const (&tab)[EPL], int* id,
                                             float* w, const uint8_t** blob) {
    wave_group_topk_values<EPL>(sv, key, a.E, a.G, a.TG, a.K, a.rsf, a.top_p, lane, id, w);
    // lane j < K: the blob of its choice, held by lane id / EPL (none for a
    // choice the top-p cut dropped)
    const bool chosen = lane < a.K && *id >= 0;
    const int owner = chosen ? *id / EPL : 0, idx = chosen ? *id % EPL : -1;
    const uint8_t* b = nullptr;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const uint8_t* t = shfl_ptr(tab[i], owner);
        if (i == idx) b = t;
    }
    *blob = chosen ? b : nullptr;
    if (a.kept) {
        // the kept routed slots, in increasing order, for the gate/up launch
        const unsigned long long m = __ballot(chosen);
        if (chosen) a.kept[1 + __popcll(m & ((1ull << lane) - 1))] = lane;
        if (lane == 0) a.kept[0] = __popcll(m);
    }
}

template <int EPL>
__device__ __forceinline__ void route_token(const DecodeArgs& a, int lane, int* id, float* w, const uint8_t** blob) {
    float sv[EPL], key[EPL];
    const uint8_t* tab[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        sv[i] = e < a.E ? __hip_atomic_load(a.s + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;
        key[i] = e < a.E ? __hip_atomic_load(a.sb + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : -__builtin_inff();
        tab[i] = a.table && e < a.E ? a.table[e] : nullptr;
    }
    route_values<EPL>(a, lane, sv, key, tab, id, w, blob);
}

// ---------------------------------------------------------------- kernel 1
// Three kinds of workgroups in one launch (the first two stream HBM side by
// side, so the routing's serial tail overlaps the shared expert's weights):
//  * router blocks [0, router_blocks(E)): W_r rows (one per wave by default),
//    logit[e] = sum_h W_r[e][h] x[h] in fp32 (fixed-order sums), turned into
//    s and sb.  The block that takes the last ticket of a device-scope
//    counter derives the group-limited top-k and writes ids, w and the
//    routed slots' blobs, then resets the counter;
//  * the next shared_blocks blocks: gate/up + SwiGLU of the shared expert
//    (it does not depend on the routing), each wave converting the
//    activations for itself;
//  * the last block: the activations' integer operands for the routed
//    experts' kernel.
template <int KG>
__host__ __device__ inline int shared_gateup_blocks(int I) {  // I: stored rows of gate
    const int per_slot = I / GateUpShape<KG>::R;
    return (per_slot + 4 * kSharedItemsPerRound - 1) / (4 * kSharedItemsPerRound);
}

template <int KG, int EPL, int F>
__global__ void __launch_bounds__(256) router_kernel(DecodeArgs a) {
    using S = GateUpShape<KG>;
    // items per round of the shared expert's waves (two planes: two items)
    constexpr int NI = code_planes(F) > 1 ? 2 : kSharedItemsPerRound;
    const int lane = threadIdx.x & 63;
    const int wave = wave_in_block();
    const int n_shared_blocks = a.S > 0 ? shared_gateup_blocks<KG>(a.I / row_pack(F)) : 0;
    const int n_router_blocks = router_blocks(a.E);
    const int b = blockIdx.x;
    if (b >= n_router_blocks + n_shared_blocks) {
        // activations -> integer operands for the routed experts' kernel
        if (wave != 0) return;
        HI8 xa[S::CPL];
        float xs[S::CPL];
        convert_activations<KG, F>(a.x, lane, xa, xs);
        store_activations<KG>(a.xq, lane, xa, xs);
        return;
    }
    if (b >= n_router_blocks) {
        // shared expert gate/up: items of R rows, rounds of NI per wave
        const int per_slot = a.I / row_pack(F) / S::R;
        const int wave_id = (b - n_router_blocks) * 4 + wave;
        const int n_waves = n_shared_blocks * 4;
        if (wave_id >= per_slot) return;
        const BlobLayout L = blob_layout(a.H, a.I, F);
        GateUpBuf<KG, F> buf[NI];
#pragma unroll
        for (int k = 0; k < NI; ++k) {
            const int it = wave_id + k * n_waves;
            gateup_issue<KG, F>(a.shared_blob, L, it < per_slot ? it : per_slot - 1, lane, buf[k]);
        }
        HI8 xa[S::CPL];
        float xs[S::CPL];
        convert_activations<KG, F>(a.x, lane, xa, xs);
        float* h = a.h + (size_t)a.K * a.I;
#pragma unroll
        for (int k = 0; k < NI; ++k) {
            const int it = wave_id + k * n_waves;
            gateup_compute<KG, F>(buf[k], it < per_slot ? it : per_slot - 1, lane, xa, xs, h, a.I / 32, it < per_slot);
        }
        for (int base = wave_id + NI * n_waves; base < per_slot; base += NI * n_waves) {
#pragma unroll
            for (int k = 0; k < NI; ++k) {
                const int it = base + k * n_waves;
                gateup_issue<KG, F>(a.shared_blob, L, it < per_slot ? it : per_slot - 1, lane, buf[k]);
            }
#pragma unroll
            for (int k = 0; k < NI; ++k) {
                const int it = base + k * n_waves;
                gateup_compute<KG, F>(buf[k], it < per_slot ? it : per_slot - 1, lane, xa, xs, h, a.I / 32, it < per_slot);
            }
        }
        return;
    }
    // router rows: kRouterWavesPerRow waves per row, wave q of a row taking
    // chunks c = q, q + kRouterWavesPerRow, ... (lane l covering floats
    // [4l + 256c, +4)); fixed-order sums (per wave, then over the row's waves)
    constexpr int CR = KG / 8;  // 16-byte chunks per lane of a row
    constexpr int WPR = kRouterWavesPerRow;
    constexpr int NC = (CR + WPR - 1) / WPR;
    const int e = b * (4 / WPR) + wave / WPR;
    const int q = wave % WPR;
    float acc = 0.0f;
    if (e < a.E) {
        const float* row = a.router_w + (size_t)e * a.H;
        f32x4 wv[NC];
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int c = q + k * WPR;
            if (c < CR) wv[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + 4 * lane + 256 * c));
        }
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int c = q + k * WPR;
            if (c < CR) {
                const u32x2 xb = *reinterpret_cast<const u32x2*>(a.x + 4 * lane + 256 * c);
                acc = fmaf(wv[k][0], __builtin_bit_cast(float, xb[0] << 16), acc);
                acc = fmaf(wv[k][1], __builtin_bit_cast(float, xb[0] & 0xFFFF0000u), acc);
                acc = fmaf(wv[k][2], __builtin_bit_cast(float, xb[1] << 16), acc);
                acc = fmaf(wv[k][3], __builtin_bit_cast(float, xb[1] & 0xFFFF0000u), acc);
            }
        }
        acc = wave_sum(acc);
    }
    if constexpr (WPR > 1) {
        __shared__ float part[4];
        if (lane == 0) part[wave] = acc;
        __syncthreads();
        if (q == 0) {
            acc = part[wave];
#pragma unroll
            for (int j = 1; j < WPR; ++j) acc += part[wave + j];
        }
    }
    // Hand-off of the scores to the last router block without cache-wide
    // fences: the scores are written and read with device-scope atomic
    // accesses (coherent across the XCDs' L2s), every wave waits until its
    // stores are acknowledged before the workgroup takes its ticket, so a
    // block that draws the last ticket sees every score.  (A release fence
    // would also write back the whole L2, about 1 us per router block.)
    if (e < a.E && q == 0 && lane == 0) {
        const float sv = 1.0f / (1.0f + expf(-acc));
        __hip_atomic_store(a.s + e, sv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.sb + e, sv + a.bias[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __shared__ int is_last;
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned ticket = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = ticket == (unsigned)(n_router_blocks - 1);
        if (last) a.counter[0] = 0u;  // ready for the next call (the launch boundary publishes it)
        is_last = last;
    }
    __syncthreads();
    if (!is_last || wave != 0) return;
    int id;
    float w;
    const uint8_t* blob;
    route_token<EPL>(a, lane, &id, &w, &blob);
    if (lane < a.K) {
        a.ids[lane] = id;
        a.w[lane] = w;
        if (a.table) a.slot_blobs[lane] = blob;
    }
}

// The routed gate/up items of one wave: items wave_id, wave_id + n_waves,
// ... of n_items (wave_id < n_items).  kept is the wave's LDS copy of the
// kept-slot list (read when a.kept is set) and blobs a 16-entry LDS row
// that receives the slots' blobs.  With SC the h values are stored with
// device-scope atomic stores, for workgroups of the same launch to read.
template <int KG, int F, bool SC>
__device__ __forceinline__ void routed_gateup_wave(const DecodeArgs& a, int lane, int wave_id, int n_waves,
                                                   int n_items, const int* kept, const uint8_t** blobs) {
    using S = GateUpShape<KG>;
    constexpr int NI = kGateUpItemsPerRound;
    const BlobLayout L = blob_layout(a.H, a.I, F);
    const int per_slot = a.I / row_pack(F) / S::R;

    // Small dependent inputs first (vector loads complete in order, so
    // waiting for them must not mean waiting for weight streams issued
    // before them): activation operands, the routed blobs.
    HI8 xa[S::CPL];
    float xs[S::CPL];
    load_activations<KG>(a.xq, lane, xa, xs);
    // The slot -> blob table goes to this wave's LDS row: looking it up per
    // item then waits only on the LDS counter, whereas reading a register
    // that a global load filled earlier can make the compiler drain every
    // outstanding weight load first.
    if (lane < 16)
        blobs[lane] = a.direct ? lane_pick(a.blobs, lane) : (lane < a.K ? a.slot_blobs[lane] : nullptr);
    __builtin_amdgcn_wave_barrier();
    // Settle the activation registers here, once: an empty asm that reads
    // and rewrites each of them makes the compiler wait for their loads at
    // this point and treat them as ready afterwards, instead of re-waiting
    // for them behind weight loads.
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        asm volatile("" : "+v"(xa[c].he), "+v"(xa[c].ho), "+v"(xa[c].le), "+v"(xa[c].lo));
        asm volatile("" : "+v"(xa[c].corr), "+v"(xs[c]));
    }
    GateUpBuf<KG, F> b[NI];

    // item -> (slot, row block)
    auto slot_of = [&](int item) {
        const int k = item / per_slot;
        int s = k;
        if (a.kept) {
            s = kept[1 + k];
        } else if (a.use_slot_list) {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (j == k) s = a.slot_list[j];
        }
        return s;
    };
    auto rb_of = [&](int item) { return item % per_slot; };
    auto blob_of = [&](int slot) { return blobs[slot]; };
    auto issue = [&](int item, GateUpBuf<KG, F>& buf) {
        const int it = item < n_items ? item : n_items - 1;
        gateup_issue<KG, F>(blob_of(slot_of(it)), L, rb_of(it), lane, buf);
    };
    auto compute = [&](int item, const GateUpBuf<KG, F>& buf) {
        const int it = item < n_items ? item : n_items - 1;
        gateup_compute<KG, F, SC>(buf, rb_of(it), lane, xa, xs, a.h + (size_t)slot_of(it) * a.I, a.I / 32, item < n_items);
    };

    // One to four items for this wave (every wave gets four at 4 x 4096
    // items, three when the top-p cut keeps 6 of 8 slots, ...): a
    // straight-line two-buffer pipeline for each count keeps one item's loads
    // in flight while the other is computed, and loads nothing beyond the
    // wave's own items.
    const int n_mine = (n_items - wave_id + n_waves - 1) / n_waves;
    if (NI == 2 && n_mine <= 4) {
        const int i0 = wave_id, i1 = wave_id + n_waves, i2 = wave_id + 2 * n_waves, i3 = wave_id + 3 * n_waves;
        if (n_mine == 4) {
            issue(i0, b[0]);
            issue(i1, b[1]);
            compute(i0, b[0]);
            issue(i2, b[0]);
            compute(i1, b[1]);
            issue(i3, b[1]);
            compute(i2, b[0]);
            compute(i3, b[1]);
        } else if (n_mine == 3) {
            issue(i0, b[0]);
            issue(i1, b[1]);
            compute(i0, b[0]);
            issue(i2, b[0]);
            compute(i1, b[1]);
            compute(i2, b[0]);
        } else if (n_mine == 2) {
            issue(i0, b[0]);
            issue(i1, b[1]);
            compute(i0, b[0]);
            compute(i1, b[1]);
        } else {
            issue(i0, b[0]);
            compute(i0, b[0]);
        }
        return;
    }
    // Rounds of NI items: issue the round's loads, then compute it (the
    // other waves of the SIMD overlap their loads with this compute).
#pragma unroll
    for (int k = 0; k < NI; ++k) issue(wave_id + k * n_waves, b[k]);
#pragma unroll
    for (int k = 0; k < NI; ++k) compute(wave_id + k * n_waves, b[k]);
    for (int base = wave_id + NI * n_waves; base < n_items; base += NI * n_waves) {
#pragma unroll
        for (int k = 0; k < NI; ++k) issue(base + k * n_waves, b[k]);
#pragma unroll
        for (int k = 0; k < NI; ++k) compute(base + k * n_waves, b[k]);
    }
}

// ---------------------------------------------------------------- kernel 2
// Items: (routed slot, block of R rows); blobs from the router's top-k, or
// given directly by the expert cache.  A wave takes items wave_id + j *
// n_waves in rounds of NI, in straight-line code (items past the end are
// clamped to the last item and their results not stored), so the
// compiler's wait counts stay exact.
template <int KG, int F>
__global__ void __launch_bounds__(256) gateup_kernel(DecodeArgs a) {
    using S = GateUpShape<KG>;
    const int lane = threadIdx.x & 63;
    const int wave = wave_in_block();
    const int wave_id = blockIdx.x * 4 + wave;
    const int n_waves = gridDim.x * 4;
    const int per_slot = a.I / row_pack(F) / S::R;
    // With the router's kept-slot list (top-p cut) the items cover only the
    // kept slots; the list goes to this wave's LDS row.
    // (the slot count from the arguments first, so that all argument loads
    // go out together before the kept-list branch)
    __shared__ int wave_kept[4][17];
    int n_routed_slots = a.use_slot_list ? a.n_slot_list : a.K;
    if (a.kept) {
        if (lane < 17) wave_kept[wave][lane] = lane <= a.K ? a.kept[lane] : 0;
        __builtin_amdgcn_wave_barrier();
        n_routed_slots = wave_kept[wave][0];
    }
    const int n_items = n_routed_slots * per_slot;
    if (wave_id >= n_items) return;
    __shared__ const uint8_t* wave_blobs[4][16];
    routed_gateup_wave<KG, F, false>(a, lane, wave_id, n_waves, n_items, wave_kept[wave], wave_blobs[wave]);
}

// ---------------------------------------------------------------- kernel 3
template <int KG, int NLD>
struct DownShape {
    static constexpr int CPL = chunks_per_lane(KG);
    static constexpr int RPL = rows_per_load(KG);
    static constexpr int NL = NLD;          // wave-load steps per chunk column
    static constexpr int R = NL * RPL;      // rows per workgroup
    static constexpr int B = KG >= kWave ? 6 : ilog2(KG);
    static constexpr int WIN = NL < 8 ? NL : 8;  // load steps per round
};

// h of one slot, this lane's groups (32 floats per chunk column), stored
// in h_index order so that every load is 64 lanes x 16 contiguous bytes.
template <int CPL, int KG>
__device__ __forceinline__ void load_h(const float* __restrict__ h, int g0, float (&hv)[CPL][32]) {
    constexpr int G = KG < kWave ? KG : kWave;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(h + ((size_t)(c * 8 + q) * G + g0) * 4);
            hv[c][4 * q + 0] = t[0];
            hv[c][4 * q + 1] = t[1];
            hv[c][4 * q + 2] = t[2];
            hv[c][4 * q + 3] = t[3];
        }
    }
}

// Down-projection work of one wave: one slot's blob over the R rows of row
// block rb.  Code loads go in rounds of WIN steps; compute_round folds a
// round into the per-step partials v, store_part reduces them over the
// lanes into the workgroup's part row of this slot.
template <int KG, int NLD, int F>
struct DownWork {
    using S = DownShape<KG, NLD>;
    static constexpr int WIN = S::WIN;
    static constexpr int NR = (S::NL + WIN - 1) / WIN;  // rounds
    static constexpr int RP = row_pack(F);               // matrix rows per stored row (int2: 2)
    static constexpr int P = code_planes(F);
    static constexpr int NVP = pow2_at_least(S::NL * RP);
    const uint8_t* blob;
    BlobLayout L;
    int rb, g0, row_sub;
    u32x4 code[S::NL][S::CPL][P];
    unsigned sc[RP][S::CPL][(S::NL + 1) / 2];

    __device__ __forceinline__ void init(const uint8_t* b, int H, int I, int block, int lane) {
        blob = b;
        L = blob_layout(H, I, F);
        rb = block;
        g0 = KG >= kWave ? lane : (lane & (KG - 1));
        row_sub = KG >= kWave ? 0 : (lane / KG);
    }
    __device__ __forceinline__ void init(const uint8_t* b, const DecodeArgs& a, int block, int lane) {
        init(b, a.H, a.I, block, lane);
    }
    __device__ __forceinline__ size_t code_off(int step, int c) const {
        const size_t row = (size_t)rb * S::R + step * S::RPL + row_sub;
        return (row * KG + g0 + kWave * c) * 16;
    }
    __device__ __forceinline__ void issue_round(int r) {
#pragma unroll
        for (int n = r * WIN; n < (r + 1) * WIN && n < S::NL; ++n)
#pragma unroll
            for (int c = 0; c < S::CPL; ++c)
#pragma unroll
                for (int p = 0; p < P; ++p)
                    code[n][c][p] = load_stream16(blob + (p ? L.down_lo : L.down_q) + code_off(n, c));
    }
    __device__ __forceinline__ void load_scales() {
#pragma unroll
        for (int h = 0; h < RP; ++h)
#pragma unroll
            for (int c = 0; c < S::CPL; ++c) {
                const size_t si = ((size_t)rb * KG + g0 + kWave * c) * S::R + (size_t)row_sub * S::NL;
                load_scales_c<F, S::NL>(blob + (h ? L.down_s2 : L.down_s) + si * scale_bytes(F), sc[h][c]);
            }
    }
    __device__ __forceinline__ void compute_round(int r, const HI8 (&ha)[S::CPL], const float (&hscale)[S::CPL],
                                                  float (&v)[NVP]) const {
#pragma unroll
        for (int n = r * WIN; n < (r + 1) * WIN && n < S::NL; ++n) {
            if constexpr (F == kCodecInt2) {
                float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
                for (int c = 0; c < S::CPL; ++c) {
                    float d0, d1;
                    dot_chunk_int2(code[n][c][0], ha[c], d0, d1);
                    acc0 = fmaf(scale_at<F>(sc[0][c], n) * hscale[c], d0, acc0);
                    acc1 = fmaf(scale_at<F>(sc[RP - 1][c], n) * hscale[c], d1, acc1);
                }
                v[n] = acc0;
                v[S::NL + n] = acc1;
            } else {
                float acc = 0.0f;
#pragma unroll
                for (int c = 0; c < S::CPL; ++c)
                    acc = fmaf(scale_at<F>(sc[0][c], n) * hscale[c], dot_planes<F>(code[n][c], ha[c]), acc);
                v[n] = acc;
            }
        }
    }
    // part[row parity * R + stored row of the block]
    __device__ __forceinline__ void store_part(float (&v)[NVP], int lane, float* part) const {
        const float r = reduce_scatter<NVP, S::B>(v, lane);
        const int low_bits = S::B - ilog2(NVP);
        const int vi = (lane >> low_bits) & (NVP - 1);
        // value index: row parity, then step
        if ((lane & ((1 << low_bits) - 1)) == 0 && vi < RP * S::NL)
            part[(vi / S::NL) * S::R + (vi % S::NL) * S::RPL + row_sub] = r;
    }
    // Every round already issued: h to operands, the rounds computed in order.
    __device__ __forceinline__ void finish_issued(const float (&hraw)[S::CPL][32], int lane, float* part) {
        HI8 ha[S::CPL];
        float hscale[S::CPL];
        to_operands<F, S::CPL>(hraw, ha, hscale);
        float v[NVP];
#pragma unroll
        for (int n = 0; n < NVP; ++n) v[n] = 0.0f;
#pragma unroll
        for (int r = 0; r < NR; ++r) compute_round(r, ha, hscale, v);
        store_part(v, lane, part);
    }
    // The whole row block after the first rounds were issued: h to operands,
    // the rounds computed in order with round r + 2 issued after round r.
    __device__ __forceinline__ void finish(const float (&hraw)[S::CPL][32], int lane, float* part) {
        HI8 ha[S::CPL];
        float hscale[S::CPL];
        to_operands<F, S::CPL>(hraw, ha, hscale);
        float v[NVP];
#pragma unroll
        for (int n = 0; n < NVP; ++n) v[n] = 0.0f;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            __builtin_amdgcn_sched_barrier(0);
            compute_round(r, ha, hscale, v);
            __builtin_amdgcn_sched_barrier(0);
            if (r + 2 < NR) issue_round(r + 2);
        }
        store_part(v, lane, part);
    }
};

// One workgroup = one wave per slot (the routed slots, then the shared
// expert) over a block of R output rows.  Row loads go in rounds of WIN
// steps, the next round issued before the current one is computed
// (sched_barrier keeps that order); the first R threads combine the block in
// slot order.  Nine waves of at most 170 registers fit one CU.
template <int KG, int NLD, int F>
__global__ void __launch_bounds__(576) down_combine_kernel(DecodeArgs a) {
    using S = DownShape<KG, NLD>;
    using D = DownWork<KG, NLD, F>;
    constexpr int MAXW = 9;
    constexpr int RP = D::RP;
    const int lane = threadIdx.x & 63;
    const int slot = wave_in_block();
    const int K = a.K;
    const int g0 = KG >= kWave ? lane : (lane & (KG - 1));
    const int rb = blockIdx.x;
    const uint8_t* blob = slot >= K ? a.shared_blob
                                    : (a.direct ? readlane_ptr(lane_pick(a.blobs, lane), slot) : a.slot_blobs[slot]);
    __shared__ float part[MAXW][RP * S::R];  // [slot][row parity * R + stored row of the block]
    // h does not depend on the blob: its loads go out before the blob
    // pointer arrives (a dropped slot's h is stale workspace and unused)
    float hraw[S::CPL][32];
    load_h<S::CPL, KG>(a.h + (size_t)slot * a.I, g0, hraw);
    asm volatile("" ::: "memory");  // keeps the h loads here (not sunk into the branch)
    if (blob == nullptr) {
        // a routed slot that the top-p cut dropped: weight 0, nothing read
        for (int t = lane; t < RP * S::R; t += kWave) part[slot][t] = 0.0f;
    } else {
        D d;
        d.init(blob, a, rb, lane);
        __builtin_amdgcn_sched_barrier(0);
        d.issue_round(0);
        d.load_scales();
        if constexpr (D::NR > 1) d.issue_round(1);
        __builtin_amdgcn_sched_barrier(0);
        d.finish(hraw, lane, part[slot]);
    }
    __syncthreads();
    if ((int)threadIdx.x < RP * S::R) {
        const int t = threadIdx.x;
        float y = 0.0f;
        for (int j = 0; j < K; ++j) y = fmaf(a.w[j], part[j][t], y);
        if (a.S > 0) y += part[K][t];
        a.y[(size_t)RP * (rb * S::R + t % S::R) + t / S::R] = y;
    }
}

// ---------------------------------------------------------------- single-entry experts of batched calls
// An expert that exactly one entry of a batched call routes to (the
// dispatch's singles list, calls with 16-entry tiles) skips the grouped MFMA
// kernels, whose tile it would fill to one sixteenth: its gate/up and down
// run as the GEMVs above, one (token, expert) pair at a time.

// Gate/up + SwiGLU of the singles: the grid's waves are spread evenly over
// the pairs (waves_per_pair = waves / pairs); wave sub of a pair takes items
// (blocks of R rows) sub, sub + waves_per_pair, ... with two items' loads in
// flight, after converting the pair's token into integer operands itself.
// h goes to the pair's row of the batched h buffer in the order
// pair_down_kernel's lanes read it (h_index).
template <int KG, int F>
__global__ void __launch_bounds__(256) pair_gateup_kernel(BatchArgs a) {
    using S = GateUpShape<KG>;
    const int n = a.n_singles[0];
    if (n == 0) return;
    const int lane = threadIdx.x & 63;
    const int wave_id = blockIdx.x * 4 + wave_in_block();
    const int n_waves = gridDim.x * 4;
    const int wpp = n_waves >= n ? n_waves / n : 1;
    const int j = wave_id / wpp, sub = wave_id - j * wpp;
    const int per_slot = a.I / row_pack(F) / S::R;
    if (j >= n || sub >= per_slot) return;
    const int n_mine = (per_slot - sub + wpp - 1) / wpp;
    const Tile t = a.singles[j];
    const int p = t.first_pair;
    const uint8_t* blob = a.table[t.expert];
    const BlobLayout L = blob_layout(a.H, a.I, F);
    HI8 xa[S::CPL];
    float xs[S::CPL];
    convert_activations_by_column<KG, F>(a.x + (size_t)(a.perm[p] / a.K) * a.H, lane, xa, xs);
    // settle the operands once (as in gateup_kernel), so that no later
    // weight load waits on them
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        asm volatile("" : "+v"(xa[c].he), "+v"(xa[c].ho), "+v"(xa[c].le), "+v"(xa[c].lo));
        asm volatile("" : "+v"(xa[c].corr), "+v"(xs[c]));
    }
    float* h = a.h + (size_t)p * a.I;
    GateUpBuf<KG, F> b[2];
    // items past the wave's last repeat its last item (loads from L2, nothing stored)
    auto rb_of = [&](int k) { return sub + (k < n_mine ? k : n_mine - 1) * wpp; };
    run_items_loop<2>(
        n_mine, [&](int k, GateUpBuf<KG, F>& buf) { gateup_issue<KG, F>(blob, L, rb_of(k), lane, buf); },
        [&](int k, const GateUpBuf<KG, F>& buf) {
            gateup_compute<KG, F>(buf, rb_of(k), lane, xa, xs, h, a.I / 32, k < n_mine);
        },
        b);
}

// Down projection of the singles: one wave per (pair, block of R output
// rows) item, taken in turn by the grid's waves; the wave loads the pair's h
// and converts it to integer operands, streams the block's rows as
// down_combine_kernel does, and writes the R results to the pair's row of
// the per-entry output d (the batched combine applies the routing weight).
template <int KG, int NLD, int F>
__global__ void __launch_bounds__(256) pair_down_kernel(BatchArgs a) {
    using S = DownShape<KG, NLD>;
    using D = DownWork<KG, NLD, F>;
    constexpr int RP = D::RP;
    __shared__ float part[4][RP * S::R];
    const int n = a.n_singles[0];
    const int lane = threadIdx.x & 63, wv = wave_in_block();
    const int g0 = KG >= kWave ? lane : (lane & (KG - 1));
    const int rblocks = a.H / RP / S::R;
    const int items = n * rblocks;
    for (int it = blockIdx.x * 4 + wv; it < items; it += gridDim.x * 4) {
        const int j = it / rblocks, rb = it - j * rblocks;
        const Tile t = a.singles[j];
        const int p = t.first_pair;
        float hraw[S::CPL][32];
        load_h<S::CPL, KG>(a.h + (size_t)p * a.I, g0, hraw);
        D d;
        d.init(a.table[t.expert], a.H, a.I, rb, lane);
        __builtin_amdgcn_sched_barrier(0);
        d.issue_round(0);
        d.load_scales();
        if constexpr (D::NR > 1) d.issue_round(1);
        __builtin_amdgcn_sched_barrier(0);
        d.finish(hraw, lane, part[wv]);
        __builtin_amdgcn_wave_barrier();
        for (int q = lane; q < RP * S::R; q += kWave)
            a.d[(size_t)p * a.H + (size_t)RP * (rb * S::R + q % S::R) + q / S::R] = part[wv][q];
        __builtin_amdgcn_wave_barrier();
    }
}

// ---------------------------------------------------------------- fused decode
// One launch per token running the three stages above on workgroups that
// are all resident at once, with the two hand-offs done inside the kernel.
// A workgroup has one wave per routed slot (K waves, two per SIMD for
// K = 8) and owns the down rows of one row block:
//   phase 0  router rows (one W_r row per wave, as router_kernel), each
//            score published as a (value, call number) record, and the
//            shared expert's gate/up items, spread over every wave; the
//            token's activation operands are converted once per
//            workgroup into LDS;
//   routing  wave 0 polls the score records until all E carry this call's
//            number and runs the group-limited top-k (every workgroup
//            derives the same routing); workgroup 0 writes ids and w;
//   phase 1  the routed gate/up items, the same number per wave;
//   phase 2  wave w: the down rows of slot w over the block, and the shared
//            expert's rows of the block congruent to w modulo K; all code
//            loads are issued, then the workgroup waits until every
//            workgroup has published its h values, reads h and finishes.
// Hand-off data (score records, h) is written with device-scope atomic
// stores; h writers wait for the stores' acknowledgement (s_waitcnt) before
// a device-scope counter increment, and readers poll, then read with
// device-scope loads.  Every value is computed exactly as on the
// three-launch path (the shared expert's rows sit at the same places of the
// same wave reduction), so both paths give bit-identical results.
//
// Global wave index gw = wave * grid + block: consecutive work units land on
// different workgroups (and CUs), so a ragged last round spreads over the
// chip.

// Adds one to a spread count (contribution index i).
__device__ __forceinline__ void count_up(unsigned* ctr, int i) {
    __hip_atomic_fetch_add(ctr + (i % kSyncCounters) * kSyncStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls a spread count until its words sum to target (one device-scope load
// per lane, a wave sum); false after limit polls.  Called by a whole wave.
__device__ __forceinline__ bool wait_count(const unsigned* ctr, unsigned target, unsigned limit, int lane) {
    for (unsigned i = 0; i < limit; ++i) {
        unsigned v = lane < kSyncCounters
                         ? __hip_atomic_load(ctr + lane * kSyncStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : 0u;
#pragma unroll
        for (int o = 1; o < kSyncCounters; o <<= 1) v += __shfl_xor(v, o);
        if (__builtin_amdgcn_readfirstlane(v) == target) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// Chunk column c of the token's activation operands (the values
// convert_activations gives), converted by one wave into LDS in
// structure-of-arrays order: xo[c][q][lane] (he, ho, le, lo) and
// xm[c][lane] (corr, factor).
template <int KG, int F>
__device__ __forceinline__ void convert_column_to_lds(const uint16_t* __restrict__ x, int lane, int c, u32x4* xo,
                                                      u32x2* xm) {
    const int g0 = KG >= kWave ? lane : (lane & (KG - 1));
    const uint16_t* xg = x + 32 * (g0 + kWave * c);
    float xv[1][32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(xg + 8 * q);
#pragma unroll
        for (int z = 0; z < 4; ++z) {
            const unsigned d = raw[z];
            xv[0][8 * q + 2 * z] = __builtin_bit_cast(float, d << 16);
            xv[0][8 * q + 2 * z + 1] = __builtin_bit_cast(float, d & 0xFFFF0000u);
        }
    }
    HI8 one[1];
    float one_s[1];
    to_operands<F, 1>(xv, one, one_s);
    xo[(c * 4 + 0) * kWave + lane] = one[0].he;
    xo[(c * 4 + 1) * kWave + lane] = one[0].ho;
    xo[(c * 4 + 2) * kWave + lane] = one[0].le;
    xo[(c * 4 + 3) * kWave + lane] = one[0].lo;
    xm[c * kWave + lane] = u32x2{(unsigned)one[0].corr, __builtin_bit_cast(unsigned, one_s[0])};
}

// Operand source reading column c of the LDS copy (gateup_compute_src).
struct LdsOperands {
    const u32x4* xo;
    const u32x2* xm;
    int lane;
    __device__ __forceinline__ void operator()(int c, HI8& o, float& f) const {
        o.he = xo[(c * 4 + 0) * kWave + lane];
        o.ho = xo[(c * 4 + 1) * kWave + lane];
        o.le = xo[(c * 4 + 2) * kWave + lane];
        o.lo = xo[(c * 4 + 3) * kWave + lane];
        const u32x2 m = xm[c * kWave + lane];
        // elements go through named scalars: this compiler bit-casts a vector
        // element operand (m[1]) as element 0
        const unsigned m0 = m[0], m1 = m[1];
        o.corr = (int)m0;
        f = __builtin_bit_cast(float, m1);
    }
};

// A score record: the value's bits in the low word, the call number in the
// high word, written and read as one 8-byte device-scope atomic.
__device__ __forceinline__ unsigned long long score_record(float v, unsigned seq) {
    return ((unsigned long long)seq << 32) | __builtin_bit_cast(unsigned, v);
}

// One router row as in router_kernel (one wave per row): the loads, then
// the fixed-order sum, published as records of s and sb.
template <int KG>
struct RouterRow {
    static constexpr int CR = KG / 8;  // 16-byte chunks per lane of a row
    f32x4 wv[CR];
    __device__ __forceinline__ void issue(const DecodeArgs& a, int e, int lane) {
        const float* row = a.router_w + (size_t)e * a.H;
#pragma unroll
        for (int c = 0; c < CR; ++c)
            wv[c] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + 4 * lane + 256 * c));
    }
    __device__ __forceinline__ void finish(const DecodeArgs& a, const FusedArgs& f, int e, int lane) {
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < CR; ++c) {
            const u32x2 xb = *reinterpret_cast<const u32x2*>(a.x + 4 * lane + 256 * c);
            acc = fmaf(wv[c][0], __builtin_bit_cast(float, xb[0] << 16), acc);
            acc = fmaf(wv[c][1], __builtin_bit_cast(float, xb[0] & 0xFFFF0000u), acc);
            acc = fmaf(wv[c][2], __builtin_bit_cast(float, xb[1] << 16), acc);
            acc = fmaf(wv[c][3], __builtin_bit_cast(float, xb[1] & 0xFFFF0000u), acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) {
            const float sv = 1.0f / (1.0f + expf(-acc));
            // system scope on both sides: the record goes past every cache
            // and the polls read it there
            __hip_atomic_store(f.s_rec + e, score_record(sv, f.seq), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(f.sb_rec + e, score_record(sv + a.bias[e], f.seq), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
};

// The token's routing on one wave from the score records: polls until every
// record of the lane's experts carries this call's number (system-scope
// loads, which no cache line of an earlier poll can satisfy), then runs the
// top-k.  False if the records were not all there within the spin limit.
template <int EPL>
__device__ __forceinline__ bool route_from_records(const DecodeArgs& a, const FusedArgs& f, int lane, int* id,
                                                   float* w, const uint8_t** blob) {
    const uint8_t* tab[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        tab[i] = e < a.E ? a.table[e] : nullptr;
    }
    float sv[EPL], key[EPL];
    bool ok = false;
    for (unsigned it = 0; it < f.spin_limit && !ok; ++it) {
        bool mine = true;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane * EPL + i;
            if (e < a.E) {
                const unsigned long long rs = __hip_atomic_load(f.s_rec + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                const unsigned long long rb = __hip_atomic_load(f.sb_rec + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                mine = mine && (unsigned)(rs >> 32) == f.seq && (unsigned)(rb >> 32) == f.seq;
                sv[i] = __builtin_bit_cast(float, (unsigned)rs);
                key[i] = __builtin_bit_cast(float, (unsigned)rb);
            } else {
                sv[i] = 0.0f;
                key[i] = -__builtin_inff();
            }
        }
        ok = __ballot(!mine) == 0ull;
        if (!ok) __builtin_amdgcn_s_sleep(1);
    }
    DecodeArgs ar = a;
    ar.kept = nullptr;
    route_values<EPL>(ar, lane, sv, key, tab, id, w, blob);
    return ok;
}

// h of one slot read with device-scope atomic loads of 8 bytes (written in
// this launch by workgroups on other XCDs), in the order of load_h.
template <int CPL, int KG>
__device__ __forceinline__ void load_h_device_scope(const float* h, int g0, float (&hv)[CPL][32]) {
    constexpr int G = KG < kWave ? KG : kWave;
    const uint64_t* h64 = reinterpret_cast<const uint64_t*>(h);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint64_t v = __hip_atomic_load(h64 + ((size_t)(c * 8 + q) * G + g0) * 2 + half, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                hv[c][4 * q + 2 * half] = __builtin_bit_cast(float, (unsigned)v);
                hv[c][4 * q + 2 * half + 1] = __builtin_bit_cast(float, (unsigned)(v >> 32));
            }
        }
    }
}

// Down rows of one slot over block rb owned by owner m of M (steps n with
// n mod M == m): their code loads, and their dot products placed at the
// value indices down_combine_kernel's wave for that slot uses, so that the
// same wave reduction gives the same sums (the other indices hold zeros,
// which leave every row's sum unchanged).
template <int KG, int NLD, int F, int M>
struct DownSteps {
    using S = DownShape<KG, NLD>;
    using D = DownWork<KG, NLD, F>;
    static constexpr int MAXOWN = (S::NL + M - 1) / M;
    static constexpr int P = code_planes(F);
    static_assert(row_pack(F) == 1, "one matrix row per stored row");
    u32x4 code[MAXOWN][S::CPL][P];
    unsigned sc[MAXOWN][S::CPL];
    __device__ __forceinline__ void issue(const uint8_t* blob, const BlobLayout& L, int rb, int lane, int m) {
        const int g0 = KG >= kWave ? lane : (lane & (KG - 1));
        const int row_sub = KG >= kWave ? 0 : (lane / KG);
#pragma unroll
        for (int i = 0; i < MAXOWN; ++i) {
            const int step = m + i * M;
            if (step < S::NL) {
                const size_t row = (size_t)rb * S::R + step * S::RPL + row_sub;
#pragma unroll
                for (int c = 0; c < S::CPL; ++c) {
#pragma unroll
                    for (int p = 0; p < P; ++p)
                        code[i][c][p] = load_stream16(blob + (p ? L.down_lo : L.down_q) + (row * KG + g0 + kWave * c) * 16);
                    // the step's scale inside the lane's run of NL scales
                    const size_t si = ((size_t)rb * KG + g0 + kWave * c) * S::R + (size_t)row_sub * S::NL + step;
                    if constexpr (F == kCodecMxfp4)
                        sc[i][c] = __builtin_nontemporal_load(as_global<uint8_t>(blob + L.down_s + si));
                    else
                        sc[i][c] = __builtin_nontemporal_load(as_global<uint16_t>(blob + L.down_s + 2 * si));
                }
            }
        }
    }
    __device__ __forceinline__ void finish(const float (&hraw)[S::CPL][32], int lane, int m, float* part) {
        HI8 ha[S::CPL];
        float hscale[S::CPL];
        to_operands<F, S::CPL>(hraw, ha, hscale);
        finish_ops(ha, hscale, lane, m, part);
    }
    // The same from h already converted to operands.
    __device__ __forceinline__ void finish_ops(const HI8 (&ha)[S::CPL], const float (&hscale)[S::CPL], int lane, int m,
                                               float* part) {
        float acc[MAXOWN];
#pragma unroll
        for (int i = 0; i < MAXOWN; ++i) {
            acc[i] = 0.0f;
            if (m + i * M < S::NL) {
#pragma unroll
                for (int c = 0; c < S::CPL; ++c) {
                    const float scale = F == kCodecMxfp4 ? e8m0_to_float(sc[i][c]) : half_bits_to_float(sc[i][c]);
                    acc[i] = fmaf(scale * hscale[c], dot_planes<F>(code[i][c], ha[c]), acc[i]);
                }
            }
        }
        // value j is step j: owned when j mod M == m
        float v[D::NVP];
#pragma unroll
        for (int j = 0; j < D::NVP; ++j) v[j] = (j < S::NL && j % M == m) ? acc[j / M] : 0.0f;
        const float r = reduce_scatter<D::NVP, S::B>(v, lane);
        const int low_bits = S::B - ilog2(D::NVP);
        const int vi = (lane >> low_bits) & (D::NVP - 1);
        const int row_sub = KG >= kWave ? 0 : (lane / KG);
        if ((lane & ((1 << low_bits) - 1)) == 0 && vi < S::NL && vi % M == m) part[vi * S::RPL + row_sub] = r;
    }
};

// gateup_issue through buffer loads on a resource over the blob; with live
// false the resource has no records, so every load returns zeros without
// touching memory (the same loads are issued either way, which keeps the
// compiler's load counts exact when a wave may run out of items).  For
// shapes whose rows span whole wave loads (one row per load) with one code
// plane and one row per stored row.
constexpr int kLoadNonTemporal = 2;  // cache-policy bits: nt
template <int KG, int F>
__device__ __forceinline__ void gateup_issue_buf(const uint8_t* blob, bool live, const BlobLayout& L, int rb, int lane,
                                                 GateUpBuf<KG, F>& b) {
    using S = GateUpShape<KG>;
    static_assert(S::RPL == 1 && code_planes(F) == 1 && row_pack(F) == 1, "one row per wave load");
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blob), (short)0, live ? 0x7FFFFFF0 : 0, 0x00020000);
    const int g0 = lane;
#pragma unroll
    for (int n = 0; n < S::NL; ++n) {
        const int row = rb * S::R + n;
#pragma unroll
        for (int c = 0; c < S::CPL; ++c) {
            const int off = (row * KG + g0 + kWave * c) * 16;
            b.cg[n][c][0] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)L.gate_q + off, 0, kLoadNonTemporal);
            b.cu[n][c][0] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)L.up_q + off, 0, kLoadNonTemporal);
        }
    }
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) {
        // the 2 NL gate and up scales of the lane's group, as in gateup_issue
        const int p = (int)L.gu_s + (rb * KG + g0 + kWave * c) * 2 * S::R * scale_bytes(F);
        static_assert(2 * S::NL * (F == kCodecMxfp4 ? 1 : 2) == 4, "one scale dword per chunk column");
        b.sgu[0][c][0] = __builtin_amdgcn_raw_buffer_load_b32(r, p, 0, kLoadNonTemporal);
    }
}

// A wave's N items with up to NB items' loads in flight: item k + NB is
// issued once item k is computed, in straight-line code (compile-time buffer
// choice keeps the compiler's load waits exact); nothing beyond the wave's
// own items is loaded.
template <int N, int NB, typename Issue, typename Compute, typename Buf>
__device__ __forceinline__ void run_items(const Issue& issue, const Compute& compute, Buf (&b)[NB]) {
#pragma unroll
    for (int k = 0; k < (N < NB ? N : NB); ++k) issue(k, b[k]);
#pragma unroll
    for (int k = 0; k < N; ++k) {
        compute(k, b[k % NB]);
        if (k + NB < N) issue(k + NB, b[k % NB]);
    }
}

// More items than the straight-line cases cover: two buffers in a loop;
// the pair after the last is clamped by the caller's issue (loads repeated,
// results not stored).
template <int NB, typename Issue, typename Compute, typename Buf>
__device__ __forceinline__ void run_items_loop(int n, const Issue& issue, const Compute& compute, Buf (&b)[NB]) {
    static_assert(NB >= 2, "two buffers");
    issue(0, b[0]);
    issue(1, b[1]);
#pragma unroll 1
    for (int k = 0; k < n; k += 2) {
        compute(k, b[0]);
        issue(k + 2, b[0]);
        compute(k + 1, b[1]);
        issue(k + 3, b[1]);
    }
}

constexpr int kFusedMaxSlots = 8;        // routed slots (top_k <= 8)
constexpr int kFusedWavesPerSlot = 1;    // waves per routed slot (one wave per slot: two per SIMD at top_k 8)
constexpr int kFusedItemsInFlight = 4;   // gate/up items per wave with loads in flight

template <int KG, int KGI, int NLD, int EPL, int F, int NK>
__global__ void __launch_bounds__(64 * kFusedWavesPerSlot * NK) fused_decode_kernel(DecodeArgs a, FusedArgs f) {
    using SG = GateUpShape<KG>;
    using SD = DownShape<KGI, NLD>;
    using D = DownWork<KGI, NLD, F>;
    const int lane = threadIdx.x & 63;
    const int wave = wave_in_block();
    constexpr int nw = kFusedWavesPerSlot * NK;  // waves per workgroup
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int gw = wave * G + b;
    const int NW = nw * G;
    const BlobLayout L = blob_layout(a.H, a.I, F);
    const int per_slot = a.I / row_pack(F) / SG::R;  // gate/up items per slot
    const int n_shared = a.S > 0 ? per_slot : 0;
    float* const h_shared = a.h + (size_t)a.K * a.I;

    __shared__ const uint8_t* s_blob[16];  // routed slot -> blob (null: dropped)
    __shared__ float s_w[16];
    __shared__ int s_kept[17];             // kept routed slots: count, then slots ascending
    __shared__ int s_fail;
    __shared__ int s_next;                 // next unclaimed gate/up item of this workgroup
    __shared__ float part[kFusedMaxSlots + 1][D::RP * SD::R];
    __shared__ u32x4 xo[SG::CPL * 4 * kWave];  // activation operands, converted once per workgroup
    __shared__ u32x2 xm[SG::CPL * kWave];
    const LdsOperands xsrc{xo, xm, lane};

    // ---- phase 0: a router row (waves with gw < E), shared gate/up items;
    // the loads go out before the activation columns are converted into LDS
    // (column c by wave nw - 1 - c mod nw: the last waves, which have no
    // phase-0 unit when units are fewer than waves)
    if (threadIdx.x == 0) {
        s_fail = 0;
        s_next = 0;
    }
    {
        // A router-row wave and an item wave keep their loads in separate
        // code paths (each with the workgroup's one barrier: a workgroup
        // barrier counts every wave that reaches any barrier instruction), so
        // the row's registers and the item's never overlap.
        const int n_units = a.E + n_shared;
        int u = gw;
        if (u < a.E) {
            RouterRow<KG> row;
            row.issue(a, u, lane);
            for (int c = nw - 1 - wave; c >= 0; c -= nw)
                if (c < SG::CPL) convert_column_to_lds<KG, F>(a.x, lane, c, xo, xm);
            __syncthreads();
            row.finish(a, f, u, lane);
            // further router rows (shapes with more rows than waves)
            for (u += NW; u < a.E; u += NW) {
                row.issue(a, u, lane);
                row.finish(a, f, u, lane);
            }
        } else {
            GateUpBuf<KG, F> buf;
            if (u < n_units) gateup_issue<KG, F>(a.shared_blob, L, u - a.E, lane, buf);
            for (int c = nw - 1 - wave; c >= 0; c -= nw)
                if (c < SG::CPL) convert_column_to_lds<KG, F>(a.x, lane, c, xo, xm);
            __syncthreads();
            if (u < n_units) {
                gateup_compute_src<KG, F, true>(buf, u - a.E, lane, xsrc, h_shared, a.I / 32, true);
                u += NW;
            }
        }
        // further shared items (shapes with more units than waves)
        for (; u < n_units; u += NW) {
            GateUpBuf<KG, F> buf;
            gateup_issue<KG, F>(a.shared_blob, L, u - a.E, lane, buf);
            gateup_compute_src<KG, F, true>(buf, u - a.E, lane, xsrc, h_shared, a.I / 32, true);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's shared h stores are acknowledged

    // ---- routing on wave 0
    if (wave == 0) {
        int id;
        float w;
        const uint8_t* blob;
        if (!route_from_records<EPL>(a, f, lane, &id, &w, &blob) && lane == 0) s_fail = 1;
        const bool chosen = lane < a.K && id >= 0;
        const unsigned long long m = __ballot(chosen);
        if (lane < 16) {
            s_blob[lane] = lane < a.K ? blob : nullptr;
            s_w[lane] = lane < a.K ? w : 0.0f;
        }
        if (chosen) s_kept[1 + __popcll(m & ((1ull << lane) - 1))] = lane;
        if (lane == 0) s_kept[0] = __popcll(m);
        if (b == 0 && lane < a.K) {
            a.ids[lane] = id;
            a.w[lane] = w;
        }
    }
    __syncthreads();
    // this workgroup's shared expert h values are all published
    if (threadIdx.x == 0 && a.S > 0) count_up(f.shared_done, b);

    // ---- phase 1: routed gate/up items
    if constexpr (SG::RPL == 1 && code_planes(F) == 1 && row_pack(F) == 1) {
        // items b, b + G, b + 2G, ... belong to this workgroup; its waves
        // claim them one at a time from an LDS counter, so faster waves take
        // more of them and all finish together
        const int n_items = s_kept[0] * per_slot;
        const int n_wg = b < n_items ? (n_items - 1 - b) / G + 1 : 0;
        auto claim = [&]() {
            int j = 0;
            if (lane == 0) j = atomicAdd(&s_next, 1);
            return __builtin_amdgcn_readfirstlane(j);
        };
        constexpr int NB = kFusedItemsInFlight;
        GateUpBuf<KG, F> bufs[NB];
        int item[NB];
        auto issue = [&](int i) {
            const int j = claim();
            const bool live = j < n_wg;
            item[i] = live ? b + j * G : -1;
            const int it = live ? item[i] : 0;
            const int slot = __builtin_amdgcn_readfirstlane(s_kept[1 + it / per_slot]);
            gateup_issue_buf<KG, F>(readlane_ptr(s_blob[slot], 0), live, L, it % per_slot, lane, bufs[i]);
        };
#pragma unroll
        for (int i = 0; i < NB; ++i) issue(i);
        bool more = true;
        while (more) {
            more = false;
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                if (item[i] >= 0) {
                    const int it = item[i];
                    const int slot = __builtin_amdgcn_readfirstlane(s_kept[1 + it / per_slot]);
                    gateup_compute_src<KG, F, true>(bufs[i], it % per_slot, lane, xsrc, a.h + (size_t)slot * a.I,
                                                    a.I / 32, true);
                    more = true;
                }
                issue(i);
            }
        }
    } else {
        const int n_items = s_kept[0] * per_slot;
        const int n_mine = gw < n_items ? (n_items - 1 - gw) / NW + 1 : 0;
        auto item_of = [&](int k) {
            const int item = gw + k * NW;
            return item < n_items ? item : n_items - 1;
        };
        // slot and blob of an item as wave-uniform values (scalar
        // registers), so the loads take a scalar base and one lane offset
        auto slot_of = [&](int it) { return __builtin_amdgcn_readfirstlane(s_kept[1 + it / per_slot]); };
        auto issue = [&](int k, GateUpBuf<KG, F>& buf) {
            const int it = item_of(k);
            gateup_issue<KG, F>(readlane_ptr(s_blob[slot_of(it)], 0), L, it % per_slot, lane, buf);
        };
        auto compute = [&](int k, const GateUpBuf<KG, F>& buf) {
            const int it = item_of(k);
            gateup_compute_src<KG, F, true>(buf, it % per_slot, lane, xsrc, a.h + (size_t)slot_of(it) * a.I, a.I / 32,
                                            k < n_mine);
        };
        constexpr int NB = kFusedItemsInFlight;
        GateUpBuf<KG, F> bufs[NB];
        switch (n_mine) {
            case 0: break;
            case 1: run_items<1, NB>(issue, compute, bufs); break;
            case 2: run_items<2, NB>(issue, compute, bufs); break;
            case 3: run_items<3, NB>(issue, compute, bufs); break;
            case 4: run_items<4, NB>(issue, compute, bufs); break;
            case 5: run_items<5, NB>(issue, compute, bufs); break;
            case 6: run_items<6, NB>(issue, compute, bufs); break;
            case 7: run_items<7, NB>(issue, compute, bufs); break;
            case 8: run_items<8, NB>(issue, compute, bufs); break;
            default: run_items_loop<NB>(n_mine, issue, compute, bufs); break;
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's h stores are acknowledged

    // ---- phase 2: wave w takes the steps of routed slot w / P congruent to
    // w mod P (P = kFusedWavesPerSlot) and the shared expert's steps
    // congruent to w modulo the wave count, over row block b
    const int slot = wave / kFusedWavesPerSlot;
    const uint8_t* dblob = s_blob[slot];
    DownSteps<KGI, NLD, F, kFusedWavesPerSlot> d;
    if (dblob) d.issue(dblob, L, b, lane, wave % kFusedWavesPerSlot);
    const int g0i = KGI >= kWave ? lane : (lane & (KGI - 1));
    if (a.S > 0) {
        // the shared expert's h was complete long ago (phase 0): its rows go
        // before the wait for the routed experts' h
        DownSteps<KGI, NLD, F, kFusedWavesPerSlot * NK> sh;
        sh.issue(a.shared_blob, L, b, lane, wave);
        if (!wait_count(f.shared_done, f.seq * (unsigned)G, f.spin_limit, lane) && lane == 0) s_fail = 1;
        float hraw[SD::CPL][32];
        load_h_device_scope<SD::CPL, KGI>(h_shared, g0i, hraw);
        sh.finish(hraw, lane, wave, part[a.K]);
    }
    __syncthreads();
    if (wave == 0) {
        if (lane == 0) count_up(f.h_done, b);
        if (!wait_count(f.h_done, f.seq * (unsigned)G, f.spin_limit, lane) && lane == 0) s_fail = 1;
    }
    __syncthreads();
    if (dblob) {
        float hraw[SD::CPL][32];
        load_h_device_scope<SD::CPL, KGI>(a.h + (size_t)slot * a.I, g0i, hraw);
        d.finish(hraw, lane, wave % kFusedWavesPerSlot, part[slot]);
    } else if (wave % kFusedWavesPerSlot == 0) {
        // a routed slot that the top-p cut dropped: weight 0, nothing read
        for (int t = lane; t < D::RP * SD::R; t += kWave) part[slot][t] = 0.0f;
    }
    __syncthreads();
    if ((int)threadIdx.x < D::RP * SD::R) {
        const int t = threadIdx.x;
        float y = 0.0f;
        for (int j = 0; j < a.K; ++j) y = fmaf(s_w[j], part[j][t], y);
        if (a.S > 0) y += part[a.K][t];
        a.y[(size_t)D::RP * (b * SD::R + t % SD::R) + t / SD::R] = y;
    }
    if (threadIdx.x == 0 && s_fail) __hip_atomic_store(f.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------- kernels 2 and 3 in one launch
// h of one slot as dot operands (to_operands), staged in LDS for the waves
// that share the slot; structure of arrays over the lanes (one 32-input
// group of h per lane).
struct HOperandsLds {
    u32x4 he[kWave], ho[kWave], le[kWave], lo[kWave];
    int corr[kWave];
    float scale[kWave];
    __device__ __forceinline__ void put(int lane, const HI8& o, float f) {
        he[lane] = o.he;
        ho[lane] = o.ho;
        le[lane] = o.le;
        lo[lane] = o.lo;
        corr[lane] = o.corr;
        scale[lane] = f;
    }
    __device__ __forceinline__ void get(int lane, HI8 (&o)[1], float (&f)[1]) const {
        o[0].he = he[lane];
        o[0].ho = ho[lane];
        o[0].le = le[lane];
        o[0].lo = lo[lane];
        o[0].corr = corr[lane];
        f[0] = scale[lane];
    }
};

// Routed gate/up + SwiGLU, down projections and combine of one token in one
// launch after the router launch: workgroups of 16 waves, one per block of R
// output rows, all resident at once (the host checks the occupancy).  Every
// wave first runs the gate/up items that gateup_kernel gives wave
// blockIdx * 16 + wave of a 16-wave grid, storing h with device-scope
// stores; then it issues the code loads of its down steps: routed slot
// wave / 2, the steps of the block congruent to wave mod 2, and the shared
// expert's steps congruent to wave mod 16.  Once every workgroup has counted
// its h as published (a spread counter; a bounded wait), the wave of each
// routed slot converts that slot's h into dot operands in LDS (the shared
// expert's h, complete since the router launch, was converted before the
// wait), every wave finishes its steps from them and the block is combined in
// slot order.  Dot products, reductions and combine are down_combine_kernel's,
// so y is bit-identical to the three-launch path's.
constexpr int kGdWaves = 16;        // waves per workgroup
constexpr int kGdWavesPerSlot = 2;  // waves sharing a routed slot's down steps

template <int KG, int KGI, int NLD, int F>
__global__ void __launch_bounds__(64 * kGdWaves) gateup_down_kernel(DecodeArgs a, FusedArgs f) {
    using SG = GateUpShape<KG>;
    using SD = DownShape<KGI, NLD>;
    static_assert(SD::CPL == 1 && row_pack(F) == 1, "one h group per lane, one matrix row per stored row");
    const int lane = threadIdx.x & 63;
    const int wave = wave_in_block();
    const int rb = blockIdx.x;
    const int wave_id = rb * kGdWaves + wave;
    const int n_waves = gridDim.x * kGdWaves;
    const int per_slot = a.I / SG::R;
    const BlobLayout L = blob_layout(a.H, a.I, F);
    const int g0 = KGI >= kWave ? lane : (lane & (KGI - 1));
    __shared__ int wave_kept[kGdWaves][17];
    __shared__ const uint8_t* wave_blobs[kGdWaves][16];
    __shared__ HOperandsLds hops[kFusedMaxSlots + 1];  // routed slots, then the shared expert
    __shared__ float part[kFusedMaxSlots + 1][SD::R];
    __shared__ int s_fail;
    if (threadIdx.x == 0) s_fail = 0;
    // the blobs of this wave's down slot and of the slot whose h it converts
    const int slot = wave / kGdWavesPerSlot;
    const uint8_t* dblob = slot < a.K ? a.slot_blobs[slot] : nullptr;
    const uint8_t* hblob = wave < a.K ? a.slot_blobs[wave] : nullptr;

    // ---- gate/up + SwiGLU of the routed slots (the kept ones with top-p)
    int n_routed_slots = a.K;
    if (a.kept) {
        if (lane < 17) wave_kept[wave][lane] = lane <= a.K ? a.kept[lane] : 0;
        __builtin_amdgcn_wave_barrier();
        n_routed_slots = wave_kept[wave][0];
    }
    const int n_items = n_routed_slots * per_slot;
    if (wave_id < n_items)
        routed_gateup_wave<KG, F, true>(a, lane, wave_id, n_waves, n_items, wave_kept[wave], wave_blobs[wave]);

    // ---- down: this wave's code loads go out before any wait
    DownSteps<KGI, NLD, F, kGdWavesPerSlot> d;
    if (dblob) d.issue(dblob, L, rb, lane, wave % kGdWavesPerSlot);
    DownSteps<KGI, NLD, F, kGdWaves> sh;
    if (a.S > 0) {
        sh.issue(a.shared_blob, L, rb, lane, wave);
        if (wave == kGdWaves - 1) {
            float hraw[1][32];
            load_h<1, KGI>(a.h + (size_t)a.K * a.I, g0, hraw);
            HI8 ha[1];
            float hs[1];
            to_operands<F, 1>(hraw, ha, hs);
            hops[a.K].put(lane, ha[0], hs[0]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's h stores are acknowledged
    __syncthreads();
    if (wave == 0) {
        if (lane == 0) count_up(f.h_done, rb);
        if (!wait_count(f.h_done, f.seq * (unsigned)gridDim.x, f.spin_limit, lane) && lane == 0) s_fail = 1;
    }
    __syncthreads();
    // every routed h is published
    if (hblob) {
        float hraw[1][32];
        load_h_device_scope<1, KGI>(a.h + (size_t)wave * a.I, g0, hraw);
        HI8 ha[1];
        float hs[1];
        to_operands<F, 1>(hraw, ha, hs);
        hops[wave].put(lane, ha[0], hs[0]);
    }
    __syncthreads();
    if (dblob) {
        HI8 ha[1];
        float hs[1];
        hops[slot].get(lane, ha, hs);
        d.finish_ops(ha, hs, lane, wave % kGdWavesPerSlot, part[slot]);
    } else if (slot < a.K && wave % kGdWavesPerSlot == 0) {
        // a routed slot that the top-p cut dropped: weight 0, nothing read
        for (int t = lane; t < SD::R; t += kWave) part[slot][t] = 0.0f;
    }
    if (a.S > 0) {
        HI8 ha[1];
        float hs[1];
        hops[a.K].get(lane, ha, hs);
        sh.finish_ops(ha, hs, lane, wave, part[a.K]);
    }
    __syncthreads();
    if ((int)threadIdx.x < SD::R) {
        const int t = threadIdx.x;
        float y = 0.0f;
        for (int j = 0; j < a.K; ++j) y = fmaf(a.w[j], part[j][t], y);
        if (a.S > 0) y += part[a.K][t];
        a.y[(size_t)rb * SD::R + t] = y;
    }
    if (threadIdx.x == 0 && s_fail) __hip_atomic_store(f.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------- launchers
// With timing events the launch goes through hipExtLaunchKernelGGL, which
// stamps the events with the kernel's own start and end (no gap from the
// enqueue of separate event records).
template <typename K>
hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, hipStream_t st, const LaunchTiming& tm,
                         const DecodeArgs& a) {
    if (tm.start)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, tm.start, tm.stop, 0, a);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, st, a);
    return hipGetLastError();
}

template <int KG, int F>
hipError_t launch_router_c(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm) {
    // router blocks, the shared expert's gate/up blocks, one conversion block
    const dim3 grid(router_blocks(a.E) + (a.S > 0 ? shared_gateup_blocks<KG>(a.I / row_pack(F)) : 0) + 1);
    if (a.E <= 64) return launch_kernel(router_kernel<KG, 1, F>, grid, dim3(256), st, tm, a);
    if (a.E <= 128) return launch_kernel(router_kernel<KG, 2, F>, grid, dim3(256), st, tm, a);
    return launch_kernel(router_kernel<KG, 4, F>, grid, dim3(256), st, tm, a);
}
template <int KG>
hipError_t launch_router(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm) {
    if (a.codec == kCodecMxfp4) return launch_router_c<KG, kCodecMxfp4>(a, st, tm);
    if (a.codec == kCodecInt8) return launch_router_c<KG, kCodecInt8>(a, st, tm);
    if (a.codec == kCodecInt2) return launch_router_c<KG, kCodecInt2>(a, st, tm);
    return launch_router_c<KG, kCodecInt4>(a, st, tm);
}

template <int KG>
hipError_t launch_gateup(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm) {
    const int per_slot = a.I / row_pack(a.codec) / GateUpShape<KG>::R;
    const int n_slots = a.use_slot_list ? a.n_slot_list : a.K;
    if (n_slots == 0) return hipSuccess;
    const int items = n_slots * per_slot;
    // at least one round of kGateUpItemsPerRound items per wave, at most
    // 4096 waves (16 per CU), at least 256 waves when there are enough items
    int waves = (items + kGateUpItemsPerRound - 1) / kGateUpItemsPerRound;
    if (waves < 256) waves = items < 256 ? items : 256;
    if (waves > 4096) waves = 4096;
    waves = (waves + 3) / 4 * 4;
    if (a.codec == kCodecMxfp4)
        return launch_kernel(gateup_kernel<KG, kCodecMxfp4>, dim3(waves / 4), dim3(256), st, tm, a);
    if (a.codec == kCodecInt8)
        return launch_kernel(gateup_kernel<KG, kCodecInt8>, dim3(waves / 4), dim3(256), st, tm, a);
    if (a.codec == kCodecInt2)
        return launch_kernel(gateup_kernel<KG, kCodecInt2>, dim3(waves / 4), dim3(256), st, tm, a);
    return launch_kernel(gateup_kernel<KG, kCodecInt4>, dim3(waves / 4), dim3(256), st, tm, a);
}

template <int KG, int NLD, int F>
hipError_t launch_down_c(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm) {
    using S = DownShape<KG, NLD>;
    if constexpr (ilog2(pow2_at_least(S::NL * row_pack(F))) <= S::B &&
                  S::NL * S::CPL * code_planes(F) <= down_max_loads(code_planes(F), S::CPL)) {
        const int grid = a.H / row_pack(F) / S::R;
        return launch_kernel(down_combine_kernel<KG, NLD, F>, dim3(grid), dim3((a.K + a.S) * 64), st, tm, a);
    } else {
        return hipErrorInvalidValue;  // never chosen by down_rows
    }
}
template <int KG, int NLD>
hipError_t launch_down_nl(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm) {
    if (a.codec == kCodecMxfp4) return launch_down_c<KG, NLD, kCodecMxfp4>(a, st, tm);
    if (a.codec == kCodecInt8) return launch_down_c<KG, NLD, kCodecInt8>(a, st, tm);
    if (a.codec == kCodecInt2) return launch_down_c<KG, NLD, kCodecInt2>(a, st, tm);
    return launch_down_c<KG, NLD, kCodecInt4>(a, st, tm);
}

template <int KG>
hipError_t launch_down(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm) {
    const int nl = down_rows(a.H, KG, a.codec) / rows_per_load(KG);
    switch (nl) {
        case 1: return launch_down_nl<KG, 1>(a, st, tm);
        case 2: return launch_down_nl<KG, 2>(a, st, tm);
        case 4: return launch_down_nl<KG, 4>(a, st, tm);
        case 8: return launch_down_nl<KG, 8>(a, st, tm);
        case 12: return launch_down_nl<KG, 12>(a, st, tm);
        case 16: return launch_down_nl<KG, 16>(a, st, tm);
        case 24: return launch_down_nl<KG, 24>(a, st, tm);
        case 32: return launch_down_nl<KG, 32>(a, st, tm);
        default: return hipErrorInvalidValue;
    }
}


// Fused kernel instances: (hidden/32, inter/32, experts per router lane)
// of the GLM-5.2-shaped layer and of the smaller parity shapes, int4
// experts; other shapes and codecs take the three launches.
template <int KG, int KGI, int EPL, int F, int NK>
const void* fused_fn_shape() {
    // the down step count down_rows gives at hidden = 32 KG
    constexpr int NLD = down_rows(32 * KG, KGI, F) / rows_per_load(KGI);
    return reinterpret_cast<const void*>(fused_decode_kernel<KG, KGI, NLD, EPL, F, NK>);
}

const void* fused_fn(const DecodeArgs& a) {
    const int kg = a.H / 32, kgi = a.I / 32;
    const int epl = a.E <= 64 ? 1 : (a.E <= 128 ? 2 : 4);
    if (a.S > 1) return nullptr;
    // int4 only: the instances are sized for its registers
    if (a.codec != kCodecInt4) return nullptr;
    if (kg == 192 && kgi == 64 && epl == 4 && a.K == 8) return fused_fn_shape<192, 64, 4, kCodecInt4, 8>();
    if (kg == 8 && kgi == 4 && epl == 1 && a.K == 4) return fused_fn_shape<8, 4, 1, kCodecInt4, 4>();
    if (kg == 32 && kgi == 8 && epl == 1 && a.K == 6) return fused_fn_shape<32, 8, 1, kCodecInt4, 6>();
    if (kg == 128 && kgi == 32 && epl == 2 && a.K == 8) return fused_fn_shape<128, 32, 2, kCodecInt4, 8>();
    if (kg == 16 && kgi == 4 && epl == 4 && a.K == 8) return fused_fn_shape<16, 4, 4, kCodecInt4, 8>();
    return nullptr;
}

// Instances of the gate/up + down launch: the fused kernel's shapes, int4
// experts; other shapes and codecs take the three launches.
template <int KG, int KGI, int F>
const void* gateup_down_fn_shape() {
    constexpr int NLD = down_rows(32 * KG, KGI, F) / rows_per_load(KGI);
    return reinterpret_cast<const void*>(gateup_down_kernel<KG, KGI, NLD, F>);
}

const void* gateup_down_fn(const DecodeArgs& a) {
    const int kg = a.H / 32, kgi = a.I / 32;
    if (a.S > 1 || a.K > kFusedMaxSlots || a.direct || a.use_slot_list || !a.table) return nullptr;
    if (a.codec != kCodecInt4) return nullptr;
    if (kg == 192 && kgi == 64) return gateup_down_fn_shape<192, 64, kCodecInt4>();
    if (kg == 8 && kgi == 4) return gateup_down_fn_shape<8, 4, kCodecInt4>();
    if (kg == 32 && kgi == 8) return gateup_down_fn_shape<32, 8, kCodecInt4>();
    if (kg == 128 && kgi == 32) return gateup_down_fn_shape<128, 32, kCodecInt4>();
    if (kg == 16 && kgi == 4) return gateup_down_fn_shape<16, 4, kCodecInt4>();
    return nullptr;
}

template <typename K>
hipError_t launch_batch_kernel(K kernel, dim3 grid, dim3 block, hipStream_t st, const LaunchTiming& tm,
                               const BatchArgs& a) {
    if (tm.start)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, tm.start, tm.stop, 0, a);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, st, a);
    return hipGetLastError();
}

// 4096 waves (16 per CU) for the singles' gate/up, spread over the pairs;
// the same for their down items.
constexpr int kPairGrid = 1024;

template <int KG>
hipError_t launch_pair_gateup(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm) {
    const dim3 g(kPairGrid), b(256);
    if (a.codec == kCodecMxfp4) return launch_batch_kernel(pair_gateup_kernel<KG, kCodecMxfp4>, g, b, st, tm, a);
    if (a.codec == kCodecInt8) return launch_batch_kernel(pair_gateup_kernel<KG, kCodecInt8>, g, b, st, tm, a);
    if (a.codec == kCodecInt2) return launch_batch_kernel(pair_gateup_kernel<KG, kCodecInt2>, g, b, st, tm, a);
    return launch_batch_kernel(pair_gateup_kernel<KG, kCodecInt4>, g, b, st, tm, a);
}

template <int KG, int NLD, int F>
hipError_t launch_pair_down_c(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm) {
    using S = DownShape<KG, NLD>;
    if constexpr (ilog2(pow2_at_least(S::NL * row_pack(F))) <= S::B &&
                  S::NL * S::CPL * code_planes(F) <= down_max_loads(code_planes(F), S::CPL)) {
        return launch_batch_kernel(pair_down_kernel<KG, NLD, F>, dim3(kPairGrid), dim3(256), st, tm, a);
    } else {
        return hipErrorInvalidValue;  // never chosen by down_rows
    }
}
template <int KG, int NLD>
hipError_t launch_pair_down_nl(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm) {
    if (a.codec == kCodecMxfp4) return launch_pair_down_c<KG, NLD, kCodecMxfp4>(a, st, tm);
    if (a.codec == kCodecInt8) return launch_pair_down_c<KG, NLD, kCodecInt8>(a, st, tm);
    if (a.codec == kCodecInt2) return launch_pair_down_c<KG, NLD, kCodecInt2>(a, st, tm);
    return launch_pair_down_c<KG, NLD, kCodecInt4>(a, st, tm);
}
template <int KG>
hipError_t launch_pair_down(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm) {
    switch (down_rows(a.H, KG, a.codec) / rows_per_load(KG)) {
        case 1: return launch_pair_down_nl<KG, 1>(a, st, tm);
        case 2: return launch_pair_down_nl<KG, 2>(a, st, tm);
        case 4: return launch_pair_down_nl<KG, 4>(a, st, tm);
        case 8: return launch_pair_down_nl<KG, 8>(a, st, tm);
        case 12: return launch_pair_down_nl<KG, 12>(a, st, tm);
        case 16: return launch_pair_down_nl<KG, 16>(a, st, tm);
        case 24: return launch_pair_down_nl<KG, 24>(a, st, tm);
        case 32: return launch_pair_down_nl<KG, 32>(a, st, tm);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Kernels are instantiated for H/32 in {8,16,32,64,128,192,256} and
// I/32 in {4,8,16,32,64,128}.
hipError_t decode_router(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm) {
    switch (a.H / 32) {
        case 8: return launch_router<8>(a, st, tm);
        case 16: return launch_router<16>(a, st, tm);
        case 32: return launch_router<32>(a, st, tm);
        case 64: return launch_router<64>(a, st, tm);
        case 128: return launch_router<128>(a, st, tm);
        case 192: return launch_router<192>(a, st, tm);
        case 256: return launch_router<256>(a, st, tm);
        default: return hipErrorInvalidValue;
    }
}

hipError_t decode_routed_gateup(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm) {
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

hipError_t batch_pair_gateup(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm) {
    switch (a.H / 32) {
        case 8: return launch_pair_gateup<8>(a, st, tm);
        case 16: return launch_pair_gateup<16>(a, st, tm);
        case 32: return launch_pair_gateup<32>(a, st, tm);
        case 64: return launch_pair_gateup<64>(a, st, tm);
        case 128: return launch_pair_gateup<128>(a, st, tm);
        case 192: return launch_pair_gateup<192>(a, st, tm);
        case 256: return launch_pair_gateup<256>(a, st, tm);
        default: return hipErrorInvalidValue;
    }
}

hipError_t batch_pair_down(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm) {
    switch (a.I / 32) {
        case 4: return launch_pair_down<4>(a, st, tm);
        case 8: return launch_pair_down<8>(a, st, tm);
        case 16: return launch_pair_down<16>(a, st, tm);
        case 32: return launch_pair_down<32>(a, st, tm);
        case 64: return launch_pair_down<64>(a, st, tm);
        case 128: return launch_pair_down<128>(a, st, tm);
        default: return hipErrorInvalidValue;
    }
}

hipError_t decode_down_combine(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm) {
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

int fused_grid(const DecodeArgs& a, int* threads) {
    if (!fused_fn(a)) return 0;
    *threads = 64 * kFusedWavesPerSlot * a.K;
    return a.H / row_pack(a.codec) / down_rows(a.H, a.I / 32, a.codec);
}

const void* fused_kernel_function(const DecodeArgs& a) { return fused_fn(a); }

hipError_t decode_fused(const DecodeArgs& a, const FusedArgs& f, hipStream_t st, const LaunchTiming& tm) {
    const void* fn = fused_fn(a);
    int threads = 0;
    const int grid = fused_grid(a, &threads);
    if (!fn || grid == 0) return hipErrorInvalidValue;
    DecodeArgs args = a;
    FusedArgs fargs = f;
    void* params[] = {&args, &fargs};
    if (tm.start)
        return hipExtLaunchKernel(fn, dim3(grid), dim3(threads), params, 0, st, tm.start, tm.stop, 0);
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), params, 0, st);
}

int gateup_down_grid(const DecodeArgs& a, int* threads) {
    if (!gateup_down_fn(a)) return 0;
    *threads = 64 * kGdWaves;
    return a.H / down_rows(a.H, a.I / 32, a.codec);
}

const void* gateup_down_kernel_function(const DecodeArgs& a) { return gateup_down_fn(a); }

hipError_t decode_gateup_down(const DecodeArgs& a, const FusedArgs& f, hipStream_t st, const LaunchTiming& tm) {
    const void* fn = gateup_down_fn(a);
    int threads = 0;
    const int grid = gateup_down_grid(a, &threads);
    if (!fn || grid == 0) return hipErrorInvalidValue;
    DecodeArgs args = a;
    FusedArgs fargs = f;
    void* params[] = {&args, &fargs};
    if (tm.start)
        return hipExtLaunchKernel(fn, dim3(grid), dim3(threads), params, 0, st, tm.start, tm.stop, 0);
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), params, 0, st);
}

bool decode_shape_supported(int hidden, int inter, int top_k, int n_shared) {
    const int kh = hidden / 32, ki = inter / 32;
    const bool h_ok = kh == 8 || kh == 16 || kh == 32 || kh == 64 || kh == 128 || kh == 192 || kh == 256;
    const bool i_ok = ki == 4 || ki == 8 || ki == 16 || ki == 32 || ki == 64 || ki == 128;
    return h_ok && i_ok && hidden % 256 == 0 && hidden % down_rows(hidden, ki, kCodecInt4) == 0 &&
           hidden % down_rows(hidden, ki, kCodecInt8) == 0 && (hidden / 2) % down_rows(hidden, ki, kCodecInt2) == 0 &&
           (inter / 2) % gateup_rows(kh) == 0 &&
           inter % gateup_rows(kh) == 0 && top_k <= 8;
}

}  // namespace moe
