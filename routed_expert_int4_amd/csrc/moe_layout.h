// Private device layout of a packed expert blob, shared by the host packer
// and the kernels (both are the library; the CPU oracle never sees this).
//
// A blob holds, in order:
//   gate codes [I][H/2], up codes [I][H/2], down codes [H][I/2]
//       the public row-major bytes; int4 nibbles are stored as q + 8
//       (offset binary, the kernels take the offset off with a per-group
//       correction), MXFP4 (E2M1) nibbles as they are, int8 codes q as the
//       int4 planes of their high nibbles q >> 4 (signed, stored + 8);
//   gate and up scales (interleaved per block of rows), down scales
//       (fp16 bits for int4, E8M0 bytes for MXFP4), permuted so that each
//       lane of a wave finds the scales it needs for one work item in
//       consecutive bytes (see scale_index and gateup_scale_index);
//   int8 only: gate, up and down planes of the low nibbles q & 15
//       (unsigned), shaped as the high planes, so q = 16 hi + lo and every
//       kernel keeps the int4 lane mapping with two loads per chunk.
// Int2 matrices are stored as int4-shaped planes of half the rows: nibble
// (virtual row p, column c) holds the codes of rows 2p (bits 0-1) and 2p + 1
// (bits 2-3), each + 2, and the scales of the even and the odd rows go to
// two arrays, each packed as an int4 matrix of rows/2 rows would be (the
// odd rows' arrays follow the even rows' ones).
// The blob is exactly as large as the public layout.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace moe {

constexpr int kWave = 64;
// Weight codecs (the moe_config_t codec values).
constexpr int kCodecInt4 = 0;   // int4 codes, fp16 scale per 32 inputs
constexpr int kCodecMxfp4 = 1;  // E2M1 codes, E8M0 scale per 32 inputs
constexpr int kCodecInt8 = 2;   // int8 codes, fp16 scale per 32 inputs
constexpr int kCodecInt2 = 3;   // int2 codes, fp16 scale per 32 inputs
__host__ __device__ constexpr int scale_bytes(int codec) { return codec == kCodecMxfp4 ? 1 : 2; }
// Nibble planes per matrix in the blob (int8: high and low nibbles).
__host__ __device__ constexpr int code_planes(int codec) { return codec == kCodecInt8 ? 2 : 1; }
// Matrix rows per stored (virtual) row (int2: two rows share a nibble).
__host__ __device__ constexpr int row_pack(int codec) { return codec == kCodecInt2 ? 2 : 1; }
// Rows of gate (and of up) per gate/up work item when a row fits in one
// wave load or more.
constexpr int kGateUpRowsBase = 1;

// A wave load covers 64 lanes x 16 bytes = 64 scale groups (32 codes each).
// A matrix with kg groups per row needs rows_per_load rows per wave load when
// kg < 64, and chunks_per_lane loads per row when kg >= 64.
__host__ __device__ constexpr int rows_per_load(int kg) { return kg >= kWave ? 1 : kWave / kg; }
__host__ __device__ constexpr int chunks_per_lane(int kg) { return kg >= kWave ? kg / kWave : 1; }
__host__ __device__ constexpr int gateup_rows(int kg_h) {
    return rows_per_load(kg_h) > kGateUpRowsBase ? rows_per_load(kg_h) : kGateUpRowsBase;
}
// Wave-load steps a down-projection wave may take over its row block; the
// down kernel is instantiated for each of these counts.
__host__ __device__ constexpr int down_step_option(int i) {
    return i == 0 ? 32 : i == 1 ? 24 : i == 2 ? 16 : i == 3 ? 12 : i == 4 ? 8 : i == 5 ? 4 : i == 6 ? 2 : 1;
}
constexpr int kDownStepOptions = 8;
// Code loads a down-projection wave keeps in registers at most (steps x
// chunk columns x planes): 24 with one chunk column and one plane, else 16
// (a second chunk column or nibble plane needs the registers for its own
// operands and dot chain).
constexpr int kDownMaxLoads = 24;
__host__ __device__ constexpr int down_max_loads(int planes, int cpl) {
    return planes > 1 || cpl > 1 ? 16 : kDownMaxLoads;
}

__host__ __device__ constexpr int pow2_at_least(int v) { return v <= 1 ? 1 : 2 * pow2_at_least((v + 1) / 2); }

// Rows per down-projection workgroup: about hidden/256 (so one round of
// workgroups covers the 256 CUs), a multiple of rows_per_load(inter/32) that
// divides hidden, with a step count s from down_step_option such that the
// wave's s x chunks_per_lane code loads stay within kDownMaxLoads and its s
// row partials, rounded up to a power of two, fit the lanes that share a row
// (min(inter/32, 64)).  With two nibble planes (int8) every step loads
// twice as many chunks; with two rows per stored row (int2) the rows are
// stored rows (hidden / 2 of them) and every step yields two partials.
__host__ __device__ constexpr int down_rows(int hidden, int kg_i, int codec) {
    const int planes = code_planes(codec), rp = row_pack(codec);
    const int vrows = hidden / rp;
    const int rpl = rows_per_load(kg_i);
    const int lanes_per_row = kg_i < kWave ? kg_i : kWave;
    const int target = vrows / 256 > rpl ? vrows / 256 : rpl;
    for (int i = 0; i < kDownStepOptions; ++i) {
        const int steps = down_step_option(i);
        const int r = steps * rpl;
        if (r <= target && vrows % r == 0 && steps * chunks_per_lane(kg_i) * planes <= down_max_loads(planes, chunks_per_lane(kg_i)) &&
            pow2_at_least(steps * rp) <= lanes_per_row)
            return r;
    }
    return rpl;
}

// Position of the scale of (row r, group g) in a packed scale array of a
// matrix with kg groups per row, packed in blocks of p rows.  Inside a block
// the p scales of one group are ordered so that the rows one lane visits
// (row_sub, row_sub + rpl, row_sub + 2 rpl, ...) are adjacent.
__host__ __device__ inline size_t scale_index(int r, int g, int kg, int p) {
    const int rpl = rows_per_load(kg);
    const int i = r % p;
    return ((size_t)(r / p) * kg + g) * p + (size_t)(i % rpl) * (p / rpl) + i / rpl;
}

// Gate (m = 0) and up (m = 1) scales share one array: for each block of p
// rows and each group, the p gate scales then the p up scales, each in the
// order of scale_index, so a lane that visits one row per load finds the
// gate and up scales of its rows in one contiguous run.
__host__ __device__ inline size_t gateup_scale_index(int r, int g, int m, int kg, int p) {
    const int rpl = rows_per_load(kg);
    const int i = r % p;
    return (((size_t)(r / p) * kg + g) * 2 + m) * p + (size_t)(i % rpl) * (p / rpl) + i / rpl;
}

struct BlobLayout {
    size_t gate_q, up_q, down_q;     // byte offsets of the code arrays (int8: high-nibble planes)
    size_t gu_s, down_s;             // byte offsets of the scale arrays (int2: even rows)
    size_t gate_lo, up_lo, down_lo;  // int8 low-nibble planes (0 otherwise)
    size_t gu_s2, down_s2;           // int2 scales of the odd rows (0 otherwise)
    size_t total;
};

__host__ __device__ inline BlobLayout blob_layout(int hidden, int inter, int codec) {
    BlobLayout L;
    const size_t codes = (size_t)hidden * inter / 2 / row_pack(codec);
    const size_t scales = (size_t)hidden * (inter / 32) * scale_bytes(codec);
    L.gate_q = 0;
    L.up_q = codes;
    L.down_q = 2 * codes;
    L.gu_s = 3 * codes;
    L.down_s = 3 * codes + 2 * scales;
    L.total = 3 * codes + 3 * scales;
    L.gate_lo = L.up_lo = L.down_lo = 0;
    L.gu_s2 = L.down_s2 = 0;
    if (codec == kCodecInt2) {
        // even rows: gate/up then down, then the odd rows' arrays
        L.down_s = L.gu_s + scales;
        L.gu_s2 = L.down_s + scales / 2;
        L.down_s2 = L.gu_s2 + scales;
    }
    if (codec == kCodecInt8) {
        L.gate_lo = L.total;
        L.up_lo = L.total + codes;
        L.down_lo = L.total + 2 * codes;
        L.total += 3 * codes;
    }
    return L;
}

}  // namespace moe
