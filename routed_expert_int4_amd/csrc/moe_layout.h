// Private device layout of a packed expert blob, shared by the host packer
// and the kernels (both are the library; the CPU oracle never sees this).
//
// A blob holds, in order:
//   gate codes [I][H/2], up codes [I][H/2], down codes [H][I/2]
//       the public row-major bytes with every nibble stored as q + 8
//       (offset binary), so a kernel can place a nibble straight into the
//       mantissa of an fp16 constant and subtract the offset exactly;
//   gate scales, up scales, down scales (fp16 bits)
//       permuted so that each lane of a wave finds the scales it needs for
//       one work item in consecutive bytes (see scale_index).
// The blob is exactly as large as the public layout.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace moe {

constexpr int kWave = 64;
// Rows of the down projection per workgroup (and per scale pack) when a row
// fits in one wave load or more.
constexpr int kDownRowsBase = 16;
// Rows of gate (and of up) per gate/up work item when a row fits in one wave
// load or more.
constexpr int kGateUpRowsBase = 4;

// A wave load covers 64 lanes x 16 bytes = 64 scale groups (32 codes each).
// A matrix with kg groups per row needs rows_per_load rows per wave load when
// kg < 64, and chunks_per_lane loads per row when kg >= 64.
__host__ __device__ constexpr int rows_per_load(int kg) { return kg >= kWave ? 1 : kWave / kg; }
__host__ __device__ constexpr int chunks_per_lane(int kg) { return kg >= kWave ? kg / kWave : 1; }
__host__ __device__ constexpr int gateup_rows(int kg_h) {
    return rows_per_load(kg_h) > kGateUpRowsBase ? rows_per_load(kg_h) : kGateUpRowsBase;
}
__host__ __device__ constexpr int down_rows(int kg_i) {
    return rows_per_load(kg_i) > kDownRowsBase ? rows_per_load(kg_i) : kDownRowsBase;
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

struct BlobLayout {
    size_t gate_q, up_q, down_q;  // byte offsets of the code arrays
    size_t gate_s, up_s, down_s;  // byte offsets of the scale arrays
    size_t total;
};

__host__ __device__ inline BlobLayout blob_layout(int hidden, int inter) {
    BlobLayout L;
    const size_t codes = (size_t)hidden * inter / 2;
    const size_t scales = (size_t)hidden * (inter / 32) * 2;
    L.gate_q = 0;
    L.up_q = codes;
    L.down_q = 2 * codes;
    L.gate_s = 3 * codes;
    L.up_s = 3 * codes + scales;
    L.down_s = 3 * codes + 2 * scales;
    L.total = 3 * codes + 3 * scales;
    return L;
}

}  // namespace moe
