// Launch interface between the host library and the HIP kernels.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "moe_layout.h"

namespace moe {

// Arguments of the one-token decode path.  Every pointer is device memory.
struct DecodeArgs {
    const uint16_t* x;               // [H] bf16 bits
    const float* router_w;           // [E][H]
    const float* bias;               // [E]
    const uint8_t* const* table;     // [E] packed routed expert blobs (null with an expert cache)
    const uint8_t* shared_blob;      // packed shared expert (when S == 1)
    float* s;                        // [E] router affinities sigmoid(logit) (scratch)
    float* sb;                       // [E] biased scores s + bias (scratch)
    unsigned* xq;                    // activations as integer dot operands, per lane (scratch)
    int32_t* ids;                    // [K] routing output
    float* w;                        // [K]
    const uint8_t** slot_blobs;      // [16] blobs of the routed slots, resolved once (scratch)
    // With top_p < 1 and a table: the router writes kept[0] = number of
    // routed slots that survive the top-p cut and kept[1 ..] = those slots in
    // increasing order, and the gate/up launch covers only them (null
    // otherwise).
    int* kept;
    float* h;                        // [(K + S) * I] scratch
    float* y;                        // [H] output
    unsigned* counter;               // router blocks done (workspace control word, 0 between calls)
    int H, I, E, G, TG, K, S;
    float rsf;
    float top_p;                     // adaptive expert top-p (1: plain top-k)
    int codec;                       // weight codec (kCodecInt4 .. kCodecInt2)
    // Expert-cache mode: routed slot j reads blobs[j] instead of
    // table[ids[j]] (the host resolved the routing before the launch).
    int direct;
    const uint8_t* blobs[16];
    // Optional subset of routed slots for the gate/up launch: with
    // use_slot_list the launch covers slot_list[0 .. n_slot_list-1] only
    // (possibly none).
    int use_slot_list;
    int n_slot_list;
    int slot_list[16];
};

// Optional timing of one launch: when start is set the launch stamps start
// and stop with the kernel's own begin and end.
struct LaunchTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// Control of the fused one-token decode launch (decode_fused), in the
// workspace's sync region (cleared when a workspace is bound).  The router
// rows publish s and sb as records (value bits, call number) that the
// routing waves poll.  The counts of workgroups whose shared expert h, and
// whose routed h, values are published are each spread over kSyncCounters words kSyncStride words apart (one cache line
// each): workgroup b increments word b mod kSyncCounters, and a waiting wave
// reads all of them at once and sums them (device-scope atomics on one
// address are serialised where they execute, so hundreds of increments of
// a single word would take microseconds).  Nothing is reset between calls:
// the call with number seq (1, 2, ... since the workspace was bound) looks
// for records carrying seq and waits for the sums seq * grid.  A wait that
// does not succeed within spin_limit polls gives up, sets *status
// (host-visible memory) to 1 and the launch finishes without blocking.
constexpr int kSyncCounters = 32;
constexpr int kSyncStride = 64;  // words (256 bytes)
constexpr int kSyncMaxExperts = 256;
constexpr size_t kSyncCounterBytes = kSyncCounters * kSyncStride * sizeof(unsigned);
// Offsets in the sync region: the fused launch's h and shared-expert
// counts, its score records, and the count of the gate/up + down launch.
constexpr size_t kSyncHDone = 0;
constexpr size_t kSyncSharedDone = kSyncCounterBytes;
constexpr size_t kSyncScoreRecords = 2 * kSyncCounterBytes;
constexpr size_t kSyncGateUpDownDone = kSyncScoreRecords + 2 * kSyncMaxExperts * sizeof(unsigned long long);
constexpr size_t kSyncBytes = kSyncGateUpDownDone + kSyncCounterBytes;
struct FusedArgs {
    unsigned* h_done;               // kSyncCounters words
    unsigned* shared_done;          // kSyncCounters words: workgroups whose shared expert h is published
    unsigned long long* s_rec;      // [E] records of s
    unsigned long long* sb_rec;     // [E] records of sb
    unsigned* status;               // set to 1 when a wait gives up
    unsigned seq;
    unsigned spin_limit;
};

// Router logits -> s, sb; group-limited top-k -> ids, w (and slot_blobs
// from table when it is set); gate/up + SwiGLU of the shared expert;
// activation pairs.
hipError_t decode_router(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm = {});
// Gate/up + SwiGLU of the routed experts (blobs from slot_blobs, or from
// blobs in direct mode).
hipError_t decode_routed_gateup(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm = {});
// Down projection of every slot and the weighted combine into y.
hipError_t decode_down_combine(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm = {});
bool decode_shape_supported(int hidden, int inter, int top_k, int n_shared);
// The whole one-token layer in one launch of co-resident workgroups (router
// and shared gate/up, the top-k, routed gate/up, down and combine, with the
// hand-offs done in the kernel).  fused_grid returns the launch's workgroups
// and threads per workgroup for this shape, or 0 when the fused kernel has
// no instance for it; fused_kernel_function returns the kernel (for the
// occupancy query).
int fused_grid(const DecodeArgs& a, int* threads);
const void* fused_kernel_function(const DecodeArgs& a);
hipError_t decode_fused(const DecodeArgs& a, const FusedArgs& f, hipStream_t st, const LaunchTiming& tm = {});
// Routed gate/up + SwiGLU, down projections and combine of one token in one
// launch of co-resident workgroups after decode_router (the hand-off from h
// to the down projections done in the kernel; f.h_done, f.seq, f.spin_limit
// and f.status are used).  gateup_down_grid returns the launch's workgroups
// and threads per workgroup, or 0 when the kernel has no instance for this
// shape and codec; gateup_down_kernel_function returns the kernel.
int gateup_down_grid(const DecodeArgs& a, int* threads);
const void* gateup_down_kernel_function(const DecodeArgs& a);
hipError_t decode_gateup_down(const DecodeArgs& a, const FusedArgs& f, hipStream_t st, const LaunchTiming& tm = {});

// ------------------------------------------------------------ batched path
// Tokens per MFMA row block (the smallest tile) and rows per gate/up
// workgroup of the grouped kernels.
constexpr int kTileTokens = 16;
constexpr int kBlockRows = 128;
// Largest number of (token, routed slot) entries one dispatch sorts in LDS.
constexpr int kMaxDispatchEntries = 8192;

// Entries per tile of the grouped kernels for a call of T tokens: 32 (two
// MFMA row blocks per weight fragment, so an expert with up to 32 entries is
// read once) when the call averages at least 8 entries per expert and the
// codec's registers allow it, else 16 (a mostly empty second row block would
// only add work; the two-fragment codecs, int8 planes and int2 rows, have no
// registers for it).
__host__ __device__ constexpr int batch_tile_tokens(int codec, int T, int K, int E) {
    return codec == kCodecInt8 || codec == kCodecInt2 || T * K < 8 * E ? 16 : 32;
}

// One tile of the grouped kernels: up to batch_tile_tokens consecutive entries
// ("pairs") of one expert.  expert == E marks the shared expert.
struct Tile {
    int expert;
    int first_pair;
    int count;
    int pad;
};

// Arguments of a batched call of T tokens.  Pairs p in [0, T*K) are the
// routed (token, slot) entries sorted by expert then token; pairs T*K + t
// are the shared expert's (one per token).
struct BatchArgs {
    const uint16_t* x;           // [T][H] bf16 bits
    const float* router_w;       // [E][H]
    const float* bias;           // [E]
    const uint8_t* const* table; // [E] packed routed expert blobs
    const uint8_t* shared_blob;  // packed shared expert (S == 1)
    float* logit_part;           // [router_splits][T][E] partial router logits
    uint16_t* xa;                // [T][H/32][4][8] scaled fp16 activations, MFMA order
    int* kx;                     // [T] their scaling exponents
    int32_t* ids;                // [T][K]
    float* w;                    // [T][K]
    int32_t* counts;             // [E]
    int32_t* offsets;            // [E + 1]
    int32_t* perm;               // [T*K] pair -> token*K + slot (-1 past the kept entries)
    int32_t* inv;                // [T*K] token*K + slot -> pair (-1 for a dropped choice)
    int32_t* distinct;           // [E] experts with at least one entry, ascending
    int32_t* n_distinct;         // [1]
    Tile* tiles;                 // [max_tiles]
    int32_t* n_tiles;            // [1]
    Tile* singles;               // [min(T*K, E)] experts with 1..single_max entries (GEMV path)
    int32_t* n_singles;          // [1]
    float* h;                    // [P][I] SwiGLU outputs
    uint16_t* ha_hi;             // [P][I/32][4][8] h as scaled fp16 hi part, MFMA order
    uint16_t* ha_lo;             // [P][I/32][4][8] lo part
    int* kh;                     // [P] scaling exponents of h
    float* d;                    // [P][H] down projections
    float* y;                    // [T][H]
    int T, H, I, E, G, TG, K, S;
    int down_p;                  // row-block size of the down scale packing
    int router_splits;           // column splits of the router (power of two, hidden % (64 * splits) == 0)
    float rsf;
    float top_p;                 // adaptive expert top-p (1: plain top-k); dropped choices get id -1
    int codec;                   // weight codec (kCodecInt4 .. kCodecInt2)
    int tile_tokens;             // batch_tile_tokens(codec, T, K, E): 16 or 32
    int single_max;              // batch_single_max(tile_tokens): entries of an expert that takes the GEMV path
};

// Experts with at most this many entries in a call skip the grouped MFMA
// kernels and run the one-token GEMVs per (token, expert) pair: 1 in calls
// with 16-entry tiles (a single entry fills a sixteenth of its tile; two or
// more would read the expert once per pair), none with 32-entry tiles.
__host__ __device__ constexpr int batch_single_max(int tile_tokens) { return tile_tokens == 16 ? 1 : 0; }

// Upper bound of the tiles of a call of T tokens.
inline int batch_max_tiles(int T, int K, int E, int S) {
    const int n = T * K;
    return (n < E ? n : E) + (n + kTileTokens - 1) / kTileTokens + S * ((T + kTileTokens - 1) / kTileTokens);
}

// Router column splits for a hidden size: the largest power of two <=
// kMaxRouterSplits with hidden % (64 * splits) == 0.
constexpr int kMaxRouterSplits = 16;
inline int batch_router_splits(int hidden) {
    int s = kMaxRouterSplits;
    while (s > 1 && hidden % (64 * s)) s /= 2;
    return s;
}

hipError_t batch_router(const BatchArgs& a, hipStream_t st);
// Group-limited top-k of every token (ids, w); with convert, also the
// tokens' activations in MFMA order (xa, kx).
hipError_t batch_topk(const BatchArgs& a, bool convert, hipStream_t st);
// counts, offsets, perm, inv, distinct, tiles from ids (T*K <= kMaxDispatchEntries).
hipError_t batch_dispatch(const BatchArgs& a, hipStream_t st);
hipError_t batch_gateup(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm = {});
hipError_t batch_hprep(const BatchArgs& a, hipStream_t st);
// Gate/up + SwiGLU and down of the singles (one-token GEMVs per pair; no-ops
// when the dispatch found none).
hipError_t batch_pair_gateup(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm = {});
hipError_t batch_pair_down(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm = {});
hipError_t batch_down(const BatchArgs& a, hipStream_t st, const LaunchTiming& tm = {});
hipError_t batch_combine(const BatchArgs& a, hipStream_t st);
// Writes n (<= 256) expert blob pointers into a device table, in stream order.
struct ExpertTable {
    const uint8_t* p[256];
};
hipError_t batch_set_table(const ExpertTable& t, int n, const uint8_t** table, hipStream_t st);
bool batch_shape_supported(int hidden, int inter);
// The batched kernels serve this codec at this shape (int2: hidden a
// multiple of 512 and inter of 256, a workgroup's stored rows being twice
// as many matrix rows).
bool batch_codec_supported(int codec, int hidden, int inter);

}  // namespace moe
