// Compile-time tile geometry of the gfx950 prefill attention kernel.  Every
// size the kernel and the host planner use is derived from these constants,
// so the planner's LDS request is by construction the sum of the planes the
// kernel lays out (the pages' launcher once requested more shared memory than
// its planes used and silently halved occupancy: "49 · r46 (FAP1) — FA audit",
// §2.5; a tail stage outside the formula under-allocated it in "53 · r50 —
// FA_TKV 32→16", §3.1).
#pragma once

namespace fa {

// Key/value tile width and wavefronts per work-group are build-time
// parameters (FA_KV_TILE in {32, 64, 128}, FA_WAVES in {4, 8}; build.py
// --kv-tile / --waves).  The library ships 64 and 4: of the six
// combinations, measured on every benchmark shape with rocprof counters
// (MFMA-busy cycles, dependency waits, LDS bank conflicts, occupancy), it is
// the fastest everywhere.
#ifndef FA_KV_TILE
#define FA_KV_TILE 64
#endif
#ifndef FA_WAVES
#define FA_WAVES 4
#endif
constexpr int kWaveSize = 64;          // CDNA wavefront
constexpr int kQRowsPerWave = 32;      // one 32x32 MFMA column block of queries
constexpr int kWaves = FA_WAVES;       // wavefronts per work-group
constexpr int kThreads = kWaves * kWaveSize;
constexpr int kQTile = kWaves * kQRowsPerWave;  // query rows per work-group (128)
constexpr int kKvTile = FA_KV_TILE;    // key/value rows per LDS tile (64)
constexpr int kKb = kKvTile / 32;      // 32-key accumulator blocks per tile
constexpr int kKs = kKvTile / 16;      // 16-key MFMA k-steps per tile
static_assert(kKvTile == 32 || kKvTile == 64 || kKvTile == 128, "FA_KV_TILE must be 32, 64 or 128");
static_assert(kWaves == 4 || kWaves == 8, "FA_WAVES must be 4 or 8");
constexpr int kStages = 2;             // LDS tiles in flight (double buffer)


// Split-KV for grids that would leave work-group slots idle (a short chunk over
// a long KV cache, or a prefill of few heads): each query tile's key range is
// divided over up to kMaxSplits work-groups, each part at least
// kMinSplitTiles shared key tiles long.
constexpr int kMaxSplits = 8;
constexpr int kMinSplitTiles = 20;
// Relative time per key tile of a work-group that shares its CU with another
// (the older of the two), against one alone on its CU (measured 1.69 vs 1.37 us).
constexpr double kSharedPartCost = 1.25;

// Phase-A issue priority is used when the heaviest work-group carries at most
// this many times the average key tiles per resident work-group slot.
constexpr double kPriorityMaxImbalance = 1.25;

// LDS planes.  K and V tiles are both stored key-major with unpadded rows of
// head_dim 16-bit elements; the 16-byte chunks of a row are permuted by
// chunk ^ swizzle(row) (see the kernel), which keeps both the K operand
// reads and the transposed V reads free of bank conflicts.
constexpr int row_bytes(int hd) { return hd * 2; }
constexpr int tile_bytes(int hd) { return kKvTile * row_bytes(hd); }   // one K or V tile
constexpr int lds_k_bytes(int hd) { return kStages * tile_bytes(hd); }
constexpr int lds_v_bytes(int hd) { return kStages * tile_bytes(hd); }
// Query plane.  Each wave copies its 32 query rows into LDS (the K tiles'
// direct-to-LDS loads and chunk permutation: whole rows per instruction) and
// reads its Q^T fragments from there once.  The first kQWavesInStage waves
// use the second V stage, which is free until the first step stages V(1);
// the others use this plane.  A split launch's merge-election flag reuses the
// plane after the prologue, so it is at least 16 bytes.
constexpr int kQWavesInStage = kKvTile / kQRowsPerWave < kWaves ? kKvTile / kQRowsPerWave : kWaves;
constexpr int kLdsFlagBytes = 16;
constexpr int lds_q_bytes(int hd) {
    return (kWaves - kQWavesInStage) * kQRowsPerWave * row_bytes(hd) > kLdsFlagBytes
               ? (kWaves - kQWavesInStage) * kQRowsPerWave * row_bytes(hd)
               : kLdsFlagBytes;
}
// The epilogue reuses the planes to write each wave's 32 f32 output rows
// row-major; a work-group needs the larger of the two.
constexpr int lds_epilogue_bytes(int hd) { return kWaves * kQRowsPerWave * hd * 4; }
constexpr int lds_planes_bytes(int hd) { return lds_k_bytes(hd) + lds_v_bytes(hd) + lds_q_bytes(hd); }
constexpr int lds_bytes(int hd) {
    return lds_planes_bytes(hd) > lds_epilogue_bytes(hd) ? lds_planes_bytes(hd) : lds_epilogue_bytes(hd);
}
// Shipped geometry: 40 KiB (head_dim 64), 80 KiB (128), 160 KiB (256)
constexpr int kCuLdsBytes = 160 * 1024;  // LDS of one gfx950 compute unit

// Head dimensions built: the pages' model uses 128 throughout; 64 and 256
// are the same kernel with narrower or wider rows.  A geometry supports a
// head dimension when each wave's share of a key tile is a whole number of
// direct-to-LDS copies (64 lanes x 16 B: 64 / (hd / 8) rows each) and the
// work-group's LDS fits a compute unit.
constexpr bool head_dim_supported(int hd) {
    return (hd == 64 || hd == 128 || hd == 256) && (kKvTile / kWaves) % (64 / (hd / 8)) == 0 &&
           lds_bytes(hd) <= kCuLdsBytes;
}

// Resident work-groups per CU: two (2 waves per SIMD, 256 registers each)
// for 4-wave groups whose LDS fits twice (head_dim <= 128 with 64-key
// tiles); otherwise one: head_dim 256's 160 KiB of planes and 8 output
// blocks per wave need a whole CU's LDS and a SIMD's full register file, and
// an 8-wave group already puts 2 waves on each SIMD.
constexpr int groups_per_cu(int hd) { return (kWaves == 4 && 2 * lds_bytes(hd) <= kCuLdsBytes) ? 2 : 1; }

// Work-groups are dispatched round-robin over the 8 XCDs of an MI355X.
constexpr int kXcds = 8;

}  // namespace fa
