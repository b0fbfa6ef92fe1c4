// Compile-time tile geometry of the gfx950 prefill attention kernel.  Every
// size the kernel and the host planner use is derived from these constants,
// so the planner's LDS request is by construction the sum of the planes the
// kernel lays out (the pages' launcher once requested more shared memory than
// its planes used and silently halved occupancy: "49 · r46 (FAP1) — FA audit",
// §2.5; a tail stage outside the formula under-allocated it in "53 · r50 —
// FA_TKV 32→16", §3.1).
#pragma once

namespace fa {

constexpr int kHeadDim = 128;          // the only head_dim built
constexpr int kWaveSize = 64;          // CDNA wavefront
constexpr int kQRowsPerWave = 32;      // one 32x32 MFMA column block of queries
constexpr int kWaves = 4;              // wavefronts per work-group
constexpr int kThreads = kWaves * kWaveSize;
constexpr int kQTile = kWaves * kQRowsPerWave;  // 128 query rows per work-group
constexpr int kKvTile = 64;            // key/value rows per LDS tile
constexpr int kStages = 2;             // LDS tiles in flight (double buffer)
constexpr int kGroupsPerCu = 2;        // resident work-groups per CU (VGPRs: 2 waves per SIMD)

// Split-KV for grids that would leave work-group slots idle (a short chunk over
// a long KV cache): each query tile's key range is divided over up to
// kMaxSplits work-groups, each part at least kMinSplitTiles key tiles long.
constexpr int kMaxSplits = 8;
constexpr int kMinSplitTiles = 4;

// LDS planes.  K and V tiles are both stored key-major with unpadded
// 256-byte rows; the sixteen 16-byte chunks of a row are permuted by
// chunk ^ swizzle(row) (see fa_prefill.hip), which keeps both the K operand
// reads and the transposed V reads free of bank conflicts.
constexpr int kRowBytes = kHeadDim * 2;
constexpr int kTileBytes = kKvTile * kRowBytes;           // one K or one V tile: 16 KiB
constexpr int kLdsKBytes = kStages * kTileBytes;
constexpr int kLdsVBytes = kStages * kTileBytes;
constexpr int kLdsMiscBytes = 16;                         // the merge-election flag
constexpr int kLdsBytes = kLdsKBytes + kLdsVBytes + kLdsMiscBytes;  // 64 KiB + 16 B

// Work-groups are dispatched round-robin over the 8 XCDs of an MI355X.
constexpr int kXcds = 8;

}  // namespace fa
