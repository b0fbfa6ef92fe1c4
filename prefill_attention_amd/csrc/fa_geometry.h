// Compile-time tile geometry of the gfx950 prefill attention kernel.  Every
// size the kernel and the host planner use is derived from these constants,
// so the planner's LDS request is by construction the sum of the planes the
// kernel lays out (the pages' launcher once requested more shared memory than
// its planes used and silently halved occupancy: "49 · r46 (FAP1) — FA audit",
// §2.5; a tail stage outside the formula under-allocated it in "53 · r50 —
// FA_TKV 32→16", §3.1).
#pragma once

namespace fa {

constexpr int kWaveSize = 64;          // CDNA wavefront
constexpr int kQRowsPerWave = 32;      // one 32x32 MFMA column block of queries
constexpr int kWaves = 4;              // wavefronts per work-group
constexpr int kThreads = kWaves * kWaveSize;
constexpr int kQTile = kWaves * kQRowsPerWave;  // 128 query rows per work-group
constexpr int kKvTile = 64;            // key/value rows per LDS tile
constexpr int kStages = 2;             // LDS tiles in flight (double buffer)

// Head dimensions built: the pages' model uses 128 throughout; 64 and 256
// are the same kernel with narrower or wider rows.
constexpr bool head_dim_supported(int hd) { return hd == 64 || hd == 128 || hd == 256; }

// Resident work-groups per CU: two (2 waves per SIMD, 256 registers each)
// for head_dim <= 128; one for 256, whose 128 KiB of K/V planes and 8 output
// blocks per wave need a whole CU's LDS and a SIMD's full register file.
constexpr int groups_per_cu(int hd) { return hd > 128 ? 1 : 2; }

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
constexpr int kLdsMiscBytes = 16;                                       // the merge-election flag
constexpr int lds_bytes(int hd) { return lds_k_bytes(hd) + lds_v_bytes(hd) + kLdsMiscBytes; }
// 32 KiB + 16 B (64), 64 KiB + 16 B (128), 128 KiB + 16 B (256)
constexpr int kLdsBytesMax = lds_bytes(256);

// Work-groups are dispatched round-robin over the 8 XCDs of an MI355X.
constexpr int kXcds = 8;

}  // namespace fa
