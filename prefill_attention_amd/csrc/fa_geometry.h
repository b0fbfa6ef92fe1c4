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

// LDS planes (f16 elements).  K is stored as rows of head_dim, V transposed
// as rows of kv_tile; the pads make consecutive rows start 16 bytes apart
// modulo 128 bytes, so the eight 16-byte row fragments read by one group of
// lanes fall on distinct banks.
constexpr int kKStride = kHeadDim + 8;   // 136 halves = 272 B per key row
constexpr int kVtStride = kKvTile + 8;   // 72 halves = 144 B per head-dim row
constexpr int kLdsKBytes = kKvTile * kKStride * 2;
constexpr int kLdsVtBytes = kHeadDim * kVtStride * 2;
constexpr int kLdsBytes = kLdsKBytes + kLdsVtBytes;

// Work-groups are dispatched round-robin over the 8 XCDs of an MI355X.
constexpr int kXcds = 8;

}  // namespace fa
