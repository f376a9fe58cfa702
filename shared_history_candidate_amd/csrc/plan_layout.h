// Layout of the varlen plan inside the caller's workspace (host and device).
#pragma once

namespace xattn {

// A 256-byte header of int32 fields, then one int4 {r, s, c0, nc} per tile.
constexpr int kPlanHeaderBytes = 256;
constexpr int kPlanNTiles = 0;          // header[0]: number of tiles
constexpr int kPlanError = 1;           // header[1]: validation bitmask (0 = ok)
constexpr int kPlanTileM = 2;           // header[2]: candidates per tile
constexpr int kPlanMaxRequests = 4096;  // requests the single-work-group planner holds in LDS

constexpr int kErrCuKv = 1;    // cu_seqlens_kv: cu[0] != 0, decreasing, or cu[R] != total_kv
constexpr int kErrCuCand = 2;  // cu_cand: cu[0] != 0, decreasing, or cu[R] != total_cand

}  // namespace xattn
