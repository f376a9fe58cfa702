// Layout of the varlen plan inside the caller's workspace (host and device).
#pragma once

namespace xattn {

// A 256-byte header of int32 fields, then one int4 work item per tile:
//   {kv0, L, c0, nc | (s << 16)}
// = first memory row and memory length of the tile's request, first candidate,
// candidate count (nc <= 128) and query slot (s < 64).  The attention kernels
// read everything they need about a tile in this one load.  (xattn_plan's
// public tile list is {r, s, c0, nc}.)
constexpr int kPlanHeaderBytes = 256;
constexpr int kPlanNTiles = 0;          // header[0]: number of tiles
constexpr int kPlanError = 1;           // header[1]: validation bitmask (0 = ok)
constexpr int kPlanTileM = 2;           // header[2]: candidates per tile
constexpr int kPlanMaxRequests = 4096;  // requests the single-work-group planner holds in LDS
constexpr int kInPlanMaxRequests = 16;  // batches whose attention waves plan for themselves

constexpr int kItemNcMask = 0xFFFF;     // low half of item.w: nc; high half: slot s

constexpr int kErrCuKv = 1;    // cu_seqlens_kv: cu[0] != 0, decreasing, or cu[R] != total_kv
constexpr int kErrCuCand = 2;  // cu_cand: cu[0] != 0, decreasing, or cu[R] != total_cand

}  // namespace xattn
