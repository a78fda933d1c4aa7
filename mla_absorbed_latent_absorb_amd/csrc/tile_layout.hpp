// LDS tile of cached rows shared by the decode kernels.
#pragma once

#include "device_common.hpp"

namespace mla {

constexpr int kTile = 32;                                 // cache rows per tile
constexpr int kKvRow = kDc * 2;                           // 1024-byte latent row in LDS
constexpr int kPeRow = kDr * 2;                           // 128-byte RoPE row in LDS
constexpr int kPeRegion = kTile * kKvRow;                 // RoPE rows follow the 32 latent rows
constexpr int kTileBytes = kTile * (kKvRow + kPeRow);     // 36864
constexpr int kTileDma = kTile + kTile * kPeRow / 1024;   // 36 wave-wide 1 KiB copies per tile
constexpr float kRescaleLog2 = 8.0f;                      // lazy-rescale threshold (exp2 domain)

// LDS tile (per ring buffer):
//   [0, 32 KiB)      latent rows: row r holds 16-byte chunk c of token r at a
//                    chunk slot given by an XOR swizzle of c with a function of r
//   [32, 36 KiB)     RoPE rows: row r holds chunk c at slot c ^ pe_swizzle(r)
// A wave-wide 1 KiB direct-to-LDS copy fills one latent row (one token, so a
// scalar base address) or eight RoPE rows.

}  // namespace mla
