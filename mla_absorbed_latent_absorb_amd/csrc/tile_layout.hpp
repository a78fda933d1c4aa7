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

// Raw E4M3 tile (one byte per element, as stored in the cache):
constexpr int kRawPeOff = kTile * kDc;                    // 16384: RoPE rows after 32 latent rows of 512 B
constexpr int kRawScaleOff = kRawPeOff + kTile * kDr;     // 18432: fp32 token scales (x2: every lane copies)
constexpr int kRawDummyOff = kRawScaleOff + 256;          // 18688: target of the padding copies
constexpr int kRawTileBytes = kRawDummyOff + 256;         // 18944

// LDS tile (per ring buffer):
//   [0, 32 KiB)      latent rows: row r holds 16-byte chunk c of token r at a
//                    chunk slot given by an XOR swizzle of c with a function of r
//   [32, 36 KiB)     RoPE rows: row r holds chunk c at slot c ^ pe_swizzle(r)
// A wave-wide 1 KiB direct-to-LDS copy fills one latent row (one token, so a
// scalar base address) or eight RoPE rows.
// E4M3 caches land unswizzled in a raw tile (latent row r at 512 r, RoPE row
// r at kRawPeOff + 64 r, scale of row r at kRawScaleOff + 4 r) and are
// expanded to the bf16 tile above before use.

}  // namespace mla
