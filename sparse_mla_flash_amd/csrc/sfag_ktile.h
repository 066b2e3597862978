// sfag_ktile.h -- LDS layout of a gathered tile of 32 key rows (576 16-bit elements each:
// 512 value dims + 64 rope dims) and the lane offsets that read and fill it (gfx950).
//
// A key row is 72 16-byte chunks; chunk ch of tile key k is stored at byte
//     ((ch / 8) * 32 + k) * 128 + ((ch % 8) ^ ktile_swz(k)) * 16,
// i.e. [9 groups of 8 chunks][32 keys][8 slots of 16 B], the slot XOR-swizzled per key.
//
// Filling: one direct-to-LDS load of 64 lanes x 16 bytes writes 1 KB of LDS in lane order;
// instruction (group cg, key octet q) covers keys 8 q .. 8 q + 7, each lane one slot, so it
// reads 8 whole 128-byte runs of key rows (8 keys x 8 consecutive chunks).  Loads that touch
// a few full 128-byte runs move far more data per cycle than loads that touch a 32-byte piece
// of 32 different rows.  A gathering wave that owns key octet q keeps one key per lane
// (8 q + lane / 8) for all 9 groups, so each of its loads is one add to that key's row address.
//
// Reading: LDS has 32 banks of 4 bytes; a 16-byte read is served 8 lanes per cycle, an 8-byte
// read 16 lanes per cycle.  A key row of a chunk group is 128 bytes, so every key starts at bank
// 0 and only the slot swizzle spreads them:
//   - 16-byte reads of MFMA operand fragments (8 lanes: one chunk of 8 consecutive keys):
//     ktile_swz is a bijection on each run of 8 keys;
//   - transposing reads (ds_read_b64_tr_b16; 16 lanes: two adjacent chunks, i.e. one 32-byte
//     slot pair, of 4 consecutive keys 4 g .. 4 g + 3): the slot-pair bits of ktile_swz are
//     key bits 0-1, different for the 4 keys.
// ktile_swz ignores key bits 3 and up, so key k + 16 sits exactly 2 KB after key k: a contraction
// over the tile's keys can read keys 4 g + j and 4 g + 16 + j as one MFMA fragment (any key order
// serves, as long as both operands use the same one).
#pragma once
#include <stdint.h>

namespace sfag {

constexpr int kTileKeys = 32;
constexpr int kTileGroups = 9;                         // 8 value groups + 1 rope group
constexpr int kTileBytes = kTileGroups * kTileKeys * 128;

// slot swizzle of key k: slot bits 1, 2 <- key bits 0, 1; slot bit 0 <- key bit 2
__device__ __forceinline__ int ktile_swz(int k) { return ((k & 3) << 1) | ((k >> 2) & 1); }

// Element offset (16-bit units) of chunk ch of key k.
__device__ __forceinline__ int ktile_off(int ch, int k) {
  return ((ch >> 3) * kTileKeys + k) * 64 + (((ch & 7) ^ ktile_swz(k)) << 3);
}

// Gathering lane of key octet q: its key within the tile ...
__device__ __forceinline__ int ktile_gather_key(int q, int lane) { return 8 * q + (lane >> 3); }
// ... and the byte offset inside a 128-byte run of that key's row that it loads (the same for
// every group).  The LDS destination of group cg is tile + (4 cg + q) * 1024 bytes.
__device__ __forceinline__ uint32_t ktile_gather_col(int q, int lane) {
  return (uint32_t)(((lane & 7) ^ ktile_swz(ktile_gather_key(q, lane))) << 4);
}

}  // namespace sfag
