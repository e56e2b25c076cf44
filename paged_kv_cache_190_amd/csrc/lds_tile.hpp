// LDS staging of 32-key K/V tiles for the matrix-core kernels (chunked prefill, and the shared
// prefix chunks of the prefix-aware decode): the DMA (global_load_lds) writes each wave's 64
// lanes to 1 KiB of consecutive LDS, 16 bytes per lane, so tile rows cannot be padded; their
// 16-byte chunks are XOR-permuted instead.
#pragma once

#include "common.hpp"

namespace pkv {

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding and
// leaves the other counters alone (gfx9 encoding: vmcnt split over bits 3:0 and 15:14).
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// s_waitcnt immediate that waits for every LDS (and scalar-memory) operation and leaves the
// vector-memory and export counters alone.
constexpr int waitcnt_lgkm0() { return 0xF | (0x3 << 14) | (0x7 << 4); }

// XOR swizzles of the 16-byte chunks of the LDS tiles, chosen so that the sixteen lanes a
// 128-bit LDS read serves together (64 banks x 4 bytes) hit sixteen different 16-byte bank
// groups. K tiles are [32 keys][D]; their rows are read in the order krow(col) of the kernels,
// i.e. rows {0..3, 16..19, 4..7, 20..23} for lanes 0..15 and {8..11, 24..27, 12..15, 28..31}
// for lanes 16..31. V tiles are [D][32 keys], rows d read in order.
// (constexpr: also callable on the host, where a test checks the layout)
template <int D>
constexpr int kswz(int row) {
  if constexpr (D == 128) return (row & 7) | ((row >> 1) & 8);       // 16 chunks per row
  else return ((row >> 1) & 3) | ((row >> 2) & 4);                   // 8 chunks, 2 rows per line
}
constexpr int vswz(int d) { return (d >> 2) & 3; }  // 4 chunks, 4 rows per line

}  // namespace pkv
