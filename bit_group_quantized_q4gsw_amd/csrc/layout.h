// Packed q4gsw weight layout for gfx950 (layout version 2, Q4GSW_LAYOUT_VERSION).
//
// The pages prepack the weight once and let the backward read the forward's
// packed buffer without a re-pack (Vulkan q4gsw-backward PR body, "Solution" and
// "Key changes"; the WebGPU BK64 QKV PR body packs constant weights and scales
// once).  This layout is our own, chosen so one buffer feeds all three kernels:
//
//   [0, 256)                      header written by the pack kernel (flags)
//   nibble plane                  n_pad * k_pad / 2 bytes
//   scale plane                   g_pad * n_pad scales in the input dtype, row-octet major:
//                                 [n / 8][group][n % 8], so the scales of one row-octet (the
//                                 unit a decode block streams) are contiguous
//
// Nibble plane: 8x8 micro-blocks.  Micro-block (row-octet R, k-octet O) sits at
// byte 32 * (R * (k_pad / 8) + O).  Its word i (bytes 4i..4i+3) holds row 8R+i,
// columns k = 8O..8O+7.  Inside a word, k-offset j lives in nibble position
//   p(j) = (j >> 1) + 4 * (j & 1)        (bits 4p..4p+3)
// so that (word >> 4s) & 0x000F000F yields the pair (k = 2s, k = 2s+1) in the two
// 16-bit halves: a consecutive-k pair for the forward and decode kernels.  The
// input-gradient kernel builds consecutive-n pairs with one byte permute across
// two rows' words.  Byte b of a word holds, in its low and high nibble, the
// k-offsets (0,2), (4,6), (1,3), (5,7) for b = 0, 1, 2, 3.
//
// Padding: rows n >= N and columns k >= K hold code 8 (value 0); scales of
// padded rows and of groups past K are 0.  Kernels still mask activations
// beyond K and N, so padding never reads caller memory out of bounds.
#pragma once
#include <stdint.h>

namespace q4gsw {

constexpr int64_t kTileRows = 128;   // n_pad multiple
constexpr int64_t kTileCols = 128;   // k_pad multiple
constexpr uint64_t kHeaderBytes = 256;
constexpr uint64_t kAlign = 256;

// Header words (uint32) written by the pack kernels.
constexpr int kHdrBadCode = 0;      // nonzero: some code > 15
constexpr int kHdrNoFold = 1;       // nonzero: some fp16 scale cannot be folded exactly enough

struct Layout {
    int64_t n_pad, k_pad, g_pad;
    uint64_t nibble_offset, nibble_bytes, scale_offset, scale_bytes, total;
};

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

inline Layout make_layout(int64_t N, int64_t K, int64_t group_size, int scale_bytes_per) {
    Layout L;
    L.n_pad = round_up(N, kTileRows);
    L.k_pad = round_up(K, kTileCols);
    L.g_pad = (L.k_pad + group_size - 1) / group_size;
    L.nibble_offset = kHeaderBytes;
    L.nibble_bytes = (uint64_t)L.n_pad * (uint64_t)L.k_pad / 2;
    L.scale_offset = (uint64_t)round_up((int64_t)(L.nibble_offset + L.nibble_bytes), (int64_t)kAlign);
    L.scale_bytes = (uint64_t)L.g_pad * (uint64_t)L.n_pad * (uint64_t)scale_bytes_per;
    L.total = (uint64_t)round_up((int64_t)(L.scale_offset + L.scale_bytes), (int64_t)kAlign);
    return L;
}

// Index of scale[group g, row n] in the scale plane.
__host__ __device__ inline int64_t scale_index(int64_t g_pad, int64_t n, int64_t g) {
    return (n >> 3) * (g_pad * 8) + g * 8 + (n & 7);
}

// Nibble position of k-offset j (0..7) inside a word.
__host__ __device__ constexpr inline int nib_pos(int j) { return (j >> 1) + 4 * (j & 1); }

// Byte offset, inside the nibble plane, of the word holding row n, k-octet o.
__host__ __device__ inline uint64_t word_offset(int64_t k_pad, int64_t n, int64_t o) {
    return 32ull * (uint64_t)((n >> 3) * (k_pad >> 3) + o) + 4ull * (uint64_t)(n & 7);
}

}  // namespace q4gsw
