// Packed W4 weight and activation layouts (internal to libexactverify).
//
// Weights of an N x K W4 linear (group size G) are repacked once, exactly, into
// tiles of 16 output rows and chunks of 128 k, chunk-major (the tiles of
// chunk 0, then those of chunk 1, ...; see w4_tc_offset):
//   blob[chunk][tile] = 1024 B of nibbles + 64*(128/G) B of (scale, bias)
//   * nibbles: lane L = ln + 16 j of a wave reads 16 B at 16 L; dword t holds
//     the 8 codes q0..q7 of row 16*tile + ln for k = 128 c + 32 t + 8 j .. +7,
//     nibbles low to high q0 q2 q4 q6 q1 q3 q5 q7 (even k in the low half, odd
//     k in the high half, so that one shift and mask decodes a k-ordered pair);
//   * (scale, bias): for row ln and group g of the chunk, the fp16 pair
//     (scale | bias << 16) at 1024 + 4 (ln * GPC + g).
// Rows >= N and k >= K are padding: codes, scales and biases 0, which adds
// exactly 0 to every output.  Without padding the blob has exactly the bytes
// of the standard layout: N*K/2 + 4*N*K/G.
//
// Inside the kernel, the activations of a chunk are staged in LDS as MFMA A
// fragments: [step][lane L][16 B] = the 8 bf16 x[ln][128 c + 32 st + 8 j + i]
// for i = 0..7, a plain copy of 16 B of the row; rows >= R and k >= K are 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ev {

constexpr int kKC = 128;         // k per chunk
constexpr int kXChunkBytes = 4096;  // staged activations (A fragments) per chunk

__host__ __device__ inline int w4_tiles(int N) { return (N + 15) / 16; }
__host__ __device__ inline int w4_chunks(int K) { return (K + kKC - 1) / kKC; }
__host__ __device__ inline int w4_chunk_bytes(int G) { return 1024 + 64 * (kKC / G); }
__host__ __device__ inline size_t w4_blob_bytes(int N, int K, int G) {
    return (size_t)w4_tiles(N) * (size_t)w4_chunks(K) * (size_t)w4_chunk_bytes(G);
}

// Byte offset of tile-chunk (tile, c) in the blob: chunk-major (a chunk's
// tiles are adjacent).
__host__ __device__ inline size_t w4_tc_offset(long tile, int c, int tiles, int G) {
    return ((size_t)c * tiles + tile) * (size_t)w4_chunk_bytes(G);
}

}  // namespace ev
