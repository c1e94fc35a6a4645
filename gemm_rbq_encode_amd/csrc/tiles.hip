// tiles.hip -- the tile layout of the sign planes (RBQ_LAYOUT_TILES).
//
// The planes are the pages' packed binary matrices, 32 columns per 32-bit
// word ("RaBiT" summary, paperlayer.ai, section D "GPU implementation").
// The one-token kernels split a matrix into units of 16 rows by 512
// columns; in the row layout one unit of one plane is 16 runs of 64 bytes
// (half a 128-byte line each), in the tile layout it is one contiguous 1 KB
// block, in the order in which the 64 lanes of a wave take it: lane
// (i, g) = (lane % 16, lane / 16) holds words 4g .. 4g+3 of row i of the
// unit, at block offset 16 * (16 g + i) bytes.
//
//   tiles[k][t][c][g][i][j] = planes[k][16t + i][16c + 4g + j]   (0 outside)
//
// The copy is a permutation of 16-byte pieces: one thread per piece of the
// output, reading 16 bytes (or none, for padding) and writing 16.  The scales
// of a layer with one scale per 128-column group get a tile layout of their
// own below.
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int TL_THREADS = 256;

__global__ __launch_bounds__(TL_THREADS) void pack_tiles_kernel(const uint32_t *__restrict__ planes, int K,
                                                                int out, int words, int T, int C,
                                                                v4u *__restrict__ tiles) {
    // pieces: K * T * C blocks of 64
    const size_t n = (size_t)K * T * C * 64;
    for (size_t p = (size_t)blockIdx.x * TL_THREADS + threadIdx.x; p < n; p += (size_t)gridDim.x * TL_THREADS) {
        const int lane = (int)(p & 63);
        const size_t blk = p >> 6;                  // (k, t, c)
        const int c = (int)(blk % C);
        const size_t kt = blk / C;
        const int t = (int)(kt % T), k = (int)(kt / T);
        const int row = 16 * t + (lane & 15);
        const int w = 16 * c + 4 * (lane >> 4);
        v4u v = (v4u){0u, 0u, 0u, 0u};
        if (row < out && w < words)                 // words % 4 == 0: a piece is all in or all out
            v = *reinterpret_cast<const v4u *>(planes + ((size_t)k * out + row) * words + w);
        tiles[p] = v;
    }
}

// Scale tiles of a g128 layer: per unit (16 rows x 512 columns = 4 groups)
// the K planes' scales of its 16 rows and 4 groups, 128 bytes per plane, so
// that the one-token kernels load them with the unit's planes:
//   stiles[t][c][p][g][q][kk][v] = scales[2p + kk][16t + 4q + v][4c + g]
// (p < K/2 plane pairs, g < 4 groups, q < 4 row quads, v < 4 rows; 0 outside).
// Lane (i, q) of a wave -- MFMA column i = 3g + limb -- reads the 16 bytes at
// [p][min(i / 3, 3)][q]: both planes of pair p, rows 4q .. 4q+3 of group g.
__global__ __launch_bounds__(TL_THREADS) void pack_scale_tiles_kernel(const uint16_t *__restrict__ scales, int K,
                                                                      int out, int G, int T, int C,
                                                                      v4u *__restrict__ stiles) {
    const int KS = K / 2;
    const size_t n = (size_t)T * C * KS * 16;      // 16-byte pieces
    for (size_t p = (size_t)blockIdx.x * TL_THREADS + threadIdx.x; p < n; p += (size_t)gridDim.x * TL_THREADS) {
        const int q = (int)(p & 3), g = (int)((p >> 2) & 3);
        const size_t up = p >> 4;                   // (unit, pair)
        const int pp = (int)(up % KS);
        const size_t unit = up / KS;
        const int c = (int)(unit % C), t = (int)(unit / C);
        const int grp = 4 * c + g;
        uint16_t h[8];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 16 * t + 4 * q + v;
                h[4 * kk + v] = (row < out && grp < G) ? scales[((size_t)(2 * pp + kk) * out + row) * G + grp]
                                                       : (uint16_t)0;
            }
        stiles[p] = (v4u){h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                          h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
    }
}

}  // namespace

size_t scale_tiles_bytes(int K, int out, int in) {
    const size_t T = ((size_t)out + 15) / 16, C = ((size_t)in + 511) / 512;
    return T * C * (size_t)K * 128;
}

hipError_t launch_pack_scale_tiles(const uint16_t *scales, int K, int out, int in, uint16_t *stiles,
                                   hipStream_t st) {
    const int T = (out + 15) / 16, C = (in + 511) / 512;
    const size_t pieces = (size_t)T * C * (K / 2) * 16;
    const size_t want = (pieces + TL_THREADS - 1) / TL_THREADS;
    const int grid = (int)(want < 8192 ? want : 8192);
    hipLaunchKernelGGL(pack_scale_tiles_kernel, dim3(grid), dim3(TL_THREADS), 0, st, scales, K, out, in / 128, T, C,
                       reinterpret_cast<v4u *>(stiles));
    return hipGetLastError();
}

size_t tiles_bytes(int K, int out, int in) {
    const size_t T = ((size_t)out + 15) / 16, C = ((size_t)in + 511) / 512;
    return (size_t)K * T * C * 1024;
}

hipError_t launch_pack_tiles(const uint32_t *planes, int K, int out, int in, uint32_t *tiles, hipStream_t st) {
    const int words = in / 32;
    const int T = (out + 15) / 16, C = (in + 511) / 512;
    const size_t pieces = (size_t)K * T * C * 64;
    const size_t want = (pieces + TL_THREADS - 1) / TL_THREADS;
    const int grid = (int)(want < 8192 ? want : 8192);
    hipLaunchKernelGGL(pack_tiles_kernel, dim3(grid), dim3(TL_THREADS), 0, st, planes, K, out, words, T, C,
                       reinterpret_cast<v4u *>(tiles));
    return hipGetLastError();
}

}  // namespace rbq
