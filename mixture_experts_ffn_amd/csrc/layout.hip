// Tiled weight layout (the storage the block kernels stream).
//
// A row-major W [rows, cols] becomes 16-row x 64-column tiles, tile-row-major.
// In a tile, lane l = 16 * (c / 16) + r owns the 16 values (r, 16 (l / 16) ..
// 16 (l / 16) + 15): bf16 tiles hold the first 8 of every lane in bytes
// [0, 1024) and the last 8 in [1024, 2048), 16 bytes per lane; int8 tiles hold
// all 16 of a lane in one 16-byte piece. Each 16-byte piece a lane of a
// wavefront loads for one MFMA operand is then part of a contiguous 1 KB run.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// one thread per 16-byte output piece
template <bool INT8>
__global__ __launch_bounds__(256) void tile_weights_kernel(const char* __restrict__ src, int64_t rows,
                                                           int cols, char* __restrict__ dst) {
    constexpr int kPieces = INT8 ? 64 : 128;  // 16-byte pieces per tile
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n_tiles = (rows / 16) * (cols / 64);
    if (i >= n_tiles * kPieces) return;
    const int64_t tile = i / kPieces;
    const int piece = (int)(i - tile * kPieces);
    const int half = INT8 ? 0 : piece >> 6, lane = piece & 63;
    const int64_t cb = cols / 64;
    const int64_t ti = tile / cb, tj = tile - ti * cb;
    const int64_t r = ti * 16 + (lane & 15);
    const int64_t c = tj * 64 + (lane >> 4) * 16 + half * 8;  // first column of the piece
    const int esz = INT8 ? 1 : 2;
    *reinterpret_cast<uint4*>(dst + i * 16) =
        *reinterpret_cast<const uint4*>(src + (r * cols + c) * esz);
}

}  // namespace

hipError_t launch_tile_weights(const void* src, int64_t rows, int cols, bool int8, void* dst,
                               hipStream_t stream) {
    const int64_t pieces = (rows / 16) * (cols / 64) * (int8 ? 64 : 128);
    if (pieces <= 0) return hipSuccess;
    const dim3 grid((unsigned)((pieces + 255) / 256));
    if (int8)
        hipLaunchKernelGGL(tile_weights_kernel<true>, grid, dim3(256), 0, stream, (const char*)src,
                           rows, cols, (char*)dst);
    else
        hipLaunchKernelGGL(tile_weights_kernel<false>, grid, dim3(256), 0, stream, (const char*)src,
                           rows, cols, (char*)dst);
    return hipGetLastError();
}

}  // namespace moe
