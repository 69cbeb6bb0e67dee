// kv_copy.hpp -- measurement aid: the calibration copy with one side's blocks
// permuted.  The movers touch one side in whole pages scattered over a pool
// (the gather reads them, the chunk-major scatter writes them) and the other
// side contiguously; a copy that does the same with no block table, no plan
// and no per-unit arithmetic bounds what that access pattern allows.
#pragma once

#include "kv_move_bf16.hpp"

namespace kvmove {

// Tile b of a copy of nbytes (a multiple of the block size 2^block_shift, each
// block a multiple of the tile): block k of the permuted side is block
// (k * mult) mod n_blocks of the buffer -- a bijection, the host picks mult
// coprime with n_blocks.  kPermuteSrc: the source side is permuted, else the
// destination side.
template <int kBlock, int kVpt, bool kPermuteSrc>
__global__ __launch_bounds__(kBlock) void copy_permuted(uint64_t src, uint64_t dst, int64_t nbytes,
                                                        uint32_t block_shift, uint64_t mult)
{
    constexpr int64_t tile = (int64_t)kBlock * kVpt * 16;
    const int64_t lo = (int64_t)xcd_contiguous(blockIdx.x, gridDim.x) * tile;
    const uint64_t n_blocks = (uint64_t)nbytes >> block_shift;
    const uint64_t blk = (uint64_t)lo >> block_shift;
    const int64_t plo = (int64_t)(((blk * mult) % n_blocks) << block_shift) | (lo & ((int64_t(1) << block_shift) - 1));
    copy_tile<kBlock, kVpt, kCpolNt | kCpolSc1, kCpolNt | kCpolSc1>(src + (kPermuteSrc ? plo : lo),
                                                                   dst + (kPermuteSrc ? lo : plo), (uint32_t)tile);
}

}  // namespace kvmove
