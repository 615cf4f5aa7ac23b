// Device compile of a block-code mask whose blocks are the tiles (mask_blocks_dev.hip):
// the launch arguments and entry points shared by the C ABI and the kernels.
#pragma once

#include "bsfa_internal.h"

namespace bsfa {

struct DcsrBlockArgs {
    int32_t sq, sk, bq, bk, n_qt, n_kt, nbq, nbk;
    const uint8_t *codes;              // [nbq][nbk]: 0 empty, 1 full, 2 causal
    int32_t *row_cnt, *row_pcnt;       // [n_qt + 1]: entries / pieces per query tile
    int32_t *row_ptr, *row_poff;       // [n_qt + 1]: their exclusive scans
    void *temp;                        // scan scratch
    size_t temp_bytes;
    int32_t *col;                      // [nnz]
    uint8_t *tag;                      // [nnz]
    int32_t *piece_ptr;                // [nnz + 1]
    Piece *pieces;                     // [n_pieces]
    unsigned long long *totals;        // [8]: nnz, n_full, n_partial, n_pieces, pairs
};
size_t dcsr_blocks_scan_temp_bytes(int32_t n);
hipError_t launch_dcsr_blocks(const DcsrBlockArgs &a, hipStream_t stream);

}  // namespace bsfa
