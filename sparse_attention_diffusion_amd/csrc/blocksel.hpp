// Launcher interface of the block-sparse selector (blocksel.hip), the baseline
// of the matched-density comparison.
#pragma once

#include "kernels.hpp"

namespace mcs {

// Workspace: the fp32 block means of Q and K, 2 * H * (N / 64) * D floats.
size_t block_select_ws_bytes(int H, int N, int D);
// Whether one (head, query block) selection fits in LDS (N / 64 sort keys).
bool block_select_fits(int N, int D);
// N a multiple of 64; kb = K / 64 key blocks per query block; idx [H][N/64][kpad].
hipError_t launch_block_select(const void* q, const void* k, int dtype, int H, int N, int D, int kb, int kpad,
                               float scale, int32_t* idx, void* ws, hipStream_t s);

}  // namespace mcs
