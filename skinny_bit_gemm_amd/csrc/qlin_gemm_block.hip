// qlin_gemm_block.hip -- the GEMM kernel variants of one format (FMT_BLOCK), and
// their dispatch; one source file per format so the variants build in
// parallel.
#include "qlin_gemm_big.h"

namespace qlin {

template <bool SWAP>
static gemm_fn pick(int tile_m, int nr, int xc) {
    // token tiles of 64 / 128: the large-M kernel (Standard operand roles)
    if (tile_m == 64 || tile_m == 128) {
        if (SWAP || xc != 0) return nullptr;
        return tile_m == 64 ? gemm_big_kernel<FMT_BLOCK, 64> : gemm_big_kernel<FMT_BLOCK, 128>;
    }
#define QLIN_PICK(MT_, NR_, XC_) \
    if (tile_m == 16 * MT_ && nr == NR_ && xc == XC_) return gemm_kernel<FMT_BLOCK, SWAP, MT_, NR_, QLIN_PF_BLOCK(NR_, XC_), XC_>;
    QLIN_PICK(1, 1, 0) QLIN_PICK(1, 2, 0) QLIN_PICK(1, 4, 0)
    QLIN_PICK(2, 1, 0) QLIN_PICK(2, 2, 0) QLIN_PICK(2, 4, 0)
    QLIN_PICK(1, 1, 2) QLIN_PICK(1, 2, 2) QLIN_PICK(1, 4, 2)
    QLIN_PICK(1, 1, 4) QLIN_PICK(1, 2, 4) QLIN_PICK(1, 4, 4)
    QLIN_PICK(1, 1, 8) QLIN_PICK(1, 2, 8) QLIN_PICK(1, 4, 8)
#undef QLIN_PICK
    return nullptr;
}

gemm_fn gemm_pick_block(bool swap, int tile_m, int nr, int xc) {
    return swap ? pick<true>(tile_m, nr, xc) : pick<false>(tile_m, nr, xc);
}

}  // namespace qlin
