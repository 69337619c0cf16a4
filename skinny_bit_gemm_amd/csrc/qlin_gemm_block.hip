// qlin_gemm_block.hip -- the GEMM kernel variants of one format (FMT_BLOCK), and
// their dispatch; one source file per format so the variants build in
// parallel.
#include "qlin_gemm_big.h"

namespace qlin {

template <bool SWAP>
static gemm_fn pick(int tile_m, int nr, int xc, bool nt) {
    // token tiles of 64 / 128: the large-M kernel (Standard operand roles).
    // Direct weights for 128-token tiles only: with 64-token tiles the block
    // format's per-fragment scale reads measured 1.4 % slower on geometric
    // mean than weights staged in the LDS (7.6 % faster with 128-token tiles).
    if ((tile_m == 64 || tile_m == 128) && nr == 0) {
        if (SWAP || xc != 0) return nullptr;
        return tile_m == 64 ? gemm_big_kernel<FMT_BLOCK, 64, false> : gemm_big_kernel<FMT_BLOCK, 128, true>;
    }
#define QLIN_PICK(MT_, NR_, XC_)                                                                  \
    if (tile_m == 16 * MT_ && nr == NR_ && xc == XC_) {                                               \
        constexpr int PF_ = XC_ < 0 ? QLIN_PF_DIRECT(QLIN_PF_BLOCK(NR_, XC_), MT_) : QLIN_PF_BLOCK(NR_, XC_);   \
        return nt ? gemm_kernel<FMT_BLOCK, SWAP, MT_, NR_, PF_, XC_, true>                               \
                  : gemm_kernel<FMT_BLOCK, SWAP, MT_, NR_, PF_, XC_, false>;                             \
    }
    QLIN_PICK(1, 1, 0) QLIN_PICK(1, 2, 0) QLIN_PICK(1, 4, 0)
    QLIN_PICK(2, 1, 0) QLIN_PICK(2, 2, 0) QLIN_PICK(2, 4, 0)
    // 64-token tiles of the skinny kernel (codes staged in the LDS)
    QLIN_PICK(4, 1, 0) QLIN_PICK(4, 2, 0)
    QLIN_PICK(1, 1, 2) QLIN_PICK(1, 2, 2) QLIN_PICK(1, 4, 2)
    QLIN_PICK(1, 1, 4) QLIN_PICK(1, 2, 4) QLIN_PICK(1, 4, 4)
    QLIN_PICK(1, 1, 8) QLIN_PICK(1, 2, 8) QLIN_PICK(1, 4, 8)
    // direct activations (xc = -1); the block format's Standard roles would
    // need 4 token scales per lane and block, so Swap-AB only
    if constexpr (SWAP) {
        QLIN_PICK(1, 1, -1) QLIN_PICK(1, 2, -1) QLIN_PICK(1, 4, -1)
        QLIN_PICK(2, 1, -1) QLIN_PICK(2, 2, -1) QLIN_PICK(2, 4, -1)
    }
#undef QLIN_PICK
    return nullptr;
}

gemm_fn gemm_pick_block(bool swap, int tile_m, int nr, int xc, bool nt) {
    return swap ? pick<true>(tile_m, nr, xc, nt) : pick<false>(tile_m, nr, xc, nt);
}

}  // namespace qlin
