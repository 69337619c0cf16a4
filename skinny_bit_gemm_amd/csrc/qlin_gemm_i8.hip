// qlin_gemm_i8.hip -- the GEMM kernel variants of one format (FMT_I8), and
// their dispatch; one source file per format so the variants build in
// parallel.
#include "qlin_gemm_big.h"

namespace qlin {

template <bool SWAP>
static gemm_fn pick(int tile_m, int nr, int xc, bool nt) {
    // token tiles of 64 / 128: the large-M kernel (Standard operand roles,
    // weights loaded straight into registers)
    if ((tile_m == 64 || tile_m == 128) && nr == 0) {
        if (SWAP || xc != 0) return nullptr;
        return tile_m == 64 ? gemm_big_kernel<FMT_I8, 64, true> : gemm_big_kernel<FMT_I8, 128, true>;
    }
#define QLIN_PICK(MT_, NR_, XC_)                                                                  \
    if (tile_m == 16 * MT_ && nr == NR_ && xc == XC_) {                                               \
        constexpr int PF_ = XC_ < 0 ? QLIN_PF_DIRECT(QLIN_PF(NR_, XC_), MT_) : QLIN_PF(NR_, XC_);   \
        return nt ? gemm_kernel<FMT_I8, SWAP, MT_, NR_, PF_, XC_, true>                               \
                  : gemm_kernel<FMT_I8, SWAP, MT_, NR_, PF_, XC_, false>;                             \
    }
    QLIN_PICK(1, 1, 0) QLIN_PICK(1, 2, 0) QLIN_PICK(1, 4, 0)
    QLIN_PICK(2, 1, 0) QLIN_PICK(2, 2, 0) QLIN_PICK(2, 4, 0)
    // 64-token tiles of the skinny kernel (codes staged in the LDS)
    QLIN_PICK(4, 1, 0) QLIN_PICK(4, 2, 0)
    QLIN_PICK(1, 1, 2) QLIN_PICK(1, 2, 2) QLIN_PICK(1, 4, 2)
    QLIN_PICK(1, 1, 4) QLIN_PICK(1, 2, 4) QLIN_PICK(1, 4, 4)
    QLIN_PICK(1, 1, 8) QLIN_PICK(1, 2, 8) QLIN_PICK(1, 4, 8)
    // direct activations (xc = -1)
    QLIN_PICK(1, 1, -1) QLIN_PICK(1, 2, -1) QLIN_PICK(1, 4, -1)
    QLIN_PICK(2, 1, -1) QLIN_PICK(2, 2, -1) QLIN_PICK(2, 4, -1)
#undef QLIN_PICK
    return nullptr;
}

gemm_fn gemm_pick_i8(bool swap, int tile_m, int nr, int xc, bool nt) {
    return swap ? pick<true>(tile_m, nr, xc, nt) : pick<false>(tile_m, nr, xc, nt);
}

}  // namespace qlin
