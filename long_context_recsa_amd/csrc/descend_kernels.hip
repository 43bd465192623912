// Level-wise descent, one query head per row (the RecSA rule: every head selects for
// itself), for decode and row-wise prefill.  The kernels are in descend_impl.hpp.
#include "descend_impl.hpp"

namespace recsa {
namespace {
using namespace descend;

// Launch shape: (waves per row, ranks per slot per pass).
// RECSA_DESCEND_SHAPE="NW,CB" overrides the choice (for tuning sweeps).
template <typename T, int D>
hipError_t dispatch(const TreeView &tv, const DescendArgs &a, const DebugView &dbg, hipStream_t s) {
    int nw = 4, cb = a.ctx_step == 0 ? 4 : 2;
    if (const char *e = getenv("RECSA_DESCEND_SHAPE")) {
        int x = 0, y = 0;
        if (sscanf(e, "%d,%d", &x, &y) == 2) { nw = x; cb = y; }
    }
    // decode (one context length for all rows): more candidates per slot in flight;
    // prefill (many rows): fewer registers, more rows resident per CU
    if (nw == 8 && cb == 4) return launch_kt<T, D, 8, 4, 1>(tv, a, dbg, s);
    if (nw == 4 && cb == 2) return launch_kt<T, D, 4, 2, 1>(tv, a, dbg, s);
    return launch_kt<T, D, 4, 4, 1>(tv, a, dbg, s);
}

}  // namespace

size_t descend_lds_bytes(int32_t maxc, int32_t k, int32_t b, int32_t D, int32_t gs) {
    switch (gs) {
        case 1: return Smem<8, 1>::bytes(maxc, k, b, D);
        case 2: return Smem<8, 2>::bytes(maxc, k, b, D);
        case 4: return Smem<8, 4>::bytes(maxc, k, b, D);
        case 8: return Smem<8, 8>::bytes(maxc, k, b, D);
        default: return ~(size_t)0;
    }
}
int32_t descend_max_candidates() { return kMaxCandidates; }

hipError_t launch_descend(const TreeView &tv, recsa_dtype st, int32_t D, const DescendArgs &a,
                          const DebugView &dbg, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    if (a.gs > 1) {
        return st == RECSA_BF16 ? launch_descend_grouped_bf16(tv, D, a, dbg, s)
                                : launch_descend_grouped_f32(tv, D, a, dbg, s);
    }
    if (st == RECSA_BF16) {
        if (D == 128) return dispatch<bf16_t, 128>(tv, a, dbg, s);
        return dispatch<bf16_t, 64>(tv, a, dbg, s);
    }
    if (D == 128) return dispatch<float, 128>(tv, a, dbg, s);
    return dispatch<float, 64>(tv, a, dbg, s);
}

}  // namespace recsa
