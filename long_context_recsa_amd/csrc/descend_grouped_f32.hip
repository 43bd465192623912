// Level-wise descent with one selection per (query, KV group): the G query heads of
// a group share each level's top-k and every key and value row they read, and keep
// their own logits and softmax (the kernels are in descend_impl.hpp).  Storage f32.
#include "descend_impl.hpp"

namespace recsa {
namespace {
using namespace descend;

// Launch shape: 8 waves per row by default (a group's row carries G heads' work, and
// there are G times fewer rows than with one head per row); RECSA_DESCEND_SHAPE="4,x"
// selects 4 waves (for tuning sweeps).  fp32 rows take twice the registers of bf16
// ones, so fewer ranks per slot are in flight than in the bf16 variant.
template <int D>
hipError_t dispatch_grouped(const TreeView &tv, const DescendArgs &a, const DebugView &dbg,
                            hipStream_t s) {
    int nw = 8;
    if (const char *e = getenv("RECSA_DESCEND_SHAPE")) {
        int x = 0, y = 0;
        if (sscanf(e, "%d,%d", &x, &y) == 2) nw = x;
    }
    switch (a.gs) {
        case 2:
            if (nw == 4) return launch_kt<float, D, 4, 4, 2>(tv, a, dbg, s);
            return launch_kt<float, D, 8, 4, 2>(tv, a, dbg, s);
        case 4:
            if (nw == 4) return launch_kt<float, D, 4, 4, 4>(tv, a, dbg, s);
            return launch_kt<float, D, 8, 2, 4>(tv, a, dbg, s);
        case 8:
            if (nw == 4) return launch_kt<float, D, 4, 2, 8>(tv, a, dbg, s);
            return launch_kt<float, D, 8, 1, 8>(tv, a, dbg, s);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_descend_grouped_f32(const TreeView &tv, int32_t D, const DescendArgs &a,
                                      const DebugView &dbg, hipStream_t s) {
    if (D == 128) return dispatch_grouped<128>(tv, a, dbg, s);
    return dispatch_grouped<64>(tv, a, dbg, s);
}

}  // namespace recsa
