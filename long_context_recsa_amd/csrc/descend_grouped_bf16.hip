// Level-wise descent with one selection per (query, KV group): the G query heads of
// a group share each level's top-k and every key and value row they read, and keep
// their own logits and softmax (the kernels are in descend_impl.hpp).  Storage bf16.
#include "descend_impl.hpp"

namespace recsa {
namespace {
using namespace descend;

// Launch shape: 8 waves per row (a group's row carries G heads' work, and there are
// G times fewer rows than with one head per row).
template <int D>
hipError_t dispatch_grouped(const TreeView &tv, const DescendArgs &a, const DebugView &dbg,
                            hipStream_t s) {
    switch (a.gs) {
        case 2: return launch_kt<bf16_t, D, 8, 4, 2>(tv, a, dbg, s);
        case 4: return launch_kt<bf16_t, D, 8, 2, 4>(tv, a, dbg, s);
        case 8: return launch_kt<bf16_t, D, 8, 1, 8>(tv, a, dbg, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_descend_grouped_bf16(const TreeView &tv, int32_t D, const DescendArgs &a,
                                      const DebugView &dbg, hipStream_t s) {
    if (D == 128) return dispatch_grouped<128>(tv, a, dbg, s);
    return dispatch_grouped<64>(tv, a, dbg, s);
}

}  // namespace recsa
