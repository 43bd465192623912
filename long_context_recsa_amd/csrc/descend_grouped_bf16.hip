// Level-wise descent with one selection per (query, KV group): the G query heads of
// a group share each level's top-k and every key and value row they read, and keep
// their own logits and softmax (the kernels are in descend_impl.hpp).  Storage bf16.
#include "descend_impl.hpp"

namespace recsa {
namespace {
using namespace descend;

// Launch shape: 8 waves per row (a group's row carries G heads' work, and there are
// G times fewer rows than with one head per row); groups of four heads take 12 waves
// with one rank per batch within 168 registers (three waves per SIMD), which gives a
// row 1.5 times the issue slots (524K, B = 16: 50.2 -> 49.2 us; 2M, B = 32: 122 -> 116).
template <int D>
hipError_t dispatch_grouped(const TreeView &tv, const DescendArgs &a, const DebugView &dbg,
                            hipStream_t s) {
    switch (a.gs) {
        case 2: return launch_kt<bf16_t, D, 8, 4, 2>(tv, a, dbg, s);
        case 4: return launch_kt<bf16_t, D, 12, 1, 4, 3>(tv, a, dbg, s);
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
