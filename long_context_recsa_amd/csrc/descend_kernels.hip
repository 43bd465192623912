// Level-wise descent, one query head per row (the RecSA rule: every head selects for
// itself), for decode and row-wise prefill.  The kernels are in descend_impl.hpp.
#include <atomic>

#include "descend_impl.hpp"

namespace recsa {
namespace {
using namespace descend;

// Compute units of the current device (0 if unknown), queried once per device.
int device_cus() {
    constexpr int kDevs = 64;
    static std::atomic<int> cached[kDevs];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < kDevs) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < kDevs) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Launch shape for decode (one context length for all rows).  At most one row per
// CU: bf16 rows take 12 waves and 2 ranks per slot within 168 registers (the slots
// walk a flat sequence of (child offset, rank group) pairs; 131K, B = 8: 33.5 -> 29.9
// us, 2M, B = 1: 68.5 -> 62.1 us against 8 waves and 4 ranks), fp32 rows 8 waves and
// 2 ranks.  Up to
// two rows per CU, bf16: 8 waves and 2 ranks per slot within 128 registers, so that
// two rows share a CU at 4 waves per SIMD: a row's passes are bound by its own
// instruction stream, and 8 waves give it twice the issue slots of 4 (524K, B = 16:
// 52.3 -> 45.6 us).  More rows, bf16: 4 waves and 2 ranks within 128 registers, four
// rows per CU (2M, B = 32: 213 -> 200 us against two 8-wave rows).  fp32 rows of more
// than one per CU keep 4 waves and 4 ranks.  Row-wise prefill (many rows): 4 waves, 2
// ranks.  A query keeps its selections whatever batch it is decoded in; its output
// can differ in the last bits between launch shapes, which fold the softmax in other
// groupings.
template <typename T, int D>
hipError_t dispatch(const TreeView &tv, const DescendArgs &a, const DebugView &dbg, hipStream_t s) {
    if (a.ctx_step != 0) return launch_kt<T, D, 4, 2, 1>(tv, a, dbg, s);
    if (a.rows <= device_cus()) {
        // (fp32 rows: 2 ranks per batch, or 8 waves' 256 registers would spill)
        if constexpr (sizeof(T) == 2) return launch_kt<T, D, 12, 2, 1, 3>(tv, a, dbg, s);
        else return launch_kt<T, D, 8, 2, 1>(tv, a, dbg, s);
    }
    if constexpr (sizeof(T) == 2) {
        if (a.rows > 2 * device_cus()) return launch_kt<T, D, 4, 2, 1, 4>(tv, a, dbg, s);
        return launch_kt<T, D, 8, 2, 1, 4>(tv, a, dbg, s);
    }
    else return launch_kt<T, D, 4, 4, 1>(tv, a, dbg, s);
}

}  // namespace

size_t descend_lds_bytes(int32_t maxc, int32_t k, int32_t b, int32_t D, int32_t gs) {
    switch (gs) {
        case 1: return Smem<12, 1>::bytes(maxc, k, b, D);
        case 2: return Smem<8, 2>::bytes(maxc, k, b, D);
        case 4: return Smem<12, 4>::bytes(maxc, k, b, D);
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
