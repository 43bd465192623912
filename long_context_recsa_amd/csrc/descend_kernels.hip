// Level-wise descent with candidate-index RoPE and the mixed softmax, for
// decode and (row by row) for causal prefill, on gfx950.
//
// RecSA, abstract: each level above the tokens keeps at most k candidates;
// the summaries of the candidates not kept share one softmax with the exact
// tokens; each entry's RoPE position is its index among its level's
// candidates.  The query's position at a level is that level's candidate
// count.
//
// One workgroup owns one row (a query and a query head) and walks its levels
// top-down.  A wave is four 16-lane groups; a lane group is a "slot" that
// takes every NSLOT-th candidate.  A lane holds D/32 RoPE pairs (i, i + D/2)
// of a row, so a key's rotation never crosses lanes; a key row is two
// contiguous half-row loads per lane group.  Per level:
//   1. every slot scores its candidates into LDS (rotation from the fp32
//      table computed in double at build time);
//   2. wave 0 picks the min(k, n) best (fp32 logits mapped to ordered
//      integers, packed with the inverted index so equal logits go to the
//      lower index) and writes the kept nodes, in ascending order, for the
//      next level's candidate list;
//   3. every slot folds the candidates not kept (all of them at level 0) into
//      its running softmax state; the running max is shared, so the partial
//      states of the slots add up at the end without rescaling.
#include <math.h>

#include "recsa_internal.hpp"

namespace recsa {
namespace {

constexpr int kWaves = 8;
constexpr int kSlots = kWaves * 4;
constexpr int kMaxCandidates = 4096;   // one taken-bit per lane and 64-candidate stride

__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;                     // -0 and +0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    #pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(v, off);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
    #pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

struct LevelGeom {
    int32_t n;          // candidates at this level
    int32_t nchild;     // candidates that are children of kept parents (b * kept)
    int64_t orphan0;    // node id of the first orphan
    int32_t top;        // 1 at the top level (candidate i is node i)
};

__device__ __forceinline__ int64_t cand_node(int32_t i, const LevelGeom &lg, const int32_t *parents,
                                             int32_t b, int32_t b_shift) {
    if (lg.top) return i;
    if (i < lg.nchild) {
        int32_t q, r;
        if (b_shift >= 0) {
            q = i >> b_shift;
            r = i & (b - 1);
        } else {
            q = i / b;
            r = i - q * b;
        }
        return (int64_t)parents[q] * b + r;
    }
    return lg.orphan0 + (i - lg.nchild);
}

template <typename T, int D>
__global__ __launch_bounds__(kWaves * 64) void descend_kernel(TreeView tv, DescendArgs a,
                                                              DebugView dbg, int32_t b_shift) {
    constexpr int H2 = D / 2;
    constexpr int PP = D / 32;                 // RoPE pairs per lane
    extern __shared__ __align__(16) unsigned char smem[];
    const int32_t maxc = a.max_cand;
    float *z = reinterpret_cast<float *>(smem);                           // [maxc]
    float *red = z + maxc;                                                // [kWaves][D]
    float *red_l = red + kWaves * D;                                      // [kWaves]
    float *misc = red_l + kWaves;                                         // [4]
    int32_t *kept = reinterpret_cast<int32_t *>(misc + 4);                // [2][k]
    uint8_t *flag = reinterpret_cast<uint8_t *>(kept + 2 * a.k);          // [maxc]

    const int64_t row = blockIdx.x;
    const int64_t qi = row / a.Hq;
    const int h = (int)(row - qi * a.Hq);
    const int g = h / a.G;
    const int64_t n_ctx = a.ctx_base + qi * a.ctx_step;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> 4, sub = lane & 15;
    const int slot = wave * 4 + grp;
    const int j0 = sub * PP;
    const int b = a.b;

    // levels above the tokens for this row: H = max{l : n_ctx / b^l >= 1}
    int H = 0;
    int64_t pw = 1;
    while (n_ctx / (pw * b) >= 1) { pw *= b; ++H; }

    float qa[PP], qb[PP];
    {
        const T *qp = static_cast<const T *>(a.q) + row * D;
        Vec<T, PP>::load(qp + j0, qa);
        Vec<T, PP>::load(qp + H2 + j0, qb);
    }
    const float2 *rope = tv.rope;

    float M = -INFINITY, lsum = 0.f, acc_a[PP], acc_b[PP];
    #pragma unroll
    for (int p = 0; p < PP; ++p) { acc_a[p] = 0.f; acc_b[p] = 0.f; }

    if (dbg.selected != nullptr && threadIdx.x == 0) {
        for (int l = H + 1; l <= tv.n_levels; ++l)
            for (int t = 0; t < a.k; ++t) dbg.selected[(row * tv.n_levels + l - 1) * a.k + t] = -1;
    }
    if (dbg.kth_gap != nullptr && threadIdx.x == 0) {
        for (int l = H + 1; l <= tv.n_levels; ++l) dbg.kth_gap[row * tv.n_levels + l - 1] = NAN;
    }

    int32_t kept_prev = 0;
    int64_t keys_scored = 0;
    for (int l = H; l >= 0; --l, pw /= b) {
        const int64_t Nl = n_ctx / pw;
        LevelGeom lg;
        lg.top = (l == H);
        if (lg.top) {
            lg.n = (int32_t)Nl;
            lg.nchild = 0;
            lg.orphan0 = 0;
        } else {
            const int64_t Nup = n_ctx / (pw * b);
            lg.nchild = b * kept_prev;
            lg.orphan0 = Nup * b;
            lg.n = lg.nchild + (int32_t)(Nl - Nup * b);
        }
        const int32_t n = lg.n;
        const int32_t *parents = kept + ((l + 1) & 1) * a.k;
        int32_t *kept_now = kept + (l & 1) * a.k;
        const T *kbase, *vbase;
        if (l == 0) {
            kbase = static_cast<const T *>(tv.k_cache) + (int64_t)g * tv.cap * D;
            vbase = static_cast<const T *>(tv.v_cache) + (int64_t)g * tv.cap * D;
        } else {
            kbase = static_cast<const T *>(tv.key[l]) + (int64_t)g * tv.node_cap[l] * D;
            vbase = static_cast<const T *>(tv.val[l]) + (int64_t)g * tv.node_cap[l] * D;
        }

        // query at position n (this level's candidate count)
        float qra[PP], qrb[PP];
        #pragma unroll
        for (int p = 0; p < PP; ++p) {
            const float2 cs = rope[(int64_t)n * H2 + j0 + p];
            qra[p] = qa[p] * cs.x - qb[p] * cs.y;
            qrb[p] = qb[p] * cs.x + qa[p] * cs.y;
        }

        // 1. score every candidate
        for (int32_t i = slot; i < n; i += kSlots) {
            const int64_t node = cand_node(i, lg, parents, b, b_shift);
            float ka[PP], kb[PP];
            Vec<T, PP>::load(kbase + node * D + j0, ka);
            Vec<T, PP>::load(kbase + node * D + H2 + j0, kb);
            float dot = 0.f;
            #pragma unroll
            for (int p = 0; p < PP; ++p) {
                const float2 cs = rope[(int64_t)i * H2 + j0 + p];
                const float ra = ka[p] * cs.x - kb[p] * cs.y;
                const float rb = kb[p] * cs.x + ka[p] * cs.y;
                dot += qra[p] * ra + qrb[p] * rb;
            }
            dot += __shfl_xor(dot, 8, 16);
            dot += __shfl_xor(dot, 4, 16);
            dot += __shfl_xor(dot, 2, 16);
            dot += __shfl_xor(dot, 1, 16);
            if (sub == 0) {
                z[i] = a.scale * dot;
                flag[i] = 0;
            }
        }
        keys_scored += n;
        __syncthreads();

        // 2. selection (wave 0)
        const int32_t m = (l > 0) ? (a.k < n ? a.k : n) : 0;
        if (wave == 0) {
            if (l > 0) {
                uint64_t taken = 0;
                float zmax = 0.f, zm = 0.f, zm1 = NAN;
                const int rounds = (n > m) ? m + 1 : m;
                for (int r = 0; r < rounds; ++r) {
                    uint64_t best = 0;
                    int t = 0;
                    for (int32_t i = lane; i < n; i += 64, ++t) {
                        if (!((taken >> t) & 1ull)) {
                            const uint64_t key = ((uint64_t)ordered_bits(z[i]) << 32) |
                                                 (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
                            best = key > best ? key : best;
                        }
                    }
                    best = wave_max_u64(best);
                    const int32_t idx = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
                    const float zv = z[idx];
                    if (r == 0) zmax = zv;
                    if (r < m) {
                        if ((idx & 63) == lane) taken |= 1ull << (idx >> 6);
                        if (r == m - 1) zm = zv;
                    } else {
                        zm1 = zv;
                    }
                }
                // ascending compaction of the kept candidates
                int32_t cnt = 0;
                int t = 0;
                for (int32_t base = 0; base < n; base += 64, ++t) {
                    const int32_t i = base + lane;
                    const bool f = (i < n) && ((taken >> t) & 1ull);
                    const uint64_t mask = __ballot(f);
                    if (f) {
                        const int32_t pos = cnt + __popcll(mask & ((1ull << lane) - 1ull));
                        const int64_t node = cand_node(i, lg, parents, b, b_shift);
                        kept_now[pos] = (int32_t)node;
                        flag[i] = 1;
                        if (dbg.selected != nullptr)
                            dbg.selected[(row * tv.n_levels + l - 1) * a.k + pos] = (int32_t)node;
                    }
                    cnt += __popcll(mask);
                }
                if (lane == 0) {
                    misc[0] = zmax;
                    if (dbg.kth_gap != nullptr)
                        dbg.kth_gap[row * tv.n_levels + l - 1] = (n > m) ? zm - zm1 : NAN;
                    if (dbg.selected != nullptr)
                        for (int q = m; q < a.k; ++q)
                            dbg.selected[(row * tv.n_levels + l - 1) * a.k + q] = -1;
                }
            } else {
                float mx = -INFINITY;
                for (int32_t i = lane; i < n; i += 64) mx = fmaxf(mx, z[i]);
                mx = wave_max_f32(mx);
                if (lane == 0) misc[0] = mx;
            }
        }
        __syncthreads();

        // 3. fold the entries of this level into the running softmax
        const float Mn = fmaxf(M, misc[0]);
        const float corr = (M == -INFINITY) ? 0.f : expf(M - Mn);
        lsum *= corr;
        #pragma unroll
        for (int p = 0; p < PP; ++p) { acc_a[p] *= corr; acc_b[p] *= corr; }
        M = Mn;
        for (int32_t i = slot; i < n; i += kSlots) {
            if (l > 0 && flag[i]) continue;
            const int64_t node = cand_node(i, lg, parents, b, b_shift);
            const float pz = expf(z[i] - M);
            float va[PP], vb[PP];
            Vec<T, PP>::load(vbase + node * D + j0, va);
            Vec<T, PP>::load(vbase + node * D + H2 + j0, vb);
            lsum += pz;
            #pragma unroll
            for (int p = 0; p < PP; ++p) {
                acc_a[p] += pz * va[p];
                acc_b[p] += pz * vb[p];
            }
        }
        kept_prev = m;
    }

    // combine the slots: four lane groups by shuffles, the waves through LDS
    #pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
        lsum += __shfl_xor(lsum, off);
        #pragma unroll
        for (int p = 0; p < PP; ++p) {
            acc_a[p] += __shfl_xor(acc_a[p], off);
            acc_b[p] += __shfl_xor(acc_b[p], off);
        }
    }
    if (grp == 0) {
        #pragma unroll
        for (int p = 0; p < PP; ++p) {
            red[wave * D + j0 + p] = acc_a[p];
            red[wave * D + H2 + j0 + p] = acc_b[p];
        }
        if (sub == 0) red_l[wave] = lsum;
    }
    __syncthreads();
    if (wave == 0 && grp == 0) {
        float oa[PP], ob[PP], L = 0.f;
        #pragma unroll
        for (int p = 0; p < PP; ++p) { oa[p] = 0.f; ob[p] = 0.f; }
        for (int w = 0; w < kWaves; ++w) {
            L += red_l[w];
            #pragma unroll
            for (int p = 0; p < PP; ++p) {
                oa[p] += red[w * D + j0 + p];
                ob[p] += red[w * D + H2 + j0 + p];
            }
        }
        #pragma unroll
        for (int p = 0; p < PP; ++p) { oa[p] /= L; ob[p] /= L; }
        if (a.out_bf16) {
            bf16_t *o = static_cast<bf16_t *>(a.out) + row * D;
            Vec<bf16_t, PP>::store(o + j0, oa);
            Vec<bf16_t, PP>::store(o + H2 + j0, ob);
        } else {
            float *o = static_cast<float *>(a.out) + row * D;
            Vec<float, PP>::store(o + j0, oa);
            Vec<float, PP>::store(o + H2 + j0, ob);
        }
        if (sub == 0 && dbg.n_keys != nullptr) dbg.n_keys[row] = (int32_t)keys_scored;
    }
}

size_t descend_smem(int32_t maxc, int32_t k, int D) {
    return sizeof(float) * ((size_t)maxc + (size_t)kWaves * D + kWaves + 4) +
           sizeof(int32_t) * 2 * (size_t)k + (size_t)maxc;
}

template <typename T, int D>
hipError_t launch_descend_t(const TreeView &tv, const DescendArgs &a, const DebugView &dbg,
                            hipStream_t s) {
    const size_t smem = descend_smem(a.max_cand, a.k, D);
    if (smem > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)descend_kernel<T, D>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    int32_t b_shift = -1;
    if ((a.b & (a.b - 1)) == 0) {
        b_shift = 0;
        while ((1 << b_shift) < a.b) ++b_shift;
    }
    hipLaunchKernelGGL((descend_kernel<T, D>), dim3((unsigned)a.rows), dim3(kWaves * 64), smem, s,
                       tv, a, dbg, b_shift);
    return hipGetLastError();
}

}  // namespace

size_t descend_lds_bytes(int32_t maxc, int32_t k, int32_t D) { return descend_smem(maxc, k, D); }
int32_t descend_max_candidates() { return kMaxCandidates; }

hipError_t launch_descend(const TreeView &tv, recsa_dtype st, int32_t D, const DescendArgs &a,
                          const DebugView &dbg, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    if (st == RECSA_BF16) {
        if (D == 128) return launch_descend_t<bf16_t, 128>(tv, a, dbg, s);
        return launch_descend_t<bf16_t, 64>(tv, a, dbg, s);
    }
    if (D == 128) return launch_descend_t<float, 128>(tv, a, dbg, s);
    return launch_descend_t<float, 64>(tv, a, dbg, s);
}

}  // namespace recsa
