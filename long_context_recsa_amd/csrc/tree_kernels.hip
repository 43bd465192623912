// Tree build and append kernels for gfx950.
//
// RecSA, abstract (sentences on the tree and the pooler): a node of the tree
// over the KV cache stands for its whole subtree through a single key and the
// average of the subtree's token values; one pooler per layer, the same at every
// level, makes the keys.  The pooler here is attention
// pooling with a per-KV-head vector w: alpha_c = softmax_c(pool_scale * w .
// child_c), key = sum_c alpha_c child_c.
//
// Level 1 is the one full scan of K and V (HBM-bound).  A wave owns one node:
// its b child rows are read with 16-byte loads, 16 lanes per row and four
// rows per wave instruction, so every 64-byte segment is consumed whole.  The
// pooler logits are reduced across the 16 lanes of a row, and softmax and the
// weighted sum run online over the rows a lane group owns; the four lane
// groups are merged with cross-lane shuffles.  Upper levels run the same
// kernel over the stored child keys and the fp32 child means.
#include <math.h>

#include "recsa_internal.hpp"

namespace recsa {
namespace {

constexpr int kNodesPerBlock = 4;     // one wave per node
constexpr int kRowsInFlight = 4;      // child rows per lane group loaded before use

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// E consecutive elements of a child row, widened to fp32.  NT (the token caches, which
// the build reads once): nontemporal loads, so the scan of K and V does not push out
// of the caches the tree levels and tables that the descent reads next.
template <typename T, int E, bool NT>
__device__ __forceinline__ void row_load(const T *p, float *out) {
    if constexpr (!NT) {
        Vec<T, E>::load(p, out);
    } else if constexpr (sizeof(T) == 2) {
        static_assert(E == 4 || E == 8, "bf16 row slice");
        uint32_t w[E / 2];
        if constexpr (E == 8) {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else {
            const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
            w[0] = v.x; w[1] = v.y;
        }
        #pragma unroll
        for (int i = 0; i < E / 2; ++i) {
            out[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
            out[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        }
    } else {
        static_assert(E % 4 == 0, "fp32 row slice");
        #pragma unroll
        for (int i = 0; i < E; i += 4) {
            const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(p + i));
            out[i] = v.x; out[i + 1] = v.y; out[i + 2] = v.z; out[i + 3] = v.w;
        }
    }
}

// KO (keys only): the pooled keys alone, for a pooler vector that changed while the
// cache did not (the means do not depend on it); child values are not read.  NT: the
// children are the token caches (level 1), read with nontemporal loads.
template <typename TK, typename TVC, typename TS, int D, bool KO, bool NT>
__global__ __launch_bounds__(64 * kNodesPerBlock) void level_kernel(
    const TK *__restrict__ child_key, int64_t child_key_stride,
    const TVC *__restrict__ child_val, int64_t child_val_stride,
    TS *__restrict__ out_key, TS *__restrict__ out_val, float *__restrict__ out_mean,
    int64_t out_stride, const float *__restrict__ pool_w, float pool_scale, int b,
    int64_t n0, int64_t n1) {
    constexpr int E = D / 16;                       // elements of a row per lane
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int grp = lane >> 4, sub = lane & 15;
    const int g = blockIdx.y;
    const int64_t node = n0 + (int64_t)blockIdx.x * kNodesPerBlock + wave;
    if (node >= n1) return;                          // whole wave leaves; no block barrier used

    const TK *ck = child_key + (int64_t)g * child_key_stride + node * b * D + sub * E;
    const TVC *cv = child_val + (int64_t)g * child_val_stride + node * b * D + sub * E;
    float w[E];
    Vec<float, E>::load(pool_w + (int64_t)g * D + sub * E, w);

    float m = -INFINITY, l = 0.f, acc[E], vacc[E];
    #pragma unroll
    for (int e = 0; e < E; ++e) { acc[e] = 0.f; vacc[e] = 0.f; }

    for (int r0 = grp; r0 < b; r0 += 4 * kRowsInFlight) {
        float kf[kRowsInFlight][E], vf[kRowsInFlight][E];
        #pragma unroll
        for (int t = 0; t < kRowsInFlight; ++t) {
            const int r = r0 + 4 * t;
            if (r < b) {
                row_load<TK, E, NT>(ck + (int64_t)r * D, kf[t]);
                if constexpr (!KO) row_load<TVC, E, NT>(cv + (int64_t)r * D, vf[t]);
            }
        }
        #pragma unroll
        for (int t = 0; t < kRowsInFlight; ++t) {
            const int r = r0 + 4 * t;
            if (r < b) {                                         // uniform within a lane group
                float s = 0.f;
                #pragma unroll
                for (int e = 0; e < E; ++e) s += w[e] * kf[t][e];
                s += __shfl_xor(s, 8, 16);
                s += __shfl_xor(s, 4, 16);
                s += __shfl_xor(s, 2, 16);
                s += __shfl_xor(s, 1, 16);
                s *= pool_scale;
                const float mn = fmaxf(m, s);
                const float c = expf(m - mn);                    // m = -inf on the first row: 0
                const float p = expf(s - mn);
                l = l * c + p;
                #pragma unroll
                for (int e = 0; e < E; ++e) {
                    acc[e] = acc[e] * c + p * kf[t][e];
                    if constexpr (!KO) vacc[e] += vf[t][e];
                }
                m = mn;
            }
        }
    }
    // merge the four lane groups (rows grp, grp+4, ...)
    #pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
        const float mo = __shfl_xor(m, off);
        const float lo = __shfl_xor(l, off);
        const float mn = fmaxf(m, mo);
        const float ca = (m == -INFINITY) ? 0.f : expf(m - mn);
        const float cb = (mo == -INFINITY) ? 0.f : expf(mo - mn);
        l = l * ca + lo * cb;
        #pragma unroll
        for (int e = 0; e < E; ++e) {
            const float ao = __shfl_xor(acc[e], off);
            acc[e] = acc[e] * ca + ao * cb;
            if constexpr (!KO) vacc[e] += __shfl_xor(vacc[e], off);
        }
        m = mn;
    }
    if (grp == 0) {
        float key[E], mean[E];
        #pragma unroll
        for (int e = 0; e < E; ++e) {
            key[e] = acc[e] / l;
            mean[e] = vacc[e] / (float)b;
        }
        const int64_t o = (int64_t)g * out_stride + node * D + sub * E;
        Vec<TS, E>::store(out_key + o, key);
        if constexpr (!KO) {
            Vec<TS, E>::store(out_val + o, mean);
            if (out_mean != nullptr) Vec<float, E>::store(out_mean + o, mean);
        }
    }
}

template <typename TK, typename TVC, typename TS, int D, bool NT>
hipError_t launch_level_t(const TK *ck, int64_t cks, const TVC *cv, int64_t cvs, TS *ok, TS *ov,
                          float *om, int64_t os, int32_t Hkv, int32_t b, int64_t n0, int64_t n1,
                          const float *pool_w, float pool_scale, bool keys_only, hipStream_t s) {
    const int64_t nodes = n1 - n0;
    dim3 grid((unsigned)((nodes + kNodesPerBlock - 1) / kNodesPerBlock), (unsigned)Hkv);
    if (keys_only)
        hipLaunchKernelGGL((level_kernel<TK, TVC, TS, D, true, NT>), grid, dim3(64 * kNodesPerBlock), 0, s,
                           ck, cks, cv, cvs, ok, ov, om, os, pool_w, pool_scale, b, n0, n1);
    else
        hipLaunchKernelGGL((level_kernel<TK, TVC, TS, D, false, NT>), grid, dim3(64 * kNodesPerBlock), 0, s,
                           ck, cks, cv, cvs, ok, ov, om, os, pool_w, pool_scale, b, n0, n1);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_level_d(const TreeView &tv, int32_t Hkv, int32_t b, int32_t level, int64_t n0,
                          int64_t n1, const float *pool_w, float pool_scale, bool ko, hipStream_t s) {
    T *ok = static_cast<T *>(tv.key[level]);
    T *ov = static_cast<T *>(tv.val[level]);
    float *om = tv.mean[level];
    const int64_t os = tv.node_cap[level] * D;
    if (level == 1) {
        return launch_level_t<T, T, T, D, true>(static_cast<const T *>(tv.k_cache), tv.cap * D,
                                          static_cast<const T *>(tv.v_cache), tv.cap * D, ok, ov,
                                          om, os, Hkv, b, n0, n1, pool_w, pool_scale, ko, s);
    }
    const T *ck = static_cast<const T *>(tv.key[level - 1]);
    const int64_t cs = tv.node_cap[level - 1] * D;
    if (tv.mean[level - 1] != nullptr)                   // bf16 storage: fp32 child means
        return launch_level_t<T, float, T, D, false>(ck, cs, tv.mean[level - 1], cs, ok, ov, om, os, Hkv,
                                              b, n0, n1, pool_w, pool_scale, ko, s);
    return launch_level_t<T, T, T, D, false>(ck, cs, static_cast<const T *>(tv.val[level - 1]), cs, ok,
                                      ov, om, os, Hkv, b, n0, n1, pool_w, pool_scale, ko, s);
}

// ---- scatter of token-major new rows into the head-major cache -------------
// K and V in one launch.  Block (x, g): head g, tokens x * tpb .. x * tpb + tpb - 1 of
// the chunk (tpb = 256 / row16), one 16-byte piece of a row per thread, so a thread's
// token and piece come from its index by a shift and a mask (row16 is a power of two).
__global__ __launch_bounds__(256) void scatter_kernel(const uint4 *__restrict__ k_src,
                                                      const uint4 *__restrict__ v_src,
                                                      uint4 *__restrict__ k_dst,
                                                      uint4 *__restrict__ v_dst, int64_t n,
                                                      int32_t Hkv, int32_t log_row16,
                                                      int64_t cap16, int64_t at16) {
    // src: [n][Hkv][row16] 16-byte pieces; dst: [Hkv][cap][row16]
    const int32_t row16 = 1 << log_row16;
    const int32_t tpb = 256 >> log_row16;
    const int64_t t = (int64_t)blockIdx.x * tpb + (threadIdx.x >> log_row16);
    if (t >= n) return;
    const int32_t c = threadIdx.x & (row16 - 1);
    const int64_t g = blockIdx.y;
    const int64_t si = (t * Hkv + g) * row16 + c;
    const int64_t di = g * cap16 + at16 + t * row16 + c;
    // the new rows are read once: nontemporal
    const u32x4 kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(k_src + si));
    const u32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(v_src + si));
    *reinterpret_cast<u32x4 *>(k_dst + di) = kv;
    *reinterpret_cast<u32x4 *>(v_dst + di) = vv;
}

// ---- RoPE table: (cos, sin) of pos * base^(-2j/D), computed in double --------
__global__ __launch_bounds__(256) void rope_table_kernel(float2 *__restrict__ table, int32_t rows,
                                                         int32_t D, double base) {
    const int h = D / 2;
    const int64_t total = (int64_t)rows * h;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t pos = i / h;
        const int j = (int)(i % h);
        const double theta = pow(base, -2.0 * (double)j / (double)D);
        const double a = (double)pos * theta;
        table[i] = make_float2((float)cos(a), (float)sin(a));
    }
}

}  // namespace

hipError_t launch_level(const TreeView &tv, recsa_dtype st, int32_t Hkv, int32_t D, int32_t b,
                        int32_t level, int64_t n0, int64_t n1, const float *pool_w,
                        float pool_scale, bool keys_only, hipStream_t s) {
    if (n1 <= n0) return hipSuccess;
    const bool ko = keys_only;
    if (st == RECSA_BF16) {
        if (D == 128) return launch_level_d<bf16_t, 128>(tv, Hkv, b, level, n0, n1, pool_w, pool_scale, ko, s);
        return launch_level_d<bf16_t, 64>(tv, Hkv, b, level, n0, n1, pool_w, pool_scale, ko, s);
    }
    if (D == 128) return launch_level_d<float, 128>(tv, Hkv, b, level, n0, n1, pool_w, pool_scale, ko, s);
    return launch_level_d<float, 64>(tv, Hkv, b, level, n0, n1, pool_w, pool_scale, ko, s);
}

hipError_t launch_scatter(const TreeView &tv, recsa_dtype st, int32_t Hkv, int32_t D,
                          const void *k_new, const void *v_new, int64_t at, int64_t n,
                          hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int32_t row16 = D * (st == RECSA_BF16 ? 2 : 4) / 16;   // 8, 16 or 32 (D = 64 or 128)
    int32_t log_row16 = 0;
    while ((1 << log_row16) < row16) ++log_row16;
    if ((1 << log_row16) != row16 || row16 > 256 || Hkv > 65535) return hipErrorInvalidValue;
    const int64_t tpb = 256 / row16;
    const int64_t bx = (n + tpb - 1) / tpb;
    if (bx > 0x7fffffff) return hipErrorInvalidValue;
    const int64_t cap16 = tv.cap * row16, at16 = at * row16;
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)bx, (unsigned)Hkv), dim3(256), 0, s,
                       static_cast<const uint4 *>(k_new), static_cast<const uint4 *>(v_new),
                       (uint4 *)tv.k_cache, (uint4 *)tv.v_cache, n, Hkv, log_row16, cap16, at16);
    return hipGetLastError();
}

hipError_t launch_rope_table(float2 *table, int32_t rows, int32_t D, double base, hipStream_t s) {
    const int64_t total = (int64_t)rows * (D / 2);
    const unsigned blocks = (unsigned)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
    hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, s, table, rows, D, base);
    return hipGetLastError();
}

}  // namespace recsa
