// Dense causal attention for decode queries, for gfx950: the teacher of the
// pooler's distillation (RecSA, abstract: the pooler is distilled from dense
// attention).  out = softmax over tokens t < n of s <rope(q, n), rope(K_t, t)>,
// applied to V, with n = the cache's length.
//
// Split over the tokens, flash-decoding style: a workgroup takes one KV head, one
// span of tokens and up to kRows query rows of that head (query i, head g*G + u).
// The rows' rotated queries sit in LDS; per 64 tokens the workgroup rotates the
// keys once (cos/sin of t * theta_j in double precision, as the tree's RoPE table
// is made, since t reaches millions of radians) and stages keys and values in
// LDS.  Each wave then owns a quarter of the rows: a lane scores one token
// against a row, the wave updates that row's running (max, sum), and lane j
// accumulates output dimensions j and j + 64.  A second kernel merges the spans'
// (max, sum, acc) per row.
#include <math.h>

#include "recsa_internal.hpp"

namespace recsa {
namespace {

constexpr int kRows = 64;       // query rows per workgroup
constexpr int kTok = 64;        // tokens staged per step

__device__ __forceinline__ float ld1(const float *p) { return *p; }
__device__ __forceinline__ float ld1(const bf16_t *p) { return bf16_to_f32(*p); }

template <typename T, int D>
__global__ __launch_bounds__(256) void dense_part(DenseArgs a) {
    constexpr int DP = D + 1;                 // padded LDS row (conflict-free column reads)
    constexpr int NV = D / 64;                // output dimensions per lane
    __shared__ float qr[kRows][DP];
    __shared__ float kr[kTok][DP];
    __shared__ float vv[kTok][DP];
    __shared__ double theta[D / 2];
    __shared__ float accs[kRows][D];
    __shared__ float ml[kRows][2];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int split = blockIdx.x, g = blockIdx.y;
    const int32_t rows_g = a.B * a.G;
    const int32_t r0 = blockIdx.z * kRows;
    const int32_t nr = rows_g - r0 < kRows ? rows_g - r0 : kRows;
    const int64_t n = a.length;
    const int64_t t_begin = (int64_t)split * a.span;
    const int64_t t_end = t_begin + a.span < n ? t_begin + a.span : n;
    constexpr int H = D / 2;
    for (int j = threadIdx.x; j < H; j += 256) theta[j] = pow(a.base, -2.0 * (double)j / (double)D);
    __syncthreads();
    // the rows' queries, rotated to position n
    for (int e = threadIdx.x; e < nr * H; e += 256) {
        const int r = e / H, j = e - r * H;
        const int32_t rg = r0 + r;
        const int64_t qi = rg / a.G;
        const int h = g * a.G + (int)(rg - qi * a.G);
        const T *qp = static_cast<const T *>(a.q) + (qi * a.Hq + h) * D;
        const float x1 = ld1(qp + j), x2 = ld1(qp + H + j);
        const double ang = (double)n * theta[j];
        const float c = (float)cos(ang), s = (float)sin(ang);
        qr[r][j] = x1 * c - x2 * s;
        qr[r][H + j] = x2 * c + x1 * s;
    }
    // per wave: rows wave, wave + 4, ...; each row's running (max, sum) and output
    // accumulator live in LDS between token steps
    for (int e = threadIdx.x; e < kRows * D; e += 256) accs[e / D][e % D] = 0.f;
    for (int e = threadIdx.x; e < kRows; e += 256) {
        ml[e][0] = -INFINITY;
        ml[e][1] = 0.f;
    }
    const T *kc = static_cast<const T *>(a.k_cache) + (int64_t)g * a.cap * D;
    const T *vc = static_cast<const T *>(a.v_cache) + (int64_t)g * a.cap * D;
    constexpr float kLog2e = 1.4426950408889634f;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += kTok) {
        __syncthreads();        // the previous tokens' LDS is free (and qr, the state are written)
        for (int e = threadIdx.x; e < kTok * H; e += 256) {
            const int tt = e / H, jj = e - tt * H;
            const int64_t t = t0 + tt;
            float k1 = 0.f, k2 = 0.f, v1 = 0.f, v2 = 0.f;
            if (t < t_end) {
                k1 = ld1(kc + t * D + jj);
                k2 = ld1(kc + t * D + H + jj);
                v1 = ld1(vc + t * D + jj);
                v2 = ld1(vc + t * D + H + jj);
            }
            const double ang = (double)t * theta[jj];
            const float c = (float)cos(ang), sn = (float)sin(ang);
            kr[tt][jj] = k1 * c - k2 * sn;
            kr[tt][H + jj] = k2 * c + k1 * sn;
            vv[tt][jj] = v1;
            vv[tt][H + jj] = v2;
        }
        __syncthreads();
        const bool live = t0 + lane < t_end;
        for (int r = wave; r < nr; r += 4) {
            float dot = 0.f;
            #pragma unroll 8
            for (int jj = 0; jj < D; ++jj) dot += qr[r][jj] * kr[lane][jj];
            const float z = live ? a.scale * dot : -INFINITY;
            float mx = z;
            #pragma unroll
            for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            const float mo = ml[r][0];
            const float mn = fmaxf(mo, mx);
            const float corr = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mo - mn) * kLog2e);
            const float p = __builtin_amdgcn_exp2f((z - mn) * kLog2e);    // 0 for dead tokens
            float ps = p;
            #pragma unroll
            for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
            float o[NV];
            #pragma unroll
            for (int v = 0; v < NV; ++v) o[v] = accs[r][lane + 64 * v] * corr;
            #pragma unroll 8
            for (int tt = 0; tt < kTok; ++tt) {
                const float pt = __shfl(p, tt);
                #pragma unroll
                for (int v = 0; v < NV; ++v) o[v] += pt * vv[tt][lane + 64 * v];
            }
            #pragma unroll
            for (int v = 0; v < NV; ++v) accs[r][lane + 64 * v] = o[v];
            if (lane == 0) {
                ml[r][0] = mn;
                ml[r][1] = ml[r][1] * corr + ps;
            }
        }
    }
    __syncthreads();
    // partial state of each row: [D] acc, then m, l
    for (int r = wave; r < nr; r += 4) {
        float *dst = a.part + (((int64_t)g * a.nspan + split) * rows_g + r0 + r) * (D + 2);
        #pragma unroll
        for (int v = 0; v < NV; ++v) dst[lane + 64 * v] = accs[r][lane + 64 * v];
        if (lane == 0) {
            dst[D] = ml[r][0];
            dst[D + 1] = ml[r][1];
        }
    }
}

template <int D>
__global__ __launch_bounds__(64) void dense_merge(DenseArgs a) {
    const int lane = threadIdx.x;
    const int32_t rows_g = a.B * a.G;
    const int64_t rr = blockIdx.x;             // over Hkv * rows_g
    const int g = (int)(rr / rows_g);
    const int32_t rg = (int32_t)(rr - (int64_t)g * rows_g);
    const int64_t qi = rg / a.G;
    const int h = g * a.G + (int)(rg - qi * a.G);
    float M = -INFINITY;
    for (int sp = 0; sp < a.nspan; ++sp) {
        const float *src = a.part + (((int64_t)g * a.nspan + sp) * rows_g + rg) * (D + 2);
        M = fmaxf(M, src[D]);
    }
    constexpr int NV = D / 64;
    float o[NV] = {}, L = 0.f;
    for (int sp = 0; sp < a.nspan; ++sp) {
        const float *src = a.part + (((int64_t)g * a.nspan + sp) * rows_g + rg) * (D + 2);
        const float ms = src[D];
        const float w = ms == -INFINITY ? 0.f : expf(ms - M);
        L += w * src[D + 1];
        #pragma unroll
        for (int v = 0; v < NV; ++v) o[v] += w * src[lane + 64 * v];
    }
    const int64_t orow = (qi * a.Hq + h) * D;
    #pragma unroll
    for (int v = 0; v < NV; ++v) {
        const float x = o[v] / L;
        if (a.out_bf16) static_cast<bf16_t *>(a.out)[orow + lane + 64 * v] = (bf16_t)f32_to_bf16(x);
        else static_cast<float *>(a.out)[orow + lane + 64 * v] = x;
    }
}

template <typename T, int D>
hipError_t launch_t(const DenseArgs &a, hipStream_t s) {
    const int32_t rows_g = a.B * a.G;
    dim3 grid((unsigned)a.nspan, (unsigned)a.Hkv, (unsigned)((rows_g + kRows - 1) / kRows));
    hipLaunchKernelGGL((dense_part<T, D>), grid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dense_merge<D>), dim3((unsigned)((int64_t)a.Hkv * rows_g)), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int64_t dense_span(int64_t length) {
    // spans of a multiple of the staging step, about 1024 of them over the cache
    int64_t span = (length + 1023) / 1024;
    span = (span + kTok - 1) / kTok * kTok;
    return span < kTok ? kTok : span;
}

hipError_t launch_dense(recsa_dtype st, int32_t D, const DenseArgs &a, hipStream_t s) {
    if (a.B <= 0 || a.length <= 0) return hipSuccess;
    if (st == RECSA_BF16) return D == 128 ? launch_t<bf16_t, 128>(a, s) : launch_t<bf16_t, 64>(a, s);
    return D == 128 ? launch_t<float, 128>(a, s) : launch_t<float, 64>(a, s);
}

}  // namespace recsa
