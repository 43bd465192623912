// Dense causal attention for decode queries, for gfx950: the teacher of the
// pooler's distillation (RecSA, abstract, sentence on the pooler: full attention
// is the pooler's teacher).  out = softmax over tokens t < n of s <rope(q, n), rope(K_t, t)>,
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
//
// bf16 storage takes dense_mfma instead: the same spans and per-span states, with a
// wave per 16 query rows and q.K and P.V on bf16 MFMA (16x16x32, fp32 accumulate).
// The rotated queries and keys are fp32, so each is split into a bf16 high and low
// part and the logits take three products (about 16 significant bits); P is split
// the same way against the values, which are exact in bf16.  Key rotations use
// cos/sin of (t0 + tt) theta_j from the step's base angle t0 theta_j (double
// precision) and a table of tt theta_j, tt < 64, by angle addition.
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
__global__ __launch_bounds__(256) void dense_merge(DenseArgs a) {
    // one row per workgroup; wave w merges the spans w, w + 4, ... online (running max,
    // rescaled sums), then the four partial states combine through LDS
    constexpr int NV = D / 64;
    __shared__ float wm[4], wl[4];
    __shared__ float wo[4][D];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int32_t rows_g = a.B * a.G;
    const int64_t rr = blockIdx.x;             // over Hkv * rows_g
    const int g = (int)(rr / rows_g);
    const int32_t rg = (int32_t)(rr - (int64_t)g * rows_g);
    float M = -INFINITY, L = 0.f, o[NV] = {};
    for (int sp = wave; sp < a.nspan; sp += 4) {
        const float *src = a.part + (((int64_t)g * a.nspan + sp) * rows_g + rg) * (D + 2);
        const float ms = src[D];
        if (ms == -INFINITY) continue;
        const float mn = fmaxf(M, ms);
        const float cold = M == -INFINITY ? 0.f : expf(M - mn), cnew = expf(ms - mn);
        L = L * cold + cnew * src[D + 1];
        #pragma unroll
        for (int v = 0; v < NV; ++v) o[v] = o[v] * cold + cnew * src[lane + 64 * v];
        M = mn;
    }
    if (lane == 0) {
        wm[wave] = M;
        wl[wave] = L;
    }
    #pragma unroll
    for (int v = 0; v < NV; ++v) wo[wave][lane + 64 * v] = o[v];
    __syncthreads();
    if (wave != 0) return;
    float Mt = -INFINITY;
    for (int w = 0; w < 4; ++w) Mt = fmaxf(Mt, wm[w]);
    float Lt = 0.f, ot[NV] = {};
    for (int w = 0; w < 4; ++w) {
        if (wm[w] == -INFINITY) continue;
        const float c = expf(wm[w] - Mt);
        Lt += c * wl[w];
        #pragma unroll
        for (int v = 0; v < NV; ++v) ot[v] += c * wo[w][lane + 64 * v];
    }
    const int64_t qi = rg / a.G;
    const int h = g * a.G + (int)(rg - qi * a.G);
    const int64_t orow = (qi * a.Hq + h) * D;
    #pragma unroll
    for (int v = 0; v < NV; ++v) {
        const float x = ot[v] / Lt;
        if (a.out_bf16) static_cast<bf16_t *>(a.out)[orow + lane + 64 * v] = (bf16_t)f32_to_bf16(x);
        else static_cast<float *>(a.out)[orow + lane + 64 * v] = x;
    }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// x ~ hi + lo with both parts bf16
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
    #pragma unroll
    for (int v = 0; v < 8; ++v) {
        const __bf16 h = (__bf16)x[v];
        hi[v] = h;
        lo[v] = (__bf16)(x[v] - (float)h);
    }
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// (cos, sin) of tt * theta_j for tt < kTok, row-major [tt][j], double precision angles.
__global__ void dense_incr(float2 *incr, int D, double base) {
    const int H = D / 2;
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= kTok * H) return;
    const int tt = e / H, j = e - tt * H;
    const double ang = (double)tt * pow(base, -2.0 * (double)j / (double)D);
    incr[e] = make_float2((float)cos(ang), (float)sin(ang));
}

constexpr int kMRows = 64;      // query rows per workgroup: 4 waves x 16

// MFMA 16x16x32: lane L supplies A row L%16 and B column L%16 for the 8 k-slots of lane
// group grp = L/16, and gets D rows 4*grp .. 4*grp + 3 of column L%16.
template <int D>
__global__ __launch_bounds__(256) void dense_mfma(DenseArgs a) {
    constexpr int H = D / 2, KC = D / 32, NT = D / 16;
    constexpr int KP = D + 8;             // padded key row (bf16)
    constexpr int VP = kTok + 8;          // padded transposed value row (bf16)
    constexpr int PS = kTok + 4;          // padded P row (fp32)
    __shared__ __align__(16) __bf16 khi[kTok][KP];
    __shared__ __align__(16) __bf16 klo[kTok][KP];
    __shared__ __align__(16) uint16_t vt[D][VP];
    __shared__ __align__(16) float pbuf[4][16][PS];
    __shared__ float2 cs0[2][H];          // (cos, sin) of t0 theta_j for the step, by step parity
    __shared__ float2 csn[H];             // (cos, sin) of n theta_j
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int i16 = lane & 15, grp = lane >> 4;
    const int split = blockIdx.x, g = blockIdx.y;
    const int32_t rows_g = a.B * a.G;
    const int32_t r0 = blockIdx.z * kMRows;
    const int64_t n = a.length;
    const int64_t t_begin = (int64_t)split * a.span;
    const int64_t t_end = t_begin + a.span < n ? t_begin + a.span : n;
    const uint16_t *kc = static_cast<const uint16_t *>(a.k_cache) + (int64_t)g * a.cap * D;
    const uint16_t *vc = static_cast<const uint16_t *>(a.v_cache) + (int64_t)g * a.cap * D;

    // lanes j < H: the steps' base rotations by angle addition in double precision,
    // cos/sin(t0 theta_j) for t0 = t_begin, t_begin + kTok, ... (no slow large-argument
    // cos/sin per step)
    double2 csd = make_double2(1.0, 0.0), rot = make_double2(1.0, 0.0);
    if (threadIdx.x < H) {
        const int j = threadIdx.x;
        const double th = pow(a.base, -2.0 * (double)j / (double)D);
        const double an = (double)n * th, a0 = (double)t_begin * th, ak = (double)kTok * th;
        csn[j] = make_float2((float)cos(an), (float)sin(an));
        csd = make_double2(cos(a0), sin(a0));
        rot = make_double2(cos(ak), sin(ak));
        cs0[0][j] = make_float2((float)csd.x, (float)csd.y);
    }
    __syncthreads();
    // this lane's query row (A row i16 of the wave's tile), rotated to position n
    const int32_t rw = r0 + wave * 16 + i16;
    const int32_t rg = rw < rows_g ? rw : rows_g - 1;
    const int64_t qi = rg / a.G;
    const int h = g * a.G + (int)(rg - qi * a.G);
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + (qi * a.Hq + h) * D;
    bf16x8 ah[KC], al[KC];
    #pragma unroll
    for (int c = 0; c < KC; ++c) {
        float u[8];
        #pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int d = 32 * c + 8 * grp + v;
            const int j = d < H ? d : d - H;
            const float2 cs = csn[j];
            const float x1 = bf16_to_f32(qp[j]), x2 = bf16_to_f32(qp[j + H]);
            u[v] = d < H ? x1 * cs.x - x2 * cs.y : x2 * cs.x + x1 * cs.y;
        }
        split8(u, ah[c], al[c]);
    }
    float m_r[4], l_r[4];
    f32x4 acc[NT];
    #pragma unroll
    for (int v = 0; v < 4; ++v) { m_r[v] = -INFINITY; l_r[v] = 0.f; }
    #pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // this thread's share of a step's keys and values (NE groups of 4 pairs), raw: the
    // next step's are loaded while the current step computes
    constexpr int NE = kTok * (H / 4) / 256;
    uint2 rk1[NE], rk2[NE], rv1[NE], rv2[NE];
    auto load_raw = [&](int64_t tb) {
        #pragma unroll
        for (int q = 0; q < NE; ++q) {
            const int e = threadIdx.x + 256 * q;
            const int tt = e / (H / 4), j = (e - tt * (H / 4)) * 4;
            const int64_t t = tb + tt;
            rk1[q] = rk2[q] = rv1[q] = rv2[q] = make_uint2(0u, 0u);
            if (t < t_end) {
                rk1[q] = *reinterpret_cast<const uint2 *>(kc + t * D + j);
                rk2[q] = *reinterpret_cast<const uint2 *>(kc + t * D + H + j);
                rv1[q] = *reinterpret_cast<const uint2 *>(vc + t * D + j);
                rv2[q] = *reinterpret_cast<const uint2 *>(vc + t * D + H + j);
            }
        }
    };
    load_raw(t_begin);
    int step = 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += kTok, ++step) {
        __syncthreads();            // the previous step's LDS reads are done; cs0[step & 1] is written
        const float2 *cb = cs0[step & 1];
        // keys rotated to their positions and split; values transposed
        #pragma unroll
        for (int q = 0; q < NE; ++q) {
            const int e = threadIdx.x + 256 * q;
            const int tt = e / (H / 4), j = (e - tt * (H / 4)) * 4;
            const uint2 k1 = rk1[q], k2 = rk2[q], v1 = rv1[q], v2 = rv2[q];
            const uint16_t ka[4] = {(uint16_t)(k1.x & 0xFFFFu), (uint16_t)(k1.x >> 16),
                                    (uint16_t)(k1.y & 0xFFFFu), (uint16_t)(k1.y >> 16)};
            const uint16_t kb[4] = {(uint16_t)(k2.x & 0xFFFFu), (uint16_t)(k2.x >> 16),
                                    (uint16_t)(k2.y & 0xFFFFu), (uint16_t)(k2.y >> 16)};
            const uint16_t va[4] = {(uint16_t)(v1.x & 0xFFFFu), (uint16_t)(v1.x >> 16),
                                    (uint16_t)(v1.y & 0xFFFFu), (uint16_t)(v1.y >> 16)};
            const uint16_t vb[4] = {(uint16_t)(v2.x & 0xFFFFu), (uint16_t)(v2.x >> 16),
                                    (uint16_t)(v2.y & 0xFFFFu), (uint16_t)(v2.y >> 16)};
            __bf16 h1[4], l1[4], h2[4], l2[4];
            #pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float2 b0 = cb[j + u], inc = a.incr[tt * H + j + u];
                const float cn = b0.x * inc.x - b0.y * inc.y, sn = b0.y * inc.x + b0.x * inc.y;
                const float x1 = bf16_to_f32(ka[u]), x2 = bf16_to_f32(kb[u]);
                const float r1 = x1 * cn - x2 * sn, r2 = x2 * cn + x1 * sn;
                h1[u] = (__bf16)r1;
                h2[u] = (__bf16)r2;
                l1[u] = (__bf16)(r1 - (float)h1[u]);
                l2[u] = (__bf16)(r2 - (float)h2[u]);
                vt[j + u][tt] = va[u];
                vt[H + j + u][tt] = vb[u];
            }
            // four consecutive elements per array: one 8-byte store each (rows are 8-byte aligned)
            *reinterpret_cast<uint2 *>(&khi[tt][j]) = __builtin_bit_cast(uint2, h1);
            *reinterpret_cast<uint2 *>(&klo[tt][j]) = __builtin_bit_cast(uint2, l1);
            *reinterpret_cast<uint2 *>(&khi[tt][H + j]) = __builtin_bit_cast(uint2, h2);
            *reinterpret_cast<uint2 *>(&klo[tt][H + j]) = __builtin_bit_cast(uint2, l2);
        }
        // the next step's base rotation (the other buffer) and its keys and values, in
        // flight while this step computes
        if (threadIdx.x < H) {
            const double cx = csd.x * rot.x - csd.y * rot.y, sx = csd.y * rot.x + csd.x * rot.y;
            csd = make_double2(cx, sx);
            cs0[(step + 1) & 1][threadIdx.x] = make_float2((float)cx, (float)sx);
        }
        if (t0 + kTok < t_end) load_raw(t0 + kTok);
        __syncthreads();
        // logits of the wave's 16 rows against the step's 64 tokens: 4 tiles of 16
        f32x4 st[4];
        #pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            f32x4 c4 = {0.f, 0.f, 0.f, 0.f};
            #pragma unroll
            for (int c = 0; c < KC; ++c) {
                const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(&khi[16 * nt + i16][32 * c + 8 * grp]);
                const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(&klo[16 * nt + i16][32 * c + 8 * grp]);
                c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[c], bh, c4, 0, 0, 0);
                c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[c], bl, c4, 0, 0, 0);
                c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[c], bh, c4, 0, 0, 0);
            }
            st[nt] = c4;
        }
        // online softmax per row 4*grp + v; the row's 64 logits sit in the 16 lanes of
        // the group, 4 per lane
        #pragma unroll
        for (int v = 0; v < 4; ++v) {
            float mx = -INFINITY;
            #pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const float z = (t0 + 16 * nt + i16 < t_end) ? a.scale * st[nt][v] : -INFINITY;
                st[nt][v] = z;
                mx = fmaxf(mx, z);
            }
            #pragma unroll
            for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            const float mn = fmaxf(m_r[v], mx);          // finite: token t0 is in the span
            const float corr = m_r[v] == -INFINITY ? 0.f : __expf(m_r[v] - mn);
            float ps = 0.f;
            #pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const float p = st[nt][v] == -INFINITY ? 0.f : __expf(st[nt][v] - mn);
                st[nt][v] = p;
                ps += p;
            }
            #pragma unroll
            for (int o = 1; o < 16; o <<= 1) ps += __shfl_xor(ps, o);
            l_r[v] = l_r[v] * corr + ps;
            m_r[v] = mn;
            #pragma unroll
            for (int t = 0; t < NT; ++t) acc[t][v] *= corr;
        }
        // P to the A operand's layout (row i16, 8 consecutive tokens) through LDS
        #pragma unroll
        for (int nt = 0; nt < 4; ++nt)
            #pragma unroll
            for (int v = 0; v < 4; ++v) pbuf[wave][4 * grp + v][16 * nt + i16] = st[nt][v];
        wave_sync();
        #pragma unroll
        for (int c = 0; c < kTok / 32; ++c) {
            float pr[8];
            const float4 p0 = *reinterpret_cast<const float4 *>(&pbuf[wave][i16][32 * c + 8 * grp]);
            const float4 p1 = *reinterpret_cast<const float4 *>(&pbuf[wave][i16][32 * c + 8 * grp + 4]);
            pr[0] = p0.x; pr[1] = p0.y; pr[2] = p0.z; pr[3] = p0.w;
            pr[4] = p1.x; pr[5] = p1.y; pr[6] = p1.z; pr[7] = p1.w;
            bf16x8 ph, pl;
            split8(pr, ph, pl);
            #pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bf16x8 vv = *reinterpret_cast<const bf16x8 *>(&vt[16 * t + i16][32 * c + 8 * grp]);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vv, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vv, acc[t], 0, 0, 0);
            }
        }
    }
    // partial state of each row: [D] acc (dimension 16 t + i16 of row 4 grp + v), m, l
    #pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int32_t rr = r0 + wave * 16 + 4 * grp + v;
        if (rr < rows_g) {
            float *dst = a.part + (((int64_t)g * a.nspan + split) * rows_g + rr) * (D + 2);
            #pragma unroll
            for (int t = 0; t < NT; ++t) dst[16 * t + i16] = acc[t][v];
            if (i16 == 0) {
                dst[D] = m_r[v];
                dst[D + 1] = l_r[v];
            }
        }
    }
}

template <int D>
hipError_t launch_mfma(const DenseArgs &a, hipStream_t s) {
    const int32_t rows_g = a.B * a.G;
    hipLaunchKernelGGL(dense_incr, dim3((unsigned)((kTok * D / 2 + 255) / 256)), dim3(256), 0, s, a.incr, D,
                       a.base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)a.nspan, (unsigned)a.Hkv, (unsigned)((rows_g + kMRows - 1) / kMRows));
    hipLaunchKernelGGL((dense_mfma<D>), grid, dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dense_merge<D>), dim3((unsigned)((int64_t)a.Hkv * rows_g)), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_t(const DenseArgs &a, hipStream_t s) {
    const int32_t rows_g = a.B * a.G;
    dim3 grid((unsigned)a.nspan, (unsigned)a.Hkv, (unsigned)((rows_g + kRows - 1) / kRows));
    hipLaunchKernelGGL((dense_part<T, D>), grid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dense_merge<D>), dim3((unsigned)((int64_t)a.Hkv * rows_g)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int64_t dense_span(int64_t length) {
    // spans of a multiple of the staging step, at most kDenseMaxSpans (256) of them over
    // the cache: with 8 KV heads that is 2048 workgroups, four rounds of what the chip
    // holds at once, and a quarter of the per-span states 1024 spans would leave to
    // write and merge
    int64_t span = (length + kDenseMaxSpans - 1) / kDenseMaxSpans;
    span = (span + kTok - 1) / kTok * kTok;
    return span < kTok ? kTok : span;
}

hipError_t launch_dense(recsa_dtype st, int32_t D, const DenseArgs &a, hipStream_t s) {
    if (a.B <= 0 || a.length <= 0) return hipSuccess;
    if (st == RECSA_BF16) return D == 128 ? launch_mfma<128>(a, s) : launch_mfma<64>(a, s);
    return D == 128 ? launch_t<float, 128>(a, s) : launch_t<float, 64>(a, s);
}

}  // namespace recsa
