// AdaRMSNorm, its conditioning MLP, and the two projections around attention.
//
// "Reflex: Real-Time VLA Control through Streaming Inference" paper review:
// §3 Architecture, Eq. 2 -- AdaRMSNorm(x, c) = x / RMS(x) * gamma(c),
// gamma(c) = 1 + MLP(c), RMS(x) = sqrt(mean(x^2) + eps), c = [sinusoidal
// t_k; robot state]; the RMS is computed in FP32 and the gating MLP runs in
// BF16. §3 component table -- MLP = Linear(cond -> hidden) -> SiLU ->
// Linear(hidden -> model). §5 Code analysis -- the module squares x.float(),
// averages over the last axis, scales by rsqrt(ms + eps), multiplies by
// 1 + dense(cond). §2 / §4 -- a packed QKV kernel is one of the fused ops.
//
// Readings (the pages are silent): the embedding is the 128-wide sinusoid
// [sin(t w_i)] ++ [cos(t w_i)], w_i = 10000^(-i/64); the Linear layers have
// biases; c and the hidden activation are rounded to bf16 (the inputs of
// bf16 Linear layers) and accumulation is FP32; gamma stays FP32; the
// normalised row is rounded to bf16 once, as the input of the projection.
//
// gamma depends only on (t_k, state), so a frame's ten gammas per layer are
// produced by one batched call before its denoising loop, and the per-step
// kernels only read them.

#include <math.h>

#include "gemm.h"

namespace pa {

constexpr int MAX_T = 16;            // timesteps per ada_gamma call
struct TArr { float t[MAX_T]; };



// ------------------------------------------------------------- gamma MLP ----
// Both layers are n_t dot products per output row over an operand held in LDS
// as [n_t][K] bf16. KL adjacent lanes share one output row: lane q of the
// group takes the 8-wide k chunks q, q + KL, q + 2 KL, ... (weight loads of a
// group are KL x 16 B contiguous), NF chunk loads per lane in flight at once
// (16-lane groups and 8 loads measured fastest for the 1024-wide output layer),
// products by v_dot2c_f32_bf16 (two bf16 pairs into an FP32 accumulator); a
// few row-local lane exchanges then finish each sum.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int KL, int NF>
struct RowDots {
    const uint16_t* w;    // this lane group's weight row
    int nc;               // chunks of 8 k in the row
    int q;                // lane within the group
    uint4 wv[NF];

    __device__ __forceinline__ void load(int c0) {
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const int c = c0 + u * KL;
            wv[u] = c < nc ? *reinterpret_cast<const uint4*>(w + c * 8) : make_uint4(0, 0, 0, 0);
        }
    }
    // acc[i] += the row's dot product with x_i over every chunk of this lane;
    // the first group's loads must already be issued by load(q).
    __device__ __forceinline__ void run(const uint16_t* xs, int n_t, float (&acc)[MAX_T]) {
        const int K = nc * 8;
        for (int c0 = q; c0 < nc; c0 += KL * NF) {
            if (c0 != q) load(c0);
#pragma unroll
            for (int u = 0; u < NF; ++u) {
                const int c = c0 + u * KL;
                if (c >= nc) break;
#pragma unroll
                for (int i = 0; i < MAX_T; ++i) {
                    if (i < n_t) {
                        const uint4 xv = *reinterpret_cast<const uint4*>(xs + i * K + c * 8);
                        float a = acc[i];
                        a = dot2_bf16(wv[u].x, xv.x, a);
                        a = dot2_bf16(wv[u].y, xv.y, a);
                        a = dot2_bf16(wv[u].z, xv.z, a);
                        acc[i] = dot2_bf16(wv[u].w, xv.w, a);
                    }
                }
            }
        }
    }
};

// Sum over the KL (4, 8 or 16) adjacent lanes of a group, the same value in each.
template <int KL>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(KL == 4 || KL == 8 || KL == 16, "lane group of 4, 8 or 16");
#define PA_DPP(x, ctrl) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false))
    v += PA_DPP(v, 0xB1);                     // quad_perm [1, 0, 3, 2]
    v += PA_DPP(v, 0x4E);                     // quad_perm [2, 3, 0, 1]
    if (KL >= 8) v += PA_DPP(v, 0x141);       // row_half_mirror: the other quad of the 8
    if (KL == 16) v += PA_DPP(v, 0x140);      // row_mirror: the other half of the 16
#undef PA_DPP
    return v;
}

constexpr int GH_KL = 4, GH_NF = 8;    // hidden layer: K = cond <= 512
constexpr int GO_KL = 16, GO_NF = 8;   // output layer: K = hidden <= 4096
constexpr int GH_ROWS = 256 / 64 * (64 / GH_KL);   // hidden units per workgroup (64)
constexpr int GO_ROWS = 256 / 64 * (64 / GO_KL);   // outputs per workgroup (16)

// Hidden layer: a[l][i][j] = bf16(SiLU(W1[l][j] . c_i + b1[l][j])), with
// c_i = bf16([emb(t_i); state]) built in LDS by each workgroup (one sincos
// per timestep and frequency).
// grid (hidden / GH_ROWS, L), block 256, dynamic LDS n_t * cond bf16.
__global__ __launch_bounds__(256) void gamma_hidden(const uint16_t* w1, const uint16_t* b1, const uint16_t* state,
                                                    TArr ts, int n_t, int cond_emb, int state_dim, int hidden,
                                                    uint16_t* a_out) {
    extern __shared__ uint16_t cs[];
    const int cond = cond_emb + state_dim, half = cond_emb / 2;
    const int l = blockIdx.y, lane = threadIdx.x & 63;
    const int j = blockIdx.x * GH_ROWS + (threadIdx.x >> 6) * (64 / GH_KL) + lane / GH_KL;
    RowDots<GH_KL, GH_NF> rd{w1 + ((long long)l * hidden + j) * cond, cond / 8, lane % GH_KL, {}};
    rd.load(rd.q);
    const float log2_base = 13.287712379549449f;   // log2(10000)
    for (int idx = threadIdx.x; idx < n_t * half; idx += blockDim.x) {
        const int i = idx / half, f = idx - i * half;
        float sn, cn;
        sincosf(ts.t[i] * exp2f(-(float)f / (float)half * log2_base), &sn, &cn);
        cs[i * cond + f] = f2bf(sn);
        cs[i * cond + half + f] = f2bf(cn);
    }
    for (int idx = threadIdx.x; idx < n_t * state_dim; idx += blockDim.x) {
        const int i = idx / state_dim, k = idx - i * state_dim;
        cs[i * cond + cond_emb + k] = state[k];
    }
    __syncthreads();
    float acc[MAX_T];
#pragma unroll
    for (int i = 0; i < MAX_T; ++i) acc[i] = 0.f;
    rd.run(cs, n_t, acc);
    const float bias = bf2f(b1[(long long)l * hidden + j]);
#pragma unroll
    for (int i = 0; i < MAX_T; ++i) {
        if (i < n_t) {
            const float h = group_sum<GH_KL>(acc[i]) + bias;
            if (rd.q == 0) a_out[((long long)l * n_t + i) * hidden + j] = f2bf(h / (1.f + expf(-h)));
        }
    }
}

// Output layer: gamma[l][i][m] = 1 + b2[l][m] + W2[l][m] . a[l][i].
// grid (model / GO_ROWS, L), block 256, dynamic LDS n_t * hidden bf16.
__global__ __launch_bounds__(256) void gamma_out(const uint16_t* w2, const uint16_t* b2, const uint16_t* a_in, int n_t,
                                                 int hidden, int model, float* gamma) {
    extern __shared__ uint16_t as[];
    const int l = blockIdx.y, lane = threadIdx.x & 63;
    const int m = blockIdx.x * GO_ROWS + (threadIdx.x >> 6) * (64 / GO_KL) + lane / GO_KL;
    RowDots<GO_KL, GO_NF> rd{w2 + ((long long)l * model + m) * hidden, hidden / 8, lane % GO_KL, {}};
    rd.load(rd.q);       // in flight across the barrier that publishes the staged activations
    const uint16_t* a_l = a_in + (long long)l * n_t * hidden;
    for (int idx = threadIdx.x * 8; idx < n_t * hidden; idx += blockDim.x * 8)
        *reinterpret_cast<uint4*>(&as[idx]) = *reinterpret_cast<const uint4*>(a_l + idx);
    __syncthreads();
    float acc[MAX_T];
#pragma unroll
    for (int i = 0; i < MAX_T; ++i) acc[i] = 0.f;
    rd.run(as, n_t, acc);
    const float bias = bf2f(b2[(long long)l * model + m]);
#pragma unroll
    for (int i = 0; i < MAX_T; ++i) {
        if (i < n_t) {
            const float sum = group_sum<GO_KL>(acc[i]);
            if (rd.q == 0) gamma[((long long)l * n_t + i) * model + m] = 1.f + bias + sum;
        }
    }
}

// ------------------------------------------------------------- RMS norm -----
// y[r] = x[r] * rsqrt(mean(x[r]^2) + eps) * gamma, FP32 arithmetic.
// grid (rows), block 256.
template <typename TO> __device__ __forceinline__ void store_y(TO* p, float v);
template <> __device__ __forceinline__ void store_y<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_y<uint16_t>(uint16_t* p, float v) { *p = f2bf(v); }

template <typename TO>
__global__ __launch_bounds__(256) void rmsnorm_rows(const uint16_t* x, const float* gamma, int model, float eps, TO* y,
                                                    uint32_t* nonfinite) {
    __shared__ float red[4];
    const int r = blockIdx.x;
    const uint16_t* xr = x + (long long)r * model;
    float ss = 0.f;
    for (int k = threadIdx.x; k < model; k += blockDim.x) {
        const float v = bf2f(xr[k]);
        ss += v * v;
    }
    ss = wsum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float ms = (red[0] + red[1] + red[2] + red[3]) / (float)model;
    const float rinv = 1.f / sqrtf(ms + eps);
    bool bad = false;
    for (int k = threadIdx.x; k < model; k += blockDim.x) {
        const float v = bf2f(xr[k]) * rinv * gamma[k];
        bad |= !finite_f(v);
        store_y(y + (long long)r * model + k, v);
    }
    if (nonfinite && __any(bad) && (threadIdx.x & 63) == 0) atomicOr(nonfinite, 1u);
}

// ------------------------------------------------- skinny GEMM, A W^T -------
// C[m][n] = sum_k A[m][k] W[n][k] for m < rows <= 64, bf16 in, FP32 accumulate,
// W in nn.Linear layout [N][K]. Weight streaming: every W element is read
// once, by one lane, and used by two MFMAs (row blocks 0-31 and 32-63).
// A workgroup of 8 waves owns 32 output columns; wave w owns the k-range
// [w K/8, (w+1) K/8) = KS k-steps of 16, issues all of its weight loads at
// once (so the whole weight matrix is in flight across the GPU), and the
// eight partial sums meet in LDS.
//   A operand (32 rows x 16 k): lane row l32, k 8hi..8hi+7 -> 16 B of A's row
//   B operand (16 k x 32 cols): lane col l32, k 8hi..8hi+7 -> 16 B of W's row
// With NORM the A operand is AdaRMSNorm's output formed on the fly,
// bf16(x[m][k] * rsqrt(mean_k x[m]^2 + eps) * gamma[k]), the mean of
// squares taken in FP32 by the workgroup before the products.
enum GemmMode { GEMM_QKV = 0, GEMM_OPROJ = 1 };

// AdaRMSNorm formed on the fly as the A operand of a skinny GEMM over K =
// GEMM_WAVES * KS * 16: the FP32 mean of squares of every row (wave w takes
// rows w, w + 8, ..., all of its loads in flight before any is used), then
// each lane's fragments bf16(x[m][k] * rsqrt(ms + eps) * gamma[k]) for rows
// l32 and 32 + l32 and its k-range. With HALVES, only the rows of 32-row half
// `half` (fragments in a0, a1 zero): each row's arithmetic is the same. Ends
// with every wave past a barrier.
template <int KS, bool HALVES = false>
__device__ __forceinline__ void norm_fragments(const uint16_t* __restrict__ a, const float* __restrict__ gamma,
                                               float eps, int rows, float* rinv_s, bf16x8 (&a0)[KS],
                                               bf16x8 (&a1)[KS], int half = 0) {
    constexpr int K = GEMM_WAVES * KS * 16;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    const int k0 = wave * KS * 16 + 8 * hi, base = HALVES ? 32 * half : 0;
    const bool r0 = base + l32 < rows, r1 = !HALVES && 32 + l32 < rows;
    constexpr int RPW = (HALVES ? 32 : 64) / GEMM_WAVES;        // rows per wave
    constexpr int LPR = (K + 511) / 512;        // 16-byte loads per lane and row
    // Every load leaves before the first is used. Up to K = 1024 (KS <= 8) a
    // row past `rows` or a chunk past K re-reads row 0's first chunk (in
    // bounds) and is zeroed after the load, so that no branch sits around a
    // load; wider rows keep the guarded loads (their registers are full).
    uint4 raw[RPW][LPR];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
        const int r = base + wave + rr * GEMM_WAVES;
#pragma unroll
        for (int c = 0; c < LPR; ++c) {
            const bool in = r < rows && c * 512 + lane * 8 < K;
            if constexpr (KS <= 8)
                raw[rr][c] = *reinterpret_cast<const uint4*>(a + (in ? (long long)r * K + c * 512 + lane * 8 : 0));
            else
                raw[rr][c] = in ? *reinterpret_cast<const uint4*>(a + (long long)r * K + c * 512 + lane * 8)
                                : make_uint4(0, 0, 0, 0);
        }
    }
    if constexpr (KS <= 8) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
            const int r = base + wave + rr * GEMM_WAVES;
#pragma unroll
            for (int c = 0; c < LPR; ++c)
                if (!(r < rows && c * 512 + lane * 8 < K)) raw[rr][c] = make_uint4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < LPR; ++c) {
            const uint16_t* e = reinterpret_cast<const uint16_t*>(&raw[rr][c]);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float v = bf2f(e[u]);
                ss += v * v;
            }
        }
        ss = wsum(ss);
        const int r = base + wave + rr * GEMM_WAVES;
        if (lane == 0 && r < rows) rinv_s[r] = 1.f / sqrtf(ss / (float)K + eps);
    }
    __syncthreads();
    const float ri0 = r0 ? rinv_s[base + l32] : 0.f, ri1 = r1 ? rinv_s[32 + l32] : 0.f;
    if constexpr (KS <= 8) {
        // Every fragment and gamma load leaves before the first is used (one
        // memory round trip, not one per k-step); a row past `rows` reads row
        // `base` (in bounds) and is scaled by 0. Without HALVES the second
        // rows' loads exist only when a second 32-row block does.
        const uint16_t* p0 = a + (long long)(r0 ? base + l32 : base) * K + k0;
        const uint16_t* p1 = a + (long long)(r1 ? 32 + l32 : 0) * K + k0;
        uint4 x0[KS], x1[KS];
        float4 g[KS][2];
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            x0[i] = *reinterpret_cast<const uint4*>(p0 + 16 * i);
            if (!HALVES) x1[i] = *reinterpret_cast<const uint4*>(p1 + 16 * i);
            g[i][0] = *reinterpret_cast<const float4*>(gamma + k0 + 16 * i);
            g[i][1] = *reinterpret_cast<const float4*>(gamma + k0 + 16 * i + 4);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            const float gg[8] = {g[i][0].x, g[i][0].y, g[i][0].z, g[i][0].w,
                                 g[i][1].x, g[i][1].y, g[i][1].z, g[i][1].w};
            const uint4 xa = x0[i], xb = HALVES ? make_uint4(0, 0, 0, 0) : x1[i];
            const uint16_t* e0 = reinterpret_cast<const uint16_t*>(&xa);
            const uint16_t* e1 = reinterpret_cast<const uint16_t*>(&xb);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                a0[i][u] = (__bf16)(bf2f(e0[u]) * ri0 * gg[u]);
                a1[i][u] = (__bf16)(bf2f(e1[u]) * ri1 * gg[u]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            const int k = k0 + 16 * i;
            const float4 g0 = *reinterpret_cast<const float4*>(gamma + k);
            const float4 g1 = *reinterpret_cast<const float4*>(gamma + k + 4);
            const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
            if (r0) x0 = *reinterpret_cast<const uint4*>(a + (long long)(base + l32) * K + k);
            if (r1) x1 = *reinterpret_cast<const uint4*>(a + (long long)(32 + l32) * K + k);
            const uint16_t* e0 = reinterpret_cast<const uint16_t*>(&x0);
            const uint16_t* e1 = reinterpret_cast<const uint16_t*>(&x1);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                a0[i][u] = (__bf16)(bf2f(e0[u]) * ri0 * gg[u]);
                a1[i][u] = (__bf16)(bf2f(e1[u]) * ri1 * gg[u]);
            }
        }
    }
}

template <int KS>
__device__ __forceinline__ void report_nonfinite(const bf16x8 (&a0)[KS], const bf16x8 (&a1)[KS], uint32_t* flag) {
    bool bad = false;
#pragma unroll
    for (int i = 0; i < KS; ++i)
#pragma unroll
        for (int u = 0; u < 8; ++u) bad |= !finite_f((float)a0[i][u]) || !finite_f((float)a1[i][u]);
    if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, 1u);
}

template <int MODE, int KS, bool NORM>
__global__ __launch_bounds__(GEMM_WAVES * 64, 2) void gemm_skinny(const uint16_t* __restrict__ a,
                                                                 const float* __restrict__ gamma, float eps,
                                                                 const uint16_t* __restrict__ w, int rows, int N,
                                                                 GemmOut out) {
    constexpr int K = GEMM_WAVES * KS * 16;
    __shared__ float red[GEMM_WAVES][2][16][64];
    __shared__ float rinv_s[64];
    // the QKV projection: one 32-row half per workgroup (row_half_grid); the
    // out-projection's residual epilogue takes all 64 row slots
    constexpr bool HALVES = MODE == GEMM_QKV;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    int nb = blockIdx.x, half = 0;
    if (HALVES) {
        row_half_block(rows, nb, half);
        if (nb >= N / 32) return;                                   // id padding, whole workgroup
    }
    const int n0 = nb * 32;
    const int k0 = wave * KS * 16 + 8 * hi;
    // the out-projection's residual rows, loaded with the operands
    ResidualRows rres{};
    if constexpr (MODE == GEMM_OPROJ) rres = residual_rows(n0, rows, N, out);

    bf16x8 wf[KS];
    const uint16_t* wp = w + (long long)(n0 + l32) * K + k0;
#pragma unroll
    for (int i = 0; i < KS; ++i) wf[i] = *reinterpret_cast<const bf16x8*>(wp + 16 * i);

    const bool r0 = 32 * half + l32 < rows, r1 = !HALVES && 32 + l32 < rows;
    bf16x8 a0[KS], a1[KS];
    if (!NORM) {
        // rows past `rows` re-read row 0 (in bounds) and are zeroed after the
        // loads, which all leave before the first product
        const uint16_t* p0 = a + (long long)(r0 ? 32 * half + l32 : 0) * K + k0;
        const uint16_t* p1 = a + (long long)(r1 ? 32 + l32 : 0) * K + k0;
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            a0[i] = *reinterpret_cast<const bf16x8*>(p0 + 16 * i);
            if (!HALVES) a1[i] = *reinterpret_cast<const bf16x8*>(p1 + 16 * i);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            if (!r0) a0[i] = bf16x8{};
            if (HALVES || !r1) a1[i] = bf16x8{};
        }
    } else {
        norm_fragments<KS, HALVES>(a, gamma, eps, rows, rinv_s, a0, a1, half);
        // every workgroup of a row half forms the same normalised rows; those
        // of column block 0 report a non-finite element (padding rows are zeros)
        if (nb == 0 && out.nonfinite) report_nonfinite<KS>(a0, a1, out.nonfinite);
    }

    f32x16 c0 = f32x16{}, c1 = f32x16{};
    const bool two = !HALVES && rows > 32;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], wf[i], c0, 0, 0, 0);
        if (two) c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], wf[i], c1, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        red[wave][0][r][lane] = c0[r];
        red[wave][1][r][lane] = c1[r];
    }
    __syncthreads();
    // wave w finishes 4 of the 32 (block, register) pairs (2 of the 16 of its
    // row half with HALVES)
    if (MODE == GEMM_QKV) {
        constexpr int NU = HALVES ? 2 : 4;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int idx = wave * NU + u, blk = idx >> 4, r = idx & 15;
            const int m = 32 * (blk + half) + 8 * (r >> 2) + 4 * hi + (r & 3);
            const int n = n0 + l32;
            if (m >= rows) continue;
            float v = 0.f;
#pragma unroll
            for (int ww = 0; ww < GEMM_WAVES; ++ww) v += red[ww][blk][r][lane];
            if (n < out.nq)
                out.q[(long long)m * out.nq + n] = f2bf(v);
            else if (n < out.nq + out.nk)
                out.k[(long long)m * out.nk + (n - out.nq)] = f2bf(v);
            else
                out.v[(long long)m * out.nk + (n - out.nq - out.nk)] = f2bf(v);
        }
    } else {
        residual_epilogue(red, rres, out);
    }
}

// ----------------------------------------------------- FFN with SwiGLU -----
// The FFN of the full action-expert layer: the pages name "SwiGLU fusion",
// "FlashNorm" and "FusedAdaLN" among their fused operators (Reflex review,
// §2 and the §3 system-optimisation row; ablated in Fig. 11) without giving
// the layer. Reading: y = bf16(AdaRMSNorm(h, gamma_ffn)) with its own gamma,
// act = bf16(SiLU(y W_gate^T) * (y W_up^T)) (FP32 products, one rounding),
// h <- bf16(h + act W_down^T). The norm is fused into the gate/up GEMM and
// SwiGLU into its epilogue, so y and the gate/up products never reach memory.
//
// gemm_gateup: a workgroup owns 32 act columns; its 8 waves split K = model
// (KS k-steps of 16 each) and compute both products for those columns; the
// gate and up partial sums meet in LDS one after the other. A workgroup owns
// one 32-row half of the operand (row_half_grid). Without NORM, x is the
// already normalised operand.
template <int KS, bool NORM = true>
__global__ __launch_bounds__(GEMM_WAVES * 64, 1) void gemm_gateup(const uint16_t* __restrict__ x,
                                                                  const float* __restrict__ gamma, float eps,
                                                                  const uint16_t* __restrict__ w_gate,
                                                                  const uint16_t* __restrict__ w_up, int rows, int F,
                                                                  uint16_t* __restrict__ act, uint32_t* nonfinite) {
    constexpr int K = GEMM_WAVES * KS * 16;
    __shared__ float red[GEMM_WAVES][16][64];
    __shared__ float rinv_s[64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    int nb, half;
    row_half_block(rows, nb, half);
    if (nb >= F / 32) return;                                       // id padding, whole workgroup
    const int n0 = nb * 32;
    const int k0 = wave * KS * 16 + 8 * hi;
    bf16x8 wg[KS], wu[KS];
    const long long wrow = (long long)(n0 + l32) * K + k0;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        wg[i] = *reinterpret_cast<const bf16x8*>(w_gate + wrow + 16 * i);
        wu[i] = *reinterpret_cast<const bf16x8*>(w_up + wrow + 16 * i);
    }
    bf16x8 a0[KS], a1[KS];
    if (NORM) {
        norm_fragments<KS, true>(x, gamma, eps, rows, rinv_s, a0, a1, half);
        if (nb == 0 && nonfinite) report_nonfinite<KS>(a0, a1, nonfinite);
    } else {
        const int row = 32 * half + l32;
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            a0[i] = row < rows ? *reinterpret_cast<const bf16x8*>(x + (long long)row * K + k0 + 16 * i) : bf16x8{};
            a1[i] = bf16x8{};
        }
    }
    f32x16 g0 = f32x16{}, u0 = f32x16{};
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        g0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], wg[i], g0, 0, 0, 0);
        u0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], wu[i], u0, 0, 0, 0);
    }
    // wave w finishes 2 of the 16 (register) rows of its row half: the gate
    // sums first
    constexpr int NU = 2;
    float gs[NU];
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][r][lane] = g0[r];
    __syncthreads();
#pragma unroll
    for (int uix = 0; uix < NU; ++uix) {
        const int r = wave * NU + uix;
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < GEMM_WAVES; ++ww) v += red[ww][r][lane];
        gs[uix] = v;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][r][lane] = u0[r];
    __syncthreads();
#pragma unroll
    for (int uix = 0; uix < NU; ++uix) {
        const int r = wave * NU + uix;
        const int m = 32 * half + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (m >= rows) continue;
        float u = 0.f;
#pragma unroll
        for (int ww = 0; ww < GEMM_WAVES; ++ww) u += red[ww][r][lane];
        const float g = gs[uix];
        act[(long long)m * F + n0 + l32] = f2bf(g / (1.f + __expf(-g)) * u);
    }
}

// K = 128 * KS; the k-step counts the library is built for.
static bool gemm_k_supported(int K) {
    if (K % 128) return false;
    const int ks = K / 128;
    return ks == 2 || ks == 4 || ks == 6 || ks == 8 || ks == 12 || ks == 16;
}

template <int MODE, bool NORM>
static hipError_t launch_gemm(const uint16_t* a, const float* gamma, float eps, const uint16_t* w, int rows, int K,
                              int N, const GemmOut& o, hipStream_t s) {
    const dim3 grid(MODE == GEMM_QKV ? row_half_grid(rows, N) : N / 32), block(GEMM_WAVES * 64);
    switch (K / 128) {
        case 2: gemm_skinny<MODE, 2, NORM><<<grid, block, 0, s>>>(a, gamma, eps, w, rows, N, o); break;
        case 4: gemm_skinny<MODE, 4, NORM><<<grid, block, 0, s>>>(a, gamma, eps, w, rows, N, o); break;
        case 6: gemm_skinny<MODE, 6, NORM><<<grid, block, 0, s>>>(a, gamma, eps, w, rows, N, o); break;
        case 8: gemm_skinny<MODE, 8, NORM><<<grid, block, 0, s>>>(a, gamma, eps, w, rows, N, o); break;
        case 12: gemm_skinny<MODE, 12, NORM><<<grid, block, 0, s>>>(a, gamma, eps, w, rows, N, o); break;
        default: gemm_skinny<MODE, 16, NORM><<<grid, block, 0, s>>>(a, gamma, eps, w, rows, N, o); break;
    }
    return hipGetLastError();
}

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static pa_status check_mlp(const ada_mlp* m) {
    PA_CHECK_ARG(m && m->w1 && m->b1 && m->w2 && m->b2, PA_EINVAL, "ada: null MLP pointer");
    PA_CHECK_ARG(al16(m->w1) && al16(m->w2), PA_EINVAL, "ada: MLP weights must be 16-byte aligned");
    PA_CHECK_ARG(m->num_layers >= 1, PA_ESHAPE, "ada: num_layers must be >= 1");
    PA_CHECK_ARG(m->cond_emb >= 2 && m->cond_emb % 2 == 0 && m->state_dim >= 0 && m->state_dim <= 128 &&
                     (m->cond_emb + m->state_dim) % 8 == 0 && m->cond_emb + m->state_dim <= 512,
                 PA_ESHAPE, "ada: cond_emb must be even, state_dim <= 128, cond_emb + state_dim a multiple of 8 (<= 512)");
    PA_CHECK_ARG(m->hidden_dim >= 64 && m->hidden_dim % 64 == 0 && m->hidden_dim <= 4096, PA_ESHAPE,
                 "ada: hidden_dim must be a multiple of 64 in [64, 4096]");
    PA_CHECK_ARG(m->model_dim >= 64 && m->model_dim % 64 == 0, PA_ESHAPE, "ada: model_dim must be a multiple of 64");
    return PA_OK;
}

static pa_status launch_gamma(const ada_mlp* m, const uint16_t* w1, const uint16_t* b1, const uint16_t* w2,
                              const uint16_t* b2, int n_layers, const float* t, int n_t, const uint16_t* state,
                              float* gamma, uint16_t* a_ws, hipStream_t s) {
    TArr ts{};
    for (int i = 0; i < n_t; ++i) ts.t[i] = t[i];
    const int cond = m->cond_emb + m->state_dim;
    gamma_hidden<<<dim3(m->hidden_dim / GH_ROWS, n_layers), 256, n_t * cond * sizeof(uint16_t), s>>>(
        w1, b1, state, ts, n_t, m->cond_emb, m->state_dim, m->hidden_dim, a_ws);
    PA_LAUNCHED();
    gamma_out<<<dim3(m->model_dim / GO_ROWS, n_layers), 256, n_t * m->hidden_dim * sizeof(uint16_t), s>>>(
        w2, b2, a_ws, n_t, m->hidden_dim, m->model_dim, gamma);
    PA_LAUNCHED();
    return PA_OK;
}

// Stack-internal projections on an operand the residual kernel has already
// normalised (nn.Linear layouts; the packed forms are in packed.hip).
pa_status qkv_proj(const void* y, int rows, int model_dim, const void* w_qkv, int hq, int hkv, int d, void* q,
                   void* k, void* v, hipStream_t s) {
    PA_CHECK_ARG(gemm_k_supported(model_dim) && rows >= 1 && rows <= 64, PA_ESHAPE,
                 "qkv projection: model_dim must be 128 x {2, 4, 6, 8, 12, 16} (got %d)", model_dim);
    GemmOut o{};
    o.q = static_cast<uint16_t*>(q);
    o.k = static_cast<uint16_t*>(k);
    o.v = static_cast<uint16_t*>(v);
    o.nq = hq * d;
    o.nk = hkv * d;
    const hipError_t e = launch_gemm<GEMM_QKV, false>(static_cast<const uint16_t*>(y), nullptr, 0.f,
                                                      static_cast<const uint16_t*>(w_qkv), rows, model_dim,
                                                      (hq + 2 * hkv) * d, o, s);
    PA_CHECK_ARG(e == hipSuccess, PA_EDEVICE, "qkv projection: launch failed (%s)", hipGetErrorString(e));
    return PA_OK;
}

pa_status gateup_proj(const void* y, int rows, int model_dim, int ffn_dim, const void* w_gate, const void* w_up,
                      void* act, hipStream_t s) {
    const uint16_t* yy = static_cast<const uint16_t*>(y);
    const uint16_t* wg = static_cast<const uint16_t*>(w_gate);
    const uint16_t* wu = static_cast<const uint16_t*>(w_up);
    uint16_t* a = static_cast<uint16_t*>(act);
    const dim3 block(GEMM_WAVES * 64);
    switch (model_dim / 128) {
        case 2: gemm_gateup<2, false><<<row_half_grid(rows, ffn_dim), block, 0, s>>>(yy, nullptr, 0.f, wg, wu, rows, ffn_dim, a, nullptr); break;
        case 4: gemm_gateup<4, false><<<row_half_grid(rows, ffn_dim), block, 0, s>>>(yy, nullptr, 0.f, wg, wu, rows, ffn_dim, a, nullptr); break;
        case 6: gemm_gateup<6, false><<<row_half_grid(rows, ffn_dim), block, 0, s>>>(yy, nullptr, 0.f, wg, wu, rows, ffn_dim, a, nullptr); break;
        default: gemm_gateup<8, false><<<row_half_grid(rows, ffn_dim), block, 0, s>>>(yy, nullptr, 0.f, wg, wu, rows, ffn_dim, a, nullptr); break;
    }
    PA_LAUNCHED();
    return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" size_t ada_gamma_workspace_bytes(const ada_mlp* m, int32_t n_t) {
    if (check_mlp(m) != PA_OK || n_t < 1 || n_t > MAX_T) return 0;
    return align_up((size_t)m->num_layers * n_t * m->hidden_dim * sizeof(uint16_t), 256);
}

extern "C" pa_status ada_gamma(const ada_mlp* m, const float* t, int32_t n_t, const void* state, float* gamma,
                               void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    pa_status st = check_mlp(m);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(t && gamma && ws && (state || m->state_dim == 0), PA_EINVAL, "ada_gamma: null argument");
    PA_CHECK_ARG(n_t >= 1 && n_t <= MAX_T, PA_ESHAPE, "ada_gamma: n_t %d not in [1, %d]", n_t, MAX_T);
    PA_CHECK_ARG(n_t * m->hidden_dim * 2 <= 65536, PA_ESHAPE, "ada_gamma: n_t * hidden_dim too large for one call");
    const size_t need = ada_gamma_workspace_bytes(m, n_t);
    PA_CHECK_ARG(ws_bytes >= need, PA_ERANGE, "ada_gamma: workspace %zu < %zu bytes", ws_bytes, need);
    for (int i = 0; i < n_t; ++i) PA_CHECK_ARG(isfinite(t[i]), PA_EINVAL, "ada_gamma: t[%d] is not finite", i);
    return launch_gamma(m, static_cast<const uint16_t*>(m->w1), static_cast<const uint16_t*>(m->b1),
                        static_cast<const uint16_t*>(m->w2), static_cast<const uint16_t*>(m->b2), m->num_layers, t,
                        n_t, static_cast<const uint16_t*>(state), gamma, static_cast<uint16_t*>(ws),
                        static_cast<hipStream_t>(stream));
}

extern "C" size_t ada_rmsnorm_workspace_bytes(const ada_mlp* m) {
    if (check_mlp(m) != PA_OK) return 0;
    return align_up((size_t)m->hidden_dim * sizeof(uint16_t), 256) + align_up((size_t)m->model_dim * sizeof(float), 256);
}

extern "C" pa_status ada_rmsnorm(const void* x, int32_t rows, const ada_mlp* m, int32_t layer, float t,
                                 const void* state, float eps, void* y, int32_t y_dtype, uint32_t* nonfinite, void* ws,
                                 size_t ws_bytes, void* stream) {
    clear_error();
    pa_status st = check_mlp(m);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(x && y && ws && (state || m->state_dim == 0), PA_EINVAL, "ada_rmsnorm: null argument");
    PA_CHECK_ARG(y_dtype == PA_F32 || y_dtype == PA_BF16, PA_EINVAL, "ada_rmsnorm: bad y_dtype");
    PA_CHECK_ARG(rows >= 1, PA_ESHAPE, "ada_rmsnorm: rows must be >= 1");
    PA_CHECK_ARG(layer >= 0 && layer < m->num_layers, PA_ESHAPE, "ada_rmsnorm: layer %d outside [0, %d)", layer,
                 m->num_layers);
    PA_CHECK_ARG(eps >= 0.f && isfinite(t), PA_EINVAL, "ada_rmsnorm: eps must be >= 0 and t finite");
    PA_CHECK_ARG(ws_bytes >= ada_rmsnorm_workspace_bytes(m), PA_ERANGE, "ada_rmsnorm: workspace too small");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int cond = m->cond_emb + m->state_dim;
    const uint16_t* w1 = static_cast<const uint16_t*>(m->w1) + (long long)layer * m->hidden_dim * cond;
    const uint16_t* b1 = static_cast<const uint16_t*>(m->b1) + (long long)layer * m->hidden_dim;
    const uint16_t* w2 = static_cast<const uint16_t*>(m->w2) + (long long)layer * m->model_dim * m->hidden_dim;
    const uint16_t* b2 = static_cast<const uint16_t*>(m->b2) + (long long)layer * m->model_dim;
    uint16_t* a_ws = static_cast<uint16_t*>(ws);
    float* g = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)m->hidden_dim * 2, 256));
    st = launch_gamma(m, w1, b1, w2, b2, 1, &t, 1, static_cast<const uint16_t*>(state), g, a_ws, s);
    if (st != PA_OK) return st;
    if (y_dtype == PA_F32)
        rmsnorm_rows<float><<<rows, 256, 0, s>>>(static_cast<const uint16_t*>(x), g, m->model_dim, eps,
                                                 static_cast<float*>(y), nonfinite);
    else
        rmsnorm_rows<uint16_t><<<rows, 256, 0, s>>>(static_cast<const uint16_t*>(x), g, m->model_dim, eps,
                                                    static_cast<uint16_t*>(y), nonfinite);
    PA_LAUNCHED();
    return PA_OK;
}

extern "C" size_t ada_rmsnorm_qkv_workspace_bytes(int32_t rows, int32_t model_dim) {
    (void)rows;
    (void)model_dim;
    return 0;   // the norm is fused into the projection; kept for ABI stability
}

extern "C" pa_status ada_rmsnorm_qkv(const void* x, int32_t rows, int32_t model_dim, const float* gamma, float eps,
                                     const void* w_qkv, int32_t hq, int32_t hkv, int32_t d, void* q, void* k_dyn,
                                     void* v_dyn, uint32_t* nonfinite, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    (void)ws;
    (void)ws_bytes;
    PA_CHECK_ARG(x && gamma && w_qkv && q && k_dyn && v_dyn, PA_EINVAL, "ada_rmsnorm_qkv: null argument");
    PA_CHECK_ARG(al16(x) && al16(w_qkv) && al16(gamma), PA_EINVAL,
                 "ada_rmsnorm_qkv: x, gamma and w_qkv must be 16-byte aligned");
    PA_CHECK_ARG(rows >= 1 && rows <= 64, PA_ESHAPE, "ada_rmsnorm_qkv: rows %d not in [1, 64]", rows);
    PA_CHECK_ARG(gemm_k_supported(model_dim), PA_ESHAPE,
                 "ada_rmsnorm_qkv: model_dim %d must be 128 x {2, 4, 6, 8, 12, 16}", model_dim);
    PA_CHECK_ARG(hq >= 1 && hkv >= 1 && hq % hkv == 0 && d >= 32 && d % 32 == 0, PA_ESHAPE,
                 "ada_rmsnorm_qkv: need Hq a multiple of Hkv and D a multiple of 32");
    PA_CHECK_ARG(eps >= 0.f, PA_EINVAL, "ada_rmsnorm_qkv: eps must be >= 0");
    GemmOut o{};
    o.nonfinite = nonfinite;
    o.q = static_cast<uint16_t*>(q);
    o.k = static_cast<uint16_t*>(k_dyn);
    o.v = static_cast<uint16_t*>(v_dyn);
    o.nq = hq * d;
    o.nk = hkv * d;
    const int n = (hq + 2 * hkv) * d;
    const hipError_t e = launch_gemm<GEMM_QKV, true>(static_cast<const uint16_t*>(x), gamma, eps,
                                                     static_cast<const uint16_t*>(w_qkv), rows, model_dim, n, o,
                                                     static_cast<hipStream_t>(stream));
    PA_CHECK_ARG(e == hipSuccess, PA_EDEVICE, "ada_rmsnorm_qkv: launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

extern "C" pa_status oproj_residual(const void* o, const void* w_o, void* h, int32_t rows, int32_t in_dim,
                                    int32_t model_dim, void* x, float dt, uint32_t* nonfinite, void* stream) {
    clear_error();
    PA_CHECK_ARG(o && w_o && h, PA_EINVAL, "oproj_residual: null argument");
    PA_CHECK_ARG(al16(o) && al16(w_o), PA_EINVAL, "oproj_residual: o and w_o must be 16-byte aligned");
    PA_CHECK_ARG(rows >= 1 && rows <= 64, PA_ESHAPE, "oproj_residual: rows %d not in [1, 64]", rows);
    PA_CHECK_ARG(gemm_k_supported(in_dim), PA_ESHAPE, "oproj_residual: in_dim %d must be 128 x {2, 4, 6, 8, 12, 16}",
                 in_dim);
    PA_CHECK_ARG(model_dim >= 32 && model_dim % 32 == 0, PA_ESHAPE, "oproj_residual: model_dim must be a multiple of 32");
    PA_CHECK_ARG(isfinite(dt), PA_EINVAL, "oproj_residual: dt must be finite");
    GemmOut g{};
    g.h = static_cast<uint16_t*>(h);
    g.x = static_cast<uint16_t*>(x);
    g.dt = dt;
    g.nonfinite = nonfinite;
    const hipError_t e = launch_gemm<GEMM_OPROJ, false>(static_cast<const uint16_t*>(o), nullptr, 0.f,
                                                        static_cast<const uint16_t*>(w_o), rows, in_dim, model_dim, g,
                                                        static_cast<hipStream_t>(stream));
    PA_CHECK_ARG(e == hipSuccess, PA_EDEVICE, "oproj_residual: launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

// ---------------------------------------------------------------- FFN -------
static bool ffn_dims_ok(int model_dim, int ffn_dim) {
    const int ks = model_dim / 128, kc = ffn_dim / 1024;
    return model_dim % 128 == 0 && (ks == 2 || ks == 4 || ks == 6 || ks == 8) && ffn_dim % 1024 == 0 &&
           (kc == 1 || kc == 2 || kc == 3 || kc == 4 || kc == 6 || kc == 8);
}

extern "C" size_t ffn_swiglu_workspace_bytes(int32_t rows, int32_t model_dim, int32_t ffn_dim) {
    if (rows < 1 || rows > 64 || !ffn_dims_ok(model_dim, ffn_dim)) return 0;
    // the SwiGLU activation, then the down projection's split-K partials
    return align_up((size_t)rows * ffn_dim * sizeof(uint16_t), 256) + residual_splitk_bytes(rows, ffn_dim, model_dim);
}

extern "C" pa_status ffn_swiglu(void* h, int32_t rows, int32_t model_dim, int32_t ffn_dim, const float* gamma,
                                float eps, const void* w_gate, const void* w_up, const void* w_down, void* x, float dt,
                                uint32_t* nonfinite, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    PA_CHECK_ARG(h && gamma && w_gate && w_up && w_down && ws, PA_EINVAL, "ffn_swiglu: null argument");
    PA_CHECK_ARG(al16(h) && al16(gamma) && al16(w_gate) && al16(w_up) && al16(w_down) && al16(ws), PA_EINVAL,
                 "ffn_swiglu: h, gamma, the weights and the workspace must be 16-byte aligned");
    PA_CHECK_ARG(rows >= 1 && rows <= 64, PA_ESHAPE, "ffn_swiglu: rows %d not in [1, 64]", rows);
    PA_CHECK_ARG(ffn_dims_ok(model_dim, ffn_dim), PA_ESHAPE,
                 "ffn_swiglu: model_dim must be 128 x {2, 4, 6, 8} and ffn_dim 1024 x {1, 2, 3, 4, 6, 8} (got %d, %d)",
                 model_dim, ffn_dim);
    PA_CHECK_ARG(eps >= 0.f && isfinite(dt), PA_EINVAL, "ffn_swiglu: eps must be >= 0 and dt finite");
    const size_t need = ffn_swiglu_workspace_bytes(rows, model_dim, ffn_dim);
    PA_CHECK_ARG(ws_bytes >= need, PA_ERANGE, "ffn_swiglu: workspace %zu < %zu bytes", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint16_t* act = static_cast<uint16_t*>(ws);
    const uint16_t* xin = static_cast<const uint16_t*>(h);
    const uint16_t* wg = static_cast<const uint16_t*>(w_gate);
    const uint16_t* wu = static_cast<const uint16_t*>(w_up);
    const dim3 block(GEMM_WAVES * 64);
    switch (model_dim / 128) {
        case 2: gemm_gateup<2><<<row_half_grid(rows, ffn_dim), block, 0, s>>>(xin, gamma, eps, wg, wu, rows, ffn_dim, act, nonfinite); break;
        case 4: gemm_gateup<4><<<row_half_grid(rows, ffn_dim), block, 0, s>>>(xin, gamma, eps, wg, wu, rows, ffn_dim, act, nonfinite); break;
        case 6: gemm_gateup<6><<<row_half_grid(rows, ffn_dim), block, 0, s>>>(xin, gamma, eps, wg, wu, rows, ffn_dim, act, nonfinite); break;
        default: gemm_gateup<8><<<row_half_grid(rows, ffn_dim), block, 0, s>>>(xin, gamma, eps, wg, wu, rows, ffn_dim, act, nonfinite); break;
    }
    PA_LAUNCHED();
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                           align_up((size_t)rows * ffn_dim * sizeof(uint16_t), 256));
    return residual_splitk(act, w_down, false, h, rows, ffn_dim, model_dim, x, dt, nonfinite, part, s);
}

