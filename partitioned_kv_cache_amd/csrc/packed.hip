// Skinny GEMMs of the layer glue on fragment-packed operands.
//
// The projections around attention and the FFN (norm + packed QKV, the
// out-projection, the SwiGLU gate/up and down projections; readings of the
// Reflex review's fused operators, §2 and the §3 system-optimisation row) have
// M = 51 rows and stream one weight matrix each. Reading nn.Linear rows
// directly in the MFMA operand layout makes every 16-byte lane load touch a
// different row, so a wave instruction gathers 32 B from 32-64 cache lines
// and the kernels are bound by memory-request rate, not bytes. Here the
// weights are packed once (pa_pack_weight) so that each lane block of one
// 16-k step is 1 KB contiguous; activations produced inside the stack are
// written packed by their producer; and the AdaRMSNorm operand, formed from
// user-layout rows, is normalised into LDS by the rows' own waves (coalesced
// 1 KB loads) and read back in the operand layout.
//
// The two residual projections (the out-projection and the FFN's down
// projection) split K across workgroups instead, for either weight layout:
// a 32-column workgroup that walks all of K would stream up to 256 KB of
// weights and re-read the whole activation through one CU.

#include <math.h>

#include "gemm.h"

namespace pa {

// ------------------------------------------------------------ packing -------
// One thread per 16-byte chunk of the packed output.
__global__ __launch_bounds__(256) void pack_weight(const uint4* __restrict__ w, uint4* __restrict__ wp, int N, int K) {
    const long long c = (long long)blockIdx.x * 256 + threadIdx.x;      // packed chunk index
    const long long total = (long long)N * K / 8;
    if (c >= total) return;
    const int lane = (int)(c & 63);
    const long long blk = c >> 6;                                        // nb * (K / 16) + s
    const int s = (int)(blk % (K >> 4)), nb = (int)(blk / (K >> 4));
    const int n = nb * 32 + (lane & 31), k = s * 16 + (lane >> 5) * 8;
    wp[c] = w[((long long)n * K + k) >> 3];
}

// ------------------------------------------------ projection (packed) ----
// A workgroup owns 32 output columns (W block nb) and one 32-row half of the
// packed operand y (both halves of a column block get ids congruent mod 8, so
// they run on one XCD and its L2 serves the weight block to both; a call of at
// most 32 rows launches the first halves only). Its 8 waves split K into KS
// 16-k steps each, load their operand fragments straight from y (1 KB
// contiguous per wave load) and meet in LDS for the reduction over waves, in
// wave order.
enum PackedMode { PK_QKV = 0, PK_GATEUP = 1 };

template <int MODE, int KS>
__global__ __launch_bounds__(GEMM_WAVES * 64, 1) void gemm_packed(const uint16_t* __restrict__ y,
                                                                  const uint16_t* __restrict__ wp1,
                                                                  const uint16_t* __restrict__ wp2, int rows, int N,
                                                                  GemmOut out, uint16_t* __restrict__ act_p) {
    constexpr int K = GEMM_WAVES * KS * 16, S = K / 16;
    __shared__ float red[GEMM_WAVES][16][64];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    int nb, half;
    row_half_block(rows, nb, half);
    if (nb >= N / 32) return;                                       // id padding, whole workgroup
    const int n0 = nb * 32;
    bf16x8 a0[KS], w1[KS], w2[MODE == PK_GATEUP ? KS : 1];
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        const long long st = wave * KS + i;
        a0[i] = *reinterpret_cast<const bf16x8*>(y + ((st * 2 + half) * 64 + lane) * 8);
    }
    const long long wb = ((long long)nb * S + wave * KS) * 512 + lane * 8;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        w1[i] = *reinterpret_cast<const bf16x8*>(wp1 + wb + i * 512);
        if (MODE == PK_GATEUP) w2[i] = *reinterpret_cast<const bf16x8*>(wp2 + wb + i * 512);
    }
    // every fragment load leaves before the first product (the scheduler
    // would otherwise hold later loads behind waits for earlier ones: one
    // memory round trip per few steps instead of one in all)
    __builtin_amdgcn_sched_barrier(0);
    f32x16 c0 = f32x16{}, u0 = f32x16{};
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], w1[i], c0, 0, 0, 0);
        if (MODE == PK_GATEUP) u0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], w2[i], u0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][r][lane] = c0[r];
    __syncthreads();
    float cs[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int r = wave * 2 + u;
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < GEMM_WAVES; ++ww) v += red[ww][r][lane];
        cs[u] = v;
    }
    if (MODE == PK_GATEUP) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 16; ++r) red[wave][r][lane] = u0[r];
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int r = wave * 2 + u;
        const int m = 32 * half + 8 * (r >> 2) + 4 * hi + (r & 3);
        const int n = n0 + l32;
        if (MODE == PK_QKV && out.q_nrb && n < out.nq) {
            // packed q: the padding rows of its last 32-row block are written
            // too (they are zero rows of the product)
            const int h = n / out.q_d;
            if (m * out.q_group + h % out.q_group < out.q_nrb * 32)
                out.q[qpack_index(m, h, n % out.q_d, out.q_group, out.q_nrb, out.q_d)] = f2bf(cs[u]);
            continue;
        }
        if (m >= rows) continue;
        if (MODE == PK_QKV) {
            const float v = cs[u];
            if (n < out.nq)
                out.q[(long long)m * out.nq + n] = f2bf(v);
            else if (n < out.nq + out.nk)
                out.k[(long long)m * out.nk + (n - out.nq)] = f2bf(v);
            else
                out.v[(long long)m * out.nk + (n - out.nq - out.nk)] = f2bf(v);
        } else {
            float up = 0.f;
#pragma unroll
            for (int ww = 0; ww < GEMM_WAVES; ++ww) up += red[ww][r][lane];
            const float gt = cs[u];
            act_p[apack_index(m, n)] = f2bf(gt / (1.f + __expf(-gt)) * up);
        }
    }
}

// ------------------------------------------ split-K residual projection ---
// Workgroup (column block nb, chunk c; with rows > 32 one per 32-row half,
// placed as in gemm_packed) sums k in [SPLITK_CHUNK c, SPLITK_CHUNK (c + 1)):
// wave w the slice of KS MFMA steps from SPLITK_CHUNK c + 16 KS w, the 8
// waves merged in wave order, into part[c][m][n] (FP32, rows m < rows).
template <bool PACKED>
__global__ __launch_bounds__(GEMM_WAVES * 64, 2) void gemm_splitk_part(const uint16_t* __restrict__ a,
                                                                     const uint16_t* __restrict__ w, int rows, int N,
                                                                     int K, float* __restrict__ part) {
    constexpr int KS = SPLITK_KS;
    __shared__ float red[GEMM_WAVES][16][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    const int c = blockIdx.y;
    int nb, half;
    row_half_block(rows, nb, half);
    if (nb >= N / 32) return;                                       // id padding, whole workgroup
    const int n0 = nb * 32;
    bf16x8 wf[KS], a0[KS];
    if (PACKED) {
        const long long S = K / 16;
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            const long long st = (c * GEMM_WAVES + wave) * KS + i;
            wf[i] = *reinterpret_cast<const bf16x8*>(w + ((nb * S + st) * 64 + lane) * 8);
            a0[i] = *reinterpret_cast<const bf16x8*>(a + ((st * 2 + half) * 64 + lane) * 8);
        }
    } else {
        const int k0 = c * SPLITK_CHUNK + wave * KS * 16 + 8 * hi, row = 32 * half + l32;
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            wf[i] = *reinterpret_cast<const bf16x8*>(w + (long long)(n0 + l32) * K + k0 + 16 * i);
            a0[i] = row < rows ? *reinterpret_cast<const bf16x8*>(a + (long long)row * K + k0 + 16 * i) : bf16x8{};
        }
    }
    f32x16 c0 = f32x16{};
#pragma unroll
    for (int i = 0; i < KS; ++i) c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], wf[i], c0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][r][lane] = c0[r];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int r = wave * 2 + u;
        const int m = 32 * half + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (m >= rows) continue;
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < GEMM_WAVES; ++ww) v += red[ww][r][lane];
        part[((long long)c * rows + m) * N + n0 + l32] = v;
    }
}

// h <- bf16(h + sum_c part[c]) in chunk order, x <- bf16(x - dt h) when x is
// set, with the residual epilogue's arithmetic. One thread per element. KC:
// chunk slots (kc <= KC). Every load is issued before the first add, with no
// branch around it (a slot past kc re-reads chunk 0 and is not added), so
// the partials cost one memory round trip.
template <int KC>
__global__ __launch_bounds__(256) void residual_reduce(const float* __restrict__ part, int kc, int rows, int N,
                                                       GemmOut out) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = (long long)rows * N;
    const bool in = i < total;
    const long long ii = in ? i : 0;
    float p[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) p[c] = part[(c < kc ? c : 0) * total + ii];
    const float h0 = bf2f(out.h[ii]);
    const float x0 = out.x ? bf2f(out.x[ii]) : 0.f;
    bool bad = false;
    if (in) {
        float v = 0.f;
#pragma unroll
        for (int c = 0; c < KC; ++c)
            if (c < kc) v += p[c];
        const float hn = bf2f(f2bf(h0 + v));
        out.h[i] = f2bf(hn);
        bad = !finite_f(hn);
        if (out.x) {
            const float xn = x0 - out.dt * hn;
            bad |= !finite_f(xn);
            out.x[i] = f2bf(xn);
        }
    }
    if (out.nonfinite && __any(bad) && (threadIdx.x & 63) == 0) atomicOr(out.nonfinite, 1u);
}

// The same residual with the next AdaRMSNorm: one workgroup per row, 4
// consecutive elements per thread (threads past N / 4 only join the row
// sum). h_out <- bf16(h_in + sum_c part[c]) (chunk order, as residual_reduce;
// kc may be 0), x <- bf16(x - dt h) when x is set, and with nn.gamma set
// y <- bf16(h * rsqrt(mean(h^2) + eps) * gamma): the row's sum of squares in
// FP32, each thread's four in order, then the wave sum, then the waves in
// order. With a packed y, workgroups past `rows` write the padding rows of
// its 64 row slots as zeros. Reports a non-finite h, x or y element.
// KC: chunk slots (kc <= KC). Every operand (the partials, h, x and gamma)
// is loaded up front with no branch around the loads (a slot past kc
// re-reads chunk 0 and is not added; a thread past N / 4 reads the row's
// first elements and stores nothing), so the row costs one memory round
// trip before its sum of squares.
template <int KC>
__global__ __launch_bounds__(512) void residual_norm_rows(const float* __restrict__ part, int kc,
                                                          const uint16_t* h_in, uint16_t* h_out, int rows, int N,
                                                          uint16_t* __restrict__ x, float dt, NormNext nn,
                                                          uint32_t* nonfinite) {
    __shared__ float wsums[8];
    const int m = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6, nw = blockDim.x >> 6;
    const int k0 = 4 * t;
    const bool own = k0 < N;
    uint16_t* y = static_cast<uint16_t*>(nn.y);
    if (m >= rows) {                     // packed padding rows (whole workgroup)
        if (own) *reinterpret_cast<uint2*>(y + apack_index(m, k0)) = make_uint2(0, 0);
        return;
    }
    const int kl = own ? k0 : 0;         // this thread's load column (in the row)
    const long long off = (long long)m * N + k0, loff = (long long)m * N + kl, total = (long long)rows * N;
    float4 p[KC > 0 ? KC : 1];
#pragma unroll
    for (int c = 0; c < KC; ++c) p[c] = *reinterpret_cast<const float4*>(part + (c < kc ? c : 0) * total + loff);
    const uint2 hr = *reinterpret_cast<const uint2*>(h_in + loff);
    const uint2 xr = x ? *reinterpret_cast<const uint2*>(x + loff) : make_uint2(0, 0);
    const float4 g = nn.gamma ? *reinterpret_cast<const float4*>(nn.gamma + kl) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float h0[4] = {__uint_as_float(hr.x << 16), __uint_as_float(hr.x & 0xffff0000u),
                         __uint_as_float(hr.y << 16), __uint_as_float(hr.y & 0xffff0000u)};
    const float x0[4] = {__uint_as_float(xr.x << 16), __uint_as_float(xr.x & 0xffff0000u),
                         __uint_as_float(xr.y << 16), __uint_as_float(xr.y & 0xffff0000u)};
    float hn[4];
    bool bad = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float v = 0.f;
#pragma unroll
        for (int c = 0; c < KC; ++c)
            if (c < kc) v += (e == 0 ? p[c].x : e == 1 ? p[c].y : e == 2 ? p[c].z : p[c].w);
        hn[e] = own ? bf2f(f2bf(h0[e] + v)) : 0.f;
        bad |= !finite_f(hn[e]);
    }
    if (own) *reinterpret_cast<uint2*>(h_out + off) = make_uint2(pack2_bf16(hn[0], hn[1]), pack2_bf16(hn[2], hn[3]));
    if (own && x) {
        float xn[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xn[e] = x0[e] - dt * hn[e];
            bad |= !finite_f(xn[e]);
        }
        *reinterpret_cast<uint2*>(x + off) = make_uint2(pack2_bf16(xn[0], xn[1]), pack2_bf16(xn[2], xn[3]));
    }
    if (nn.gamma) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += hn[e] * hn[e];
        ss = wsum(ss);
        if (lane == 0) wsums[wave] = ss;
        __syncthreads();
        float tot = 0.f;
        for (int w = 0; w < nw; ++w) tot += wsums[w];
        const float rinv = 1.f / sqrtf(tot / (float)N + nn.eps);
        if (own) {
            const uint32_t y01 = pack2_bf16(hn[0] * rinv * g.x, hn[1] * rinv * g.y);
            const uint32_t y23 = pack2_bf16(hn[2] * rinv * g.z, hn[3] * rinv * g.w);
            bad |= nonfinite_seen(nonfinite_bits(y01) | nonfinite_bits(y23)) != 0;
            *reinterpret_cast<uint2*>(y + (nn.packed ? apack_index(m, k0) : off)) = make_uint2(y01, y23);
        }
    }
    if (nonfinite && __any(bad) && lane == 0) atomicOr(nonfinite, 1u);
}

// ------------------------------------------------------------ host side -----
static void launch_norm_rows(const float* part, int kc, const void* h_in, void* h_out, int rows, int N, void* x,
                             float dt, const NormNext& nn, uint32_t* nonfinite, hipStream_t s) {
    const int threads = ((N / 4 + 63) / 64) * 64;
    const int grid = nn.gamma && nn.packed ? 64 : rows;
#define PA_NORM_ROWS(KC)                                                                                     \
    residual_norm_rows<KC><<<grid, threads, 0, s>>>(part, kc, static_cast<const uint16_t*>(h_in),              \
                                                    static_cast<uint16_t*>(h_out), rows, N,                    \
                                                    static_cast<uint16_t*>(x), dt, nn, nonfinite)
    if (kc == 0)
        PA_NORM_ROWS(0);
    else if (kc <= 4)
        PA_NORM_ROWS(4);
    else if (kc <= 8)
        PA_NORM_ROWS(8);
    else
        PA_NORM_ROWS(16);
#undef PA_NORM_ROWS
}

pa_status norm_rows(const void* h_in, void* h_out, int rows, int N, const NormNext& nn, uint32_t* nonfinite,
                    hipStream_t s) {
    PA_CHECK_ARG(nn.gamma && nn.y && N % 128 == 0 && N <= 2048 && rows >= 1 && rows <= 64, PA_ESHAPE,
                 "norm: unsupported shape rows %d, N %d", rows, N);
    launch_norm_rows(nullptr, 0, h_in, h_out, rows, N, nullptr, 0.f, nn, nonfinite, s);
    PA_LAUNCHED();
    return PA_OK;
}

pa_status residual_splitk(const void* a, const void* w, bool packed, void* h, int rows, int K, int N, void* x,
                          float dt, uint32_t* nonfinite, float* part, hipStream_t s, const NormNext* nn) {
    const int kc = K / SPLITK_CHUNK;
    PA_CHECK_ARG(K % SPLITK_CHUNK == 0 && kc >= 1 && K <= 8192 && N % 32 == 0 && rows >= 1 && rows <= 64, PA_ESHAPE,
                 "residual projection: unsupported shape rows %d, K %d, N %d", rows, K, N);
    PA_CHECK_ARG(!nn || (nn->gamma && nn->y && N % 128 == 0 && N <= 2048), PA_ESHAPE,
                 "residual projection: the fused norm needs N a multiple of 128, at most 2048 (got %d)", N);
    const uint16_t* aa = static_cast<const uint16_t*>(a);
    const uint16_t* ww = static_cast<const uint16_t*>(w);
    const dim3 grid(row_half_grid(rows, N), kc), block(GEMM_WAVES * 64);
    if (packed)
        gemm_splitk_part<true><<<grid, block, 0, s>>>(aa, ww, rows, N, K, part);
    else
        gemm_splitk_part<false><<<grid, block, 0, s>>>(aa, ww, rows, N, K, part);
    PA_LAUNCHED();
    if (nn) {
        launch_norm_rows(part, kc, h, h, rows, N, x, dt, *nn, nonfinite, s);
        PA_LAUNCHED();
        return PA_OK;
    }
    GemmOut o{};
    o.h = static_cast<uint16_t*>(h);
    o.x = static_cast<uint16_t*>(x);
    o.dt = dt;
    o.nonfinite = nonfinite;
    const long long total = (long long)rows * N;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (kc <= 4)
        residual_reduce<4><<<blocks, 256, 0, s>>>(part, kc, rows, N, o);
    else if (kc <= 8)
        residual_reduce<8><<<blocks, 256, 0, s>>>(part, kc, rows, N, o);
    else
        residual_reduce<16><<<blocks, 256, 0, s>>>(part, kc, rows, N, o);
    PA_LAUNCHED();
    return PA_OK;
}

bool packed_norm_supported(int model_dim) {
    const int ks = model_dim / 128;
    return model_dim % 512 == 0 && (ks == 4 || ks == 8);
}
bool packed_residual_supported(int K, int N) {
    const int kc = K / 1024;
    return K % 1024 == 0 && (kc == 1 || kc == 2 || kc == 3 || kc == 4 || kc == 6 || kc == 8) && N % 32 == 0;
}

pa_status packed_qkv(const void* y_p, int rows, int model_dim, const void* w_p, int hq, int hkv, int d, void* q,
                     void* k, void* v, bool q_packed, hipStream_t s) {
    GemmOut o{};
    if (q_packed) {
        o.q_nrb = qpack_blocks(rows, hq, hkv);
        o.q_group = hq / hkv;
        o.q_d = d;
    }
    o.q = static_cast<uint16_t*>(q);
    o.k = static_cast<uint16_t*>(k);
    o.v = static_cast<uint16_t*>(v);
    o.nq = hq * d;
    o.nk = hkv * d;
    const int n = (hq + 2 * hkv) * d;
    const uint16_t* yy = static_cast<const uint16_t*>(y_p);
    const uint16_t* ww = static_cast<const uint16_t*>(w_p);
    const int grid = row_half_grid(rows, n);
    if (model_dim == 512)
        gemm_packed<PK_QKV, 4><<<grid, GEMM_WAVES * 64, 0, s>>>(yy, ww, nullptr, rows, n, o, nullptr);
    else
        gemm_packed<PK_QKV, 8><<<grid, GEMM_WAVES * 64, 0, s>>>(yy, ww, nullptr, rows, n, o, nullptr);
    PA_LAUNCHED();
    return PA_OK;
}

pa_status packed_gateup(const void* y_p, int rows, int model_dim, int ffn_dim, const void* wg_p, const void* wu_p,
                        void* act_p, hipStream_t s) {
    GemmOut o{};
    const uint16_t* yy = static_cast<const uint16_t*>(y_p);
    const uint16_t* g = static_cast<const uint16_t*>(wg_p);
    const uint16_t* u = static_cast<const uint16_t*>(wu_p);
    uint16_t* a = static_cast<uint16_t*>(act_p);
    const int grid = row_half_grid(rows, ffn_dim);
    if (model_dim == 512)
        gemm_packed<PK_GATEUP, 4><<<grid, GEMM_WAVES * 64, 0, s>>>(yy, g, u, rows, ffn_dim, o, a);
    else
        gemm_packed<PK_GATEUP, 8><<<grid, GEMM_WAVES * 64, 0, s>>>(yy, g, u, rows, ffn_dim, o, a);
    PA_LAUNCHED();
    return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_pack_weight(const void* w, int32_t n, int32_t k, void* w_packed, void* stream) {
    clear_error();
    PA_CHECK_ARG(w && w_packed, PA_EINVAL, "pa_pack_weight: null argument");
    PA_CHECK_ARG(w != w_packed, PA_EINVAL, "pa_pack_weight: packing cannot be done in place");
    PA_CHECK_ARG((reinterpret_cast<uintptr_t>(w) & 15) == 0 && (reinterpret_cast<uintptr_t>(w_packed) & 15) == 0,
                 PA_EINVAL, "pa_pack_weight: buffers must be 16-byte aligned");
    PA_CHECK_ARG(n >= 32 && n % 32 == 0 && k >= 16 && k % 16 == 0 && (long long)n * k < (1LL << 40), PA_ESHAPE,
                 "pa_pack_weight: need N a multiple of 32 and K a multiple of 16 (got %d x %d)", n, k);
    const long long chunks = (long long)n * k / 8;
    pack_weight<<<(unsigned)((chunks + 255) / 256), 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint4*>(w), static_cast<uint4*>(w_packed), n, k);
    PA_LAUNCHED();
    return PA_OK;
}
