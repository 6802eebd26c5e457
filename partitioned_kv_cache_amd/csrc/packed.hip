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

// -------------------------------------------- norm + projection (packed) ----
// A workgroup owns 32 output columns (W block nb) and all 64 row slots; its
// 8 waves split K into KS 16-k steps each. Wave w normalises rows w, w + 8,
// ... into LDS (its own rows, so no barrier between the mean of squares and
// the scaling); after one barrier every wave reads its operand fragments
// from LDS. The LDS is then reused for the split-K reduction.
enum PackedMode { PK_QKV = 0, PK_GATEUP = 1 };

template <int MODE, int KS>
__global__ __launch_bounds__(GEMM_WAVES * 64, 1) void gemm_norm_packed(
    const uint16_t* __restrict__ x, const float* __restrict__ gamma, float eps, const uint16_t* __restrict__ wp1,
    const uint16_t* __restrict__ wp2, int rows, int N, GemmOut out, uint16_t* __restrict__ act_p) {
    constexpr int K = GEMM_WAVES * KS * 16, S = K / 16;
    constexpr int XS = K + 8;                         // staged row stride in bf16 elements (16 B of padding)
    constexpr int LPR = K / 512;                      // 1 KB row pieces per wave load
    constexpr int RED = GEMM_WAVES * 2 * 16 * 64 * 4;
    constexpr int SMEM = 64 * XS * 2 > RED ? 64 * XS * 2 : RED;
    __shared__ __attribute__((aligned(16))) char smem[SMEM];
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: row choices are scalar branches
    const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    const int nb = blockIdx.x, n0 = nb * 32;

    // normalise rows w, w + 8, ... into LDS (rows >= `rows` are zeros)
    static_assert(K % 512 == 0, "rows are staged in 1 KB pieces");
    float4 g[LPR][2];
#pragma unroll
    for (int c = 0; c < LPR; ++c) {
        g[c][0] = *reinterpret_cast<const float4*>(gamma + c * 512 + lane * 8);
        g[c][1] = *reinterpret_cast<const float4*>(gamma + c * 512 + lane * 8 + 4);
    }
    constexpr int RPW = 64 / GEMM_WAVES;
    uint4 raw[RPW][LPR];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
        const int r = wave + rr * GEMM_WAVES;
#pragma unroll
        for (int c = 0; c < LPR; ++c)
            raw[rr][c] = r < rows ? *reinterpret_cast<const uint4*>(x + (long long)r * K + c * 512 + lane * 8)
                                  : make_uint4(0, 0, 0, 0);
    }
    // Then this wave's weight blocks (KS consecutive 1 KB blocks): issued after
    // x, so the normalisation waits only for x (loads return in issue order)
    // while the weights stream in.
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 w1[KS], w2[MODE == PK_GATEUP ? KS : 1];
    const long long wb = ((long long)nb * S + wave * KS) * 512 + lane * 8;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        w1[i] = *reinterpret_cast<const bf16x8*>(wp1 + wb + i * 512);
        if (MODE == PK_GATEUP) w2[i] = *reinterpret_cast<const bf16x8*>(wp2 + wb + i * 512);
    }
    __builtin_amdgcn_sched_barrier(0);
    uint32_t bad = 0;                  // nonfinite_bits of every rounded operand, as the MFMA sees it
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
        const int r = wave + rr * GEMM_WAVES;          // wave-uniform
        if (r >= rows) {                               // padding rows are zeros
#pragma unroll
            for (int c = 0; c < LPR; ++c)
                *reinterpret_cast<uint4*>(xs + r * XS + c * 512 + lane * 8) = make_uint4(0, 0, 0, 0);
            continue;
        }
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
        const float rinv = 1.f / sqrtf(ss / (float)K + eps);
#pragma unroll
        for (int c = 0; c < LPR; ++c) {
            const uint16_t* e = reinterpret_cast<const uint16_t*>(&raw[rr][c]);
            const float gg[8] = {g[c][0].x, g[c][0].y, g[c][0].z, g[c][0].w, g[c][1].x, g[c][1].y, g[c][1].z, g[c][1].w};
            uint32_t pk[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                pk[u] = pack2_bf16(bf2f(e[2 * u]) * rinv * gg[2 * u], bf2f(e[2 * u + 1]) * rinv * gg[2 * u + 1]);
                bad |= nonfinite_bits(pk[u]);
            }
            *reinterpret_cast<uint4*>(xs + r * XS + c * 512 + lane * 8) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
    }
    if (blockIdx.x == 0 && out.nonfinite && __any(nonfinite_seen(bad)) && lane == 0) atomicOr(out.nonfinite, 1u);
    __syncthreads();
    const int k0 = wave * KS * 16 + 8 * hi;
    bf16x8 a0[KS], a1[KS];
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        a0[i] = *reinterpret_cast<const bf16x8*>(xs + l32 * XS + k0 + 16 * i);
        a1[i] = *reinterpret_cast<const bf16x8*>(xs + (32 + l32) * XS + k0 + 16 * i);
    }
    __syncthreads();                                   // the staging area becomes the reduction buffer
    auto& red = *reinterpret_cast<float (*)[GEMM_WAVES][2][16][64]>(smem);
    const bool two = rows > 32;
    f32x16 c0 = f32x16{}, c1 = f32x16{}, u0 = f32x16{}, u1 = f32x16{};
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], w1[i], c0, 0, 0, 0);
        if (two) c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], w1[i], c1, 0, 0, 0);
        if (MODE == PK_GATEUP) {
            u0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], w2[i], u0, 0, 0, 0);
            if (two) u1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], w2[i], u1, 0, 0, 0);
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        red[wave][0][r][lane] = c0[r];
        red[wave][1][r][lane] = c1[r];
    }
    __syncthreads();
    float cs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int idx = wave * 4 + u, blk = idx >> 4, r = idx & 15;
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < GEMM_WAVES; ++ww) v += red[ww][blk][r][lane];
        cs[u] = v;
    }
    if (MODE == PK_GATEUP) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            red[wave][0][r][lane] = u0[r];
            red[wave][1][r][lane] = u1[r];
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int idx = wave * 4 + u, blk = idx >> 4, r = idx & 15;
        const int m = 32 * blk + 8 * (r >> 2) + 4 * hi + (r & 3);
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
            for (int ww = 0; ww < GEMM_WAVES; ++ww) up += red[ww][blk][r][lane];
            const float gt = cs[u];
            act_p[apack_index(m, n)] = f2bf(gt / (1.f + __expf(-gt)) * up);
        }
    }
}

// ------------------------------------------ split-K residual projection ---
// Workgroup (column block nb, chunk c) sums k in [SPLITK_CHUNK c,
// SPLITK_CHUNK (c + 1)): wave w the slice of KS MFMA steps from
// SPLITK_CHUNK c + 16 KS w, the 8 waves merged in wave order, into
// part[c][m][n] (FP32, rows m < rows).
template <bool PACKED>
__global__ __launch_bounds__(GEMM_WAVES * 64, 2) void gemm_splitk_part(const uint16_t* __restrict__ a,
                                                                     const uint16_t* __restrict__ w, int rows, int N,
                                                                     int K, float* __restrict__ part) {
    constexpr int KS = SPLITK_KS;
    __shared__ float red[GEMM_WAVES][2][16][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    const int nb = blockIdx.x, c = blockIdx.y, n0 = nb * 32;
    const bool two = rows > 32;
    bf16x8 wf[KS], a0[KS], a1[KS];
    if (PACKED) {
        const long long S = K / 16;
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            const long long st = (c * GEMM_WAVES + wave) * KS + i;
            wf[i] = *reinterpret_cast<const bf16x8*>(w + ((nb * S + st) * 64 + lane) * 8);
            a0[i] = *reinterpret_cast<const bf16x8*>(a + ((st * 2) * 64 + lane) * 8);
            a1[i] = two ? *reinterpret_cast<const bf16x8*>(a + ((st * 2 + 1) * 64 + lane) * 8) : bf16x8{};
        }
    } else {
        const int k0 = c * SPLITK_CHUNK + wave * KS * 16 + 8 * hi;
        const bool r0 = l32 < rows, r1 = 32 + l32 < rows;
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            wf[i] = *reinterpret_cast<const bf16x8*>(w + (long long)(n0 + l32) * K + k0 + 16 * i);
            a0[i] = r0 ? *reinterpret_cast<const bf16x8*>(a + (long long)l32 * K + k0 + 16 * i) : bf16x8{};
            a1[i] = r1 ? *reinterpret_cast<const bf16x8*>(a + (long long)(32 + l32) * K + k0 + 16 * i) : bf16x8{};
        }
    }
    f32x16 c0 = f32x16{}, c1 = f32x16{};
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
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int idx = wave * 4 + u, blk = idx >> 4, r = idx & 15;
        const int m = 32 * blk + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (m >= rows) continue;
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < GEMM_WAVES; ++ww) v += red[ww][blk][r][lane];
        part[((long long)c * rows + m) * N + n0 + l32] = v;
    }
}

// h <- bf16(h + sum_c part[c]) in chunk order, x <- bf16(x - dt h) when x is
// set, with the residual epilogue's arithmetic. One thread per element.
__global__ __launch_bounds__(256) void residual_reduce(const float* __restrict__ part, int kc, int rows, int N,
                                                       GemmOut out) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = (long long)rows * N;
    bool bad = false;
    if (i < total) {
        // every load issued before the first add
        constexpr int MAXC = 8192 / SPLITK_CHUNK;
        float p[MAXC];
#pragma unroll
        for (int c = 0; c < MAXC; ++c) p[c] = c < kc ? part[c * total + i] : 0.f;
        const float h0 = bf2f(out.h[i]);
        const float x0 = out.x ? bf2f(out.x[i]) : 0.f;
        float v = 0.f;
#pragma unroll
        for (int c = 0; c < MAXC; ++c)
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

// ------------------------------------------------------------ host side -----
pa_status residual_splitk(const void* a, const void* w, bool packed, void* h, int rows, int K, int N, void* x,
                           float dt, uint32_t* nonfinite, float* part, hipStream_t s) {
    const int kc = K / SPLITK_CHUNK;
    PA_CHECK_ARG(K % SPLITK_CHUNK == 0 && kc >= 1 && K <= 8192 && N % 32 == 0 && rows >= 1 && rows <= 64, PA_ESHAPE,
                 "residual projection: unsupported shape rows %d, K %d, N %d", rows, K, N);
    const uint16_t* aa = static_cast<const uint16_t*>(a);
    const uint16_t* ww = static_cast<const uint16_t*>(w);
    const dim3 grid(N / 32, kc), block(GEMM_WAVES * 64);
    if (packed)
        gemm_splitk_part<true><<<grid, block, 0, s>>>(aa, ww, rows, N, K, part);
    else
        gemm_splitk_part<false><<<grid, block, 0, s>>>(aa, ww, rows, N, K, part);
    PA_LAUNCHED();
    GemmOut o{};
    o.h = static_cast<uint16_t*>(h);
    o.x = static_cast<uint16_t*>(x);
    o.dt = dt;
    o.nonfinite = nonfinite;
    const long long total = (long long)rows * N;
    residual_reduce<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(part, kc, rows, N, o);
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

pa_status packed_norm_qkv(const void* x, int rows, int model_dim, const float* gamma, float eps, const void* w_p,
                          int hq, int hkv, int d, void* q, void* k, void* v, uint32_t* nonfinite, bool q_packed,
                          hipStream_t s) {
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
    o.nonfinite = nonfinite;
    const int n = (hq + 2 * hkv) * d;
    const uint16_t* xx = static_cast<const uint16_t*>(x);
    const uint16_t* ww = static_cast<const uint16_t*>(w_p);
    if (model_dim == 512)
        gemm_norm_packed<PK_QKV, 4><<<n / 32, GEMM_WAVES * 64, 0, s>>>(xx, gamma, eps, ww, nullptr, rows, n, o, nullptr);
    else
        gemm_norm_packed<PK_QKV, 8><<<n / 32, GEMM_WAVES * 64, 0, s>>>(xx, gamma, eps, ww, nullptr, rows, n, o, nullptr);
    PA_LAUNCHED();
    return PA_OK;
}

pa_status packed_norm_gateup(const void* h, int rows, int model_dim, int ffn_dim, const float* gamma, float eps,
                             const void* wg_p, const void* wu_p, void* act_p, uint32_t* nonfinite, hipStream_t s) {
    GemmOut o{};
    o.nonfinite = nonfinite;
    const uint16_t* xx = static_cast<const uint16_t*>(h);
    const uint16_t* g = static_cast<const uint16_t*>(wg_p);
    const uint16_t* u = static_cast<const uint16_t*>(wu_p);
    uint16_t* a = static_cast<uint16_t*>(act_p);
    if (model_dim == 512)
        gemm_norm_packed<PK_GATEUP, 4><<<ffn_dim / 32, GEMM_WAVES * 64, 0, s>>>(xx, gamma, eps, g, u, rows, ffn_dim, o, a);
    else
        gemm_norm_packed<PK_GATEUP, 8><<<ffn_dim / 32, GEMM_WAVES * 64, 0, s>>>(xx, gamma, eps, g, u, rows, ffn_dim, o, a);
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
