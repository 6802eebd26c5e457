// Pieces shared by the skinny GEMMs of the layer glue (adanorm.hip and
// packed.hip): the output descriptor, the wave count, a wave sum and the
// residual epilogue.
#pragma once

#include "internal.h"

namespace pa {

__device__ __forceinline__ float wsum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

constexpr int GEMM_WAVES = 8;

struct GemmOut {
    // GEMM_QKV: columns [0, nq) -> q, [nq, nq+nk) -> k, [nq+nk, nq+2nk) -> v
    uint16_t* q; uint16_t* k; uint16_t* v; int nq; int nk;
    // GEMM_OPROJ: h += C (rounded to bf16); x -= dt * h when x != null
    uint16_t* h; uint16_t* x; float dt;
    uint32_t* nonfinite;
};

// h <- bf16(h + C) and, when x is set, x <- bf16(x - dt h), for the 4 of the
// 32 (row block, register) pairs wave w finishes; C's partial sums per wave
// are in red. Every load of h and x is issued before the first store.
__device__ __forceinline__ void residual_epilogue(const float (&red)[GEMM_WAVES][2][16][64], int n0, int rows, int N,
                                                  const GemmOut& out) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    const int n = n0 + l32;
    long long off[4];
    bool ok[4];
    float hv[4], xv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int idx = wave * 4 + u, blk = idx >> 4, r = idx & 15;
        const int m = 32 * blk + 8 * (r >> 2) + 4 * hi + (r & 3);
        ok[u] = m < rows;
        off[u] = (long long)(ok[u] ? m : 0) * N + n;
        hv[u] = ok[u] ? bf2f(out.h[off[u]]) : 0.f;
        xv[u] = ok[u] && out.x ? bf2f(out.x[off[u]]) : 0.f;
    }
    bool bad = false;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (!ok[u]) continue;
        const int idx = wave * 4 + u, blk = idx >> 4, r = idx & 15;
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < GEMM_WAVES; ++ww) v += red[ww][blk][r][lane];
        const float hn = bf2f(f2bf(hv[u] + v));
        out.h[off[u]] = f2bf(hn);
        bad |= !finite_f(hn);
        if (out.x) {
            const float xn = xv[u] - out.dt * hn;
            bad |= !finite_f(xn);
            out.x[off[u]] = f2bf(xn);
        }
    }
    if (out.nonfinite && __any(bad) && lane == 0) atomicOr(out.nonfinite, 1u);
}

// ---- fragment-packed operands (packed.hip) ------------------------------
// One 1 KB block holds the 64 lanes' 16-byte operand of one 16-k step of
// v_mfma_f32_32x32x16_bf16 (lane = 32 * ((k % 16) / 8) + row % 32):
//   weight W [N][K] -> [N / 32][K / 16][64 lanes][8]
//   activation A [M <= 64][K] -> [K / 16][2 row halves][64 lanes][8]
// so every load of the GEMMs below is 1 KB contiguous across a wave.
__host__ __device__ inline long long wpack_index(int n, int k, int K) {
    return (((long long)(n >> 5) * (K >> 4) + (k >> 4)) * 64 + ((k >> 3) & 1) * 32 + (n & 31)) * 8 + (k & 7);
}
__host__ __device__ inline long long apack_index(int m, int k) {
    return (((long long)(k >> 4) * 2 + (m >> 5)) * 64 + ((k >> 3) & 1) * 32 + (m & 31)) * 8 + (k & 7);
}

// Stack-internal GEMMs on packed operands (rows <= 64).
//   q|k|v = bf16(AdaRMSNorm(x, gamma)) W_qkv^T           (W_qkv packed)
pa_status packed_norm_qkv(const void* x, int rows, int model_dim, const float* gamma, float eps, const void* w_qkv_p,
                          int hq, int hkv, int d, void* q, void* k, void* v, uint32_t* nonfinite, hipStream_t s);
//   act_p = packed bf16(SiLU(y W_gate^T) * (y W_up^T)), y = bf16(AdaRMSNorm(h, gamma))
pa_status packed_norm_gateup(const void* h, int rows, int model_dim, int ffn_dim, const float* gamma, float eps,
                             const void* w_gate_p, const void* w_up_p, void* act_p, uint32_t* nonfinite,
                             hipStream_t s);
//   h <- bf16(h + A W^T); x <- bf16(x - dt h) when x is set   (A and W packed, K = 1024 * KC)
//   wave_major: sum in the order of oproj_residual, else in that of ffn_swiglu's down projection
pa_status packed_residual(const void* a_p, const void* w_p, void* h, int rows, int K, int N, void* x, float dt,
                          uint32_t* nonfinite, bool wave_major, hipStream_t s);
bool packed_residual_supported(int K, int N);
bool packed_norm_supported(int model_dim);

// pattn_step writing its bf16 output in the packed activation layout
// [K = Hq * D] for the out-projection (rows = suffix tokens <= 64).
pa_status pattn_step_apacked(const rb_ring* ring, const pattn_args* a, const void* q, const void* k_dyn,
                             const void* v_dyn, void* out_p, void* ws, size_t ws_bytes, void* stream);

}  // namespace pa
