// Pieces shared by the skinny GEMMs of the layer glue (adanorm.hip and
// packed.hip): the output descriptor, the wave count, a wave sum and the
// residual epilogue.
#pragma once

#include "internal.h"

namespace pa {

// Sum over the 64 lanes of a wave, the same value in every lane. Partners at
// lane distance 1, 2 (quad permutes), 4 (half-row mirror), 8 (row mirror),
// 16 (a swizzled shuffle) and 32 (permlane32 swap): vector ALU steps, except
// the one at 16, instead of six LDS permutes. Each step adds the same pair in
// every lane of the pair, so all lanes end with bit-identical sums.
__device__ __forceinline__ float wsum(float v) {
#define PA_DPP(x, ctrl) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false))
    v += PA_DPP(v, 0xB1);    // quad_perm [1, 0, 3, 2]
    v += PA_DPP(v, 0x4E);    // quad_perm [2, 3, 0, 1]
    v += PA_DPP(v, 0x141);   // row_half_mirror
    v += PA_DPP(v, 0x140);   // row_mirror
#undef PA_DPP
    v += __shfl_xor(v, 16);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Two floats to packed bf16 words (round to nearest even), low word first.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, b2));
}

// Non-finite test on two packed bf16 words: an all-ones exponent (0x7F80)
// carries into the word's top bit when 0x80 is added to the masked exponent,
// and no other exponent does. OR the results; test with nonfinite_seen().
__device__ __forceinline__ uint32_t nonfinite_bits(uint32_t w) { return (w & 0x7F807F80u) + 0x00800080u; }
__device__ __forceinline__ bool nonfinite_seen(uint32_t acc) { return (acc & 0x80008000u) != 0; }

constexpr int GEMM_WAVES = 8;

// Workgroups of a 64-row projection that gives each workgroup 32 output
// columns and one 32-row half of the operand: ids 16 j + 8 h + x take column
// block 8 j + x and half h (both halves of a block on one XCD, sharing its
// weights in L2), padded to whole groups of 16; with at most 32 rows, one per
// column block. row_half_block decodes an id (nb >= N / 32 marks padding).
inline int row_half_grid(int rows, int n) { return rows > 32 ? 16 * ((n / 32 + 7) / 8) : n / 32; }
__device__ __forceinline__ void row_half_block(int rows, int& nb, int& half) {
    nb = blockIdx.x;
    half = 0;
    if (rows > 32) {
        nb = ((blockIdx.x >> 4) << 3) | (blockIdx.x & 7);
        half = (blockIdx.x >> 3) & 1;
    }
}

struct GemmOut {
    // GEMM_QKV: columns [0, nq) -> q, [nq, nq+nk) -> k, [nq+nk, nq+2nk) -> v
    uint16_t* q; uint16_t* k; uint16_t* v; int nq; int nk;
    // q_nrb > 0: q goes to the attention kernel's B-operand order (qpack_index),
    // q_nrb 32-row blocks per KV head, q_group query heads per KV head, head dim q_d
    int q_nrb, q_group, q_d;
    // GEMM_OPROJ: h += C (rounded to bf16); x -= dt * h when x != null
    uint16_t* h; uint16_t* x; float dt;
    uint32_t* nonfinite;
};

// h <- bf16(h + C) and, when x is set, x <- bf16(x - dt h), for the 4 of the
// 32 (row block, register) pairs wave w finishes; C's partial sums per wave
// are in red. Every load of h and x is issued before the first store.
// The h (and x) elements of the (block, register) pairs a wave finishes,
// loaded up front: every load is issued (a row past `rows` reads row 0, in
// bounds, and is zeroed), so they share the operand loads' round trip.
struct ResidualRows {
    long long off[4];
    bool ok[4];
    float hv[4], xv[4];
};
__device__ __forceinline__ ResidualRows residual_rows(int n0, int rows, int N, const GemmOut& out) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    const int n = n0 + l32;
    ResidualRows rr;
    uint16_t hb[4], xb[4];
    const uint16_t* xs = out.x ? out.x : out.h;     // no x: a second read of h, unused
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int idx = wave * 4 + u, blk = idx >> 4, r = idx & 15;
        const int m = 32 * blk + 8 * (r >> 2) + 4 * hi + (r & 3);
        rr.ok[u] = m < rows;
        rr.off[u] = (long long)(rr.ok[u] ? m : 0) * N + n;
        hb[u] = out.h[rr.off[u]];
        xb[u] = xs[rr.off[u]];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        rr.hv[u] = rr.ok[u] ? bf2f(hb[u]) : 0.f;
        rr.xv[u] = rr.ok[u] && out.x ? bf2f(xb[u]) : 0.f;
    }
    return rr;
}

__device__ __forceinline__ void residual_epilogue(const float (&red)[GEMM_WAVES][2][16][64], const ResidualRows& rr,
                                                  const GemmOut& out) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    bool bad = false;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (!rr.ok[u]) continue;
        const int idx = wave * 4 + u, blk = idx >> 4, r = idx & 15;
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < GEMM_WAVES; ++ww) v += red[ww][blk][r][lane];
        const float hn = bf2f(f2bf(rr.hv[u] + v));
        out.h[rr.off[u]] = f2bf(hn);
        bad |= !finite_f(hn);
        if (out.x) {
            const float xn = rr.xv[u] - out.dt * hn;
            bad |= !finite_f(xn);
            out.x[rr.off[u]] = f2bf(xn);
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
// Query (token m, head h, dim d) in the attention kernel's Q operand order:
// row r = m * group + h % group of KV head g = h / group, in 32-row blocks.
__host__ __device__ inline long long qpack_index(int m, int h, int d, int group, int nrb, int D) {
    const int g = h / group, r = m * group + h % group;
    return ((((long long)g * nrb + (r >> 5)) * (D >> 4) + (d >> 4)) * 64 + ((d >> 3) & 1) * 32 + (r & 31)) * 8 + (d & 7);
}
__host__ __device__ inline long long apack_index(int m, int k) {
    return (((long long)(k >> 4) * 2 + (m >> 5)) * 64 + ((k >> 3) & 1) * 32 + (m & 31)) * 8 + (k & 7);
}

// Stack-internal GEMMs (rows <= 64) on an operand y = bf16(AdaRMSNorm(h))
// that the residual kernel before them has already formed (NormNext):
//   q|k|v = y W_qkv^T
//   act   = bf16(SiLU(y W_gate^T) * (y W_up^T))
// packed_*: y and the weights in fragment order (y over 64 row slots, the
// padding rows zero), q in operand order when q_packed, act written packed;
// *_proj (adanorm.hip): y [rows][model_dim], nn.Linear weights. Both sum in
// the same order.
pa_status packed_qkv(const void* y_p, int rows, int model_dim, const void* w_qkv_p, int hq, int hkv, int d, void* q,
                     void* k, void* v, bool q_packed, hipStream_t s);
pa_status packed_gateup(const void* y_p, int rows, int model_dim, int ffn_dim, const void* w_gate_p,
                        const void* w_up_p, void* act_p, hipStream_t s);
pa_status qkv_proj(const void* y, int rows, int model_dim, const void* w_qkv, int hq, int hkv, int d, void* q,
                   void* k, void* v, hipStream_t s);
pa_status gateup_proj(const void* y, int rows, int model_dim, int ffn_dim, const void* w_gate, const void* w_up,
                      void* act, hipStream_t s);
// 32-row blocks per KV head of the packed Q of `rows` tokens
inline int qpack_blocks(int rows, int hq, int hkv) { return (rows * (hq / hkv) + 31) / 32; }

// The AdaRMSNorm of the next GEMM's operand, fused into the kernel that
// finishes h: y = bf16(h / sqrt(mean(h^2) + eps) * gamma), FP32 arithmetic,
// written in fragment order over 64 row slots (packed; padding rows zero) or
// as [rows][N].
struct NormNext {
    const float* gamma;
    float eps;
    void* y;
    bool packed;
};
// Residual projection h <- bf16(h + A W^T); x <- bf16(x - dt h) when x is
// set -- the stack's out-projection and the FFN's down projection -- split
// over K: KC = K / SPLITK_CHUNK workgroups per 32 columns each sum one chunk
// (their 8 waves one SPLITK_CHUNK / 8 slice each, merged in wave order) into
// FP32 partials part[KC][rows][N]; a second kernel adds the chunks in order
// and applies the residual. A and W packed (fragment order) or in row-major /
// nn.Linear layout; both sum in the same order, so the two agree bit for bit.
// With nn, the reduction runs one workgroup per row and also forms the next
// operand y (the h it writes is the same).
pa_status residual_splitk(const void* a, const void* w, bool packed, void* h, int rows, int K, int N, void* x,
                          float dt, uint32_t* nonfinite, float* part, hipStream_t s, const NormNext* nn = nullptr);
// h_out <- h_in and y <- AdaRMSNorm(h_in) (the first layer's operand; h_out
// may be h_in).
pa_status norm_rows(const void* h_in, void* h_out, int rows, int N, const NormNext& nn, uint32_t* nonfinite,
                    hipStream_t s);
constexpr int SPLITK_KS = 4;                                // MFMA k-steps per wave and chunk
constexpr int SPLITK_CHUNK = GEMM_WAVES * SPLITK_KS * 16;   // k per workgroup
inline bool residual_splitk_supported(int K, int N) {
    return K % SPLITK_CHUNK == 0 && K >= SPLITK_CHUNK && K <= 8192 && N % 32 == 0;
}
inline size_t residual_splitk_bytes(int rows, int K, int N) {
    return align_up((size_t)(K / SPLITK_CHUNK) * rows * N * 4, 256);
}
bool packed_residual_supported(int K, int N);
bool packed_norm_supported(int model_dim);

// pattn_step writing its bf16 output in the packed activation layout
// [K = Hq * D] for the out-projection (rows = suffix tokens <= 64); with
// q_packed, q is in the attention kernel's operand order (qpack_index).
pa_status pattn_step_apacked(const rb_ring* ring, const pattn_args* a, const void* q, const void* k_dyn,
                             const void* v_dyn, void* out_p, void* ws, size_t ws_bytes, void* stream,
                             bool q_packed);

}  // namespace pa
