// Partitioned attention over [pin | sliding window | dynamic suffix].
//
// "Reflex: Real-Time VLA Control through Streaming Inference" paper review,
// §3 Architecture, Eq. 1 (softmax over the concatenation of the three
// regions) and Prop. A.1 (softmax is invariant to how its keys are
// partitioned and ordered, so per-region or per-split partial results merged
// exactly reproduce full-batch attention).
//
// Work split: the keys of one (layer, KV head) are cut into contiguous
// splits; each workgroup reduces one split for a block of query rows to a
// partial (running max m, running sum l, unnormalised accumulator O) kept in
// FP32, in base-2 units (logits are pre-multiplied by scale * log2 e).
// `combine` merges the partials of every split:
//     m* = max_s m_s,  l* = sum_s l_s 2^(m_s - m*),  out = sum_s O_s 2^(m_s - m*) / l*.
//
// Query rows: every query head that shares a KV head reads the same keys, so
// the rows of one (layer, KV head) are all (token, head-in-group) pairs:
// row r -> token r / G, head g*G + r % G, with G = Hq / Hkv. For the
// Pi0.5-like shape (8 heads, 1 KV head, 51 tokens) that is one 408 x 256
// query matrix against each K/V tile, which is what makes bf16 MFMA pay.

#include <math.h>

#include "internal.h"

namespace pa {

constexpr int KT = 32;           // keys per MFMA tile
constexpr int MFMA_WAVES = 4;    // waves per workgroup, 32 query rows each
constexpr int ROWS_PER_WG = MFMA_WAVES * 32;
constexpr int VALU_ROWS = 4;     // query rows per workgroup of the vector kernels

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <typename T> __device__ __forceinline__ float ldf(const T* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p) { return bf2f(*p); }

struct Partials {
    float* o;        // [parts][lg][mpad][D]
    float2* ml;      // [parts][lg][mpad]   (m, l)
    int mpad;
    int lg_count;    // call-layers x KV heads
    __device__ __forceinline__ long long idx(int part, int lg, int row) const {
        return ((long long)part * lg_count + lg) * mpad + row;
    }
};

// ---------------------------------------------------------------------------
// Vector (VALU) partial: one wave per query row, FP32 arithmetic. Used for
// f32 rings, where parity is held to 1e-5 absolute.
// grid (splits, ceil(M / 4), Lb * Hkv), block 256, dynamic LDS 4 * D floats.
template <typename T>
__global__ __launch_bounds__(256) void partial_valu(const T* q, long long q_layer, int hq, int group, int m_rows,
                                                    KvSource src, int chunk, float scale_log2, Partials part) {
    extern __shared__ float qs[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int split = blockIdx.x, lg = blockIdx.z;
    const int lb = lg / src.hkv, g = lg % src.hkv;
    const int row = blockIdx.y * VALU_ROWS + wave;
    const int D = src.d;
    const bool row_ok = row < m_rows;
    const int tok = row / group, head = g * group + row % group;
    for (int d = lane; d < D; d += 64)
        qs[wave * D + d] = row_ok ? ldf(q + lb * q_layer + ((long long)tok * hq + head) * D + d) : 0.f;
    __syncthreads();

    const int k_begin = split * chunk, k_end = min(k_begin + chunk, src.total());
    float m = -INFINITY, l = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int base = k_begin; base < k_end; base += 64) {
        const int j = base + lane;
        float s = -INFINITY;
        if (j < k_end) {
            bool dyn;
            const long long off = src.offset(lb, g, j, dyn);
            const T* kp = static_cast<const T*>(dyn ? src.dyn_k : src.ring_k) + off;
            float z = 0.f;
            for (int d = 0; d < D; ++d) z += qs[wave * D + d] * ldf(kp + d);
            s = z * scale_log2;
        }
        const float mn = fmaxf(m, wave_max(s));      // finite: base < k_end
        const float alpha = exp2f(m - mn);
        const float p = j < k_end ? exp2f(s - mn) : 0.f;
        l = l * alpha + wave_sum(p);
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] *= alpha;
        const int nvalid = min(64, k_end - base);
        for (int jj = 0; jj < nvalid; ++jj) {
            const float pj = __shfl(p, jj);
            bool dyn;
            const long long off = src.offset(lb, g, base + jj, dyn);
            const T* vp = static_cast<const T*>(dyn ? src.dyn_v : src.ring_v) + off;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int d = lane + 64 * c;
                if (d < D) o[c] += pj * ldf(vp + d);
            }
        }
        m = mn;
    }
    if (row_ok) {
        float* op = part.o + part.idx(split, lg, row) * D;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int d = lane + 64 * c;
            if (d < D) op[d] = o[c];
        }
        if (lane == 0) part.ml[part.idx(split, lg, row)] = make_float2(m, l);
    }
}

// ---------------------------------------------------------------------------
// bf16 MFMA partial. Each wave owns 32 query rows; the workgroup stages one
// tile of KT keys at a time in LDS (K row-major, V transposed) and every
// wave computes
//     S^T (KT x 32)  = K_tile (KT x D) . Q^T (D x 32)        v_mfma_f32_32x32x16_bf16
//     O^T (D x 32)  += V_tile^T (D x KT) . P^T (KT x 32)
// In the transposed form each lane holds one query row's scores, so the
// softmax statistics are per lane plus one swap with lane ^ 32, and P feeds
// the second product straight from registers. The K rows fed to the first
// product are permuted (bits 2 and 3 of the row index swapped) so that
// after the product every lane holds 8 consecutive keys per 16-key step:
// exactly the B-operand layout of the second product.
//
// MFMA 32x32x16 operand layout (64 lanes, l32 = lane % 32, hi = lane / 32):
//   A[m][k]: lane holds m = l32, k = 8 hi .. 8 hi + 7
//   B[k][n]: lane holds n = l32, k = 8 hi .. 8 hi + 7
//   C[m][n]: lane holds n = l32, m = 8 (r / 4) + 4 hi + r % 4, r = 0 .. 15
//
// grid (splits, ceil(M / 128), Lb * Hkv), block 256.
template <int D>
__global__ __launch_bounds__(MFMA_WAVES * 64, 2) void partial_mfma(const uint16_t* __restrict__ q, long long q_layer,
                                                                   int hq, int group, int m_rows, KvSource src,
                                                                   int chunk, float scale_log2, Partials part) {
    constexpr int KD = D / 16;    // k-steps over the head dimension
    constexpr int DB = D / 32;    // 32-wide blocks of the output
    constexpr int KP = D + 8;     // K tile pitch (elements): 16-byte skew per row
    constexpr int VP = KT + 8;    // V^T tile pitch
    constexpr int CH = KT * D / 8;  // 16-byte chunks per tile
    __shared__ __attribute__((aligned(16))) uint16_t ks[KT * KP];
    __shared__ __attribute__((aligned(16))) uint16_t vt[D * VP];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int split = blockIdx.x, lg = blockIdx.z;
    const int lb = lg / src.hkv, g = lg % src.hkv;
    const int row = blockIdx.y * ROWS_PER_WG + wave * 32 + l32;

    bf16x8 qf[KD];
    if (row < m_rows) {
        const uint16_t* qp = q + lb * q_layer + ((long long)(row / group) * hq + g * group + row % group) * D + 8 * hi;
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
    } else {
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) qf[kk] = bf16x8{};
    }

    f32x16 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const int k_begin = split * chunk, k_end = min(k_begin + chunk, src.total());
    const int prow = (l32 & ~0xC) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);

    for (int base = k_begin; base < k_end; base += KT) {
        for (int c = tid; c < CH; c += MFMA_WAVES * 64) {       // K: row-major
            const int key = c / (D / 8), dc = c % (D / 8), j = base + key;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (j < k_end) {
                bool dyn;
                const long long off = src.offset(lb, g, j, dyn);
                val = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(dyn ? src.dyn_k : src.ring_k) + off + dc * 8);
            }
            *reinterpret_cast<uint4*>(&ks[key * KP + dc * 8]) = val;
        }
        for (int c = tid; c < CH; c += MFMA_WAVES * 64) {       // V: transposed
            const int key = c % KT, dc = c / KT, j = base + key;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (j < k_end) {
                bool dyn;
                const long long off = src.offset(lb, g, j, dyn);
                val = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(dyn ? src.dyn_v : src.ring_v) + off + dc * 8);
            }
            const uint16_t* e = reinterpret_cast<const uint16_t*>(&val);
#pragma unroll
            for (int i = 0; i < 8; ++i) vt[(dc * 8 + i) * VP + key] = e[i];
        }
        __syncthreads();

        f32x16 s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&ks[prow * KP + 16 * kk + 8 * hi]);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s, 0, 0, 0);
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = base + 16 * (r >> 3) + 8 * hi + (r & 7);
            const float x = key < k_end ? s[r] * scale_log2 : -INFINITY;
            s[r] = x;
            tmax = fmaxf(tmax, x);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = exp2f(m_run - m_new);
        float psum = 0.f;
        bf16x8 pf[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = exp2f(s[r] - m_new);
            psum += p;
            pf[r >> 3][r & 7] = (__bf16)p;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int b = 0; b < DB; ++b) acc[b] *= alpha;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(&vt[(32 * b + l32) * VP + 16 * s2 + 8 * hi]);
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[s2], acc[b], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    l_run += __shfl_xor(l_run, 32);
    if (row < m_rows) {
        float* op = part.o + part.idx(split, lg, row) * D;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<float4*>(op + 32 * b + 8 * j + 4 * hi) =
                    make_float4(acc[b][4 * j], acc[b][4 * j + 1], acc[b][4 * j + 2], acc[b][4 * j + 3]);
        if (hi == 0) part.ml[part.idx(split, lg, row)] = make_float2(m_run, l_run);
    }
}

// ---------------------------------------------------------------------------
// Private-tail partial of the decode readers: one wave per (stream, head)
// row over that stream's own appended tokens. Writes partial slot `slot`.
// grid (ceil(M / 4), Lb * Hkv), block 256, dynamic LDS 4 * D floats.
template <typename T>
__global__ __launch_bounds__(256) void partial_tail(const T* q, long long q_layer, int hq, int group, int m_rows,
                                                    const T* tail_k, const T* tail_v, const int32_t* tail_len,
                                                    int n_streams, int cap, int hkv, int D, float scale_log2,
                                                    int slot, Partials part) {
    extern __shared__ float qs[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lg = blockIdx.y, lb = lg / hkv, g = lg % hkv;
    const int row = blockIdx.x * VALU_ROWS + wave;
    const bool row_ok = row < m_rows;
    const int strm = row_ok ? row / group : 0, head = g * group + row % group;
    for (int d = lane; d < D; d += 64)
        qs[wave * D + d] = row_ok ? ldf(q + lb * q_layer + ((long long)strm * hq + head) * D + d) : 0.f;
    __syncthreads();
    int n = row_ok ? tail_len[strm] : 0;
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const long long tok_base = ((long long)lb * n_streams + strm) * cap;
    float m = -INFINITY, l = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int base = 0; base < n; base += 64) {
        const int j = base + lane;
        float s = -INFINITY;
        if (j < n) {
            const T* kp = tail_k + ((tok_base + j) * hkv + g) * D;
            float z = 0.f;
            for (int d = 0; d < D; ++d) z += qs[wave * D + d] * ldf(kp + d);
            s = z * scale_log2;
        }
        const float mn = fmaxf(m, wave_max(s));
        const float alpha = exp2f(m - mn);
        const float p = j < n ? exp2f(s - mn) : 0.f;
        l = l * alpha + wave_sum(p);
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] *= alpha;
        const int nvalid = min(64, n - base);
        for (int jj = 0; jj < nvalid; ++jj) {
            const float pj = __shfl(p, jj);
            const T* vp = tail_v + ((tok_base + base + jj) * hkv + g) * D;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int d = lane + 64 * c;
                if (d < D) o[c] += pj * ldf(vp + d);
            }
        }
        m = mn;
    }
    if (row_ok) {
        float* op = part.o + part.idx(slot, lg, row) * D;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int d = lane + 64 * c;
            if (d < D) op[d] = o[c];
        }
        if (lane == 0) part.ml[part.idx(slot, lg, row)] = make_float2(m, l);
    }
}

// ---------------------------------------------------------------------------
// Log-sum-exp combine of `n_parts` partials per row (Prop. A.1), FP32.
// One wave per query row; writes out[lb][token][head][d] in the output dtype.
// grid (ceil(M / 4), Lb * Hkv), block 256.
template <typename TO> __device__ __forceinline__ void st(TO* p, float v);
template <> __device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<uint16_t>(uint16_t* p, float v) { *p = f2bf(v); }

template <typename TO>
__global__ __launch_bounds__(256) void combine(Partials part, int n_parts, int m_rows, int group, int hq, int hkv,
                                               int D, long long out_layer, TO* out) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = blockIdx.x * VALU_ROWS + wave, lg = blockIdx.y;
    if (row >= m_rows) return;
    const int lb = lg / hkv, g = lg % hkv;
    float mx = -INFINITY;
    for (int s = 0; s < n_parts; ++s) mx = fmaxf(mx, part.ml[part.idx(s, lg, row)].x);
    float lsum = 0.f;
    for (int s = 0; s < n_parts; ++s) {
        const float2 ml = part.ml[part.idx(s, lg, row)];
        if (ml.x != -INFINITY) lsum += ml.y * exp2f(ml.x - mx);
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    TO* op = out + lb * out_layer + ((long long)(row / group) * hq + g * group + row % group) * D;
    for (int d = lane * 4; d < D; d += 256) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s = 0; s < n_parts; ++s) {
            const float ms = part.ml[part.idx(s, lg, row)].x;
            if (ms == -INFINITY) continue;
            const float w = exp2f(ms - mx);
            const float4 v = *reinterpret_cast<const float4*>(part.o + part.idx(s, lg, row) * D + d);
            a.x += w * v.x; a.y += w * v.y; a.z += w * v.z; a.w += w * v.w;
        }
        st(op + d + 0, a.x * inv);
        st(op + d + 1, a.y * inv);
        st(op + d + 2, a.z * inv);
        st(op + d + 3, a.w * inv);
    }
}

// ---------------------------------------------------------------------------
// Append one token per decode stream to its private tail, in every layer.
// grid (G), block 256.
template <typename T>
__global__ __launch_bounds__(256) void append_tail(T* tail_k, T* tail_v, int32_t* tail_len, const T* k_new,
                                                   const T* v_new, int n_layers, int n_streams, int cap,
                                                   int tok_elems, uint32_t* overflow) {
    const int strm = blockIdx.x;
    const int n = tail_len[strm];
    const bool ok = n >= 0 && n < cap;
    if (ok) {
        for (int lb = 0; lb < n_layers; ++lb) {
            const long long src = ((long long)lb * n_streams + strm) * tok_elems;
            const long long dst = (((long long)lb * n_streams + strm) * cap + n) * tok_elems;
            for (int e = threadIdx.x; e < tok_elems; e += blockDim.x) {
                tail_k[dst + e] = k_new[src + e];
                tail_v[dst + e] = v_new[src + e];
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        if (ok)
            tail_len[strm] = n + 1;
        else if (overflow)
            atomicOr(overflow, 1u << (strm & 31));
    }
}

// ================================================================ host side ==

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

struct Plan {
    int group, m_rows, mpad, lg_count, total, chunk, parts, max_parts;
    bool mfma;
};

static int valu_row_blocks(int m) { return (m + VALU_ROWS - 1) / VALU_ROWS; }

// Choose the split count: enough workgroups for two per CU on 256 CUs, but
// no split shorter than 128 keys.
static int default_splits(int lg_count, int row_blocks, int max_keys) {
    const int base = lg_count * row_blocks;
    int s = (512 + base - 1) / base;
    int by_len = max_keys / 128;
    if (by_len < 1) by_len = 1;
    if (s > by_len) s = by_len;
    if (s > 64) s = 64;
    return s < 1 ? 1 : s;
}

static size_t partial_bytes(const Plan& p, int d) {
    const size_t o = align_up((size_t)p.max_parts * p.lg_count * p.mpad * d * sizeof(float), 256);
    const size_t ml = align_up((size_t)p.max_parts * p.lg_count * p.mpad * sizeof(float2), 256);
    return o + ml;
}

static Partials partials_in(void* ws, const Plan& p, int d) {
    Partials part;
    part.o = static_cast<float*>(ws);
    part.ml = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                        align_up((size_t)p.max_parts * p.lg_count * p.mpad * d * sizeof(float), 256));
    part.mpad = p.mpad;
    part.lg_count = p.lg_count;
    return part;
}

// `extra` is the number of extra partial slots after the cached-key splits.
static pa_status plan_for(const Ring* r, int layer_begin, int num_layers, int hq, int n_rows_tokens, int n_dyn,
                          int req_splits, int extra, Plan* p) {
    const rb_config& c = r->cfg;
    PA_CHECK_ARG(num_layers >= 1 && layer_begin >= 0 && layer_begin + num_layers <= c.num_layers, PA_ESHAPE,
                 "layers [%d, %d) outside the ring's %d layers", layer_begin, layer_begin + num_layers, c.num_layers);
    PA_CHECK_ARG(hq >= 1 && hq % c.num_kv_heads == 0, PA_ESHAPE, "n_q_heads %d is not a multiple of num_kv_heads %d",
                 hq, c.num_kv_heads);
    PA_CHECK_ARG(n_rows_tokens >= 1, PA_ESHAPE, "need at least one query token");
    PA_CHECK_ARG(req_splits >= 0 && req_splits <= 256, PA_EINVAL, "num_splits %d not in [0, 256]", req_splits);
    p->mfma = c.dtype == PA_BF16;
    if (p->mfma)
        PA_CHECK_ARG(c.head_dim == 64 || c.head_dim == 128 || c.head_dim == 256, PA_ESHAPE,
                     "bf16 attention supports head_dim 64, 128 or 256 (got %d)", c.head_dim);
    p->group = hq / c.num_kv_heads;
    p->m_rows = n_rows_tokens * p->group;
    p->lg_count = num_layers * c.num_kv_heads;
    const int row_blocks = p->mfma ? (p->m_rows + ROWS_PER_WG - 1) / ROWS_PER_WG : valu_row_blocks(p->m_rows);
    p->mpad = (p->m_rows + 31) / 32 * 32;
    const int max_keys = (int)(r->seq_len() + n_dyn);
    const int s_max = req_splits ? req_splits : default_splits(p->lg_count, row_blocks, max_keys);
    p->max_parts = s_max + extra;
    p->total = r->cached_tokens() + n_dyn;
    if (p->total > 0) {
        int chunk = (p->total + s_max - 1) / s_max;
        chunk = (chunk + KT - 1) / KT * KT;
        p->chunk = chunk;
        p->parts = (p->total + chunk - 1) / chunk;
    } else {
        p->chunk = KT;
        p->parts = 0;
    }
    return PA_OK;
}

static KvSource source_for(const Ring* r, int layer_begin, const void* k_dyn, const void* v_dyn, int n_dyn) {
    KvSource s;
    const long long le = r->layer_elems();
    const int eb = (int)r->elem_bytes();
    s.ring_k = static_cast<const char*>(r->k) + (long long)layer_begin * le * eb;
    s.ring_v = static_cast<const char*>(r->v) + (long long)layer_begin * le * eb;
    s.ring_layer = le;
    s.dyn_k = k_dyn;
    s.dyn_v = v_dyn;
    s.dyn_layer = (long long)n_dyn * r->cfg.num_kv_heads * r->cfg.head_dim;
    s.pinned = r->pinned;
    s.pin_cap = r->cfg.pin_capacity;
    s.n_slide = r->count * r->cfg.tokens_per_frame;
    s.n_dyn = n_dyn;
    s.hkv = r->cfg.num_kv_heads;
    s.d = r->cfg.head_dim;
    return s;
}

static pa_status launch_partials(const Ring* r, const Plan& p, const void* q, long long q_layer, int hq,
                                 const KvSource& src, float scale, const Partials& part, hipStream_t stream) {
    if (p.parts == 0) return PA_OK;
    const float scale_log2 = scale * 1.4426950408889634f;
    const int d = r->cfg.head_dim;
    if (p.mfma) {
        dim3 grid(p.parts, (p.m_rows + ROWS_PER_WG - 1) / ROWS_PER_WG, p.lg_count);
        const uint16_t* qq = static_cast<const uint16_t*>(q);
        if (d == 256)
            partial_mfma<256><<<grid, MFMA_WAVES * 64, 0, stream>>>(qq, q_layer, hq, p.group, p.m_rows, src, p.chunk, scale_log2, part);
        else if (d == 128)
            partial_mfma<128><<<grid, MFMA_WAVES * 64, 0, stream>>>(qq, q_layer, hq, p.group, p.m_rows, src, p.chunk, scale_log2, part);
        else
            partial_mfma<64><<<grid, MFMA_WAVES * 64, 0, stream>>>(qq, q_layer, hq, p.group, p.m_rows, src, p.chunk, scale_log2, part);
    } else {
        dim3 grid(p.parts, valu_row_blocks(p.m_rows), p.lg_count);
        partial_valu<float><<<grid, 256, VALU_ROWS * d * sizeof(float), stream>>>(
            static_cast<const float*>(q), q_layer, hq, p.group, p.m_rows, src, p.chunk, scale_log2, part);
    }
    PA_LAUNCHED();
    return PA_OK;
}

static pa_status launch_combine(const Ring* r, const Plan& p, int n_parts, int hq, long long out_layer, void* out,
                                int out_dtype, const Partials& part, hipStream_t stream) {
    dim3 grid(valu_row_blocks(p.m_rows), p.lg_count);
    const int d = r->cfg.head_dim, hkv = r->cfg.num_kv_heads;
    if (out_dtype == PA_F32)
        combine<float><<<grid, 256, 0, stream>>>(part, n_parts, p.m_rows, p.group, hq, hkv, d, out_layer,
                                                 static_cast<float*>(out));
    else
        combine<uint16_t><<<grid, 256, 0, stream>>>(part, n_parts, p.m_rows, p.group, hq, hkv, d, out_layer,
                                                    static_cast<uint16_t*>(out));
    PA_LAUNCHED();
    return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" size_t pattn_workspace_bytes(const rb_ring* ring, const pattn_args* a) {
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    if (!r || !a) return 0;
    Plan p;
    if (plan_for(r, a->layer_begin, a->num_layers, a->n_q_heads, a->n_dyn, a->n_dyn, a->num_splits, 0, &p) != PA_OK)
        return 0;
    return partial_bytes(p, r->cfg.head_dim);
}

static pa_status step_impl(const rb_ring* ring, const pattn_args* a, const void* q, const void* k_dyn,
                           const void* v_dyn, void* out, void* ws, size_t ws_bytes, void* stream, void* ev_begin,
                           void* ev_end) {
    clear_error();
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    PA_CHECK_ARG(r && a && q && k_dyn && v_dyn && out && ws, PA_EINVAL, "pattn_step: null argument");
    PA_CHECK_ARG(aligned16(q) && aligned16(k_dyn) && aligned16(v_dyn) && aligned16(out) && aligned16(ws) &&
                     aligned16(r->k) && aligned16(r->v),
                 PA_EINVAL, "pattn_step: every buffer must be 16-byte aligned");
    PA_CHECK_ARG(a->out_dtype == PA_F32 || a->out_dtype == PA_BF16, PA_EINVAL, "pattn_step: bad out_dtype");
    PA_CHECK_ARG(a->scale > 0.f && a->scale < 1e30f, PA_EINVAL, "pattn_step: scale must be positive and finite");
    PA_CHECK_ARG(a->n_dyn >= 1, PA_ESHAPE, "pattn_step: n_dyn must be >= 1");
    Plan p;
    pa_status st = plan_for(r, a->layer_begin, a->num_layers, a->n_q_heads, a->n_dyn, a->n_dyn, a->num_splits, 0, &p);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(!(r->cfg.pin_capacity > 0 && r->pinned == 0), PA_ESTATE,
                 "pattn_step: the prefix is not pinned yet (rb_pin_prefix first)");
    const size_t need = partial_bytes(p, r->cfg.head_dim);
    PA_CHECK_ARG(ws_bytes >= need, PA_ERANGE, "pattn_step: workspace %zu bytes < %zu needed", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const KvSource src = source_for(r, a->layer_begin, k_dyn, v_dyn, a->n_dyn);
    const Partials part = partials_in(ws, p, r->cfg.head_dim);
    const long long q_layer = (long long)a->n_dyn * a->n_q_heads * r->cfg.head_dim;
    if (ev_begin) PA_HIP(hipEventRecord(static_cast<hipEvent_t>(ev_begin), s));
    st = launch_partials(r, p, q, q_layer, a->n_q_heads, src, a->scale, part, s);
    if (st != PA_OK) return st;
    if (ev_end) PA_HIP(hipEventRecord(static_cast<hipEvent_t>(ev_end), s));
    return launch_combine(r, p, p.parts, a->n_q_heads, q_layer, out, a->out_dtype, part, s);
}

extern "C" pa_status pattn_step(const rb_ring* ring, const pattn_args* a, const void* q, const void* k_dyn,
                                const void* v_dyn, void* out, void* ws, size_t ws_bytes, void* stream) {
    return step_impl(ring, a, q, k_dyn, v_dyn, out, ws, ws_bytes, stream, nullptr, nullptr);
}

extern "C" pa_status pattn_step_timed(const rb_ring* ring, const pattn_args* a, const void* q, const void* k_dyn,
                                      const void* v_dyn, void* out, void* ws, size_t ws_bytes, void* stream,
                                      void* ev_begin, void* ev_end) {
    return step_impl(ring, a, q, k_dyn, v_dyn, out, ws, ws_bytes, stream, ev_begin, ev_end);
}

// ------------------------------------------------------------ decode readers --

static pa_status check_decode(const Ring* r, const pattn_decode_args* a) {
    PA_CHECK_ARG(r && a, PA_EINVAL, "decode: null argument");
    PA_CHECK_ARG(a->n_streams >= 1 && a->tail_capacity >= 1, PA_ESHAPE, "decode: n_streams and tail_capacity must be >= 1");
    PA_CHECK_ARG(a->out_dtype == PA_F32 || a->out_dtype == PA_BF16, PA_EINVAL, "decode: bad out_dtype");
    PA_CHECK_ARG(a->scale > 0.f && a->scale < 1e30f, PA_EINVAL, "decode: scale must be positive and finite");
    PA_CHECK_ARG(a->num_layers >= 1 && a->layer_begin >= 0 && a->layer_begin + a->num_layers <= r->cfg.num_layers,
                 PA_ESHAPE, "decode: layer range outside the ring");
    return PA_OK;
}

extern "C" pa_status pattn_append_private(const rb_ring* ring, const pattn_decode_args* a, void* tail_k, void* tail_v,
                                          int32_t* tail_len, const void* k_new, const void* v_new,
                                          uint32_t* overflow, void* stream) {
    clear_error();
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    pa_status st = check_decode(r, a);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(tail_k && tail_v && tail_len && k_new && v_new, PA_EINVAL, "pattn_append_private: null argument");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int tok = r->cfg.num_kv_heads * r->cfg.head_dim;
    if (r->cfg.dtype == PA_F32)
        append_tail<float><<<a->n_streams, 256, 0, s>>>(static_cast<float*>(tail_k), static_cast<float*>(tail_v), tail_len,
                                                        static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                                                        a->num_layers, a->n_streams, a->tail_capacity, tok, overflow);
    else
        append_tail<uint16_t><<<a->n_streams, 256, 0, s>>>(
            static_cast<uint16_t*>(tail_k), static_cast<uint16_t*>(tail_v), tail_len, static_cast<const uint16_t*>(k_new),
            static_cast<const uint16_t*>(v_new), a->num_layers, a->n_streams, a->tail_capacity, tok, overflow);
    PA_LAUNCHED();
    return PA_OK;
}

extern "C" size_t pattn_decode_workspace_bytes(const rb_ring* ring, const pattn_decode_args* a) {
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    if (check_decode(r, a) != PA_OK) return 0;
    Plan p;
    if (plan_for(r, a->layer_begin, a->num_layers, a->n_q_heads, a->n_streams, 0, a->num_splits, 1, &p) != PA_OK) return 0;
    return partial_bytes(p, r->cfg.head_dim);
}

extern "C" pa_status pattn_decode(const rb_ring* ring, const pattn_decode_args* a, const void* q, const void* tail_k,
                                  const void* tail_v, const int32_t* tail_len, void* out, void* ws, size_t ws_bytes,
                                  void* stream) {
    clear_error();
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    pa_status st = check_decode(r, a);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(q && tail_k && tail_v && tail_len && out && ws, PA_EINVAL, "pattn_decode: null argument");
    PA_CHECK_ARG(aligned16(q) && aligned16(out) && aligned16(ws) && aligned16(r->k) && aligned16(r->v), PA_EINVAL,
                 "pattn_decode: buffers must be 16-byte aligned");
    Plan p;
    st = plan_for(r, a->layer_begin, a->num_layers, a->n_q_heads, a->n_streams, 0, a->num_splits, 1, &p);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(!(r->cfg.pin_capacity > 0 && r->pinned == 0), PA_ESTATE, "pattn_decode: the prefix is not pinned yet");
    const size_t need = partial_bytes(p, r->cfg.head_dim);
    PA_CHECK_ARG(ws_bytes >= need, PA_ERANGE, "pattn_decode: workspace %zu bytes < %zu needed", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const KvSource src = source_for(r, a->layer_begin, nullptr, nullptr, 0);
    const Partials part = partials_in(ws, p, r->cfg.head_dim);
    const int d = r->cfg.head_dim, hkv = r->cfg.num_kv_heads;
    const long long q_layer = (long long)a->n_streams * a->n_q_heads * d;
    st = launch_partials(r, p, q, q_layer, a->n_q_heads, src, a->scale, part, s);
    if (st != PA_OK) return st;
    const float scale_log2 = a->scale * 1.4426950408889634f;
    dim3 grid(valu_row_blocks(p.m_rows), p.lg_count);
    if (r->cfg.dtype == PA_F32)
        partial_tail<float><<<grid, 256, VALU_ROWS * d * sizeof(float), s>>>(
            static_cast<const float*>(q), q_layer, a->n_q_heads, p.group, p.m_rows, static_cast<const float*>(tail_k),
            static_cast<const float*>(tail_v), tail_len, a->n_streams, a->tail_capacity, hkv, d, scale_log2, p.parts, part);
    else
        partial_tail<uint16_t><<<grid, 256, VALU_ROWS * d * sizeof(float), s>>>(
            static_cast<const uint16_t*>(q), q_layer, a->n_q_heads, p.group, p.m_rows,
            static_cast<const uint16_t*>(tail_k), static_cast<const uint16_t*>(tail_v), tail_len, a->n_streams,
            a->tail_capacity, hkv, d, scale_log2, p.parts, part);
    PA_LAUNCHED();
    return launch_combine(r, p, p.parts + 1, a->n_q_heads, q_layer, out, a->out_dtype, part, s);
}
