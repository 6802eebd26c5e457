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

#include <mutex>
#include <type_traits>

#include "gemm.h"

namespace pa {

constexpr int KT = 32;           // key granularity of splits, keys per LDS tile
constexpr int MFMA_WAVES = 8;    // waves per workgroup: two per SIMD, 32 query rows each
constexpr int MFMA_OCC = 1;      // workgroups per CU
constexpr int NBUF = 2;          // K/V tile buffers in the LDS ring: NBUF - 1 tiles in flight
constexpr int N_XCD = 8;         // accelerator complex dies, one L2 each
constexpr int ROWS_PER_WG = MFMA_WAVES * 32;
constexpr float RESCALE_SLACK = 8.f;   // log2 units the running max may lag the true max
constexpr int VALU_ROWS = 4;     // query rows per workgroup of the vector kernels
// Launch shapes of the matrix-core partial kernel. The throughput form is 8
// waves over 256 query rows. A launch that would leave CUs idle with it (a
// single layer) runs 128-row workgroups instead, more of them, if they still
// fit the chip at once (at most HALVES_MAX_WGS): with splits of at least
// HALVES_MIN_TILES tiles, 8 waves as four row blocks x two key halves, each
// half walking every other tile, merged through LDS; with shorter splits (in
// launches of at most NARROW_MAX_WGS 256-row workgroups), 4 waves, one per
// SIMD, since with one tile per wave the merge would cost more than the tile
// it saves. The halves pay only through the extra workgroups: on a grid of
// the same size (the 128 rows of the decode readers) the merge made the
// launch slower.
constexpr int HALVES_MIN_TILES = 4;
constexpr int HALVES_MAX_WGS = 256;
constexpr int NARROW_MAX_WGS = 64;

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
__device__ __forceinline__ void stp(float* p, float v) { *p = v; }
__device__ __forceinline__ void stp(uint16_t* p, float v) { *p = f2bf(v); }
// two floats -> two bf16 (round to nearest even), first in the low half
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// Split partials in the workspace. (m, l) per row in FP32; the unnormalised
// accumulator O in MFMA-fragment order, so that a wave's accumulator tile is
// stored and reloaded with fully contiguous accesses. O is FP32 for f32 rings
// and bf16 for bf16 rings (whose products already round P to bf16; the extra
// rounding of O is of the same relative size, 2^-9):
//   O[part][lg][row / 32][d / 32][j][lane][e],  lane = row % 32 + 32 hi,
//   (d % 32) = 8 j + 4 hi + e   (j < 4, hi < 2, e < 4)
// which is the C/D register layout of v_mfma_f32_32x32x16 for O^T.
struct Partials {
    void* o;         // float (f32 rings) or bf16 bits (bf16 rings)
    float2* ml;      // [parts][lg][mpad]   (m, l)
    int mpad;        // rows padded to a multiple of 32
    int lg_count;    // call-layers x KV heads
    int d;           // head dim
    __device__ __forceinline__ long long idx(int part, int lg, int row) const {
        return ((long long)part * lg_count + lg) * mpad + row;
    }
    template <typename PO> __device__ __forceinline__ PO* optr() const { return static_cast<PO*>(o); }
    // first element of the 32-row block holding `row`
    __device__ __forceinline__ long long oblock(int part, int lg, int row) const {
        return (((long long)part * lg_count + lg) * mpad + (row & ~31)) * d;
    }
    // element offset of (row, dim) within that block
    __device__ __forceinline__ int oelem(int row, int dim) const {
        const int dd = dim & 31;
        return (((dim >> 5) * 4 + (dd >> 3)) * 64 + (row & 31) + 32 * ((dd >> 2) & 1)) * 4 + (dd & 3);
    }
};

// ---------------------------------------------------------------------------
// Vector (VALU) attention of one query row per wave over keys [k_begin,
// k_end), FP32 arithmetic. Keys go 64 at a time, lane j scoring key j:
// its K row is read with 16-byte loads, all of a group in flight at once.
// For O += P V, lane i owns dims 4i .. 4i + 3, and the rows of eight keys are
// loaded before any is used. `row_of(j, v)` gives key j's K (v = false) or V
// (v = true) row. Updates the running (m, l, O) in base-2 units.
template <typename T> __device__ __forceinline__ float4 ld4f(const T* p);
template <> __device__ __forceinline__ float4 ld4f<float>(const float* p) { return *reinterpret_cast<const float4*>(p); }
template <> __device__ __forceinline__ float4 ld4f<uint16_t>(const uint16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                       __uint_as_float(u.y & 0xffff0000u));
}

template <typename T, int D, typename RowOf>
__device__ __forceinline__ void valu_row(const float* qrow, int k_begin, int k_end, float scale_log2, RowOf row_of,
                                         float& m, float& l, float4& o) {
    constexpr int EG = D < 64 ? D : 64;           // K elements per group of loads in flight
    const int lane = threadIdx.x & 63;
    for (int base = k_begin; base < k_end; base += 64) {
        const int j = base + lane;
        const bool jv = j < k_end;
        const T* kp = row_of(jv ? j : k_end - 1, false);
        float z = 0.f;
#pragma unroll 1
        for (int g0 = 0; g0 < D; g0 += EG) {
            float4 kv[EG / 4];
#pragma unroll
            for (int i = 0; i < EG / 4; ++i) kv[i] = ld4f<T>(kp + g0 + 4 * i);
            // the group's loads all leave before the first is used (the
            // scheduler would otherwise reuse one register: one load in flight)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < EG / 4; ++i) {
                const float4 qq = *reinterpret_cast<const float4*>(qrow + g0 + 4 * i);
                z = fmaf(qq.x, kv[i].x, z);
                z = fmaf(qq.y, kv[i].y, z);
                z = fmaf(qq.z, kv[i].z, z);
                z = fmaf(qq.w, kv[i].w, z);
            }
        }
        const float sc = jv ? z * scale_log2 : -INFINITY;
        const float mn = fmaxf(m, wave_max(sc));      // finite: base < k_end
        const float alpha = exp2f(m - mn);
        const float p = jv ? exp2f(sc - mn) : 0.f;
        l = l * alpha + wave_sum(p);
        o.x *= alpha; o.y *= alpha; o.z *= alpha; o.w *= alpha;
        const int nvalid = min(64, k_end - base);
        for (int j0 = 0; j0 < nvalid; j0 += 8) {
            float4 v[8];
            float pj[8];
            // lanes past D / 4 re-read the row's first four elements (no
            // branch around the loads) and are zeroed below
            const int dl = 4 * lane < D ? 4 * lane : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int jj = j0 + u;                      // < 64; p is 0 past nvalid
                pj[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), jj));
                const T* vp = row_of(base + min(jj, nvalid - 1), true);
                v[u] = ld4f<T>(vp + dl);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (4 * lane >= D)
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                o.x = fmaf(pj[u], v[u].x, o.x); o.y = fmaf(pj[u], v[u].y, o.y);
                o.z = fmaf(pj[u], v[u].z, o.z); o.w = fmaf(pj[u], v[u].w, o.w);
            }
        }
        m = mn;
    }
}

// Store one row's partial: O (lane i: dims 4i .. 4i + 3) and (m, l).
template <typename PO>
__device__ __forceinline__ void store_row_partial(const Partials& part, int slot, int lg, int row, int D, float m,
                                                  float l, float4 o) {
    const int lane = threadIdx.x & 63;
    PO* op = part.optr<PO>() + part.oblock(slot, lg, row);
    if (4 * lane < D) {
        const int d = 4 * lane;
        stp(op + part.oelem(row, d), o.x);
        stp(op + part.oelem(row, d + 1), o.y);
        stp(op + part.oelem(row, d + 2), o.z);
        stp(op + part.oelem(row, d + 3), o.w);
    }
    if (lane == 0) part.ml[part.idx(slot, lg, row)] = make_float2(m, l);
}

// Vector partial for f32 rings (parity held to 1e-5 absolute): one wave per
// query row of one split.
// grid (splits, ceil(M / 4), Lb * Hkv), block 256.
template <int D>
__global__ __launch_bounds__(256) void partial_valu(const float* q, long long q_layer, int hq, int group, int m_rows,
                                                    KvSource src, int chunk, float scale_log2, Partials part) {
    __shared__ __attribute__((aligned(16))) float qs[VALU_ROWS][D];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int split = blockIdx.x, lg = blockIdx.z;
    const int lb = lg / src.hkv, g = lg % src.hkv;
    const int row = blockIdx.y * VALU_ROWS + wave;
    const bool row_ok = row < m_rows;
    const int tok = row / group, head = g * group + row % group;
    for (int d = lane; d < D; d += 64) qs[wave][d] = row_ok ? q[lb * q_layer + ((long long)tok * hq + head) * D + d] : 0.f;
    __syncthreads();
    const int k_begin = split * chunk, k_end = min(k_begin + chunk, src.total());
    const float* rk = static_cast<const float*>(src.ring_k);
    const float* rv = static_cast<const float*>(src.ring_v);
    const float* dk = static_cast<const float*>(src.dyn_k);
    const float* dv = static_cast<const float*>(src.dyn_v);
    KvSource sr = src;
    sr.skip_at = src.window_skip();
    auto row_of = [&](int j, bool v) -> const float* {
        bool dyn;
        const long long off = sr.offset(lb, g, j, dyn);
        return (dyn ? (v ? dv : dk) : (v ? rv : rk)) + off;
    };
    float m = -INFINITY, l = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    valu_row<float, D>(qs[wave], k_begin, k_end, scale_log2, row_of, m, l, o);
    if (row_ok) store_row_partial<float>(part, split, lg, row, D, m, l, o);
}

// ---------------------------------------------------------------------------
// bf16 MFMA partial. Each wave owns 32 query rows; the workgroup streams the
// split's keys through LDS in tiles of KT keys and every wave computes
//     S^T (KT x 32)  = K_tile (KT x D) . Q^T (D x 32)        v_mfma_f32_32x32x16_bf16
//     O^T (D x 32)  += V_tile^T (D x KT) . P^T (KT x 32)
// In the transposed form each lane holds one query row's scores, so the
// softmax statistics are per lane plus one swap with lane ^ 32, and P feeds
// the second product straight from registers. The K rows fed to the first
// product are permuted (bits 2 and 3 of the row index swapped) so that after
// it every lane holds 8 consecutive keys per 16-key step: exactly the
// B-operand layout of the second product.
//
// MFMA 32x32x16 operand layout (64 lanes, l32 = lane % 32, hi = lane / 32):
//   A[m][k]: lane holds m = l32, k = 8 hi .. 8 hi + 7
//   B[k][n]: lane holds n = l32, k = 8 hi .. 8 hi + 7
//   C[m][n]: lane holds n = l32, m = 8 (r / 4) + 4 hi + r % 4, r = 0 .. 15
//
// Data movement (gfx950):
// * tiles go global -> LDS by direct-to-LDS loads (global_load_lds, 16 bytes
//   per lane, lane i landing at base + 16 i), double-buffered: the next
//   tile's loads are in flight while the current tile is multiplied, and
//   they cost no registers;
// * K and V stay token-major, as the ring stores them. A tile is kept in
//   "planes" of 32 dims: plane p holds dims [32p, 32p + 32) of all KT keys,
//   64 bytes per key. In a K plane the four 16-byte chunks of key r are
//   rotated by XOR with (r / 4) % 4, which makes the A-operand reads of 16
//   different keys hit 16 different bank groups;
// * V^T operands come from ds_read_b64_tr_b16. Within 16 lanes, lane i
//   addresses 4 dims of one key (key R + i / 4, dims D0 + 4 (i % 4)); the
//   transposed read hands lane l the 4 keys R .. R + 3 of dim D0 + l, i.e.
//   the A operand of O^T = V^T P^T, straight from the token-major tile.
// Waves whose 32 rows are all padding skip the arithmetic but still load.
//
// grid: 1-D, ceil(layers x KV heads x splits / 8) x 8 x row blocks workgroups of 256 threads.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

// Per-wave arithmetic on one LDS tile of KT = 32 keys for the wave's 32
// query rows:
//   qk_scores:    S^T = K_tile . Q^T       (16 MFMAs, K from LDS)
//   softmax_tile: online softmax of S -> P (VALU)
//   pv_tile:      O^T += V^T P^T           (16 MFMAs, V from LDS)
template <int D>
__device__ __forceinline__ f32x16 qk_scores(const char* kb, int koff0, int koff1, const bf16x8 (&qf)[D / 16]) {
    constexpr int KD = D / 16, PLANE = KT * 64;
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + (kk >> 1) * PLANE + ((kk & 1) ? koff1 : koff0));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s, 0, 0, 0);
    }
    return s;
}

// Online softmax of one tile's scores: updates the running (m, l), rescales
// O when the reference max moves, and returns P in bf16 in the B-operand
// layout of the PV product.
// With FUSED, rows differ in how many keys they see (k_lim per lane, the
// wave's smallest in k_lim_wave): a row can have every key of a tile masked
// while its running max is still -inf, which the rescale and the exponent
// must then treat as "nothing yet" instead of producing NaN.
template <int D, bool FUSED = false>
__device__ __forceinline__ void softmax_tile(f32x16 s, int base, int k_end, int hi, float scale_log2,
                                             f32x16 (&acc)[D / 32], float& m_run, float& l_run, bf16x8 (&pf)[2],
                                             int k_lim_wave = 0) {
    constexpr int DB = D / 32;
    // Row max on the raw scores (scale > 0 keeps the order); keys past the
    // split's end exist only in its last tile and are masked there alone.
    float rmax = -INFINITY;
    if (base + KT <= (FUSED ? k_lim_wave : k_end)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) rmax = fmaxf(rmax, s[r]);
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = base + 16 * (r >> 3) + 8 * hi + (r & 7);
            s[r] = key < k_end ? s[r] : -INFINITY;
            rmax = fmaxf(rmax, s[r]);
        }
    }
    float tmax = rmax * scale_log2;
    {   // the other half of the row's keys sits in lane ^ 32: swap the wave's halves
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // Lazy rescale: keep the reference max unless some row's max got more than
    // RESCALE_SLACK above it. Exact (numerator and denominator share the
    // reference); probabilities stay below 2^RESCALE_SLACK.
    if (__any(tmax > m_run + RESCALE_SLACK)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = FUSED && m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        // a row whose reference is still -inf has accumulated nothing (O = 0):
        // on a wave's first tile the 128 accumulator products are skipped
        if (!__all(m_run == -INFINITY)) {
#pragma unroll
            for (int b = 0; b < DB; ++b) acc[b] *= alpha;
        }
        m_run = m_new;
    }
    // p = 2^(scale log2e s - m): one FMA and the hardware exp2 (v_exp_f32);
    // results below 2^-126 flush to zero, far below what a bf16 P can carry.
    const float m_e = FUSED ? fmaxf(m_run, -3.0e38f) : m_run;   // a row with nothing yet: p = 0
#pragma unroll
    for (int r = 0; r < 16; ++r) pf[r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -m_e));
    // The row sum is taken over the rounded P that the P.V product uses, two
    // values per instruction (a bf16 dot product against (1, 1), FP32 sum),
    // in two chains.
    const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[0][2 * i], pf[0][2 * i + 1]}, one, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[1][2 * i], pf[1][2 * i + 1]}, one, ps1, false);
    }
    l_run += ps0 + ps1;
}

// O^T += V^T P^T for one tile (16 MFMAs; V^T straight from the token-major
// tile by transposed LDS reads).
template <int D>
__device__ __forceinline__ void pv_tile(const char* vb, int voff, const bf16x8 (&pf)[2], f32x16 (&acc)[D / 32]) {
    constexpr int DB = D / 32, PLANE = KT * 64;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            const char* vp = vb + b * PLANE + (16 * s2) * 64 + voff;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(vp));
            const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(vp + 4 * 64));
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[s2], acc[b], 0, 0, 0);
        }
    }
}

// One LDS tile buffer per (index, size): distinct objects, so the compiler
// can prove that loads in flight into one buffer never alias reads of another.
template <int I, int BYTES>
__device__ __forceinline__ char* lds_buffer() {
    __shared__ __attribute__((aligned(1024))) char b[BYTES];
    return b;
}

// Wait until at most N vector-memory operations of this wave are in flight
// (they complete in issue order), leaving the LDS and export counters alone.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// FUSED: rows [0, m1) are the action suffix's (queries from q, keys
// [pin | window | suffix]); rows [m1, m_rows) are decode streams' (queries
// from q2, keys [pin | window] only: the suffix keys are masked for them).
// QPK: q is already in the B-operand order of the S = K Q^T product,
// [call layer x KV head][32-row block][D / 16][64 lanes][8] (rows padded to
// whole blocks), so each Q load is 1 KB contiguous across the wave instead of
// 32 B from each of 32 rows. The stack's QKV projection writes it that way.
// WAVES: 8 (two per SIMD, the throughput form) or 4 (one per SIMD, for
// launches too small to fill the chip: each wave's key loop then runs at the
// single-wave rate).
// KH: key halves per workgroup. With KH = 2 the waves form two groups of
// WAVES / 2 over the same query rows; group h takes tiles h, h + 2, ... of
// the split, and group 1 hands its (m, l, O) to group 0 through LDS at the
// end, which merges the two and stores one partial. Each wave then walks half
// the split's tiles, two waves per SIMD, without more partials to combine.
template <int D, bool FUSED = false, bool QPK = false, int WAVES = MFMA_WAVES, bool F32P = false, int KH = 1>
__global__ __launch_bounds__(WAVES * 64, MFMA_OCC) void partial_mfma(const uint16_t* __restrict__ q,
                                                                          long long q_layer, int hq, int group,
                                                                          int m_rows, KvSource src, int chunk,
                                                                          float scale_log2, Partials part, int parts,
                                                                          int row_blocks,
                                                                          const uint16_t* __restrict__ q2 = nullptr,
                                                                          long long q2_layer = 0, int m1 = 0) {
    constexpr int KD = D / 16;               // k-steps over the head dimension
    constexpr int DB = D / 32;               // 32-wide output blocks = planes
    constexpr int PLANE = KT * 64;           // bytes per plane (KT keys x 32 dims x 2 B)
    constexpr int TILE = DB * PLANE;         // bytes per K or V tile
    constexpr int NBLK = TILE / 1024;        // 1 KB direct-to-LDS loads per tile and tensor
    constexpr int WR = WAVES / KH;                    // waves per key half, one 32-row block each
    constexpr int DPW = (NBLK + WR - 1) / WR;         // loads per wave, per tile and tensor
    constexpr int RPW = WR * 32;                      // query rows per workgroup
    static_assert(NBLK % 2 == 0 && (NBLK <= WR || NBLK % WR == 0) && WR % 2 == 0, "tile / wave split");
    static_assert(KH == 1 || (KH == 2 && !FUSED && D == 256 && WR * 32 * D * 4 <= 2 * NBUF * KH * TILE),
                  "key halves: single-reader bf16 step, exchange fits the tile buffers");

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = KH == 1 ? 0 : wave / WR;     // key half (wave-uniform)
    const int wr = KH == 1 ? wave : wave % WR;  // row block within the workgroup
    // XCD-aware placement. Workgroups go to the 8 XCDs round-robin by id, and
    // each XCD has its own L2. All row blocks of one (layer, split) read the
    // same keys, so they are given ids congruent mod 8: same XCD, same L2,
    // dispatched back to back, and the split's K/V leaves HBM once.
    const int xcd = blockIdx.x & (N_XCD - 1), slot = blockIdx.x / N_XCD;
    const int unit = (slot / row_blocks) * N_XCD + xcd;       // (layer, split) index
    if (unit >= parts * part.lg_count) return;                 // id padding, whole workgroup
    const int split = unit % parts, lg = unit / parts, rblk = slot % row_blocks;
    const int lb = lg / src.hkv, g = lg % src.hkv;
    const int row0 = rblk * RPW + wr * 32;
    const int row = row0 + l32;
    const bool active = row0 < m_rows;       // wave-uniform

    bf16x8 qf[KD];
    if (QPK) {
        static_assert(!(QPK && FUSED), "packed Q is for the single-reader step");
        const uint16_t* qp = q + ((long long)(lg * (part.mpad >> 5) + (row0 >> 5)) * KD) * 512 + lane * 8;
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) qf[kk] = active ? *reinterpret_cast<const bf16x8*>(qp + kk * 512) : bf16x8{};
    } else if (row < m_rows) {
        const bool second = FUSED && row >= m1;
        const int r = second ? row - m1 : row;
        const uint16_t* qp = (second ? q2 + lb * q2_layer : q + lb * q_layer) +
                             ((long long)(r / group) * hq + g * group + r % group) * D + 8 * hi;
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
    } else {
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) qf[kk] = bf16x8{};
    }

    const int k_begin = split * chunk, k_end = min(k_begin + chunk, src.total());
    // FUSED: this lane's key limit (decode rows stop before the suffix) and the wave's smallest
    const int k_lim = FUSED && row >= m1 ? min(k_end, src.pinned + src.n_slide) : k_end;
    int k_lim_wave = k_lim;
    if (FUSED) {
        k_lim_wave = min(k_lim_wave, __shfl_xor(k_lim_wave, 16));
        k_lim_wave = min(k_lim_wave, __shfl_xor(k_lim_wave, 8));
        k_lim_wave = min(k_lim_wave, __shfl_xor(k_lim_wave, 4));
        k_lim_wave = min(k_lim_wave, __shfl_xor(k_lim_wave, 2));
        k_lim_wave = min(k_lim_wave, __shfl_xor(k_lim_wave, 1));
        k_lim_wave = __builtin_amdgcn_readfirstlane(k_lim_wave);
    }

    // Base pointers of this (layer, KV head), hoisted so that choosing between
    // the ring and the suffix buffer is a register select, not a memory load.
    const int stride = src.hkv * D;                     // elements per token
    const uint16_t* rk = static_cast<const uint16_t*>(src.ring_k) + lb * src.ring_layer + g * D;
    const uint16_t* rv = static_cast<const uint16_t*>(src.ring_v) + lb * src.ring_layer + g * D;
    const uint16_t* dk = static_cast<const uint16_t*>(src.dyn_k) + lb * src.dyn_layer + g * D;
    const uint16_t* dv = static_cast<const uint16_t*>(src.dyn_v) + lb * src.dyn_layer + g * D;
    const int n_cached = src.pinned + src.n_slide, pinned = src.pinned, gap = src.pin_cap - src.pinned;
    const int skip_at = pinned + src.window_skip(), skip_len = src.skip_len;   // in context-key units

    // Direct-to-LDS loads: one 1 KB load = 16 keys x 64 B of one plane, lane
    // -> (key, 16-byte chunk). Wave w of a key half loads blocks w, w + WR,
    // ... of that half's tile; block b is plane b / 2, keys 16 (b % 2) .. + 15.
    // With an even wave count every block a wave loads has the same keys, so
    // one address per tile serves.
    const int dma_key = lane >> 2, dma_pos = lane & 3;
    const int kq = wr & 1;
    const int key_in_tile = kq * 16 + dma_key;
    const int kchunk = (dma_pos ^ ((key_in_tile >> 2) & 3)) << 3;   // K plane rotation
    // this lane's element offsets inside a tile whose keys are consecutive tokens
    const int lane_k = key_in_tile * stride + (wr >> 1) * 32 + kchunk;
    const int lane_v = key_in_tile * stride + (wr >> 1) * 32 + (dma_pos << 3);
    auto issue_tile = [&](int t, char* kbuf, char* vbuf) {
        if (DPW * WR > NBLK && wr >= NBLK) return;                     // fewer blocks than waves
        const int j0 = k_begin + t * KT;                               // the tile's first key (uniform)
        const uint16_t* kp;
        const uint16_t* vp;
        // A tile inside one region (pin, a window run, or the suffix) and
        // inside the split maps to KT consecutive tokens: one scalar base
        // address plus this lane's fixed offset (scalar work instead of
        // per-lane vector work). Otherwise (the ragged tail, a tile across a
        // region boundary) each lane maps its own key.
        const bool in_pin = j0 + KT <= pinned;
        const bool in_win = j0 >= pinned && j0 + KT <= n_cached && (j0 + KT <= skip_at || j0 >= skip_at);
        const bool in_dyn = j0 >= n_cached;
        if (j0 + KT <= k_end && (in_pin || in_win || in_dyn)) {
            const int tok0 = in_dyn ? j0 - n_cached : (in_pin ? j0 : j0 + gap + (j0 >= skip_at ? skip_len : 0));
            const long long base = (long long)tok0 * stride;
            kp = (in_dyn ? dk : rk) + base + lane_k;
            vp = (in_dyn ? dv : rv) + base + lane_v;
        } else {
            const int j = min(j0 + key_in_tile, k_end - 1);            // ragged tail: a valid key, masked later
            const bool dyn = j >= n_cached;
            const int tok = dyn ? j - n_cached : (j < pinned ? j : j + gap + (j >= skip_at ? skip_len : 0));
            const int off = tok * stride + (wr >> 1) * 32;
            kp = (dyn ? dk : rk) + off + kchunk;
            vp = (dyn ? dv : rv) + off + (dma_pos << 3);
        }
#pragma unroll
        for (int i = 0; i < DPW; ++i) {
            const int blk = __builtin_amdgcn_readfirstlane(wr + i * WR);
            __builtin_amdgcn_global_load_lds((const GLB_AS void*)(kp + i * (WR / 2) * 32),
                                             (LDS_AS void*)(kbuf + blk * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const GLB_AS void*)(vp + i * (WR / 2) * 32),
                                             (LDS_AS void*)(vbuf + blk * 1024), 16, 0, 0);
        }
    };

    // per-lane LDS read offsets (key rows within a 32-key block)
    const int prow = (l32 & ~0xC) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
    const int koff0 = prow * 64 + (((0 + hi) ^ ((prow >> 2) & 3)) << 4);
    const int koff1 = prow * 64 + (((2 + hi) ^ ((prow >> 2) & 3)) << 4);
    const int gi = lane >> 4, li = lane & 15;
    const int voff = (8 * (gi >> 1) + (li >> 2)) * 64 + ((2 * (gi & 1) + ((li & 3) >> 1)) << 4) + ((li & 1) << 3);

    f32x16 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    const int n_tiles = (k_end - k_begin + KT - 1) / KT;
    // Key half kh walks the split's tiles kh, kh + KH, ...: n_mine of them,
    // in n_steps steps, the same count for every wave of the workgroup (the
    // barriers below are met by all of them).
    const int n_steps = (n_tiles + KH - 1) / KH;
    const int n_mine = (n_tiles - kh + KH - 1) / KH;
    // this half's region of each tile buffer
    const int hoff = kh * TILE;
    // Step through local tile t held in ring buffer J: wait for its loads,
    // meet at the barrier (which also frees buffer J - 1 for reuse), refill
    // that buffer with local tile t + NBUF - 1, then S = K Q^T, softmax, O += V P.
    auto step = [&](auto J_, int t) {
        constexpr int J = decltype(J_)::value;
        constexpr int JN = (J + NBUF - 1) % NBUF;
        if (t >= n_steps) return;
        wait_vmem<0>();    // with two buffers no later tile of this wave is in flight yet
        __syncthreads();
        if (t + NBUF - 1 < n_mine)
            issue_tile((t + NBUF - 1) * KH + kh, lds_buffer<JN, KH * TILE>() + hoff,
                       lds_buffer<NBUF + JN, KH * TILE>() + hoff);
        if (active && t < n_mine) {
            bf16x8 pf[2];
            const f32x16 sc = qk_scores<D>(lds_buffer<J, KH * TILE>() + hoff, koff0, koff1, qf);
            softmax_tile<D, FUSED>(sc, k_begin + (t * KH + kh) * KT, k_lim, hi, scale_log2, acc, m_run, l_run, pf,
                                   k_lim_wave);
            pv_tile<D>(lds_buffer<NBUF + J, KH * TILE>() + hoff, voff, pf, acc);
        }
    };
    // One tile in flight while one is consumed: two buffers measured faster
    // than three or four (fewer loads outstanding per CU) on every launch
    // shape here.
    static_assert(NBUF == 2, "the prologue and the unrolled loop below assume two buffers");
    if (n_mine > 0) issue_tile(kh, lds_buffer<0, KH * TILE>() + hoff, lds_buffer<NBUF + 0, KH * TILE>() + hoff);
    for (int t = 0; t < n_steps; t += NBUF) {
        step(std::integral_constant<int, 0>{}, t);
        step(std::integral_constant<int, 1>{}, t + 1);
    }

    l_run += __shfl_xor(l_run, 32);
    if constexpr (KH == 2) {
        // Merge the two halves: half 1 writes its running (m, l) and its FP32
        // accumulators into the (now idle) tile buffers, half 0 rescales both
        // to the larger reference max and adds. 32 KB per wave: one whole
        // K/V buffer object per row block.
        __syncthreads();    // every wave is past its last tile
        char* xb = wr == 0 ? lds_buffer<0, KH * TILE>()
                 : wr == 1 ? lds_buffer<1, KH * TILE>()
                 : wr == 2 ? lds_buffer<NBUF, KH * TILE>() : lds_buffer<NBUF + 1, KH * TILE>();
        f32x4* xo = reinterpret_cast<f32x4*>(xb) + lane;
        float2* xml = reinterpret_cast<float2*>(lds_buffer<2 * NBUF, WR * 64 * 8>()) + wr * 64 + lane;
        if (kh == 1 && active) {
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xo[(b * 4 + j) * 64] = f32x4{acc[b][4 * j], acc[b][4 * j + 1], acc[b][4 * j + 2], acc[b][4 * j + 3]};
            *xml = make_float2(m_run, l_run);
        }
        __syncthreads();
        if (kh == 1) return;
        if (active) {
            const float2 ml1 = *xml;
            const float mm = fmaxf(m_run, ml1.x);
            const float mref = mm == -INFINITY ? 0.f : mm;     // neither half saw a key
            const float a0 = __builtin_amdgcn_exp2f(m_run - mref), a1 = __builtin_amdgcn_exp2f(ml1.x - mref);
            l_run = l_run * a0 + ml1.y * a1;
            m_run = mm;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 x = xo[(b * 4 + j) * 64];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[b][4 * j + e] = acc[b][4 * j + e] * a0 + x[e] * a1;
                }
        }
    }
    if (active) {       // whole 32-row block, fragment order: each store is contiguous across the wave
        // Non-temporal: the partials are read once, by the combine kernel,
        // which runs on other CUs (measured 1.5% faster than plain stores).
        if constexpr (F32P) {       // FP32 partial O (16 B per lane and store)
            float* op = part.optr<float>() + part.oblock(split, lg, row0) + lane * 4;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 w = {acc[b][4 * j], acc[b][4 * j + 1], acc[b][4 * j + 2], acc[b][4 * j + 3]};
                    __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(op + (b * 4 + j) * 256));
                }
        } else {                    // bf16 partial O (8 B per lane and store)
            uint16_t* op = part.optr<uint16_t>() + part.oblock(split, lg, row0) + lane * 4;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const unsigned long long w =
                        (unsigned long long)pack_bf16(acc[b][4 * j], acc[b][4 * j + 1]) |
                        ((unsigned long long)pack_bf16(acc[b][4 * j + 2], acc[b][4 * j + 3]) << 32);
                    __builtin_nontemporal_store(w, reinterpret_cast<unsigned long long*>(op + (b * 4 + j) * 256));
                }
        }
        if (hi == 0 && row < m_rows) part.ml[part.idx(split, lg, row)] = make_float2(m_run, l_run);
    }
}

// ---------------------------------------------------------------------------
// Private-tail partial of the decode readers: one wave per (stream, head)
// row over that stream's own appended tokens. Writes partial slot `slot`,
// partial row row_base + row.
// grid (ceil(M / 4), Lb * Hkv), block 256.
template <typename T, int D>
__global__ __launch_bounds__(256) void partial_tail(const T* q, long long q_layer, int hq, int group, int m_rows,
                                                    const T* tail_k, const T* tail_v, const int32_t* tail_len,
                                                    int n_streams, int cap, int hkv, float scale_log2, int slot,
                                                    Partials part, int row_base) {
    __shared__ __attribute__((aligned(16))) float qs[VALU_ROWS][D];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lg = blockIdx.y, lb = lg / hkv, g = lg % hkv;
    const int row = blockIdx.x * VALU_ROWS + wave;
    const bool row_ok = row < m_rows;
    const int strm = row_ok ? row / group : 0, head = g * group + row % group;
    for (int d = lane; d < D; d += 64)
        qs[wave][d] = row_ok ? ldf(q + lb * q_layer + ((long long)strm * hq + head) * D + d) : 0.f;
    __syncthreads();
    int n = row_ok ? tail_len[strm] : 0;
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const long long tok_base = ((long long)lb * n_streams + strm) * cap;
    auto row_of = [&](int j, bool v) -> const T* { return (v ? tail_v : tail_k) + ((tok_base + j) * hkv + g) * D; };
    float m = -INFINITY, l = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    valu_row<T, D>(qs[wave], 0, n, scale_log2, row_of, m, l, o);
    if (row_ok) store_row_partial<T>(part, slot, lg, row_base + row, D, m, l, o);
}

// Four consecutive outputs of one row: one 8-byte (bf16) or 16-byte (f32) store.
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ void st4(uint16_t* p, float4 v) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16(v.x, v.y), pack_bf16(v.z, v.w));
}

// Splits merged per batch: every load of a batch is issued before the first
// one is used, so a batch costs one memory round trip. bf16 partials are held
// as raw words until used (two registers per four values), so their batch is
// twice as long: up to 16 splits in one round trip.
template <typename PO> struct CombineRaw;
template <> struct CombineRaw<float> {
    using T = float4;
    static constexpr int BATCH = 8;
    __device__ __forceinline__ static T load(const float* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ static float4 widen(T v) { return v; }
};
template <> struct CombineRaw<uint16_t> {
    using T = uint2;
    static constexpr int BATCH = 16;
    __device__ __forceinline__ static T load(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ static float4 widen(T u) {
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
    }
};

// Merges partial rows [row_lo, row_hi); output row index row - row_lo.
// APK: the output (bf16, one layer) goes to the fragment-packed activation
// layout of the out-projection's operand (token m < 64, column head * D + d).
// A wave takes JW of the four 8-dim slices of a (32-row, 32-dim) block: 4
// (256 B contiguous per slice and split) when the launch is large, 1 when it
// would leave most CUs idle, so that the per-wave merge is a quarter as long.
// SW > 1 (many splits): the SW waves of a workgroup share one slice, wave w
// merging splits w, w + SW, ... (each set in one batch, one memory round
// trip, where one wave alone would need several in sequence); the SW
// partial merges are then merged through LDS by the first wave.
// NB: splits per batch (at most the raw type's BATCH; the launch picks the
// smallest that holds a wave's splits, so no registers sit idle).
template <typename TO, int D, typename PO, bool APK = false, int JW = 4, int SW = 1,
          int NB = CombineRaw<PO>::BATCH>
__global__ __launch_bounds__(256) void combine(Partials part, int n_parts, int row_lo, int row_hi, int group, int hq,
                                               int hkv, long long out_layer, TO* out) {
    constexpr int DB = D / 32, NJ = 4 / JW, UPB = 4 / SW;
    static_assert(JW == 1 || JW == 2 || JW == 4, "slices per wave");
    static_assert(SW == 1 || SW == 2 || SW == 4, "split waves per slice");
    static_assert(NB >= 1 && NB <= CombineRaw<PO>::BATCH, "splits per batch");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    const int sub = wave % SW;                          // this wave's share of the splits
    const int unit = blockIdx.x * UPB + wave / SW, lg = blockIdx.y;
    const int row0 = (row_lo & ~31) + (unit / (DB * NJ)) * 32, b = (unit / NJ) % DB, j0 = (unit % NJ) * JW;
    // a slice past the end (the last workgroup of an odd count) merges
    // nothing; with SW > 1 its waves still meet the others at the barrier
    const bool live = row0 < row_hi;
    if (SW == 1 && !live) return;
    const int row = row0 + l32;
    const bool ok = row >= row_lo && row < row_hi;
    const int lb = lg / hkv, g = lg % hkv;
    // Split s of this lane's row and slice: (m, l) at ml0 + s * ml_stride,
    // the O words at o0 + s * o_stride (rows of padded blocks are in bounds).
    const long long ml_stride = (long long)part.lg_count * part.mpad, o_stride = ml_stride * part.d;
    const float2* ml0 = part.ml + part.idx(0, lg, row);
    const PO* o0 = part.optr<PO>() + part.oblock(0, lg, row0) + (b * 4 + j0) * 256 + lane * 4;
    // Online merge over batches of splits: (mx, lsum, acc) is the merge of
    // the splits seen so far, referenced to mx.
    float mx = -INFINITY, lsum = 0.f;
    float4 acc[JW];
#pragma unroll
    for (int j = 0; j < JW; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    using R = CombineRaw<PO>;
    const int n_mine = live ? (n_parts - sub + SW - 1) / SW : 0;   // splits sub, sub + SW, ...
    for (int s0 = 0; s0 < n_mine; s0 += NB) {
        // Every load of the batch is issued, in order: the (m, l) of all
        // slots, then their O words, so the merge of slot i waits only for
        // its own words. A slot past the end re-reads the batch's first
        // split (in bounds, cached) and weighs 0.
        float2 ml[NB];
        typename R::T v[NB][JW];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int s = (s0 + i < n_mine ? s0 + i : s0) * SW + sub;
            ml[i] = ml0[s * ml_stride];
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int s = (s0 + i < n_mine ? s0 + i : s0) * SW + sub;
#pragma unroll
            for (int j = 0; j < JW; ++j) v[i][j] = R::load(o0 + s * o_stride + j * 256);
        }
        // all of the batch's loads leave before any merging starts (the
        // scheduler would otherwise hold some back to save registers)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (!ok || s0 + i >= n_mine) ml[i] = make_float2(-INFINITY, 0.f);
        float bm = mx;
#pragma unroll
        for (int i = 0; i < NB; ++i) bm = fmaxf(bm, ml[i].x);
        // Weights 2^(m - bm) <= 1 on the hardware exp2 (results below 2^-126
        // flush to zero, far below what the merge can carry). With nothing
        // non-empty yet (bm = -inf) every weight and the rescale are 0.
        const float bref = bm == -INFINITY ? 0.f : bm;
        const float sc = __builtin_amdgcn_exp2f(mx - bref);   // 0 while mx is -inf
        lsum *= sc;
#pragma unroll
        for (int j = 0; j < JW; ++j) { acc[j].x *= sc; acc[j].y *= sc; acc[j].z *= sc; acc[j].w *= sc; }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const float w = ml[i].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[i].x - bref);   // empty: 0
            lsum += w * ml[i].y;
#pragma unroll
            for (int j = 0; j < JW; ++j) {
                const float4 vv = R::widen(v[i][j]);
                acc[j].x += w * vv.x; acc[j].y += w * vv.y;
                acc[j].z += w * vv.z; acc[j].w += w * vv.w;
            }
        }
        mx = bm;
    }
    if constexpr (SW > 1) {
        // merge the SW waves' (mx, lsum, acc) of this slice (waves w0 ..
        // w0 + SW - 1 of the block), referenced to the largest mx
        __shared__ float2 sh_ml[4][64];
        __shared__ float4 sh_acc[4][JW][64];
        const int w0 = wave - sub;
        sh_ml[wave][lane] = make_float2(mx, lsum);
#pragma unroll
        for (int j = 0; j < JW; ++j) sh_acc[wave][j][lane] = acc[j];
        __syncthreads();
        if (sub != 0 || !live) return;
        float m_all = mx;
#pragma unroll
        for (int w = 1; w < SW; ++w) m_all = fmaxf(m_all, sh_ml[w0 + w][lane].x);
        if (m_all != -INFINITY) {
            lsum = 0.f;
#pragma unroll
            for (int j = 0; j < JW; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int w = 0; w < SW; ++w) {
                const float2 mlw = sh_ml[w0 + w][lane];
                const float wt = mlw.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mlw.x - m_all);
                lsum += wt * mlw.y;
#pragma unroll
                for (int j = 0; j < JW; ++j) {
                    const float4 a = sh_acc[w0 + w][j][lane];
                    acc[j].x += wt * a.x; acc[j].y += wt * a.y; acc[j].z += wt * a.z; acc[j].w += wt * a.w;
                }
            }
        }
    }
    if (!ok) return;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int r = row - row_lo;
    if (APK) {
        const int col = (g * group + r % group) * D + 32 * b + 4 * hi;
#pragma unroll
        for (int j = 0; j < JW; ++j)
            st4(out + apack_index(r / group, col + 8 * (j0 + j)),
                make_float4(acc[j].x * inv, acc[j].y * inv, acc[j].z * inv, acc[j].w * inv));
        return;
    }
    TO* orow = out + lb * out_layer + ((long long)(r / group) * hq + g * group + r % group) * D + 32 * b + 4 * hi;
#pragma unroll
    for (int j = 0; j < JW; ++j)
        st4(orow + 8 * (j0 + j), make_float4(acc[j].x * inv, acc[j].y * inv, acc[j].z * inv, acc[j].w * inv));
}

// ---------------------------------------------------------------------------
// Private-tail partial on the matrix cores (bf16 rings): one wave per (stream,
// call layer x KV head). The G = Hq / Hkv query heads of the stream are the
// columns of S^T = K_tail . Q^T, so each tail key is read once for all of
// them. The wave streams its tail in 32-key tiles through its own LDS buffers
// in the partial kernel's layout (direct-to-LDS loads, K plane rotation) and
// runs the same per-tile arithmetic (qk_scores, softmax_tile, pv_tile).
// Partial rows row_base + stream * G + c go to slot `slot`.
// grid (ceil(streams / TAIL_WAVES), Lb * Hkv), block TAIL_WAVES * 64.
constexpr int TAIL_WAVES = 4;

template <int D>
__global__ __launch_bounds__(TAIL_WAVES * 64) void partial_tail_mfma(
    const uint16_t* __restrict__ q, long long q_layer, int hq, int group, const uint16_t* __restrict__ tail_k,
    const uint16_t* __restrict__ tail_v, const int32_t* __restrict__ tail_len, int n_streams, int cap, int hkv,
    float scale_log2, int slot, Partials part, int row_base) {
    constexpr int KD = D / 16, DB = D / 32, PLANE = KT * 64, TILE = DB * PLANE, NBLK = TILE / 1024;
    __shared__ __attribute__((aligned(1024))) char lds[TAIL_WAVES][2][TILE];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
    const int strm = blockIdx.x * TAIL_WAVES + wave, lg = blockIdx.y, lb = lg / hkv, g = lg % hkv;
    if (strm >= n_streams) return;                                  // whole wave; no barriers below
    char* kbuf = lds[wave][0];
    char* vbuf = lds[wave][1];
    int n = tail_len[strm];
    n = n < 0 ? 0 : (n > cap ? cap : n);

    // B operand: column c = l32 is query head g * G + c of this stream (c < G)
    bf16x8 qf[KD];
    const bool col_ok = l32 < group;
    const uint16_t* qp = q + lb * q_layer + ((long long)strm * hq + g * group + (col_ok ? l32 : 0)) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) qf[kk] = col_ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * kk) : bf16x8{};

    const long long tok_base = ((long long)lb * n_streams + strm) * cap;
    const int stride = hkv * D;
    const uint16_t* tk = tail_k + tok_base * stride + g * D;
    const uint16_t* tv = tail_v + tok_base * stride + g * D;
    // direct-to-LDS copy of one tile: block b = plane b / 2, keys 16 (b % 2) .. + 15
    const int dma_key = lane >> 2, dma_pos = lane & 3;
    auto load_tile = [&](int t) {
#pragma unroll
        for (int b = 0; b < NBLK; ++b) {
            const int key = 16 * (b & 1) + dma_key;
            const int j = min(t * KT + key, n - 1);                 // past the tail: a valid key, masked later
            const int kchunk = (dma_pos ^ ((key >> 2) & 3)) << 3;   // K plane rotation
            const uint16_t* row_k = tk + (long long)j * stride + (b >> 1) * 32;
            const uint16_t* row_v = tv + (long long)j * stride + (b >> 1) * 32;
            __builtin_amdgcn_global_load_lds((const GLB_AS void*)(row_k + kchunk), (LDS_AS void*)(kbuf + b * 1024), 16,
                                             0, 0);
            __builtin_amdgcn_global_load_lds((const GLB_AS void*)(row_v + (dma_pos << 3)),
                                             (LDS_AS void*)(vbuf + b * 1024), 16, 0, 0);
        }
    };
    // LDS read offsets of the partial kernel
    const int prow = (l32 & ~0xC) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
    const int koff0 = prow * 64 + (((0 + hi) ^ ((prow >> 2) & 3)) << 4);
    const int koff1 = prow * 64 + (((2 + hi) ^ ((prow >> 2) & 3)) << 4);
    const int gi = lane >> 4, li = lane & 15;
    const int voff = (8 * (gi >> 1) + (li >> 2)) * 64 + ((2 * (gi & 1) + ((li & 3) >> 1)) << 4) + ((li & 1) << 3);

    f32x16 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    for (int t = 0; t * KT < n; ++t) {
        load_tile(t);           // the previous tile's LDS reads were consumed by its MFMAs already
        wait_vmem<0>();
        bf16x8 pf[2];
        const f32x16 sc = qk_scores<D>(kbuf, koff0, koff1, qf);
        softmax_tile<D>(sc, t * KT, n, hi, scale_log2, acc, m_run, l_run, pf);
        pv_tile<D>(vbuf, voff, pf, acc);
    }
    l_run += __shfl_xor(l_run, 32);
    if (!col_ok) return;
    const int row = row_base + strm * group + l32;
    uint16_t* op = part.optr<uint16_t>() + part.oblock(slot, lg, row) + ((row & 31) + 32 * hi) * 4;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<uint2*>(op + (b * 4 + j) * 256) =
                make_uint2(pack_bf16(acc[b][4 * j], acc[b][4 * j + 1]), pack_bf16(acc[b][4 * j + 2], acc[b][4 * j + 3]));
    if (hi == 0) part.ml[part.idx(slot, lg, row)] = make_float2(m_run, l_run);
}

// ---------------------------------------------------------------------------
// Append one token per decode stream to its private tail, in every layer.
// 16-byte chunks; each thread copies up to APPEND_BATCH chunks (of any
// layers) with every load issued before the first store.
// grid (G), block 256.
constexpr int APPEND_BATCH = 8;

__global__ __launch_bounds__(256) void append_tail(uint4* __restrict__ tail_k, uint4* __restrict__ tail_v,
                                                   int32_t* tail_len, const uint4* __restrict__ k_new,
                                                   const uint4* __restrict__ v_new, int n_layers, int n_streams,
                                                   int cap, int tok_chunks, int retire_full, uint32_t* overflow) {
    const int strm = blockIdx.x;
    int n = tail_len[strm];
    if (retire_full && n >= cap) n = 0;                 // the request ended: a new one starts here
    const bool ok = n >= 0 && n < cap;
    if (ok) {
        const int total = n_layers * tok_chunks;       // (layer, chunk) items of this stream
        for (int i0 = threadIdx.x; i0 < total; i0 += 256 * APPEND_BATCH) {
            uint4 kk[APPEND_BATCH], vv[APPEND_BATCH];
#pragma unroll
            for (int u = 0; u < APPEND_BATCH; ++u) {
                const int it = min(i0 + 256 * u, total - 1);
                const int lb = it / tok_chunks, c = it % tok_chunks;
                const long long src = ((long long)lb * n_streams + strm) * tok_chunks + c;
                kk[u] = k_new[src];
                vv[u] = v_new[src];
            }
#pragma unroll
            for (int u = 0; u < APPEND_BATCH; ++u) {
                const int it = i0 + 256 * u;
                if (it < total) {
                    const int lb = it / tok_chunks, c = it % tok_chunks;
                    const long long dst = (((long long)lb * n_streams + strm) * cap + n) * tok_chunks + c;
                    tail_k[dst] = kk[u];
                    tail_v[dst] = vv[u];
                }
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


struct Plan {
    int group, m_rows, mpad, lg_count, total, chunk, parts, max_parts;
    bool mfma;
    int o_bytes;     // bytes per partial-O element: 2 (bf16 rings) or 4 (f32 rings)
};

static int valu_row_blocks(int m) { return (m + VALU_ROWS - 1) / VALU_ROWS; }

// Choose the split count: as many workgroups as fit at once (one per CU on
// 256 CUs) without a partial second wave, and no split shorter than
// min_keys: 48 keys for the matrix-core kernel, which the 32-key rounding of
// the split length makes two tiles (a single-layer call of the Pi0.5-like
// stack then runs 26 splits of 2 tiles: 496 -> 458 us per 18-layer step,
// against 13 splits of 4 tiles, once the combine merged many splits in one
// round trip); half a tile for the vector kernel, whose waves walk their
// keys one at a time (splits are still whole 32-key chunks: the 88-key fp32
// call went from 1 to 3 splits, 24.6 to 12.7 us).
static int default_splits(int lg_count, int row_blocks, int max_keys, int min_keys) {
    const int base = lg_count * row_blocks;
    int s = 256 * MFMA_OCC / base;
    int by_len = max_keys / min_keys;
    if (by_len < 1) by_len = 1;
    if (s > by_len) s = by_len;
    if (s > 64) s = 64;
    return s < 1 ? 1 : s;
}

static size_t partial_bytes(const Plan& p, int d) {
    const size_t o = align_up((size_t)p.max_parts * p.lg_count * p.mpad * d * p.o_bytes, 256);
    const size_t ml = align_up((size_t)p.max_parts * p.lg_count * p.mpad * sizeof(float2), 256);
    return o + ml;
}

static Partials partials_in(void* ws, const Plan& p, int d) {
    Partials part;
    part.o = ws;
    part.ml = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                        align_up((size_t)p.max_parts * p.lg_count * p.mpad * d * p.o_bytes, 256));
    part.mpad = p.mpad;
    part.lg_count = p.lg_count;
    part.d = d;
    return part;
}

// `extra` is the number of extra partial slots after the cached-key splits.
static pa_status plan_for(const Ring* r, int layer_begin, int num_layers, int hq, int n_rows_tokens, int n_dyn,
                          int req_splits, int extra, Plan* p, bool f32_partials = false) {
    const rb_config& c = r->cfg;
    PA_CHECK_ARG(num_layers >= 1 && layer_begin >= 0 && layer_begin + num_layers <= c.num_layers, PA_ESHAPE,
                 "layers [%d, %d) outside the ring's %d layers", layer_begin, layer_begin + num_layers, c.num_layers);
    PA_CHECK_ARG(hq >= 1 && hq % c.num_kv_heads == 0, PA_ESHAPE, "n_q_heads %d is not a multiple of num_kv_heads %d",
                 hq, c.num_kv_heads);
    PA_CHECK_ARG(n_rows_tokens >= 1, PA_ESHAPE, "need at least one query token");
    PA_CHECK_ARG(req_splits >= 0 && req_splits <= 127, PA_EINVAL, "num_splits %d not in [0, 127]", req_splits);
    p->mfma = c.dtype == PA_BF16;
    p->o_bytes = p->mfma && !f32_partials ? 2 : 4;
    if (p->mfma)
        PA_CHECK_ARG(c.head_dim == 64 || c.head_dim == 128 || c.head_dim == 256, PA_ESHAPE,
                     "bf16 attention supports head_dim 64, 128 or 256 (got %d)", c.head_dim);
    p->group = hq / c.num_kv_heads;
    p->m_rows = n_rows_tokens * p->group;
    p->lg_count = num_layers * c.num_kv_heads;
    const int row_blocks = p->mfma ? (p->m_rows + ROWS_PER_WG - 1) / ROWS_PER_WG : valu_row_blocks(p->m_rows);
    p->mpad = (p->m_rows + 31) / 32 * 32;
    const int max_keys = (int)(r->seq_len() + n_dyn);
    const int s_max = req_splits ? req_splits : default_splits(p->lg_count, row_blocks, max_keys, p->mfma ? 48 : KT / 2);
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
    s.skip_at = r->skip_at();
    s.skip_len = r->cfg.spare_slots ? r->cfg.tokens_per_frame : 0;
    s.head_word = r->cfg.spare_slots ? r->state_word : nullptr;
    s.n_dyn = n_dyn;
    s.hkv = r->cfg.num_kv_heads;
    s.d = r->cfg.head_dim;
    return s;
}

// Token-major q [Lb][N][Hq][D] (bf16) into the matrix-core kernel's operand
// order (PA_Q_OPERAND): one thread per 16-byte chunk of the output; padding
// rows of the last 32-row block are zeros.
__global__ __launch_bounds__(256) void pack_q(const uint4* __restrict__ q, uint4* __restrict__ qo, int n_tok, int hq,
                                              int hkv, int d, int nrb, long long chunks) {
    const long long c = (long long)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks) return;
    const int lane = (int)(c & 63), kd = d >> 4, group = hq / hkv;
    long long blk = c >> 6;
    const int kk = (int)(blk % kd);
    blk /= kd;
    const int rb = (int)(blk % nrb);
    const long long lg = blk / nrb;
    const long long lb = lg / hkv;
    const int g = (int)(lg % hkv);
    const int r = rb * 32 + (lane & 31), d0 = kk * 16 + (lane >> 5) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < n_tok * group) {
        const int t = r / group, h = g * group + r % group;
        v = q[((lb * n_tok + t) * hq + h) * (d >> 3) + (d0 >> 3)];
    }
    qo[c] = v;
}

static pa_status launch_partials(const Ring* r, const Plan& p, const void* q, long long q_layer, int hq,
                                 const KvSource& src, float scale, const Partials& part, hipStream_t stream,
                                 const void* q2 = nullptr, long long q2_layer = 0, int m1 = 0,
                                 bool q_packed = false) {
    if (p.parts == 0) return PA_OK;
    const float scale_log2 = scale * 1.4426950408889634f;
    const int d = r->cfg.head_dim;
    if (p.mfma) {
        const int units = p.parts * p.lg_count;
        const int wide_wgs = units * ((p.m_rows + ROWS_PER_WG - 1) / ROWS_PER_WG);
        const int half_wgs = units * ((p.m_rows + ROWS_PER_WG / 2 - 1) / (ROWS_PER_WG / 2));
        const bool halves = d == 256 && !q2 && p.chunk >= HALVES_MIN_TILES * KT && half_wgs > wide_wgs &&
                            half_wgs <= HALVES_MAX_WGS;
        const bool narrow = d == 256 && !q2 && !halves && wide_wgs <= NARROW_MAX_WGS;
        const int rpw = halves || narrow ? ROWS_PER_WG / 2 : ROWS_PER_WG;
        const int threads = halves ? rpw * 4 : rpw * 2;
        const int row_blocks = (p.m_rows + rpw - 1) / rpw;
        const dim3 grid(((units + N_XCD - 1) / N_XCD) * N_XCD * row_blocks);
        const uint16_t* qq = static_cast<const uint16_t*>(q);
        const uint16_t* qq2 = static_cast<const uint16_t*>(q2);
#define PA_MFMA_(DD, FU, QP, WV, FP, ...)                                                                     \
    partial_mfma<DD, FU, QP, WV, FP, ##__VA_ARGS__><<<grid, threads, 0, stream>>>(                            \
        qq, q_layer, hq, p.group, p.m_rows, src, p.chunk, scale_log2, part, p.parts, row_blocks, qq2, q2_layer, m1)
#define PA_MFMA(DD, FU, QP, ...) PA_MFMA_(DD, FU, QP, ##__VA_ARGS__)
        // FP32 partial O (optional, single-reader steps): the same kernels
        // with wider partial stores; the combine reads FP32 partials
        const bool f32p = p.o_bytes == 4;
        if (f32p && q2) return fail(PA_EINVAL, "FP32 partials are for the single-reader step");
        if (halves) {
            if (f32p) {
                if (q_packed) PA_MFMA(256, false, true, MFMA_WAVES, true, 2);
                else PA_MFMA(256, false, false, MFMA_WAVES, true, 2);
            } else if (q_packed) PA_MFMA(256, false, true, MFMA_WAVES, false, 2);
            else PA_MFMA(256, false, false, MFMA_WAVES, false, 2);
        } else if (narrow) {
            if (f32p) {
                if (q_packed) PA_MFMA(256, false, true, MFMA_WAVES / 2, true);
                else PA_MFMA(256, false, false, MFMA_WAVES / 2, true);
            } else if (q_packed) PA_MFMA(256, false, true, MFMA_WAVES / 2, false);
            else PA_MFMA(256, false, false, MFMA_WAVES / 2, false);
        } else if (f32p) {
            if (d == 256) { if (q_packed) PA_MFMA(256, false, true, MFMA_WAVES, true); else PA_MFMA(256, false, false, MFMA_WAVES, true); }
            else if (d == 128) { if (q_packed) PA_MFMA(128, false, true, MFMA_WAVES, true); else PA_MFMA(128, false, false, MFMA_WAVES, true); }
            else { if (q_packed) PA_MFMA(64, false, true, MFMA_WAVES, true); else PA_MFMA(64, false, false, MFMA_WAVES, true); }
        } else if (q_packed) {
            if (d == 256) PA_MFMA(256, false, true, MFMA_WAVES, false);
            else if (d == 128) PA_MFMA(128, false, true, MFMA_WAVES, false);
            else PA_MFMA(64, false, true, MFMA_WAVES, false);
        } else if (q2) {
            if (d == 256) PA_MFMA(256, true, false, MFMA_WAVES, false);
            else if (d == 128) PA_MFMA(128, true, false, MFMA_WAVES, false);
            else PA_MFMA(64, true, false, MFMA_WAVES, false);
        } else {
            if (d == 256) PA_MFMA(256, false, false, MFMA_WAVES, false);
            else if (d == 128) PA_MFMA(128, false, false, MFMA_WAVES, false);
            else PA_MFMA(64, false, false, MFMA_WAVES, false);
        }
#undef PA_MFMA
#undef PA_MFMA_
    } else {
        dim3 grid(p.parts, valu_row_blocks(p.m_rows), p.lg_count);
        const float* qf = static_cast<const float*>(q);
#define PA_VALU(DD) partial_valu<DD><<<grid, 256, 0, stream>>>(qf, q_layer, hq, p.group, p.m_rows, src, p.chunk, \
                                                                scale_log2, part)
        if (d == 256) PA_VALU(256);
        else if (d == 128) PA_VALU(128);
        else if (d == 64) PA_VALU(64);
        else PA_VALU(32);
#undef PA_VALU
    }
    PA_LAUNCHED();
    return PA_OK;
}

// out_dtype PA_BF16_APACKED: bf16 in the packed activation layout (one layer).
constexpr int PA_BF16_APACKED = -1;

static pa_status launch_combine(const Ring* r, const Plan& p, int n_parts, int hq, long long out_layer, void* out,
                                int out_dtype, const Partials& part, hipStream_t stream, int row_lo = 0,
                                int row_hi = -1) {
    const int d = r->cfg.head_dim, hkv = r->cfg.num_kv_heads;
    if (row_hi < 0) row_hi = p.m_rows;
    const int units = (row_hi - (row_lo & ~31) + 31) / 32 * (d / 32);   // (32-row, 32-dim) blocks
    // at most 64 workgroups of whole blocks (a single-layer call): one slice
    // per wave instead (larger launches, the 18-layer decode pass included,
    // measured no gain)
    const bool thin = units * p.lg_count <= 256;
    // more splits than one batch of loads holds (16 bf16 or 8 FP32 partials):
    // two or four waves share each slice, one batch each
    const int batch = p.o_bytes == 2 ? 16 : 8;
    const int sw = n_parts <= batch ? 1 : (n_parts <= 2 * batch ? 2 : 4);
    // a wave's splits fit a batch of 8 (fewer registers, more waves resident)?
    const bool nb8 = (n_parts + sw - 1) / sw <= 8;
    const int slices = units * (thin ? 4 : 1);
    const dim3 grid((slices * sw + 3) / 4, p.lg_count);
#define PA_COMBINE_NB(TO, DD, PO, APK, NB)                                                                     \
    do {                                                                                                       \
        if (sw == 4 && thin)                                                                                   \
            combine<TO, DD, PO, APK, 1, 4, NB><<<grid, 256, 0, stream>>>(part, n_parts, row_lo, row_hi, p.group, \
                                                                         hq, hkv, out_layer, static_cast<TO*>(out)); \
        else if (sw == 4)                                                                                      \
            combine<TO, DD, PO, APK, 4, 4, NB><<<grid, 256, 0, stream>>>(part, n_parts, row_lo, row_hi, p.group, \
                                                                         hq, hkv, out_layer, static_cast<TO*>(out)); \
        else if (sw == 2 && thin)                                                                              \
            combine<TO, DD, PO, APK, 1, 2, NB><<<grid, 256, 0, stream>>>(part, n_parts, row_lo, row_hi, p.group, \
                                                                         hq, hkv, out_layer, static_cast<TO*>(out)); \
        else if (sw == 2)                                                                                      \
            combine<TO, DD, PO, APK, 4, 2, NB><<<grid, 256, 0, stream>>>(part, n_parts, row_lo, row_hi, p.group, \
                                                                         hq, hkv, out_layer, static_cast<TO*>(out)); \
        else if (thin)                                                                                         \
            combine<TO, DD, PO, APK, 1, 1, NB><<<grid, 256, 0, stream>>>(part, n_parts, row_lo, row_hi, p.group, \
                                                                         hq, hkv, out_layer, static_cast<TO*>(out)); \
        else                                                                                                   \
            combine<TO, DD, PO, APK, 4, 1, NB><<<grid, 256, 0, stream>>>(part, n_parts, row_lo, row_hi, p.group, \
                                                                         hq, hkv, out_layer, static_cast<TO*>(out)); \
    } while (0)
#define PA_COMBINE_JW(TO, DD, PO, APK)                                                                         \
    do {                                                                                                       \
        if (nb8 || CombineRaw<PO>::BATCH == 8) PA_COMBINE_NB(TO, DD, PO, APK, 8);                              \
        else PA_COMBINE_NB(TO, DD, PO, APK, CombineRaw<PO>::BATCH);                                            \
    } while (0)
#define PA_COMBINE(TO, DD)                                                                                  \
    do {                                                                                                    \
        if (p.o_bytes == 2) PA_COMBINE_JW(TO, DD, uint16_t, false);                                          \
        else PA_COMBINE_JW(TO, DD, float, false);                                                            \
    } while (0)
#define PA_COMBINE_APK(DD)                                                                                   \
    do {                                                                                                     \
        if (p.o_bytes == 2) PA_COMBINE_JW(uint16_t, DD, uint16_t, true);                                      \
        else PA_COMBINE_JW(uint16_t, DD, float, true);                                                        \
    } while (0)
    if (out_dtype == PA_BF16_APACKED) {
        if (d == 256) PA_COMBINE_APK(256);
        else if (d == 128) PA_COMBINE_APK(128);
        else if (d == 64) PA_COMBINE_APK(64);
        else if (d == 32) PA_COMBINE_APK(32);
        else return fail(PA_ESHAPE, "combine: head_dim %d must be 32, 64, 128 or 256", d);
    } else if (out_dtype == PA_F32) {
        if (d == 256) PA_COMBINE(float, 256);
        else if (d == 128) PA_COMBINE(float, 128);
        else if (d == 64) PA_COMBINE(float, 64);
        else if (d == 32) PA_COMBINE(float, 32);
        else return fail(PA_ESHAPE, "combine: head_dim %d must be 32, 64, 128 or 256", d);
    } else {
        if (d == 256) PA_COMBINE(uint16_t, 256);
        else if (d == 128) PA_COMBINE(uint16_t, 128);
        else if (d == 64) PA_COMBINE(uint16_t, 64);
        else if (d == 32) PA_COMBINE(uint16_t, 32);
        else return fail(PA_ESHAPE, "combine: head_dim %d must be 32, 64, 128 or 256", d);
    }
#undef PA_COMBINE
#undef PA_COMBINE_APK
#undef PA_COMBINE_JW
#undef PA_COMBINE_NB
    PA_LAUNCHED();
    return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" size_t pattn_workspace_bytes(const rb_ring* ring, const pattn_args* a) {
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    if (!r || !a) return 0;
    Plan p;
    if (a->partials_f32 != 0 && a->partials_f32 != 1) return 0;
    if (plan_for(r, a->layer_begin, a->num_layers, a->n_q_heads, a->n_dyn, a->n_dyn, a->num_splits, 0, &p,
                 a->partials_f32 == 1) != PA_OK)
        return 0;
    return partial_bytes(p, r->cfg.head_dim);
}

static pa_status step_impl(const rb_ring* ring, const pattn_args* a, const void* q, const void* k_dyn,
                           const void* v_dyn, void* out, void* ws, size_t ws_bytes, void* stream, void* ev_begin,
                           void* ev_end, bool apacked = false, bool q_packed = false) {
    clear_error();
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    PA_CHECK_ARG(r && a && q && k_dyn && v_dyn && out && ws, PA_EINVAL, "pattn_step: null argument");
    PA_CHECK_ARG(aligned16(q) && aligned16(k_dyn) && aligned16(v_dyn) && aligned16(out) && aligned16(ws) &&
                     aligned16(r->k) && aligned16(r->v),
                 PA_EINVAL, "pattn_step: every buffer must be 16-byte aligned");
    PA_CHECK_ARG(a->out_dtype == PA_F32 || a->out_dtype == PA_BF16, PA_EINVAL, "pattn_step: bad out_dtype");
    PA_CHECK_ARG(a->q_layout == PA_Q_TOKEN_MAJOR || (a->q_layout == PA_Q_OPERAND && r->cfg.dtype == PA_BF16),
                 PA_EINVAL, "pattn_step: q_layout must be PA_Q_TOKEN_MAJOR, or PA_Q_OPERAND on a bf16 ring");
    PA_CHECK_ARG(a->scale > 0.f && a->scale < 1e30f, PA_EINVAL, "pattn_step: scale must be positive and finite");
    PA_CHECK_ARG(a->n_dyn >= 1, PA_ESHAPE, "pattn_step: n_dyn must be >= 1");
    PA_CHECK_ARG(a->partials_f32 == 0 || a->partials_f32 == 1, PA_EINVAL, "pattn_step: partials_f32 must be 0 or 1");
    Plan p;
    pa_status st = plan_for(r, a->layer_begin, a->num_layers, a->n_q_heads, a->n_dyn, a->n_dyn, a->num_splits, 0, &p,
                            a->partials_f32 == 1);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(!(r->cfg.pin_capacity > 0 && r->pinned == 0), PA_ESTATE,
                 "pattn_step: the prefix is not pinned yet (rb_pin_prefix first)");
    const size_t need = partial_bytes(p, r->cfg.head_dim);
    PA_CHECK_ARG(ws_bytes >= need, PA_ERANGE, "pattn_step: workspace %zu bytes < %zu needed", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = check_capture(r, s, "pattn_step");
    if (st != PA_OK) return st;
    const KvSource src = source_for(r, a->layer_begin, k_dyn, v_dyn, a->n_dyn);
    const Partials part = partials_in(ws, p, r->cfg.head_dim);
    const long long q_layer = (long long)a->n_dyn * a->n_q_heads * r->cfg.head_dim;
    if (ev_begin) PA_HIP(hipEventRecord(static_cast<hipEvent_t>(ev_begin), s));
    st = launch_partials(r, p, q, q_layer, a->n_q_heads, src, a->scale, part, s, nullptr, 0, 0,
                         q_packed || a->q_layout == PA_Q_OPERAND);
    if (st != PA_OK) return st;
    if (ev_end) PA_HIP(hipEventRecord(static_cast<hipEvent_t>(ev_end), s));
    return launch_combine(r, p, p.parts, a->n_q_heads, q_layer, out, apacked ? PA_BF16_APACKED : a->out_dtype, part,
                          s);
}

pa_status pa::pattn_step_apacked(const rb_ring* ring, const pattn_args* a, const void* q, const void* k_dyn,
                                 const void* v_dyn, void* out_p, void* ws, size_t ws_bytes, void* stream,
                                 bool q_packed) {
    clear_error();
    PA_CHECK_ARG(a && a->num_layers == 1 && a->n_dyn <= 64 && a->out_dtype == PA_BF16, PA_EINVAL,
                 "pattn_step (packed output): one layer, at most 64 suffix tokens, bf16 output");
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    PA_CHECK_ARG(!q_packed || (r && r->cfg.dtype == PA_BF16), PA_EINVAL, "pattn_step (packed Q): bf16 rings only");
    return step_impl(ring, a, q, k_dyn, v_dyn, out_p, ws, ws_bytes, stream, nullptr, nullptr, true, q_packed);
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

// ---------------------------------------------------------------------------
// pattn_step for callers that cannot allocate: the split partials go to a
// file-scope device array instead of a caller workspace. Each GPU holds its
// own copy of the array (allocated with the code object, kept until the
// process ends); its address on a device is looked up once, with that
// device current, and cached. The array's name is only a host-side stand-in:
// host code uses the looked-up address, never the name.
namespace pa {
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(32) << 20;   // covers 18 layers x 416 rows x 7 splits, bf16
constexpr int NOALLOC_MAX_DEVICES = 64;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];
static void* g_scratch_dev[NOALLOC_MAX_DEVICES];
static std::mutex g_scratch_mu;

static pa_status noalloc_scratch(void** out) {
    int dev = -1;
    PA_HIP(hipGetDevice(&dev));
    PA_CHECK_ARG(dev >= 0 && dev < NOALLOC_MAX_DEVICES, PA_EDEVICE, "pattn_step_noalloc: device %d beyond %d", dev,
                 NOALLOC_MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        PA_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        PA_CHECK_ARG(p, PA_EDEVICE, "pattn_step_noalloc: no address for the scratch array on device %d", dev);
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return PA_OK;
}
}  // namespace pa

extern "C" size_t pattn_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

extern "C" pa_status pattn_step_noalloc(const rb_ring* ring, const pattn_args* a, const void* q, const void* k_dyn,
                                        const void* v_dyn, void* out, void* stream) {
    clear_error();
    PA_CHECK_ARG(ring && a, PA_EINVAL, "pattn_step_noalloc: null argument");
    const size_t need = pattn_workspace_bytes(ring, a);
    PA_CHECK_ARG(need > 0, PA_ESHAPE, "pattn_step_noalloc: arguments rejected (see pattn_workspace_bytes)");
    PA_CHECK_ARG(need <= NOALLOC_SCRATCH_BYTES, PA_ERANGE,
                 "pattn_step_noalloc: the call needs %zu bytes of partials, above the fixed %zu-byte scratch; "
                 "use pattn_step with a workspace", need, NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    pa_status st = noalloc_scratch(&ws);
    if (st != PA_OK) return st;
    return step_impl(ring, a, q, k_dyn, v_dyn, out, ws, NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr);
}

// Chunks of 16 bytes in the PA_Q_OPERAND form of q, 0 if not applicable.
static long long operand_q_chunks(const Ring* r, const pattn_args* a) {
    if (!r || !a || r->cfg.dtype != PA_BF16 || a->num_layers < 1 || a->n_dyn < 1 || a->n_q_heads < 1 ||
        a->n_q_heads % r->cfg.num_kv_heads)
        return 0;
    const long long group = a->n_q_heads / r->cfg.num_kv_heads;
    const long long nrb = (a->n_dyn * group + 31) / 32;
    return (long long)a->num_layers * r->cfg.num_kv_heads * nrb * 32 * r->cfg.head_dim / 8;
}

extern "C" size_t pattn_operand_q_bytes(const rb_ring* ring, const pattn_args* a) {
    return (size_t)operand_q_chunks(reinterpret_cast<const Ring*>(ring), a) * 16;
}

extern "C" pa_status pattn_pack_q(const rb_ring* ring, const pattn_args* a, const void* q, void* q_operand,
                                  void* stream) {
    clear_error();
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    PA_CHECK_ARG(r && a && q && q_operand, PA_EINVAL, "pattn_pack_q: null argument");
    PA_CHECK_ARG(r->cfg.dtype == PA_BF16, PA_EINVAL, "pattn_pack_q: the operand order is for bf16 rings");
    PA_CHECK_ARG(aligned16(q) && aligned16(q_operand), PA_EINVAL, "pattn_pack_q: buffers must be 16-byte aligned");
    const long long chunks = operand_q_chunks(r, a);
    PA_CHECK_ARG(chunks > 0, PA_ESHAPE, "pattn_pack_q: need layers >= 1, n_dyn >= 1 and Hq a multiple of Hkv");
    const int hkv = r->cfg.num_kv_heads, d = r->cfg.head_dim, nrb = (a->n_dyn * (a->n_q_heads / hkv) + 31) / 32;
    const char* qb = static_cast<const char*>(q);
    const char* ob = static_cast<const char*>(q_operand);
    const long long in_bytes = (long long)a->num_layers * a->n_dyn * a->n_q_heads * d * 2;
    PA_CHECK_ARG(ob + chunks * 16 <= qb || qb + in_bytes <= ob, PA_EINVAL, "pattn_pack_q: buffers overlap");
    pack_q<<<(unsigned)((chunks + 255) / 256), 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint4*>(q), static_cast<uint4*>(q_operand), a->n_dyn, a->n_q_heads, hkv, d, nrb, chunks);
    PA_LAUNCHED();
    return PA_OK;
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
    PA_CHECK_ARG(aligned16(tail_k) && aligned16(tail_v) && aligned16(k_new) && aligned16(v_new), PA_EINVAL,
                 "pattn_append_private: buffers must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    // a token of one layer is Hkv * D elements: a whole number of 16-byte chunks (D >= 32)
    const int tok_chunks = (int)((size_t)r->cfg.num_kv_heads * r->cfg.head_dim * r->elem_bytes() / 16);
    append_tail<<<a->n_streams, 256, 0, s>>>(static_cast<uint4*>(tail_k), static_cast<uint4*>(tail_v), tail_len,
                                             static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                                             a->num_layers, a->n_streams, a->tail_capacity, tok_chunks,
                                             a->retire_full, overflow);
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

// Private-tail partials of decode rows [row_base, row_base + G * group) into slot `slot`.
static pa_status launch_tails(const Ring* r, const Plan& p, const void* q, long long q_layer, int hq, const void* tail_k,
                              const void* tail_v, const int32_t* tail_len, int n_streams, int cap, float scale,
                              int slot, const Partials& part, int row_base, hipStream_t s) {
    const int d = r->cfg.head_dim, hkv = r->cfg.num_kv_heads;
    const int m_rows = n_streams * p.group;
    const float scale_log2 = scale * 1.4426950408889634f;
    dim3 grid(valu_row_blocks(m_rows), p.lg_count);
#define PA_TAIL(T, DD)                                                                                           \
    partial_tail<T, DD><<<grid, 256, 0, s>>>(static_cast<const T*>(q), q_layer, hq, p.group, m_rows,               \
                                             static_cast<const T*>(tail_k), static_cast<const T*>(tail_v), tail_len, \
                                             n_streams, cap, hkv, scale_log2, slot, part, row_base)
    if (r->cfg.dtype == PA_F32) {
        if (d == 256) PA_TAIL(float, 256);
        else if (d == 128) PA_TAIL(float, 128);
        else if (d == 64) PA_TAIL(float, 64);
        else PA_TAIL(float, 32);
    } else if (p.group <= 32) {
        // bf16: the stream's query heads are the columns of one MFMA tile
        const dim3 tgrid((n_streams + TAIL_WAVES - 1) / TAIL_WAVES, p.lg_count);
#define PA_TAIL_MFMA(DD)                                                                                        \
    partial_tail_mfma<DD><<<tgrid, TAIL_WAVES * 64, 0, s>>>(                                                    \
        static_cast<const uint16_t*>(q), q_layer, hq, p.group, static_cast<const uint16_t*>(tail_k),            \
        static_cast<const uint16_t*>(tail_v), tail_len, n_streams, cap, hkv, scale_log2, slot, part, row_base)
        if (d == 256) PA_TAIL_MFMA(256);
        else if (d == 128) PA_TAIL_MFMA(128);
        else PA_TAIL_MFMA(64);
#undef PA_TAIL_MFMA
    } else {
        if (d == 256) PA_TAIL(uint16_t, 256);
        else if (d == 128) PA_TAIL(uint16_t, 128);
        else PA_TAIL(uint16_t, 64);
    }
#undef PA_TAIL
    PA_LAUNCHED();
    return PA_OK;
}

extern "C" pa_status pattn_decode(const rb_ring* ring, const pattn_decode_args* a, const void* q, const void* tail_k,
                                  const void* tail_v, const int32_t* tail_len, void* out, void* ws, size_t ws_bytes,
                                  void* stream) {
    clear_error();
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    pa_status st = check_decode(r, a);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(q && tail_k && tail_v && tail_len && out && ws, PA_EINVAL, "pattn_decode: null argument");
    PA_CHECK_ARG(aligned16(q) && aligned16(out) && aligned16(ws) && aligned16(r->k) && aligned16(r->v) &&
                     aligned16(tail_k) && aligned16(tail_v), PA_EINVAL,
                 "pattn_decode: buffers must be 16-byte aligned");
    Plan p;
    st = plan_for(r, a->layer_begin, a->num_layers, a->n_q_heads, a->n_streams, 0, a->num_splits, 1, &p);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(!(r->cfg.pin_capacity > 0 && r->pinned == 0), PA_ESTATE, "pattn_decode: the prefix is not pinned yet");
    const size_t need = partial_bytes(p, r->cfg.head_dim);
    PA_CHECK_ARG(ws_bytes >= need, PA_ERANGE, "pattn_decode: workspace %zu bytes < %zu needed", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = check_capture(r, s, "pattn_decode");
    if (st != PA_OK) return st;
    const KvSource src = source_for(r, a->layer_begin, nullptr, nullptr, 0);
    const Partials part = partials_in(ws, p, r->cfg.head_dim);
    const int d = r->cfg.head_dim;
    const long long q_layer = (long long)a->n_streams * a->n_q_heads * d;
    st = launch_partials(r, p, q, q_layer, a->n_q_heads, src, a->scale, part, s);
    if (st != PA_OK) return st;
    st = launch_tails(r, p, q, q_layer, a->n_q_heads, tail_k, tail_v, tail_len, a->n_streams, a->tail_capacity,
                      a->scale, p.parts, part, 0, s);
    if (st != PA_OK) return st;
    return launch_combine(r, p, p.parts + 1, a->n_q_heads, q_layer, out, a->out_dtype, part, s);
}

// ---------------------------------------------------------------------------
// One pass for both kinds of reader (OxyGen review, core method: the action
// expert and the language expert read one shared cache): the action
// suffix's rows and the decode streams' rows stacked into one query matrix
// per (layer, KV head), so the shared
// [pin | window] keys stream through the chip once for both.

static pa_status check_fused(const Ring* r, const pattn_args* a, const pattn_decode_args* d) {
    pa_status st = check_decode(r, d);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(a, PA_EINVAL, "pattn_fused_step: null argument");
    PA_CHECK_ARG(r->cfg.dtype == PA_BF16, PA_EINVAL, "pattn_fused_step: needs a bf16 ring");
    PA_CHECK_ARG(a->layer_begin == d->layer_begin && a->num_layers == d->num_layers && a->n_q_heads == d->n_q_heads &&
                     a->scale == d->scale,
                 PA_EINVAL, "pattn_fused_step: action and decode arguments must agree on layers, heads and scale");
    PA_CHECK_ARG(a->out_dtype == PA_F32 || a->out_dtype == PA_BF16, PA_EINVAL, "pattn_fused_step: bad out_dtype");
    PA_CHECK_ARG(a->n_dyn >= 1, PA_ESHAPE, "pattn_fused_step: n_dyn must be >= 1");
    PA_CHECK_ARG(a->q_layout == PA_Q_TOKEN_MAJOR, PA_EINVAL, "pattn_fused_step: queries are token-major");
    PA_CHECK_ARG(a->partials_f32 == 0, PA_EINVAL, "pattn_fused_step: FP32 partials are for pattn_step");
    return PA_OK;
}

extern "C" size_t pattn_fused_workspace_bytes(const rb_ring* ring, const pattn_args* a, const pattn_decode_args* d) {
    clear_error();
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    if (!r || check_fused(r, a, d) != PA_OK) return 0;
    Plan p;
    if (plan_for(r, a->layer_begin, a->num_layers, a->n_q_heads, a->n_dyn + d->n_streams, a->n_dyn, a->num_splits, 1,
                 &p) != PA_OK)
        return 0;
    return partial_bytes(p, r->cfg.head_dim);
}

extern "C" pa_status pattn_fused_step(const rb_ring* ring, const pattn_args* a, const void* q, const void* k_dyn,
                                      const void* v_dyn, void* out, const pattn_decode_args* d, const void* q_dec,
                                      const void* tail_k, const void* tail_v, const int32_t* tail_len, void* out_dec,
                                      void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    PA_CHECK_ARG(r, PA_EINVAL, "pattn_fused_step: null ring");
    pa_status st = check_fused(r, a, d);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(q && k_dyn && v_dyn && out && q_dec && tail_k && tail_v && tail_len && out_dec && ws, PA_EINVAL,
                 "pattn_fused_step: null argument");
    PA_CHECK_ARG(aligned16(q) && aligned16(k_dyn) && aligned16(v_dyn) && aligned16(out) && aligned16(q_dec) &&
                     aligned16(tail_k) && aligned16(tail_v) && aligned16(out_dec) && aligned16(ws) &&
                     aligned16(r->k) && aligned16(r->v),
                 PA_EINVAL, "pattn_fused_step: every buffer must be 16-byte aligned");
    Plan p;
    st = plan_for(r, a->layer_begin, a->num_layers, a->n_q_heads, a->n_dyn + d->n_streams, a->n_dyn, a->num_splits, 1,
                  &p);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(!(r->cfg.pin_capacity > 0 && r->pinned == 0), PA_ESTATE, "pattn_fused_step: the prefix is not pinned yet");
    const size_t need = partial_bytes(p, r->cfg.head_dim);
    PA_CHECK_ARG(ws_bytes >= need, PA_ERANGE, "pattn_fused_step: workspace %zu bytes < %zu needed", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = check_capture(r, s, "pattn_fused_step");
    if (st != PA_OK) return st;
    const KvSource src = source_for(r, a->layer_begin, k_dyn, v_dyn, a->n_dyn);
    const Partials part = partials_in(ws, p, r->cfg.head_dim);
    const int D = r->cfg.head_dim;
    const int m_act = a->n_dyn * p.group;                       // action rows first, then decode rows
    const long long qa_layer = (long long)a->n_dyn * a->n_q_heads * D;
    const long long qd_layer = (long long)d->n_streams * a->n_q_heads * D;
    st = launch_partials(r, p, q, qa_layer, a->n_q_heads, src, a->scale, part, s, q_dec, qd_layer, m_act);
    if (st != PA_OK) return st;
    st = launch_tails(r, p, q_dec, qd_layer, a->n_q_heads, tail_k, tail_v, tail_len, d->n_streams, d->tail_capacity,
                      a->scale, p.parts, part, m_act, s);
    if (st != PA_OK) return st;
    st = launch_combine(r, p, p.parts, a->n_q_heads, qa_layer, out, a->out_dtype, part, s, 0, m_act);
    if (st != PA_OK) return st;
    return launch_combine(r, p, p.parts + 1, a->n_q_heads, qd_layer, out_dec, d->out_dtype, part, s, m_act, p.m_rows);
}

