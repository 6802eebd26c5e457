// One denoising step of the whole stack, every layer, launched from C++.
//
// The pages time the denoising loop as one component -- ten steps per
// action chunk ("Reflex: Real-Time VLA Control through Streaming Inference"
// paper review, §6 Table 7) -- and describe each step's suffix as recomputed
// while the cached regions are only read (§3 Eq. 1 text). Per layer the
// chain is AdaRMSNorm (§3 Eq. 2) and the packed QKV projection, partitioned
// attention (Eq. 1), and a residual out-projection, optionally followed by
// the SwiGLU FFN; the Euler update of the flow state is fused into the last
// projection of the last layer. The norm is fused (§2/§4 fused operators)
// into the kernel that finishes h, which writes the normalised operand of the
// next GEMM, so no GEMM workgroup renormalises the rows. The out-projection,
// the FFN, the velocity (last layer's stream) and the Euler step are
// readings: the pages give no layer glue.
//
// Everything is enqueued on one stream with no host synchronisation and no
// allocation, so a caller can capture the whole step in a graph and replay
// it while frames are pushed into the ring between replays.

#include "gemm.h"

namespace pa {

struct StackWs {
    size_t h, y, q, k, v, o, attn, part, ffn, total;
};

// the out-projection runs split over K when Hq * D allows it (always on
// packed weights); otherwise the unpacked path falls back to oproj_residual
static bool oproj_split(const Ring* r, const pa_stack* st) {
    return residual_splitk_supported(st->n_q_heads * r->cfg.head_dim, st->model_dim);
}

static StackWs stack_layout(const Ring* r, const pa_stack* st, size_t attn_bytes) {
    const size_t n = st->rows, m = st->model_dim, d = r->cfg.head_dim, hkv = r->cfg.num_kv_heads;
    StackWs w;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += align_up(bytes, 256);
        return at;
    };
    w.h = take(n * m * 2);
    // the normalised operand of the next QKV or gate/up GEMM (packed: 64 row slots)
    w.y = take((st->packed ? 64 : n) * m * 2);
    // packed Q (operand order) pads each KV head's rows to whole 32-row blocks
    const size_t qpk = st->packed ? (size_t)qpack_blocks(st->rows, st->n_q_heads, (int)hkv) * 32 * hkv * d : 0;
    w.q = take((qpk > n * st->n_q_heads * d ? qpk : n * st->n_q_heads * d) * 2);
    w.k = take(n * hkv * d * 2);
    w.v = take(n * hkv * d * 2);
    // packed activations always span the 64 row slots of the operand
    w.o = take((st->packed ? 64 : n) * st->n_q_heads * d * 2);
    w.attn = take(attn_bytes);
    // FP32 partials of the split-K out-projection
    w.part = take(oproj_split(r, st) ? residual_splitk_bytes(st->rows, st->n_q_heads * (int)d, st->model_dim) : 0);
    // SwiGLU activation (packed: 64 row slots), then the down projection's split-K partials
    w.ffn = take(st->ffn_dim ? align_up((size_t)(st->packed ? 64 : n) * st->ffn_dim * 2, 256) +
                                   residual_splitk_bytes(st->rows, st->ffn_dim, st->model_dim)
                             : 0);
    w.total = off;
    return w;
}

static pa_status check_stack(const Ring* r, const pa_stack* st) {
    PA_CHECK_ARG(r && st && st->w_qkv && st->w_o, PA_EINVAL, "pa_denoise_step: null argument");
    PA_CHECK_ARG(r->cfg.dtype == PA_BF16, PA_EINVAL, "pa_denoise_step: the stack runs on a bf16 ring");
    PA_CHECK_ARG(st->num_layers >= 1 && st->num_layers <= r->cfg.num_layers, PA_ESHAPE,
                 "pa_denoise_step: %d layers but the ring has %d", st->num_layers, r->cfg.num_layers);
    PA_CHECK_ARG(st->rows >= 1 && st->rows <= 64, PA_ESHAPE, "pa_denoise_step: rows %d not in [1, 64]", st->rows);
    PA_CHECK_ARG(st->model_dim % 128 == 0 && st->model_dim >= 256 && st->model_dim <= 2048, PA_ESHAPE,
                 "pa_denoise_step: model_dim must be a multiple of 128 in [256, 2048]");
    PA_CHECK_ARG(st->n_q_heads >= 1 && st->n_q_heads % r->cfg.num_kv_heads == 0, PA_ESHAPE,
                 "pa_denoise_step: n_q_heads must be a multiple of num_kv_heads");
    PA_CHECK_ARG((st->n_q_heads * r->cfg.head_dim) % 256 == 0, PA_ESHAPE,
                 "pa_denoise_step: n_q_heads * head_dim must be a multiple of 256");
    if (st->ffn_dim) {
        PA_CHECK_ARG(st->w_gate && st->w_up && st->w_down, PA_EINVAL, "pa_denoise_step: null FFN weights");
        PA_CHECK_ARG(ffn_swiglu_workspace_bytes(st->rows, st->model_dim, st->ffn_dim) > 0, PA_ESHAPE,
                     "pa_denoise_step: FFN needs model_dim 128 x {2, 4, 6, 8} and ffn_dim 1024 x {1, 2, 3, 4, 6, 8}");
    }
    PA_CHECK_ARG(st->packed == 0 || st->packed == 1, PA_EINVAL, "pa_denoise_step: packed must be 0 or 1");
    if (st->packed) {
        PA_CHECK_ARG(packed_norm_supported(st->model_dim), PA_ESHAPE,
                     "pa_denoise_step: packed weights need model_dim 512 or 1024 (got %d)", st->model_dim);
        PA_CHECK_ARG(packed_residual_supported(st->n_q_heads * r->cfg.head_dim, st->model_dim), PA_ESHAPE,
                     "pa_denoise_step: packed weights need Hq * D = 1024 x {1, 2, 3, 4, 6, 8}");
        PA_CHECK_ARG(!st->ffn_dim || packed_residual_supported(st->ffn_dim, st->model_dim), PA_ESHAPE,
                     "pa_denoise_step: packed weights need ffn_dim = 1024 x {1, 2, 3, 4, 6, 8}");
        const void* ws[5] = {st->w_qkv, st->w_o, st->w_gate, st->w_up, st->w_down};
        for (int i = 0; i < (st->ffn_dim ? 5 : 2); ++i)
            PA_CHECK_ARG(aligned16(ws[i]), PA_EINVAL, "pa_denoise_step: packed weights must be 16-byte aligned");
    }
    return PA_OK;
}

static pattn_args attn_args(const pa_stack* st, int layer) {
    pattn_args a;
    a.layer_begin = layer;
    a.num_layers = 1;
    a.n_q_heads = st->n_q_heads;
    a.n_dyn = st->rows;
    a.scale = st->scale;
    a.out_dtype = PA_BF16;
    a.num_splits = st->num_splits;
    a.q_layout = PA_Q_TOKEN_MAJOR;       // the packed path passes its operand-order Q internally
    a.partials_f32 = 0;
    return a;
}

}  // namespace pa

using namespace pa;

extern "C" size_t pa_denoise_step_workspace_bytes(const rb_ring* ring, const pa_stack* st) {
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    if (check_stack(r, st) != PA_OK) return 0;
    const pattn_args a = attn_args(st, 0);
    const size_t attn = pattn_workspace_bytes(ring, &a);
    if (!attn) return 0;
    return stack_layout(r, st, attn).total;
}

extern "C" pa_status pa_denoise_step(const rb_ring* ring, const pa_stack* st, void* x, const float* gamma,
                                     const float* gamma_ffn, int64_t gamma_layer_stride, uint32_t* nonfinite,
                                     void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    pa_status s = check_stack(r, st);
    if (s != PA_OK) return s;
    PA_CHECK_ARG(x && gamma && ws && (gamma_ffn || !st->ffn_dim), PA_EINVAL, "pa_denoise_step: null argument");
    PA_CHECK_ARG(gamma_layer_stride >= st->model_dim, PA_ESHAPE, "pa_denoise_step: gamma stride below model_dim");
    const pattn_args a0 = attn_args(st, 0);
    const size_t attn = pattn_workspace_bytes(ring, &a0);
    PA_CHECK_ARG(attn > 0, PA_ESHAPE, "pa_denoise_step: attention arguments rejected");
    const StackWs w = stack_layout(r, st, attn);
    PA_CHECK_ARG(ws_bytes >= w.total, PA_ERANGE, "pa_denoise_step: workspace %zu < %zu bytes", ws_bytes, w.total);
    char* base = static_cast<char*>(ws);
    void *h = base + w.h, *y = base + w.y, *q = base + w.q, *k = base + w.k, *v = base + w.v, *o = base + w.o;
    void* aws = base + w.attn;
    float* opart = reinterpret_cast<float*>(base + w.part);
    const bool osplit = oproj_split(r, st);
    void* fws = base + w.ffn;
    hipStream_t strm = static_cast<hipStream_t>(stream);
    const int d = r->cfg.head_dim, hkv = r->cfg.num_kv_heads;
    const int in_dim = st->n_q_heads * d;
    const size_t wqkv_layer = (size_t)(st->n_q_heads + 2 * hkv) * d * st->model_dim;
    const size_t wo_layer = (size_t)st->model_dim * in_dim;
    const size_t wf_layer = (size_t)st->ffn_dim * st->model_dim;
    void* act = fws;
    float* fpart = reinterpret_cast<float*>(static_cast<char*>(fws) +
                                            align_up((size_t)(st->packed ? 64 : st->rows) * st->ffn_dim * 2, 256));
    const bool pk = st->packed != 0;
    // Every GEMM that starts from h reads y = bf16(AdaRMSNorm(h)), formed by
    // the kernel that finished h (the first layer's by a norm pass that also
    // copies x into h), in the GEMM's own operand layout. Packed and unpacked
    // weights run the same normalisation and the same summation orders, so
    // their x agree bit for bit.
    auto norm_of = [&](const float* g) { return NormNext{g, st->eps, y, pk}; };
    NormNext nn = norm_of(gamma);
    s = norm_rows(x, h, st->rows, st->model_dim, nn, nonfinite, strm);
    if (s != PA_OK) return s;
    for (int l = 0; l < st->num_layers; ++l) {
        const bool last = l + 1 == st->num_layers;
        const uint16_t* wq = static_cast<const uint16_t*>(st->w_qkv) + l * wqkv_layer;
        const uint16_t* wo = static_cast<const uint16_t*>(st->w_o) + l * wo_layer;
        s = pk ? packed_qkv(y, st->rows, st->model_dim, wq, st->n_q_heads, hkv, d, q, k, v, true, strm)
               : qkv_proj(y, st->rows, st->model_dim, wq, st->n_q_heads, hkv, d, q, k, v, strm);
        if (s != PA_OK) return s;
        const pattn_args a = attn_args(st, l);
        s = pk ? pattn_step_apacked(ring, &a, q, k, v, o, aws, attn, stream, true)
               : pattn_step(ring, &a, q, k, v, o, aws, attn, stream);
        if (s != PA_OK) return s;
        // the out-projection's residual forms the FFN's operand, or the next
        // layer's, and applies the Euler update after the last projection
        const float* g_next = st->ffn_dim ? gamma_ffn + l * gamma_layer_stride
                                          : (last ? nullptr : gamma + (l + 1) * gamma_layer_stride);
        nn = norm_of(g_next);
        void* xl = last && !st->ffn_dim ? x : nullptr;
        if (osplit) {
            s = residual_splitk(o, wo, pk, h, st->rows, in_dim, st->model_dim, xl, st->dt, nonfinite, opart, strm,
                                g_next ? &nn : nullptr);
        } else {   // unpacked weights only: single-kernel out-projection, then the norm in place
            s = oproj_residual(o, wo, h, st->rows, in_dim, st->model_dim, xl, st->dt, nonfinite, stream);
            if (s == PA_OK && g_next) s = norm_rows(h, h, st->rows, st->model_dim, nn, nonfinite, strm);
        }
        if (s != PA_OK) return s;
        if (st->ffn_dim) {
            const uint16_t* wg = static_cast<const uint16_t*>(st->w_gate) + l * wf_layer;
            const uint16_t* wu = static_cast<const uint16_t*>(st->w_up) + l * wf_layer;
            const uint16_t* wd = static_cast<const uint16_t*>(st->w_down) + l * wf_layer;
            s = pk ? packed_gateup(y, st->rows, st->model_dim, st->ffn_dim, wg, wu, act, strm)
                   : gateup_proj(y, st->rows, st->model_dim, st->ffn_dim, wg, wu, act, strm);
            if (s != PA_OK) return s;
            const float* g2 = last ? nullptr : gamma + (l + 1) * gamma_layer_stride;
            nn = norm_of(g2);
            s = residual_splitk(act, wd, pk, h, st->rows, st->ffn_dim, st->model_dim, last ? x : nullptr, st->dt,
                                nonfinite, fpart, strm, g2 ? &nn : nullptr);
            if (s != PA_OK) return s;
        }
    }
    return PA_OK;
}
