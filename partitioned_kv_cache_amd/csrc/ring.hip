// Static ring-buffer KV cache: handle, pinned prefix, frame push.
//
// "Reflex: Real-Time VLA Control through Streaming Inference" paper review,
// §3 Architecture (ring-buffer diagram: a pinned prefix, then a FIFO window
// where every frame enqueues the newest frame and evicts the oldest; the
// component table gives buffer_k as num_layers x max_seq_len x num_heads x
// head_dim) and §5 Code analysis (the buffers are allocated zeroed, once,
// beside a write pointer that starts at 0).
//
// The buffers are the caller's. A push is one strided device-to-device copy
// of the frame's [L][F][Hkv][D] block into slot `head` of every layer; only
// host metadata changes otherwise. Nothing is ever allocated or moved. A
// captured attention launch reads the window length and (on a spare-slot
// ring) its position as they were when it was enqueued, so capture is
// allowed only where neither can change under a replay: the window must be
// full, and a spare-slot ring must keep its head in a bound device state
// word, which the kernels read when they run (rb_bind_state_word). The calls
// that change the ring's host metadata cannot be captured at all.

#include <stdarg.h>

#include <algorithm>
#include <new>

#include "internal.h"

namespace pa {

static thread_local char g_err[512] = "";

pa_status fail(pa_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

void clear_error() { g_err[0] = 0; }

pa_status stream_capturing(hipStream_t stream, bool* capturing) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    // A runtime that cannot answer (no device) cannot be capturing either;
    // the call's own launches then report the device error.
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        cs = hipStreamCaptureStatusNone;
    }
    *capturing = cs != hipStreamCaptureStatusNone;
    return PA_OK;
}

pa_status check_capture(const Ring* r, hipStream_t stream, const char* who) {
    bool cap = false;
    pa_status st = stream_capturing(stream, &cap);
    if (st != PA_OK || !cap) return st;
    PA_CHECK_ARG(r->count == r->cfg.num_slots, PA_ESTATE,
                 "%s: capture needs a full window (%d of %d frames): a replay after the next push would read a "
                 "stale window length", who, r->count, r->cfg.num_slots);
    PA_CHECK_ARG(!r->cfg.spare_slots || r->state_word, PA_ESTATE,
                 "%s: capture on a spare-slot ring needs a bound state word (rb_bind_state_word): a replay after "
                 "the next commit would read a stale window position", who);
    return PA_OK;
}

// The calls that change host metadata at enqueue time cannot be captured.
static pa_status refuse_capture(hipStream_t stream, const char* who) {
    bool cap = false;
    pa_status st = stream_capturing(stream, &cap);
    if (st != PA_OK) return st;
    PA_CHECK_ARG(!cap, PA_ESTATE, "%s: changes the ring's host metadata when enqueued and cannot be captured", who);
    return PA_OK;
}

// One thread writes the ring's state word {head, count, pinned, 0} (a
// vector store; 16-byte aligned).
__global__ void write_state_word(int4* w, int head, int count, int pinned) {
    *w = make_int4(head, count, pinned, 0);
}

static pa_status publish_state(Ring* r, hipStream_t s) {
    if (!r->state_word) return PA_OK;
    write_state_word<<<1, 1, 0, s>>>(reinterpret_cast<int4*>(r->state_word), r->head, r->count, r->pinned);
    PA_LAUNCHED();
    return PA_OK;
}

static pa_status ensure_events(Ring* r) {
    if (!r->ev_staged) {
        PA_HIP(hipEventCreateWithFlags(&r->ev_staged, hipEventDisableTiming));
        PA_HIP(hipEventCreateWithFlags(&r->ev_free, hipEventDisableTiming));
    }
    return PA_OK;
}

// A spare-slot ring's next spare (slot `head`) may still be read by steps
// enqueued on `s` before this point: the next rb_stage_frame waits for them.
static pa_status fence_spare(Ring* r, hipStream_t s) {
    if (!r->cfg.spare_slots) return PA_OK;
    pa_status st = ensure_events(r);
    if (st != PA_OK) return st;
    PA_HIP(hipEventRecord(r->ev_free, s));
    r->free_recorded = true;
    return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" const char* pa_last_error(void) { return pa::g_err; }

extern "C" pa_status rb_create(const rb_config* cfg, void* k_buf, void* v_buf, rb_ring** out) {
    clear_error();
    PA_CHECK_ARG(cfg && k_buf && v_buf && out, PA_EINVAL, "rb_create: null argument");
    PA_CHECK_ARG(cfg->dtype == PA_F32 || cfg->dtype == PA_BF16, PA_EINVAL, "rb_create: bad dtype %d", cfg->dtype);
    PA_CHECK_ARG(cfg->num_layers > 0 && cfg->num_kv_heads > 0 && cfg->head_dim > 0 && cfg->num_slots > 0 &&
                     cfg->tokens_per_frame > 0 && cfg->pin_capacity >= 0,
                 PA_ESHAPE, "rb_create: sizes must be positive (pin capacity >= 0)");
    PA_CHECK_ARG(cfg->head_dim == 32 || cfg->head_dim == 64 || cfg->head_dim == 128 || cfg->head_dim == 256,
                 PA_ESHAPE, "rb_create: head_dim %d must be 32, 64, 128 or 256", cfg->head_dim);
    PA_CHECK_ARG(cfg->spare_slots == 0 || cfg->spare_slots == 1, PA_EINVAL, "rb_create: spare_slots %d must be 0 or 1",
                 cfg->spare_slots);
    int64_t seq = (int64_t)cfg->pin_capacity + (int64_t)(cfg->num_slots + cfg->spare_slots) * cfg->tokens_per_frame;
    PA_CHECK_ARG(seq * cfg->num_kv_heads * cfg->head_dim < (1LL << 31), PA_ESHAPE,
                 "rb_create: (P + W*F) * Hkv * D must stay below 2^31 elements per layer");
    Ring* r = new (std::nothrow) Ring();
    PA_CHECK_ARG(r, PA_EINVAL, "rb_create: out of host memory");
    r->cfg = *cfg;
    r->k = k_buf;
    r->v = v_buf;
    *out = reinterpret_cast<rb_ring*>(r);
    return PA_OK;
}

extern "C" pa_status rb_destroy(rb_ring* ring) {
    clear_error();
    Ring* r = reinterpret_cast<Ring*>(ring);
    if (r) {
        if (r->ev_staged) (void)hipEventDestroy(r->ev_staged);
        if (r->ev_free) (void)hipEventDestroy(r->ev_free);
    }
    delete r;
    return PA_OK;
}

// Copy [L][n][Hkv][D] (contiguous) into tokens [tok0, tok0 + n) of every layer.
static pa_status copy_tokens(Ring* r, void* dst_base, const void* src, int64_t tok0, int64_t n, hipStream_t s) {
    const int64_t tok_bytes = (int64_t)r->cfg.num_kv_heads * r->cfg.head_dim * r->elem_bytes();
    const size_t width = (size_t)(n * tok_bytes);
    const size_t dpitch = (size_t)(r->seq_len() * tok_bytes);
    char* dst = static_cast<char*>(dst_base) + tok0 * tok_bytes;
    PA_HIP(hipMemcpy2DAsync(dst, dpitch, src, width, width, (size_t)r->cfg.num_layers, hipMemcpyDeviceToDevice, s));
    return PA_OK;
}

// Workgroup (x, 2 l + t) of copy_kv_runs moves words [x * 1024, x * 1024 +
// 1024) of tensor t's run in layer l, four per thread, all four loaded before
// any is stored (a word past the run re-reads word 0 and is not stored). The
// source is read once, so its loads are non-temporal; the stores stay cached
// for the steps that read them next.
constexpr int COPY_THREADS = 256, COPY_WORDS = 4;

__global__ __launch_bounds__(COPY_THREADS) void pa::copy_kv_runs(RunCopy c) {
    const int t = blockIdx.y & 1, l = blockIdx.y >> 1;
    const word16* src = (t ? c.src[1] : c.src[0]) + (long long)l * c.run;
    word16* dst = (t ? c.dst[1] : c.dst[0]) + (long long)l * c.dst_stride;
    const long long base = (long long)blockIdx.x * (COPY_THREADS * COPY_WORDS) + threadIdx.x;
    word16 w[COPY_WORDS];
#pragma unroll
    for (int u = 0; u < COPY_WORDS; ++u) {
        const long long i = base + u * COPY_THREADS;
        w[u] = __builtin_nontemporal_load(src + (i < c.run ? i : 0));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < COPY_WORDS; ++u) {
        const long long i = base + u * COPY_THREADS;
        if (i < c.run) dst[i] = w[u];
    }
}

// tokens [tok0, tok0 + n) of every layer of both tensors from contiguous
// [L][n][Hkv][D] sources; the 2-D copy engine path when a source is not
// 16-byte aligned
static pa_status copy_kv_tokens(Ring* r, const void* k, const void* v, int64_t tok0, int64_t n, hipStream_t s) {
    const int64_t tok_bytes = (int64_t)r->cfg.num_kv_heads * r->cfg.head_dim * r->elem_bytes();
    if (!aligned16(k) || !aligned16(v) || (n * tok_bytes) % 16 != 0 || tok_bytes % 16 != 0 ||
        !aligned16(r->k) || !aligned16(r->v)) {
        pa_status st = copy_tokens(r, r->k, k, tok0, n, s);
        if (st != PA_OK) return st;
        return copy_tokens(r, r->v, v, tok0, n, s);
    }
    RunCopy c;
    c.src[0] = static_cast<const word16*>(k);
    c.src[1] = static_cast<const word16*>(v);
    c.dst[0] = reinterpret_cast<word16*>(static_cast<char*>(r->k) + tok0 * tok_bytes);
    c.dst[1] = reinterpret_cast<word16*>(static_cast<char*>(r->v) + tok0 * tok_bytes);
    c.run = n * tok_bytes / 16;
    c.dst_stride = r->seq_len() * tok_bytes / 16;
    const long long per_block = (long long)COPY_THREADS * COPY_WORDS;
    const dim3 grid((unsigned)((c.run + per_block - 1) / per_block), 2u * (unsigned)r->cfg.num_layers);
    copy_kv_runs<<<grid, COPY_THREADS, 0, s>>>(c);
    PA_LAUNCHED();
    return PA_OK;
}

extern "C" pa_status rb_pin_prefix(rb_ring* ring, const void* k, const void* v, int32_t n_tokens, void* stream) {
    clear_error();
    Ring* r = reinterpret_cast<Ring*>(ring);
    PA_CHECK_ARG(r && k && v, PA_EINVAL, "rb_pin_prefix: null argument");
    PA_CHECK_ARG(r->pinned == 0, PA_ESTATE, "rb_pin_prefix: prefix already pinned (%d tokens)", r->pinned);
    PA_CHECK_ARG(n_tokens > 0 && n_tokens <= r->cfg.pin_capacity, PA_ESHAPE,
                 "rb_pin_prefix: n_tokens %d not in [1, %d]", n_tokens, r->cfg.pin_capacity);
    hipStream_t s = static_cast<hipStream_t>(stream);
    pa_status st = refuse_capture(s, "rb_pin_prefix");
    if (st != PA_OK) return st;
    st = copy_kv_tokens(r, k, v, 0, n_tokens, s);
    if (st != PA_OK) return st;
    r->pinned = n_tokens;
    return publish_state(r, s);
}

// Copy a frame into slot `head` of every layer.
static pa_status write_head_slot(Ring* r, const void* k, const void* v, hipStream_t s) {
    const int64_t tok0 = (int64_t)r->cfg.pin_capacity + (int64_t)r->head * r->cfg.tokens_per_frame;
    return copy_kv_tokens(r, k, v, tok0, r->cfg.tokens_per_frame, s);
}

// The frame in slot `head` joins the window; the oldest leaves it.
static int64_t advance(Ring* r) {
    const int W = r->cfg.num_slots;
    const int64_t ev = r->frames_pushed >= W ? r->frames_pushed - W : -1;
    r->frames_pushed += 1;
    r->head = (int32_t)(r->frames_pushed % r->phys_slots());
    r->count = r->count < W ? r->count + 1 : W;
    return ev;
}

extern "C" pa_status rb_push_frame(rb_ring* ring, const void* k, const void* v, void* stream, int64_t* evicted) {
    clear_error();
    Ring* r = reinterpret_cast<Ring*>(ring);
    PA_CHECK_ARG(r && k && v, PA_EINVAL, "rb_push_frame: null argument");
    PA_CHECK_ARG(!r->staged, PA_ESTATE, "rb_push_frame: a staged frame is pending; commit it first");
    hipStream_t s = static_cast<hipStream_t>(stream);
    pa_status st = refuse_capture(s, "rb_push_frame");
    if (st != PA_OK) return st;
    st = write_head_slot(r, k, v, s);
    if (st != PA_OK) return st;
    const int64_t ev = advance(r);
    st = fence_spare(r, s);
    if (st == PA_OK) st = publish_state(r, s);
    if (st != PA_OK) return st;
    if (evicted) *evicted = ev;
    return PA_OK;
}

extern "C" pa_status rb_stage_frame(rb_ring* ring, const void* k, const void* v, void* stream) {
    clear_error();
    Ring* r = reinterpret_cast<Ring*>(ring);
    PA_CHECK_ARG(r && k && v, PA_EINVAL, "rb_stage_frame: null argument");
    PA_CHECK_ARG(r->cfg.spare_slots == 1, PA_ESTATE, "rb_stage_frame: the ring has no spare slot");
    PA_CHECK_ARG(!r->staged, PA_ESTATE, "rb_stage_frame: a staged frame is already pending");
    hipStream_t s = static_cast<hipStream_t>(stream);
    pa_status st = refuse_capture(s, "rb_stage_frame");
    if (st != PA_OK) return st;
    st = ensure_events(r);
    if (st != PA_OK) return st;
    if (r->free_recorded) PA_HIP(hipStreamWaitEvent(s, r->ev_free, 0));
    st = write_head_slot(r, k, v, s);
    if (st != PA_OK) return st;
    PA_HIP(hipEventRecord(r->ev_staged, s));
    r->staged = true;
    return PA_OK;
}

extern "C" pa_status rb_commit_frame(rb_ring* ring, void* stream, int64_t* evicted) {
    clear_error();
    Ring* r = reinterpret_cast<Ring*>(ring);
    PA_CHECK_ARG(r, PA_EINVAL, "rb_commit_frame: null argument");
    PA_CHECK_ARG(r->staged, PA_ESTATE, "rb_commit_frame: no staged frame");
    hipStream_t s = static_cast<hipStream_t>(stream);
    pa_status st = refuse_capture(s, "rb_commit_frame");
    if (st != PA_OK) return st;
    // Everything enqueued on the consumer so far may read the slot this
    // commit frees (the oldest of the window): the next stage waits for it.
    PA_HIP(hipEventRecord(r->ev_free, s));
    PA_HIP(hipStreamWaitEvent(s, r->ev_staged, 0));
    r->free_recorded = true;
    r->staged = false;
    const int64_t ev = advance(r);
    st = publish_state(r, s);
    if (st != PA_OK) return st;
    if (evicted) *evicted = ev;
    return PA_OK;
}

extern "C" pa_status rb_bind_state_word(rb_ring* ring, int32_t* state_word, void* stream) {
    clear_error();
    Ring* r = reinterpret_cast<Ring*>(ring);
    PA_CHECK_ARG(r, PA_EINVAL, "rb_bind_state_word: null ring");
    PA_CHECK_ARG(aligned16(state_word), PA_EINVAL, "rb_bind_state_word: the state word must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    pa_status st = refuse_capture(s, "rb_bind_state_word");
    if (st != PA_OK) return st;
    r->state_word = state_word;
    return publish_state(r, s);
}

extern "C" pa_status rb_get_state(const rb_ring* ring, rb_state* out) {
    clear_error();
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    PA_CHECK_ARG(r && out, PA_EINVAL, "rb_get_state: null argument");
    out->head = r->head;
    out->count = r->count;
    out->pinned = r->pinned;
    out->reserved = 0;
    out->frames_pushed = r->frames_pushed;
    return PA_OK;
}

// ---------------------------------------------------------------------------
// Capsules: FlashRT article (PaperDaily, "FlashRT开源：27倍加速…"), the
// section on what a capsule is and Fig. 2 (snapshot, restore, fork and
// rollback as operations on a set of static buffers). For this ring the live
// state at a frame boundary is the valid K/V region plus (head, count,
// pinned, frames_pushed). A capsule stores that region compactly, K then V,
// each [L][pinned + count * F][Hkv][D]: the pinned tokens of a layer, then
// its first count slots (the slots a ring fills before it wraps, or all of
// them once full).

static int64_t capsule_tokens(const Ring* r) { return (int64_t)r->pinned + (int64_t)r->count * r->cfg.tokens_per_frame; }

static size_t capsule_bytes_of(const Ring* r, int64_t ctok) {
    return (size_t)(2 * r->cfg.num_layers * ctok * r->cfg.num_kv_heads * r->cfg.head_dim * r->elem_bytes());
}

// Copy the valid region between the ring (layer pitch P + S*F tokens) and a
// capsule (layer pitch ctok tokens), one 2-D copy per run and tensor: the
// pinned tokens, then the window's slots in physical order, which with a
// spare slot form up to two runs around slot `head`.
static pa_status capsule_copy(Ring* r, char* cap, int32_t pinned, int64_t count, int32_t head, bool to_capsule,
                              hipStream_t s) {
    const int64_t F = r->cfg.tokens_per_frame, P = r->cfg.pin_capacity;
    const int64_t tok = (int64_t)r->cfg.num_kv_heads * r->cfg.head_dim * r->elem_bytes();
    const int64_t ctok = pinned + count * F;
    const size_t rpitch = (size_t)(r->seq_len() * tok), cpitch = (size_t)(ctok * tok);
    const size_t layers = (size_t)r->cfg.num_layers;
    const int64_t n_win = count * F;
    const int64_t skip = r->cfg.spare_slots ? (int64_t)head * F : n_win;   // window tokens before the spare
    const int64_t run1 = skip < n_win ? skip : n_win;
    for (int t = 0; t < 2; ++t) {
        char* ring = static_cast<char*>(t == 0 ? r->k : r->v);
        char* c = cap + (size_t)t * layers * cpitch;
        struct { int64_t ring_tok, cap_tok, n; } reg[3] = {
            {0, 0, pinned}, {P, pinned, run1}, {P + run1 + F, pinned + run1, n_win - run1}};
        for (const auto& g : reg) {
            if (g.n == 0) continue;
            char* rp = ring + g.ring_tok * tok;
            char* cp = c + g.cap_tok * tok;
            const size_t w = (size_t)(g.n * tok);
            if (to_capsule)
                PA_HIP(hipMemcpy2DAsync(cp, cpitch, rp, rpitch, w, layers, hipMemcpyDefault, s));
            else
                PA_HIP(hipMemcpy2DAsync(rp, rpitch, cp, cpitch, w, layers, hipMemcpyDefault, s));
        }
    }
    return PA_OK;
}

extern "C" size_t rb_capsule_bytes(const rb_ring* ring) {
    clear_error();
    const Ring* r = reinterpret_cast<const Ring*>(ring);
    return r ? capsule_bytes_of(r, capsule_tokens(r)) : 0;
}

extern "C" pa_status rb_snapshot(const rb_ring* ring, void* capsule, size_t capsule_bytes, rb_state* state,
                                 void* stream) {
    clear_error();
    Ring* r = const_cast<Ring*>(reinterpret_cast<const Ring*>(ring));
    PA_CHECK_ARG(r && state, PA_EINVAL, "rb_snapshot: null argument");
    const size_t need = capsule_bytes_of(r, capsule_tokens(r));
    PA_CHECK_ARG(capsule || need == 0, PA_EINVAL, "rb_snapshot: null capsule");
    PA_CHECK_ARG(capsule_bytes >= need, PA_ERANGE, "rb_snapshot: capsule %zu bytes < %zu needed", capsule_bytes, need);
    pa_status st = refuse_capture(static_cast<hipStream_t>(stream), "rb_snapshot");
    if (st != PA_OK) return st;
    st = capsule_copy(r, static_cast<char*>(capsule), r->pinned, r->count, r->head, true,
                      static_cast<hipStream_t>(stream));
    if (st != PA_OK) return st;
    return rb_get_state(ring, state);
}

extern "C" pa_status rb_restore(rb_ring* ring, const void* capsule, size_t capsule_bytes, const rb_state* state,
                                void* stream) {
    clear_error();
    Ring* r = reinterpret_cast<Ring*>(ring);
    PA_CHECK_ARG(r && state, PA_EINVAL, "rb_restore: null argument");
    PA_CHECK_ARG(!r->staged, PA_ESTATE, "rb_restore: a staged frame is pending; commit it first");
    const int W = r->cfg.num_slots;
    const int64_t fp = state->frames_pushed;
    PA_CHECK_ARG(state->pinned >= 0 && state->pinned <= r->cfg.pin_capacity, PA_EINVAL,
                 "rb_restore: pinned %d not in [0, %d]", state->pinned, r->cfg.pin_capacity);
    PA_CHECK_ARG(fp >= 0 && state->count == (fp < W ? fp : W) && state->head == (int32_t)(fp % r->phys_slots()), PA_EINVAL,
                 "rb_restore: state (head %d, count %d, frames_pushed %lld) is not one a ring of %d slots reaches",
                 state->head, state->count, (long long)fp, W);
    const size_t need = capsule_bytes_of(r, state->pinned + (int64_t)state->count * r->cfg.tokens_per_frame);
    PA_CHECK_ARG(capsule || need == 0, PA_EINVAL, "rb_restore: null capsule");
    PA_CHECK_ARG(capsule_bytes >= need, PA_ERANGE, "rb_restore: capsule %zu bytes < %zu needed", capsule_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    pa_status st = refuse_capture(s, "rb_restore");
    if (st != PA_OK) return st;
    st = capsule_copy(r, const_cast<char*>(static_cast<const char*>(capsule)), state->pinned, state->count,
                      state->head, false, s);
    if (st != PA_OK) return st;
    r->head = state->head;
    r->count = state->count;
    r->pinned = state->pinned;
    r->frames_pushed = fp;
    st = fence_spare(r, s);
    if (st != PA_OK) return st;
    return publish_state(r, s);
}

