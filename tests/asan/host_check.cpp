// Host-side checks of the library's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer, on a machine without a GPU: the library's host
// code (ring metadata, pin / push / staging, capsules, the state word,
// capture refusals, argument validation and launch planning) runs against a
// host-memory double of the HIP runtime (hip_host_double.cpp), with every
// "device" buffer in host memory. Ring bytes are checked against an
// independent model written here: frame f of a ring with S physical slots
// sits in slot f mod S, the pin occupies tokens [0, pinned).
//
// Prints one line per failed check and exits with the number of failures.

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/pattn.h"
#include "hip_host_double.h"

static int g_fail = 0;
#define CHECK(cond, ...)                                         \
    do {                                                         \
        if (!(cond)) {                                           \
            ++g_fail;                                            \
            printf("FAIL %s:%d: ", __FILE__, __LINE__);          \
            printf(__VA_ARGS__);                                 \
            printf(" [%s]\n", pa_last_error());                  \
        }                                                        \
    } while (0)

// 256-byte aligned, zeroed host buffer standing in for device memory
struct Buf {
    void* p = nullptr;
    size_t n = 0;
    explicit Buf(size_t bytes) : n(bytes) {
        const size_t r = (bytes + 255) / 256 * 256;
        p = aligned_alloc(256, r ? r : 256);
        memset(p, 0, r ? r : 256);
    }
    ~Buf() { free(p); }
    Buf(const Buf&) = delete;
    Buf& operator=(const Buf&) = delete;
    template <typename T> T* as() const { return static_cast<T*>(p); }
};

static uint16_t word(int tag, int f, int l, int t, int d) {
    return (uint16_t)((tag * 7919 + f * 1009 + l * 101 + t * 13 + d * 3 + 1) & 0xffff);
}

// frame f's K (tag 1) or V (tag 2): [L][F][1][D]
static void fill_frame(Buf& b, int tag, int f, int L, int F, int D) {
    for (int l = 0; l < L; ++l)
        for (int t = 0; t < F; ++t)
            for (int d = 0; d < D; ++d) b.as<uint16_t>()[((size_t)l * F + t) * D + d] = word(tag, f, l, t, d);
}

struct Model {
    int L, P, S, F, D, W;
    int pinned = 0;
    std::vector<int> slot_frame;   // frame held by each physical slot, -1 if none
    Model(int l, int p, int w, int spare, int f, int d) : L(l), P(p), S(w + spare), F(f), D(d), W(w), slot_frame(S, -1) {}
    // expected word at (layer, token, dim) of the K (tag 1) or V (tag 2) buffer
    uint16_t at(int tag, int l, int tok, int d) const {
        if (tok < P) return tok < pinned ? word(tag + 10, 0, l, tok, d) : 0;
        const int s = (tok - P) / F, t = (tok - P) % F;
        return slot_frame[s] < 0 ? 0 : word(tag, slot_frame[s], l, t, d);
    }
};

static int compare_ring(const Model& m, const Buf& k, const Buf& v) {
    int bad = 0;
    const int seq = m.P + m.S * m.F;
    for (int l = 0; l < m.L; ++l)
        for (int tok = 0; tok < seq; ++tok)
            for (int d = 0; d < m.D; ++d) {
                const size_t i = ((size_t)l * seq + tok) * m.D + d;
                bad += k.as<uint16_t>()[i] != m.at(1, l, tok, d);
                bad += v.as<uint16_t>()[i] != m.at(2, l, tok, d);
            }
    return bad;
}

static void test_ring(int spare) {
    const int L = 2, D = 32, P = 4, W = 3, F = 2, S = W + spare;
    const size_t seq = P + (size_t)S * F;
    Buf kb(L * seq * D * 2), vb(L * seq * D * 2);
    rb_config cfg = {L, 1, D, P, W, F, PA_BF16, spare};
    rb_ring* r = nullptr;
    CHECK(rb_create(&cfg, kb.p, vb.p, &r) == PA_OK && r, "rb_create");
    Model m(L, P, W, spare, F, D);
    Buf pk(L * 3 * D * 2), pv(L * 3 * D * 2);
    for (int l = 0; l < L; ++l)
        for (int t = 0; t < 3; ++t)
            for (int d = 0; d < D; ++d) {
                pk.as<uint16_t>()[(l * 3 + t) * D + d] = word(11, 0, l, t, d);
                pv.as<uint16_t>()[(l * 3 + t) * D + d] = word(12, 0, l, t, d);
            }
    CHECK(rb_pin_prefix(r, pk.p, pv.p, 3, nullptr) == PA_OK, "pin");
    CHECK(rb_pin_prefix(r, pk.p, pv.p, 3, nullptr) == PA_ESTATE, "second pin refused");
    m.pinned = 3;
    CHECK(compare_ring(m, kb, vb) == 0, "bytes after pin");
    Buf fk(L * F * D * 2), fv(L * F * D * 2);
    const int events0 = dbl::g.live_events;
    for (int f = 0; f < 11; ++f) {
        fill_frame(fk, 1, f, L, F, D);
        fill_frame(fv, 2, f, L, F, D);
        int64_t ev = -7;
        if (spare && f % 2) {       // alternate staged pushes with synchronous ones
            const long long waits = dbl::g.waits;
            CHECK(rb_stage_frame(r, fk.p, fv.p, nullptr) == PA_OK, "stage %d", f);
            CHECK(f < 2 || dbl::g.waits == waits + 1, "stage %d waits for the fence", f);
            CHECK(rb_push_frame(r, fk.p, fv.p, nullptr, nullptr) == PA_ESTATE, "push while staged refused");
            CHECK(rb_commit_frame(r, nullptr, &ev) == PA_OK, "commit %d", f);
        } else {
            const long long rec = dbl::g.records;
            CHECK(rb_push_frame(r, fk.p, fv.p, nullptr, &ev) == PA_OK, "push %d", f);
            CHECK(!spare || dbl::g.records == rec + 1, "push %d on a spare ring records the fence", f);
        }
        m.slot_frame[f % S] = f;
        CHECK(ev == (f >= W ? f - W : -1), "evicted id at frame %d: %lld", f, (long long)ev);
        rb_state st;
        CHECK(rb_get_state(r, &st) == PA_OK, "state");
        CHECK(st.head == (f + 1) % S && st.count == (f + 1 < W ? f + 1 : W) && st.pinned == 3 &&
                  st.frames_pushed == f + 1,
              "state after frame %d: head %d count %d", f, st.head, st.count);
        CHECK(compare_ring(m, kb, vb) == 0, "ring bytes after frame %d", f);
    }
    CHECK(!spare || dbl::g.live_events == events0 + 2, "a spare ring holds its two fence events");
    // capsule round trip: snapshot, two more frames, restore
    const size_t cb = rb_capsule_bytes(r);
    CHECK(cb == (size_t)2 * L * (3 + W * F) * D * 2, "capsule bytes %zu", cb);
    Buf cap(cb);
    rb_state snap;
    CHECK(rb_snapshot(r, cap.p, cb - 1, &snap, nullptr) == PA_ERANGE, "small capsule refused");
    CHECK(rb_snapshot(r, cap.p, cb, &snap, nullptr) == PA_OK, "snapshot");
    const std::vector<int> saved = m.slot_frame;
    for (int f = 11; f < 13; ++f) {
        fill_frame(fk, 1, f, L, F, D);
        fill_frame(fv, 2, f, L, F, D);
        CHECK(rb_push_frame(r, fk.p, fv.p, nullptr, nullptr) == PA_OK, "push %d", f);
        m.slot_frame[f % S] = f;
    }
    rb_state bad = snap;
    bad.head = (bad.head + 1) % S;
    CHECK(rb_restore(r, cap.p, cb, &bad, nullptr) == PA_EINVAL, "unreachable state refused");
    const long long rec = dbl::g.records;
    CHECK(rb_restore(r, cap.p, cb, &snap, nullptr) == PA_OK, "restore");
    CHECK(!spare || dbl::g.records == rec + 1, "restore on a spare ring records the fence");
    // the valid region is back; the slot outside it (the spare) keeps what it held
    const std::vector<int> cur = m.slot_frame;
    m.slot_frame = saved;
    if (spare) m.slot_frame[snap.head] = cur[snap.head];
    CHECK(compare_ring(m, kb, vb) == 0, "ring bytes after restore");
    rb_state st;
    rb_get_state(r, &st);
    CHECK(st.head == snap.head && st.count == snap.count && st.frames_pushed == snap.frames_pushed, "state restored");
    // state word: written on bind and on every push
    alignas(16) int32_t sw[4] = {-1, -1, -1, -1};
    long long writes = dbl::g.state_writes;
    CHECK(rb_bind_state_word(r, sw + 1, nullptr) == PA_EINVAL, "misaligned state word refused");
    CHECK(rb_bind_state_word(r, sw, nullptr) == PA_OK, "bind state word");
    CHECK(dbl::g.state_writes == writes + 1 && dbl::g.last_ptr == sw && dbl::g.last_int[0] == st.head &&
              dbl::g.last_int[1] == st.count && dbl::g.last_int[2] == 3,
          "state word written on bind");
    CHECK(rb_push_frame(r, fk.p, fv.p, nullptr, nullptr) == PA_OK, "push with a state word");
    rb_get_state(r, &st);
    CHECK(dbl::g.state_writes == writes + 2 && dbl::g.last_int[0] == st.head, "state word rewritten by a push");
    CHECK(rb_bind_state_word(r, nullptr, nullptr) == PA_OK, "unbind");
    CHECK(rb_push_frame(r, fk.p, fv.p, nullptr, nullptr) == PA_OK, "push unbound");
    CHECK(dbl::g.state_writes == writes + 2, "no state word write once unbound");
    // capture: calls that change host metadata are refused and change nothing
    dbl::g.capturing = true;
    rb_state before, after;
    rb_get_state(r, &before);
    CHECK(rb_push_frame(r, fk.p, fv.p, nullptr, nullptr) == PA_ESTATE, "push under capture refused");
    CHECK(rb_snapshot(r, cap.p, cb, &snap, nullptr) == PA_ESTATE, "snapshot under capture refused");
    rb_get_state(r, &after);
    CHECK(memcmp(&before, &after, sizeof before) == 0, "refused calls change nothing");
    dbl::g.capturing = false;
    CHECK(rb_destroy(r) == PA_OK, "destroy");
    CHECK(dbl::g.live_events == events0, "destroy releases the fence events");
}

struct Step {
    Buf q, k, v, out;
    Step(int L, int N, int hq, int D)
        : q((size_t)L * N * hq * D * 2), k((size_t)L * N * D * 2), v((size_t)L * N * D * 2),
          out((size_t)L * N * hq * D * 4) {}
};

static void test_attention_planning() {
    // the long-history shape: 18 layers, pin 256, 8 x 768 window, 51 x 8 queries
    const int L = 18, D = 256, P = 256, W = 8, F = 768, N = 51, HQ = 8;
    const size_t seq = P + (size_t)W * F;
    Buf kb(L * seq * D * 2), vb(L * seq * D * 2);
    rb_config cfg = {L, 1, D, P, W, F, PA_BF16, 0};
    rb_ring* r = nullptr;
    CHECK(rb_create(&cfg, kb.p, vb.p, &r) == PA_OK, "rb_create long");
    Step st(L, N, HQ, D);
    pattn_args a = {0, L, HQ, N, 1.f / 16.f, PA_F32, 0, PA_Q_TOKEN_MAJOR, 0};
    size_t wsb = pattn_workspace_bytes(r, &a);
    CHECK(wsb > 0, "workspace bytes");
    {
        Buf ws(wsb);
        CHECK(pattn_step(r, &a, st.q.p, st.k.p, st.v.p, st.out.p, ws.p, wsb, nullptr) == PA_ESTATE,
              "step before the pin refused");
        Buf pk(L * P * D * 2), pv(L * P * D * 2);
        CHECK(rb_pin_prefix(r, pk.p, pv.p, P, nullptr) == PA_OK, "pin long");
        // nothing pushed: context [pin; suffix]
        CHECK(pattn_step(r, &a, st.q.p, st.k.p, st.v.p, st.out.p, ws.p, wsb, nullptr) == PA_OK, "step, empty window");
        Buf fk(L * F * D * 2), fv(L * F * D * 2);
        for (int f = 0; f < W; ++f) CHECK(rb_push_frame(r, fk.p, fv.p, nullptr, nullptr) == PA_OK, "push");
        const long long l0 = dbl::g.launches, b0 = dbl::g.bad_launches;
        CHECK(pattn_step(r, &a, st.q.p, st.k.p, st.v.p, st.out.p, ws.p, wsb, nullptr) == PA_OK, "step");
        CHECK(dbl::g.launches == l0 + 2 && dbl::g.bad_launches == b0, "partials + combine launched");
        CHECK(pattn_step(r, &a, st.q.p, st.k.p, st.v.p, st.out.p, ws.p, wsb - 1, nullptr) == PA_ERANGE,
              "small workspace refused");
        pattn_args bad = a;
        bad.scale = -1.f;
        CHECK(pattn_step(r, &bad, st.q.p, st.k.p, st.v.p, st.out.p, ws.p, wsb, nullptr) == PA_EINVAL, "bad scale");
        bad = a;
        bad.partials_f32 = 2;
        CHECK(pattn_step(r, &bad, st.q.p, st.k.p, st.v.p, st.out.p, ws.p, wsb, nullptr) == PA_EINVAL, "bad flag");
        bad = a;
        bad.layer_begin = 10;
        CHECK(pattn_step(r, &bad, st.q.p, st.k.p, st.v.p, st.out.p, ws.p, wsb, nullptr) == PA_ESHAPE, "layers");
        CHECK(pattn_step(r, &a, nullptr, st.k.p, st.v.p, st.out.p, ws.p, wsb, nullptr) == PA_EINVAL, "null q");
        CHECK(pattn_step(r, &a, static_cast<char*>(st.q.p) + 2, st.k.p, st.v.p, st.out.p, ws.p, wsb, nullptr) ==
                  PA_EINVAL, "misaligned q");
        // capture: a full window without a spare slot may be captured
        dbl::g.capturing = true;
        CHECK(pattn_step(r, &a, st.q.p, st.k.p, st.v.p, st.out.p, ws.p, wsb, nullptr) == PA_OK, "capture, full");
        dbl::g.capturing = false;
    }
    // every split count, both Q layouts, FP32 partials, layer sub-ranges
    for (int splits = 0; splits <= 127; splits += (splits < 16 ? 1 : 37))
        for (int layout = 0; layout < 2; ++layout)
            for (int f32p = 0; f32p < 2; ++f32p) {
                pattn_args b = {3, 5, HQ, N, 1.f / 16.f, PA_BF16, splits, layout, f32p};
                const size_t n = pattn_workspace_bytes(r, &b);
                CHECK(n > 0, "workspace %d %d %d", splits, layout, f32p);
                Buf ws(n);
                Buf qo(layout ? pattn_operand_q_bytes(r, &b) : 16);
                const long long b0 = dbl::g.bad_launches;
                if (layout) CHECK(pattn_pack_q(r, &b, st.q.p, qo.p, nullptr) == PA_OK, "pack q");
                CHECK(pattn_step(r, &b, layout ? qo.p : st.q.p, st.k.p, st.v.p, st.out.p, ws.p, n, nullptr) == PA_OK,
                      "step splits %d layout %d f32p %d", splits, layout, f32p);
                CHECK(dbl::g.bad_launches == b0, "launch shape splits %d", splits);
            }
    // the entry point that allocates nothing: fits, and refuses beyond its scratch
    CHECK(pattn_step_noalloc(r, &a, st.q.p, st.k.p, st.v.p, st.out.p, nullptr) == PA_OK, "noalloc");
    pattn_args big = a;
    big.num_splits = 16;
    CHECK(pattn_workspace_bytes(r, &big) > pattn_noalloc_scratch_bytes(), "16 splits exceed the scratch");
    CHECK(pattn_step_noalloc(r, &big, st.q.p, st.k.p, st.v.p, st.out.p, nullptr) == PA_ERANGE, "noalloc refuses");
    // decode readers and the fused pass: 16 streams, 30-token tails
    const int G = 16, CAP = 30;
    pattn_decode_args da = {0, L, HQ, G, CAP, 1.f / 16.f, PA_BF16, 0, 1};
    Buf tk((size_t)L * G * CAP * D * 2), tv((size_t)L * G * CAP * D * 2), tl(G * 4), ovf(4);
    Buf kn((size_t)L * G * D * 2), vn((size_t)L * G * D * 2), qd((size_t)L * G * HQ * D * 2),
        od((size_t)L * G * HQ * D * 2);
    CHECK(pattn_append_private(r, &da, tk.p, tv.p, tl.as<int32_t>(), kn.p, vn.p, ovf.as<uint32_t>(), nullptr) == PA_OK,
          "append");
    {
        const size_t n = pattn_decode_workspace_bytes(r, &da);
        Buf ws(n);
        CHECK(n > 0 && pattn_decode(r, &da, qd.p, tk.p, tv.p, tl.as<int32_t>(), od.p, ws.p, n, nullptr) == PA_OK,
              "decode");
    }
    {
        pattn_args fa = a;
        fa.out_dtype = PA_BF16;
        const size_t n = pattn_fused_workspace_bytes(r, &fa, &da);
        Buf ws(n);
        CHECK(n > 0 && pattn_fused_step(r, &fa, st.q.p, st.k.p, st.v.p, st.out.p, &da, qd.p, tk.p, tv.p,
                                        tl.as<int32_t>(), od.p, ws.p, n, nullptr) == PA_OK,
              "fused");
        fa.partials_f32 = 1;
        CHECK(pattn_fused_step(r, &fa, st.q.p, st.k.p, st.v.p, st.out.p, &da, qd.p, tk.p, tv.p, tl.as<int32_t>(),
                               od.p, ws.p, n, nullptr) == PA_EINVAL,
              "fused refuses FP32 partials");
    }
    CHECK(rb_destroy(r) == PA_OK, "destroy long");
}

static void test_stack_planning() {
    // the Pi0.5-like ring (pin 48, 2 x 768 window), a 3-layer stack of width 1024
    const int L = 3, D = 256, P = 48, W = 2, F = 768, N = 51, HQ = 8, M = 1024, FF = 4096;
    const size_t seq = P + (size_t)W * F;
    Buf kb(L * seq * D * 2), vb(L * seq * D * 2);
    rb_config cfg = {L, 1, D, P, W, F, PA_BF16, 0};
    rb_ring* r = nullptr;
    CHECK(rb_create(&cfg, kb.p, vb.p, &r) == PA_OK, "rb_create stack");
    Buf pk(L * P * D * 2), pv(L * P * D * 2), fk(L * F * D * 2), fv(L * F * D * 2);
    rb_pin_prefix(r, pk.p, pv.p, P, nullptr);
    for (int f = 0; f < W; ++f) rb_push_frame(r, fk.p, fv.p, nullptr, nullptr);
    const size_t nqkv = (size_t)(HQ + 2) * D;
    Buf wqkv(L * nqkv * M * 2), wo((size_t)L * M * HQ * D * 2), wg((size_t)L * FF * M * 2), wu((size_t)L * FF * M * 2),
        wd((size_t)L * M * FF * 2), x(N * M * 2), gamma((size_t)L * 10 * M * 4), flag(4);
    for (int packed = 0; packed < 2; ++packed)
        for (int ffn = 0; ffn < 2; ++ffn) {
            pa_stack s = {L, N, M, HQ, wqkv.p, wo.p, 1e-6f, 1.f / 16.f, 0.1f, 0, ffn ? FF : 0,
                          wg.p, wu.p, wd.p, packed};
            const size_t n = pa_denoise_step_workspace_bytes(r, &s);
            CHECK(n > 0, "stack workspace packed %d ffn %d", packed, ffn);
            Buf ws(n);
            const long long b0 = dbl::g.bad_launches;
            CHECK(pa_denoise_step(r, &s, x.p, gamma.as<float>(), ffn ? gamma.as<float>() : nullptr, 10 * M,
                                  flag.as<uint32_t>(), ws.p, n, nullptr) == PA_OK,
                  "denoise step packed %d ffn %d", packed, ffn);
            CHECK(dbl::g.bad_launches == b0, "stack launch shapes");
            CHECK(pa_denoise_step(r, &s, x.p, gamma.as<float>(), ffn ? gamma.as<float>() : nullptr, M - 1,
                                  flag.as<uint32_t>(), ws.p, n, nullptr) == PA_ESHAPE, "gamma stride refused");
        }
    pa_stack bad = {L + 1, N, M, HQ, wqkv.p, wo.p, 1e-6f, 1.f / 16.f, 0.1f, 0, 0, nullptr, nullptr, nullptr, 0};
    CHECK(pa_denoise_step_workspace_bytes(r, &bad) == 0, "more layers than the ring");
    CHECK(pa_pack_weight(wqkv.p, (int)nqkv, M, wo.p, nullptr) == PA_OK, "pack weight");
    CHECK(pa_pack_weight(wqkv.p, 33, M, wo.p, nullptr) != PA_OK, "pack weight needs n % 32 == 0");
    // the per-op entry points
    Buf q(N * HQ * D * 2), k(N * D * 2), v(N * D * 2), h(N * M * 2), y(N * M * 4);
    CHECK(ada_rmsnorm_qkv(x.p, N, M, gamma.as<float>(), 1e-6f, wqkv.p, HQ, 1, D, q.p, k.p, v.p, flag.as<uint32_t>(),
                          nullptr, 0, nullptr) == PA_OK, "ada_rmsnorm_qkv");
    CHECK(ada_rmsnorm_qkv(x.p, 65, M, gamma.as<float>(), 1e-6f, wqkv.p, HQ, 1, D, q.p, k.p, v.p, nullptr, nullptr, 0,
                          nullptr) != PA_OK, "65 rows refused");
    CHECK(oproj_residual(q.p, wo.p, h.p, N, HQ * D, M, x.p, 0.1f, flag.as<uint32_t>(), nullptr) == PA_OK, "oproj");
    {
        const size_t n = ffn_swiglu_workspace_bytes(N, M, FF);
        Buf ws(n);
        CHECK(n > 0 && ffn_swiglu(h.p, N, M, FF, gamma.as<float>(), 1e-6f, wg.p, wu.p, wd.p, x.p, 0.1f,
                                  flag.as<uint32_t>(), ws.p, n, nullptr) == PA_OK, "ffn_swiglu");
    }
    Buf w1((size_t)L * 1024 * 160 * 2), b1((size_t)L * 1024 * 2), w2((size_t)L * M * 1024 * 2), b2((size_t)L * M * 2),
        state(32 * 2);
    ada_mlp mlp = {w1.p, b1.p, w2.p, b2.p, L, 128, 32, 1024, M};
    float t[10];
    for (int i = 0; i < 10; ++i) t[i] = 1.f - i / 10.f;
    {
        const size_t n = ada_gamma_workspace_bytes(&mlp, 10);
        Buf ws(n ? n : 1);
        CHECK(ada_gamma(&mlp, t, 10, state.p, gamma.as<float>(), ws.p, n, nullptr) == PA_OK, "ada_gamma");
        CHECK(ada_gamma(&mlp, t, 17, state.p, gamma.as<float>(), ws.p, n, nullptr) == PA_ESHAPE, "17 timesteps");
    }
    {
        const size_t n = ada_rmsnorm_workspace_bytes(&mlp);
        Buf ws(n ? n : 1);
        CHECK(ada_rmsnorm(x.p, N, &mlp, 1, 0.5f, state.p, 1e-6f, y.p, PA_F32, flag.as<uint32_t>(), ws.p, n,
                          nullptr) == PA_OK, "ada_rmsnorm");
        CHECK(ada_rmsnorm(x.p, N, &mlp, L, 0.5f, state.p, 1e-6f, y.p, PA_F32, nullptr, ws.p, n, nullptr) != PA_OK,
              "layer beyond the MLP stack");
    }
    CHECK(rb_destroy(r) == PA_OK, "destroy stack ring");
}

int main() {
    test_ring(0);
    test_ring(1);
    test_attention_planning();
    test_stack_planning();
    printf("host checks: %d failure(s); %lld launches recorded, %lld copies, %lld bad launch shapes\n", g_fail,
           dbl::g.launches, dbl::g.copies, dbl::g.bad_launches);
    return g_fail;
}
