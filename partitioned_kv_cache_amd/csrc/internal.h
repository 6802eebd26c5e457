// Internal helpers shared by the library's translation units: status and
// error text, bf16 words, MFMA operand vector types, the KV-source descriptor
// used by every attention kernel, and the ring handle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/pattn.h"

namespace pa {

// ---------------------------------------------------------------- errors --
pa_status fail(pa_status st, const char* fmt, ...);
void clear_error();

#define PA_CHECK_ARG(cond, st, ...)            \
    do {                                       \
        if (!(cond)) return ::pa::fail(st, __VA_ARGS__); \
    } while (0)

#define PA_HIP(call)                                                          \
    do {                                                                      \
        hipError_t e_ = (call);                                               \
        if (e_ != hipSuccess)                                                 \
            return ::pa::fail(PA_EDEVICE, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

// After a launch: report a launch failure as PA_EDEVICE.
#define PA_LAUNCHED()                                                         \
    do {                                                                      \
        hipError_t e_ = hipGetLastError();                                    \
        if (e_ != hipSuccess)                                                 \
            return ::pa::fail(PA_EDEVICE, "kernel launch failed: %s", hipGetErrorString(e_)); \
    } while (0)

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// ------------------------------------------------------------- ring handle --
struct Ring {
    rb_config cfg;
    void* k;              // device [L][P + S*F][Hkv][D], S = W + spare_slots physical slots
    void* v;
    int32_t head = 0;     // physical slot the next frame goes to: frames_pushed mod S
    int32_t count = 0;    // frames in the window, min(frames_pushed, W)
    int32_t pinned = 0;
    int64_t frames_pushed = 0;
    // asynchronous pushes (spare_slots = 1): a frame staged into slot `head`
    // by one stream and committed on another, fenced by two events
    bool staged = false;
    bool free_recorded = false;
    hipEvent_t ev_staged = nullptr;   // the staging copy is done
    hipEvent_t ev_free = nullptr;     // every step that could read the freed slot is done
    // Optional caller-owned device copy of the state, int32 {head, count,
    // pinned, 0}, rewritten stream-ordered by every call that moves head.
    // Attention kernels on a spare-slot ring read the window position from
    // it when it is bound, so a captured step stays valid across commits.
    int32_t* state_word = nullptr;
    int64_t elem_bytes() const { return cfg.dtype == PA_F32 ? 4 : 2; }
    int32_t phys_slots() const { return cfg.num_slots + cfg.spare_slots; }
    int64_t seq_len() const { return (int64_t)cfg.pin_capacity + (int64_t)phys_slots() * cfg.tokens_per_frame; }
    int64_t layer_elems() const { return seq_len() * cfg.num_kv_heads * cfg.head_dim; }
    int32_t cached_tokens() const { return pinned + count * cfg.tokens_per_frame; }
    // The window's slots in physical order skip slot `head` (the spare, which
    // may be being written); with no spare the window is slots [0, count).
    // Window token u (of count * F) lives at slide token u + (u >= skip_at ? F : 0).
    int32_t skip_at() const { return cfg.spare_slots ? head * cfg.tokens_per_frame : count * cfg.tokens_per_frame; }
};

// ------------------------------------------------------------ device types --
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

// float -> bf16 word, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ bool finite_f(float x) { return (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u; }

// Where the keys of one (layer, kv-head) live. Logical key j of the context
// [pin | window | dyn] maps to
//   j <  pinned                     ring token j
//   j <  pinned + n_slide           ring token P + u (+ F if u >= skip_at), u = j - pinned
//   otherwise                       dyn token j - pinned - n_slide
// n_slide = count * F. Frame f sits in slot f mod S and slots fill from 0,
// so the window is the leading `count` slots, except that a ring with a
// spare slot (S = W + 1) leaves out slot `head`, the one a push may be
// filling (physical slot order; softmax does not depend on key order).
// One launch that copies both tensors' per-layer runs of a frame (or of the
// pinned prefix) into the ring: for tensor t and layer l, `run` 16-byte
// words from src[t] + l * run to dst[t] + l * dst_stride (ring.hip).
typedef unsigned int word16 __attribute__((ext_vector_type(4)));   // one 16-byte word
struct RunCopy {
    const word16* src[2];
    word16* dst[2];
    long long run;          // 16-byte words per layer (a contiguous run in the source)
    long long dst_stride;   // 16-byte words from one layer's run to the next in the ring
};
__global__ void copy_kv_runs(RunCopy c);

struct KvSource {
    const void* ring_k;        // element 0 of layer `layer_begin`
    const void* ring_v;
    long long ring_layer;      // elements per ring layer
    const void* dyn_k;         // element 0 of call-layer 0, may be null if n_dyn == 0
    const void* dyn_v;
    long long dyn_layer;       // elements per dyn layer (N * Hkv * D)
    int pinned, pin_cap, n_slide, n_dyn;
    int skip_at, skip_len;     // window token u >= skip_at sits skip_len tokens further on
    int hkv, d;
    // Spare-slot rings with a bound state word: skip_at is head * F, read
    // from the word (element 0 = head) when the kernel runs, not when it is
    // enqueued. Null otherwise.
    const int32_t* head_word;

    __device__ __forceinline__ int total() const { return pinned + n_slide + n_dyn; }
    // skip_at as the kernel must use it (reads the state word when bound)
    __device__ __forceinline__ int window_skip() const {
        return head_word ? *head_word * skip_len : skip_at;
    }

    // element offset of (call-layer lb, kv head g, logical key j) and which
    // buffer; skip_at must already be resolved (window_skip)
    __device__ __forceinline__ long long offset(int lb, int g, int j, bool& is_dyn) const {
        if (j < pinned + n_slide) {
            const int u = j - pinned;
            int tok = j < pinned ? j : pin_cap + u + (u >= skip_at ? skip_len : 0);
            is_dyn = false;
            return (long long)lb * ring_layer + ((long long)tok * hkv + g) * d;
        }
        is_dyn = true;
        return (long long)lb * dyn_layer + ((long long)(j - pinned - n_slide) * hkv + g) * d;
    }
};

// Is `stream` being captured into a graph? (false when HIP cannot tell.)
pa_status stream_capturing(hipStream_t stream, bool* capturing);

// Attention reads the ring's host metadata (window length, and the window
// position of a spare-slot ring) when it is enqueued. A captured launch
// stays valid across later pushes only if neither can change under it: the
// window must be full, and a spare-slot ring must have a bound state word.
pa_status check_capture(const Ring* r, hipStream_t stream, const char* who);

}  // namespace pa
