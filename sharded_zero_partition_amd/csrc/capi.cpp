// capi.cpp -- C ABI glue: errors, per-device workspace, the shard step's host
// control (argument checks, Adam constants, overflow decision, loss scale).
//
// The step follows the Stage 1/2 paragraphs of the ZeRO explainer page
// ("ZeRO: Memory Optimizations Toward Training Trillion Parameter Models",
// azimuth.plus): the rank sums the gradient contributions of its own slice,
// updates its own partition of the fp32 Adam state and writes its fp16
// parameters into its slot of the gather buffer.  The skip-on-overflow loss
// scaling around it is not on the page (standard mixed-precision practice).
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "zp_internal.hpp"

namespace zp {

namespace {
thread_local std::string g_last_error;
thread_local int g_last_hip_error = 0;
}  // namespace

int fail(int status, const std::string& msg) {
    g_last_error = msg;
    return status;
}

int fail_hip(hipError_t err, const char* what) {
    g_last_hip_error = int(err);
    g_last_error = std::string(what) + ": " + hipGetErrorString(err);
    return ZERO_ERR_HIP;
}

void clear_error() { g_last_error.clear(); }

int check_stream_device(void* stream, int dev, const char* what) {
    if (!stream) return ZERO_OK;
    hipDevice_t sdev = -1;
    const hipError_t e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return fail_hip(e, "hipStreamGetDevice");
    if (int(sdev) != dev)
        return fail(ZERO_ERR_STATE, std::string(what) + ": the stream belongs to another device");
    return ZERO_OK;
}

namespace {

int env_int(const char* name, int dflt, int lo, int hi) {
    const char* s = std::getenv(name);
    if (!s || !*s) return dflt;
    const long v = std::strtol(s, nullptr, 10);
    if (v < lo || v > hi) return dflt;
    return int(v);
}

}  // namespace

int blocks_per_cu_step() {
    static const int v = env_int("ZERO_BLOCKS_PER_CU", 8, 1, 4096);
    return v;
}



namespace {

// Per-thread kernel timing: a ring of HIP event pairs, one pair per timed
// call, so that calls can be timed back to back and read afterwards.
constexpr size_t kTimingRing = 4096;

struct EventPair {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
    int device = -1;
};

struct ThreadTiming {
    bool enabled = false;
    std::vector<EventPair> ring;   // grows up to kTimingRing entries, then wraps
    size_t count = 0;              // calls recorded since timing was enabled
    bool open = false;             // a start event recorded, its stop not yet
    // the events are not destroyed at thread exit: the HIP runtime may
    // already be shutting down then
};
thread_local ThreadTiming g_timing;

EventPair* current_pair() { return &g_timing.ring[(g_timing.count - 1) % kTimingRing]; }

}  // namespace

hipError_t timing_events(KernelEvents* ev) {
    ev->start = ev->stop = nullptr;
    if (!g_timing.enabled) return hipSuccess;
    if (g_timing.open) {   // the previous call failed before closing its pair: reuse it
        g_timing.count -= 1;
        g_timing.open = false;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const size_t slot = g_timing.count % kTimingRing;
    if (slot >= g_timing.ring.size()) {
        try {
            g_timing.ring.emplace_back();
        } catch (...) {
            return hipErrorOutOfMemory;
        }
    }
    EventPair& p = g_timing.ring[slot];
    if (p.device != dev) {
        if (p.start) (void)hipEventDestroy(p.start);
        if (p.stop) (void)hipEventDestroy(p.stop);
        p.start = p.stop = nullptr;
        p.device = -1;
        e = hipEventCreate(&p.start);
        if (e == hipSuccess) e = hipEventCreate(&p.stop);
        if (e != hipSuccess) return e;
        p.device = dev;
    }
    g_timing.count += 1;
    g_timing.open = true;
    ev->start = p.start;
    ev->stop = p.stop;
    return hipSuccess;
}

void timing_done() { g_timing.open = false; }

namespace {

// Per-device workspace: the overflow flag word and the blocks-done counter
// (device, 64 bytes apart) and the pinned, coherent host word that the last
// block of a pass writes the decision into.  Created on a device's first
// shard step and kept until the process ends; `mu` serialises shard steps on
// the device (they share these words).
struct DeviceWorkspace {
    std::mutex mu;
    uint32_t* d_flag = nullptr;             // d_flag[0] flag; d_flag[16..17] the 64-bit counter
    unsigned long long* h_word = nullptr;   // host address
    unsigned long long* h_word_dev = nullptr;   // the same word, device address
    uint32_t epoch = 0;
    int cu_count = 0;
};

constexpr int kMaxDevices = 64;
std::mutex g_ws_mu;
DeviceWorkspace* g_ws[kMaxDevices] = {};
std::mutex g_noalloc_mu[kMaxDevices];   // zero_shard_step_noalloc, per device

int get_workspace(int dev, DeviceWorkspace** out) {
    if (dev < 0 || dev >= kMaxDevices) return fail(ZERO_ERR_INVALID_ARG, "device index out of range");
    std::lock_guard<std::mutex> lock(g_ws_mu);
    if (!g_ws[dev]) {
        std::unique_ptr<DeviceWorkspace> ws(new (std::nothrow) DeviceWorkspace());
        if (!ws) return fail(ZERO_ERR_OUT_OF_MEMORY, "workspace allocation failed");
        hipError_t e = hipDeviceGetAttribute(&ws->cu_count, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute");
        static_assert(kStaticScratchWords * sizeof(uint32_t) == 256, "clear_scratch zeroes the whole workspace");
        e = hipMalloc(reinterpret_cast<void**>(&ws->d_flag), 256);
        if (e != hipSuccess) return fail_hip(e, "hipMalloc (flag)");
        e = hipMemset(ws->d_flag, 0, 256);
        if (e == hipSuccess)
            e = hipHostMalloc(reinterpret_cast<void**>(&ws->h_word), 64,
                              hipHostMallocMapped | hipHostMallocCoherent);
        if (e == hipSuccess) {
            *ws->h_word = 0;
            e = hipHostGetDevicePointer(reinterpret_cast<void**>(&ws->h_word_dev), ws->h_word, 0);
        }
        if (e != hipSuccess) {
            if (ws->h_word) (void)hipHostFree(ws->h_word);
            (void)hipFree(ws->d_flag);
            return fail_hip(e, "workspace set-up");
        }
        g_ws[dev] = ws.release();
    }
    *out = g_ws[dev];
    return ZERO_OK;
}

// Waits until the last block of the pass launched with `epoch` has written
// (epoch << 1) | flag into the host word.  Every 1024 polls the stream is
// queried: an error there is returned, and a stream that has drained without
// the word being written is reported rather than waited on.
int wait_for_flag(DeviceWorkspace* ws, hipStream_t s, uint32_t epoch, int32_t* flag) {
    const unsigned long long want = epoch;
    for (unsigned poll = 1;; ++poll) {
        const unsigned long long w = __atomic_load_n(ws->h_word, __ATOMIC_ACQUIRE);
        if ((w >> 1) == want) {
            *flag = int32_t(w & 1ull);
            return ZERO_OK;
        }
        if ((poll & 1023u) == 0) {
            const hipError_t e = hipStreamQuery(s);
            if (e == hipSuccess) {
                const unsigned long long w2 = __atomic_load_n(ws->h_word, __ATOMIC_ACQUIRE);
                if ((w2 >> 1) == want) {
                    *flag = int32_t(w2 & 1ull);
                    return ZERO_OK;
                }
                return fail(ZERO_ERR_STATE, "the step's stream drained without the overflow flag being published");
            }
            if (e != hipErrorNotReady) return fail_hip(e, "waiting for the shard step");
        }
        __builtin_ia32_pause();
    }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool finite_f(float x) { return std::isfinite(x); }

// Scalar checks shared by the step entry points (nothing is modified).
int check_step_scalars(const zero_shard_state* st, const zero_adam_hparams* hp,
                       const zero_loss_scaler* sc, bool* pingpong) {
    const int64_t S = st->shard_elems;
    if (S < 0) return fail(ZERO_ERR_INVALID_ARG, "shard_elems < 0");
    if (S > ZERO_MAX_SHARD_ELEMS)
        return fail(ZERO_ERR_INVALID_ARG, "shard_elems above ZERO_MAX_SHARD_ELEMS (one launch's grid)");
    if (st->cur != 0 && st->cur != 1) return fail(ZERO_ERR_INVALID_ARG, "cur must be 0 or 1");
    if (st->t < 0 || st->t == std::numeric_limits<int64_t>::max())
        return fail(ZERO_ERR_INVALID_ARG, "step count out of range");
    const bool has1[3] = {st->p[1] != nullptr, st->m[1] != nullptr, st->v[1] != nullptr};
    *pingpong = has1[0];
    if (has1[1] != *pingpong || has1[2] != *pingpong)
        return fail(ZERO_ERR_INVALID_ARG, "p[1], m[1], v[1] must be all set or all NULL");
    if (!*pingpong && st->cur != 0) return fail(ZERO_ERR_INVALID_ARG, "cur must be 0 in place");
    if (!std::isfinite(sc->scale) || !(sc->scale >= ZERO_MIN_LOSS_SCALE))
        return fail(ZERO_ERR_INVALID_ARG, "loss scale must be finite and >= 2^-24");
    if (!finite_f(sc->min_scale) || !(sc->min_scale >= ZERO_MIN_LOSS_SCALE))
        return fail(ZERO_ERR_INVALID_ARG, "min_scale must be finite and >= 2^-24");
    if (!finite_f(sc->backoff) || !(sc->backoff > 0.0f) || !finite_f(sc->growth) ||
        !(sc->growth > 0.0f) || sc->growth_interval < 0 || sc->good_steps < 0)
        return fail(ZERO_ERR_INVALID_ARG, "invalid loss-scaler settings");
    if (!finite_f(hp->lr) || !finite_f(hp->eps) || !(hp->eps > 0.0f) || !finite_f(hp->weight_decay) ||
        !(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
        return fail(ZERO_ERR_INVALID_ARG, "invalid Adam hyper-parameters (finite; eps > 0; betas in [0, 1))");
    return ZERO_OK;
}

// Pointer checks of the state sets and the slot over their first n
// elements: non-NULL, aligned, pairwise disjoint.  Their byte ranges go to
// rs[0 .. *nr).
int check_state_arrays(const zero_shard_state* st, bool pingpong, const uint16_t* out_slot, int64_t n,
                       Range rs[7], int* nr) {
    *nr = 0;
    const int sets = pingpong ? 2 : 1;
    for (int k = 0; k < sets; ++k) {
        const float* arr[3] = {st->p[k], st->m[k], st->v[k]};
        for (const float* a : arr) {
            if (!a) return fail(ZERO_ERR_INVALID_ARG, "a state pointer is NULL");
            if (!aligned(a, 16)) return fail(ZERO_ERR_ALIGNMENT, "state array not 16-byte aligned");
            const uintptr_t lo = reinterpret_cast<uintptr_t>(a);
            rs[(*nr)++] = {lo, lo + uintptr_t(n) * 4};
        }
    }
    if (!out_slot) return fail(ZERO_ERR_INVALID_ARG, "out_slot is NULL");
    if (!aligned(out_slot, 2)) return fail(ZERO_ERR_ALIGNMENT, "out_slot not 2-byte aligned");
    const uintptr_t olo = reinterpret_cast<uintptr_t>(out_slot);
    rs[(*nr)++] = {olo, olo + uintptr_t(n) * 2};
    for (int i = 0; i < *nr; ++i)
        for (int j = i + 1; j < *nr; ++j)
            if (overlap(rs[i], rs[j])) return fail(ZERO_ERR_INVALID_ARG, "state arrays and slot must not overlap");
    return ZERO_OK;
}

// Device, stream check and workspace of a step call; advances the epoch (the
// flag words hold epochs, so after wrap-around they are cleared first).
// The caller holds (*ws)->mu from here on through `lock`.
int begin_step(void* stream, const char* who, DeviceWorkspace** ws, std::unique_lock<std::mutex>* lock,
               int* dev_out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    int rc = check_stream_device(stream, dev, who);
    if (rc != ZERO_OK) return rc;
    rc = get_workspace(dev, ws);
    if (rc != ZERO_OK) return rc;
    *lock = std::unique_lock<std::mutex>((*ws)->mu);
    if (++(*ws)->epoch == 0) {
        // the workspace is 256 bytes, the size clear_scratch zeroes
        e = clear_scratch((*ws)->d_flag, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail_hip(e, "clearing the flag word");
        __atomic_store_n((*ws)->h_word, 0ull, __ATOMIC_RELEASE);
        (*ws)->epoch = 1;
    }
    *dev_out = dev;
    return ZERO_OK;
}

// State pointers and Adam constants for step t + 1 (used only if the step is
// taken).
void step_constants(StepLaunch* a, const zero_shard_state* st, bool pingpong, const zero_adam_hparams* hp,
                    const zero_loss_scaler* sc, uint16_t* out_slot, int64_t n) {
    const int64_t t_new = st->t + 1;
    const int cur = st->cur;
    a->p_in = st->p[cur];
    a->m_in = st->m[cur];
    a->v_in = st->v[cur];
    a->p_out = pingpong ? st->p[1 - cur] : st->p[0];
    a->m_out = pingpong ? st->m[1 - cur] : st->m[0];
    a->v_out = pingpong ? st->v[1 - cur] : st->v[0];
    a->out16 = out_slot;
    a->n = n;
    a->inv_scale = 1.0f / sc->scale;
    a->lr = hp->lr;
    a->beta1 = hp->beta1;
    a->beta2 = hp->beta2;
    a->one_minus_beta1 = 1.0f - hp->beta1;
    a->one_minus_beta2 = 1.0f - hp->beta2;
    a->bias_corr1 = float(1.0 - std::pow(double(hp->beta1), double(t_new)));
    a->bias_corr2 = float(1.0 - std::pow(double(hp->beta2), double(t_new)));
    a->eps = hp->eps;
    a->weight_decay = hp->weight_decay;
}

// The flag words of `ws` at its current epoch.
void workspace_words(StepLaunch* a, const DeviceWorkspace* ws) {
    a->flag = ws->d_flag;
    a->epoch = ws->epoch;
    a->done = reinterpret_cast<unsigned long long*>(ws->d_flag + 16);
    a->host_word = ws->h_word_dev;
}

// Commit or skip, and the loss scale.
void commit_step(zero_shard_state* st, bool pingpong, zero_loss_scaler* sc, int32_t flag) {
    if (flag) {
        float ns = sc->scale * sc->backoff;
        if (ns < sc->min_scale) ns = sc->min_scale;
        sc->scale = ns;
        sc->good_steps = 0;
    } else {
        st->t += 1;
        if (pingpong) st->cur = 1 - st->cur;
        if (sc->good_steps < std::numeric_limits<int32_t>::max()) sc->good_steps += 1;   // saturates
        if (sc->growth_interval > 0 && sc->good_steps >= sc->growth_interval) {
            const float ns = sc->scale * sc->growth;
            if (std::isfinite(ns)) sc->scale = ns;   // never grow into inf
            sc->good_steps = 0;
        }
    }
}

// Argument checks of a shard step call (nothing is modified).
int check_shard_step_call(const zero_shard_state* st, const uint16_t* const* grads, int32_t R,
                          const zero_adam_hparams* hp, const zero_loss_scaler* sc, const uint16_t* out_slot,
                          const char* who, bool* pingpong) {
    if (!st || !hp || !sc) return fail(ZERO_ERR_INVALID_ARG, std::string(who) + ": NULL state, hparams or scaler");
    if (R < 1 || R > kMaxContrib) return fail(ZERO_ERR_INVALID_ARG, "R must be in 1..16");
    int rc = check_step_scalars(st, hp, sc, pingpong);
    if (rc != ZERO_OK) return rc;
    const int64_t S = st->shard_elems;
    if (S == 0) return ZERO_OK;
    if (!grads) return fail(ZERO_ERR_INVALID_ARG, "grads is NULL");
    for (int r = 0; r < R; ++r) {
        if (!grads[r]) return fail(ZERO_ERR_INVALID_ARG, "a gradient pointer is NULL");
        if (!aligned(grads[r], 16)) return fail(ZERO_ERR_ALIGNMENT, "gradient not 16-byte aligned");
    }
    Range rs[7];
    int nr = 0;
    rc = check_state_arrays(st, *pingpong, out_slot, S, rs, &nr);
    if (rc != ZERO_OK) return rc;
    for (int r = 0; r < R; ++r) {
        const uintptr_t lo = reinterpret_cast<uintptr_t>(grads[r]);
        const Range g = {lo, lo + uintptr_t(S) * 2};
        for (int i = 0; i < nr; ++i)
            if (overlap(g, rs[i])) return fail(ZERO_ERR_INVALID_ARG, "a gradient overlaps a written array");
    }
    return ZERO_OK;
}

}  // namespace
}  // namespace zp

using zp::fail;

extern "C" int zero_shard_step(zero_shard_state* st, const uint16_t* const* grads, int32_t R,
                               const zero_adam_hparams* hp, zero_loss_scaler* sc,
                               uint16_t* out_slot, void* stream, int32_t* overflow) {
    zp::clear_error();
    bool pingpong = false;
    int rc = zp::check_shard_step_call(st, grads, R, hp, sc, out_slot, "zero_shard_step", &pingpong);
    if (rc != ZERO_OK) return rc;
    const int64_t S = st->shard_elems;

    int32_t flag = 0;
    if (S > 0) {
        zp::DeviceWorkspace* ws = nullptr;
        std::unique_lock<std::mutex> lock;
        int dev = 0;
        rc = zp::begin_step(stream, "zero_shard_step", &ws, &lock, &dev);
        if (rc != ZERO_OK) return rc;
        hipStream_t s = static_cast<hipStream_t>(stream);

        zp::StepLaunch a;
        std::memset(&a, 0, sizeof(a));
        for (int r = 0; r < R; ++r) a.grad[r] = grads[r];
        a.R = R;
        zp::step_constants(&a, st, pingpong, hp, sc, out_slot, S);
        zp::workspace_words(&a, ws);

        zp::KernelEvents ev;
        hipError_t e = zp::timing_events(&ev);
        if (e != hipSuccess) return zp::fail_hip(e, "timing event");
        if (pingpong) {
            e = zp::launch_fused_step(a, s, ev);
            if (e != hipSuccess) return zp::fail_hip(e, "shard step kernel launch");
        } else {
            e = zp::launch_check(a, ws->cu_count, s, ev.start);
            if (e != hipSuccess) return zp::fail_hip(e, "check kernel launch");
            e = zp::launch_update_in_place(a, s, ev.stop);
            if (e != hipSuccess) return zp::fail_hip(e, "update kernel launch");
        }
        zp::timing_done();
        rc = zp::wait_for_flag(ws, s, ws->epoch, &flag);
        if (rc != ZERO_OK) return rc;
        if (!pingpong) {
            // the update pass reads the flag word: let it finish before the
            // next call on this device can raise that word again
            e = hipStreamSynchronize(s);
            if (e != hipSuccess) return zp::fail_hip(e, "waiting for the in-place update");
        }

        if (flag && pingpong) {
            // the pass wrote the slot speculatively; restore fp16(master)
            e = zp::launch_slot_from_master(a, ws->cu_count, s);
            if (e != hipSuccess) return zp::fail_hip(e, "slot restore kernel launch");
        }
    }

    zp::commit_step(st, pingpong, sc, flag);
    if (overflow) *overflow = flag;
    return ZERO_OK;
}

extern "C" int zero_shard_step_noalloc(zero_shard_state* st, const uint16_t* const* grads, int32_t R,
                                       const zero_adam_hparams* hp, zero_loss_scaler* sc,
                                       uint16_t* out_slot, void* stream, int32_t* overflow) {
    zp::clear_error();
    bool pingpong = false;
    int rc = zp::check_shard_step_call(st, grads, R, hp, sc, out_slot, "zero_shard_step_noalloc", &pingpong);
    if (rc != ZERO_OK) return rc;
    const int64_t S = st->shard_elems;

    int32_t flag = 0;
    if (S > 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return zp::fail_hip(e, "hipGetDevice");
        rc = zp::check_stream_device(stream, dev, "zero_shard_step_noalloc");
        if (rc != ZERO_OK) return rc;
        if (dev >= zp::kMaxDevices) return fail(ZERO_ERR_INVALID_ARG, "device index out of range");
        uint32_t* w = nullptr;
        rc = zp::static_scratch(dev, &w);
        if (rc != ZERO_OK) return rc;
        int cu_count = 0;
        e = hipDeviceGetAttribute(&cu_count, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return zp::fail_hip(e, "hipDeviceGetAttribute");
        // one call at a time per device in this process: the calls share the
        // device's scratch words
        std::lock_guard<std::mutex> lock(zp::g_noalloc_mu[dev]);
        hipStream_t s = static_cast<hipStream_t>(stream);
        // the flag, the counter and the decision word start at 0
        e = zp::clear_scratch(w, s);
        if (e != hipSuccess) return zp::fail_hip(e, "clearing the scratch words");

        zp::StepLaunch a;
        std::memset(&a, 0, sizeof(a));
        for (int r = 0; r < R; ++r) a.grad[r] = grads[r];
        a.R = R;
        zp::step_constants(&a, st, pingpong, hp, sc, out_slot, S);
        a.flag = w;
        a.epoch = 1;
        a.done = reinterpret_cast<unsigned long long*>(w + 16);
        a.host_word = reinterpret_cast<unsigned long long*>(w + 32);
        const zp::KernelEvents none;
        if (pingpong) {
            e = zp::launch_fused_step(a, s, none);
            if (e != hipSuccess) return zp::fail_hip(e, "shard step kernel launch");
        } else {
            e = zp::launch_check(a, cu_count, s, nullptr);
            if (e != hipSuccess) return zp::fail_hip(e, "check kernel launch");
            e = zp::launch_update_in_place(a, s, nullptr);
            if (e != hipSuccess) return zp::fail_hip(e, "update kernel launch");
        }
        unsigned long long word = 0;
        e = hipMemcpyAsync(&word, a.host_word, sizeof(word), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return zp::fail_hip(e, "reading the overflow decision");
        if ((word >> 1) != 1ull)
            return fail(ZERO_ERR_STATE, "the pass ended without writing the overflow decision");
        flag = int32_t(word & 1ull);
        if (flag && pingpong) {
            // the pass wrote the slot speculatively; restore fp16(master)
            e = zp::launch_slot_from_master(a, cu_count, s);
            if (e != hipSuccess) return zp::fail_hip(e, "slot restore kernel launch");
        }
    }

    zp::commit_step(st, pingpong, sc, flag);
    if (overflow) *overflow = flag;
    return ZERO_OK;
}

extern "C" int zero_owner_step(const zero_layout* layout, int32_t rank, zero_shard_state* st,
                               const zero_adam_hparams* hp, zero_loss_scaler* sc,
                               uint16_t* out_slot, void* stream, int32_t* overflow) {
    zp::clear_error();
    if (!layout || !st || !hp || !sc)
        return fail(ZERO_ERR_INVALID_ARG, "zero_owner_step: NULL layout, state, hparams or scaler");
    bool pingpong = false;
    int rc = zp::check_step_scalars(st, hp, sc, &pingpong);
    if (rc != ZERO_OK) return rc;
    if (!pingpong) return fail(ZERO_ERR_INVALID_ARG, "the owner step needs ping-pong state (p[1], m[1], v[1])");
    zp::OwnerLaunch a;
    std::memset(&a, 0, sizeof(a));
    int bound_dev = -1;
    rc = zp::owner_tables(layout, rank, &a, &bound_dev);
    if (rc != ZERO_OK) return rc;
    zero_layout_info info;
    rc = zero_layout_get_info(layout, &info);
    if (rc != ZERO_OK) return rc;
    if (st->shard_elems != info.shard_elems)
        return fail(ZERO_ERR_INVALID_ARG, "shard_elems differs from the layout's shard size");
    // the whole shard is written: its real elements from the contributions,
    // its padding with a zero gradient
    const int64_t S = st->shard_elems;

    if (S > 0) {
        zp::Range rs[7];
        int nr = 0;
        rc = zp::check_state_arrays(st, pingpong, out_slot, S, rs, &nr);
        if (rc != ZERO_OK) return rc;
        for (int i = 0; i < nr; ++i)
            if (zp::contributions_overlap(layout, rs[i].lo, rs[i].hi))
                return fail(ZERO_ERR_INVALID_ARG, "a contribution tensor overlaps the state or the slot");
    }

    int32_t flag = 0;
    if (S > 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return zp::fail_hip(e, "hipGetDevice");
        if (dev != bound_dev) return fail(ZERO_ERR_STATE, "contributions were bound on another device");
        zp::DeviceWorkspace* ws = nullptr;
        std::unique_lock<std::mutex> lock;
        rc = zp::begin_step(stream, "zero_owner_step", &ws, &lock, &dev);
        if (rc != ZERO_OK) return rc;
        hipStream_t s = static_cast<hipStream_t>(stream);
        zp::step_constants(&a.st, st, pingpong, hp, sc, out_slot, S);
        zp::workspace_words(&a.st, ws);
        a.st.R = a.R;

        zp::KernelEvents ev;
        e = zp::timing_events(&ev);
        if (e != hipSuccess) return zp::fail_hip(e, "timing event");
        e = zp::launch_owner_step(a, s, ev);
        if (e != hipSuccess) return zp::fail_hip(e, "owner step kernel launch");
        zp::timing_done();
        rc = zp::wait_for_flag(ws, s, ws->epoch, &flag);
        if (rc != ZERO_OK) return rc;
        if (flag) {
            // the pass wrote the slot speculatively; restore fp16(master)
            e = zp::launch_slot_from_master(a.st, ws->cu_count, s);
            if (e != hipSuccess) return zp::fail_hip(e, "slot restore kernel launch");
        }
    }

    zp::commit_step(st, pingpong, sc, flag);
    if (overflow) *overflow = flag;
    return ZERO_OK;
}

extern "C" int zero_set_kernel_timing(int32_t enable) {
    zp::clear_error();
    zp::g_timing.enabled = enable != 0;
    zp::g_timing.count = 0;
    zp::g_timing.open = false;
    return ZERO_OK;
}

namespace zp {
namespace {

int pair_ms(const EventPair& p, float* ms) {
    hipError_t e = hipEventSynchronize(p.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, p.start, p.stop);
    if (e != hipSuccess) return fail_hip(e, "reading kernel timing events");
    return ZERO_OK;
}

}  // namespace
}  // namespace zp

extern "C" int zero_last_kernel_ms(float* ms) {
    zp::clear_error();
    if (!ms) return fail(ZERO_ERR_INVALID_ARG, "ms is NULL");
    const size_t complete = zp::g_timing.count - (zp::g_timing.open ? 1 : 0);
    if (complete == 0) return fail(ZERO_ERR_STATE, "no kernel timed since timing was enabled");
    return zp::pair_ms(zp::g_timing.ring[(complete - 1) % zp::kTimingRing], ms);
}

extern "C" int zero_kernel_times(float* ms, int64_t cap, int64_t* n) {
    zp::clear_error();
    if (!n) return fail(ZERO_ERR_INVALID_ARG, "zero_kernel_times: n is NULL");
    const size_t count = zp::g_timing.count - (zp::g_timing.open ? 1 : 0);
    const size_t kept = count < zp::kTimingRing ? count : zp::kTimingRing;
    *n = int64_t(kept);
    if (kept == 0) return ZERO_OK;
    if (!ms || cap < int64_t(kept)) return fail(ZERO_ERR_CAPACITY, "timing array too small");
    for (size_t i = 0; i < kept; ++i) {
        const size_t call = count - kept + i;   // oldest kept call first
        const int rc = zp::pair_ms(zp::g_timing.ring[call % zp::kTimingRing], ms + i);
        if (rc != ZERO_OK) return rc;
    }
    return ZERO_OK;
}

extern "C" int zero_version(void) { return ZERO_PARTITION_VERSION; }

extern "C" const char* zero_last_error(void) { return zp::g_last_error.c_str(); }

extern "C" int zero_last_hip_error(void) { return zp::g_last_hip_error; }

extern "C" int64_t zero_abi_struct_size(int32_t which) {
    switch (which) {
        case 0: return int64_t(sizeof(zero_layout_info));
        case 1: return int64_t(sizeof(zero_segment));
        case 2: return int64_t(sizeof(zero_shard_state));
        case 3: return int64_t(sizeof(zero_adam_hparams));
        case 4: return int64_t(sizeof(zero_loss_scaler));
        case 5: return int64_t(sizeof(zero_arena_plan));
        default: return -1;
    }
}

extern "C" int zero_device_info(int32_t* arch, int64_t* hbm_bytes) {
    zp::clear_error();
    if (!arch || !hbm_bytes) return fail(ZERO_ERR_INVALID_ARG, "zero_device_info: NULL argument");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return zp::fail_hip(e, "hipGetDevice");
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return zp::fail_hip(e, "hipGetDeviceProperties");
    int num = 0;
    if (std::sscanf(prop.gcnArchName, "gfx%d", &num) != 1) num = 0;
    *arch = num;
    *hbm_bytes = int64_t(prop.totalGlobalMem);
    return ZERO_OK;
}
