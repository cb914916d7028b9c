// Per-exact-shape autotuning of the GEMM launch configuration, with the
// winners cached in process memory (nothing is written to disk).  LightX2V
// "模型量化技术", "MiniMax-H3 FP8 FP16 累加": that kernel tunes its tile and
// swizzle per exact GEMM shape over built-in candidates on first sight of a
// shape, keeps the winner in an in-process C++ cache and relies on warm-up
// to absorb the first call.  Here the choices are the tile order's band
// height and, for small grids, the tile shape.
//
// With autotuning on, the first GEMM call of a (device, kind, m, n, k,
// epilogue, groups) shape times every candidate configuration on the
// caller's own buffers and stream -- each candidate writes the same result
// bits, so running them is harmless -- with HIP events (one warm-up run,
// then the best of three), keeps the fastest and launches it.  That call
// waits for the stream (a warm-up step absorbs the cost); later calls of the
// shape launch the cached configuration asynchronously.  A stream that is
// being captured into a graph is never tuned: such calls use the cached or
// the default configuration.
#include <hip/hip_runtime.h>

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

#include "tfq_internal.h"

namespace tfq {
namespace {

std::atomic<int> g_mode{0};

// (device, qtype, scale_block, epi, groups, m, n, k)
typedef std::tuple<int, int, int, int, int, int64_t, int64_t, int64_t> Key;

std::mutex g_cache_mu;  // guards g_cache
std::map<Key, GemmConfig> g_cache;
std::mutex g_tune_mu;  // one tuning at a time

Key key_of(int dev, const GemmArgs& g)
{
    return Key{dev, g.qtype, g.scale_block, g.epi, g.groups, g.m, g.n, g.k};
}

bool find(const Key& k, GemmConfig* out)
{
    std::lock_guard<std::mutex> lk(g_cache_mu);
    auto it = g_cache.find(k);
    if (it == g_cache.end()) return false;
    *out = it->second;
    return true;
}

// Times one candidate: one warm-up launch, then the best of three.
hipError_t time_config(const GemmArgs& g, GemmConfig c, hipStream_t s, hipEvent_t e0,
                       hipEvent_t e1, float* best_ms)
{
    hipError_t err = launch_scaled_gemm_with(g, c, s);
    if (err != hipSuccess) return err;
    *best_ms = 3.4e38f;
    for (int r = 0; r < 3; ++r) {
        if ((err = hipEventRecord(e0, s)) != hipSuccess) return err;
        if ((err = launch_scaled_gemm_with(g, c, s)) != hipSuccess) return err;
        if ((err = hipEventRecord(e1, s)) != hipSuccess) return err;
        if ((err = hipEventSynchronize(e1)) != hipSuccess) return err;
        float ms = 0.0f;
        if ((err = hipEventElapsedTime(&ms, e0, e1)) != hipSuccess) return err;
        if (ms < *best_ms) *best_ms = ms;
    }
    return hipSuccess;
}

hipError_t tune(const GemmArgs& g, hipStream_t s, GemmConfig* best)
{
    GemmConfig cand[32];
    const int n = candidate_configs(g, cand, 32);
    *best = default_config(g);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t err = hipEventCreate(&e0);
    if (err == hipSuccess) err = hipEventCreate(&e1);
    float best_ms = 3.4e38f;
    for (int i = 0; i < n && err == hipSuccess; ++i) {
        float ms = 0.0f;
        err = time_config(g, cand[i], s, e0, e1, &ms);
        if (err == hipSuccess && ms < best_ms) {
            best_ms = ms;
            *best = cand[i];
        }
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    return err;
}

}  // namespace

void set_autotune(int mode) { g_mode.store(mode); }

int autotune_mode() { return g_mode.load(); }

bool autotune_lookup(int dev, const GemmArgs& g, GemmConfig* out)
{
    return find(key_of(dev, g), out);
}

void autotune_set(int dev, const GemmArgs& g, GemmConfig c)
{
    std::lock_guard<std::mutex> lk(g_cache_mu);
    g_cache[key_of(dev, g)] = c;
}

void autotune_clear()
{
    std::lock_guard<std::mutex> lk(g_cache_mu);
    g_cache.clear();
}

GemmConfig config_without_tuning(const GemmArgs& g)
{
    GemmConfig c = default_config(g);
    int dev = 0;
    if (g_mode.load() != 0 && hipGetDevice(&dev) == hipSuccess) (void)find(key_of(dev, g), &c);
    return c;
}

hipError_t launch_scaled_gemm(const GemmArgs& g, hipStream_t stream)
{
    if (g_mode.load() == 0) return launch_scaled_gemm_with(g, default_config(g), stream);
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const Key k = key_of(dev, g);
    GemmConfig c;
    if (find(k, &c)) return launch_scaled_gemm_with(g, c, stream);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if ((err = hipStreamIsCapturing(stream, &cs)) != hipSuccess) return err;
    if (cs != hipStreamCaptureStatusNone) return launch_scaled_gemm_with(g, default_config(g), stream);
    {
        std::lock_guard<std::mutex> lk(g_tune_mu);
        if (!find(k, &c)) {
            if ((err = tune(g, stream, &c)) != hipSuccess) return err;
            std::lock_guard<std::mutex> lk2(g_cache_mu);
            g_cache[k] = c;
        }
    }
    return launch_scaled_gemm_with(g, c, stream);
}

}  // namespace tfq
