// Host side of the causal launch order: how many workgroups one XCD runs at
// once (a generation, see odd_generation) and how many heads it takes at a
// time.  The counts come from the kernel's occupancy and the device's CU
// count, which the runtime reports once per device and kernel; they are
// cached so a launch pays for a lookup only.
#include <mutex>
#include <vector>

#include "fa_launch.h"

namespace fa {

namespace {
constexpr int kXcds = 8;                       // workgroup ids are dealt to XCDs mod 8

struct Entry {
    int device;
    const void* kernel;
    int threads;
    int gen;
};
std::mutex g_mu;
std::vector<Entry> g_cache;

// L2 bytes of one XCD (the runtime reports the per-XCD cache); 4 MiB if it
// cannot say
long l2_bytes(hipStream_t stream) {
    int dev = 0, bytes = 0;
    if (hipStreamGetDevice(stream, &dev) == hipSuccess &&
        hipDeviceGetAttribute(&bytes, hipDeviceAttributeL2CacheSize, dev) == hipSuccess && bytes > 0)
        return bytes;
    (void)hipGetLastError();
    return 4l << 20;
}

}  // namespace

int xcd_slots(const void* kernel, int threads, hipStream_t stream) {
    int dev = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    {
        std::lock_guard<std::mutex> lk(g_mu);
        for (const Entry& e : g_cache)
            if (e.device == dev && e.kernel == kernel && e.threads == threads) return e.gen;
    }
    int per_cu = 0, cus = 0;
    int gen = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
        gen = per_cu * (cus / kXcds);
    else
        (void)hipGetLastError();               // a failed query leaves no error for the launch
    std::lock_guard<std::mutex> lk(g_mu);
    g_cache.push_back(Entry{dev, kernel, threads, gen});
    return gen;
}

Schedule causal_schedule(const void* kernel, int threads, int nb, int d, int N, bool window,
                         hipStream_t stream) {
    // Heads taken together when the sweeps do not alternate: pairs at
    // d = 128, all heads at d = 64 (fewer heads at once made the d = 64
    // kernels 6 - 10% slower).
    const Schedule plain{0, d == 128 ? 2 : 1 << 20};
    if (window) return plain;
    // While a head's streamed operands (two N x d bf16 tensors: K and V, or
    // Q and dO) fit in one XCD's L2, the plain order re-reads them from L2
    // already, and at those sizes one head per generation measured 2.5%
    // slower in the backward; past that the L2 cannot hold them and the
    // generations' sweeps must line up.
    if ((long)N * d * 4 < (long)l2_bytes(stream)) return plain;
    const int gen = xcd_slots(kernel, threads, stream);
    if (gen <= 0) return plain;
    // enough heads that one generation holds the blocks of whole heads
    const int group = d == 64 ? plain.group : nb >= gen ? 1 : (gen + nb - 1) / nb;
    return Schedule{gen, group};
}

}  // namespace fa
