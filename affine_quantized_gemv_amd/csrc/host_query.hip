// Cached host-side device queries (declared in host_query.h).
#include "host_query.h"

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

namespace aqg {
namespace detail {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];   // 0 = not yet queried

std::mutex g_mu;
// (device, kernel, threads, LDS bytes) -> blocks per CU
std::map<std::tuple<int, const void*, int, size_t>, int> g_occ;
// (device, kernel) -> LDS limit raised to at least this many bytes
std::map<std::pair<int, const void*>, size_t> g_lds;

hipError_t current(int& dev)
{
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
    return e;
}

}  // namespace

hipError_t device_cus(int& cus)
{
    int dev = 0;
    hipError_t e = current(dev);
    if (e != hipSuccess) return e;
    int v = g_cus[dev].load(std::memory_order_acquire);
    if (v == 0) {
        e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (v < 1) v = 1;
        g_cus[dev].store(v, std::memory_order_release);
    }
    cus = v;
    return hipSuccess;
}

hipError_t occupancy(int& blocks_per_cu, const void* fn, int threads, size_t lds_bytes)
{
    int dev = 0;
    hipError_t e = current(dev);
    if (e != hipSuccess) return e;
    const auto key = std::make_tuple(dev, fn, threads, lds_bytes);
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_occ.find(key);
        if (it != g_occ.end()) {
            blocks_per_cu = it->second;
            return hipSuccess;
        }
    }
    int v = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, fn, threads, lds_bytes);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_mu);
    g_occ[key] = v;
    blocks_per_cu = v;
    return hipSuccess;
}

hipError_t raise_lds_limit(const void* fn, size_t bytes)
{
    int dev = 0;
    hipError_t e = current(dev);
    if (e != hipSuccess) return e;
    const auto key = std::make_pair(dev, fn);
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_lds.find(key);
        if (it != g_lds.end() && it->second >= bytes) return hipSuccess;
    }
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_mu);
    size_t& have = g_lds[key];
    if (have < bytes) have = bytes;
    return hipSuccess;
}

}  // namespace detail
}  // namespace aqg
