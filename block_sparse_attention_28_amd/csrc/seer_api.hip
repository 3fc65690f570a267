// seer_api.hip -- library-wide entry points of the C ABI: status names,
// version, and the per-device compute-unit cache used to size launches.
#include "seer_host.hpp"

#include <mutex>

namespace seer {

int device_cu_count() {
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev < 64) cached[dev] = cus;
    return cus;
}

}  // namespace seer

extern "C" const char *seer_status_string(int status) {
    switch (status) {
        case SEER_OK: return "SEER_OK";
        case SEER_ERR_INVALID_ARG: return "SEER_ERR_INVALID_ARG";
        case SEER_ERR_UNSUPPORTED: return "SEER_ERR_UNSUPPORTED";
        case SEER_ERR_WORKSPACE: return "SEER_ERR_WORKSPACE";
        case SEER_ERR_LAUNCH: return "SEER_ERR_LAUNCH";
    }
    return "SEER_ERR_UNKNOWN";
}

extern "C" int seer_version(void) { return 100; }
