// Dispatch of the chunk-scan kernel on the chunk size (kernel in k_chunk_scan.h,
// one instantiation file per chunk size so that they compile in parallel).
#include <atomic>

#include "k_chunk_scan.h"

namespace cssd {

template <int C>
hipError_t launch_chunk_scan_c(const FwdArgs& f, hipStream_t s);
extern template hipError_t launch_chunk_scan_c<16>(const FwdArgs&, hipStream_t);
extern template hipError_t launch_chunk_scan_c<32>(const FwdArgs&, hipStream_t);
extern template hipError_t launch_chunk_scan_c<64>(const FwdArgs&, hipStream_t);
extern template hipError_t launch_chunk_scan_c<128>(const FwdArgs&, hipStream_t);

hipError_t device_cu_count(int* cus) {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64 && cache[dev].load() > 0) {
        *cus = cache[dev].load();
        return hipSuccess;
    }
    e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (*cus < 1) return hipErrorInvalidDevice;
    if (dev >= 0 && dev < 64) cache[dev].store(*cus);
    return hipSuccess;
}

hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t stream) {
    switch (a.C) {
        case 16: return launch_chunk_scan_c<16>(a, stream);
        case 32: return launch_chunk_scan_c<32>(a, stream);
        case 64: return launch_chunk_scan_c<64>(a, stream);
        default: return launch_chunk_scan_c<128>(a, stream);
    }
}

}  // namespace cssd
