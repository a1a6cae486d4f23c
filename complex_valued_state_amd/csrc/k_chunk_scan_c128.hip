// Instantiation of the chunk-scan kernel for chunk size 128 (see k_chunk_scan.h).
#include "k_chunk_scan.h"

namespace cssd {
template hipError_t launch_chunk_scan_c<128>(const FwdArgs& f, hipStream_t s);
}  // namespace cssd
