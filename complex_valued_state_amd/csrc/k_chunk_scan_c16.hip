// Instantiation of the chunk-scan kernel for chunk size 16 (see k_chunk_scan.h).
#include "k_chunk_scan.h"

namespace cssd {
template hipError_t launch_chunk_scan_c<16>(const FwdArgs& f, hipStream_t s);
}  // namespace cssd
