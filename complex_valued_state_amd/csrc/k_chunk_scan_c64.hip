// Instantiation of the chunk-scan kernel for chunk size 64 (see k_chunk_scan.h).
#include "k_chunk_scan.h"

namespace cssd {
template hipError_t launch_chunk_scan_c<64>(const FwdArgs& f, hipStream_t s);
}  // namespace cssd
