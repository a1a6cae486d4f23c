// Instantiation of the chunk-scan kernel for chunk size 16 (kernels in k_chunk_scan.h, k_chunk_scan_lds.h and k_chunk_scan_bf16.h).
#include "k_chunk_scan_bf16.h"

namespace cssd {
template hipError_t launch_chunk_scan_c<16>(const FwdArgs& f, hipStream_t s);
}  // namespace cssd
