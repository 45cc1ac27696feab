// One compiled variant of the chunked scan: the I/O dtype and the delta
// activation are fixed by -DMAMBA_VARIANT_IO=<0|1> (fp32|bf16) and
// -DMAMBA_VARIANT_SP=<0|1> (softplus off|on), so the four variants build in
// parallel as separate objects.
#include "scan_chunked.h"

#if !defined(MAMBA_VARIANT_IO) || !defined(MAMBA_VARIANT_SP)
#error "compile with -DMAMBA_VARIANT_IO=<0|1> -DMAMBA_VARIANT_SP=<0|1>"
#endif

namespace mamba {
template hipError_t launch_scan_variant<MAMBA_VARIANT_IO, (MAMBA_VARIANT_SP != 0)>(
    const ScanArgs&, const ScanPlan&, void*, hipStream_t);
}  // namespace mamba
