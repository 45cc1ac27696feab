// One compiled variant of the chunked scan: the I/O dtype, the delta
// activation and the half of the dstate range are fixed by
// -DMAMBA_VARIANT_IO=<0|1> (fp32|bf16), -DMAMBA_VARIANT_SP=<0|1> (softplus
// off|on) and -DMAMBA_VARIANT_PART=<0|1> (dstate 1..8|9..16), so the eight
// objects build in parallel.
#include "scan_chunked.h"

#if !defined(MAMBA_VARIANT_IO) || !defined(MAMBA_VARIANT_SP) || !defined(MAMBA_VARIANT_PART)
#error "compile with -DMAMBA_VARIANT_IO=<0|1> -DMAMBA_VARIANT_SP=<0|1> -DMAMBA_VARIANT_PART=<0|1>"
#endif

namespace mamba {
template hipError_t launch_scan_variant<MAMBA_VARIANT_IO, (MAMBA_VARIANT_SP != 0), MAMBA_VARIANT_PART>(
    const ScanArgs&, const ScanPlan&, void*, hipStream_t);
}  // namespace mamba
