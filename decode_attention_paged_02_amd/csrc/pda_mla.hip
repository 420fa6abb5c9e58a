// pda_mla.hip -- MLA latent decode kernels (placeholder until they land).
#include "pda_internal.h"

namespace pda {

hipError_t launch_mla(const MlaArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pda
