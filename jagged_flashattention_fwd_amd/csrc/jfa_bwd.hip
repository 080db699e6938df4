// Placeholder until the backward kernels land.
#include "jfa_internal.hpp"
namespace jfa {
hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace jfa
