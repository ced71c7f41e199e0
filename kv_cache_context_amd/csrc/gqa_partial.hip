// placeholder until the GQA kernel lands
#include "dcp_internal.hpp"
namespace dcp {
hipError_t launch_gqa_partial(const GqaArgs&, hipStream_t) { return hipErrorNotSupported; }
}
