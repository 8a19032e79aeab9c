// The LUT rung's expert kernels: the shared templates (expert_body.h) instantiated with the
// LUT rung's decoder (a 9-bit pair state indexing a 512 x 2 codebook held in LDS as one copy per
// bank).  A translation unit of its own so that the two rungs compile in parallel.
//
// Source of the rung: m-tile page, PR #167, "The regression" (the LUT rung's grouped kernel) and
// "Applied to both rungs" (one dispatch gate for both); its bit format is a reading, stated with
// the C ABI (include/qtip_moe.h).
#include "expert_body.h"

namespace qtip {

hipError_t launch_expert_lut(int mode, int arm, int variant, const ExpertParams& p, int grid, int waves,
                             hipStream_t stream) {
  return launch_expert_rung<kRungLut>(mode, arm, variant, p, grid, waves, stream);
}

hipError_t launch_dequant_lut(const DequantParams& q, int grid, hipStream_t stream) {
  return launch_dequant_rung<kRungLut>(q, grid, stream);
}

}  // namespace qtip
