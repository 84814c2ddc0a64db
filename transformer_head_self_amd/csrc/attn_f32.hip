// fp32 instantiations of the fused attention kernel.
#include "attn_launch.hpp"

namespace mha {
hipError_t launch_attention_f32(const AttnParams& p, hipStream_t stream) {
  return launch_attn_typed<float>(p, stream);
}
hipError_t launch_attention_split_f32(const AttnParams& p, hipStream_t stream) {
  return launch_attn_split_typed<float>(p, stream);
}
}  // namespace mha
