// fp16 instantiations of the fused attention kernel.
#include "attn_launch.hpp"

namespace mha {
hipError_t launch_attention_f16(const AttnParams& p, hipStream_t stream) {
  return launch_attn_typed<f16>(p, stream);
}
hipError_t launch_attention_split_f16(const AttnParams& p, hipStream_t stream) {
  return launch_attn_split_typed<f16>(p, stream);
}
}  // namespace mha
