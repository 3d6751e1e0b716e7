// Size limits shared by the host-side validation and the kernels (no HIP types).
#pragma once

namespace csa {

constexpr int kCompressNormMaxChannels = 4096;   // RMSNorm of produced entries: channels staged in LDS

}  // namespace csa
