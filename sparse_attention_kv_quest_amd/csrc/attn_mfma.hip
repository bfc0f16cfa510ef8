// bf16 GQA decode attention on MFMA (placeholder until the kernel lands).
#include "attn_common.hpp"

namespace se {

bool attn_mfma_supported(const AttnArgs&) { return false; }
se_status launch_attn_mfma(const AttnArgs&, hipStream_t) { return SE_ERR_UNSUPPORTED; }

}  // namespace se
