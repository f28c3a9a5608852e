// Anchor-only decode attention (placeholder until the fused kernel lands).
#include "../../include/lynx.h"
#include "lynx_kernels.hpp"

namespace lynx {

size_t attn_workspace_bytes(int, int, int, int, int, int, int) { return 0; }

int attn_anchor_launch(const void*, const void*, const void*, int, int, int, int, int, int, int, float, float,
                       void*, size_t, int, void*, hipStream_t) {
  return LYNX_EUNSUPPORTED;
}

}  // namespace lynx
