// block_sparse.hip -- GQA block-sparse decode (placeholder until implemented).
#include "common.hpp"
#include "launch.hpp"

namespace sa {
bool block_supported(const BlockArgs&) { return false; }
size_t block_workspace_bytes(int, int, int, int, int, int, int) { return 0; }
hipError_t launch_block_pool(const void*, int, int, int, int, int, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_block_decode(const BlockArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace sa
