// Instantiates the gfx950 kernels and dispatchers for head dimension 64.
#include "kvq_kernels.hpp"

namespace kvq {
KVQ_INSTANTIATE(64)
}  // namespace kvq
