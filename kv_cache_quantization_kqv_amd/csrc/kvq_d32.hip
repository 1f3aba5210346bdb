// Instantiates the gfx950 kernels and dispatchers for head dimension 32.
#include "kvq_kernels.hpp"

namespace kvq {
KVQ_INSTANTIATE(32)
}  // namespace kvq
