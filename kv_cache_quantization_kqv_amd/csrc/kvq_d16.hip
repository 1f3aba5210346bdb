// Instantiates the gfx950 kernels and dispatchers for head dimension 16.
#include "kvq_kernels.hpp"

namespace kvq {
KVQ_INSTANTIATE(16)
}  // namespace kvq
