// Instantiates the gfx950 kernels and dispatchers for head dimension 8.
#include "kvq_kernels.hpp"

namespace kvq {
KVQ_INSTANTIATE(8)
}  // namespace kvq
