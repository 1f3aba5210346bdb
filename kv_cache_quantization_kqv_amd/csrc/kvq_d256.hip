// Instantiates the gfx950 kernels and dispatchers for head dimension 256.
#include "kvq_kernels.hpp"

namespace kvq {
KVQ_INSTANTIATE(256)
}  // namespace kvq
