// Instantiates the gfx950 kernels and dispatchers for head dimension 128.
#include "kvq_kernels.hpp"

namespace kvq {
KVQ_INSTANTIATE(128)
}  // namespace kvq
