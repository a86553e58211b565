// Kernels for dk = 128 (see gdn_dk_impl.hpp).
#define GDN_DK 128
#include "gdn_dk_impl.hpp"
