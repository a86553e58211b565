// Kernels for dk = 32 (see gdn_dk_impl.hpp).
#define GDN_DK 32
#include "gdn_dk_impl.hpp"
