// Kernels for dk = 64 (see gdn_dk_impl.hpp).
#define GDN_DK 64
#include "gdn_dk_impl.hpp"
