// Kernels for dk = 16 (see gdn_dk_impl.hpp).
#define GDN_DK 16
#include "gdn_dk_impl.hpp"
