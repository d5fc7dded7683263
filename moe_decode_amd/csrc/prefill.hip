// prefill.hip -- placeholder, filled in with the MFMA grouped GEMM
#include "common.hpp"
