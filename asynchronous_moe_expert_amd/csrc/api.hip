// Host-only helpers of the C ABI: status strings, version, struct sizes.
#include "common.hpp"

extern "C" const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL_NULL: return "a required pointer is NULL";
    case MOE_EINVAL_SIZE: return "a size is negative or over a documented limit";
    case MOE_EINVAL_DTYPE: return "unsupported dtype or dtype combination";
    case MOE_EINVAL_ALIGN: return "a pointer or pitch is not 16-byte aligned";
    case MOE_EINVAL_SHAPE: return "H or I is not a multiple of the required granule";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_ELAUNCH: return "kernel launch failed";
    case MOE_ESCRATCH: return "more arrivals than the library's static scratch holds";
    default: return "unknown status";
  }
}

extern "C" int moe_version(void) { return MOE_STEP_VERSION; }

extern "C" size_t moe_struct_size(int which) {
  switch (which) {
    case 0: return sizeof(moe_assemble_args);
    case 1: return sizeof(moe_pack_args);
    case 2: return sizeof(moe_ffn_args);
    case 3: return sizeof(moe_combine_state);
    case 4: return sizeof(moe_combine_args);
    default: return 0;
  }
}
