// Library-wide entry points that launch nothing (contract in include/tg.h).
#include "tg_abi.hpp"

extern "C" const char* tg_status_string(tg_status status)
{
    switch (tg::abi_int(status)) {
    case TG_OK: return "TG_OK: success";
    case TG_ERR_INVALID_VALUE: return "TG_ERR_INVALID_VALUE: invalid size, leading dimension, pointer or enum";
    case TG_ERR_NOT_SUPPORTED: return "TG_ERR_NOT_SUPPORTED: valid request that this library does not implement";
    case TG_ERR_MISALIGNED: return "TG_ERR_MISALIGNED: base pointer or leading dimension not 16-byte aligned";
    case TG_ERR_LAUNCH: return "TG_ERR_LAUNCH: the HIP runtime refused the kernel launch";
    case TG_ERR_SCRATCH: return "TG_ERR_SCRATCH: the problem needs more scratch than the library's static buffer holds";
    default: return "unknown tg_status";
    }
}

extern "C" int32_t tg_version(void) { return 100; /* 0.1.0 */ }
