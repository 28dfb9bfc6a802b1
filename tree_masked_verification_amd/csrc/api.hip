// api.hip -- library-wide entry points of libtmv (status names, ABI version).
#include "tmv_device.hpp"

extern "C" const char *tmv_status_string(int code)
{
    switch (code) {
    case TMV_OK: return "ok";
    case TMV_ERR_ARG: return "invalid argument";
    case TMV_ERR_RANGE: return "parent index out of range";
    case TMV_ERR_CYCLE: return "parent chain has a cycle";
    case TMV_ERR_DEPTH: return "node deeper than D_max";
    case TMV_ERR_CLOSURE: return "valid node under an invalid parent";
    case TMV_ERR_INPUT: return "malformed input data";
    case TMV_ERR_DEVICE: return "kernel launch failed";
    default: return "unknown status";
    }
}

extern "C" int tmv_abi_version(void) { return 2; }
