// status.cpp -- names of the C ABI's status codes.
#include "../../include/w8a8.h"

extern "C" const char *w8a8_status_str(w8a8_status status) {
    switch (status) {
    case W8A8_OK: return "W8A8_OK";
    case W8A8_ERR_INVALID_ARG: return "W8A8_ERR_INVALID_ARG: null pointer, negative size or bad enum";
    case W8A8_ERR_SHAPE: return "W8A8_ERR_SHAPE: size or stride outside the layout rules";
    case W8A8_ERR_ALIGN: return "W8A8_ERR_ALIGN: pointer not 16-byte aligned";
    case W8A8_ERR_UNSUPPORTED: return "W8A8_ERR_UNSUPPORTED: combination not implemented";
    case W8A8_ERR_HIP: return "W8A8_ERR_HIP: the HIP runtime reported a launch error";
    case W8A8_ERR_SCRATCH_LIMIT:
        return "W8A8_ERR_SCRATCH_LIMIT: the call needs more than the no-alloc entry point's fixed scratch";
    }
    return "unknown w8a8_status";
}
