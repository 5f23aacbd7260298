// Status strings of the C ABI.
#include "../../include/s2a.h"

extern "C" const char* s2a_status_string(int status) {
  switch (status) {
    case S2A_OK: return "ok";
    case S2A_ERR_INVALID_ARG: return "invalid argument";
    case S2A_ERR_UNSUPPORTED: return "unsupported configuration";
    case S2A_ERR_WORKSPACE: return "workspace missing or too small";
    case S2A_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}
