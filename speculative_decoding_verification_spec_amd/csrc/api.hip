// Library identity and status names for the verification-step C ABI.
#include "spec_verify.h"

extern "C" const char* spec_version(void) { return "specverify 0.1.0 gfx950"; }

extern "C" const char* spec_status_string(spec_status_t s) {
  switch (s) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_ARG: return "SPEC_ERR_ARG";
    case SPEC_ERR_OVERFLOW: return "SPEC_ERR_OVERFLOW";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED";
    case SPEC_ERR_LAUNCH: return "SPEC_ERR_LAUNCH";
    case SPEC_ERR_SCRATCH: return "SPEC_ERR_SCRATCH";
  }
  return "SPEC_ERR_UNKNOWN";
}
