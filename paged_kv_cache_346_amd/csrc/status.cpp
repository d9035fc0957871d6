// Status names for the C ABI.
#include "../../include/pkv.h"

extern "C" const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "PKV_OK";
    case PKV_EINVAL: return "PKV_EINVAL: invalid argument";
    case PKV_ENOBLOCKS: return "PKV_ENOBLOCKS: not enough free KV blocks";
    case PKV_ENOSEQ: return "PKV_ENOSEQ: unknown sequence id";
    case PKV_EEXIST: return "PKV_EEXIST: sequence id already in use";
    case PKV_EUNSUPPORTED: return "PKV_EUNSUPPORTED: no kernel for this shape or dtype";
    case PKV_EHIP: return "PKV_EHIP: HIP launch or runtime error";
    case PKV_ENOSCRATCH: return "PKV_ENOSCRATCH: needs more than the library's static scratch";
  }
  return "unknown pkv_status";
}
