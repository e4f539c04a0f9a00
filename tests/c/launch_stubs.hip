// Stand-ins for the library's kernel launchers, linked with the ABI file alone for the
// host sanitizer build: the test program makes only calls that are rejected, or accepted with
// nothing to enqueue, before a launcher would run, so reaching one is an error.
#include <stdio.h>
#include <stdlib.h>

#include "qmoe_internal.h"

namespace qmoe {

static hipError_t unexpected(const char* what) {
  fprintf(stderr, "launcher reached in the host-only build: %s\n", what);
  abort();
}

hipError_t launch_route(const float*, int, int, int, const moe_routing*, void*, hipStream_t) {
  return unexpected("launch_route");
}
hipError_t launch_decode(const DecodeArgs&) { return unexpected("launch_decode"); }
hipError_t launch_prefill(const PrefillArgs&) { return unexpected("launch_prefill"); }

}  // namespace qmoe
