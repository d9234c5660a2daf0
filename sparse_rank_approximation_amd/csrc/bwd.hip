// bwd.hip -- backward of the ELSAA operator (in progress).
#include "common.hpp"
#include "launch.hpp"

namespace elsaa {

size_t bwd_ws_bytes(const Problem&) { return 0; }
size_t bwd_lds_need(const Problem&) { return 0; }
void launch_bwd(const Problem&, const void*, const void*, const void*, const void*, const void*,
                const void*, const float*, const int32_t*, const int32_t*, const float*,
                const float*, const float*, const float*, const float*, const float*,
                const float*, void*, void*, void*, float*, float*, float*, void*, hipStream_t) {}

}  // namespace elsaa
