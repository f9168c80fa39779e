// placeholder: chunked path not built yet
#include "internal.h"
namespace chm {
bool kda_chunked_supported(const KdaArgs&) { return false; }
int64_t kda_chunked_segments(int64_t, int64_t, int64_t, bool) { return 1; }
size_t kda_chunked_workspace(int64_t, int64_t, int64_t, bool) { return 0; }
hipError_t launch_kda_chunked(const KdaArgs&, bool, void*, hipStream_t) { return hipErrorInvalidValue; }
}
