// Score and attend kernels (not yet built).
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
size_t scores128_workspace(int segs, int group) { return (size_t)segs * group * 0 + 256; }
size_t attend128_workspace(int segs, int group, int64_t T) { (void)T; return (size_t)segs * group * 0 + 256; }
}  // namespace tq
