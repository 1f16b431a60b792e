// engram_apply_signsgd.hip -- the sorted scatter-add's apply into the
// SignSGD step on the bf16 table (each distinct row
// updated in place); the kernel is in engram_apply_dev.h.
#include "engram_apply_dev.h"

void engram::walk_signsgd(const WalkArgs &a, hipStream_t s) { dispatch_walkers<kOutSignSGD>(a, s); }
