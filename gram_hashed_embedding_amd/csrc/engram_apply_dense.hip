// engram_apply_dense.hip -- the sorted scatter-add's apply into the
// dense fp32 gradient table (a read-modify-write of
// each distinct row); the kernel is in engram_apply_dev.h.
#include "engram_apply_dev.h"

void engram::walk_dense(const WalkArgs &a, hipStream_t s) { dispatch_walkers<kOutDense>(a, s); }
