// engram_apply_sparse.hip -- the sorted scatter-add's apply into the
// row-sparse output (the ascending distinct rows and
// their fp32 sums); the kernel is in engram_apply_dev.h.
#include "engram_apply_dev.h"

void engram::walk_sparse(const WalkArgs &a, hipStream_t s) { dispatch_walkers<kOutSparse>(a, s); }
