// host_launch_stub.cpp -- stand-ins for the HIP launchers of libengram.so,
// so that the library's host side (csrc/engram_host.cpp: every extern "C"
// entry point and its argument checks) builds and runs on a CPU alone, under
// host sanitizers.  Test infrastructure: each stand-in only checks that the
// entry point handed it a consistent call, touches no pointer, and enqueues
// nothing.
#include <cstdlib>

#include "engram_host.h"

namespace engram {

namespace {
void require(bool ok) {
  if (!ok) std::abort();  // an entry point launched with arguments it should have refused
}
}  // namespace

int launch_hash(const HashParams &hp, int64_t tokens, int64_t *d_row_ids, void *) {
  require(tokens > 0 && d_row_ids != nullptr && hp.tokens != nullptr && hp.H >= 1);
  return ENGRAM_OK;
}

int launch_gather(const int64_t *d_row_ids, int64_t n, const void *d_table, int64_t,
                  int64_t head_dim, void *d_out, int64_t *, void *) {
  require(n > 0 && d_row_ids != nullptr && d_table != nullptr && d_out != nullptr &&
          head_dim % 8 == 0);
  return ENGRAM_OK;
}

int launch_lookup(const HashParams &hp, int64_t n, const void *d_table, int64_t head_dim,
                  void *d_out, int64_t *, void *) {
  require(n > 0 && hp.tokens != nullptr && d_table != nullptr && d_out != nullptr &&
          head_dim % 8 == 0);
  return ENGRAM_OK;
}

int launch_plan(const int64_t *d_row_ids, const HashParams *hp, int64_t n, int64_t,
                const Plan &p, void *d_workspace, int64_t *, void *) {
  require(n > 0 && (d_row_ids != nullptr || hp != nullptr) && d_workspace != nullptr &&
          p.total > 0);
  return ENGRAM_OK;
}

int launch_apply(const void *d_grads, int64_t n, int64_t head_dim, int64_t, const Plan &p,
                 void *d_workspace, const ApplyOut &o, int64_t *, void *) {
  require(n > 0 && d_grads != nullptr && d_workspace != nullptr && head_dim % 8 == 0);
  require(grid_fits(apply_blocks(p, head_dim), kWalkThreads));
  require(o.mode == kOutSignSGD ? o.table != nullptr
          : o.mode == kOutDense ? o.grad_table != nullptr
                                : o.unique_ids != nullptr && o.unique_grads != nullptr &&
                                      o.num_unique != nullptr);
  return ENGRAM_OK;
}

int launch_scatter_atomic(const int64_t *d_row_ids, int64_t n, const void *d_grads, int64_t,
                          float *d_grad_table, int64_t, int64_t *, void *) {
  require(n > 0 && d_row_ids != nullptr && d_grads != nullptr && d_grad_table != nullptr);
  return ENGRAM_OK;
}

int launch_write_zero(int64_t *d_value, void *) {
  require(d_value != nullptr);
  return ENGRAM_OK;
}

int launch_signsgd(const int64_t *d_unique_ids, const float *d_unique_grads,
                   const int64_t *d_num_unique, int64_t capacity, int64_t, void *d_table, int64_t,
                   float, int64_t *, void *) {
  require(capacity > 0 && d_unique_ids != nullptr && d_unique_grads != nullptr &&
          d_num_unique != nullptr && d_table != nullptr);
  return ENGRAM_OK;
}

int launch_ple_conv(const ConvCall &c, void *) {
  require(c.batch > 0 && c.seq > 0 && c.x != nullptr && c.out != nullptr);
  return ENGRAM_OK;
}

// A fake, 256-aligned address: the stand-in launchers never dereference it.
void *static_scratch() { return reinterpret_cast<void *>(uintptr_t(1) << 20); }

int record_event(void *event, void *) {
  require(event != nullptr);
  return ENGRAM_OK;
}

int wait_event(void *, void *event) {
  require(event != nullptr);
  return ENGRAM_OK;
}

}  // namespace engram
