// engram_stream.hip -- the stream-event operations of engram_run_ops: the
// two HIP calls a schedule of this library's calls needs to order work
// across streams.
#include "engram_internal.h"

int engram::record_event(void *event, void *stream) {
  return hipEventRecord(static_cast<hipEvent_t>(event), as_stream(stream)) == hipSuccess
             ? ENGRAM_OK
             : ENGRAM_EHIP;
}

int engram::wait_event(void *stream, void *event) {
  return hipStreamWaitEvent(as_stream(stream), static_cast<hipEvent_t>(event), 0) == hipSuccess
             ? ENGRAM_OK
             : ENGRAM_EHIP;
}
