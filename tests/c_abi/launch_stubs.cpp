// Stand-ins for the device launchers, for a host-only build of api.cpp under
// the address and undefined-behaviour sanitizers. The host checks driver only
// reaches calls that fail their argument checks, so none of these may run.
#include <stdio.h>
#include <stdlib.h>

#include "../../zero_dp_partitioned_amd/csrc/zero_dp_internal.h"

namespace zdp {

static hipError_t never(const char* what) {
  fprintf(stderr, "host checks: %s reached a launch\n", what);
  abort();
}

hipError_t launch_adam(const AdamArgs&, int, bool, int, size_t, hipStream_t, int*) { return never("adam"); }
hipError_t launch_reduce(const ReduceArgs&, int, bool, size_t, hipStream_t, int*) { return never("reduce"); }
hipError_t launch_scan(const ReduceArgs&, int, hipStream_t, int*) { return never("scan"); }
int scan_grid(int64_t) { return 1; }
hipError_t launch_fold(const FoldArgs&, hipStream_t) { return never("fold"); }
hipError_t launch_finalize(const FinalizeArgs&, hipStream_t) { return never("finalize"); }
hipError_t launch_commit(const CommitArgs&, hipStream_t) { return never("commit"); }
hipError_t launch_redo_commit(const CommitArgs&, hipStream_t) { return never("redo commit"); }
hipError_t launch_state_init(zero_step_state*, float, hipStream_t) { return never("state init"); }
hipError_t launch_cast(const CastArgs&, bool, hipStream_t) { return never("cast"); }
hipError_t launch_restore(const RestoreArgs&, bool, hipStream_t) { return never("restore"); }
hipError_t static_scratch(void**) { return never("static scratch"); }
hipError_t launch_copy_probe(const void*, const void*, void*, void*, int64_t, hipStream_t) { return never("copy probe"); }

}  // namespace zdp
