// Kernel launchers of libgdn replaced by counters, so that the host code of gdn_api.hip (argument
// checks, the AutoCP planner, workspace layout, launch sequence) runs under the host sanitizers
// without a GPU. Test infrastructure only: linked into tests/sanitize/plan_driver.cpp's binary.
#include "gdn_kernels.h"
#include "gdn_norm.h"

int g_launches = 0;

namespace gdn {
hipError_t launch_tables(const TableArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_intra(const IntraArgs&, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decide(const DecideArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_recur(const RecurArgs&, int, int, int64_t, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_scan(const ScanArgs&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fused(const RecurArgs&, int, int64_t, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_reverse(const RevArgs&, int, int, int64_t, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_bwd_chunk(const BwdChunkArgs&, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs&, int, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode_qk_l2norm(const DecodeArgs&, int, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_l2norm_bwd(const NormArgs&, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
}  // namespace gdn
