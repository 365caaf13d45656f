// NT kernel instances: bf16 operands, direct-to-LDS loader (and the persistent schedule).
#include "launch_impl.hpp"

namespace pgemm {

pgemm_status launch_bf16_direct(const NtLaunch &a) { return launch_detail::launch_any<__bf16, false>(a); }

}  // namespace pgemm
