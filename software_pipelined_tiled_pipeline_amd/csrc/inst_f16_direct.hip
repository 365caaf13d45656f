// NT kernel instances: f16 operands, direct-to-LDS loader (and the persistent schedule).
#include "launch_impl.hpp"

namespace pgemm {

pgemm_status launch_f16_direct(const NtLaunch &a) { return launch_detail::launch_any<_Float16, false>(a); }

}  // namespace pgemm
