// NT kernel instances: f16 operands, register-staged element-guarded loader.
#include "launch_impl.hpp"

namespace pgemm {

pgemm_status launch_f16_staged(const NtLaunch &a) { return launch_detail::launch_any<_Float16, true>(a); }

}  // namespace pgemm
