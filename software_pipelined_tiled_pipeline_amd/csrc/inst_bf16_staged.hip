// NT kernel instances: bf16 operands, register-staged element-guarded loader.
#include "launch_impl.hpp"

namespace pgemm {

pgemm_status launch_bf16_staged(const NtLaunch &a) { return launch_detail::launch_any<__bf16, true>(a); }

}  // namespace pgemm
