// gqa_prefill.hip -- bf16 MFMA flash prefill (not yet enabled).
#include "gqa_common.hpp"
#include "gqa_internal.hpp"

namespace gqa {

hipError_t launch_prefill_mfma(const Problem &p, hipStream_t stream) {
    return launch_generic(p, stream);
}

} // namespace gqa
