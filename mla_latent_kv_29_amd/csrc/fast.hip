// MFMA kernels for the DeepSeek-V3 MLA shape (placeholder: not yet enabled).
#include "internal.hpp"

namespace mla {
bool fast_append_supported(const mla_dims&, int) { return false; }
bool fast_decode_supported(const mla_dims&, int, int, int) { return false; }
hipError_t fast_append(const AppendArgs&) { return hipErrorNotSupported; }
hipError_t fast_decode(const DecodeArgs&) { return hipErrorNotSupported; }
hipError_t fast_combine(const CombineArgs&) { return hipErrorNotSupported; }
}  // namespace mla
