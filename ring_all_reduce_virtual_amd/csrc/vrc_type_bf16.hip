// vrc_type_bf16.hip -- the bf16 kernels and their launchers.  One translation
// unit per element type, so the library's kernels compile in parallel.
#include "vrc_launch.hpp"

namespace vrc {
namespace host {
template vrc_status_t run_typed<vrc::BF16>(Coll, vrc_mode_t, const char* const*, char* const*, int, uint64_t, uint64_t,
                                          int, hipStream_t);
}  // namespace host
}  // namespace vrc
