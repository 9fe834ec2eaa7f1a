// vrc_type_f32.hip -- the f32 kernels and their launchers.  One translation
// unit per element type, so the library's kernels compile in parallel.
#include "vrc_launch.hpp"

namespace vrc {
namespace host {
template vrc_status_t run_typed<vrc::F32>(Coll, vrc_mode_t, const char* const*, char* const*, int, uint64_t, uint64_t,
                                          int, hipStream_t);
}  // namespace host
}  // namespace vrc
