// Persistent step kernel instantiated for 2 batch column(s) per GEMV item.
#include "qd_step_impl.h"

namespace qd {
template hipError_t step_dispatch<2>(int, int, const StepArgs*, int, size_t, hipStream_t,
                                       int*, int);
}  // namespace qd
