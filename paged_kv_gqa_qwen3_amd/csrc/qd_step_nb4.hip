// Persistent step kernel instantiated for 4 batch column(s) per GEMV item.
#include "qd_step_impl.h"

namespace qd {
template hipError_t step_dispatch<4>(int, int, const StepArgs*, int, size_t, hipStream_t,
                                       int*, int);
}  // namespace qd
