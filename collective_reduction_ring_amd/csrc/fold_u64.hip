// Fold kernels instantiated for one element type (see fold_impl.h).
#include "fold_impl.h"

namespace rsx {

hipError_t launch_fold_u64(int op, int world, bool rs, bool vec, int tpw, const FoldArgs& a, dim3 grid, uint32_t lds,
                           hipStream_t s) {
  return launch_fold<U64T>(op, world, rs, vec, tpw, a, grid, lds, s);
}

hipError_t launch_list_u64(int op, int world, const ListArgs& a, dim3 grid, uint32_t lds, hipStream_t s) {
  return launch_list<U64T>(op, world, a, grid, lds, s);
}

}  // namespace rsx
