// iir_frames_16_v2.hip -- the motion v2 frames kernels of 16-bit storage at depths 9 to 15 (the
// depth from the launch's scale shift): the 12-row tile, with and without moments. Every shape
// takes the generic path: the fast path's kernel runs out of registers here (it schedules the
// rows' 64-bit squares together and spills), and the generic path is exact for every shape.
#include "iir_frames.h"

namespace iir {

FramesFn frames_pick_16_v2(int th, bool /*generic*/, bool moments)
{
    return moments ? frames_fn<16, true, true, true>(th) : frames_fn<16, true, false, true>(th);
}

}  // namespace iir
