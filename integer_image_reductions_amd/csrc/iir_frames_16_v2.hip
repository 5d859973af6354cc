// iir_frames_16_v2.hip -- the motion v2 frames kernels of 16-bit storage: depths 9 to 15 (the
// depth from the launch's scale shift) and 16 (halved differences), the 12-row tile, with and
// without moments. Every shape takes the generic path: the fast path's kernel runs out of
// registers here (it schedules the rows' 64-bit squares together and spills), and the generic
// path is exact for every shape.
#include "iir_frames.h"

namespace iir {

FramesFn frames_pick_16_v2(int th, bool /*generic*/, bool moments, bool wide)
{
    if (wide)
        return moments ? frames_fn<16, true, true, 2>(th) : frames_fn<16, true, false, 2>(th);
    return moments ? frames_fn<16, true, true, 1>(th) : frames_fn<16, true, false, 1>(th);
}

}  // namespace iir
