// iir_frames_8_v2.hip -- the motion v2 frames kernels of 8-bit samples: every tile height,
// both paths, with and without moments.
#include "iir_frames.h"

namespace iir {

FramesFn frames_pick_8_v2(int th, bool generic, bool moments)
{
    if (moments)
        return generic ? frames_fn<8, true, true, true>(th)
                       : frames_fn<8, false, true, true>(th);
    return generic ? frames_fn<8, true, false, true>(th)
                   : frames_fn<8, false, false, true>(th);
}

}  // namespace iir
