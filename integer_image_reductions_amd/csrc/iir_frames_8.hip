// iir_frames_8.hip -- the frames kernels of 8-bit samples: every tile height, both paths, with
// and without moments.
#include "iir_frames.h"

namespace iir {

FramesFn frames_pick_8(int th, bool generic, bool moments)
{
    if (moments)
        return generic ? frames_fn<8, true, true>(th) : frames_fn<8, false, true>(th);
    return generic ? frames_fn<8, true, false>(th) : frames_fn<8, false, false>(th);
}

}  // namespace iir
