// iir_frames_10.hip -- the frames kernels of 10-bit samples: every tile height, both paths, with
// and without moments.
#include "iir_frames.h"

namespace iir {

FramesFn frames_pick_10(int th, bool generic, bool moments)
{
    if (moments)
        return generic ? frames_fn<10, true, true>(th) : frames_fn<10, false, true>(th);
    return generic ? frames_fn<10, true, false>(th) : frames_fn<10, false, false>(th);
}

}  // namespace iir
