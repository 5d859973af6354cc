// iir_frames_16.hip -- the frames kernels of 9- to 16-bit (other than 10) samples: every tile height, both paths, with
// and without moments.
#include "iir_frames.h"

namespace iir {

FramesFn frames_pick_16(int th, bool generic, bool moments)
{
    if (moments)
        return generic ? frames_fn<16, true, true>(th) : frames_fn<16, false, true>(th);
    return generic ? frames_fn<16, true, false>(th) : frames_fn<16, false, false>(th);
}

}  // namespace iir
