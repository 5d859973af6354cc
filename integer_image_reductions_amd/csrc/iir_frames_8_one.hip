// iir_frames_8_one.hip -- the frames kernels of one-frame launches of 8-bit samples (a frame
// pair per submission): every tile height, both paths, with and without moments. They issue the
// previous launch's blurred tile behind the frame's own loads and load one luma group only.
#include "iir_frames.h"

namespace iir {

FramesFn frames_pick_8_one(int th, bool generic, bool moments)
{
    if (moments)
        return generic ? frames_fn_one<true, true>(th) : frames_fn_one<false, true>(th);
    return generic ? frames_fn_one<true, false>(th) : frames_fn_one<false, false>(th);
}

}  // namespace iir
