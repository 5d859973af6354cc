// iir_frames_16_v2.hip -- the motion v2 frames kernels of 16-bit storage: depths 9 to 15 (the
// depth from the launch's scale shift) and 16 (halved differences), the 12-row tile. With moments
// every shape takes the generic path: the fast path's kernel then spills ~700 bytes per lane
// (it schedules the rows' 64-bit squares together) and measured twice as slow at 4K 16-bit
// (1,952 against 982 us). Without moments the fast path spills 12 bytes and is the faster one
// (661 against 821 us), so aligned shapes take it.
#include "iir_frames.h"

namespace iir {

FramesFn frames_pick_16_v2(int th, bool generic, bool moments, bool wide)
{
    if (moments)
        return wide ? frames_fn<16, true, true, 2>(th) : frames_fn<16, true, true, 1>(th);
    if (wide)
        return generic ? frames_fn<16, true, false, 2>(th) : frames_fn<16, false, false, 2>(th);
    return generic ? frames_fn<16, true, false, 1>(th) : frames_fn<16, false, false, 1>(th);
}

}  // namespace iir
