// iir_internal.h -- the contract between the host library (iir_host.cpp) and the gfx950 kernels
// (iir_frames.h, iir_frames_*.hip, iir_kernels.hip): tile geometry constants and the one argument
// struct every launch takes by value. One header for both sides, so the host sizes grids and buffers with the numbers the
// kernels assume ("ADR-1392: CUDA motion, PSNR and moment kernels add one atomic per block ...",
// Decision 2 keeps the PSNR block geometry in one header shared by the kernel and its dispatch).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "iir.h"

namespace iir {

constexpr int kWave = 64;          // CDNA wavefront; one wavefront is one workgroup
constexpr int kSumSlots = 64;      // partial slots per sum: the slot of workgroup b is b mod 64
constexpr int kSumGroups = 8;      // slot groups (slot mod 8), each folded by its last workgroup
// finished-workgroup counters: one per slot, then one per slot group
constexpr int kArrivals = kSumSlots + kSumGroups;
constexpr int kSums = 4;           // SAD, SSE_Y, SSE_U, SSE_V
constexpr int kMoments = 4;        // optional: sum ref Y, sum dist Y, sum ref Y^2, sum dist Y^2
constexpr int kMaxSums = kSums + kMoments;
constexpr int kLumaCols = 4;       // luma columns per lane
constexpr int kStripCols = kWave * kLumaCols;  // luma columns per tile (one per 4 per lane)

// Device pointers of one frame pair: ref Y, U, V, then dist Y, U, V.
struct FramePtrs {
    const uint8_t *p[6];
};

struct KernelArgs {
    // frames: plane k of frame t is base[k] + t * fstride[k], unless table is set, in which
    // case it is table[t].p[k]; every frame uses pitch[k]
    const uint8_t *base[6];
    int64_t fstride[6];
    int32_t pitch[6];
    uint32_t span[6];  // readable bytes of each plane (rows * pitch), below 2^32
    const FramePtrs *table;
    // blurred reference luma of the frame before this launch (read when has_prev), and of the
    // launch's last frame (written); tiled: uint2 at [(tile * TH + row) * kWave + lane], TH the
    // launch's rows per tile
    const uint32_t *ring_in;
    uint32_t *ring_out;  // null: the launch keeps no state (its last frame is not stored)
    // per-frame partial sums [nframes][S][kSumSlots], S = kSums, or kMaxSums when the launch
    // also sums the luma moments; zero at launch; the last workgroup of each slot group folds
    // the group's slots and writes its totals to `publish`
    unsigned long long *sums;
    // the other slot buffer (the previous launch's), whose first zero_n words the launch clears
    unsigned long long *zero;
    int64_t zero_n;
    // host-visible [nframes][S][kSumGroups] group totals of this launch (pinned host memory)
    unsigned long long *publish;
    // [kArrivals] zero at launch: finished workgroups of each slot (kSumSlots), then finished
    // slots of each slot group (kSumGroups); the last arrival at a counter resets it
    unsigned int *arrivals;
    int32_t W, H, Wc, Hc;
    int32_t strips, row_tiles, tiles;
    int32_t nframes, chunks, chunk_len;
    int32_t has_prev;
    int32_t shift;  // 16-bit samples: 16 - bit depth, the left shift that scales them to 16 bits
};

// The frames kernel of one configuration, or nullptr: one function per sample type and motion
// variant, each in its own translation unit (iir_frames_8.hip, iir_frames_10.hip,
// iir_frames_16.hip, and the motion v2 units iir_frames_8_v2.hip, iir_frames_10_v2.hip,
// iir_frames_16_v2.hip).
typedef void (*FramesFn)(KernelArgs);
FramesFn frames_pick_8(int th, bool generic, bool moments);
FramesFn frames_pick_8_one(int th, bool generic, bool moments);  // launches of one frame
FramesFn frames_pick_10(int th, bool generic, bool moments);
FramesFn frames_pick_16(int th, bool generic, bool moments);
FramesFn frames_pick_8_v2(int th, bool generic, bool moments);
FramesFn frames_pick_10_v2(int th, bool generic, bool moments);
FramesFn frames_pick_16_v2(int th, bool generic, bool moments, bool wide);

// Host-side launchers (iir_kernels.hip). Each returns the launch's hipError_t.
bool supported_rows_per_tile(int th);           // 12, 16 or 20
bool fast_path_ok(int W, int H, int th);         // the uniform fast path applies
// `moments`: the launch also sums the luma moments (S = kMaxSums); `v2`: the motion sum is the
// motion v2 one (8 to 16 bits), with ring_in / ring_out holding the last frame's reference
// luma as a plane of strips * 256 samples per row instead of the tiled blurred state
hipError_t frames_occupancy(int bpc, int th, bool generic, bool moments, bool v2,
                            int *waves_per_cu);
// start / stop (both or neither): events the launch records as the kernel's own start and end
hipError_t launch_frames(int bpc, int th, bool generic, bool moments, bool v2,
                         const KernelArgs &a, hipStream_t stream, hipEvent_t start = nullptr,
                         hipEvent_t stop = nullptr);
hipError_t launch_export(const uint32_t *ring, uint16_t *dst, int64_t pitch, int W, int H,
                         int strips, int th, hipStream_t stream);
hipError_t launch_probe(int mode, const void *src, void *dst, int64_t bytes, hipStream_t stream);
// Input-range check of a launch's frames (16-bit storage, bpc 9 to 15): a sample >= 2^bpc
// inside a plane's width stores (t * 6 + k) + 1 to *flag, frame t and plane k (ref Y, U, V,
// dist Y, U, V) of one offending sample; *flag is left alone when every sample is in range.
hipError_t launch_check_range(const KernelArgs &a, int bpc, uint32_t *flag, hipStream_t stream);

// Working memory of the entry point that allocates nothing (iir_run_clip_static): one
// file-scope device array per GPU, holding the regions below at 256-byte boundaries. The clip
// runs standalone (no previous frame, no state kept), so no region depends on the frame size.
constexpr int kStaticMaxFrames = IIR_STATIC_MAX_FRAMES;
struct StaticScratch {
    unsigned long long *sums;     // [frames][kMaxSums][kSumSlots] partial slots
    unsigned long long *publish;  // [frames][kMaxSums][kSumGroups] group totals
    iir_result *results;          // [frames] folded results
    FramePtrs *table;             // [frames] plane pointers of a non-uniformly strided clip
    unsigned int *arrivals;       // [kArrivals] finished-workgroup counters
};
// The scratch regions as addressed on the current device (looked up once per device).
hipError_t static_scratch(int device, StaticScratch *out);
// Zero words [0, n) of `sums` and the kArrivals arrival counters (a fill kernel, not a memset,
// so the clearing is an ordinary kernel node for callers that capture the stream).
hipError_t launch_clear(unsigned long long *sums, int64_t n, unsigned int *arrivals,
                        hipStream_t stream);
// Fold each frame's `groups` group totals of `nsums` sums into iir_result rows (has_motion = 1
// for every frame after the first; frame 0 has none).
hipError_t launch_fold(const unsigned long long *publish, int nframes, int nsums, int groups,
                       iir_result *out, hipStream_t stream);

}  // namespace iir
