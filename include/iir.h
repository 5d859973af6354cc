/*
 * iir.h -- C ABI of the integer motion + PSNR library for AMD MI355X (gfx950).
 *
 * Per frame pair of an 8- to 16-bit planar 4:2:0 video, the library returns four exact 64-bit sums:
 *
 *   SAD     sum over the luma plane of |Bl_t - Bl_(t-1)|, where Bl is the reference luma after a
 *           5-tap separable fixed-point Gaussian blur with mirrored edges: the vertical pass is
 *           rounded by a shift of the bit depth and the horizontal pass by a shift of 16
 *           ("ADR-1392: CUDA motion, PSNR and moment kernels add one atomic per block ...",
 *           Context and Decision 4; "Research-0735: CUDA motion kernel ncu hotpath analysis
 *           (576x324)", Key observations 2). Taps (3571, 16004, 26386, 16004, 3571), whole-sample
 *           mirror and round-half-up are this library's readings where the pages give no numbers.
 *   SSE[c]  sum over plane c in {Y, U, V} of (ref - dist)^2 ("ADR-1392", Context and Decision 2).
 *
 * Optionally (IIR_FLAG_MOMENTS) four more: the sums and sums of squares of the reference and the
 * distorted luma, in the same pass. Clip-level scores (iir_motion2, iir_aggregate_of) are host
 * functions of the per-frame results.
 *
 * Every sum is computed exactly in integers, so the order of the reduction does not matter
 * ("ADR-1392", Context: the sums are order-independent). Derived doubles (iir_scores_of) are
 * computed on the host.
 *
 * Frames stay on the device: the caller owns all frame memory (device pointers, e.g. torch
 * tensors); nothing returns to the host inside a frame, and each submission's kernel writes its
 * small per-frame totals straight into pinned host memory, where iir_collect finds them ("ADR-1380:
 * The CUDA SpEED twins are device-resident ...", Decision: the work is enqueued on the picture's
 * stream, a small result per frame comes back, and collect waits once; the pages wait on an event,
 * this library on the totals themselves).
 *
 * Conventions for every call:
 *   - the return value is IIR_OK (0) or a negative IIR_E* code; no call throws or aborts;
 *   - on IIR_EDEVICE the HIP error text is available from iir_last_error() (thread-local);
 *   - a context is used by one host thread at a time and is bound to one HIP stream;
 *   - argument checks happen on the host before any device work is enqueued.
 */
#ifndef IIR_H
#define IIR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IIR_API __attribute__((visibility("default")))

enum {
    IIR_OK = 0,
    IIR_EINVAL = -1,  /* bad argument: null pointer, size, bit depth, pitch or alignment */
    IIR_ENODEV = -2,  /* no usable gfx950 device with that index */
    IIR_ENOMEM = -3,  /* device or pinned host allocation failed (iir_create only) */
    IIR_EDEVICE = -4, /* a HIP call failed; see iir_last_error() */
    IIR_EBUSY = -5,   /* the submission would exceed max_batch uncollected frames */
    IIR_ESTATE = -6,  /* call not valid in the context's current state */
    IIR_ERANGE = -7   /* IIR_FLAG_CHECK_RANGE found a sample >= 2^bpc (iir_collect) */
};

#define IIR_CHROMA_420 420

/* iir_config.flags */
/* time each main kernel with HIP events attached to its dispatch (its own start and end; see
   iir_kernel_time) */
#define IIR_FLAG_TIMING 1u
/*
 * Also sum the luma moments of every frame pair in the same pass (iir_result.moment): the sums
 * and sums of squares of the reference and distorted luma, the four accumulators of the moment
 * kernel ("ADR-1392", Context, and Decision 6).
 */
#define IIR_FLAG_MOMENTS 2u
/*
 * Motion v2 instead of the blurred-frame SAD (every depth, 8 to 16 bits): iir_result.sad becomes
 * SAD2 = sum over the luma plane of |F|, F the same separable filter applied to the difference
 * prev - cur of consecutive reference luma frames, with both rounded shifts taken as floor
 * ("ADR-1392", Decision 4: the kernel stages prev - cur and filters it separably). The context
 * then keeps the last reference luma frame instead of the blurred one; iir_export_blur is not
 * available (IIR_ESTATE).
 */
#define IIR_FLAG_MOTION_V2 4u
/*
 * Debug mode: check that every input sample lies in the bit depth's range, a precondition the
 * kernels do not verify. The pages fix the depths (8, 10 and 16-bit inputs, "ADR-1392",
 * Consequences) but no check of the samples; this one is the library's own. At 9 to 15 bits each
 * submission first runs a check kernel over its frames (every plane, every sample inside the
 * plane's width; pitch padding is ignored), which costs one more read of the frames. At 8 and 16
 * bits every stored value is a valid sample and nothing runs. iir_collect then returns IIR_ERANGE
 * when a frame it returns held a sample >= 2^bpc, after writing all of its results as usual
 * (those frames' sums are unspecified, and so is the motion state after them: call iir_reset);
 * iir_last_error names the result, the frame within its launch, and the plane. Not available
 * in iir_run_clip_static (IIR_EINVAL).
 */
#define IIR_FLAG_CHECK_RANGE 8u

/*
 * One plane of one frame. data is a DEVICE pointer, pitch is the distance between rows in bytes.
 * Samples are uint8 (bpc 8) or little-endian uint16 holding 0..2^bpc - 1 (bpc 9 to 16; the pages
 * check their outputs at 8, 10 and 16 bits, "ADR-1392", Consequences). data and pitch must
 * both be multiples of 16 bytes, pitch >= width * bytes-per-sample, and height * pitch < 2^32.
 * The whole height * pitch bytes must be readable device memory (the kernels load whole 16-byte
 * aligned groups, which may reach past the last column of a row up to its pitch; those bytes never
 * affect a result). Samples >= 2^bpc are a precondition violation: the sums are then unspecified
 * (the kernels still stay in bounds).
 */
typedef struct iir_plane {
    const void *data;
    int64_t pitch;
    int32_t width;
    int32_t height;
} iir_plane;

/* A 4:2:0 frame: plane[0] = Y (W x H), plane[1] = U, plane[2] = V (ceil(W/2) x ceil(H/2)). */
typedef struct iir_frame {
    iir_plane plane[3];
} iir_frame;

typedef struct iir_config {
    int32_t width;     /* luma width, >= 3 and <= 32768 */
    int32_t height;    /* luma height, >= 3 and <= 32768 */
    int32_t bpc;       /* bit depth, 8 to 16 */
    int32_t chroma;    /* IIR_CHROMA_420 */
    int32_t max_batch; /* max frames uncollected at once, over at most 64 pending submissions */
    uint32_t flags;    /* IIR_FLAG_* */
} iir_config;

/*
 * Exact sums of one frame pair. has_motion is 0 for the first frame after iir_create or iir_reset
 * (there is no previous blurred frame; sad is then 0) and 1 otherwise. moment = {sum of ref Y,
 * sum of dist Y, sum of ref Y^2, sum of dist Y^2} over the luma plane with IIR_FLAG_MOMENTS, else
 * all 0.
 */
typedef struct iir_result {
    uint64_t sad;
    uint64_t sse[3];
    uint64_t moment[4];
    int32_t has_motion;
    int32_t reserved;
} iir_result;

/*
 * Scores derived from one iir_result on the host in IEEE double ("ADR-1392", Consequences names
 * the psnr_*, mse_* and motion outputs; the formulas are this library's readings):
 *   motion    = sad / (256 * W * H)   (mean absolute blurred difference in 8-bit units; 0 when
 *                                      has_motion is 0)
 *   mse[c]    = sse[c] / (W_c * H_c)
 *   psnr[c]   = 10 * log10(peak^2 / mse[c]), peak = 2^bpc - 1; +infinity when sse[c] == 0
 *   moment[k] = result moment[k] / (W * H): the first and second moments of ref and dist luma
 *               (0 unless the result came from a context with IIR_FLAG_MOMENTS).
 */
typedef struct iir_scores {
    double motion;
    double mse[3];
    double psnr[3];
    double moment[4];
} iir_scores;

/*
 * Clip aggregates of n consecutive results (pure host code; "ADR-1392", Consequences names the
 * apsnr_* and integer_motion2 outputs without formulas, so these are this library's readings):
 *   sse[c]       = the clip's total squared error of plane c (exact)
 *   apsnr[c]     = 10 * log10(peak^2 / (sse[c] / (n * W_c * H_c))); +infinity when sse[c] == 0
 *   mean_motion  = the mean of the frames' motion scores (iir_scores.motion)
 *   mean_motion2 = the mean of the frames' motion2 scores (iir_motion2)
 */
typedef struct iir_aggregate {
    uint64_t sse[3];
    double apsnr[3];
    double mean_motion;
    double mean_motion2;
    int32_t frames;
    int32_t reserved;
} iir_aggregate;

typedef struct iir_ctx iir_ctx;

/*
 * Create a context for one frame geometry on HIP device `device`, enqueuing all of its work on
 * `hip_stream` (a hipStream_t; NULL means the device's null stream). Allocates everything the
 * context will ever use: the blurred-luma state (two planes of uint16 in a tiled layout), the
 * device sum slots, pinned readback and descriptor staging, and (IIR_FLAG_TIMING) events; with
 * IIR_FLAG_CHECK_RANGE, a pinned word per pending submission. Nothing is allocated
 * afterwards ("Making it fast: three rounds on one pipeline", Round 2: allocation and freeing on
 * the hot path were the largest single cost, removed by keeping and reusing the buffers). The
 * launch geometry is sized from the device's compute units and checked here, once ("ADR-1226:
 * Size the CUDA AIM CM launch by SM count ...", Decision; "ADR-1380: The CUDA SpEED twins are
 * device-resident ...", Consequences: an oversized launch failed only at run time).
 * Errors: IIR_EINVAL (config), IIR_ENODEV (no such device or not gfx950), IIR_ENOMEM,
 * IIR_EDEVICE. *out is set only on success.
 */
IIR_API int iir_create(const iir_config *cfg, int32_t device, void *hip_stream, iir_ctx **out);

/*
 * Enqueue one frame pair (asynchronous: returns before the GPU runs it). ref and dist are host
 * structs describing device planes; the planes must stay valid and unmodified until the result
 * has been collected. One kernel launch, which writes the frame's totals into pinned host memory
 * itself; no copy and no host wait ("ADR-1380", Decision: the work is enqueued on the picture's
 * stream with a small result per frame).
 * Errors: IIR_EINVAL, IIR_EBUSY (the pending results would exceed max_batch frames or 64
 * submissions), IIR_EDEVICE.
 */
IIR_API int iir_submit(iir_ctx *ctx, const iir_frame *ref, const iir_frame *dist);

/*
 * Opt-in coalescing of one-frame submissions, for callers that can wait for a result until a few
 * more frames have been submitted. With frames = K > 1, iir_submit records the frame pair's
 * descriptors on the host and enqueues nothing until K pairs are recorded; those then go out as
 * one launch of K frames, with the sums of K separate submissions. iir_submit_clip, iir_collect,
 * iir_reset, iir_export_blur and iir_set_coalesce itself first enqueue whatever is recorded; a
 * recorded frame counts as pending (iir_run_clip returns IIR_ESTATE, iir_submit IIR_EBUSY when it
 * would not fit). The frames must stay valid until collected, as always. Default 1 (every
 * iir_submit is its own launch, as "ADR-1380", Decision, enqueues every frame's chain on its
 * picture's stream); K = 1 switches it off again. A launch has a fixed cost beside its per-frame
 * cost, and K frames share it. Errors: IIR_EINVAL (K outside 1..min(64, max_batch)), and those of
 * the launch that enqueues the recorded frames.
 */
IIR_API int iir_set_coalesce(iir_ctx *ctx, int32_t frames);

/*
 * Enqueue nframes consecutive frame pairs in one launch (asynchronous). ref[t] and dist[t]
 * describe frame t; every frame of a clip must use frame 0's pitches. When every plane advances
 * by a constant byte stride from frame to frame (e.g. one (F, H, W) tensor per plane), the
 * pointers travel in the kernel arguments; otherwise a descriptor table is copied to the device
 * first. Results are appended to the pending queue in frame order. Motion continues from the
 * previous submission's last frame. Errors: IIR_EINVAL (nframes < 1 or > max_batch, bad frame),
 * IIR_EBUSY, IIR_EDEVICE.
 */
IIR_API int iir_submit_clip(iir_ctx *ctx, const iir_frame *ref, const iir_frame *dist,
                            int32_t nframes);

/*
 * Copy up to `max` pending results, oldest first, into the HOST array `out`; *n_out receives the
 * number copied. Waits once, for the submission holding the last result returned (later
 * submissions keep running; "ADR-1380", Consequences (Positive): one small readback and one wait
 * per frame, no host work inside it). Results beyond `max` stay queued for the next call. With nothing
 * pending it returns IIR_OK with *n_out = 0. Errors: IIR_EINVAL (null out or n_out, max < 0),
 * IIR_EDEVICE, IIR_ERANGE (IIR_FLAG_CHECK_RANGE: a returned frame held an out-of-range sample;
 * out and *n_out are filled all the same).
 */
IIR_API int iir_collect(iir_ctx *ctx, iir_result *out, int32_t max, int32_t *n_out);

/*
 * iir_submit_clip followed by iir_collect of exactly those nframes results into the host array
 * `out` (which must hold nframes entries). Requires nothing else pending (IIR_ESTATE otherwise).
 * One launch for the whole clip, one wait ("ADR-1380", Consequences (Positive); the clip stays
 * resident on the device, "ADR-1392", Consequences (Negative): copying frames in dominates).
 */
IIR_API int iir_run_clip(iir_ctx *ctx, const iir_frame *ref, const iir_frame *dist,
                         int32_t nframes, iir_result *out);

/* Derive the scores of one result for a configuration (pure host code). Errors: IIR_EINVAL. */
IIR_API int iir_scores_of(const iir_config *cfg, const iir_result *r, iir_scores *s);

/*
 * Second motion score of each of n consecutive frames from their motion scores (reading of the
 * integer_motion2 output named by "ADR-1392", Consequences): motion2[t] = min(motion[t],
 * motion[t + 1]); the last frame keeps its own motion. motion2 may alias motion. Errors:
 * IIR_EINVAL (NULL array, n < 1).
 */
IIR_API int iir_motion2(const double *motion, int32_t n, double *motion2);

/* Aggregate n >= 1 consecutive results of one clip (see iir_aggregate). Errors: IIR_EINVAL. */
IIR_API int iir_aggregate_of(const iir_config *cfg, const iir_result *r, int32_t n,
                             iir_aggregate *out);

/*
 * Forget the previous frame: the next submitted frame gets has_motion = 0, as the first frame of a
 * clip does. Enqueues nothing. (The context keeps the previous frame's state on the device between
 * submissions, as the temporal extractor keeps the previous luma in a slot: "ADR-1380",
 * Decision, second item.)
 */
IIR_API int iir_reset(iir_ctx *ctx);

/*
 * Write the blurred reference luma of the most recently submitted frame as a W x H uint16 plane
 * into the DEVICE buffer dst (row pitch `pitch` bytes, >= 2 W, multiple of 4), enqueued on the
 * context's stream. IIR_ESTATE if no frame has been submitted since create/reset, or with
 * IIR_FLAG_MOTION_V2 (which keeps no blurred frame).
 */
IIR_API int iir_export_blur(iir_ctx *ctx, void *dst, int64_t pitch);

/*
 * Duration in milliseconds of the main kernel of the most recently collected submission, from the
 * HIP start and stop events attached to its dispatch (hipExtLaunchKernelGGL) on the context's
 * stream: the kernel's own time, as the pages' kernel traces report it ("ADR-1392",
 * Consequences (Positive)). Needs IIR_FLAG_TIMING; IIR_ESTATE until a timed submission has been
 * collected.
 */
IIR_API int iir_kernel_time(iir_ctx *ctx, float *ms);

/*
 * Number of collected timed launches and their summed kernel milliseconds since create or the
 * last reset (reset != 0 clears the counters after reading them). Needs IIR_FLAG_TIMING for
 * non-zero counts.
 */
IIR_API int iir_kernel_stats(iir_ctx *ctx, int32_t reset, int64_t *launches, double *total_ms);

/* Launch geometry chosen at create from the device's compute units, for reports and tests
   ("ADR-1226", Decision: the launch is sized by the processor count). Three environment variables,
   read at create, override the choice for tuning and tests: IIR_ROWS_PER_TILE (12, 16 or 20),
   IIR_TARGET_WAVES (a cap on the wavefronts a launch's time chunks may fill) and IIR_MIN_CHUNK
   (the fewest frames per time chunk, default 2). */
typedef struct iir_geometry {
    int32_t rows_per_tile;     /* output luma rows per wavefront tile */
    int32_t lanes_out;         /* output lanes per wavefront (4 luma columns each): 64 */
    int32_t strips;            /* tiles across: ceil(W / 256) */
    int32_t row_tiles;         /* tiles down */
    int32_t tiles;             /* strips * row_tiles */
    int32_t sum_slots;         /* partial accumulators per sum (64), folded on the device in 8
                                  groups whose totals the host adds */
    int32_t max_chunks;        /* most time chunks one launch may split a clip into */
} iir_geometry;
IIR_API int iir_get_geometry(const iir_ctx *ctx, iir_geometry *out);

/* Time chunks the next iir_submit_clip of nframes frames will use (1 = no split); small frames
   are split so the launch fills the GPU ("ADR-1226", Decision). */
IIR_API int iir_plan_chunks(const iir_ctx *ctx, int32_t nframes, int32_t *chunks);

/*
 * Memory-ceiling probe in the manner of "Making it fast: three rounds on one pipeline", section
 * "First, find the ceiling": a kernel that only moves memory. mode 0 reads `bytes` from src,
 * mode 1 writes `bytes` to dst, mode 2 copies src to dst. src/dst are DEVICE buffers of at least
 * `bytes` (multiple of 4096, 16-byte aligned). Runs `iters` launches on hip_stream between two
 * events and returns the mean milliseconds per launch in *ms. Errors: IIR_EINVAL, IIR_EDEVICE.
 */
IIR_API int iir_probe_bandwidth(int32_t device, void *hip_stream, int32_t mode, const void *src,
                                void *dst, int64_t bytes, int32_t iters, float *ms);

/*
 * For callers that cannot allocate device memory (code running under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): iir_run_clip without a context. Computes the
 * sums of nframes consecutive frame pairs of a standalone clip -- frame 0 has no previous frame
 * (has_motion 0), exactly as the first iir_run_clip after iir_create -- and writes them to `out`
 * (nframes entries, host or device memory), then waits for the stream. cfg as for iir_create
 * (max_batch is not used; IIR_FLAG_TIMING is ignored); ref/dist as for iir_submit_clip. Enqueues
 * on hip_stream (NULL: the null stream) of HIP device `device`: a clearing kernel, the frames
 * kernel, a folding kernel and one copy into `out`.
 *
 * Calls no hipMalloc, hipFree or other allocating routine: its working memory is a fixed array of
 * about 1.2 MB in the library's device data, one copy per GPU, kept until the process ends, which
 * bounds a call to IIR_STATIC_MAX_FRAMES frames (IIR_EINVAL beyond). The frame size is not
 * bounded by it. Every call on one GPU uses that GPU's array: calls that overlap on one GPU (two
 * host threads, or two streams in flight) race and give wrong sums; serialise them. Errors:
 * IIR_EINVAL, IIR_ENODEV, IIR_EDEVICE.
 */
#define IIR_STATIC_MAX_FRAMES 256
IIR_API int iir_run_clip_static(const iir_config *cfg, int32_t device, void *hip_stream,
                                const iir_frame *ref, const iir_frame *dist, int32_t nframes,
                                iir_result *out);

/* Release everything the context owns, once, off the hot path ("Making it fast", Round 2). Waits
   for its pending work first. NULL is a no-op. */
IIR_API void iir_destroy(iir_ctx *ctx);

/* Static text for an IIR_* code. */
IIR_API const char *iir_strerror(int code);

/* Detail of the last failure on this thread (HIP error text or the failed check). */
IIR_API const char *iir_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IIR_H */
