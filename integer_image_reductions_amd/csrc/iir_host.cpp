// iir_host.cpp -- the C ABI of include/iir.h: argument checks, context lifetime, the submission
// queue and the score derivation. All device work goes to the gfx950 kernels (iir_frames.h and
// iir_kernels.hip).
//
// Per submission the context enqueues, on the caller's stream: (only for a non-uniformly strided
// clip) one host-to-device copy of the frame table, (only with IIR_FLAG_CHECK_RANGE at 9 to 15
// bits) the input-range check, and one frames kernel launch, whose last workgroups write the
// per-frame totals into pinned host memory; iir_collect waits once, until they are all there
// ("ADR-1380: The CUDA SpEED twins are device-resident ...", Decision: submit on the picture's
// stream, read the small result back, collect waits once). The totals are their own completion
// signal: an event packet per submission cost about 3 us of GPU time between one-frame launches.
// Everything is allocated in iir_create ("Making it fast: three rounds on one pipeline", Round 2:
// no allocation or free on the hot path).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "iir.h"
#include "iir_internal.h"

using namespace iir;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int fail_hip(hipError_t e, const char *what)
{
    return fail(IIR_EDEVICE, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

#define HIP_TRY(expr)                                   \
    do {                                                \
        hipError_t e_ = (expr);                         \
        if (e_ != hipSuccess)                           \
            return fail_hip(e_, #expr);                 \
    } while (0)

// Makes `device` current for the scope of one API call and restores the caller's device.
struct DeviceScope {
    int saved = -1;
    hipError_t err = hipSuccess;
    explicit DeviceScope(int device)
    {
        err = hipGetDevice(&saved);
        if (err == hipSuccess && saved != device)
            err = hipSetDevice(device);
    }
    ~DeviceScope()
    {
        if (saved >= 0)
            (void)hipSetDevice(saved);
    }
};

constexpr int kAlign = 16;

}  // namespace

struct iir_ctx {
    iir_config cfg{};
    int device = 0;
    hipStream_t stream = nullptr;
    int bps = 1;  // bytes per sample
    int Wc = 0, Hc = 0;
    int lanes_out = 0, strips = 0, row_tiles = 0, tiles = 0;
    int rows_per_tile = 16;
    int target_waves = 0;   // cap on the wavefronts chunks may fill (0: none)
    int fill = 1;           // wavefronts a launch's time chunks may fill
    int min_chunk = 2;
    int max_chunks = 1;
    bool check_range = false;  // IIR_FLAG_CHECK_RANGE at 9 to 15 bits: a check kernel runs first
    bool moments = false;  // IIR_FLAG_MOMENTS: the kernels also sum the luma moments
    bool v2 = false;       // IIR_FLAG_MOTION_V2: motion of the filtered frame difference
    int nsums = kSums;     // 64-bit sums per frame: kSums, or kMaxSums with moments
    uint32_t *ring[2] = {nullptr, nullptr};
    // ring[ring_cur] holds the blurred state of the last submitted frame (motion v2: its
    // reference luma, as a plane of strips * 256 samples per row, which fits the same bytes)
    int ring_cur = 0;
    // device, two slot buffers of [max_batch][nsums][kSumSlots] u64 that launches alternate
    // between; the one a launch uses is zero (the launch before cleared it)
    unsigned long long *sums = nullptr;
    int sums_cur = 0;         // the buffer the next launch uses
    int64_t sums_dirty = 0;   // words of the other buffer the last launch left non-zero
                                              // between launches (each launch re-zeroes it)
    unsigned int *arrivals = nullptr;         // device, [kArrivals] finished-workgroup counters, zero
    int64_t sums_n = 0;
    // pinned coherent, [max_batch][nsums][kSumGroups] group totals (the launch's last workgroup of
    // each slot group writes its group's; the host adds the groups)
    unsigned long long *host_sums = nullptr;
    unsigned long long *host_sums_dev = nullptr;  // the same memory as the device sees it
    FramePtrs *table_dev = nullptr;
    FramePtrs *table_host = nullptr;  // pinned, [max_batch]
    // pinned coherent, [kMaxPending]: per pending submission, 0 or the input-range check's code
    // (t * 6 + k) + 1 of an out-of-range sample (IIR_FLAG_CHECK_RANGE)
    uint32_t *range_host = nullptr;
    uint32_t *range_dev = nullptr;
    // Pending submissions, oldest first, in a ring of kMaxPending records. Their results sit in
    // a circular region of max_batch frame slots of host_sums (and table slots), each submission
    // contiguous, so up to max_batch frames can be in flight across several submissions.
    struct Sub {
        int first;       // first frame slot
        int n;           // frames
        int taken;       // frames already returned by iir_collect
        bool has_prev;   // frame 0 has a previous frame
        int groups;      // slot groups with workgroups in the launch (their totals are valid)
        hipEvent_t k0, k1;  // bracket the main kernel (IIR_FLAG_TIMING)
    };
    static constexpr int kMaxPending = 64;
    Sub subs[kMaxPending] = {};
    int sub_head = 0;    // oldest pending submission
    int sub_count = 0;   // pending submissions
    int slot_head = 0;   // next free frame slot
    int pending = 0;     // frames submitted and not yet returned
    // iir_set_coalesce: one-frame submissions are recorded here and enqueued `coalesce` at a time
    // as one launch (1: every submission is its own launch)
    static constexpr int kMaxCoalesce = 64;
    int coalesce = 1;
    int deferred = 0;
    iir_frame def_ref[kMaxCoalesce] = {};
    iir_frame def_dist[kMaxCoalesce] = {};
    bool has_prev = false;            // the next frame has a previous blurred frame
    bool any_frame = false;           // ring[ring_cur] is valid
    // kernel timing of collected submissions (IIR_FLAG_TIMING)
    float last_ms = -1.f;
    int64_t timed_launches = 0;
    double timed_ms = 0.0;
};

namespace {

int env_int(const char *name, int dflt, int lo, int hi)
{
    const char *v = getenv(name);
    if (!v || !*v)
        return dflt;
    long x = strtol(v, nullptr, 10);
    return (int)std::min<long>(std::max<long>(x, lo), hi);
}

int check_config(const iir_config *c)
{
    if (!c)
        return fail(IIR_EINVAL, "config is NULL");
    if (c->bpc < 8 || c->bpc > 16)
        return fail(IIR_EINVAL, "bpc must be 8 to 16, got %d", c->bpc);
    if (c->chroma != IIR_CHROMA_420)
        return fail(IIR_EINVAL, "only 4:2:0 (chroma = %d) is supported", IIR_CHROMA_420);
    if (c->width < 3 || c->height < 3 || c->width > 32768 || c->height > 32768)
        return fail(IIR_EINVAL, "frame size %dx%d outside 3..32768", c->width, c->height);
    if (c->max_batch < 1 || c->max_batch > 65536)
        return fail(IIR_EINVAL, "max_batch %d outside 1..65536", c->max_batch);
    if (c->flags &
        ~(IIR_FLAG_TIMING | IIR_FLAG_MOMENTS | IIR_FLAG_MOTION_V2 | IIR_FLAG_CHECK_RANGE))
        return fail(IIR_EINVAL, "unknown flags 0x%x", c->flags);
    return IIR_OK;
}

int check_plane(const iir_ctx *c, const iir_plane &p, int idx, const char *which)
{
    const int w = idx == 0 ? c->cfg.width : c->Wc;
    const int h = idx == 0 ? c->cfg.height : c->Hc;
    if (!p.data)
        return fail(IIR_EINVAL, "%s plane %d: data is NULL", which, idx);
    if (p.width != w || p.height != h)
        return fail(IIR_EINVAL, "%s plane %d: %dx%d, expected %dx%d", which, idx, p.width,
                    p.height, w, h);
    if (p.pitch < (int64_t)w * c->bps || p.pitch > INT32_MAX)
        return fail(IIR_EINVAL, "%s plane %d: pitch %lld outside [%lld, 2^31)", which, idx,
                    (long long)p.pitch, (long long)w * c->bps);
    if ((int64_t)h * p.pitch > (int64_t)UINT32_MAX)
        return fail(IIR_EINVAL, "%s plane %d: %d rows of pitch %lld exceed 4 GiB", which, idx, h,
                    (long long)p.pitch);
    if ((p.pitch % kAlign) || ((uintptr_t)p.data % kAlign))
        return fail(IIR_EINVAL, "%s plane %d: data and pitch must be multiples of %d bytes", which,
                    idx, kAlign);
    return IIR_OK;
}

int check_frames(const iir_ctx *c, const iir_frame *ref, const iir_frame *dist, int n)
{
    if (!ref || !dist)
        return fail(IIR_EINVAL, "frame array is NULL");
    for (int t = 0; t < n; ++t)
        for (int k = 0; k < 3; ++k) {
            int rc = check_plane(c, ref[t].plane[k], k, "ref");
            if (rc == IIR_OK)
                rc = check_plane(c, dist[t].plane[k], k, "dist");
            if (rc != IIR_OK)
                return rc;
            if (ref[t].plane[k].pitch != ref[0].plane[k].pitch ||
                dist[t].plane[k].pitch != dist[0].plane[k].pitch)
                return fail(IIR_EINVAL, "frame %d plane %d: every frame must share frame 0's pitch",
                            t, k);
        }
    return IIR_OK;
}

const uint8_t *plane_ptr(const iir_frame *ref, const iir_frame *dist, int t, int k)
{
    return static_cast<const uint8_t *>(k < 3 ? ref[t].plane[k].data : dist[t].plane[k - 3].data);
}

// Columns: strips of kStripCols luma columns, each starting on a 256-column boundary, so a
// wavefront's rows are whole aligned cache lines that no other wavefront loads.
void choose_columns(iir_ctx *c)
{
    c->strips = (c->cfg.width + kStripCols - 1) / kStripCols;
    c->lanes_out = kWave;
}

// Time chunks for a launch of n frames over `tiles` tiles, filling at most `fill` wavefronts at
// once: as many chunks as fit, each of at least min_chunk frames (every chunk after the first
// re-blurs the frame before it, so a one-frame chunk doubles its blur work). With few tiles (small
// frames) the chunks give each SIMD a second wavefront to overlap its loads with; more than two
// per SIMD measured slower (1080p: 2 chunks 87 us, 3 or 4 chunks 92 us), since more fronts of
// frames in flight push the halo rows a tile shares with its neighbours out of each XCD's L2.
int chunks_for(int64_t tiles, int64_t fill, int n, int min_chunk)
{
    if (n < 2 * min_chunk || tiles >= fill)
        return 1;
    int chunks = (int)std::max<int64_t>(1, std::min<int64_t>(fill / tiles, n / min_chunk));
    // no empty chunks
    const int len = (n + chunks - 1) / chunks;
    return (n + len - 1) / len;
}

// Rows per tile: each candidate's kernel has its own register footprint and hence its own number
// of resident wavefronts per CU (its slots). A launch whose tiles all fit at once finishes when
// its busiest SIMD does, so the estimated cost is (wavefronts per SIMD, rounded up) x (rows + the
// 4 halo rows each tile re-reads), times the number of rounds when they do not all fit. The
// generic path (ragged sizes) costs half as much again per row: at 960x544 the 12-row generic
// kernel lost to the 16-row fast one.
int choose_rows(iir_ctx *c, int cus, int forced, int *slots_out)
{
    static const int kCandidates[] = {12, 16, 20};
    int best = 0;  // none: no kernel for this configuration
    double best_cost = 1e300;
    for (int th : kCandidates) {
        if (forced && th != forced)
            continue;
        int per_cu = 0;
        const bool generic = !fast_path_ok(c->cfg.width, c->cfg.height, th);
        if (frames_occupancy(c->cfg.bpc, th, generic, c->moments, c->v2, &per_cu) !=
                hipSuccess ||
            per_cu < 1)
            continue;
        const int64_t waves = (int64_t)c->strips * ((c->cfg.height + th - 1) / th);
        const int64_t slots = (int64_t)per_cu * cus;
        const int64_t simds = 4LL * cus;
        const int64_t rounds = (waves + slots - 1) / slots;
        const int64_t per_simd = (std::min(waves, slots) + simds - 1) / simds;
        const double cost = (double)rounds * (double)per_simd * (th + 4) * (generic ? 1.5 : 1.0);
        if (cost < best_cost - 1e-9 || (cost <= best_cost + 1e-9 && th > best)) {
            best_cost = cost;
            best = th;
            *slots_out = (int)std::min<int64_t>(slots, INT32_MAX);
        }
    }
    return best;
}

int plan_chunks(const iir_ctx *c, int nframes)
{
    return chunks_for(c->tiles, c->fill, nframes, c->min_chunk);
}

// The launch geometry of a configuration on a device with `cus` compute units: sample size,
// chroma size, tile columns and rows, the time-chunk policy. Touches no device memory.
int setup_geometry(iir_ctx *c, const iir_config *cfg, int device, int cus)
{
    c->cfg = *cfg;
    c->device = device;
    c->bps = cfg->bpc == 8 ? 1 : 2;
    c->Wc = (cfg->width + 1) / 2;
    c->Hc = (cfg->height + 1) / 2;
    c->moments = (cfg->flags & IIR_FLAG_MOMENTS) != 0;
    c->v2 = (cfg->flags & IIR_FLAG_MOTION_V2) != 0;
    c->check_range = (cfg->flags & IIR_FLAG_CHECK_RANGE) != 0 && cfg->bpc > 8 && cfg->bpc < 16;
    c->nsums = c->moments ? kMaxSums : kSums;
    choose_columns(c);
    // IIR_TARGET_WAVES caps the wavefronts a launch's time chunks may fill (0: no cap beyond
    // two per SIMD)
    c->target_waves = env_int("IIR_TARGET_WAVES", 0, 0, 1 << 20);
    c->min_chunk = env_int("IIR_MIN_CHUNK", 2, 1, 65536);
    const int forced_rows = env_int("IIR_ROWS_PER_TILE", 0, 0, 64);
    int slots = 0;
    c->rows_per_tile = choose_rows(c, cus, forced_rows, &slots);
    if (c->rows_per_tile == 0)
        return fail(IIR_EINVAL, "no frames kernel for this configuration (rows per tile %d)",
                    forced_rows);
    c->row_tiles = (cfg->height + c->rows_per_tile - 1) / c->rows_per_tile;
    c->tiles = c->strips * c->row_tiles;
    // time chunks fill at most two wavefronts per SIMD (and the kernel's slots)
    c->fill = std::min(slots, 8 * cus);
    if (c->target_waves > 0)
        c->fill = std::min(c->fill, c->target_waves);
    c->max_chunks = plan_chunks(c, cfg->max_batch);
    // launch geometry must fit a 1-D grid ("ADR-1380", Consequences: an oversized launch failed
    // with an invalid-value error at 1080p and 4K; here every shape is checked once, up front)
    if ((int64_t)c->tiles * c->max_chunks > INT32_MAX / kWave)
        return fail(IIR_EINVAL, "frame too large for one grid");
    return IIR_OK;
}

void release(iir_ctx *c)
{
    if (!c)
        return;
    int saved = -1;
    if (hipGetDevice(&saved) == hipSuccess && saved != c->device)
        (void)hipSetDevice(c->device);
    (void)hipStreamSynchronize(c->stream);
    for (int i = 0; i < 2; ++i)
        if (c->ring[i])
            (void)hipFree(c->ring[i]);
    if (c->sums)
        (void)hipFree(c->sums);
    if (c->arrivals)
        (void)hipFree(c->arrivals);
    if (c->table_dev)
        (void)hipFree(c->table_dev);
    if (c->host_sums)
        (void)hipHostFree(c->host_sums);
    if (c->table_host)
        (void)hipHostFree(c->table_host);
    if (c->range_host)
        (void)hipHostFree(c->range_host);
    for (auto &sub : c->subs) {
        if (sub.k0)
            (void)hipEventDestroy(sub.k0);
        if (sub.k1)
            (void)hipEventDestroy(sub.k1);
    }

    if (saved >= 0 && saved != c->device)
        (void)hipSetDevice(saved);
    delete c;
}

// First of n contiguous free frame slots in the circular result region, or -1. Pending frames
// occupy [first slot of the oldest submission, slot_head) modulo max_batch.
int reserve_slots(const iir_ctx *c, int n)
{
    const int cap = c->cfg.max_batch;
    if (c->sub_count >= iir_ctx::kMaxPending || c->pending + n > cap)
        return -1;
    if (c->sub_count == 0)
        return 0;
    const int tail = c->subs[c->sub_head].first;
    const int head = c->slot_head;
    if (head > tail || (head == tail && c->pending == 0)) {
        if (head + n <= cap)
            return head;
        return n <= tail ? 0 : -1;  // wrap to the front
    }
    return head + n <= tail ? head : -1;
}

// No total reaches 2^63 (the largest, a sum of 2^30 squares of 16-bit differences, is below
// 2^62), so an all-ones word in host_sums means "not written yet".
constexpr unsigned long long kUnwritten = ~0ull;

// Mark the group totals of frames [first, first + n) as not yet written.
void fill_pending(iir_ctx *c, int first, int n)
{
    unsigned long long *p = c->host_sums + (size_t)first * c->nsums * kSumGroups;
    std::fill(p, p + (size_t)n * c->nsums * kSumGroups, kUnwritten);
}

// The frame part of one launch's arguments: plane pointers of n frame pairs (a base and a
// per-frame stride when every plane advances uniformly, else a descriptor table written at
// table_host and copied to table_dev on the context's stream), pitches, readable spans, the
// geometry and the time chunks. The state, sum and publish pointers are the caller's to set.
int frame_args(const iir_ctx *c, const iir_frame *ref, const iir_frame *dist, int n,
               FramePtrs *table_host, FramePtrs *table_dev, KernelArgs &a)
{
    // uniform frame stride: pointers travel in the kernel arguments
    bool uniform = true;
    for (int k = 0; k < 6 && uniform; ++k) {
        const uint8_t *p0 = plane_ptr(ref, dist, 0, k);
        const int64_t step = n > 1 ? plane_ptr(ref, dist, 1, k) - p0 : 0;
        for (int t = 2; t < n && uniform; ++t)
            uniform = plane_ptr(ref, dist, t, k) == p0 + (int64_t)t * step;
        a.base[k] = p0;
        a.fstride[k] = step;
    }
    if (!uniform) {
        for (int t = 0; t < n; ++t)
            for (int k = 0; k < 6; ++k)
                table_host[t].p[k] = plane_ptr(ref, dist, t, k);
        HIP_TRY(hipMemcpyAsync(table_dev, table_host, sizeof(FramePtrs) * n,
                               hipMemcpyHostToDevice, c->stream));
        a.table = table_dev;
    }
    for (int k = 0; k < 3; ++k) {
        const int64_t rows = k == 0 ? c->cfg.height : c->Hc;
        a.pitch[k] = (int32_t)ref[0].plane[k].pitch;
        a.pitch[k + 3] = (int32_t)dist[0].plane[k].pitch;
        a.span[k] = (uint32_t)(rows * ref[0].plane[k].pitch);
        a.span[k + 3] = (uint32_t)(rows * dist[0].plane[k].pitch);
    }
    a.W = c->cfg.width;
    a.H = c->cfg.height;
    a.Wc = c->Wc;
    a.Hc = c->Hc;
    a.strips = c->strips;
    a.row_tiles = c->row_tiles;
    a.tiles = c->tiles;
    a.nframes = n;
    a.chunks = plan_chunks(c, n);
    a.chunk_len = (n + a.chunks - 1) / a.chunks;
    a.shift = c->cfg.bpc == 8 ? 0 : 16 - c->cfg.bpc;
    return IIR_OK;
}

int submit_now(iir_ctx *c, const iir_frame *ref, const iir_frame *dist, int n)
{
    if (!c)
        return fail(IIR_EINVAL, "context is NULL");
    if (n < 1 || n > c->cfg.max_batch)
        return fail(IIR_EINVAL, "nframes %d outside 1..max_batch (%d)", n, c->cfg.max_batch);
    int rc = check_frames(c, ref, dist, n);
    if (rc != IIR_OK)
        return rc;
    const int first = reserve_slots(c, n);
    if (first < 0)
        return fail(IIR_EBUSY, "%d frames in %d submissions pending; %d more do not fit (max_batch %d)",
                    c->pending, c->sub_count, n, c->cfg.max_batch);
    DeviceScope ds(c->device);
    if (ds.err != hipSuccess)
        return fail_hip(ds.err, "hipSetDevice");

    KernelArgs a{};
    rc = frame_args(c, ref, dist, n, c->table_host + first, c->table_dev + first, a);
    if (rc != IIR_OK)
        return rc;
    a.ring_in = c->ring[c->ring_cur];
    a.ring_out = c->ring[c->ring_cur ^ 1];
    a.sums = c->sums + (size_t)c->sums_cur * c->sums_n;
    a.zero = c->sums + (size_t)(c->sums_cur ^ 1) * c->sums_n;
    a.zero_n = c->sums_dirty;
    a.publish = c->host_sums_dev + (size_t)first * c->nsums * kSumGroups;
    a.arrivals = c->arrivals;
    a.has_prev = c->has_prev ? 1 : 0;

    const bool timing = (c->cfg.flags & IIR_FLAG_TIMING) != 0;
    // untimed: the launch's totals are their own completion signal. Its rows of host_sums are
    // filled with a value no total can take before it is enqueued; iir_collect waits until every
    // one of them has been overwritten (no event packet in the stream between launches). Timed:
    // the dispatch's own end event marks it.
    if (!timing)
        fill_pending(c, first, n);
    const int sub_idx = (c->sub_head + c->sub_count) % iir_ctx::kMaxPending;
    iir_ctx::Sub &sub = c->subs[sub_idx];
    if (c->check_range) {
        // the slot's last submission has been collected, so its check kernel has finished
        c->range_host[sub_idx] = 0;
        HIP_TRY(launch_check_range(a, c->cfg.bpc, c->range_dev + sub_idx, c->stream));
    }
    // the kernel writes the totals to host_sums itself; with timing, the dispatch's own start
    // and end events also bracket it
    HIP_TRY(launch_frames(c->cfg.bpc, c->rows_per_tile,
                          !fast_path_ok(c->cfg.width, c->cfg.height, c->rows_per_tile),
                          c->moments, c->v2, a, c->stream, timing ? sub.k0 : nullptr,
                          timing ? sub.k1 : nullptr));
    // the launch is enqueued: the device state it leaves behind (the other slot buffer to clear,
    // the ring to read next) is committed
    sub.first = first;
    sub.n = n;
    sub.taken = 0;
    sub.has_prev = c->has_prev;
    sub.groups = std::min(a.tiles * a.chunks, kSumGroups);
    c->sub_count++;
    c->sums_dirty = (int64_t)n * c->nsums * kSumSlots;  // left in a.sums for the next launch
    c->sums_cur ^= 1;
    c->slot_head = first + n;
    c->pending += n;
    c->ring_cur ^= 1;
    c->has_prev = true;
    c->any_frame = true;
    return IIR_OK;
}

// Enqueue the recorded one-frame submissions as one launch (their descriptors go through the
// frame table when their planes do not advance by a constant stride). They are forgotten even if
// the launch fails: the error is the caller's.
int flush_deferred(iir_ctx *c)
{
    if (c->deferred == 0)
        return IIR_OK;
    const int n = c->deferred;
    c->deferred = 0;
    return submit_now(c, c->def_ref, c->def_dist, n);
}

bool same_pitches(const iir_frame &a, const iir_frame &b)
{
    for (int k = 0; k < 3; ++k)
        if (a.plane[k].pitch != b.plane[k].pitch)
            return false;
    return true;
}

// One submission: a clip goes out at once (after any recorded frames); with coalescing, a single
// frame pair is recorded, and the record goes out when it holds `coalesce` frames. A frame whose
// pitches differ from the recorded ones (one launch takes one set of pitches), or that would not
// fit beside them in the result slots, sends the record out first.
int submit(iir_ctx *c, const iir_frame *ref, const iir_frame *dist, int n)
{
    if (!c)
        return fail(IIR_EINVAL, "context is NULL");
    if (n != 1 || c->coalesce <= 1) {
        const int rc = flush_deferred(c);
        return rc != IIR_OK ? rc : submit_now(c, ref, dist, n);
    }
    int rc = check_frames(c, ref, dist, 1);
    if (rc != IIR_OK)
        return rc;
    if (c->deferred > 0 && (!same_pitches(c->def_ref[0], ref[0]) ||
                            !same_pitches(c->def_dist[0], dist[0]) ||
                            reserve_slots(c, c->deferred + 1) < 0)) {
        rc = flush_deferred(c);
        if (rc != IIR_OK)
            return rc;
    }
    if (reserve_slots(c, c->deferred + 1) < 0)
        return fail(IIR_EBUSY, "%d frames in %d submissions pending; one more does not fit "
                    "(max_batch %d)", c->pending, c->sub_count, c->cfg.max_batch);
    c->def_ref[c->deferred] = ref[0];
    c->def_dist[c->deferred] = dist[0];
    if (++c->deferred == c->coalesce)
        return flush_deferred(c);
    return IIR_OK;
}

// Wait until the kernel of an untimed submission has written every group total of its frames
// (each one 64-bit store, so a word is either the unwritten mark or its total). The scan resumes
// where it last found a mark. The stream is queried now and then, so a launch that failed, or one
// that finished without writing a total, ends the wait with an error instead of spinning forever.
int wait_published(iir_ctx *c, const iir_ctx::Sub &sub)
{
    const volatile unsigned long long *p = c->host_sums + (size_t)sub.first * c->nsums * kSumGroups;
    const int rows = sub.n * c->nsums;
    int row = 0, g = 0;
    for (uint64_t spin = 0;; ++spin) {
        while (row < rows && p[(size_t)row * kSumGroups + g] != kUnwritten) {
            if (++g == sub.groups) {
                g = 0;
                ++row;
            }
        }
        if (row == rows)
            return IIR_OK;
        if ((spin & 1023) == 1023) {
            const hipError_t e = hipStreamQuery(c->stream);
            if (e == hipSuccess) {
                if (p[(size_t)row * kSumGroups + g] != kUnwritten)
                    continue;
                return fail(IIR_EDEVICE, "the launch finished without writing its totals");
            }
            if (e != hipErrorNotReady)
                return fail_hip(e, "hipStreamQuery");
            if (spin > (1u << 20))
                std::this_thread::yield();
        }
        __builtin_ia32_pause();
    }
}

}  // namespace

extern "C" {

IIR_API int iir_create(const iir_config *cfg, int32_t device, void *hip_stream, iir_ctx **out)
{
    if (!out)
        return fail(IIR_EINVAL, "out is NULL");
    int rc = check_config(cfg);
    if (rc != IIR_OK)
        return rc;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0)
        return fail(IIR_ENODEV, "no HIP device visible");
    if (device < 0 || device >= count)
        return fail(IIR_ENODEV, "device %d not in [0, %d)", device, count);
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, device));
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(IIR_ENODEV, "device %d is %s; this library is built for gfx950", device,
                    prop.gcnArchName);
    DeviceScope ds(device);
    if (ds.err != hipSuccess)
        return fail_hip(ds.err, "hipSetDevice");

    iir_ctx *c = new (std::nothrow) iir_ctx;
    if (!c)
        return fail(IIR_ENOMEM, "host allocation failed");
    rc = setup_geometry(c, cfg, device, prop.multiProcessorCount);
    if (rc != IIR_OK) {
        delete c;
        return rc;
    }
    c->stream = static_cast<hipStream_t>(hip_stream);
    c->sums_n = (int64_t)cfg->max_batch * c->nsums * kSumSlots;

    const size_t ring_bytes = (size_t)c->tiles * c->rows_per_tile * kWave * sizeof(uint2);
    hipError_t e = hipSuccess;
    for (int i = 0; i < 2 && e == hipSuccess; ++i)
        e = hipMalloc(&c->ring[i], ring_bytes);
    if (e == hipSuccess)
        e = hipMalloc(&c->sums, sizeof(unsigned long long) * 2 * c->sums_n);
    if (e == hipSuccess)
        e = hipMalloc(&c->arrivals, sizeof(unsigned int) * kArrivals);
    if (e == hipSuccess)
        e = hipMalloc(&c->table_dev, sizeof(FramePtrs) * cfg->max_batch);
    if (e == hipSuccess)
        e = hipHostMalloc(&c->host_sums,
                          sizeof(unsigned long long) * cfg->max_batch * c->nsums * kSumGroups,
                          hipHostMallocCoherent | hipHostMallocMapped);
    if (e == hipSuccess)
        e = hipHostGetDevicePointer(reinterpret_cast<void **>(&c->host_sums_dev), c->host_sums, 0);
    if (e == hipSuccess)
        e = hipHostMalloc(&c->table_host, sizeof(FramePtrs) * cfg->max_batch, hipHostMallocDefault);
    if (e == hipSuccess && c->check_range)
        e = hipHostMalloc(&c->range_host, sizeof(uint32_t) * iir_ctx::kMaxPending,
                          hipHostMallocCoherent | hipHostMallocMapped);
    if (e == hipSuccess && c->check_range)
        e = hipHostGetDevicePointer(reinterpret_cast<void **>(&c->range_dev), c->range_host, 0);

    if (e != hipSuccess) {
        release(c);
        return fail(IIR_ENOMEM, "allocation failed: %s", hipGetErrorString(e));
    }
    for (auto &sub : c->subs) {
        if (e == hipSuccess && (cfg->flags & IIR_FLAG_TIMING))
            e = hipEventCreate(&sub.k0);
        if (e == hipSuccess && (cfg->flags & IIR_FLAG_TIMING))
            e = hipEventCreate(&sub.k1);
    }
    if (e == hipSuccess)
        e = hipMemsetAsync(c->sums, 0, sizeof(unsigned long long) * 2 * c->sums_n, c->stream);
    if (e == hipSuccess)
        e = hipMemsetAsync(c->arrivals, 0, sizeof(unsigned int) * kArrivals, c->stream);
    for (int i = 0; i < 2 && e == hipSuccess; ++i)
        e = hipMemsetAsync(c->ring[i], 0, ring_bytes, c->stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) {
        release(c);
        return fail_hip(e, "iir_create setup");
    }
    *out = c;
    return IIR_OK;
}

IIR_API int iir_submit(iir_ctx *ctx, const iir_frame *ref, const iir_frame *dist)
{
    return submit(ctx, ref, dist, 1);
}

IIR_API int iir_submit_clip(iir_ctx *ctx, const iir_frame *ref, const iir_frame *dist,
                            int32_t nframes)
{
    return submit(ctx, ref, dist, nframes);
}

IIR_API int iir_collect(iir_ctx *ctx, iir_result *out, int32_t max, int32_t *n_out)
{
    if (!ctx || !out || !n_out || max < 0)
        return fail(IIR_EINVAL, "bad collect arguments");
    *n_out = 0;
    const int frc = flush_deferred(ctx);
    if (frc != IIR_OK)
        return frc;
    const int n = std::min(max, ctx->pending);
    if (n == 0)
        return IIR_OK;
    // wait for the submission holding the last result returned; stream order covers the others
    {
        int need = n, k = 0;
        const iir_ctx::Sub *last = nullptr;
        while (need > 0) {
            const iir_ctx::Sub &sub = ctx->subs[(ctx->sub_head + k++) % iir_ctx::kMaxPending];
            need -= sub.n - sub.taken;
            last = &sub;
        }
        DeviceScope ds(ctx->device);
        if (ds.err != hipSuccess)
            return fail_hip(ds.err, "hipSetDevice");
        if (ctx->cfg.flags & IIR_FLAG_TIMING)
            HIP_TRY(hipEventSynchronize(last->k1));
        else {
            const int rc = wait_published(ctx, *last);
            if (rc != IIR_OK)
                return rc;
        }
    }
    int got = 0;
    int range_rc = IIR_OK;
    while (got < n) {
        iir_ctx::Sub &sub = ctx->subs[ctx->sub_head];
        const int take = std::min(n - got, sub.n - sub.taken);
        if (ctx->check_range && range_rc == IIR_OK) {
            // written by the check kernel, which finished before the frames kernel began
            const uint32_t code = __atomic_load_n(ctx->range_host + ctx->sub_head, __ATOMIC_ACQUIRE);
            const int t = code ? (int)(code - 1) / 6 : -1;
            if (code && t >= sub.taken && t < sub.taken + take) {
                static const char *const kPlanes[6] = {"ref Y", "ref U", "ref V",
                                                       "dist Y", "dist U", "dist V"};
                range_rc = fail(IIR_ERANGE, "result %d (frame %d of its launch): %s holds a "
                                "sample >= 2^%d", got + t - sub.taken, t,
                                kPlanes[(code - 1) % 6], ctx->cfg.bpc);
            }
        }
        for (int i = 0; i < take; ++i) {
            const int f = sub.taken + i;
            const volatile unsigned long long *g =
                ctx->host_sums + (size_t)(sub.first + f) * ctx->nsums * kSumGroups;
            uint64_t v[kMaxSums] = {};
            for (int k = 0; k < ctx->nsums; ++k)
                for (int j = 0; j < sub.groups; ++j)
                    v[k] += g[k * kSumGroups + j];
            iir_result &r = out[got + i];
            r.has_motion = (f > 0 || sub.has_prev) ? 1 : 0;
            r.sad = r.has_motion ? v[0] : 0;
            r.sse[0] = v[1];
            r.sse[1] = v[2];
            r.sse[2] = v[3];
            for (int k = 0; k < kMoments; ++k)
                r.moment[k] = ctx->moments ? v[kSums + k] : 0;
            r.reserved = 0;
        }
        sub.taken += take;
        got += take;
        if (sub.taken == sub.n) {
            float ms = 0.f;
            if ((ctx->cfg.flags & IIR_FLAG_TIMING) &&
                hipEventElapsedTime(&ms, sub.k0, sub.k1) == hipSuccess) {
                ctx->last_ms = ms;
                ctx->timed_launches++;
                ctx->timed_ms += ms;
            }
            ctx->sub_head = (ctx->sub_head + 1) % iir_ctx::kMaxPending;
            ctx->sub_count--;
        }
    }
    ctx->pending -= n;
    if (ctx->sub_count == 0)
        ctx->slot_head = 0;
    *n_out = n;
    return range_rc;
}

IIR_API int iir_run_clip(iir_ctx *ctx, const iir_frame *ref, const iir_frame *dist,
                         int32_t nframes, iir_result *out)
{
    if (!ctx || !out)
        return fail(IIR_EINVAL, "context or out is NULL");
    if (ctx->pending != 0 || ctx->deferred != 0)
        return fail(IIR_ESTATE, "iir_run_clip needs an empty queue (%d results pending)",
                    ctx->pending + ctx->deferred);
    int rc = submit(ctx, ref, dist, nframes);
    if (rc != IIR_OK)
        return rc;
    int32_t got = 0;
    rc = iir_collect(ctx, out, nframes, &got);
    if (rc == IIR_OK && got != nframes)
        return fail(IIR_EDEVICE, "collected %d of %d results", got, nframes);
    return rc;
}

IIR_API int iir_run_clip_static(const iir_config *cfg, int32_t device, void *hip_stream,
                                const iir_frame *ref, const iir_frame *dist, int32_t nframes,
                                iir_result *out)
{
    if (!out)
        return fail(IIR_EINVAL, "out is NULL");
    int rc = check_config(cfg);
    if (rc != IIR_OK)
        return rc;
    if (nframes < 1 || nframes > kStaticMaxFrames)
        return fail(IIR_EINVAL, "nframes %d outside 1..%d (the static working memory's bound)",
                    nframes, kStaticMaxFrames);
    if (cfg->flags & IIR_FLAG_CHECK_RANGE)
        return fail(IIR_EINVAL, "IIR_FLAG_CHECK_RANGE is not available in iir_run_clip_static");
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0)
        return fail(IIR_ENODEV, "no HIP device visible");
    if (device < 0 || device >= count)
        return fail(IIR_ENODEV, "device %d not in [0, %d)", device, count);
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, device));
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(IIR_ENODEV, "device %d is %s; this library is built for gfx950", device,
                    prop.gcnArchName);
    DeviceScope ds(device);
    if (ds.err != hipSuccess)
        return fail_hip(ds.err, "hipSetDevice");

    // geometry only: this context lives on the stack and owns no device or host memory
    iir_ctx c;
    iir_config one = *cfg;
    one.max_batch = nframes;
    rc = setup_geometry(&c, &one, device, prop.multiProcessorCount);
    if (rc != IIR_OK)
        return rc;
    c.stream = static_cast<hipStream_t>(hip_stream);
    rc = check_frames(&c, ref, dist, nframes);
    if (rc != IIR_OK)
        return rc;

    StaticScratch s;
    HIP_TRY(static_scratch(device, &s));
    // a non-uniformly strided clip's plane pointers go through this stack table (the stream is
    // synchronised before it goes out of scope)
    FramePtrs table[kStaticMaxFrames];
    KernelArgs a{};
    rc = frame_args(&c, ref, dist, nframes, table, s.table, a);
    if (rc != IIR_OK)
        return rc;
    a.ring_in = nullptr;
    a.ring_out = nullptr;
    a.has_prev = 0;
    a.sums = s.sums;
    a.zero = nullptr;
    a.zero_n = 0;
    a.publish = s.publish;
    a.arrivals = s.arrivals;
    // the partial slots and arrival counters start at zero; the array keeps the last call's values
    HIP_TRY(launch_clear(s.sums, (int64_t)nframes * c.nsums * kSumSlots, s.arrivals, c.stream));
    HIP_TRY(launch_frames(one.bpc, c.rows_per_tile,
                          !fast_path_ok(one.width, one.height, c.rows_per_tile), c.moments, c.v2,
                          a, c.stream));
    HIP_TRY(launch_fold(s.publish, nframes, c.nsums, std::min(a.tiles * a.chunks, kSumGroups),
                        s.results, c.stream));
    HIP_TRY(hipMemcpyAsync(out, s.results, sizeof(iir_result) * nframes, hipMemcpyDefault,
                           c.stream));
    HIP_TRY(hipStreamSynchronize(c.stream));
    return IIR_OK;
}

IIR_API int iir_scores_of(const iir_config *cfg, const iir_result *r, iir_scores *s)
{
    if (!cfg || !r || !s)
        return fail(IIR_EINVAL, "NULL argument");
    if (cfg->bpc < 8 || cfg->bpc > 16 || cfg->width < 1 || cfg->height < 1)
        return fail(IIR_EINVAL, "bad configuration");
    const double n_luma = (double)cfg->width * (double)cfg->height;
    const double n_chroma = (double)((cfg->width + 1) / 2) * (double)((cfg->height + 1) / 2);
    const double peak = (double)((1 << cfg->bpc) - 1);
    s->motion = r->has_motion ? (double)r->sad / (256.0 * n_luma) : 0.0;
    for (int c = 0; c < 3; ++c) {
        const double mse = (double)r->sse[c] / (c == 0 ? n_luma : n_chroma);
        s->mse[c] = mse;
        s->psnr[c] = r->sse[c] == 0 ? INFINITY : 10.0 * std::log10(peak * peak / mse);
    }
    for (int k = 0; k < 4; ++k)
        s->moment[k] = (double)r->moment[k] / n_luma;
    return IIR_OK;
}

IIR_API int iir_motion2(const double *motion, int32_t n, double *motion2)
{
    if (!motion || !motion2 || n < 1)
        return fail(IIR_EINVAL, "motion2 needs two non-NULL arrays and n >= 1");
    // in place is allowed: frame t reads motion[t + 1] before anything overwrites it
    for (int32_t t = 0; t < n; ++t) {
        const double own = motion[t];
        const double next = t + 1 < n ? motion[t + 1] : own;
        motion2[t] = std::min(own, next);
    }
    return IIR_OK;
}

IIR_API int iir_aggregate_of(const iir_config *cfg, const iir_result *r, int32_t n,
                             iir_aggregate *out)
{
    if (!cfg || !r || !out || n < 1)
        return fail(IIR_EINVAL, "aggregate needs a config, n >= 1 results and an output");
    if (cfg->bpc < 8 || cfg->bpc > 16 || cfg->width < 1 || cfg->height < 1)
        return fail(IIR_EINVAL, "bad configuration");
    const double n_luma = (double)cfg->width * (double)cfg->height;
    const double n_chroma = (double)((cfg->width + 1) / 2) * (double)((cfg->height + 1) / 2);
    const double peak = (double)((1 << cfg->bpc) - 1);
    uint64_t total[3] = {0, 0, 0};
    double sum_motion = 0.0, sum_motion2 = 0.0;
    double prev = 0.0;  // motion of frame t - 1 while frame t is read
    for (int32_t t = 0; t < n; ++t) {
        const double m = r[t].has_motion ? (double)r[t].sad / (256.0 * n_luma) : 0.0;
        for (int c = 0; c < 3; ++c)
            total[c] += r[t].sse[c];
        sum_motion += m;
        if (t > 0)
            sum_motion2 += std::min(prev, m);  // motion2 of frame t - 1
        prev = m;
    }
    sum_motion2 += prev;  // the last frame keeps its own motion
    for (int c = 0; c < 3; ++c) {
        out->sse[c] = total[c];
        const double mse = (double)total[c] / ((double)n * (c == 0 ? n_luma : n_chroma));
        out->apsnr[c] = total[c] == 0 ? INFINITY : 10.0 * std::log10(peak * peak / mse);
    }
    out->mean_motion = sum_motion / (double)n;
    out->mean_motion2 = sum_motion2 / (double)n;
    out->frames = n;
    out->reserved = 0;
    return IIR_OK;
}

IIR_API int iir_reset(iir_ctx *ctx)
{
    if (!ctx)
        return fail(IIR_EINVAL, "context is NULL");
    const int rc = flush_deferred(ctx);  // recorded frames still follow the frames before them
    if (rc != IIR_OK)
        return rc;
    ctx->has_prev = false;
    ctx->any_frame = false;
    return IIR_OK;
}

IIR_API int iir_set_coalesce(iir_ctx *ctx, int32_t frames)
{
    if (!ctx)
        return fail(IIR_EINVAL, "context is NULL");
    const int most = std::min(iir_ctx::kMaxCoalesce, ctx->cfg.max_batch);
    if (frames < 1 || frames > most)
        return fail(IIR_EINVAL, "coalesce %d outside 1..%d", frames, most);
    const int rc = flush_deferred(ctx);
    if (rc != IIR_OK)
        return rc;
    ctx->coalesce = frames;
    return IIR_OK;
}

IIR_API int iir_export_blur(iir_ctx *ctx, void *dst, int64_t pitch)
{
    if (!ctx || !dst)
        return fail(IIR_EINVAL, "context or dst is NULL");
    if (pitch < 2 * (int64_t)ctx->cfg.width || (pitch % 4) || ((uintptr_t)dst % 4))
        return fail(IIR_EINVAL, "pitch %lld: needs >= 2*W and 4-byte alignment", (long long)pitch);
    const int rc = flush_deferred(ctx);
    if (rc != IIR_OK)
        return rc;
    if (!ctx->any_frame)
        return fail(IIR_ESTATE, "no frame submitted since create or reset");
    if (ctx->v2)
        return fail(IIR_ESTATE, "motion v2 keeps no blurred frame");
    DeviceScope ds(ctx->device);
    if (ds.err != hipSuccess)
        return fail_hip(ds.err, "hipSetDevice");
    HIP_TRY(launch_export(ctx->ring[ctx->ring_cur], static_cast<uint16_t *>(dst), pitch,
                          ctx->cfg.width, ctx->cfg.height, ctx->strips,
                          ctx->rows_per_tile, ctx->stream));
    return IIR_OK;
}

IIR_API int iir_kernel_time(iir_ctx *ctx, float *ms)
{
    if (!ctx || !ms)
        return fail(IIR_EINVAL, "NULL argument");
    if (ctx->last_ms < 0.f)
        return fail(IIR_ESTATE, "no timed submission collected (IIR_FLAG_TIMING off, or collect first)");
    *ms = ctx->last_ms;
    return IIR_OK;
}

IIR_API int iir_kernel_stats(iir_ctx *ctx, int32_t reset, int64_t *launches, double *total_ms)
{
    if (!ctx || !launches || !total_ms)
        return fail(IIR_EINVAL, "NULL argument");
    *launches = ctx->timed_launches;
    *total_ms = ctx->timed_ms;
    if (reset) {
        ctx->timed_launches = 0;
        ctx->timed_ms = 0.0;
    }
    return IIR_OK;
}

IIR_API int iir_get_geometry(const iir_ctx *ctx, iir_geometry *out)
{
    if (!ctx || !out)
        return fail(IIR_EINVAL, "NULL argument");
    out->rows_per_tile = ctx->rows_per_tile;
    out->lanes_out = ctx->lanes_out;
    out->strips = ctx->strips;
    out->row_tiles = ctx->row_tiles;
    out->tiles = ctx->tiles;
    out->sum_slots = kSumSlots;
    out->max_chunks = ctx->max_chunks;
    return IIR_OK;
}

IIR_API int iir_plan_chunks(const iir_ctx *ctx, int32_t nframes, int32_t *chunks)
{
    if (!ctx || !chunks || nframes < 1 || nframes > ctx->cfg.max_batch)
        return fail(IIR_EINVAL, "bad plan_chunks arguments");
    *chunks = plan_chunks(ctx, nframes);
    return IIR_OK;
}

IIR_API int iir_probe_bandwidth(int32_t device, void *hip_stream, int32_t mode, const void *src,
                                void *dst, int64_t bytes, int32_t iters, float *ms)
{
    if (!ms || mode < 0 || mode > 2 || bytes < 4096 || (bytes % 4096) || iters < 1)
        return fail(IIR_EINVAL, "bad probe arguments");
    if ((mode != 1 && !src) || !dst || ((uintptr_t)src % 16) || ((uintptr_t)dst % 16))
        return fail(IIR_EINVAL, "probe buffers must be non-NULL and 16-byte aligned");
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count)
        return fail(IIR_ENODEV, "device %d not available", device);
    DeviceScope ds(device);
    if (ds.err != hipSuccess)
        return fail_hip(ds.err, "hipSetDevice");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    HIP_TRY(hipEventCreate(&e0));
    hipError_t e = hipEventCreate(&e1);
    if (e == hipSuccess)
        e = launch_probe(mode, src, dst, bytes, s);  // warm-up
    if (e == hipSuccess)
        e = hipEventRecord(e0, s);
    for (int i = 0; i < iters && e == hipSuccess; ++i)
        e = launch_probe(mode, src, dst, bytes, s);
    if (e == hipSuccess)
        e = hipEventRecord(e1, s);
    if (e == hipSuccess)
        e = hipEventSynchronize(e1);
    float total = 0.f;
    if (e == hipSuccess)
        e = hipEventElapsedTime(&total, e0, e1);
    (void)hipEventDestroy(e0);
    if (e1)
        (void)hipEventDestroy(e1);
    if (e != hipSuccess)
        return fail_hip(e, "bandwidth probe");
    *ms = total / (float)iters;
    return IIR_OK;
}

IIR_API void iir_destroy(iir_ctx *ctx)
{
    release(ctx);
}

IIR_API const char *iir_strerror(int code)
{
    switch (code) {
    case IIR_OK:
        return "success";
    case IIR_EINVAL:
        return "invalid argument";
    case IIR_ENODEV:
        return "no usable gfx950 device";
    case IIR_ENOMEM:
        return "out of memory";
    case IIR_EDEVICE:
        return "HIP runtime error";
    case IIR_EBUSY:
        return "too many frames pending";
    case IIR_ESTATE:
        return "invalid in the current state";
    case IIR_ERANGE:
        return "input sample out of range";
    default:
        return "unknown error";
    }
}

IIR_API const char *iir_last_error(void)
{
    return g_err.c_str();
}

}  // extern "C"
