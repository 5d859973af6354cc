// iir_kernels.hip -- launchers of the gfx950 kernels (the frames kernel itself is in
// iir_frames.h, instantiated by the iir_frames_*.hip units), the blurred-plane export, the
// input-range check and the memory-ceiling probes.
#include <hip/hip_ext.h>

#include <algorithm>
#include <mutex>

#include "iir_internal.h"

namespace iir {
namespace {

// Tiled blurred state -> W x H uint16 plane.
__global__ void export_kernel(const uint32_t *ring, uint16_t *dst, int64_t pitch, int W, int H,
                              int strips, int th)
{
    const int pairs = (W + 1) / 2;
    const int64_t n = (int64_t)pairs * H;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int row = (int)(idx / pairs);
        const int j = 2 * (int)(idx - (int64_t)row * pairs);
        const int strip = j / kStripCols;
        const int in = j - strip * kStripCols;
        const int lane = in / kLumaCols;
        const int half = (in % kLumaCols) / 2;
        const int tile = (row / th) * strips + strip;
        const uint32_t w = ring[(((int64_t)tile * th + row % th) * kWave + lane) * 2 + half];
        uint16_t *d = reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(dst) + row * pitch);
        d[j] = (uint16_t)(w & 0xffffu);
        if (j + 1 < W)
            d[j + 1] = (uint16_t)(w >> 16);
    }
}

// Blocks take (frame, plane, row) triples, grid-stride, and their 256 threads the row's 16-byte
// groups of 8 samples (data and pitch are multiples of 16 bytes and pitch >= 2 * width, so every
// group that starts inside the width ends inside the row's pitch). Samples past the width (the
// pitch padding) are not checked.
__global__ __launch_bounds__(256) void check_range_kernel(const KernelArgs a, uint32_t limit,
                                                          uint32_t *flag)
{
    const int H = a.H;
    const int64_t n = (int64_t)a.nframes * 6 * H;
    for (int64_t id = blockIdx.x; id < n; id += gridDim.x) {
        const int z = (int)(id / H), row = (int)(id - (int64_t)z * H);  // z = t * 6 + k
        const int t = z / 6, k = z - 6 * t;
        const bool luma = k % 3 == 0;
        const int w = luma ? a.W : a.Wc;
        if (row >= (luma ? H : a.Hc))
            continue;
        const uint8_t *plane = a.table ? a.table[t].p[k] : a.base[k] + (int64_t)t * a.fstride[k];
        const uint4 *r = reinterpret_cast<const uint4 *>(plane + (int64_t)row * a.pitch[k]);
        bool row_bad = false;
        for (int g = threadIdx.x; 8 * g < w; g += blockDim.x) {
            const uint4 v = r[g];
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t sample = (d[j / 2] >> (16 * (j % 2))) & 0xffffu;
                row_bad |= 8 * g + j < w && sample >= limit;
            }
        }
        if (row_bad)
            *flag = (uint32_t)z + 1u;  // any offending thread's code will do
    }
}

// Memory-ceiling probes: read-only (xor-reduced, written only if a runtime flag asks), write-only,
// copy. 16-byte non-temporal accesses; each thread keeps U independent accesses in flight per
// pass (grid-stride), then finishes the tail one at a time. The shapes (8 reads or 4 copies in
// flight, 16384 workgroups of 256) measured fastest on MI355X among 4-16 in flight and
// 1024-16384 workgroups.
constexpr int kReadUnroll = 8, kCopyUnroll = 4, kProbeBlocks = 16384;
typedef unsigned int probe_v4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void probe_read(const probe_v4 *src, int64_t n, probe_v4 *sink,
                                                  int keep)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    probe_v4 acc = {0, 0, 0, 0};
    for (; i + (U - 1) * stride < n; i += U * stride) {
        probe_v4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k)
            v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
        for (int k = 0; k < U; ++k)
            acc ^= v[k];
    }
    for (; i < n; i += stride)
        acc ^= src[i];
    if (keep)
        sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void probe_write(probe_v4 *dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const probe_v4 v = {(uint32_t)i, (uint32_t)(i >> 32), 0x9e3779b9u, 0u};
        __builtin_nontemporal_store(v, dst + i);
    }
}

template <int U>
__global__ __launch_bounds__(256) void probe_copy(const probe_v4 *src, probe_v4 *dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        probe_v4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k)
            v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
        for (int k = 0; k < U; ++k)
            __builtin_nontemporal_store(v[k], dst + i + k * stride);
    }
    for (; i < n; i += stride)
        dst[i] = src[i];
}


// Zero n 64-bit words and the group arrival counters.
__global__ __launch_bounds__(256) void clear_kernel(unsigned long long *p, int64_t n,
                                                     unsigned int *arrivals)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t i = i0; i < n; i += stride)
        p[i] = 0ull;
    if (i0 < kArrivals)
        arrivals[i0] = 0u;
}

// One thread per frame: the sum of its `groups` group totals of every sum, as an iir_result.
__global__ __launch_bounds__(256) void fold_kernel(const unsigned long long *publish, int nframes,
                                                    int nsums, int groups, iir_result *out)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nframes)
        return;
    const unsigned long long *g = publish + (size_t)t * nsums * kSumGroups;
    unsigned long long v[kMaxSums] = {};
    for (int k = 0; k < nsums; ++k)
        for (int j = 0; j < groups; ++j)
            v[k] += g[k * kSumGroups + j];
    iir_result r;
    r.has_motion = t > 0 ? 1 : 0;
    r.sad = t > 0 ? v[0] : 0ull;
    for (int c = 0; c < 3; ++c)
        r.sse[c] = v[1 + c];
    for (int k = 0; k < kMoments; ++k)
        r.moment[k] = nsums > kSums ? v[kSums + k] : 0ull;
    r.reserved = 0;
    out[t] = r;
}

// The working memory of iir_run_clip_static, in the library's own device data: each GPU the
// library runs on holds one copy until the process ends. Region sizes for kStaticMaxFrames frames,
// each rounded up to 256 bytes.
constexpr size_t round256(size_t n) { return (n + 255) / 256 * 256; }
constexpr size_t kScrSums = round256(sizeof(unsigned long long) * kStaticMaxFrames * kMaxSums *
                                     kSumSlots);
constexpr size_t kScrPublish = round256(sizeof(unsigned long long) * kStaticMaxFrames * kMaxSums *
                                        kSumGroups);
constexpr size_t kScrResults = round256(sizeof(iir_result) * kStaticMaxFrames);
constexpr size_t kScrTable = round256(sizeof(FramePtrs) * kStaticMaxFrames);
constexpr size_t kScrArrivals = round256(sizeof(unsigned int) * kArrivals);
constexpr size_t kScratchBytes = kScrSums + kScrPublish + kScrResults + kScrTable + kScrArrivals;
static_assert(kScratchBytes < (size_t)2 << 20, "the static working memory stays modest");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

}  // namespace

// The array's address on the current device. In host code `scratch` names a host-side stand-in,
// not device memory, so the device address is looked up once per device (with that device
// current) and only that address is handed to kernels and copies.
hipError_t static_scratch(int device, StaticScratch *out)
{
    constexpr int kMaxDevices = 64;
    static std::mutex lock;
    static void *addr[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices)
        return hipErrorInvalidDevice;
    void *p = nullptr;
    {
        std::lock_guard<std::mutex> g(lock);
        if (!addr[device]) {
            void *q = nullptr;
            const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            if (!q)
                return hipErrorInvalidSymbol;
            addr[device] = q;
        }
        p = addr[device];
    }
    unsigned char *b = static_cast<unsigned char *>(p);
    out->sums = reinterpret_cast<unsigned long long *>(b);
    b += kScrSums;
    out->publish = reinterpret_cast<unsigned long long *>(b);
    b += kScrPublish;
    out->results = reinterpret_cast<iir_result *>(b);
    b += kScrResults;
    out->table = reinterpret_cast<FramePtrs *>(b);
    b += kScrTable;
    out->arrivals = reinterpret_cast<unsigned int *>(b);
    return hipSuccess;
}

hipError_t launch_clear(unsigned long long *sums, int64_t n, unsigned int *arrivals,
                        hipStream_t stream)
{
    const unsigned blocks =
        (unsigned)std::min<int64_t>(std::max<int64_t>((n + 255) / 256, 1), 1024);
    hipLaunchKernelGGL(clear_kernel, dim3(blocks), dim3(256), 0, stream, sums, n, arrivals);
    return hipGetLastError();
}

hipError_t launch_fold(const unsigned long long *publish, int nframes, int nsums, int groups,
                       iir_result *out, hipStream_t stream)
{
    const unsigned blocks = (unsigned)((nframes + 255) / 256);
    hipLaunchKernelGGL(fold_kernel, dim3(blocks), dim3(256), 0, stream, publish, nframes, nsums,
                       groups, out);
    return hipGetLastError();
}


// 8-bit and 10-bit samples have kernels of their own; every other depth up to 16 bits takes the
// 16-bit one with the launch's scale shift
FramesFn pick(int bpc, int th, bool generic, bool moments, bool v2 = false)
{
    if (v2) {
        if (bpc == 8)
            return frames_pick_8_v2(th, generic, moments);
        if (bpc == 10)
            return frames_pick_10_v2(th, generic, moments);
        if (bpc >= 9 && bpc <= 16)
            return frames_pick_16_v2(th, generic, moments, bpc == 16);
        return nullptr;
    }
    if (bpc == 8)
        return frames_pick_8(th, generic, moments);
    if (bpc == 10)
        return frames_pick_10(th, generic, moments);
    if (bpc >= 9 && bpc <= 16)
        return frames_pick_16(th, generic, moments);
    return nullptr;
}


bool supported_rows_per_tile(int th)
{
    return pick(8, th, true, false) != nullptr;
}

bool fast_path_ok(int W, int H, int th)
{
    return W % 8 == 0 && H % th == 0;
}

hipError_t frames_occupancy(int bpc, int th, bool generic, bool moments, bool v2,
                            int *waves_per_cu)
{
    FramesFn f = pick(bpc, th, generic, moments, v2);
    if (!f)
        return hipErrorInvalidValue;
    int blocks = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &blocks, reinterpret_cast<const void *>(f), kWave, 0);
    *waves_per_cu = blocks;
    return e;
}

hipError_t launch_frames(int bpc, int th, bool generic, bool moments, bool v2,
                         const KernelArgs &a, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop)
{
    FramesFn f = pick(bpc, th, generic, moments, v2);
    if (!f)
        return hipErrorInvalidValue;
    // a one-frame launch of 8-bit samples (a frame pair per submission) has its own kernel
    if (a.nframes == 1 && a.chunks == 1 && bpc == 8 && !v2) {
        if (FramesFn one = frames_pick_8_one(th, generic, moments))
            f = one;
    }
    const dim3 grid((unsigned)(a.tiles * a.chunks)), block(kWave);
    if (start && stop)  // the events are the dispatch's own start and end timestamps
        hipExtLaunchKernelGGL(f, grid, block, 0, stream, start, stop, 0, a);
    else
        hipLaunchKernelGGL(f, grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_export(const uint32_t *ring, uint16_t *dst, int64_t pitch, int W, int H,
                         int strips, int th, hipStream_t stream)
{
    const int64_t n = (int64_t)((W + 1) / 2) * H;
    const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 65536);
    hipLaunchKernelGGL(export_kernel, dim3(blocks), dim3(256), 0, stream, ring, dst, pitch, W, H,
                       strips, th);
    return hipGetLastError();
}

// The probe's sink (mode 0) is dst; it must hold blocks * 256 * 16 bytes, which bytes covers.
hipError_t launch_check_range(const KernelArgs &a, int bpc, uint32_t *flag, hipStream_t stream)
{
    if (bpc <= 8 || bpc >= 16)
        return hipErrorInvalidValue;  // every stored value is a valid sample
    const int64_t rows = (int64_t)a.nframes * 6 * a.H;
    if (rows <= 0)
        return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)std::min<int64_t>(rows, 1 << 20);
    hipLaunchKernelGGL(check_range_kernel, dim3(blocks), dim3(256), 0, stream, a, 1u << bpc,
                       flag);
    return hipGetLastError();
}

hipError_t launch_probe(int mode, const void *src, void *dst, int64_t bytes, hipStream_t stream)
{
    const int64_t n = bytes / 16;
    // up to kProbeBlocks workgroups of 256, fewer for a small buffer
    const unsigned blocks =
        (unsigned)std::min<int64_t>(std::max<int64_t>(n / (256 * 8), 1), kProbeBlocks);
    if (mode == 0)
        hipLaunchKernelGGL(probe_read<kReadUnroll>, dim3(blocks), dim3(256), 0, stream,
                           static_cast<const probe_v4 *>(src), n, static_cast<probe_v4 *>(dst), 0);
    else if (mode == 1)
        hipLaunchKernelGGL(probe_write, dim3(blocks), dim3(256), 0, stream,
                           static_cast<probe_v4 *>(dst), n);
    else
        hipLaunchKernelGGL(probe_copy<kCopyUnroll>, dim3(blocks), dim3(256), 0, stream,
                           static_cast<const probe_v4 *>(src), static_cast<probe_v4 *>(dst), n);
    return hipGetLastError();
}

}  // namespace iir
