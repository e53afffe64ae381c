// Routing metadata on the GPU: expert histogram, offsets (plain, padded,
// tile) and the stable gather / scatter indices of the expert-grouped order.
//
// What is computed is the metadata the pages' grouped GEMMs consume: m_sizes,
// whose prefix sums cut the gather index into per-expert groups
// (grouped_gemm_forward docstring, unsloth grouped_gemm/interface.py), expt_hist with its cumsum
// offsets and block-padded offsets, and the inverse index pair of
// GatherIndx / ScatterIndx (triton_kernels/matmul_ogs.py).
//
// Design (three launches on the caller's stream):
//   1. route_count: every wave owns kSlotsPerWave consecutive slots (a
//      "chunk") and counts them per expert.  Lanes holding the same expert id
//      find each other with one wave ballot per id bit; the lowest such lane
//      adds the group's popcount to a wave-private LDS histogram, so there is
//      one LDS update per (expert, 64 slots) instead of one per slot.  Counts
//      go to workspace as counts[e][chunk] (expert-major).
//   2. route_scan: one wave per expert turns its row counts[e][c] into the
//      number of expert-e slots in chunks before c (wave shuffles, all loads
//      of a batch in flight at once) and writes the expert's total, m_sizes[e].
//   3. route_scatter: every workgroup scans m_sizes over the experts in LDS
//      (the offsets; workgroup 0 also writes them out with the padded and
//      tile offsets), then each wave starts a per-expert cursor at
//      offsets[e] + counts[e][chunk] and walks its chunk 64 slots at a time;
//      a slot's position is its cursor plus the number of lower lanes with
//      the same expert.  Chunks are in slot order and lanes are in slot
//      order, so the result is the stable counting sort, bit for bit.
#include <mutex>

#include "common.h"

#include "gemm_params.h"

namespace moegg {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kSlotsPerWave = 256;
constexpr int kScanThreads = 256;  // one expert row per wave

// Lanes (of the active, valid ones) that hold the same id as this lane.
__device__ __forceinline__ uint64_t same_id_lanes(int id, bool valid, int nbits)
{
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (id >> b) & 1;
        const uint64_t on = __ballot(valid && bit);
        m &= bit ? on : ~on;
    }
    return m;
}

__device__ __forceinline__ uint64_t lanes_below()
{
    const int lane = threadIdx.x & (kWave - 1);
    return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}

// The ids of a wave's chunk: step st of this lane is slot base + 64 st +
// lane (-1 past S).  All loads are issued before any is used: one memory
// round trip instead of one per step.
__device__ __forceinline__ void load_chunk_ids(const int32_t *__restrict__ ids, int64_t base,
                                               int64_t S, bool live, int (&id)[kSlotsPerWave / kWave])
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int st = 0; st < kSlotsPerWave / kWave; ++st) {
        const int64_t s = base + st * kWave + lane;
        id[st] = live ? ids[min(s, S - 1)] : -1;
        if (!live || s >= S)
            id[st] = -1;
    }
}

__global__ __launch_bounds__(kRouteThreads) void route_count(const int32_t *__restrict__ ids,
                                                             int64_t S, int E, int nbits,
                                                             int nchunks, int32_t *counts,
                                                             int32_t *err)
{
    __shared__ int hist[kRouteWaves][kMaxExperts];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int chunk = blockIdx.x * kRouteWaves + wave;
    const int64_t base = (int64_t)chunk * kSlotsPerWave;
    int ids_[kSlotsPerWave / kWave];
    load_chunk_ids(ids, base, S, chunk < nchunks, ids_);
    for (int e = lane; e < E; e += kWave)
        hist[wave][e] = 0;
    __syncthreads();
    bool dropped = false;
#pragma unroll
    for (int step = 0; step < kSlotsPerWave / kWave; ++step) {
        const int64_t s = base + step * kWave + lane;
        const bool in = chunk < nchunks && s < S;
        const int id = ids_[step];
        const bool valid = in && id >= 0 && id < E;
        dropped |= in && !valid;
        const uint64_t peers = same_id_lanes(id, valid, nbits);
        if (valid && (peers & lanes_below()) == 0)
            atomicAdd(&hist[wave][id], __popcll(peers));
    }
    __syncthreads();
    if (chunk < nchunks)
        for (int e = lane; e < E; e += kWave)
            counts[(int64_t)e * nchunks + chunk] = hist[wave][e];
    if (dropped)
        raise_error(err, kErrExpertId);
}

__global__ __launch_bounds__(kScanThreads) void route_scan(int32_t *counts, int nchunks, int E,
                                                           int32_t *m_sizes)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int e = blockIdx.x * (kScanThreads / kWave) + threadIdx.x / kWave;
    if (e >= E)
        return;
    // A lane owns kPer consecutive chunks of each batch; all loads of a batch
    // are issued before any is used, so a batch costs one memory round trip.
    constexpr int kPer = 8;
    int32_t *const row = counts + (int64_t)e * nchunks;
    int carry = 0;
    for (int c0 = 0; c0 < nchunks; c0 += kWave * kPer) {
        int v[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int c = c0 + lane * kPer + q;
            v[q] = c < nchunks ? row[c] : 0;
        }
        int local = 0;
#pragma unroll
        for (int q = 0; q < kPer; ++q)
            local += v[q];
        int incl = local;
        for (int d = 1; d < kWave; d <<= 1) {
            const int u = __shfl_up(incl, d, kWave);
            if (lane >= d)
                incl += u;
        }
        int run = carry + incl - local;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int c = c0 + lane * kPer + q;
            if (c < nchunks)
                row[c] = run;
            run += v[q];
        }
        carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0)
        m_sizes[e] = carry;
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter(
    const int32_t *__restrict__ ids, int64_t S, int E, int nbits, int nchunks, int block_m,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ m_sizes, int32_t *offsets,
    int32_t *padded_offsets, int32_t *tile_offsets, int32_t *gather, int32_t *scatter)
{
    __shared__ int cursor[kRouteWaves][kMaxExperts];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int chunk = blockIdx.x * kRouteWaves + wave;
    const int64_t base = (int64_t)chunk * kSlotsPerWave;
    __shared__ int off[kMaxExperts];
    __shared__ int totals[3];
    int ids_[kSlotsPerWave / kWave];
    load_chunk_ids(ids, base, S, chunk < nchunks, ids_);
    for (int e = threadIdx.x; e < E; e += kRouteThreads)
        off[e] = m_sizes[e];
    if (chunk < nchunks)
        for (int e = lane; e < E; e += kWave)
            cursor[wave][e] = counts[(int64_t)e * nchunks + chunk];
    if (blockIdx.x == 0) {
        // Workgroup 0 also writes out the padded and tile offsets.
        __shared__ int poff[kMaxExperts];
        __shared__ int toff[kMaxExperts];
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += kRouteThreads) {
            const int tiles = (off[e] + block_m - 1) / block_m;
            poff[e] = tiles * block_m;
            toff[e] = tiles;
        }
        wave0_exclusive_scan(poff, E, &totals[1]);
        wave0_exclusive_scan(toff, E, &totals[2]);
        for (int e = threadIdx.x; e < E; e += kRouteThreads) {
            if (padded_offsets)
                padded_offsets[e] = poff[e];
            if (tile_offsets)
                tile_offsets[e] = toff[e];
        }
    }
    wave0_exclusive_scan(off, E, &totals[0]);
    if (blockIdx.x == 0) {
        for (int e = threadIdx.x; e < E; e += kRouteThreads)
            offsets[e] = off[e];
        if (threadIdx.x == 0) {
            offsets[E] = totals[0];
            if (padded_offsets)
                padded_offsets[E] = totals[1];
            if (tile_offsets)
                tile_offsets[E] = totals[2];
        }
    }
    // Positions left over by dropped slots hold -1.
    for (int64_t p = totals[0] + (int64_t)blockIdx.x * kRouteThreads + threadIdx.x; p < S;
         p += (int64_t)gridDim.x * kRouteThreads)
        gather[p] = -1;
    if (chunk < nchunks)
        for (int e = lane; e < E; e += kWave)
            cursor[wave][e] += off[e];
    __syncthreads();
#pragma unroll
    for (int step = 0; step < kSlotsPerWave / kWave; ++step) {
        const int64_t s = base + step * kWave + lane;
        const bool in = chunk < nchunks && s < S;
        const int id = ids_[step];
        const bool valid = in && id >= 0 && id < E;
        const uint64_t peers = same_id_lanes(id, valid, nbits);
        const uint64_t below = peers & lanes_below();
        // All lanes read their cursor before any group leader advances it.
        const int start = valid ? cursor[wave][id] : 0;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            const int pos = start + __popcll(below);
            gather[pos] = (int32_t)s;
            if (scatter)
                scatter[s] = pos;
            if (below == 0)
                cursor[wave][id] = start + __popcll(peers);
        } else if (in && scatter) {
            scatter[s] = -1;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// All three phases in one workgroup, for up to kSmallWaves x kSmallSteps x
// 64 = 4096 slots (a decode step's few hundred).  The slots are cut into
// kSmallWaves consecutive chunks of `steps` x 64 slots (steps = 1 .. 4, as
// few as cover S, so that a small step spreads over all waves): wave w
// counts chunk w into hist[w], the workgroup turns the counts into
// per-chunk starts and the offsets, and wave w then scatters chunk w from
// its cursors.  Each lane loads all its ids at once and keeps them in
// registers for the scatter.  Chunks and lanes are in slot order, so this is
// the same stable counting sort as the three launches above, bit for bit, in
// one launch instead of three.
constexpr int kSmallWaves = 16;
constexpr int kSmallThreads = kSmallWaves * kWave;
constexpr int kSmallSteps = 4;  // 16 measured slower on 512 slots (6.7 against 5.5 us)
constexpr int64_t kSmallSlots = (int64_t)kSmallThreads * kSmallSteps;

__global__ __launch_bounds__(kSmallThreads) void route_small(
    const int32_t *__restrict__ ids, int64_t S, int E, int nbits, int block_m, int32_t *m_sizes,
    int32_t *offsets, int32_t *padded_offsets, int32_t *tile_offsets, int32_t *gather,
    int32_t *scatter, int32_t *err)
{
    __shared__ int hist[kSmallWaves][kMaxExperts];  // counts, then chunk starts, then cursors
    __shared__ int off[kMaxExperts];
    __shared__ int poff[kMaxExperts];
    __shared__ int toff[kMaxExperts];
    __shared__ int totals[3];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int steps = (int)((S + kSmallThreads - 1) / kSmallThreads);  // <= kSmallSteps
    const int64_t base = (int64_t)wave * steps * kWave;
    int id[kSmallSteps];
#pragma unroll
    for (int st = 0; st < kSmallSteps; ++st) {
        const int64_t sl = base + st * kWave + lane;
        id[st] = (S > 0) ? ids[min(sl, S - 1)] : -1;  // every load in flight at once
        if (st >= steps || sl >= S)
            id[st] = -1;
    }
    for (int e = lane; e < E; e += kWave)
        hist[wave][e] = 0;
    __syncthreads();
    bool dropped = false;
#pragma unroll
    for (int st = 0; st < kSmallSteps; ++st) {
        if (st >= steps)
            break;
        const bool in = base + st * kWave + lane < S;
        const bool valid = in && id[st] >= 0 && id[st] < E;
        dropped |= in && !valid;
        const uint64_t peers = same_id_lanes(id[st], valid, nbits);
        if (valid && (peers & lanes_below()) == 0)
            atomicAdd(&hist[wave][id[st]], __popcll(peers));
    }
    if (dropped)
        raise_error(err, kErrExpertId);
    __syncthreads();
    // Per expert: counts of the chunks before each chunk, and the total.
    for (int e = threadIdx.x; e < E; e += kSmallThreads) {
        int run = 0;
        for (int w = 0; w < kSmallWaves; ++w) {
            const int c = hist[w][e];
            hist[w][e] = run;
            run += c;
        }
        const int tiles = (run + block_m - 1) / block_m;
        m_sizes[e] = run;
        off[e] = run;
        poff[e] = tiles * block_m;
        toff[e] = tiles;
    }
    wave0_exclusive_scan(off, E, &totals[0]);
    wave0_exclusive_scan(poff, E, &totals[1]);
    wave0_exclusive_scan(toff, E, &totals[2]);
    for (int e = threadIdx.x; e < E; e += kSmallThreads) {
        offsets[e] = off[e];
        if (padded_offsets)
            padded_offsets[e] = poff[e];
        if (tile_offsets)
            tile_offsets[e] = toff[e];
        for (int w = 0; w < kSmallWaves; ++w)
            hist[w][e] += off[e];  // cursor of chunk w
    }
    if (threadIdx.x == 0) {
        offsets[E] = totals[0];
        if (padded_offsets)
            padded_offsets[E] = totals[1];
        if (tile_offsets)
            tile_offsets[E] = totals[2];
    }
    for (int64_t p = totals[0] + threadIdx.x; p < S; p += kSmallThreads)
        gather[p] = -1;  // positions left over by dropped slots
    __syncthreads();
#pragma unroll
    for (int st = 0; st < kSmallSteps; ++st) {
        if (st >= steps)
            break;
        const int64_t sl = base + st * kWave + lane;
        const bool in = sl < S;
        const bool valid = in && id[st] >= 0 && id[st] < E;
        const uint64_t peers = same_id_lanes(id[st], valid, nbits);
        const uint64_t below = peers & lanes_below();
        // All lanes read their cursor before any group leader advances it.
        const int start = valid ? hist[wave][id[st]] : 0;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            const int pos = start + __popcll(below);
            gather[pos] = (int32_t)sl;
            if (scatter)
                scatter[sl] = pos;
            if (below == 0)
                hist[wave][id[st]] = start + __popcll(peers);
        } else if (in && scatter) {
            scatter[sl] = -1;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

static int bits_for(int E)
{
    int b = 0;
    while ((1 << b) < E)
        ++b;
    return b;
}

int64_t route_chunks(int64_t S)
{
    return (S + kSlotsPerWave - 1) / kSlotsPerWave;
}

// Per-chunk counts of moegg_route_noalloc: a device array the library holds
// on every device it runs on (one copy per device, at its own address) until
// the process ends.  route_count writes every count route_scan and
// route_scatter read, so the array needs no clearing between calls.
static __device__ __align__(256) int32_t scratch[MOEGG_ROUTE_NOALLOC_MAX_BYTES / sizeof(int32_t)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
int32_t *g_scratch[kMaxScratchDevices];  // device address of `scratch`, per device
}  // namespace

// Device address of the current device's `scratch`, looked up once per
// device (host code must not pass the array's own name to a kernel: that is
// a host-side stand-in, not a device address).
hipError_t route_scratch(int32_t **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch[dev] = static_cast<int32_t *>(p);
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

hipError_t route_launch(const int32_t *ids, int64_t S, int E, int block_m, int32_t *m_sizes,
                        int32_t *offsets, int32_t *padded_offsets, int32_t *tile_offsets,
                        int32_t *gather, int32_t *scatter, int32_t *counts, int32_t *err,
                        hipStream_t stream)
{
    const int nchunks = (int)route_chunks(S);
    const int nbits = bits_for(E);
    const int blocks = (nchunks + kRouteWaves - 1) / kRouteWaves;
    if (S <= kSmallSlots) {
        hipLaunchKernelGGL(route_small, dim3(1), dim3(kSmallThreads), 0, stream, ids, S, E, nbits,
                           block_m, m_sizes, offsets, padded_offsets, tile_offsets, gather,
                           scatter, err);
        return hipGetLastError();
    }
    if (nchunks > 0) {
        hipLaunchKernelGGL(route_count, dim3(blocks), dim3(kRouteThreads), 0, stream, ids, S, E,
                           nbits, nchunks, counts, err);
    }
    hipLaunchKernelGGL(route_scan, dim3((E + kScanThreads / kWave - 1) / (kScanThreads / kWave)),
                       dim3(kScanThreads), 0, stream, counts, nchunks, E, m_sizes);
    hipLaunchKernelGGL(route_scatter, dim3(blocks), dim3(kRouteThreads), 0, stream, ids, S, E,
                       nbits, nchunks, block_m, counts, m_sizes, offsets, padded_offsets,
                       tile_offsets, gather, scatter);
    return hipGetLastError();
}

}  // namespace moegg
