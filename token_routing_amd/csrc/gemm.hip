// Persistent grouped-GEMM kernels for gfx950: forward (with permute_x,
// permute_y, fuse_mul_post and the gated activation), dX, dW (ragged
// reduction per expert, optionally split for hot experts) and explicit GEMM
// groups.
//
// The operations are those of grouped_gemm_forward / grouped_gemm_dX /
// grouped_gemm_dW (unsloth grouped_gemm/interface.py), whose per-expert
// meaning is the loop of matmul_ogs_torch (triton_kernels/matmul_ogs.py), and
// of asym_dual_gmm_separated (wall_x/fusions/backend.py) for the groups.
//
// One engine serves all of them.  A workgroup owns an output tile of BM x BN
// and walks the reduction in stages of BK = 64 elements:
//   * Operands whose reduction index is contiguous in HBM (X and W in the
//     forward, dY in dX) sit in LDS "reduction-contiguous": a tile row is the
//     64 reduction elements (128 bytes) of one output row or column, 16-byte
//     chunk c of row r at chunk c ^ ((r / 2) mod 8), so 16 rows read at one
//     chunk hit 16 different bank groups.
//   * Operands whose reduction index runs across HBM rows (W in dX, dY and X
//     in dW, a [K, N] weight in the groups) sit in LDS as in HBM (reduction
//     rows), chunks swizzled by (row mod 4) * 4, and their MFMA fragments are
//     read with the transposing LDS read ds_read_b64_tr_b16.
//   * Both are copied HBM -> LDS by buffer_load ... lds (no registers), 16
//     bytes per lane, whole 128-byte row segments per eight lanes; gathered
//     rows (permute_x, permute_y on load) are just per-lane row offsets.
//   * v_mfma_f32_32x32x16_bf16 with fp32 accumulators; fragment reads run one
//     16-deep step ahead of the MFMAs.  Two LDS stages: the copies of stage
//     s+1 are in flight while the MFMAs consume stage s; one barrier per
//     stage.  Long dX reductions use a four-wave engine with four 32-deep
//     slots instead (see below).
//   * bf16 epilogue: fp32 accumulators (times the gate weight under
//     fuse_mul_post) are rounded to bf16 into LDS, then written out as
//     16-byte row segments, to row gather[p] under permute_y.
//   * Persistent grid of (CUs x resident workgroups).  Every workgroup reads
//     m_sizes and builds the tile map in LDS (no host synchronisation); tile
//     t belongs to the expert whose tile range holds it.  Workgroup ids are
//     remapped so that consecutive tiles run on the same XCD (own L2), and
//     within an expert the M tiles of one N panel are consecutive, so the
//     weight panel is fetched from HBM once per XCD.
#include <type_traits>

#include "common.h"

#include "gemm_params.h"

namespace moegg {

constexpr int BK = 64;
constexpr int kChunks = BK / 8;  // 16-byte chunks per LDS row

// LDS tile rows are 128 bytes (64 bf16).  gfx950 serves a 16-byte-per-lane
// LDS access 16 lanes (256 bytes, 64 banks) at a time, so 16 consecutive rows
// read at one logical chunk must fall in 16 distinct 16-byte bank groups:
// even and odd rows occupy the two 128-byte halves, and XOR-ing the chunk
// with (row / 2) % 8 spreads each parity class over all 8 groups of its half.
__device__ __forceinline__ int swz_chunk(int row, int chunk)
{
    return chunk ^ ((row >> 1) & 7);
}

__device__ __forceinline__ int lds_swz(int row, int chunk)
{
    return row * (BK * 2) + (swz_chunk(row, chunk) << 4);
}

template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NT = kWave * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
};

__device__ __forceinline__ uint32_t dw(const uint4 &v, int d)
{
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// Operand loaders
// ---------------------------------------------------------------------------

// Raw buffer resources: a 32-bit byte offset per lane and a uniform
// descriptor.  An offset at or past num_records reads as zero, so a masked
// row or column is the offset kOOB (operands are limited to 2 GiB each).
constexpr uint32_t kOOB = 0x80000000u;

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor words (uniform): base, stride 0, num_records, format.
__device__ __forceinline__ u32x4_t rsrc_words(const void *base, int64_t bytes)
{
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    u32x4_t w;
    w.x = __builtin_amdgcn_readfirstlane((uint32_t)b);
    w.y = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu);
    w.z = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
    w.w = 0x00020000u;
    return w;
}

// 16 bytes per lane copied HBM -> LDS without passing through registers
// (buffer_load_dwordx4 ... lds): lane l writes LDS bytes [16 l, 16 l + 16)
// from lds_addr (a wave's 1 KiB window).  The copy is issued from inline
// assembly, so the compiler does not know it writes LDS and does not hold
// back LDS reads of the other stage until it lands; every loop waits for it
// explicitly (wait_vmem / wait_vmcnt) before the barrier that publishes the
// stage.  Vector-memory loads complete in issue order, so any wait the
// compiler inserts for its own loads can only wait longer.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const u32x4_t &r, uint32_t voff, uint32_t soff,
                                              uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(soff), "s"(lds_addr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a pointer into a __shared__ array: the low 32 bits of
// its flat address (the shared aperture is the high half).  Taken by
// truncation rather than an address-space cast, whose null check the
// compiler can mislower when the address is a constant under a branch.
__device__ __forceinline__ uint32_t lds_u32(const void *p)
{
    return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// ROWS tile rows, reduction contiguous in HBM, copied with copy16_to_lds.
// Lane l of a wave writes physical chunk l % 8 of window row l / 8; to land
// in the swizzled layout it fetches the logical chunk that swizzles to it
// (the swizzle is an involution).  Wave w, pass i fills rows
// 8 w + i * (NT / 8) .. + 7, so the eight lanes of a row still read one whole
// 128-byte row segment.
template <int ROWS, int NT>
struct DmaLoader {
    static constexpr int PASS = NT / kChunks;
    static constexpr int RPT = ROWS / PASS;
    static_assert(ROWS % PASS == 0, "DMA loader covers whole passes");
    uint32_t off[RPT];

    __device__ __forceinline__ static int tile_row(int i) { return (threadIdx.x >> 3) + i * PASS; }

    // Lane l of wave w fills row 8 w + l / 8 + i * PASS (PASS is a multiple of
    // 16, so the swizzle depends only on threadIdx.x / 8) at physical chunk l % 8.
    static_assert(PASS % 16 == 0, "swizzle period");
    __device__ __forceinline__ static int chunk()
    {
        return swz_chunk(threadIdx.x >> 3, threadIdx.x & 7);
    }

    __device__ __forceinline__ void set_row(int i, int64_t row, int64_t row_bytes)
    {
        off[i] = row < 0 ? kOOB : (uint32_t)(row * row_bytes) + chunk() * 16;
    }

    // Enqueue the copies of reduction stage k0 into the LDS stage `lds`.
    __device__ __forceinline__ void load(const u32x4_t &r, char *lds, int k0, int klen) const
    {
        const bool kin = k0 + chunk() * 8 < klen;
        const uint32_t wave_row = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave) * 8;
        const uint32_t base = lds_u32(lds);
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            copy16_to_lds(r, kin ? off[i] : kOOB, (uint32_t)k0 * 2,
                          __builtin_amdgcn_readfirstlane(base + (i * PASS + wave_row) * (BK * 2)));
    }
};

// Wait until this wave's outstanding vector-memory operations (including
// HBM -> LDS copies) have completed: s_waitcnt vmcnt(0), other counters free.
__device__ __forceinline__ void wait_vmem()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Operands whose reduction index runs across HBM rows (W in dX, dY and X in
// dW, a [K, N] weight in the groups) are kept in LDS as they are in HBM: BK
// reduction rows of COLS bf16 (row pitch 2 COLS bytes).  The MFMA fragments
// are then read with the gfx950 LDS transpose read (tr_frag below).  16-byte
// chunk c of row r is stored at chunk c ^ ((r % 4) * 4), so the four rows one
// transpose read touches fall in four different 64-byte bank groups.
template <int COLS>
__device__ __forceinline__ int tr_off(int row, int chunk)
{
    static_assert(COLS >= 128, "the row swizzle needs 16 chunks per row");
    return row * (COLS * 2) + ((chunk ^ ((row & 3) << 2)) << 4);
}

// A row-major tile (BK reduction rows of COLS columns) copied HBM -> LDS
// without registers.  A wave's
// 1 KiB window is RW = 64 / (COLS / 8) whole rows; lane l writes physical
// chunk l % (COLS / 8) of window row l / (COLS / 8) and therefore fetches the
// logical chunk that the row swizzle maps there.
//
// Row indices are three-phase: fetch(red0, raw) only issues the loads of the
// next stage's raw row indices (e.g. gather entries) into registers; at the
// next stage, prepare(…, fin) turns them into byte offsets and issue() starts
// the copies.  The raw values are consumed a whole stage after they were
// requested, and every prepare of a stage runs before its first copy is
// issued: the compiler (which does not see the copies) may insert a wait for
// the raw loads there, and at that point nothing else is in flight.
//
// D: reduction rows per LDS stage (BK, or a shorter slot).
template <int COLS, int NT, int D = BK>
struct TileDmaLoader {
    static constexpr int CPR = COLS / 8;
    static constexpr int RW = kWave / CPR;
    static constexpr int NWAVE = NT / kWave;
    static constexpr int RPT = D / (RW * NWAVE);
    static_assert(kWave % CPR == 0 && D % (RW * NWAVE) == 0, "whole windows per stage");
    static_assert(COLS >= 128, "the row swizzle needs 16 chunks per row");
    int32_t raw[RPT];
    int red0 = 0;

    __device__ __forceinline__ static int window(int i) { return threadIdx.x / kWave + i * NWAVE; }
    __device__ __forceinline__ static int row_of(int i)
    {
        return window(i) * RW + (int)(threadIdx.x % kWave) / CPR;
    }

    // rawfn(red) -> the raw row index of reduction index red (a load or a
    // plain value; must stay in bounds for any red).
    template <class RawFn>
    __device__ __forceinline__ void fetch(int red_base, RawFn rawfn)
    {
        red0 = red_base;
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            raw[i] = rawfn(red_base + row_of(i));
    }

    // Turn the raw indices fetched last into byte offsets: fin(red, raw) ->
    // HBM row (-1: zeros); row_bytes is the HBM pitch.  Call before issuing
    // any copy of the stage (the load callbacks of dx_kernel and dw_kernel).
    template <class FinFn>
    __device__ __forceinline__ void prepare(int col0, int ncols, int64_t row_bytes, FinFn fin)
    {
        const int pc = (int)(threadIdx.x % kWave) % CPR;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = row_of(i);
            const int idx = fin(red0 + row, raw[i]);
            const int col = col0 + (pc ^ ((row & 3) << 2)) * 8;
            voff[i] = (idx >= 0 && col < ncols)
                          ? (uint32_t)idx * (uint32_t)row_bytes + (uint32_t)col * 2
                          : kOOB;
        }
    }

    // One-phase form: rowfn(row) -> HBM row of tile row `row` (-1: zeros),
    // for row indices that need no memory load of their own.
    template <class RowFn>
    __device__ __forceinline__ void prepare_rows(int col0, int ncols, int64_t row_bytes,
                                                 RowFn rowfn)
    {
        const int pc = (int)(threadIdx.x % kWave) % CPR;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = row_of(i);
            const int idx = rowfn(row);
            const int col = col0 + (pc ^ ((row & 3) << 2)) * 8;
            voff[i] = (idx >= 0 && col < ncols)
                          ? (uint32_t)idx * (uint32_t)row_bytes + (uint32_t)col * 2
                          : kOOB;
        }
    }

    // Copy the prepared rows into the LDS tile.
    __device__ __forceinline__ void issue(const u32x4_t &r, char *lds) const
    {
        const uint32_t base = lds_u32(lds);
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            copy16_to_lds(r, voff[i], 0,
                          __builtin_amdgcn_readfirstlane(base + window(i) * (kWave * 16)));
    }

    uint32_t voff[RPT];
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// MFMA fragment (8 reduction elements of one column, lane layout of
// v_mfma_f32_32x32x16_bf16) of columns [c0, c0 + 32), reduction rows
// [16 kk, 16 kk + 16), from a row-major LDS tile.  ds_read_b64_tr_b16: in
// each 16-lane group, lane i receives element i % 4 of the 8 bytes addressed
// by lanes 4 j + i / 4 (j = 0..3).  Lane q of a group addresses reduction row
// q / 4 and columns 4 (q % 4) .. + 3 of its 16-column half, so lane i gets
// column i and four consecutive reduction rows; two reads give eight.
template <int COLS>
__device__ __forceinline__ bf16x8_t tr_frag(const char *tile, int kk, int c0)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int q = lane & 15;
    const int row = kk * 16 + 8 * (lane >> 5) + (q >> 2);
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (q & 3);
    const int within = (col & 7) * 2;
    typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(tile + tr_off<COLS>(row, col >> 3) + within));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(tile + tr_off<COLS>(row + 4, col >> 3) + within));
    const v4i16_t both[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8_t, both);
}

// ---------------------------------------------------------------------------
// MFMA stage and mainloop
// ---------------------------------------------------------------------------

// Fragments of one 16-deep step.  A_TR / B_TR: the operand's LDS tile is
// row-major (reduction rows) and is read with transpose reads; otherwise it
// is reduction-contiguous (lds_swz layout).
// ib: number of leading 32-row A blocks holding real rows (PART only; the
// others are padding of a ragged tail tile and are neither read nor used).
template <class C, bool A_TR, bool B_TR, bool PART = false>
__device__ __forceinline__ void read_step(const char *As, const char *Bs, int kk, int wm, int wn,
                                          bf16x8_t (&a)[C::FM], bf16x8_t (&b)[C::FN], int ib = 0)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int r = lane & 31, chunk = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        if (PART && i >= ib)
            continue;
        if constexpr (A_TR)
            a[i] = tr_frag<C::BM>(As, kk, wm * C::TM + i * 32);
        else
            a[i] = *reinterpret_cast<const bf16x8_t *>(As + lds_swz(wm * C::TM + i * 32 + r, chunk));
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
        if constexpr (B_TR)
            b[j] = tr_frag<C::BN>(Bs, kk, wn * C::TN + j * 32);
        else
            b[j] = *reinterpret_cast<const bf16x8_t *>(Bs + lds_swz(wn * C::TN + j * 32 + r, chunk));
    }
}

template <class C, bool PART = false>
__device__ __forceinline__ void mma_step(const bf16x8_t (&a)[C::FM], const bf16x8_t (&b)[C::FN],
                                         f32x16_t (&acc)[C::FM][C::FN], int ib = 0)
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        if (PART && i >= ib)
            continue;
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
}

// PIPE = false: each step's reads directly precede its MFMAs (fewer live
// registers).  PART: only the first ib 32-row A blocks are computed.
template <class C, bool PIPE, bool A_TR, bool B_TR, bool PART = false>
__device__ __forceinline__ void mma_stage(const char *As, const char *Bs,
                                          f32x16_t (&acc)[C::FM][C::FN], int wm, int wn,
                                          int ib = C::FM)
{
    if (!PIPE) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8_t a[C::FM], b[C::FN];
            read_step<C, A_TR, B_TR, PART>(As, Bs, kk, wm, wn, a, b, ib);
            mma_step<C, PART>(a, b, acc, ib);
        }
        return;
    }
    // sched_barrier(0) keeps the compiler from moving the reads back next to
    // their consumers.
    bf16x8_t a0[C::FM], b0[C::FN], a1[C::FM], b1[C::FN];
    read_step<C, A_TR, B_TR, PART>(As, Bs, 0, wm, wn, a0, b0, ib);
    read_step<C, A_TR, B_TR, PART>(As, Bs, 1, wm, wn, a1, b1, ib);
    __builtin_amdgcn_sched_barrier(0);
    mma_step<C, PART>(a0, b0, acc, ib);
    __builtin_amdgcn_sched_barrier(0);
    read_step<C, A_TR, B_TR, PART>(As, Bs, 2, wm, wn, a0, b0, ib);
    __builtin_amdgcn_sched_barrier(0);
    mma_step<C, PART>(a1, b1, acc, ib);
    __builtin_amdgcn_sched_barrier(0);
    read_step<C, A_TR, B_TR, PART>(As, Bs, 3, wm, wn, a1, b1, ib);
    __builtin_amdgcn_sched_barrier(0);
    mma_step<C, PART>(a0, b0, acc, ib);
    __builtin_amdgcn_sched_barrier(0);
    mma_step<C, PART>(a1, b1, acc, ib);
}

template <class C>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[C::FM][C::FN])
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;
}

// Two LDS stages.  Per stage s: start the copies of stage s+1 straight into
// the other LDS stage, run the MFMAs of stage s from LDS, wait for this
// wave's copies, and barrier.  load(s, As, Bs) starts the copies of stage s.
// The other stage was last read before the previous barrier, so it is free
// to fill.
template <class C, bool PIPE, bool A_TR, bool B_TR, bool PART, class Load>
__device__ __forceinline__ void mainloop_body(char *st0, char *st1, int nsteps,
                                              f32x16_t (&acc)[C::FM][C::FN], Load &load, int wm,
                                              int wn, int ib)
{
    load(0, st0, st0 + C::A_BYTES);
    wait_vmem();
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        char *cur = (s & 1) ? st1 : st0;
        char *nxt = (s & 1) ? st0 : st1;
        if (s + 1 < nsteps)
            load(s + 1, nxt, nxt + C::A_BYTES);
        mma_stage<C, PIPE, A_TR, B_TR, PART>(cur, cur + C::A_BYTES, acc, wm, wn, ib);
        wait_vmem();
        __syncthreads();
    }
}

// rows: tile rows (A side) holding real data.  A wave whose 32-row blocks
// are all real runs the branch-free body; a wave of a ragged tail tile skips
// the MFMAs and A reads of its padding blocks (the barriers are the same).
template <class C, bool PIPE, bool A_TR, bool B_TR, class Load>
__device__ __forceinline__ void mainloop(char *st0, char *st1, int nsteps,
                                         f32x16_t (&acc)[C::FM][C::FN], Load load,
                                         int rows = C::BM)
{
    const int wave = threadIdx.x / kWave;
    const int wm = wave / C::WN, wn = wave % C::WN;
    if (nsteps <= 0)
        return;
    const int ib = __builtin_amdgcn_readfirstlane(
        min(C::FM, max(0, (rows - wm * C::TM + 31) / 32)));
    if (ib == C::FM)
        mainloop_body<C, PIPE, A_TR, B_TR, false>(st0, st1, nsteps, acc, load, wm, wn, ib);
    else
        mainloop_body<C, PIPE, A_TR, B_TR, true>(st0, st1, nsteps, acc, load, wm, wn, ib);
}

// ---------------------------------------------------------------------------
// 32-deep LDS slots and explicit waits
// ---------------------------------------------------------------------------

constexpr int SK = 32;        // reduction elements per slot
constexpr int kSlots = 4;

// 64-byte slot rows: 16 rows read at one logical chunk land in 16 distinct
// 16-byte bank groups of a 256-byte bank window (4 rows per window, the
// chunk XOR-ed with (row / 4) % 4).
__device__ __forceinline__ int slot_off(int row, int chunk)
{
    return row * (SK * 2) + ((chunk ^ ((row >> 2) & 3)) << 4);
}

__device__ __forceinline__ void wg_barrier()
{
    asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ void wait_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One wave's share of one operand of a slot: NC windows of 16 rows x 64
// bytes.  Lane l writes window row l / 4 at physical chunk l % 4 and so
// fetches the logical chunk that slot_off maps there.
template <int NC>
struct SlotCopier {
    uint32_t off[NC];  // HBM byte offset of this lane's row + chunk (kOOB: zero row)
    int kc;            // reduction offset of this lane's chunk within a slot
    uint32_t lds0;     // LDS address of the wave's first window in slot 0

    __device__ __forceinline__ static int lane() { return threadIdx.x & (kWave - 1); }
    // Tile row of window j for this lane (first_row: the wave's first row).
    __device__ __forceinline__ static int row(int first_row, int j)
    {
        return first_row + 16 * j + (lane() >> 2);
    }
    __device__ __forceinline__ void init(char *slot0_part, int first_row)
    {
        const int lc = (lane() & 3) ^ ((lane() >> 4) & 3);
        kc = lc * 8;
        lds0 = __builtin_amdgcn_readfirstlane(lds_u32(slot0_part)) + first_row * (SK * 2);
    }
    __device__ __forceinline__ void set_row(int j, int64_t hbm_row, int64_t row_bytes)
    {
        off[j] = hbm_row < 0 ? kOOB : (uint32_t)(hbm_row * row_bytes) + (uint32_t)kc * 2;
    }
    // Copy j of reduction elements [k0, k0 + 32) into slot buffer `slot`.
    template <int SLOT_BYTES>
    __device__ __forceinline__ void issue_one(const u32x4_t &r, int j, int slot, int k0,
                                              int klen) const
    {
        copy16_to_lds(r, k0 + kc < klen ? off[j] : kOOB, (uint32_t)k0 * 2,
                      lds0 + (uint32_t)(slot * SLOT_BYTES + j * kWave * 16));
    }
    // Copies of reduction elements [k0, k0 + 32) into slot buffer `slot`.
    template <int SLOT_BYTES>
    __device__ __forceinline__ void issue(const u32x4_t &r, int slot, int k0, int klen) const
    {
        const bool kin = k0 + kc < klen;
#pragma unroll
        for (int j = 0; j < NC; ++j)
            copy16_to_lds(r, kin ? off[j] : kOOB, (uint32_t)k0 * 2,
                          lds0 + (uint32_t)(slot * SLOT_BYTES + j * kWave * 16));
    }
};

// Fragments of 16-deep step kk (0 or 1) of a slot.
template <class C, bool PART>
__device__ __forceinline__ void read_slot_step(const char *As, const char *Bs, int kk, int wm,
                                               int wn, bf16x8_t (&a)[C::FM],
                                               bf16x8_t (&b)[C::FN], int ib)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int r = lane & 31, chunk = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        if (PART && i >= ib)
            continue;
        a[i] = *reinterpret_cast<const bf16x8_t *>(As + slot_off(wm * C::TM + i * 32 + r, chunk));
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t *>(Bs + slot_off(wn * C::TN + j * 32 + r, chunk));
}

// Wait for the copy batch `newer` batches older than the newest (each batch
// is NC copies of this wave).
template <int NC>
__device__ __forceinline__ void wait_batch(int newer)
{
    if (newer >= 2)
        wait_vmcnt<2 * NC>();
    else if (newer == 1)
        wait_vmcnt<NC>();
    else
        wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Four-wave engine: one wave per SIMD, 128 x 128 outputs per wave
// ---------------------------------------------------------------------------
//
// LDS read bandwidth (about 128 bytes per clock per CU) is what bounds a
// bf16 MFMA tile on this chip.  A wave computing FM x FN blocks of 32 x 32
// reads FM + FN fragments of 1 KiB per 16-deep step for FM * FN MFMAs, so a
// 128 x 128 wave tile (4 x 4) needs 0.5 KiB of LDS reads per MFMA against
// 0.75 KiB for 128 x 64.  With 256 accumulators per wave that allows one
// wave per SIMD: four waves cover a 256 x 256 tile.
//
// The wave hides latency by itself: every MFMA of a 16-deep step is followed
// by one memory operation, reads of the next step's fragments or HBM -> LDS
// copies, in a fixed order (sched_barrier pins it).  LDS holds four 32-deep
// slots (A then B, 64-byte rows, slot_off layout).  Per slot q:
//
//   phase A: MFMAs of step 0 (fragments F0)  |  reads of step 1 -> F1, then
//            half of this wave's copies of slot q + 3 (into the buffer of q - 1)
//   wait: own LDS reads, own copies of slot q + 1; barrier
//   phase B: MFMAs of step 1 (F1)            |  reads of slot q + 1 step 0 -> F0,
//            then the other half of the copies
//
// Before the barrier of slot q every wave has finished all its reads of
// slot q - 1 (its last ones were in phase A of q - 1 and were waited for at
// that slot's barrier), so after it the buffer can take copies; and every
// wave's copies of slot q + 1 have landed, so phase B may read it.  Copies
// get one and a half to two slots (1500-2000 MFMA cycles) to arrive, and the
// address unit sees four per wave per phase.

template <class C>
struct Quad {
    static_assert(C::WM == 2 && C::WN == 2 && C::FM == 4 && C::FN == 4,
                  "2 x 2 waves of 4 x 4 blocks");
    static constexpr int A = C::BM * SK * 2, B = C::BN * SK * 2, SLOT = A + B;
    static constexpr int NCA = C::BM / 64, NCB = C::BN / 64;  // copies per wave and slot
    static constexpr int NCOPY = NCA + NCB;
    static_assert(kSlots * SLOT <= 2 * C::STAGE, "four slots fit the LDS tile buffer");
};

// 2 x 2 waves of 128 x 128 run the four-wave engine.
template <class C>
struct UseQuad {
    static constexpr bool value = C::WM == 2 && C::WN == 2 && C::FM == 4 && C::FN == 4;
};

// Per-lane LDS offsets, within an operand's slot part, of the fragments of
// the wave's four 32-wide blocks for the two 16-deep steps of a slot.
//   TR = false: reduction-contiguous rows of 32 elements (slot_off layout);
//               a fragment is one 16-byte read.
//   TR = true:  32 reduction rows of COLS elements (tr_off layout); a
//               fragment is two transpose reads, rows r and r + 4 (tr_frag).
// For TR the second step's rows are 16 below the first's with the same
// swizzle (16 is a multiple of 4), so only step 0's offsets are kept and
// step 1 adds a constant that folds into the read's immediate offset.
template <bool TR, int COLS>
struct OpFrag {
    static constexpr int KK = TR ? 1 : 2;
    uint32_t off[KK][4];

    // first: the wave's first row (TR = false) or column (TR = true).
    __device__ __forceinline__ void init(int first)
    {
        const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (TR) {
                    const int q = lane & 15;
                    const int row = 8 * (lane >> 5) + (q >> 2);
                    const int col = first + i * 32 + 16 * ((lane >> 4) & 1) + 4 * (q & 3);
                    off[kk][i] = (uint32_t)(tr_off<COLS>(row, col >> 3) + (col & 7) * 2);
                } else {
                    off[kk][i] = (uint32_t)slot_off(first + i * 32 + (lane & 31),
                                                    kk * 2 + (lane >> 5));
                }
            }
    }

    __device__ __forceinline__ bf16x8_t read(const char *part, int kk, int i) const
    {
        if constexpr (TR) {
            typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
            const char *p = part + off[0][i] + kk * 16 * COLS * 2;
            const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p);
            const v4i16_t hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p + 4 * COLS * 2));
            const v4i16_t both[2] = {lo, hi};
            return __builtin_bit_cast(bf16x8_t, both);
        } else {
            return *reinterpret_cast<const bf16x8_t *>(part + off[kk][i]);
        }
    }
};

// Fragment registers of the two 16-deep steps of a slot.
struct QuadFrags {
    bf16x8_t a0[4], b0[4], a1[4], b1[4];
};

// Fragment read r (0-3: A blocks, 4-7: B blocks) of step kk of slot q.
template <class C, bool PART, class FA, class FB>
__device__ __forceinline__ void quad_read(const char *smem, int q, int kk, int r,
                                          bf16x8_t (&ta)[4], bf16x8_t (&tb)[4], int ib,
                                          const FA &fa, const FB &fb)
{
    using Q = Quad<C>;
    const char *base = smem + (q % kSlots) * Q::SLOT;
    if (r < 4) {
        if (!PART || r < ib)
            ta[r] = fa.read(base, kk, r);
    } else {
        tb[r - 4] = fb.read(base + Q::A, kk, r - 4);
    }
}

// MFMA t (block t / 4, t % 4) of one 16-deep step.
template <bool PART>
__device__ __forceinline__ void quad_mma(int t, const bf16x8_t (&ta)[4], const bf16x8_t (&tb)[4],
                                         f32x16_t (&acc)[4][4], int ib)
{
    const int i = t / 4, j = t % 4;
    if (!PART || i < ib)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[i], tb[j], acc[i][j], 0, 0, 0);
}

// One slot q.  Each phase pairs MFMA t with fragment read t (t < 8) or,
// at odd t >= 9, with a copy: phase A issues copies 0 .. NCOPY/2 - 1 of
// slot q + 3, phase B the rest.  COPIES: slot q + 3 exists; NEXT: slot q + 1
// exists (phase B reads its step 0); WAITN: copies allowed in flight at the
// barrier (those issued after slot q + 1's: slot q + 2's, and the first half
// of slot q + 3's).
template <class C, bool PART, bool COPIES, bool NEXT, int WAITN, class Copy, class FA, class FB>
__device__ __forceinline__ void quad_slot(const char *smem, int q, f32x16_t (&acc)[4][4],
                                          QuadFrags &f, Copy &copy, int ib, const FA &fa,
                                          const FB &fb)
{
    using Q = Quad<C>;
    constexpr int HALF = Q::NCOPY / 2;
    const int cq = q + kSlots - 1, cbuf = cq % kSlots;
    __builtin_amdgcn_sched_barrier(0);
    copy.phase_a(q);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        quad_mma<PART>(t, f.a0, f.b0, acc, ib);
        if (t < 8)
            quad_read<C, PART>(smem, q, 1, t, f.a1, f.b1, ib, fa, fb);
        else if (COPIES && (t & 1) && (t - 9) / 2 < HALF)
            copy(cq, cbuf, (t - 9) / 2);
        __builtin_amdgcn_sched_barrier(0);
    }
    wait_lds();
    wait_vmcnt<WAITN>();
    __builtin_amdgcn_sched_barrier(0);
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        quad_mma<PART>(t, f.a1, f.b1, acc, ib);
        if (t < 8) {
            if (NEXT)
                quad_read<C, PART>(smem, q + 1, 0, t, f.a0, f.b0, ib, fa, fb);
        } else if (COPIES && (t & 1) && (t - 9) / 2 < Q::NCOPY - HALF) {
            copy(cq, cbuf, HALF + (t - 9) / 2);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    copy.phase_b_end(q);
}

// copy(q, buf, n): this wave's copy n (0 .. NCOPY-1) of reduction slot q into
// slot buffer buf.  Hooks (no-ops in PlainCopy): prepare(q) readies the row
// offsets of slot q before its first copy (prologue); phase_a(q) and
// phase_b_end(q) bracket slot q, for copiers that fetch row indices ahead.
template <class C, bool PART, class Copy, class FA, class FB>
__device__ __forceinline__ void quad_body(const char *smem, int nslots, f32x16_t (&acc)[4][4],
                                          Copy &copy, int ib, const FA &fa, const FB &fb)
{
    using Q = Quad<C>;
    constexpr int N = Q::NCOPY;
    static_assert(N % 2 == 0 && N / 2 <= 4, "copies fit the odd steps 9..15 of each phase");
    // Let the compiler see that none of its own memory operations is pending:
    // otherwise a load still in flight at loop entry (e.g. a register
    // reload) makes it wait for vmcnt(0) inside the loop, which would also
    // drain the copies it does not know about.
    __builtin_amdgcn_s_waitcnt(0);
    QuadFrags f;
    const int pre = min(kSlots - 1, nslots);
    for (int q = 0; q < pre; ++q) {
        copy.prepare(q);
#pragma unroll
        for (int n = 0; n < N; ++n)
            copy(q, q, n);
    }
    copy.prepare(kSlots - 1);
    wait_batch<N>(pre - 1);
    wg_barrier();
#pragma unroll
    for (int r = 0; r < 8; ++r)
        quad_read<C, PART>(smem, 0, 0, r, f.a0, f.b0, ib, fa, fb);
    int q = 0;
    for (; q + kSlots - 1 < nslots; ++q)
        quad_slot<C, PART, true, true, N + N / 2>(smem, q, acc, f, copy, ib, fa, fb);
    // The last (up to) three slots: no more copies.
    if (q + 2 < nslots)
        quad_slot<C, PART, false, true, N>(smem, q++, acc, f, copy, ib, fa, fb);
    if (q + 1 < nslots)
        quad_slot<C, PART, false, true, 0>(smem, q++, acc, f, copy, ib, fa, fb);
    quad_slot<C, PART, false, false, 0>(smem, q, acc, f, copy, ib, fa, fb);
}

// NST LDS stages of BK (a ring): the copies of stage s + NST - 1 are issued
// at stage s, right after the barrier that ends every wave's reads of stage
// s - 1, whose buffer they fill; so each stage's copies have NST - 1 stages of
// MFMAs to land instead of one.  load(s, As, Bs) issues this wave's CPS copies
// of stage s (the only vector-memory operations of the loop: the waits count
// them).  Leaves LDS free for the epilogue.
template <class C, int NST, bool A_TR, bool B_TR, int CPS, bool PART, class Load>
__device__ __forceinline__ void ring_body(char *smem, int nsteps, f32x16_t (&acc)[C::FM][C::FN],
                                          Load &load, int wm, int wn, int ib)
{
    static_assert(NST >= 2 && NST <= 4 && (NST & (NST - 1)) == 0, "2 or 4 stages");
    __builtin_amdgcn_s_waitcnt(0);
    for (int q = 0; q < NST - 1 && q < nsteps; ++q)
        load(q, smem + q * C::STAGE, smem + q * C::STAGE + C::A_BYTES);
    for (int s = 0; s < nsteps; ++s) {
        const int pending = min(NST - 2, nsteps - 1 - s);  // stages issued after s
        if (pending >= 2)
            wait_vmcnt<2 * CPS>();
        else if (pending == 1)
            wait_vmcnt<CPS>();
        else
            wait_vmcnt<0>();
        wait_lds();
        wg_barrier();
        if (s + NST - 1 < nsteps) {
            char *b = smem + ((s + NST - 1) & (NST - 1)) * C::STAGE;
            load(s + NST - 1, b, b + C::A_BYTES);
        }
        const char *cur = smem + (s & (NST - 1)) * C::STAGE;
        mma_stage<C, true, A_TR, B_TR, PART>(cur, cur + C::A_BYTES, acc, wm, wn, ib);
    }
    wait_lds();
    __syncthreads();
}

template <class C, int NST, bool A_TR, bool B_TR, int CPS, class Load>
__device__ __forceinline__ void mainloop_ring(char *smem, int nsteps,
                                              f32x16_t (&acc)[C::FM][C::FN], Load load,
                                              int rows = C::BM)
{
    const int wave = threadIdx.x / kWave;
    const int wm = wave / C::WN, wn = wave % C::WN;
    if (nsteps <= 0)
        return;
    const int ib = __builtin_amdgcn_readfirstlane(
        min(C::FM, max(0, (rows - wm * C::TM + 31) / 32)));
    if (ib == C::FM)
        ring_body<C, NST, A_TR, B_TR, CPS, false>(smem, nsteps, acc, load, wm, wn, ib);
    else
        ring_body<C, NST, A_TR, B_TR, CPS, true>(smem, nsteps, acc, load, wm, wn, ib);
}

// A copy callback f(q, buf, n) without row-index prefetching.
template <class F>
struct PlainCopy {
    F f;
    __device__ __forceinline__ void operator()(int q, int buf, int n) { f(q, buf, n); }
    __device__ __forceinline__ void prepare(int) {}
    __device__ __forceinline__ void phase_a(int) {}
    __device__ __forceinline__ void phase_b_end(int) {}
};
template <class F>
__device__ __forceinline__ PlainCopy<F> plain_copy(F f)
{
    return PlainCopy<F>{f};
}

// A_TR / B_TR: operand layout (OpFrag).  rows: real rows of the tile (A
// side); waves of a ragged tail skip the MFMAs and A reads of their padding
// 32-row blocks but keep every barrier.  Leaves LDS free for the epilogue
// (all reads and copies complete).
template <class C, bool A_TR, bool B_TR, class Copy>
__device__ __forceinline__ void mainloop_quad(const char *smem, int nslots,
                                              f32x16_t (&acc)[C::FM][C::FN], Copy &&copy, int rows)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave / C::WN, wn = wave % C::WN;
    if (nslots <= 0)
        return;
    OpFrag<A_TR, C::BM> fa;
    OpFrag<B_TR, C::BN> fb;
    fa.init(wm * C::TM);
    fb.init(wn * C::TN);
    const int ib = __builtin_amdgcn_readfirstlane(
        min(C::FM, max(0, (rows - wm * C::TM + 31) / 32)));
    if (ib == C::FM)
        quad_body<C, false>(smem, nslots, acc, copy, ib, fa, fb);
    else
        quad_body<C, true>(smem, nslots, acc, copy, ib, fa, fb);
}

// A row-major slot tile (32 reduction rows of COLS elements), copied by the
// four waves: 1 KiB windows of RW = 64 / (COLS / 8) rows, NC per wave.  Lane
// l writes window row l / CPR at physical chunk l % CPR and fetches the
// logical chunk that tr_off maps there.  The HBM rows of the reduction
// indices are contiguous (red -> first_row + red) with pitch row_bytes.
template <int COLS, int NC>
struct SlotTileCopier {
    static constexpr int CPR = COLS / 8, RW = kWave / CPR;
    static_assert(4 * NC * RW == SK, "four waves cover the slot's rows");
    uint32_t off[NC];  // HBM byte offset of (row, chunk) at slot 0 (kOOB: column outside)
    int row[NC];       // slot row of this lane in window j
    uint32_t lds0;     // LDS address of the wave's first window in slot 0
    int64_t row_bytes;

    __device__ __forceinline__ void init(char *slot0_part, int first_row, int col0, int ncols,
                                         int64_t row_bytes_)
    {
        const int lane = threadIdx.x & (kWave - 1);
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
        row_bytes = row_bytes_;
        lds0 = __builtin_amdgcn_readfirstlane(lds_u32(slot0_part)) + wave * NC * kWave * 16;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int r = (wave * NC + j) * RW + lane / CPR;
            const int lc = (lane % CPR) ^ ((r & 3) << 2);
            const int col = col0 + lc * 8;
            row[j] = r;
            off[j] = col < ncols ? (uint32_t)((first_row + r) * row_bytes) + (uint32_t)col * 2
                                 : kOOB;
        }
    }
    // Copy j of reduction slot q into slot buffer `slot`; rows at or past
    // nred are zeros.
    template <int SLOT_BYTES>
    __device__ __forceinline__ void issue_one(const u32x4_t &r, int j, int slot, int q,
                                              int nred) const
    {
        const bool in = q * SK + row[j] < nred;
        copy16_to_lds(r, in ? off[j] : kOOB,
                      __builtin_amdgcn_readfirstlane((uint32_t)(q * SK * row_bytes)),
                      lds0 + (uint32_t)(slot * SLOT_BYTES + j * kWave * 16));
    }
};

// n / d for the divisor d described by FastDiv (exact for n < 2^31).
__device__ __forceinline__ int fast_div(uint32_t n, FastDiv d)
{
    return (int)((__umulhi(n, d.mul) + n) >> d.shift);
}

// Row and column of accumulator element r of 32x32 block (i, j) for this lane.
template <class C>
__device__ __forceinline__ int acc_row(int wm, int i, int r)
{
    const int lane = threadIdx.x & (kWave - 1);
    return wm * C::TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
template <class C>
__device__ __forceinline__ int acc_col(int wn, int j)
{
    return wn * C::TN + j * 32 + (threadIdx.x & 31);
}

// bf16 epilogue through LDS.  The tile is staged as bf16 in st0 (or, when
// it does not fit in one stage, rows [0, BM/2) in st0 and [BM/2, BM) in
// st1), then copied out as 16-byte row segments.
// s_dst[i]: destination row of tile row i (-1: skip); s_scale: per-row factor
// applied when SCALE is set.  Y is bf16 with leading dimension ldy; tile
// column c maps to output column n0 + c (valid below ncols).
//
// Staging layout: row-major, BN elements per row, with the 16-byte chunks of
// row r permuted as chunk ^ g(r % 4), g(k) = 2k ^ 4k (0, 6, 12, 10).  An MFMA
// lane holds 4 adjacent rows of one column; four adjacent lanes transpose
// their 4 x 4 values with two cross-lane swaps (quad_transpose_bf16) so that
// each writes 4 adjacent columns of one row as one 8-byte LDS write, a
// quarter of the writes of one element at a time.  The four rows of a quad
// are 512 bytes apart; g gives each of them a different 32-byte bank group
// within 128 bytes (bits 1-2 of g distinct) and a different 64-byte group
// within 256 bytes (bits 2-3 distinct).  With chunk ^ 4k alone, only the
// latter held and the SQ counters showed 4-30% of LDS cycles in conflicts.
__device__ __forceinline__ int quad_perm(int k)
{
    return (k << 1) ^ (k << 2);
}

template <class C>
struct EpiLayout {
    static constexpr bool SPLIT = C::BM * C::BN * 2 > C::STAGE;
    static constexpr int ROWS_PER_BUF = SPLIT ? C::BM / 2 : C::BM;
    static_assert(ROWS_PER_BUF * C::BN * 2 <= C::STAGE, "staged rows must fit in one stage");
    static_assert(ROWS_PER_BUF % C::TM == 0, "a wave's rows must stay in one staging buffer");
    static_assert(C::BN >= 128, "the chunk permutation needs 16 chunks per row");
    // Byte offset of 16-byte chunk ch of staged row r.
    __device__ __forceinline__ static int chunk_off(int r, int ch)
    {
        return r * C::BN * 2 + ((ch ^ quad_perm(r & 3)) << 4);
    }
};

// Lanes 4q .. 4q + 3 hold x[k][c] (rows k = 0..3 in v0..v3, column c = lane
// % 4).  Returns row lane % 4, columns 0..3, as packed bf16.  Swap 1 (lanes
// c, c ^ 2) exchanges 2 x 2 blocks of row pairs; swap 2 (lanes c, c ^ 1)
// exchanges single elements.  v_perm selects bytes of {S0, S1}, S1 low.
__device__ __forceinline__ uint2 quad_transpose_bf16(float v0, float v1, float v2, float v3)
{
    const int k = threadIdx.x & 3;
    const uint32_t d0 = pack_bf16x2(v0, v1), d1 = pack_bf16x2(v2, v3);
    // Lanes 0, 1 keep rows 0-1 and receive them for columns + 2; lanes 2, 3
    // keep rows 2-3 and receive them for columns - 2.
    const bool low = (k & 2) == 0;
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(low ? d1 : d0), 0x4e,
                                                              0xf, 0xf, false);
    const uint32_t e0 = low ? d0 : r1, e1 = low ? r1 : d1;
    // e0 = (x[a][c0], x[a+1][c0]), e1 = (x[a][c0+2], x[a+1][c0+2]) with c0 =
    // the even column of the lane pair; the even lane wants row a, the odd
    // lane row a + 1.
    const bool even = (k & 1) == 0;
    const uint32_t s2 = __builtin_amdgcn_perm(e1, e0, even ? 0x07060302u : 0x05040100u);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s2, 0xb1, 0xf, 0xf, false);
    return {__builtin_amdgcn_perm(r2, e0, even ? 0x05040100u : 0x03020504u),
            __builtin_amdgcn_perm(r2, e1, even ? 0x07060100u : 0x03020706u)};
}

// SCALE: multiply row i by s_scale[i].
template <class C, bool SCALE>
__device__ __forceinline__ void stage_bf16(char *st0, char *st1,
                                           const f32x16_t (&acc)[C::FM][C::FN],
                                           const float *s_scale)
{
    using L = EpiLayout<C>;
    const int wave = threadIdx.x / kWave;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int lane = threadIdx.x & (kWave - 1);
    const int k = lane & 3;
    // Accumulator row of v0 (register r % 4 == 0) for block row 0, group 0.
    const int row0 = wm * C::TM + 4 * (lane >> 5);
    char *buf = (wm * C::TM) / L::ROWS_PER_BUF ? st1 : st0;
    // After the transpose this lane writes staged row row0 % RPB + k + 32 i +
    // 8 g, columns wn * TN + 32 j + (lane & 28) + 0..3: the chunk part
    // depends on j and k only (row % 4 == k), the row part is a constant.
    char *rowp = buf + ((row0 % L::ROWS_PER_BUF) + k) * C::BN * 2;
    int coff[C::FN];
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
        const int ch = (wn * C::TN + j * 32) / 8 + ((lane >> 3) & 3);
        coff[j] = ((ch ^ quad_perm(k)) << 4) + (lane & 4) * 2;
    }
    const float *sc = s_scale + row0;
    // Straight-line code, one group of 4 rows at a time (sched_barrier):
    // otherwise the compiler moves every accumulator out of the AGPRs, and
    // loads every row factor, up front.
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int rr = i * 32 + 8 * g;  // row offset of v0 from row0
            float f[4] = {1.0f, 1.0f, 1.0f, 1.0f};
            if (SCALE) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    f[q] = sc[rr + q];
            }
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                const f32x16_t &a = acc[i][j];
                const uint2 w = quad_transpose_bf16(a[4 * g] * f[0], a[4 * g + 1] * f[1],
                                                    a[4 * g + 2] * f[2], a[4 * g + 3] * f[3]);
                *reinterpret_cast<uint2 *>(rowp + rr * C::BN * 2 + coff[j]) = w;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
}

// 16 bytes of a staged output row to HBM with the nontemporal (streaming)
// hint: no kernel here reads its own output again, so its lines need not
// stay in L2 next to the operands.  Measured: fine-grained step forward
// 0.296 -> 0.284 ms, dX 0.280 -> 0.272, dW 0.388 -> 0.378; in the decode
// slice with backward, the next step's forward 0.101 -> 0.058 ms (dW's
// 403 MB output no longer displaces the weights); Mixtral unchanged.
typedef unsigned u32x4_nt_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_out16(char *dst, const char *lds_src)
{
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4_nt_t *>(lds_src),
                                reinterpret_cast<u32x4_nt_t *>(dst));
}

// BATCH: a thread's chunks share one column (rows r0, r0 + RSTEP, ...), and
// its LDS reads are issued in groups of up to 8 before the group's stores,
// instead of one read and one store at a time.  Measured on dW: Mixtral
// 2.49 -> 2.46 ms, fine-grained 0.385 -> 0.378 ms, decode-shaped 0.107 ->
// 0.105 ms; on Mixtral dX 1.5% slower, so dW alone uses it.
template <class C, bool SCALE = false, bool BATCH = false>
__device__ __forceinline__ void epilogue_bf16(char *st0, char *st1,
                                              const f32x16_t (&acc)[C::FM][C::FN],
                                              const int *s_dst, const float *s_scale,
                                              char *Y, int64_t ldy, int n0, int ncols)
{
    using L = EpiLayout<C>;
    stage_bf16<C, SCALE>(st0, st1, acc, s_scale);
    __syncthreads();
    constexpr int CPR = C::BN / 8;  // 16-byte chunks per tile row
    if constexpr (BATCH) {
        constexpr int PER = C::BM * CPR / C::NT, RSTEP = C::NT / CPR, B = PER < 8 ? PER : 8;
        static_assert(C::NT % CPR == 0 && (C::BM * CPR) % C::NT == 0 && PER % B == 0,
                      "whole rows per pass");
        const int ch = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
        const int col = n0 + ch * 8;
#pragma unroll
        for (int i0 = 0; i0 < PER; i0 += B) {
            u32x4_nt_t v[B];
            int dst[B];
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const int row = r0 + (i0 + i) * RSTEP;
                const char *buf = row / L::ROWS_PER_BUF ? st1 : st0;
                v[i] = *reinterpret_cast<const u32x4_nt_t *>(
                    buf + L::chunk_off(row % L::ROWS_PER_BUF, ch));
                dst[i] = s_dst[row];
            }
#pragma unroll
            for (int i = 0; i < B; ++i)
                if (dst[i] >= 0 && col < ncols)
                    __builtin_nontemporal_store(v[i], reinterpret_cast<u32x4_nt_t *>(
                                                          Y + ((int64_t)dst[i] * ldy + col) * 2));
        }
    } else {
        for (int idx = threadIdx.x; idx < C::BM * CPR; idx += C::NT) {
            const int row = idx / CPR, ch = idx % CPR;
            const int dst = s_dst[row];
            const int col = n0 + ch * 8;
            const char *buf = row / L::ROWS_PER_BUF ? st1 : st0;
            if (dst >= 0 && col < ncols)
                store_out16(Y + ((int64_t)dst * ldy + col) * 2,
                            buf + L::chunk_off(row % L::ROWS_PER_BUF, ch));
        }
    }
    __syncthreads();
}

// fp32 epilogue straight from the accumulators (32 lanes = 128 contiguous bytes).
template <class C>
__device__ __forceinline__ void epilogue_f32(const f32x16_t (&acc)[C::FM][C::FN], const int *s_dst,
                                             float *Y, int64_t ldy, int n0, int ncols)
{
    const int wave = threadIdx.x / kWave;
    const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = acc_row<C>(wm, i, r);
                const int col = n0 + acc_col<C>(wn, j);
                const int dst = s_dst[row];
                if (dst >= 0 && col < ncols)
                    Y[(int64_t)dst * ldy + col] = acc[i][j][r];
            }
}

// Gated activation on the gate_up output (reduction_n = 2): output column c
// is silu(A[:, 2c]) * A[:, 2c + 1].  The W tile is loaded with its rows
// permuted (gated_row) so that a lane's accumulator block j < FN/2 holds the
// gate and block j + FN/2 the linear partner of the same output column in the
// same register: the activation needs no data exchange between lanes.
//
// Tile row r (wave column wn = r / TN, block j, lane l = r % 32) holds W row
// n0 + 2 * (wn * TN/2 + (j mod FN/2) * 32 + l) + (j >= FN/2): a bijection of
// [0, BN) onto itself, and output column n0/2 + wn * TN/2 + (j mod FN/2) * 32 + l.
template <class C>
__device__ __forceinline__ int gated_row(int r)
{
    static_assert(C::FN % 2 == 0, "the gated epilogue pairs accumulator blocks");
    constexpr int H = C::FN / 2;
    const int wn = r / C::TN, j = (r % C::TN) / 32, l = r % 32;
    return 2 * (wn * (C::TN / 2) + (j % H) * 32 + l) + j / H;
}

__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Stages the BM x BN/2 bf16 output tile in st0 and copies it out as 16-byte
// row segments to Y (leading dimension ldy, tile column c -> o0 + c, valid
// below ncols), like epilogue_bf16.
template <class C>
__device__ __forceinline__ void epilogue_gated(char *st0, const f32x16_t (&acc)[C::FM][C::FN],
                                               const int *s_dst, char *Y, int64_t ldy, int o0,
                                               int ncols)
{
    constexpr int OC = C::BN / 2, H = C::FN / 2;
    static_assert(C::BM * OC * 2 <= C::STAGE, "the gated tile fits in one stage");
    const int wave = threadIdx.x / kWave;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int lane = threadIdx.x & (kWave - 1);
    const int row0 = wm * C::TM + 4 * (lane >> 5);
    uint16_t *base = reinterpret_cast<uint16_t *>(st0) + row0 * OC + wn * (C::TN / 2) + (lane & 31);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rr = i * 32 + 8 * (r >> 2) + (r & 3);
#pragma unroll
            for (int j = 0; j < H; ++j)
                base[rr * OC + j * 32] = to_bf16(silu_mul(acc[i][j][r], acc[i][j + H][r]));
            __builtin_amdgcn_sched_barrier(0);
        }
    __syncthreads();
    constexpr int CPR = OC / 8;
    for (int idx = threadIdx.x; idx < C::BM * CPR; idx += C::NT) {
        const int row = idx / CPR, ch = idx % CPR;
        const int dst = s_dst[row];
        const int col = o0 + ch * 8;
        if (dst >= 0 && col < ncols)
            store_out16(Y + ((int64_t)dst * ldy + col) * 2, st0 + (row * OC + ch * 8) * 2);
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Expert tables shared by the routed kernels
// ---------------------------------------------------------------------------

__device__ __forceinline__ int checked_gather(const int32_t *gather, int64_t p, int64_t S,
                                              int32_t *err)
{
    const int g = gather[p];
    if (g < 0 || g >= S) {
        raise_error(err, kErrGather);
        return -1;
    }
    return g;
}

// ---------------------------------------------------------------------------
// Tail split of the last round (dX; see TailReduceParams in gemm_params.h).
// Measured on the Mixtral shape in one process: dX 2.03 -> 1.90 ms.  The same
// split of the forward (K reduction, the gate factor and scatter applied after
// the sum) measured slower (1.75 -> 1.81 ms) and is not used.
// ---------------------------------------------------------------------------

struct TailPlan {
    int full;   // work items 0 .. full-1 are whole tiles
    int R, P;   // tail tiles after them, parts per tail tile (R = 0: none)
    int items;  // full + R * P
};

// The same plan in every workgroup (total and G are uniform).  Splitting pays
// when at least two workgroups share each tail tile.
__device__ __forceinline__ TailPlan tail_plan(int total, int G, bool enabled)
{
    TailPlan tp{total, 0, 1, total};
    if (enabled && G <= kTailMaxTiles) {
        const int R = total % G;
        if (R > 0 && G / R >= 2) {
            tp.full = total - R;
            tp.R = R;
            tp.P = G / R;
            tp.items = tp.full + R * tp.P;
        }
    }
    return tp;
}

// Work item w -> tile and part (part -1: a whole tile).
__device__ __forceinline__ void tail_item(const TailPlan &tp, int w, int &t, int &part)
{
    if (w < tp.full) {
        t = w;
        part = -1;
    } else {
        t = tp.full + (w - tp.full) / tp.P;
        part = (w - tp.full) % tp.P;
    }
}

// Sums each tail tile's parts in part order and stores it (bf16, 8 bytes per
// lane), after the GEMM launch on the same stream.
template <int BM, int BN>
__global__ __launch_bounds__(256) void tail_reduce_kernel(TailReduceParams a)
{
    const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws);
    const float4 *partials = reinterpret_cast<const float4 *>(a.ws + tail_header_bytes());
    const int R = hdr[0], P = hdr[1];
    constexpr int Q = BN / 4;  // float4 per tile row
    // All tiles' items at once (one tile at a time left most threads idle
    // and made the launch a chain of R memory round trips).  A block's 256
    // consecutive items lie in one tile, so the tile's header is uniform.
    constexpr int PER = BM * Q;  // items per tile
    static_assert(PER % 256 == 0, "a block's items stay in one tile");
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < (int64_t)R * PER;
         w += (int64_t)gridDim.x * blockDim.x) {
        const int r = __builtin_amdgcn_readfirstlane((int)(w / PER));
        const int p0 = hdr[2 + 4 * r], rows = hdr[3 + 4 * r], c0 = hdr[4 + 4 * r];
        {
            const int idx = (int)(w % PER);
            const int i = idx / Q, j = idx % Q;
            const int col = c0 + 4 * j;
            if (i >= rows || col >= a.ncols)
                continue;
            const int64_t p = p0 + i;
            int64_t dst = p;
            if (a.scatter_out) {
                const int g = a.gather[p];
                if (g < 0 || g >= a.S)
                    continue;  // reported by the GEMM launch
                dst = g;
            }
            const float4 *src = partials + (int64_t)r * P * BM * Q + i * Q + j;
            float4 s = src[0];
            for (int q = 1; q < P; ++q) {
                const float4 v = src[(int64_t)q * BM * Q];
                s.x += v.x;
                s.y += v.y;
                s.z += v.z;
                s.w += v.w;
            }
            uint2 b;
            b.x = pack_bf16x2(s.x, s.y);
            b.y = pack_bf16x2(s.z, s.w);
            *reinterpret_cast<uint2 *>(a.out + (dst * a.ldo + col) * 2) = b;
        }
    }
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------

// Raster of an expert's output tiles: tile u of mt row tiles x nt column
// tiles.  The row tiles are taken in bands of up to BAND; within a band the
// row tiles of one column tile are consecutive.  With BAND = 8 an XCD's 32
// concurrent tiles cover at most 8 row tiles and 4 or more column tiles: on
// a dense 8192 x 28672 x 4096 product, 32 row tiles of one column tile made
// each stage fetch 33 distinct slices into the XCD's L2 instead of 12 (4 and
// 16 measured no better there, 16 11% slower).  Experts of up to BAND row
// tiles keep the plain column-major order.
constexpr int kBandM = 8;    // forward
constexpr int kBandMdX = 4;  // dX: Mixtral-shaped dX 1.84 -> 1.77 ms against 8

template <int BAND>
__device__ __forceinline__ void band_raster(int u, int mt, int nt, int &m, int &n)
{
    const int band = u / (BAND * nt);
    const int first = band * BAND;
    const int gm = min(mt - first, BAND);
    const int r = u - band * BAND * nt;
    m = first + r % gm;
    n = r / gm;
}

// GATED: W rows come in (gate, linear) pairs and Y gets N/2 columns of the
// gated activation (epilogue_gated).
template <class C, bool GATED>
__global__ __launch_bounds__(C::NT) void fwd_kernel(FwdParams a)
{
    __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
    char *const st0 = smem, *const st1 = smem + C::STAGE;
    __shared__ int s_roff[kMaxExperts + 1];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_src[C::BM];
    __shared__ int s_dst[C::BM];
    __shared__ float s_scale[C::BM];
    __shared__ int s_scratch[2];

    const bool px = a.flags & MOEGG_PERMUTE_X, py = a.flags & MOEGG_PERMUTE_Y;
    const bool fm = a.flags & MOEGG_FUSE_MUL_POST;
    const int ntn = (a.N + C::BN - 1) / C::BN;
    const int total = build_expert_tables(a.m_sizes, a.E, a.S, s_roff, s_tstart, s_scratch, a.err,
                                          [&](int m) { return (m + C::BM - 1) / C::BM * ntn; });
    const int nsteps = (a.K + BK - 1) / BK;
    const int64_t row_bytes = (int64_t)a.K * 2;
    const int64_t x_rows = px ? a.S / a.topk : a.S;
    const u32x4_t xr = rsrc_words(a.X, x_rows * row_bytes);

    // Tile t: expert, first sorted position, real rows, first column.
    auto tile = [&](int t, int &e, int &p0, int &rows, int &n0) {
        e = __builtin_amdgcn_readfirstlane(upper_index(s_tstart, a.E, t));
        const int mc = __builtin_amdgcn_readfirstlane(s_roff[e + 1] - s_roff[e]);
        const int mtiles = (mc + C::BM - 1) / C::BM;
        const int u = t - __builtin_amdgcn_readfirstlane(s_tstart[e]);
        int mt, nt;
        band_raster<kBandM>(u, mtiles, ntn, mt, nt);
        p0 = __builtin_amdgcn_readfirstlane(s_roff[e]) + mt * C::BM;
        rows = min(C::BM, mc - mt * C::BM);
        n0 = nt * C::BN;
    };
    // Gather entry of tile row threadIdx.x (one row per thread; -2: none).
    // The next tile's entry is loaded before this tile's mainloop, so its
    // latency is hidden; only the gate factor, which depends on it, is read
    // when the tile starts.
    static_assert(C::BM <= C::NT, "one tile row per thread");
    auto fetch = [&](int p0, int rows) -> int {
        const int i = threadIdx.x;
        if (i >= C::BM || i >= rows)
            return -2;
        return (px || py) ? a.gather[p0 + i] : p0 + i;
    };

    int t = xcd_logical_block(blockIdx.x, gridDim.x);
    int e = 0, p0 = 0, rows = 0, n0 = 0, g = -2;
    if (t < total) {
        tile(t, e, p0, rows, n0);
        g = fetch(p0, rows);
    }
    for (; t < total; t += gridDim.x) {
        if (threadIdx.x < C::BM) {
            const int i = threadIdx.x;
            int src = -1, dst = -1;
            float scale = 1.0f;
            if (g != -2) {
                const int64_t p = p0 + i;
                if ((px || py) && (g < 0 || g >= a.S)) {
                    raise_error(a.err, kErrGather);
                } else {
                    src = px ? g / a.topk : (int)p;
                    dst = py ? g : (int)p;
                    if (fm)
                        scale = a.topk_w[g];
                }
            }
            s_src[i] = src;
            s_dst[i] = dst;
            s_scale[i] = scale;
        }
        __syncthreads();
        // The next tile's gather entries, in flight during this mainloop.
        const int tn = t + gridDim.x;
        int e_n = 0, p0_n = 0, rows_n = 0, n0_n = 0, g_n = -2;
        if (tn < total) {
            tile(tn, e_n, p0_n, rows_n, n0_n);
            g_n = fetch(p0_n, rows_n);
        }

        const u32x4_t wr =
            rsrc_words(a.W + (int64_t)e * a.N * row_bytes, (int64_t)a.N * row_bytes);
        f32x16_t acc[C::FM][C::FN];
        zero_acc<C>(acc);
        DmaLoader<C::BM, C::NT> la;
        DmaLoader<C::BN, C::NT> lb;
#pragma unroll
        for (int i = 0; i < la.RPT; ++i)
            la.set_row(i, s_src[la.tile_row(i)], row_bytes);
#pragma unroll
        for (int i = 0; i < lb.RPT; ++i) {
            const int r = lb.tile_row(i);
            int wrow = n0 + r;
            if constexpr (GATED)
                wrow = n0 + gated_row<C>(r);
            lb.set_row(i, wrow < a.N ? wrow : -1, row_bytes);
        }
        mainloop<C, true, false, false>(
            st0, st1, nsteps, acc,
            [&](int s, char *As, char *Bs) {
                la.load(xr, As, s * BK, a.K);
                lb.load(wr, Bs, s * BK, a.K);
            },
            rows);
        if constexpr (GATED)
            epilogue_gated<C>(st0, acc, s_dst, a.Y, a.N / 2, n0 / 2, a.N / 2);
        else
            epilogue_bf16<C, true>(st0, st1, acc, s_dst, s_scale, a.Y, a.N, n0, a.N);
        e = e_n;
        p0 = p0_n;
        rows = rows_n;
        n0 = n0_n;
        g = g_n;
    }
}

// ---------------------------------------------------------------------------
// dX = dY_e W_e  (reduction over N)
// ---------------------------------------------------------------------------

template <class C>
__global__ __launch_bounds__(C::NT) void dx_kernel(DxParams a)
{
    __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
    char *const st0 = smem, *const st1 = smem + C::STAGE;
    __shared__ int s_roff[kMaxExperts + 1];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_src[C::BM];
    __shared__ int s_dst[C::BM];
    __shared__ int s_scratch[2];

    const bool px = a.flags & MOEGG_PERMUTE_X, py = a.flags & MOEGG_PERMUTE_Y;
    const int ntk = (a.K + C::BN - 1) / C::BN;
    const int total = build_expert_tables(a.m_sizes, a.E, a.S, s_roff, s_tstart, s_scratch, a.err,
                                          [&](int m) { return (m + C::BM - 1) / C::BM * ntk; });
    const int nsteps = (a.N + BK - 1) / BK;
    const int64_t dy_row = (int64_t)a.N * 2, w_row = (int64_t)a.K * 2;
    const u32x4_t dyr = rsrc_words(a.dY, a.S * dy_row);
    const TailPlan tp = tail_plan(total, gridDim.x, a.ws != nullptr);
    int32_t *const hdr = reinterpret_cast<int32_t *>(a.ws);
    if (a.ws && blockIdx.x == 0 && threadIdx.x == 0) {
        hdr[0] = tp.R;
        hdr[1] = tp.P;
    }

    for (int w = xcd_logical_block(blockIdx.x, gridDim.x); w < tp.items; w += gridDim.x) {
        int t, part;
        tail_item(tp, w, t, part);
        const int e = __builtin_amdgcn_readfirstlane(upper_index(s_tstart, a.E, t));
        const int mc = __builtin_amdgcn_readfirstlane(s_roff[e + 1] - s_roff[e]);
        const int p0base = __builtin_amdgcn_readfirstlane(s_roff[e]);
        const int mtiles = (mc + C::BM - 1) / C::BM;
        const int u = t - __builtin_amdgcn_readfirstlane(s_tstart[e]);
        int mt, kt;
        band_raster<kBandMdX>(u, mtiles, ntk, mt, kt);
        const int p0 = p0base + mt * C::BM;
        const int rows = min(C::BM, mc - mt * C::BM);
        const int k0 = kt * C::BN;
        // A tail part reduces its share of the N range into a partial whose
        // row i is tile row i (the finishing launch maps rows to dX).
        const bool tail = part >= 0;
        const int r = t - tp.full;
        if (tail && part == 0 && threadIdx.x == 0) {
            hdr[2 + 4 * r] = p0;
            hdr[3 + 4 * r] = rows;
            hdr[4 + 4 * r] = k0;
            hdr[5 + 4 * r] = e;
        }

        for (int i = threadIdx.x; i < C::BM; i += C::NT) {
            int src = -1, dst = -1;
            if (i < rows) {
                const int64_t p = p0 + i;
                const int g = (px || py) ? checked_gather(a.gather, p, a.S, a.err) : (int)p;
                if (g >= 0) {
                    src = py ? g : (int)p;
                    dst = px ? g : (int)p;
                }
            }
            s_src[i] = src;
            s_dst[i] = tail ? i : dst;
        }
        __syncthreads();
        float *const partial =
            tail ? reinterpret_cast<float *>(a.ws + tail_header_bytes()) +
                       (int64_t)(r * tp.P + part) * C::BM * C::BN
                 : nullptr;

        const u32x4_t wr =
            rsrc_words(a.W + (int64_t)e * a.N * w_row, (int64_t)a.N * w_row);
        f32x16_t acc[C::FM][C::FN];
        if constexpr (UseQuad<C>::value) {
            // Wave w copies dY rows [64 w, 64 w + 64) (A, reduction-contiguous)
            // and W rows 8 w .. 8 w + 7 of each slot (B, row-major).
            using Q = Quad<C>;
            const int first = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave) * 64;
            SlotCopier<Q::NCA> ca;
            SlotTileCopier<C::BN, Q::NCB> cb;
            ca.init(smem, first);
#pragma unroll
            for (int j = 0; j < Q::NCA; ++j)
                ca.set_row(j, s_src[ca.row(first, j)], dy_row);
            cb.init(smem + Q::A, 0, k0, a.K, w_row);
            const int N = a.N;
            const int U = (N + SK - 1) / SK;
            const int u0 = tail ? part * U / tp.P : 0, u1 = tail ? (part + 1) * U / tp.P : U;
            zero_acc<C>(acc);
            mainloop_quad<C, false, true>(
                smem, u1 - u0, acc,
                plain_copy([&](int q, int buf, int n) {
                    const int qq = q + u0;
                    if (n < Q::NCA)
                        ca.template issue_one<Q::SLOT>(dyr, n, buf, qq * SK, N);
                    else
                        cb.template issue_one<Q::SLOT>(wr, n - Q::NCA, buf, qq, N);
                }),
                rows);
            if (tail) {
                epilogue_f32<C>(acc, s_dst, partial, C::BN, 0, C::BN);
                __syncthreads();
            } else {
                epilogue_bf16<C>(st0, st1, acc, s_dst, nullptr, a.dX, a.K, k0, a.K);
            }
            continue;
        }
        DmaLoader<C::BM, C::NT> la;
#pragma unroll
        for (int i = 0; i < la.RPT; ++i)
            la.set_row(i, s_src[la.tile_row(i)], dy_row);
        const int N = a.N;
        const int u0 = tail ? part * nsteps / tp.P : 0;
        const int u1 = tail ? (part + 1) * nsteps / tp.P : nsteps;
        zero_acc<C>(acc);
        TileDmaLoader<C::BN, C::NT> lb;
        auto wraw = [](int n) -> int { return n; };
        auto wfin = [=](int n, int) -> int { return n < N ? n : -1; };
        lb.fetch(u0 * BK, wraw);
        mainloop<C, true, false, true>(
            st0, st1, u1 - u0, acc,
            [&](int s, char *As, char *Bs) {
                lb.prepare(k0, a.K, w_row, wfin);
                __builtin_amdgcn_sched_barrier(0);
                la.load(dyr, As, (s + u0) * BK, a.N);
                lb.issue(wr, Bs);
                lb.fetch((s + u0 + 1) * BK, wraw);
            },
            rows);
        if (tail) {
            epilogue_f32<C>(acc, s_dst, partial, C::BN, 0, C::BN);
            __syncthreads();
        } else {
            epilogue_bf16<C>(st0, st1, acc, s_dst, nullptr, a.dX, a.K, k0, a.K);
        }
    }
}

// ---------------------------------------------------------------------------
// dW_e = dY_e^T X_e  (reduction over the expert's own rows)
// ---------------------------------------------------------------------------

constexpr int kGroupK = 8;

// The copies of a 64-row stage take longer to land than the MFMAs of the
// previous stage run: with the MFMAs removed, the two-stage loop still takes
// 1.5 us per stage on the Mixtral shape, against 0.95 us per stage with the
// copies removed.  dW therefore splits the same 128 KiB of LDS into four
// 32-row slots and issues each slot's copies three slots ahead.  Gather
// entries are staged in LDS for a segment of up to kDwGather rows at a time,
// so that the only vector-memory operations in the loop are the copies and
// each wait can count them.  Measured: fine-grained dW 0.404 -> 0.368 ms,
// decode-shaped dW 0.113 -> 0.105 ms; the Mixtral shape is unchanged (its
// copies are bound by their rate, not by how far ahead they are issued).
constexpr int kDwSlot = 32;      // reduction rows per slot
constexpr int kDwSlots = 4;
constexpr int kDwGather = 1024;  // gather entries staged per segment

// MFMAs of one 32-row slot (both operands reduction rows in LDS).
template <class C>
__device__ __forceinline__ void dw_slot_mma(const char *As, const char *Bs,
                                            f32x16_t (&acc)[C::FM][C::FN], int wm, int wn)
{
    bf16x8_t a0[C::FM], b0[C::FN], a1[C::FM], b1[C::FN];
    read_step<C, true, true>(As, Bs, 0, wm, wn, a0, b0);
    read_step<C, true, true>(As, Bs, 1, wm, wn, a1, b1);
    mma_step<C>(a0, b0, acc);
    mma_step<C>(a1, b1, acc);
}


// PX / PY: the forward's permute flags, as template parameters so that the
// per-stage row-index code has no flag branches.
template <class C, bool PX, bool PY>
__global__ __launch_bounds__(C::NT) void dw_kernel(DwParams a)
{
    __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
    char *const st0 = smem, *const st1 = smem + C::STAGE;
    __shared__ int s_roff[kMaxExperts + 1];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_order[kMaxExperts];
    __shared__ int s_crows[kMaxExperts];       // rows per chunk, by sorted position
    __shared__ int s_istart[kMaxExperts + 1];  // first work item, by sorted position
    __shared__ int s_poff[kMaxExperts + 1];    // first partial (split experts), by position
    __shared__ int s_dst[C::BM];
    __shared__ int s_scratch[4];

    const bool f32out = a.flags & MOEGG_DW_FP32_OUT;
    const int ntn = (a.N + C::BM - 1) / C::BM, ntk = (a.K + C::BN - 1) / C::BN;
    const int per_expert = ntn * ntk;
    build_expert_tables(a.m_sizes, a.E, a.S, s_roff, s_tstart, s_scratch, a.err,
                        [&](int) { return 0; });
    // Chunks: an expert longer than split_rows is cut into c chunks of cr
    // rows (a multiple of BK, the last one shorter); otherwise one chunk of
    // all its rows.  Work items (chunk x output tile) are ordered by chunk
    // length, longest first, so the long reductions start early.
    auto chunking = [&](int m, int &c, int &cr) {
        c = 1;
        cr = m;
        if (a.split_rows > 0 && m > a.split_rows) {
            c = (m + a.split_rows - 1) / a.split_rows;
            cr = ((m + c - 1) / c + BK - 1) / BK * BK;
            c = (m + cr - 1) / cr;
        }
    };
    int *const s_cnt = s_tstart;  // chunks by sorted position (s_tstart is free here)
    for (int e = threadIdx.x; e < a.E; e += C::NT) {
        int c, cr;
        chunking(s_roff[e + 1] - s_roff[e], c, cr);
        int rank = 0;
        for (int f = 0; f < a.E; ++f) {
            int cf, crf;
            chunking(s_roff[f + 1] - s_roff[f], cf, crf);
            rank += (crf > cr) || (crf == cr && f < e);
        }
        s_order[rank] = e;
        s_crows[rank] = cr;
        s_cnt[rank] = c;
        s_istart[rank] = c * per_expert;
        s_poff[rank] = c > 1 ? c : 0;
    }
    wave0_exclusive_scan(s_istart, a.E, &s_scratch[2]);
    wave0_exclusive_scan(s_poff, a.E, &s_scratch[3]);
    const int total = s_scratch[2];
    float *const partials =
        a.ws ? reinterpret_cast<float *>(a.ws + dw_header_bytes(a.E)) : nullptr;
    if (blockIdx.x == 0 && a.split_rows > 0 && a.ws) {
        // The plan for dw_reduce: split experts in sorted order.
        int32_t *hdr = reinterpret_cast<int32_t *>(a.ws);
        if (threadIdx.x < kWave) {
            int base = 0;
            for (int p0 = 0; p0 < a.E; p0 += kWave) {
                const int pos = p0 + threadIdx.x;
                const int cnt = pos < a.E ? s_cnt[pos] : 0;
                const bool split = cnt > 1;
                const uint64_t mask = __ballot(split);
                const int j = base + __popcll(mask & ((1ull << threadIdx.x) - 1));
                if (split) {
                    hdr[1 + 3 * j] = s_order[pos];
                    hdr[2 + 3 * j] = cnt;
                    hdr[3 + 3 * j] = s_poff[pos];
                }
                base += __popcll(mask);
            }
            if (threadIdx.x == 0)
                hdr[0] = base;
        }
    }
    const int64_t dy_row = (int64_t)a.N * 2, x_row = (int64_t)a.K * 2;
    const int64_t x_rows = PX ? a.S / a.topk : a.S;
    const u32x4_t dyr = rsrc_words(a.dY, a.S * dy_row);
    const u32x4_t xr = rsrc_words(a.X, x_rows * x_row);

    for (int t = xcd_logical_block(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
        const int pos = __builtin_amdgcn_readfirstlane(upper_index(s_istart, a.E, t));
        const int e = __builtin_amdgcn_readfirstlane(s_order[pos]);
        const int item = t - __builtin_amdgcn_readfirstlane(s_istart[pos]);
        const int chunk = item / per_expert;
        const int cr = __builtin_amdgcn_readfirstlane(s_crows[pos]);
        const int m_e = __builtin_amdgcn_readfirstlane(s_roff[e + 1] - s_roff[e]);
        const bool split = cr < m_e;  // chunked expert: fp32 partial into the workspace
        // Grouped raster inside the expert: runs of up to kGroupK K-panels per
        // N column, so consecutive tiles (one XCD's concurrent set) share
        // few dY (N) and X (K) panels in that XCD's L2.
        const int u = item % per_expert;
        const int span = kGroupK * ntn;
        const int first_kt = (u / span) * kGroupK;
        const int gk = min(ntk - first_kt, kGroupK);
        const int kt = first_kt + (u % span) % gk, nt = (u % span) / gk;
        const int n0 = nt * C::BM, k0 = kt * C::BN;
        const int start = __builtin_amdgcn_readfirstlane(s_roff[e]) + chunk * cr;
        const int mc = max(0, min(cr, m_e - chunk * cr));

        if (m_e == 0) {
            // An expert without rows: its tile of dW is zeros, stored as 16-byte
            // row segments straight from registers (no copies, MFMAs or LDS
            // staging; every thread of the workgroup takes this branch).
            const int esz = f32out ? 4 : 2;
            const int cpr = min(C::BN, a.K - k0) * esz / 16;  // K is a multiple of 8
            const int nrows = min(C::BM, a.N - n0);
            char *const base = a.dW + (((int64_t)e * a.N + n0) * a.K + k0) * esz;
            const u32x4_nt_t z = {0u, 0u, 0u, 0u};
            for (int idx = threadIdx.x; idx < nrows * cpr; idx += C::NT) {
                const int r = idx / cpr, c = idx % cpr;
                __builtin_nontemporal_store(
                    z, reinterpret_cast<u32x4_nt_t *>(base + (int64_t)r * a.K * esz + c * 16));
            }
            continue;
        }

        __syncthreads();
        for (int i = threadIdx.x; i < C::BM; i += C::NT)
            s_dst[i] = (n0 + i < a.N) ? (split ? 0 : e * a.N) + n0 + i : -1;
        __syncthreads();

        const int64_t S = a.S;
        const int32_t *gather = a.gather;
        int32_t *err = a.err;
        f32x16_t acc[C::FM][C::FN];
        zero_acc<C>(acc);
        {
            static_assert(kDwSlots * 2 * C::BM * kDwSlot * 2 <= 2 * C::STAGE &&
                              C::BM == C::BN && kMaxExperts + 1 >= kDwGather,
                          "four slots in the two stages; gather entries in s_tstart");
            constexpr int SLOT_A = C::BM * kDwSlot * 2, SLOT = 2 * SLOT_A;
            int *const s_g = s_tstart;  // free once the plan is built
            const FastDiv tdiv = a.topk_div;
            const uint32_t Su = (uint32_t)S;
            const int wave = threadIdx.x / kWave;
            const int wm = wave / C::WN, wn = wave % C::WN;
            bool bad = false;
            TileDmaLoader<C::BM, C::NT, kDwSlot> la;
            TileDmaLoader<C::BN, C::NT, kDwSlot> lb;
            constexpr int NC = TileDmaLoader<C::BM, C::NT, kDwSlot>::RPT +
                               TileDmaLoader<C::BN, C::NT, kDwSlot>::RPT;  // copies per wave per slot
            for (int seg0 = 0; seg0 < mc; seg0 += kDwGather) {
                const int segn = min(kDwGather, mc - seg0);
                const int ns = (segn + kDwSlot - 1) / kDwSlot;
                if constexpr (PX || PY) {
                    for (int i = threadIdx.x; i < segn; i += C::NT)
                        s_g[i] = gather[start + seg0 + i];
                    __syncthreads();
                } else {
                    wait_vmem();  // earlier stores: the waits below count copies only
                }
                // HBM rows of segment row r (-1: zeros).  A gather entry
                // outside [0, S) gives zeros and is reported once per tile.
                auto dyrow = [&](int r) -> int {
                    const bool in = r < segn;
                    if constexpr (PY) {
                        const int g = s_g[min(r, segn - 1)];
                        const bool ok = (uint32_t)g < Su;
                        bad |= in && !ok;
                        return in && ok ? g : -1;
                    }
                    return in ? start + seg0 + r : -1;
                };
                auto xrow = [&](int r) -> int {
                    const bool in = r < segn;
                    if constexpr (PX) {
                        const int g = s_g[min(r, segn - 1)];
                        const bool ok = (uint32_t)g < Su;
                        bad |= in && !ok;
                        return in && ok ? fast_div((uint32_t)g, tdiv) : -1;
                    }
                    return in ? start + seg0 + r : -1;
                };
                auto issue = [&](int q) {
                    char *sl = smem + (q % kDwSlots) * SLOT;
                    la.prepare_rows(n0, a.N, dy_row, [&](int row) { return dyrow(q * kDwSlot + row); });
                    lb.prepare_rows(k0, a.K, x_row, [&](int row) { return xrow(q * kDwSlot + row); });
                    __builtin_amdgcn_sched_barrier(0);
                    la.issue(dyr, sl);
                    lb.issue(xr, sl + SLOT_A);
                };
                for (int q = 0; q < min(ns, kDwSlots - 1); ++q)
                    issue(q);
                for (int q = 0; q < ns; ++q) {
                    // Slot q's copies are complete once at most the copies of
                    // the (up to two) slots issued after it are in flight.
                    const int after = min(kDwSlots - 2, ns - 1 - q);
                    if (after >= 2)
                        wait_vmcnt<2 * NC>();
                    else if (after == 1)
                        wait_vmcnt<NC>();
                    else
                        wait_vmcnt<0>();
                    wait_lds();
                    wg_barrier();
                    // Every wave is past slot q - 1, whose buffer slot q + 3 reuses.
                    if (q + kDwSlots - 1 < ns)
                        issue(q + kDwSlots - 1);
                    const char *sl = smem + (q % kDwSlots) * SLOT;
                    dw_slot_mma<C>(sl, sl + SLOT_A, acc, wm, wn);
                }
                __syncthreads();  // slots and s_g free for the next segment or the epilogue
            }
            if (bad)
                raise_error(err, kErrGather);
        }
        if (split) {
            const int poff = __builtin_amdgcn_readfirstlane(s_poff[pos]);
            epilogue_f32<C>(acc, s_dst, partials + (int64_t)(poff + chunk) * a.N * a.K, a.K, k0,
                            a.K);
        } else if (f32out) {
            epilogue_f32<C>(acc, s_dst, reinterpret_cast<float *>(a.dW), a.K, k0, a.K);
        } else {
            epilogue_bf16<C, false, true>(st0, st1, acc, s_dst, nullptr, a.dW, a.K, k0, a.K);
        }
    }
}

// Sums the chunk partials of the split experts in chunk order (fp32) into
// dW (bf16 or fp32), 16 bytes per lane and two positions per iteration (so
// that 2 c loads are in flight before the first add).  The plan comes from
// the workspace header written by dw_kernel's workgroup 0 earlier on the
// stream.
__device__ __forceinline__ void dw_reduce_store(const DwParams &a, int64_t o, const float4 &v)
{
    if (a.flags & MOEGG_DW_FP32_OUT) {
        reinterpret_cast<float4 *>(a.dW)[o] = v;
    } else {
        uint2 b;
        b.x = pack_bf16x2(v.x, v.y);
        b.y = pack_bf16x2(v.z, v.w);
        reinterpret_cast<uint2 *>(a.dW)[o] = b;
    }
}

__global__ __launch_bounds__(256) void dw_reduce_kernel(DwParams a)
{
    const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws);
    const float4 *partials = reinterpret_cast<const float4 *>(a.ws + dw_header_bytes(a.E));
    const int nsplit = hdr[0];
    const int64_t nk4 = (int64_t)a.N * a.K / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int j = 0; j < nsplit; ++j) {
        const int e = hdr[1 + 3 * j], c = hdr[2 + 3 * j], p0 = hdr[3 + 3 * j];
        const float4 *src = partials + (int64_t)p0 * nk4;
        for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nk4; w += 2 * stride) {
            const bool two = w + stride < nk4;
            float4 s0 = src[w];
            float4 s1 = two ? src[w + stride] : float4{};
            for (int q = 1; q < c; ++q) {
                const float4 v0 = src[q * nk4 + w];
                const float4 v1 = two ? src[q * nk4 + w + stride] : float4{};
                s0.x += v0.x; s0.y += v0.y; s0.z += v0.z; s0.w += v0.w;
                s1.x += v1.x; s1.y += v1.y; s1.z += v1.z; s1.w += v1.w;
            }
            dw_reduce_store(a, (int64_t)e * nk4 + w, s0);
            if (two)
                dw_reduce_store(a, (int64_t)e * nk4 + w + stride, s1);
        }
    }
}

// ---------------------------------------------------------------------------
// Explicit groups: y_g = x_g @ w_g
// ---------------------------------------------------------------------------

// The groups are few short products (the dual-expert layer: one tile per CU,
// 16 stages over K = 1024): a tile's copies of one stage cannot hide their
// own latency behind one stage of MFMAs, so the groups run a four-stage ring.
constexpr int kGroupStages = 4;

template <class C, bool TRANS_B>
__global__ __launch_bounds__(C::NT) void groups_kernel(GroupsParams a)
{
    constexpr int NST = kGroupStages;
    __shared__ __attribute__((aligned(16))) char smem[NST * C::STAGE];
    char *const st0 = smem, *const st1 = smem + C::STAGE;
    __shared__ int s_tstart[MOEGG_MAX_GROUPS + 1];
    __shared__ int s_dst[C::BM];

    if (threadIdx.x == 0) {
        int run = 0;
        for (int i = 0; i < a.num; ++i) {
            s_tstart[i] = run;
            run += ((a.g[i].m + C::BM - 1) / C::BM) * ((a.g[i].n + C::BN - 1) / C::BN);
        }
        s_tstart[a.num] = run;
    }
    __syncthreads();
    const int total = s_tstart[a.num];

    for (int t = xcd_logical_block(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
        const int gi = __builtin_amdgcn_readfirstlane(upper_index(s_tstart, a.num, t));
        const moegg_group &g = a.g[gi];
        const int mtiles = (g.m + C::BM - 1) / C::BM;
        const int u = t - __builtin_amdgcn_readfirstlane(s_tstart[gi]);
        const int mt = u % mtiles, nt = u / mtiles;
        const int m0 = mt * C::BM, n0 = nt * C::BN;

        __syncthreads();
        for (int i = threadIdx.x; i < C::BM; i += C::NT)
            s_dst[i] = (m0 + i < g.m) ? m0 + i : -1;
        __syncthreads();

        const int64_t x_row = (int64_t)g.ldx * 2, w_row = (int64_t)g.ldw * 2;
        const u32x4_t xr = rsrc_words(g.x, (int64_t)g.m * x_row);
        const u32x4_t wr = rsrc_words(g.w, (int64_t)(TRANS_B ? g.n : g.k) * w_row);
        DmaLoader<C::BM, C::NT> la;
#pragma unroll
        for (int i = 0; i < la.RPT; ++i) {
            const int r = la.tile_row(i);
            la.set_row(i, m0 + r < g.m ? m0 + r : -1, x_row);
        }
        f32x16_t acc[C::FM][C::FN];
        zero_acc<C>(acc);
        const int nsteps = (g.k + BK - 1) / BK;
        const int kk = g.k;
        if constexpr (TRANS_B) {
            DmaLoader<C::BN, C::NT> lb;
#pragma unroll
            for (int i = 0; i < lb.RPT; ++i) {
                const int r = lb.tile_row(i);
                lb.set_row(i, n0 + r < g.n ? n0 + r : -1, w_row);
            }
            mainloop_ring<C, NST, false, false, decltype(la)::RPT + decltype(lb)::RPT>(
                smem, nsteps, acc,
                [&](int s, char *As, char *Bs) {
                    la.load(xr, As, s * BK, kk);
                    lb.load(wr, Bs, s * BK, kk);
                },
                min(C::BM, g.m - m0));
        } else {
            TileDmaLoader<C::BN, C::NT> lb;
            const int n = g.n;
            mainloop_ring<C, NST, false, true, decltype(la)::RPT + decltype(lb)::RPT>(
                smem, nsteps, acc,
                [&](int s, char *As, char *Bs) {
                    lb.prepare_rows(n0, n, w_row, [&](int row) {
                        const int red = s * BK + row;
                        return red < kk ? red : -1;
                    });
                    __builtin_amdgcn_sched_barrier(0);
                    la.load(xr, As, s * BK, kk);
                    lb.issue(wr, Bs);
                },
                min(C::BM, g.m - m0));
        }
        epilogue_bf16<C>(st0, st1, acc, s_dst, nullptr, static_cast<char *>(g.y), g.ldy, n0, g.n);
    }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

// Tile shapes: <BM, BN, waves along M, waves along N>.
using BigCfg = Cfg<256, 256, 2, 4>;     // many rows per expert
using DxCfg = Cfg<256, 256, 2, 4>;
using DxQuadCfg = Cfg<256, 256, 2, 2>;  // long reductions: four-wave engine
using DwCfg = Cfg<256, 256, 2, 4>;
using SmallCfg = Cfg<32, 128, 1, 4>;    // few rows per expert: stream the weights
using DxSmallCfg = Cfg<32, 128, 1, 4>;     // the same for dX
using SmallGatedCfg = Cfg<32, 256, 1, 4>;  // the same with two blocks per wave to pair
// Small explicit groups: tiles of 64 x 128 so that the dual-expert layer's
// 256 tiles cover every CU (128 x 128 tiles: 15.4 us against 11.9 us there;
// each tile's copies, about 0.4 MB over K = 1024, bound a CU's time).
using GroupCfg = Cfg<64, 128, 1, 4>;

// Explicit instantiations: every kernel the launchers use is emitted here.
template __global__ void fwd_kernel<BigCfg, false>(FwdParams);
template __global__ void fwd_kernel<SmallCfg, false>(FwdParams);
template __global__ void fwd_kernel<BigCfg, true>(FwdParams);
template __global__ void fwd_kernel<SmallGatedCfg, true>(FwdParams);
template __global__ void dx_kernel<DxCfg>(DxParams);
template __global__ void dx_kernel<DxQuadCfg>(DxParams);
template __global__ void dx_kernel<DxSmallCfg>(DxParams);
template __global__ void dw_kernel<DwCfg, false, false>(DwParams);
template __global__ void dw_kernel<DwCfg, true, false>(DwParams);
template __global__ void dw_kernel<DwCfg, false, true>(DwParams);

// ---------------------------------------------------------------------------
// dW for short reductions (a decode step: a few hundred slots spread over
// many experts, most of them a handful of rows).  There the output is all
// that costs (E*N*K*2 bytes against S*(N+K)*2 of operands), and the tile
// engine spends a copy round trip and a 128 KiB LDS staging pass on every
// 256 x 256 tile whatever its reduction length, with one workgroup per CU to
// hide them.  Here every wave owns 64 (N) x 64 (K) output tiles and works
// alone (no workgroup barrier after the expert table):
//   * operands come from global memory straight into MFMA fragments.  Lane
//     l of v_mfma_f32_32x32x16_bf16 needs 8 consecutive reduction rows of one
//     column: 8 two-byte buffer loads per fragment (32 lanes read 64
//     contiguous bytes of one row; rows past the expert read zero), rows
//     gathered under permute_x / permute_y.  The operands are a few MB and
//     stay in L2.
//   * the tile is computed as its transpose (MFMA rows along K), so a lane
//     holds 4 consecutive K values of one N row; it is rounded to bf16 into
//     a wave-private LDS tile and written out as whole 128-byte row segments,
//     8 rows per store instruction (fp32 output is stored from the
//     accumulators, 16 bytes per lane).
//   * an empty expert's tiles are zeros through the same path.
// Tiles are dealt round-robin over the waves (eight per CU).  The stores
// bound it: on the decode step the same launch with every expert empty (no
// loads, no MFMAs) takes as long as the real one.
constexpr int kSdwWaves = 4;  // waves per workgroup
constexpr int kSdwT = 64;     // output tile: kSdwT rows of N by kSdwT columns of K
constexpr uint32_t kSdwOOB = 1u << 30;
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));

template <bool PX, bool PY>
__global__ __launch_bounds__(kSdwWaves * kWave) void dw_small_kernel(DwParams a)
{
    __shared__ int s_roff[kMaxExperts + 1];
    __shared__ int s_scratch[2];
    __shared__ __attribute__((aligned(16))) char s_out[kSdwWaves][kSdwT * kSdwT * 2];
    static_assert(sizeof(s_out) >= (kMaxExperts + 1) * sizeof(int), "tile table fits");
    // The table's tile starts are not used here: they go to the output tiles'
    // LDS (four workgroups per CU fit), which the barrier at its end frees.
    build_expert_tables(a.m_sizes, a.E, a.S, s_roff, reinterpret_cast<int *>(&s_out[0][0]),
                        s_scratch, a.err, [](int) { return 0; });
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int col = lane & 31, half = lane >> 5;
    const int ntn = (a.N + kSdwT - 1) / kSdwT, ntk = (a.K + kSdwT - 1) / kSdwT;
    const int per_expert = ntn * ntk;
    const int64_t total = (int64_t)per_expert * a.E;
    const bool f32out = a.flags & MOEGG_DW_FP32_OUT;
    // Operands below 1 GiB each (checked on the host): offsets of 1 GiB and
    // above (kSdwOOB, alone or added to a row or column offset) read zero.
    const uint32_t xrow = (uint32_t)a.K * 2, yrow = (uint32_t)a.N * 2;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(a.X), 0, (int)((PX ? a.S / a.topk : a.S) * xrow), 0x00020000);
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(a.dY), 0, (int)(a.S * yrow), 0x00020000);
    char *const lds = s_out[wave];
    const uint32_t Su = (uint32_t)a.S;
    bool bad = false;
    // Byte offsets of this lane's 8 reduction rows c0 + 8 * half + i of the
    // expert starting at slot `start`, in X and in dY (kSdwOOB: zeros, past
    // the expert or a bad gather entry).  The gather loads are unconditional,
    // from clamped in-bounds addresses, so all 8 are in flight together.
    auto step_rows = [&](int start, int m_e, int c0, uint32_t (&ox)[8], uint32_t (&oy)[8]) {
        int g[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int p = start + min(c0 + 8 * half + i, m_e - 1);
            g[i] = (PX || PY) ? a.gather[p] : p;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int m = c0 + 8 * half + i, p = start + m;
            const bool in = m < m_e;
            const bool ok = !(PX || PY) || (uint32_t)g[i] < Su;
            bad |= in && !ok;
            const int rx = !PX ? p : fast_div((uint32_t)g[i], a.topk_div);
            const int ry = !PY ? p : g[i];
            ox[i] = in && (ok || !PX) ? (uint32_t)rx * xrow : kSdwOOB;
            oy[i] = in && (ok || !PY) ? (uint32_t)ry * yrow : kSdwOOB;
        }
    };
    // Fragment of column c (< lim) over the 8 rows at byte offsets off[]:
    // buffer loads, so that an offset past the operand reads zero.
    auto frag = [&](__amdgpu_buffer_rsrc_t r, const uint32_t (&off)[8], int c,
                    int lim) -> bf16x8_t {
        const uint32_t co = c < lim ? (uint32_t)c * 2 : kSdwOOB;
        u16x8_t v;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = __builtin_amdgcn_raw_buffer_load_b16(r, off[i] + co, 0, 0);
        return __builtin_bit_cast(bf16x8_t, v);
    };
    // Tiles are dealt out round-robin over the waves (an expert's tiles cost
    // in proportion to its rows, so contiguous runs would leave the waves
    // of a hot expert behind the rest).
    const int64_t nwaves = (int64_t)gridDim.x * kSdwWaves;
    for (int64_t t = (int64_t)xcd_logical_block(blockIdx.x, gridDim.x) * kSdwWaves + wave;
         t < total; t += nwaves) {
        const int e = (int)(t / per_expert), u = (int)(t % per_expert);
        const int n0 = (u / ntk) * kSdwT, k0 = (u % ntk) * kSdwT;
        const int start = s_roff[e], m_e = s_roff[e + 1] - start;
        f32x16_t acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.0f;
        for (int c0 = 0; c0 < m_e; c0 += 16) {
            uint32_t ox[8], oy[8];
            step_rows(start, m_e, c0, ox, oy);
            bf16x8_t fa[2], fb[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                fa[j] = frag(xr, ox, k0 + 32 * j + col, a.K);
                fb[j] = frag(yr, oy, n0 + 32 * j + col, a.N);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j],
                                                                         0, 0, 0);
        }
        // acc[i][j][r]: K column k0 + 32 i + 8 (r / 4) + 4 half + r % 4 of
        // N row n0 + 32 j + col.
        if (f32out) {
            float *const out = reinterpret_cast<float *>(a.dW);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int n = n0 + 32 * j + col, k = k0 + 32 * i + 8 * g + 4 * half;
                        if (n < a.N && k < a.K) {
                            const float4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1],
                                              acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                            *reinterpret_cast<float4 *>(out + ((int64_t)e * a.N + n) * a.K + k) = v;
                        }
                    }
            continue;
        }
        wait_lds();  // the previous tile's reads of this wave's LDS tile are done
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int row = 32 * j + col;
                    const uint2 v = {pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                                     pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
                    *reinterpret_cast<uint2 *>(lds + row * (kSdwT * 2) +
                                               swz_chunk(row, 4 * i + g) * 16 + half * 8) = v;
                }
        wait_lds();  // every lane's writes are in LDS before any lane reads them
        char *const base = a.dW + (((int64_t)e * a.N + n0) * a.K + k0) * 2;
#pragma unroll
        for (int q = 0; q < kSdwT * kSdwT * 2 / 16 / kWave; ++q) {
            const int idx = q * kWave + lane;
            const int row = idx / 8, c = idx % 8;
            const u32x4_nt_t v = *reinterpret_cast<const u32x4_nt_t *>(
                lds + row * (kSdwT * 2) + swz_chunk(row, c) * 16);
            if (n0 + row < a.N && k0 + 8 * c < a.K)
                __builtin_nontemporal_store(
                    v, reinterpret_cast<u32x4_nt_t *>(base + ((int64_t)row * a.K + 8 * c) * 2));
        }
    }
    if (bad)
        raise_error(a.err, kErrGather);
}
template __global__ void dw_small_kernel<false, false>(DwParams);
template __global__ void dw_small_kernel<true, false>(DwParams);
template __global__ void dw_small_kernel<false, true>(DwParams);
template __global__ void groups_kernel<GroupCfg, true>(GroupsParams);
template __global__ void groups_kernel<GroupCfg, false>(GroupsParams);

static int64_t n_blocks_bound(int64_t rows, int E, int block)
{
    if (rows <= E)
        return rows;
    return (rows - E + 1 + block - 1) / block + E - 1;
}

template <class Kern>
static int resident_blocks(Kern kernel, int threads)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1)
        n = 1;
    return n;
}

static int grid_for(int64_t tiles_bound, int cus, int resident)
{
    int64_t g = (int64_t)cus * resident;
    if (tiles_bound < g)
        g = tiles_bound;
    return (int)(g < 1 ? 1 : g);
}

template <class C, bool GATED>
static void fwd_launch_cfg(const FwdParams &p, int cus, hipStream_t stream)
{
    const int64_t tiles = n_blocks_bound(p.S, p.E, C::BM) * ((p.N + C::BN - 1) / C::BN);
    static int res = resident_blocks(fwd_kernel<C, GATED>, C::NT);
    hipLaunchKernelGGL((fwd_kernel<C, GATED>), dim3(grid_for(tiles, cus, res)), dim3(C::NT), 0,
                       stream, p);
}

hipError_t fwd_launch(const FwdParams &p, int cus, hipStream_t stream)
{
    const bool small = p.S / p.E < 96;
    if (p.flags & MOEGG_GATED_SILU) {
        if (small)
            fwd_launch_cfg<SmallGatedCfg, true>(p, cus, stream);
        else
            fwd_launch_cfg<BigCfg, true>(p, cus, stream);
    } else {
        if (small)
            fwd_launch_cfg<SmallCfg, false>(p, cus, stream);
        else
            fwd_launch_cfg<BigCfg, false>(p, cus, stream);
    }
    return hipGetLastError();
}

template <class C>
static int dx_resident()
{
    static int res = resident_blocks(dx_kernel<C>, C::NT);
    return res;
}

template <class C>
static void dx_launch_cfg(const DxParams &p, int cus, hipStream_t stream)
{
    const int64_t tiles = n_blocks_bound(p.S, p.E, C::BM) * ((p.K + C::BN - 1) / C::BN);
    hipLaunchKernelGGL(dx_kernel<C>, dim3(grid_for(tiles, cus, dx_resident<C>())), dim3(C::NT), 0,
                       stream, p);
    if (p.ws) {
        TailReduceParams r;
        r.ws = p.ws;
        r.out = p.dX;
        r.gather = p.gather;
        r.S = p.S;
        r.ldo = p.K;
        r.ncols = p.K;
        r.scatter_out = p.flags & MOEGG_PERMUTE_X;
        hipLaunchKernelGGL((tail_reduce_kernel<C::BM, C::BN>), dim3(cus * 4), dim3(256), 0, stream,
                           r);
    }
}

// Measured on MI355X: the four-wave engine is faster once the reduction (N)
// is long enough to amortise its per-tile prologue (T=4096 top-2, N=28672:
// 2.16 ms against 2.44 ms); at N = 2048 the eight-wave engine is.
constexpr int kDxQuadMinN = 8192;

// Average rows per expert below which dX uses the small-M tiles: the
// weights are then streamed once per 32-row tile (a decode slice), where
// 256 x 256 tiles would leave about one long, latency-bound tile per CU
// (T=64 top-8 of E=128, N=2048, K=768: 0.064 ms against 0.114 ms).
constexpr int64_t kSmallRows = 96;

// Workspace of the tail split: the header and at most G partials of one
// tile (R * P <= G), for the grid the launch below will use.
template <class C>
static int64_t dx_ws_cfg(int cus)
{
    const int64_t G = (int64_t)cus * dx_resident<C>();
    return G > kTailMaxTiles ? 0 : tail_header_bytes() + G * C::BM * C::BN * 4;
}

// The small-M tiles are many and short (a decode slice): their last round
// costs little, and the finishing launch would cost more.
int64_t dx_workspace_bytes(int64_t S, int E, int N, int K, int cus)
{
    (void)K;
    if (S / E < kSmallRows)
        return 0;
    if (N >= kDxQuadMinN)
        return dx_ws_cfg<DxQuadCfg>(cus);
    return dx_ws_cfg<DxCfg>(cus);
}

hipError_t dx_launch(const DxParams &p, int cus, hipStream_t stream)
{
    if (p.S / p.E < kSmallRows)
        dx_launch_cfg<DxSmallCfg>(p, cus, stream);
    else if (p.N >= kDxQuadMinN)
        dx_launch_cfg<DxQuadCfg>(p, cus, stream);
    else
        dx_launch_cfg<DxCfg>(p, cus, stream);
    return hipGetLastError();
}

// Split reductions.  The target is about three work items per workgroup of
// a full 256-CU chip when the rows are spread evenly over the experts:
// chunks of S * tiles_per_expert / (256 * 3) rows (at least 4 reduction
// steps), so that with the longest items scheduled first no workgroup is
// left with one hot expert's whole reduction.  An expert splits only if it
// has more rows than that; a split expert has fewer than 2 m / split_rows
// chunks, so all of them together hold fewer than 2 S / split_rows partials.
constexpr int kSplitCus = 256, kSplitItems = 3;
constexpr int64_t kNoSplitRows = 1024;

int dw_split_rows(int64_t S, int N, int K)
{
    using C = DwCfg;
    // A launch this short has no reduction long enough to be worth cutting
    // (at most four chunks of 256 rows); without a split the reduce launch
    // is not needed either (a decode step's dW: 4.4 us saved).
    if (S <= kNoSplitRows)
        return 0;
    const int64_t tiles = (int64_t)((N + C::BM - 1) / C::BM) * ((K + C::BN - 1) / C::BN);
    int64_t rows = (S * tiles + kSplitCus * kSplitItems - 1) / (kSplitCus * kSplitItems);
    rows = (rows + BK - 1) / BK * BK;
    if (rows < 4 * BK)
        rows = 4 * BK;
    return rows >= S ? 0 : (int)rows;
}

int64_t dw_workspace_bytes(int64_t S, int E, int N, int K)
{
    const int rows = dw_split_rows(S, N, K);
    if (rows == 0)
        return 0;
    const int64_t partials = 2 * S / rows;
    return dw_header_bytes(E) + partials * N * K * 4;
}

// Byte offset of the gathered X rows in dW's workspace, after the split
// partials.
int64_t dw_gather_offset(int64_t S, int E, int N, int K)
{
    return (dw_workspace_bytes(S, E, N, K) + 255) / 256 * 256;
}

// X rows in expert order for dW under permute_x, when the caller's
// workspace has room for them: xg[p, :] = X[gather[p] / topk, :].  The
// reduction then reads xg in sorted order.  On the Mixtral shape (8192 slots,
// K 4096) the copy takes 0.020 ms and dW 2.00-2.05 ms, against 2.17-2.20 ms
// for the row gather inside dW, with the same result bit for bit: the
// scattered row reads cost dW's copy path more than one streaming pass
// costs.  One workgroup per row at a time; an entry outside [0, S) gives a
// zero row and is reported, as the gather inside dW does.  Only the
// positions the reduction reads are copied: those below the sum of m_sizes
// (negative sizes as 0, clipped to S, as the reduction's tables take them),
// so the entries routing leaves at -1 for dropped slots are not touched.
// Plain stores: dW reads the copy right after.
__global__ __launch_bounds__(256) void gather_x_kernel(DwParams a)
{
    __shared__ long long s_part[256 / kWave];
    long long part = 0;
    for (int e = threadIdx.x; e < a.E; e += blockDim.x)
        part += max(a.m_sizes[e], 0);
    for (int d = kWave / 2; d > 0; d >>= 1)
        part += __shfl_xor(part, d, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0)
        s_part[threadIdx.x / kWave] = part;
    __syncthreads();
    int64_t rows = 0;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w)
        rows += s_part[w];
    rows = min(rows, a.S);
    const int cpr = a.K / 8;  // 16-byte chunks per row
    for (int64_t p = blockIdx.x; p < rows; p += gridDim.x) {
        const int g = __builtin_amdgcn_readfirstlane(a.gather[p]);
        const bool ok = g >= 0 && g < a.S;
        if (!ok && threadIdx.x == 0)
            raise_error(a.err, kErrGather);
        const char *src = a.X + (int64_t)(ok ? g / a.topk : 0) * a.K * 2;
        char *dst = a.xg + p * a.K * 2;
        for (int c = threadIdx.x; c < cpr; c += blockDim.x)
            *reinterpret_cast<uint4 *>(dst + c * 16) =
                ok ? *reinterpret_cast<const uint4 *>(src + c * 16) : uint4{0, 0, 0, 0};
    }
}

template <bool PX, bool PY>
static void dw_launch_flags(const DwParams &p, int cus, hipStream_t stream)
{
    using C = DwCfg;
    // Work items: every (expert, output tile) plus the extra chunks of split
    // experts, fewer than 2 S / split_rows in all.
    const int64_t per_expert = (int64_t)((p.N + C::BM - 1) / C::BM) * ((p.K + C::BN - 1) / C::BN);
    int64_t tiles = p.E * per_expert;
    if (p.split_rows > 0)
        tiles += 2 * p.S / p.split_rows * per_expert;
    static int res = resident_blocks(dw_kernel<C, PX, PY>, C::NT);
    hipLaunchKernelGGL((dw_kernel<C, PX, PY>), dim3(grid_for(tiles, cus, res)), dim3(C::NT), 0,
                       stream, p);
}


// Launches of at most 1024 slots and at most 16 rows per expert on average
// take dw_small_kernel (no split, no gather copy: the rows are gathered as
// the fragments are loaded).  Measured on MI355X, 128 experts of 2048 x 768:
// a 64-token top-8 decode step (512 slots) 0.092 -> 0.080 ms; 64 experts of
// 2048 x 1408, 512 slots 0.082 -> 0.071 ms; 64 experts of 2048 x 768, 1024
// slots 0.052 -> 0.049 ms.  With 128 rows per expert (8 experts of
// 4096 x 4096, 1024 slots) it is 2.3x slower than the tile engine, whose
// cost does not grow with the reduction here.
constexpr int64_t kSmallDwSlots = 1024, kSmallDwRowsPerExpert = 16;

bool dw_short_launch(int64_t S, int64_t x_rows, int E, int N, int K)
{
    return S <= kSmallDwSlots && S <= kSmallDwRowsPerExpert * E &&
           S * N * 2 < (int64_t)kSdwOOB && x_rows * K * 2 < (int64_t)kSdwOOB;
}

template <bool PX, bool PY>
static void dw_small_launch(const DwParams &p, int cus, hipStream_t stream)
{
    const int64_t tiles = (int64_t)p.E * ((p.N + kSdwT - 1) / kSdwT) * ((p.K + kSdwT - 1) / kSdwT);
    static int res = resident_blocks(dw_small_kernel<PX, PY>, kSdwWaves * kWave);
    hipLaunchKernelGGL((dw_small_kernel<PX, PY>),
                       dim3(grid_for((tiles + kSdwWaves - 1) / kSdwWaves, cus, res)),
                       dim3(kSdwWaves * kWave), 0, stream, p);
}

hipError_t dw_launch(const DwParams &pin, int cus, hipStream_t stream)
{
    DwParams p = pin;
    if (dw_short_launch(p.S, (p.flags & MOEGG_PERMUTE_X) ? p.S / p.topk : p.S, p.E, p.N, p.K)) {
        if (p.flags & MOEGG_PERMUTE_X)
            dw_small_launch<true, false>(p, cus, stream);
        else if (p.flags & MOEGG_PERMUTE_Y)
            dw_small_launch<false, true>(p, cus, stream);
        else
            dw_small_launch<false, false>(p, cus, stream);
        return hipGetLastError();
    }
    if (p.xg && (p.flags & MOEGG_PERMUTE_X) && p.S > 0) {
        hipLaunchKernelGGL(gather_x_kernel, dim3((unsigned)std::min<int64_t>(p.S, (int64_t)cus * 16)),
                           dim3(256), 0, stream, p);
        p.X = p.xg;
        p.flags &= ~MOEGG_PERMUTE_X;
    }
    if (p.flags & MOEGG_PERMUTE_X)
        dw_launch_flags<true, false>(p, cus, stream);
    else if (p.flags & MOEGG_PERMUTE_Y)
        dw_launch_flags<false, true>(p, cus, stream);
    else
        dw_launch_flags<false, false>(p, cus, stream);
    if (p.split_rows > 0 && p.ws)
        hipLaunchKernelGGL(dw_reduce_kernel, dim3(cus * 8), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t groups_launch(const GroupsParams &p, int trans_b, int cus, hipStream_t stream)
{
    using C = GroupCfg;
    int64_t tiles = 0;
    for (int i = 0; i < p.num; ++i)
        tiles += (int64_t)((p.g[i].m + C::BM - 1) / C::BM) * ((p.g[i].n + C::BN - 1) / C::BN);
    if (trans_b) {
        static int res = resident_blocks(groups_kernel<C, true>, C::NT);
        hipLaunchKernelGGL((groups_kernel<C, true>), dim3(grid_for(tiles, cus, res)), dim3(C::NT),
                           0, stream, p);
    } else {
        static int res = resident_blocks(groups_kernel<C, false>, C::NT);
        hipLaunchKernelGGL((groups_kernel<C, false>), dim3(grid_for(tiles, cus, res)), dim3(C::NT),
                           0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace moegg
