// expert.hip -- tile-signalled return path: a stand-in expert GEMM over the
// (source, local expert) blocks of a receive buffer, whose output tiles
// publish readiness flags, and a consumer that returns each source's rows
// as soon as they are ready.
//
// Method: thecoregrid "Mixture-of-experts acceleration through overlap"
// (producer GEMM and consumer kept apart but synchronised per tile: the
// GEMM epilogue publishes a flag per tile; the consumer starts a transfer
// once enough row bands are ready and moves several bands per transfer;
// tiles are tied to one destination, remote-owner-aligned, and remote
// tiles are computed first; the GPU's compute units are split between the
// two roles); aicassindra "gpu_moe_all_to_all", "Overlapping dispatch with
// expert compute" (the strict dispatch -> compute -> combine chain that
// per-tile signalling relaxes).
//
// On one GPU the R sources are partitions of one buffer, so the "transfer"
// is a copy of a contiguous row range from the expert output y to the
// return buffer ret, which has the same layout as the sources' send
// buffers: combine then reads ret unchanged.
//
// Kernels:
//  * linear_table_kernel (one block): from the S x E_l counts, the first row
//    of every (source, expert) block, the row bands (128-row tiles of a
//    block) counted in remote-first order -- sources self+1, self+2, ...,
//    self last -- and the consumer tasks (up to band_group bands of one
//    source). It also clears the band flags and the status word, with
//    ordinary stores, so a call needs no memset.
//  * expert_linear_kernel: a persistent grouped GEMM, one block per CU. Tile
//    = 128 rows (one band) x 512 output columns, K-steps of 32; 4 waves,
//    each 128 x 128 of the tile with v_mfma_f32_32x32x16_bf16 (bf16 in,
//    fp32 accumulate, all 256 AGPRs). Operands go straight from memory to LDS
//    (buffer loads with an LDS destination) through four 40 KiB stages, so
//    a K-step's loads are issued three steps ahead and hold no registers;
//    the next step's first fragments are read while this step multiplies.
//    LDS rows carry no padding: a chunk permutation keeps the fragment reads
//    conflict-free. The epilogue rounds to bf16 (nearest even), stages the
//    tile in LDS and writes 16-byte row chunks. Work units (a band by one
//    column tile) are dealt so that each XCD takes runs of consecutive
//    units: a band's 128-row A slab is read into one L2.
//  * expert_return_kernel: the same GEMM in producer blocks, which after
//    each unit release-add one to the band's count of column tiles (one L2
//    write-back per unit, which other XCDs need to see the tile). With
//    consumer blocks, those take tasks in order, wait (bounded) until every
//    band of the task has all its column tiles, then copy the task's rows to
//    ret; a wait that exceeds its bound sets the status word and skips the
//    copy instead of spinning on. Without them, the unit that completes a
//    band counts it toward its task and the one that completes the task
//    copies it. One cooperative launch keeps every block resident, so no
//    consumer waits on a producer that cannot run.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
// GEMM tile: 128 rows (one band) x 512 output columns, K-steps of 32; each of
// the 4 waves owns 128 x 128 of the tile (16 fp32 accumulators of 32 x 32).
constexpr int kBM = 128, kBN = 512, kBK = 32, kStages = 4;
constexpr int kRowB = kBK * 2;                        // 64-byte LDS rows, no padding (swizzled)
constexpr int kABytes = kBM * kRowB;                  // 8 KiB: the band's rows of one K-step
constexpr int kBBytes = kBN * kRowB;                  // 32 KiB: the tile's W rows of one K-step
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kLdsBytes = kStages * kStageBytes;      // 160 KiB: all of a CU's LDS, one block per CU
constexpr int kCRowBytes = kBN * 2 + 16;              // LDS row of the staged output tile
static_assert(kBM * kCRowBytes <= kLdsBytes, "output stage must fit the operand space");
constexpr int kFillA = kABytes / 1024 / 4, kFillB = kBBytes / 1024 / 4;  // 1 KiB fills per wave per stage
constexpr int kFill = kFillA + kFillB;
constexpr int kTableThreads = 1024;
constexpr int kSpinLimit = 1 << 21;            // polls before a wait gives up (about 1 s)

// word 3 of a buffer resource for plain byte-addressed loads (32-bit data
// format, as raw buffer loads on this architecture require)
constexpr int kBufferFlags = 0x00020000;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Workspace layout (int32 words), for SE = S * E_l blocks and NBmax bands.
struct LinearWs {
    int32_t *status;       // [1]      0; 1 = a consumer wait expired; 2 = counts exceed the buffers
    int32_t *counts;       // [2]      total bands, total consumer tasks
    int32_t *blk_row;      // [SE]     first row of source-major block s*E_l+l
    int32_t *band_prefix;  // [SE + 1] bands before remote-first block q*E_l+l
    int32_t *task_prefix;  // [S + 1]  consumer tasks before remote-first source q
    int32_t *flags;        // [NBmax]  finished column tiles per band
    int32_t *task_flags;   // [NBmax]  finished bands per consumer task (inline return)
};

__host__ __device__ inline int64_t max_bands(int32_t S, int32_t El, int64_t max_rows)
{
    return (int64_t)S * El + (max_rows + kBM - 1) / kBM;
}

// the flag arrays' length is kept in the workspace itself (word 3)
__host__ __device__ inline int64_t max_bands_of(const int32_t *base) { return base[3]; }

__host__ __device__ inline LinearWs linear_ws(int32_t *base, int32_t S, int32_t El)
{
    const int64_t SE = (int64_t)S * El;
    LinearWs w;
    w.status = base;
    w.counts = base + 1;
    w.blk_row = base + 4;
    w.band_prefix = w.blk_row + SE;
    w.task_prefix = w.band_prefix + SE + 1;
    w.flags = w.task_prefix + S + 1;
    w.task_flags = w.flags + max_bands_of(base);
    return w;
}

__host__ __device__ inline int64_t linear_ws_words(int32_t S, int32_t El, int64_t max_rows)
{
    return 4 + 2 * (int64_t)S * El + 1 + S + 1 + 2 * max_bands(S, El, max_rows);
}

// exclusive scan of one value per thread over a 1024-thread block
__device__ int32_t block_scan(int32_t v, int32_t *wave_total, int32_t *total)
{
    constexpr int WAVES = kTableThreads / kWave;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int32_t inc = wave_inclusive_sum(v);
    __syncthreads();
    if (lane == kWave - 1)
        wave_total[w] = inc;
    __syncthreads();
    int32_t before = 0, all = 0;
#pragma unroll
    for (int u = 0; u < WAVES; ++u) {
        before += u < w ? wave_total[u] : 0;
        all += wave_total[u];
    }
    *total = all;
    return before + inc - v;
}

// Each thread owns up to 4 consecutive entries of a 4096-entry sequence.
__global__ __launch_bounds__(kTableThreads) void linear_table_kernel(
    const int32_t *__restrict__ cnt, int32_t S, int32_t El, int32_t self_rank, int32_t band_group,
    int64_t max_rows, int64_t flag_words, int32_t *__restrict__ ws_base)
{
    __shared__ int32_t wave_total[kTableThreads / kWave];
    __shared__ unsigned long long rows64;  // the row total without int32 wrap-around
    const int SE = S * El;
    const int tid = threadIdx.x;
    if (tid == 0) {
        rows64 = 0;
        ws_base[3] = (int32_t)flag_words;
    }
    __syncthreads();
    const LinearWs ws = linear_ws(ws_base, S, El);
    for (int64_t i = tid; i < 2 * flag_words; i += kTableThreads)
        ws.flags[i] = 0;  // band counts, then task counts
    // 1) first rows of the source-major blocks
    int32_t c[4], part = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int b = tid * 4 + u;
        c[u] = b < SE ? max(cnt[b], 0) : 0;
        part += c[u];
    }
    __syncthreads();
    atomicAdd(&rows64, (unsigned long long)c[0] + c[1] + c[2] + c[3]);
    int32_t total;
    int32_t run = block_scan(part, wave_total, &total);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int b = tid * 4 + u;
        if (b < SE)
            ws.blk_row[b] = run;
        run += c[u];
    }
    // 2) bands in remote-first order: block rb = q*El + l is source (self+1+q) % S
    int32_t nb[4];
    part = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int rb = tid * 4 + u;
        nb[u] = 0;
        if (rb < SE) {
            const int q = rb / El, l = rb - q * El;
            const int s = (self_rank + 1 + q) % S;
            nb[u] = (int32_t)(((int64_t)max(cnt[s * El + l], 0) + kBM - 1) / kBM);
        }
        part += nb[u];
    }
    int32_t n_bands;
    run = block_scan(part, wave_total, &n_bands);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int rb = tid * 4 + u;
        if (rb < SE)
            ws.band_prefix[rb] = run;
        run += nb[u];
    }
    // 3) consumer tasks per remote-first source q: ceil(bands of q / band_group)
    int32_t tasks = 0;
    if (tid < S) {
        int32_t bq = 0;
        for (int l = 0; l < El; ++l) {
            const int s = (self_rank + 1 + tid) % S;
            bq += (int32_t)(((int64_t)max(cnt[s * El + l], 0) + kBM - 1) / kBM);
        }
        tasks = (bq + band_group - 1) / band_group;
    }
    int32_t n_tasks;
    const int32_t tstart = block_scan(tasks, wave_total, &n_tasks);
    if (tid < S)
        ws.task_prefix[tid] = tstart;
    if (tid == 0) {
        // counts totalling more rows than the buffers hold: publish no work
        const bool fits = rows64 <= (unsigned long long)max_rows;
        ws.band_prefix[SE] = n_bands;
        ws.task_prefix[S] = n_tasks;
        ws.counts[0] = fits ? n_bands : 0;
        ws.counts[1] = fits ? n_tasks : 0;
        ws.status[0] = fits ? 0 : 2;
    }
}

// largest index i in [0, n) with a[i] <= v (a ascending, a[0] <= v)
__device__ __forceinline__ int upper_index(const int32_t *a, int n, int32_t v)
{
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a[mid] <= v)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

struct Band {
    int32_t row0;   // first row of the band
    int32_t rows;   // rows in the band (1..128)
    int32_t l;      // local expert
};

// band index (remote-first order) -> rows and expert
__device__ __forceinline__ Band band_info(const LinearWs &ws, const int32_t *cnt, int32_t S,
                                          int32_t El, int32_t self_rank, int32_t band)
{
    const int SE = S * El;
    const int rb = upper_index(ws.band_prefix, SE, band);
    const int q = rb / El, l = rb - q * El;
    const int s = (self_rank + 1 + q) % S;
    const int32_t rt = band - ws.band_prefix[rb];
    const int32_t n = max(cnt[s * El + l], 0);
    Band b;
    b.row0 = ws.blk_row[s * El + l] + rt * kBM;
    b.rows = min(kBM, n - rt * kBM);
    b.l = l;
    return b;
}

// Position of 16-byte chunk c of 64-byte LDS row i: c ^ swz(i & 15). A 16-byte
// read of one chunk from 16 consecutive rows (or from 8) then touches
// distinct banks, with no padding.
__device__ __forceinline__ int swz(int i) { return ((i >> 1) & 3) ^ (((i >> 3) & 1) * 3); }

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmem()
{
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ bf16x8 frag(const uint8_t *__restrict__ base, int row, int blk, int koff)
{
    return *reinterpret_cast<const bf16x8 *>(base + row + blk * 32 * kRowB + koff);
}

// Start the loads of one stage: x's band rows and the tile's W rows for the
// K-step at byte offset kb go straight to LDS (buffer loads with an LDS
// destination, 1 KiB per instruction and wave: 16 rows x 64 bytes).
__device__ __forceinline__ void fill_stage(uint8_t *__restrict__ fill, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, int kb,
                                           const uint32_t (&aoff)[kFillA], const uint32_t (&boff)[kFillB],
                                           int wave)
{
#pragma unroll
    for (int i = 0; i < kFillA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, fill + (i * 4 + wave) * 1024, 16, aoff[i], kb, 0, 0);
#pragma unroll
    for (int i = 0; i < kFillB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, fill + kABytes + (i * 4 + wave) * 1024, 16, boff[i], kb, 0, 0);
}

__device__ __forceinline__ void first_frags(const uint8_t *__restrict__ cur, int arow, int brow, int koff0,
                                            bf16x8 (&f0)[8])
{
#pragma unroll
    for (int q = 0; q < 8; ++q)
        f0[q] = q < 4 ? frag(cur, arow, q, koff0) : frag(cur + kABytes, brow, q - 4, koff0);
}

// One K-step of 32: multiply the first 16 of stage `cur` (fragments f0, read
// during the previous step) while reading its second 16 into f1, then
// multiply those while reading the first 16 of stage `nxt` into f0 (MORE);
// with LOAD, the fill of stage `fill` is spread over the first half. The
// groups are pinned in this order, so LDS reads and fills overlap the
// MFMAs. The stage pointers are restrict-qualified: the compiler then knows
// that reads of one stage do not depend on the fill of another and leaves
// the waits to the caller's explicit ones.
template <bool LOAD, bool MORE>
__device__ __forceinline__ void kstep(const uint8_t *__restrict__ cur, const uint8_t *__restrict__ nxt,
                                      uint8_t *__restrict__ fill, __amdgpu_buffer_rsrc_t ra,
                                      __amdgpu_buffer_rsrc_t rb, int kb, const uint32_t (&aoff)[kFillA],
                                      const uint32_t (&boff)[kFillB], int wave, int arow, int brow,
                                      const int (&koff)[2], bf16x8 (&f0)[8], bf16x8 (&f1)[8],
                                      f32x16 (&acc)[4][4])
{
    static_assert(kFillA + kFillB == 10, "the fill schedule below spreads 10 loads over 8 groups");
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        if (LOAD) {
            if (q < kFillA)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, fill + (q * 4 + wave) * 1024, 16, aoff[q], kb, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, fill + kABytes + ((q - kFillA) * 4 + wave) * 1024,
                                                         16, boff[q - kFillA], kb, 0, 0);
            if (q < 2)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, fill + kABytes + ((6 + q) * 4 + wave) * 1024, 16,
                                                         boff[6 + q], kb, 0, 0);
        }
        f1[q] = q < 4 ? frag(cur, arow, q, koff[1]) : frag(cur + kABytes, brow, q - 4, koff[1]);
        __builtin_amdgcn_sched_barrier(0);
        const int i = q >> 1, j = (q & 1) * 2;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0[i], f0[4 + j], acc[i][j], 0, 0, 0);
        acc[i][j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0[i], f0[5 + j], acc[i][j + 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        if (MORE)  // f0[q] is free: the first half's MFMAs have read it
            f0[q] = q < 4 ? frag(nxt, arow, q, koff[0]) : frag(nxt + kABytes, brow, q - 4, koff[0]);
        __builtin_amdgcn_sched_barrier(0);
        const int i = q >> 1, j = (q & 1) * 2;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1[i], f1[4 + j], acc[i][j], 0, 0, 0);
        acc[i][j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1[i], f1[5 + j], acc[i][j + 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One 128 x 512 output tile: y[row0 .. row0+rows)[n0 .. n0+512) =
// x[rows] . W[l][n0 .. n0+512)^T, accumulated over K = H in fp32, columns at
// or past H_out not stored. The K-steps stream through four LDS stages: at
// the top of step s, stage s + 1 is complete (every wave waits for its own
// fills, then a barrier), so step s reads the first fragments of stage
// s + 1 while it multiplies stage s, and fills stage s + 3. Rows past the
// band re-read its last row and W rows past H_out its last row, so no load
// carries a condition; the buffer ranges cover exactly the band's rows and
// the tile's W rows.
__device__ __forceinline__ void gemm_tile(const uint16_t *__restrict__ x, const uint16_t *__restrict__ Wl,
                                          int32_t row0, int32_t rows, int32_t n0, int32_t H, int32_t H_out,
                                          uint16_t *__restrict__ y, uint8_t *lds)
{
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    // the tile is the same for every lane; saying so keeps the buffer
    // resources in scalar registers (no per-lane loop around each load)
    row0 = __builtin_amdgcn_readfirstlane(row0);
    rows = __builtin_amdgcn_readfirstlane(rows);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    const int ncols = min(kBN, H_out - n0);
    // fill mapping: lane L of an instruction writes row L / 4, position L % 4,
    // which holds chunk position ^ swz(row)
    const int lr = lane >> 2, gc = (lane & 3) ^ swz(lr);
    uint32_t aoff[kFillA], boff[kFillB];
#pragma unroll
    for (int i = 0; i < kFillA; ++i)
        aoff[i] = (uint32_t)min((i * 4 + wave) * 16 + lr, rows - 1) * (uint32_t)H * 2u + gc * 16;
#pragma unroll
    for (int i = 0; i < kFillB; ++i)
        boff[i] = (uint32_t)min((i * 4 + wave) * 16 + lr, ncols - 1) * (uint32_t)H * 2u + gc * 16;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x + (int64_t)row0 * H), 0, rows * H * 2, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(Wl + (int64_t)n0 * H), 0, ncols * H * 2, kBufferFlags);
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x16{};
    // fragment reads: row lane % 32 of each 32-row block, chunk 2 kk + lane / 32
    const int hi = lane >> 5, sw = swz(lane & 15);
    const int arow = (lane & 31) * kRowB, brow = (wave * 128 + (lane & 31)) * kRowB;
    const int koff[2] = {(hi ^ sw) << 4, ((2 + hi) ^ sw) << 4};
    const int nsteps = H / kBK;
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st)
        if (st < nsteps)
            fill_stage(lds + st * kStageBytes, ra, rb, st * kBK * 2, aoff, boff, wave);
    if (nsteps > 2)
        wait_vmem<kFill>();
    else
        wait_vmem<0>();
    __syncthreads();
    bf16x8 f0[8], f1[8];
    first_frags(lds, arow, brow, koff[0], f0);
    // top of step s > 0: stage s + 1 complete (only stage s + 2 may be in
    // flight), then a barrier so every wave's part of it is in LDS and every
    // wave is done with the stage the next fill overwrites
    auto top = [&](int st) {
        if (st == 0)
            return;
        if (st + 2 < nsteps)
            wait_vmem<kFill>();
        else
            wait_vmem<0>();
        asm volatile("s_barrier" ::: "memory");
    };
#define MOE_KSTEP(L, M)                                                                                   \
    kstep<L, M>(lds + (st % kStages) * kStageBytes, lds + ((st + 1) % kStages) * kStageBytes,           \
                lds + ((st + kStages - 1) % kStages) * kStageBytes, ra, rb, (st + kStages - 1) * kBK * 2, \
                aoff, boff, wave, arow, brow, koff, f0, f1, acc)
    int st = 0;
    for (; st + kStages - 1 < nsteps; ++st) {
        top(st);
        MOE_KSTEP(true, true);
    }
    for (; st + 1 < nsteps; ++st) {
        top(st);
        MOE_KSTEP(false, true);
    }
    top(st);
    MOE_KSTEP(false, false);
#undef MOE_KSTEP
    __syncthreads();  // every wave is done with the stages
    // epilogue: round to bf16, stage the tile in LDS, write 16-byte chunks of rows
    uint16_t *Cs = reinterpret_cast<uint16_t *>(lds);
    constexpr int kCStride = kCRowBytes / 2;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                // accumulator r holds row 8(r/4) + 4(lane/32) + r%4, column lane%32
                const int row = i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                const int col = wave * 128 + j * 32 + (lane & 31);
                const uint32_t p = pack_bf16x2(acc[i][j][r], acc[i][j][r + 1]);
                Cs[row * kCStride + col] = (uint16_t)(p & 0xFFFFu);
                Cs[(row + 1) * kCStride + col] = (uint16_t)(p >> 16);
            }
    __syncthreads();
#pragma unroll 8
    for (int i = 0; i < kBM * kBN / 8 / kThreads; ++i) {
        const int r = (tid >> 6) + 4 * i, chunk = tid & 63;
        if (r < rows && chunk * 8 < ncols)
            *reinterpret_cast<u32x4 *>(y + (int64_t)(row0 + r) * H_out + n0 + chunk * 8) =
                *reinterpret_cast<const u32x4 *>(lds + r * kCRowBytes + chunk * 16);
    }
    __syncthreads();  // the stage is free again before the next tile's loads land
}

// the bands [b0, b1) of one consumer task (remote-first source q)
__device__ __forceinline__ void task_bands(const LinearWs &ws, int32_t S, int32_t El,
                                           int32_t band_group, int32_t task, int32_t *b0,
                                           int32_t *b1)
{
    const int q = upper_index(ws.task_prefix, S, task);
    const int32_t q_band0 = ws.band_prefix[q * El], q_band1 = ws.band_prefix[(q + 1) * El];
    *b0 = q_band0 + (task - ws.task_prefix[q]) * band_group;
    *b1 = min(*b0 + band_group, q_band1);
}

// copy the rows of bands [b0, b1) -- consecutive rows of one source -- from y to ret
__device__ void return_rows(const LinearWs &ws, const int32_t *cnt, int32_t S, int32_t El,
                            int32_t self_rank, int32_t H_out, int32_t b0, int32_t b1,
                            const uint16_t *__restrict__ y, uint16_t *__restrict__ ret)
{
    const int32_t C16 = H_out / 8;
    const Band first = band_info(ws, cnt, S, El, self_rank, b0);
    const Band last = band_info(ws, cnt, S, El, self_rank, b1 - 1);
    const int64_t r0 = first.row0, r1 = (int64_t)last.row0 + last.rows;
    const int64_t n16 = (r1 - r0) * C16;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(y) + r0 * C16;
    u32x4 *dst = reinterpret_cast<u32x4 *>(ret) + r0 * C16;
    // whole chunks of 16 loads per thread (64 KiB per block), software-
    // pipelined: chunk c + 1 is loaded before chunk c is stored, so a wait for
    // a chunk's loads never includes the stores issued after them, and two
    // chunks (128 KiB per block) are in flight -- a copy by few blocks is
    // bound by bytes in flight over memory latency. No per-load condition,
    // which would make each load wait for the last. The registers are there
    // anyway: the kernel is sized for its GEMM.
    constexpr int kInFlight = 16;
    constexpr int64_t kChunk = (int64_t)kThreads * kInFlight;
    const int64_t full = n16 / kChunk * kChunk;
    u32x4 va[kInFlight], vb[kInFlight];
    auto load = [&](u32x4 (&v)[kInFlight], int64_t base) {
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            v[u] = load_stream(src + base + u * kThreads);
    };
    auto store = [&](const u32x4 (&v)[kInFlight], int64_t base) {
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            store_stream(dst + base + u * kThreads, v[u]);
    };
    int64_t base = threadIdx.x;
    if (base < full)
        load(va, base);
    while (base < full) {
        if (base + kChunk < full)
            load(vb, base + kChunk);
        store(va, base);
        base += kChunk;
        if (base >= full)
            break;
        if (base + kChunk < full)
            load(va, base + kChunk);
        store(vb, base);
        base += kChunk;
    }
    for (int64_t i = full + threadIdx.x; i < n16; i += kThreads)
        store_stream(dst + i, load_stream(src + i));
}

// tile order: each XCD (blockIdx % 8) takes runs of consecutive tile ids
__device__ __forceinline__ int64_t dealt_tile(int64_t step, int32_t slot, int32_t n_slots)
{
    const int32_t per_xcd = n_slots / 8;
    if (per_xcd == 0 || n_slots % 8 != 0)
        return step * n_slots + slot;
    return step * n_slots + (int64_t)(slot % 8) * per_xcd + slot / 8;
}

// signal: release-add each unit's column tiles to its band's count.
// inline_return: the unit that completes a band counts the band toward its
// task, and the unit that completes a task's last band copies the task's
// rows to ret itself (acquire-release counts; no block ever waits).
__device__ void produce(const uint16_t *__restrict__ x, const int32_t *__restrict__ cnt,
                        int32_t S, int32_t El, int32_t self_rank, int32_t H, int32_t H_out,
                        const uint16_t *__restrict__ W, uint16_t *__restrict__ y,
                        const LinearWs &ws, int32_t slot, int32_t n_slots, bool signal,
                        bool inline_return, int32_t band_group, uint16_t *__restrict__ ret,
                        int32_t *copy_task, uint8_t *lds)
{
    // a work unit is one band by one column tile; it is released once (one L2
    // write-back per 512 output columns)
    const int32_t nct = (H_out + kBN - 1) / kBN;
    const int64_t n_units = (int64_t)ws.counts[0] * nct;
    for (int64_t step = 0; step * n_slots < n_units; ++step) {
        const int64_t u = dealt_tile(step, slot, n_slots);
        if (u >= n_units)
            continue;
        const int32_t band = (int32_t)(u / nct), ct = (int32_t)(u % nct);
        const Band b = band_info(ws, cnt, S, El, self_rank, band);
        const int32_t l = __builtin_amdgcn_readfirstlane(b.l);  // the same in every lane
        gemm_tile(x, W + (int64_t)l * H_out * H, b.row0, b.rows, ct * kBN, H, H_out, y, lds);
        if (signal) {
            // each thread's stores complete to its L2 (a workgroup-scope release is
            // a wait, no cache maintenance); then one agent-scope release by thread 0
            // writes the L2 back once for the whole unit before the count moves
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __syncthreads();
            if (threadIdx.x == 0) {
                const int32_t add = 1;
                int32_t task = -1;
                if (!inline_return) {
                    __hip_atomic_fetch_add(ws.flags + band, add, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                } else if (__hip_atomic_fetch_add(ws.flags + band, add, __ATOMIC_RELEASE,
                                                  __HIP_MEMORY_SCOPE_AGENT) + add == nct) {
                    // this unit completed the band (its add read the final count):
                    // acquire the other units' releases, then count the band
                    // toward its task. Only band completions pay for the acquire.
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    const int rb = upper_index(ws.band_prefix, S * El, band);
                    const int q = rb / El;
                    const int32_t t = ws.task_prefix[q] + (band - ws.band_prefix[q * El]) / band_group;
                    int32_t b0, b1;
                    task_bands(ws, S, El, band_group, t, &b0, &b1);
                    if (__hip_atomic_fetch_add(ws.task_flags + t, 1, __ATOMIC_ACQ_REL,
                                               __HIP_MEMORY_SCOPE_AGENT) + 1 == b1 - b0)
                        task = t;
                }
                *copy_task = task;
            }
            __syncthreads();
            const int32_t task = *copy_task;
            __syncthreads();  // the word lives in the tile's LDS, which the next tile's loads reuse
            if (inline_return && task >= 0) {
                int32_t b0, b1;
                task_bands(ws, S, El, band_group, task, &b0, &b1);
                return_rows(ws, cnt, S, El, self_rank, H_out, b0, b1, y, ret);
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void expert_linear_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ cnt, int32_t S, int32_t El,
    int32_t self_rank, int32_t H, int32_t H_out, const uint16_t *__restrict__ W,
    uint16_t *__restrict__ y, int32_t *__restrict__ ws_base)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    const LinearWs ws = linear_ws(ws_base, S, El);
    produce(x, cnt, S, El, self_rank, H, H_out, W, y, ws, blockIdx.x, gridDim.x, false, false, 1,
            nullptr, nullptr, lds);
}

__global__ __launch_bounds__(kThreads) void expert_return_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ cnt, int32_t S, int32_t El,
    int32_t self_rank, int32_t H, int32_t H_out, const uint16_t *__restrict__ W,
    uint16_t *__restrict__ y, uint16_t *__restrict__ ret, int32_t band_group,
    int32_t consumers, int32_t *__restrict__ ws_base)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    // the block's broadcast word shares the first bytes of the tile memory:
    // it is written only between tiles (producers) or by blocks that run no
    // tile (consumers)
    int32_t &task_ok = *reinterpret_cast<int32_t *>(lds);
    const LinearWs ws = linear_ws(ws_base, S, El);
    const int32_t producers = (int32_t)gridDim.x - consumers;
    if ((int32_t)blockIdx.x < producers) {
        produce(x, cnt, S, El, self_rank, H, H_out, W, y, ws, blockIdx.x, producers, true,
                consumers == 0, band_group, ret, &task_ok, lds);
        return;
    }
    // consumer: tasks c, c + consumers, ... in remote-first order
    const int32_t nct = (H_out + kBN - 1) / kBN;
    const int32_t n_tasks = ws.counts[1];
    for (int32_t task = (int32_t)blockIdx.x - producers; task < n_tasks; task += consumers) {
        int32_t b0, b1;
        task_bands(ws, S, El, band_group, task, &b0, &b1);
        if (threadIdx.x == 0) {
            // poll with relaxed loads (they read the coherent copy without
            // invalidating any cache the producers rely on); acquire once, below
            int32_t ok = 1;
            for (int32_t band = b0; band < b1 && ok; ++band) {
                int spins = 0;
                while (__hip_atomic_load(ws.flags + band, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nct) {
                    if (++spins > kSpinLimit) {
                        ok = 0;
                        __hip_atomic_store(ws.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(8);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            task_ok = ok;
        }
        __syncthreads();
        if (task_ok)
            return_rows(ws, cnt, S, El, self_rank, H_out, b0, b1, y, ret);
        __syncthreads();  // task_ok is rewritten for the next task
    }
}

// resident blocks per device (occupancy x CUs) for each kernel, 0 = not yet asked
int g_linear_slots[64], g_return_slots[64];

hipError_t resident_blocks(const void *kernel, int *cache, int *slots)
{
    int dev;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 64 && cache[dev] > 0) {
        *slots = cache[dev];
        return hipSuccess;
    }
    int per_cu = 0, cus = 0;
    if ((err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0)) != hipSuccess)
        return err;
    if ((err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
        return err;
    *slots = per_cu * cus;
    if (dev < 64)
        cache[dev] = *slots;
    return hipSuccess;
}

}  // namespace

hipError_t expert_return_slots(int *slots)
{
    return resident_blocks(reinterpret_cast<const void *>(expert_return_kernel), g_return_slots, slots);
}

size_t expert_linear_workspace_bytes(int32_t S, int32_t El, int64_t max_rows)
{
    return (size_t)linear_ws_words(S, El, max_rows) * sizeof(int32_t);
}

hipError_t launch_expert_linear(const uint16_t *recv, const int32_t *cnt, int32_t S, int32_t El,
                                int32_t H, int32_t H_out, const uint16_t *W, int64_t max_rows,
                                uint16_t *y, int32_t *workspace, hipStream_t stream)
{
    hipLaunchKernelGGL(linear_table_kernel, dim3(1), dim3(kTableThreads), 0, stream, cnt, S, El,
                       S - 1, 1, max_rows, max_bands(S, El, max_rows), workspace);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || max_rows == 0)
        return err;
    int slots = 0;
    if ((err = resident_blocks(reinterpret_cast<const void *>(expert_linear_kernel), g_linear_slots,
                               &slots)) != hipSuccess)
        return err;
    const int64_t tiles = max_bands(S, El, max_rows) * ((H_out + kBN - 1) / kBN);
    const int grid = (int)(tiles < slots ? tiles : slots);
    hipLaunchKernelGGL(expert_linear_kernel, dim3(grid), dim3(kThreads), 0, stream, recv, cnt, S,
                       El, S - 1, H, H_out, W, y, workspace);
    return hipGetLastError();
}

hipError_t launch_expert_return(const uint16_t *recv, const int32_t *cnt, int32_t S, int32_t El,
                                int32_t H, int32_t H_out, const uint16_t *W, int64_t max_rows,
                                int32_t self_rank, int32_t consumers, int32_t band_group,
                                uint16_t *y, uint16_t *ret, int32_t *workspace,
                                hipStream_t stream, int32_t *grid_used)
{
    hipLaunchKernelGGL(linear_table_kernel, dim3(1), dim3(kTableThreads), 0, stream, cnt, S, El,
                       self_rank, band_group, max_rows, max_bands(S, El, max_rows), workspace);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || max_rows == 0)
        return err;
    int slots = 0;
    if ((err = resident_blocks(reinterpret_cast<const void *>(expert_return_kernel), g_return_slots,
                               &slots)) != hipSuccess)
        return err;
    if (consumers < 0 || consumers >= slots)
        return hipErrorInvalidValue;
    *grid_used = slots;
    void *args[] = {(void *)&recv, (void *)&cnt, (void *)&S, (void *)&El, (void *)&self_rank,
                    (void *)&H, (void *)&H_out, (void *)&W, (void *)&y, (void *)&ret,
                    (void *)&band_group, (void *)&consumers, (void *)&workspace};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(expert_return_kernel),
                                      dim3(slots), dim3(kThreads), args, 0, stream);
}

}  // namespace moe
