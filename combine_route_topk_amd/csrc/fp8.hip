// fp8.hip -- FP8 dispatch payload: quantise inside the dispatch permute,
// and decode rows back to bf16 on the receiving side.
//
// Method: aicassindra "gpu_moe_all_to_all", "Latency-bound at decode,
// bandwidth-bound at prefill" (send fewer bytes: a lower-precision dispatch
// payload, since the expert matmul casts its input anyway) and "Bucketing"
// (the permutation fused into the kernel that stages the sends); zenaique
// Q&A "moe-hide-alltoall-techniques" (shrink the payload).
//
// Format (the pages leave it open): OCP E4M3 codes, and per 32 consecutive
// values along H one power-of-two scale 2^e stored as the byte e + 127 (the
// E8M0 scale of the OCP microscaling formats, which gfx950's scaled MFMA
// reads). e is the smallest integer >= -127 with max|x| <= 448 * 2^e, so no
// code saturates, and x * 2^-e is exact in float32: the hardware convert
// (round to nearest even) then yields the nearest E4M3 code.
//
// Row layout: H code bytes, then one 128-byte line per 4096 values holding
// that slab's 128 scale bytes (zero-padded in the last slab). For H a
// multiple of 128 every row starts on a 128-byte line, and every line of a
// send row is written whole by one store instruction. Rows that share a line,
// or lines written in pieces, cost a read-modify-write in the memory system:
// on MI355X unaligned 7392-byte rows took 84 us where 7424-byte rows took
// 62 us (32768 rows), and 16-byte pieces of scale bytes added about 35 us at
// 327680 rows. A destination's segment stays one contiguous range.
//
// permute_fp8_kernel: block (token, 4096-value slab), 16 values per lane
// (two 16-byte loads, one 16-byte code store). A quantisation block is two
// neighbouring lanes (one DPP swap for their maximum). Four scale bytes are
// packed per 8 lanes with ds_bpermute, collected in LDS, and the slab's
// 128-byte scale line leaves as eight 16-byte stores per kept replica.
// For k >= 4 each block also loads (and discards) its slab of token
// t + kPrefetchTokens, so that the block reading it later finds it in a
// cache, as the bf16 permute does (its header gives the measurements).
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kRowThreads = 256;
constexpr int kSlabValues = kRowThreads * 16;   // 4096 values per block
constexpr int kScaleLine = kSlabValues / 32;    // 128 scale bytes per slab
constexpr int64_t kPrefetchTokens = 4096;       // a multiple of 8: the reader's XCD
constexpr int32_t kPrefetchMinK = 4;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// largest |bf16| bit pattern (sign cleared) of the 8 values in v
__device__ __forceinline__ uint32_t max_abs_bits(u32x4 v)
{
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        m = max(m, max(v[i] & 0x7FFFu, (v[i] >> 16) & 0x7FFFu));
    return m;
}

// smallest e >= -127 with a <= 448 * 2^e, from the bit pattern of a = |x|
// (finite): a = 1.m * 2^(be - 127) fits 448 * 2^e = 1.75 * 2^(e + 8) when
// e = be - 135, or needs one more when the mantissa exceeds 0.75 (0x60/128)
__device__ __forceinline__ int32_t block_exponent(uint32_t abits)
{
    const int32_t be = (int32_t)(abits >> 7);
    return max(-127, be - 135 + ((abits & 0x7Fu) > 0x60u ? 1 : 0));
}

// 8 bf16 values * 2^-e -> 8 E4M3 codes (round to nearest even)
__device__ __forceinline__ u32x2 encode8(u32x4 v, float mul)
{
    u32x2 out;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t a = v[2 * i], b = v[2 * i + 1];
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(a) * mul, bf16_hi(a) * mul, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(b) * mul, bf16_hi(b) * mul, w, true);
        out[i] = (uint32_t)w;
    }
    return out;
}

// T tokens in this launch; x and pos extend n_ahead tokens further (rows a
// prefetch may touch); pf_dist: the prefetch distance in tokens, 0 for none
__global__ __launch_bounds__(kRowThreads) void permute_fp8_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ pos, int64_t T, int64_t n_ahead,
    int64_t pf_dist, int32_t C32, int32_t k, uint8_t *__restrict__ send, int64_t send_rows,
    int64_t row_bytes)
{
    __shared__ u32x4 line[kScaleLine / 16];
    const int64_t t = blockIdx.x;
    const int32_t c = blockIdx.y * kRowThreads + threadIdx.x;
    const int32_t *pr = pos + t * k;
    // lanes past the row act on zeros: their scale byte is 0, the padding
    const bool active = c < C32;
    // prefetch of token t + pf_dist's slab, if that token keeps a replica
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t tf = t + pf_dist;
    const bool ahead = pf_dist > 0 && tf < T + n_ahead;  // uniform across the block
    const int32_t pf = ahead && lane < k ? pos[tf * k + lane] : -1;
    u32x4 warm0 = {0u, 0u, 0u, 0u}, warm1 = warm0;
    if (ahead && ballot64(pf >= 0 && pf < send_rows) != 0 && active) {
        warm0 = x[(tf * C32 + c) * 2];
        warm1 = x[(tf * C32 + c) * 2 + 1];
    }
    bool any = false;
    for (int j = 0; j < k; ++j) {
        const int32_t p = pr[j];
        any |= p >= 0 && p < send_rows;
    }
    if (!any) {  // the same for the whole block: no thread reaches the barrier
        // the prefetched values are not needed; this keeps their loads
        asm volatile("" ::"v"(warm0[0]), "v"(warm0[1]), "v"(warm0[2]), "v"(warm0[3]),
                     "v"(warm1[0]), "v"(warm1[1]), "v"(warm1[2]), "v"(warm1[3]));
        return;
    }
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = v0;
    if (active) {
        v0 = x[(t * C32 + c) * 2];
        v1 = x[(t * C32 + c) * 2 + 1];
    }
    uint32_t m = max(max_abs_bits(v0), max_abs_bits(v1));
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, true));  // pair swap
    const int32_t e = block_exponent(m);
    const float mul = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, e in [-127, 120]
    const u32x2 a = encode8(v0, mul), b = encode8(v1, mul);
    const u32x4 codes = {a[0], a[1], b[0], b[1]};
    // lane 8i packs the scale bytes of quantisation blocks 4i..4i+3
    const uint32_t sbyte = (uint32_t)(e + 127);
    const int src = (lane + 2) << 2;
    const uint32_t b1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)sbyte);
    const uint32_t b2 = (uint32_t)__builtin_amdgcn_ds_bpermute(src + 8, (int)sbyte);
    const uint32_t b3 = (uint32_t)__builtin_amdgcn_ds_bpermute(src + 16, (int)sbyte);
    if ((threadIdx.x & 7) == 0)
        reinterpret_cast<uint32_t *>(line)[threadIdx.x / 8] = sbyte | (b1 << 8) | (b2 << 16) | (b3 << 24);
    __syncthreads();
    const bool line_lane = threadIdx.x < kScaleLine / 16;
    const u32x4 scales = line_lane ? line[threadIdx.x] : codes;
    const int64_t H = (int64_t)C32 * 16;
    for (int j = 0; j < k; ++j) {
        const int32_t p = pr[j];
        if (p < 0 || p >= send_rows)
            continue;
        uint8_t *row = send + (int64_t)p * row_bytes;
        if (active)
            store_stream(reinterpret_cast<u32x4 *>(row) + c, codes);
        if (line_lane)
            store_stream(reinterpret_cast<u32x4 *>(row + H + (int64_t)kScaleLine * blockIdx.y) +
                             threadIdx.x,
                         scales);
    }
    asm volatile("" ::"v"(warm0[0]), "v"(warm0[1]), "v"(warm0[2]), "v"(warm0[3]), "v"(warm1[0]),
                 "v"(warm1[1]), "v"(warm1[2]), "v"(warm1[3]));
}

// out[i] = bf16(value(code) * 2^(scale - 127)) for rows i < min(*n_rows, max_rows)
__global__ __launch_bounds__(kRowThreads) void fp8_dequant_kernel(
    const uint8_t *__restrict__ rows, const int32_t *__restrict__ n_rows, int64_t max_rows,
    int32_t C16, int64_t row_bytes, u32x4 *__restrict__ out)
{
    const int32_t c = blockIdx.y * kRowThreads + threadIdx.x;
    const int64_t N = n_rows ? min((int64_t)*n_rows, max_rows) : max_rows;
    if (c >= C16)
        return;
    const int64_t H = (int64_t)C16 * 8;
    for (int64_t i = blockIdx.x; i < N; i += gridDim.x) {
        const uint8_t *row = rows + i * row_bytes;
        const u32x2 codes = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(row) + c);
        const int32_t e = (int32_t)row[H + c / 4] - 127;
        u32x4 o;
        // exact: a code has 4 significant bits and the product stays inside
        // float32's range, down to its subnormals
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[q], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[q], true);
            o[2 * q] = pack_bf16x2(__builtin_amdgcn_ldexpf(lo[0], e), __builtin_amdgcn_ldexpf(lo[1], e));
            o[2 * q + 1] = pack_bf16x2(__builtin_amdgcn_ldexpf(hi[0], e), __builtin_amdgcn_ldexpf(hi[1], e));
        }
        store_stream(out + i * C16 + c, o);
    }
}


}  // namespace

int64_t fp8_row_bytes(int32_t H)
{
    return (int64_t)H + (int64_t)kScaleLine * ((H + kSlabValues - 1) / kSlabValues);
}

hipError_t launch_dispatch_permute_fp8(const uint16_t *x, const int32_t *pos, int64_t T,
                                       int32_t H, int32_t k, uint8_t *send, int64_t send_rows,
                                       hipStream_t stream)
{
    const int32_t C32 = H / 16;
    const int64_t pf_dist = k >= kPrefetchMinK ? kPrefetchTokens : 0;
    // one block per token; past kMaxRowBlocks tokens, one launch per chunk
    for (int64_t t0 = 0; t0 < T; t0 += kMaxRowBlocks) {
        const int64_t n = T - t0 < kMaxRowBlocks ? T - t0 : kMaxRowBlocks;
        const dim3 grid((unsigned)n, (unsigned)((H + kSlabValues - 1) / kSlabValues));
        hipLaunchKernelGGL(permute_fp8_kernel, grid, dim3(kRowThreads), 0, stream,
                           reinterpret_cast<const u32x4 *>(x) + t0 * C32 * 2, pos + t0 * k, n,
                           T - t0 - n, pf_dist, C32, k, send, send_rows, fp8_row_bytes(H));
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

hipError_t launch_fp8_dequant(const uint8_t *rows, const int32_t *n_rows, int64_t max_rows,
                              int32_t H, uint16_t *out, hipStream_t stream)
{
    if (max_rows == 0)
        return hipSuccess;
    const int32_t C16 = H / 8;
    const dim3 grid((unsigned)(max_rows < kMaxRowBlocks ? max_rows : kMaxRowBlocks),
                    (unsigned)((C16 + kRowThreads - 1) / kRowThreads));
    hipLaunchKernelGGL(fp8_dequant_kernel, grid, dim3(kRowThreads), 0, stream, rows, n_rows,
                       max_rows, C16, fp8_row_bytes(H), reinterpret_cast<u32x4 *>(out));
    return hipGetLastError();
}

}  // namespace moe
