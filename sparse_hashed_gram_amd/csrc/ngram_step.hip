// Fused lazy sparse row-wise step and window export (gfx950).
//
// Adam with beta1 = 0 on the n-gram rows a window touched, one second-moment
// float per 768-wide row, beta2 applied retroactively when a row comes back
// (the @classiclarryd post quoted on the airebao.com item; modded-nanogpt
// README technique list: sparse row-wise embedding updates).  Per touched row
// r with window gradient G and optimizer step number t:
//     k = t - t_last[r];   v[r] = beta2^k v[r] + (1 - beta2) mean(G^2)
//     W[r] -= lr G / (sqrt(v[r]) + eps);   t_last[r] = t
// One wavefront per row: a lane holds 12 of the 768 values (three 16-byte G
// loads and three 8-byte bf16 loads, all coalesced), mean(G^2) is a butterfly
// sum over the wavefront (every lane ends with the same bits).  v and t_last
// of a row share one 8-byte record, so the row's optimizer state costs one
// small read and one small write; the window is emptied by advancing its
// epoch afterwards, not by touching the slot map.
#include <algorithm>

#include "ngram_dev.hpp"

#include "../../include/ngram.h"

namespace ngram {

namespace {

struct StepArgs {
    const uint32_t *slot_rows[2];
    const float *gacc;      // [2][wrows][768]
    int64_t wrows;
    uint8_t *w[2];
    RowState *st[2];
    WsHeader *hdr;
    StepParams p;
    const StepParams *p_dev;   // if set, the parameters are read from here
};

// Row state of one touched row while it is being stepped.
struct RowIn {
    uint32_t row;
    float4 g[3];
    float w[3][4];
    RowState s;
};

template <int ELT>
__device__ __forceinline__ void load_row(RowIn &r, const float *G, uint32_t slot, const uint8_t *W,
                                         const RowState *S, int lane)
{
    // every access here touches its row once: streaming (non-temporal) forms
    const uint64_t g4 = (uint64_t)(G + (size_t)slot * kDim) + 16 * lane;
#pragma unroll
    for (int q = 0; q < 3; ++q)
        r.g[q] = ld_global_nt<float4>(g4 + q * kWave * 16);
    if (ELT == 2) {
        const uint64_t wp = (uint64_t)(W + (size_t)r.row * kDim * 2) + 8 * lane;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const uint2 x = ld_global_nt<uint2>(wp + q * kWave * 8);
            r.w[q][0] = bf16_lo(x.x);
            r.w[q][1] = bf16_hi(x.x);
            r.w[q][2] = bf16_lo(x.y);
            r.w[q][3] = bf16_hi(x.y);
        }
    } else {
        const uint64_t wp = (uint64_t)(W + (size_t)r.row * kDim * 4) + 16 * lane;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const float4 x = ld_global_nt<float4>(wp + q * kWave * 16);
            r.w[q][0] = x.x;
            r.w[q][1] = x.y;
            r.w[q][2] = x.z;
            r.w[q][3] = x.w;
        }
    }
    r.s = ld_global_nt<RowState>((uint64_t)(S + r.row));
}

template <int ELT>
__device__ __forceinline__ void step_row(RowIn &r, const StepArgs &a, const StepParams &sp, uint8_t *W,
                                         RowState *S, int lane)
{
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < 3; ++q)
        ss += r.g[q].x * r.g[q].x + r.g[q].y * r.g[q].y + r.g[q].z * r.g[q].z + r.g[q].w * r.g[q].w;
    ss = wave_sum(ss);
    float vn;
    bool order_bad;
    const float scale = step_scale(ss, r.s, sp, vn, order_bad);
    if (order_bad && lane == 0)
        atomicOr(&a.hdr->flags, NGRAM_FLAG_STEP_ORDER);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        r.w[q][0] -= scale * r.g[q].x;
        r.w[q][1] -= scale * r.g[q].y;
        r.w[q][2] -= scale * r.g[q].z;
        r.w[q][3] -= scale * r.g[q].w;
    }
    if (ELT == 2) {
        const uint64_t wp = (uint64_t)(W + (size_t)r.row * kDim * 2) + 8 * lane;
#pragma unroll
        for (int q = 0; q < 3; ++q)
            st_global_nt<uint2>(wp + q * kWave * 8,
                                make_uint2(bf16_pack(r.w[q][0], r.w[q][1]), bf16_pack(r.w[q][2], r.w[q][3])));
    } else {
        const uint64_t wp = (uint64_t)(W + (size_t)r.row * kDim * 4) + 16 * lane;
#pragma unroll
        for (int q = 0; q < 3; ++q)
            st_global_nt<float4>(wp + q * kWave * 16, make_float4(r.w[q][0], r.w[q][1], r.w[q][2], r.w[q][3]));
    }
    if (lane == 0)
        S[r.row] = RowState{vn, sp.t};
}

// Each wavefront takes 64 consecutive window slots at a time (one coalesced
// load of their row ids), then steps them two rows per iteration with both
// rows' loads in flight together.  Slots whose row was already stepped by
// the fused reduction (kSlotStepped) are skipped.
constexpr int kStepRows = 2;
template <int ELT>
__global__ __launch_bounds__(256) void step_kernel(StepArgs a)
{
    const int c = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wid = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
    const uint32_t nwaves = gridDim.x * (256 / kWave);
    const uint32_t n = a.hdr->n_slots[c];
    const uint32_t *rows = a.slot_rows[c];
    const float *G = a.gacc + (size_t)c * a.wrows * kDim;
    uint8_t *W = a.w[c];
    RowState *S = a.st[c];
    bool sp_ok;
    const StepParams sp = step_params(a.p, a.p_dev, sp_ok);
    if (!sp_ok && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
        atomicOr(&a.hdr->flags, NGRAM_FLAG_BAD_PARAMS);
    const bool live_window = sp_ok && !a.hdr->dropped;

    for (uint32_t base = wid * kWave; live_window && base < n; base += nwaves * kWave) {
        const uint32_t cnt = min((uint32_t)kWave, n - base);
        const uint32_t my_row = lane < (int)cnt ? rows[base + lane] : 0u;
        for (uint32_t u = 0; u < cnt; u += kStepRows) {
            RowIn r[kStepRows];
            bool live[kStepRows];
#pragma unroll
            for (int k = 0; k < kStepRows; ++k) {
                live[k] = false;
                if (u + k < cnt) {
                    r[k].row = (uint32_t)__builtin_amdgcn_readlane((int)my_row, (int)(u + k));
                    live[k] = !(r[k].row & kSlotStepped);
                    if (live[k])
                        load_row<ELT>(r[k], G, base + u + k, W, S, lane);
                }
            }
#pragma unroll
            for (int k = 0; k < kStepRows; ++k)
                if (live[k])
                    step_row<ELT>(r[k], a, sp, W, S, lane);
        }
    }
}

// Ends the window: the epoch advances, so every slot-map entry goes stale, and
// the window's and the burst stash's counts return to 0.
__global__ void window_clear_kernel(WsHeader *__restrict__ hdr)
{
    hdr->epoch += 1;
    hdr->n_slots[0] = 0;
    hdr->n_slots[1] = 0;
    hdr->n_next[0] = 0;
    hdr->n_next[1] = 0;
    hdr->n_stash = 0;
    hdr->n_micro = 0;
    hdr->n_keyed = 0;
    hdr->sorted_n = 0;
    hdr->dropped = 0;
}

__global__ void export_kernel(const WsHeader *__restrict__ hdr, int c, const uint32_t *__restrict__ slot_rows,
                              const float *__restrict__ G, uint32_t *__restrict__ rows_out,
                              float *__restrict__ g_out, uint32_t max_rows, uint32_t *__restrict__ count)
{
    const uint32_t total = hdr->n_slots[c];
    const uint32_t n = min(total, max_rows);
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t nthr = (uint64_t)gridDim.x * blockDim.x;
    if (tid == 0)
        *count = total;
    for (uint64_t i = tid; i < n; i += nthr)
        rows_out[i] = slot_rows[i] & ~kSlotStepped;
    if (g_out) {
        const float4 *src = reinterpret_cast<const float4 *>(G);
        float4 *dst = reinterpret_cast<float4 *>(g_out);
        for (uint64_t i = tid; i < (uint64_t)n * (kDim / 4); i += nthr)
            dst[i] = src[i];
    }
}

// ------------------------------------------------------------ touched rows
//
// The distinct rows of one channel that the current window touches, in
// ascending order: one bit per table row is set for every row the window
// accumulator holds (its slot rows) and for every key kept in the burst
// stash but not reduced yet, then the set bits are compacted in row order.
// No sort: the bit array is the order.

constexpr int kTouchThreads = 256;
constexpr int kTouchWords = 32;   // consecutive bit words per thread
constexpr int kTouchBlockWords = kTouchThreads * kTouchWords;

__global__ void touched_clear_kernel(uint32_t *__restrict__ bits, uint64_t nwords)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords;
         i += (uint64_t)gridDim.x * blockDim.x)
        bits[i] = 0u;
}

// Grid-stride over the window's slot rows (the first n_slots of slot_rows)
// and, in burst modes, the stash's packed indices of this channel (the first
// n_stash); both counts are read here and bounded by the host's capacities.
__global__ void touched_mark_kernel(const WsHeader *__restrict__ hdr, int c, const uint32_t *__restrict__ slot_rows,
                                    uint32_t slot_cap, const uint32_t *__restrict__ sidx, uint32_t stash_cap,
                                    uint32_t *__restrict__ bits)
{
    const uint32_t ns = min(hdr->n_slots[c], slot_cap);
    const uint32_t nst = sidx ? min(hdr->n_stash, stash_cap) : 0u;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (uint64_t)ns + nst; i += stride) {
        const uint32_t r = i < ns ? (slot_rows[i] & ~kSlotStepped) : (sidx[i - ns] & 0x7FFFFFFFu);
        atomicOr(&bits[r >> 5], 1u << (r & 31u));
    }
}

// Set bits per block of kTouchBlockWords words.
__global__ __launch_bounds__(kTouchThreads) void touched_count_kernel(const uint32_t *__restrict__ bits,
                                                                      uint64_t nwords, uint32_t *__restrict__ blk)
{
    __shared__ uint32_t s_wave[kTouchThreads / kWave];
    const uint64_t w0 = (uint64_t)blockIdx.x * kTouchBlockWords + (uint64_t)threadIdx.x * kTouchWords;
    uint32_t cnt = 0;
    for (int j = 0; j < kTouchWords; ++j)
        cnt += w0 + j < nwords ? (uint32_t)__popc(bits[w0 + j]) : 0u;
    uint32_t total;
    block_excl_scan<kTouchThreads>(cnt, s_wave, &total);
    if (threadIdx.x == 0)
        blk[blockIdx.x] = total;
}

// Writes the rows of the set bits in ascending order (the first max_rows of
// them) and the number of touched rows to *count.
__global__ __launch_bounds__(kTouchThreads) void touched_write_kernel(const uint32_t *__restrict__ bits,
                                                                      uint64_t nwords,
                                                                      const uint32_t *__restrict__ blk,
                                                                      uint32_t nblk, int32_t *__restrict__ rows,
                                                                      uint64_t max_rows, int64_t *__restrict__ count)
{
    __shared__ uint32_t s_wave[kTouchThreads / kWave];
    const uint32_t b = blockIdx.x;
    uint32_t part = 0, part_before = 0;
    for (uint32_t k = threadIdx.x; k < nblk; k += kTouchThreads) {
        const uint32_t x = blk[k];
        part += x;
        part_before += k < b ? x : 0u;
    }
    uint32_t before, all;
    block_excl_scan<kTouchThreads>(part_before, s_wave, &before);
    block_excl_scan<kTouchThreads>(part, s_wave, &all);
    if (b == 0 && threadIdx.x == 0)
        *count = (int64_t)all;
    const uint64_t w0 = (uint64_t)b * kTouchBlockWords + (uint64_t)threadIdx.x * kTouchWords;
    uint32_t cnt = 0;
    for (int j = 0; j < kTouchWords; ++j)
        cnt += w0 + j < nwords ? (uint32_t)__popc(bits[w0 + j]) : 0u;
    uint64_t o = (uint64_t)before + block_excl_scan<kTouchThreads>(cnt, s_wave, nullptr);
    for (int j = 0; j < kTouchWords && w0 + j < nwords; ++j) {
        uint32_t m = bits[w0 + j];
        while (m) {
            const int bit = __builtin_ctz(m);
            m &= m - 1u;
            if (o < max_rows)
                rows[o] = (int32_t)(((w0 + j) << 5) + bit);
            ++o;
        }
    }
}

__global__ void touched_none_kernel(int64_t *__restrict__ count) { *count = 0; }

}  // namespace

hipError_t launch_touched(const WsLayout &L, uint8_t *ws, int c, int32_t *rows, uint64_t max_rows, int64_t *count,
                          hipStream_t s)
{
    const WsHeader *hdr = reinterpret_cast<const WsHeader *>(ws + L.hdr);
    uint32_t *bits = reinterpret_cast<uint32_t *>(ws + L.tbits[c]);
    uint32_t *blk = reinterpret_cast<uint32_t *>(ws + L.tblk);
    const uint64_t nwords = ((uint64_t)L.rows[c] + 31) / 32;
    const uint32_t nblk = (uint32_t)((nwords + kTouchBlockWords - 1) / kTouchBlockWords);
    touched_clear_kernel<<<(unsigned)std::min<uint64_t>((nwords + 255) / 256, 4096), 256, 0, s>>>(bits, nwords);
    const uint32_t slot_cap = (uint32_t)L.wrows;
    const uint32_t stash_cap = L.burst ? (uint32_t)L.nk : 0u;
    const uint32_t *sidx = L.burst ? reinterpret_cast<const uint32_t *>(ws + L.stash_idx) + (size_t)c * L.nk : nullptr;
    const uint64_t items = (uint64_t)slot_cap + stash_cap;
    touched_mark_kernel<<<(unsigned)std::min<uint64_t>((items + 255) / 256, 8192), 256, 0, s>>>(
        hdr, c, reinterpret_cast<const uint32_t *>(ws + L.slot_rows[c]), slot_cap, sidx, stash_cap, bits);
    touched_count_kernel<<<nblk, kTouchThreads, 0, s>>>(bits, nwords, blk);
    touched_write_kernel<<<nblk, kTouchThreads, 0, s>>>(bits, nwords, blk, nblk, rows, max_rows, count);
    return hipGetLastError();
}

hipError_t launch_touched_none(int64_t *count, hipStream_t s)
{
    touched_none_kernel<<<1, 1, 0, s>>>(count);
    return hipGetLastError();
}

hipError_t launch_step(const WsLayout &L, uint8_t *ws, const FuseArgs &f, hipStream_t s)
{
    StepArgs a;
    for (int c = 0; c < 2; ++c)
        a.slot_rows[c] = reinterpret_cast<const uint32_t *>(ws + L.slot_rows[c]);
    a.gacc = reinterpret_cast<const float *>(ws + L.gacc);
    a.wrows = L.wrows;
    a.w[0] = f.w[0];
    a.w[1] = f.w[1];
    a.st[0] = f.st[0];
    a.st[1] = f.st[1];
    a.hdr = reinterpret_cast<WsHeader *>(ws + L.hdr);
    a.p = f.p;
    a.p_dev = f.p_dev;
    const int dtype = f.dtype;
    // about one resident wavefront per SIMD slot; each walks 64-slot blocks
    const int64_t want = (L.wrows + 255) / 256;
    const unsigned gx = (unsigned)(want < 1024 ? (want > 0 ? want : 1) : 1024);
    launch_prof(NGRAM_PROF_STEP, true, false, dtype == NGRAM_DTYPE_BF16 ? step_kernel<2> : step_kernel<4>,
                dim3(gx, L.nch), dim3(256), 0, s, a);
    launch_prof(NGRAM_PROF_STEP, false, true, window_clear_kernel, dim3(1), dim3(1), 0, s, a.hdr);
    return hipGetLastError();
}

hipError_t launch_export(const WsLayout &L, const uint8_t *ws, int channel, uint32_t *rows, float *G,
                         uint32_t max_rows, uint32_t *count, hipStream_t s)
{
    const WsHeader *hdr = reinterpret_cast<const WsHeader *>(ws + L.hdr);
    const float *src = reinterpret_cast<const float *>(ws + L.gacc) + (size_t)channel * L.wrows * kDim;
    export_kernel<<<1024, 256, 0, s>>>(hdr, channel,
                                       reinterpret_cast<const uint32_t *>(ws + L.slot_rows[channel]), src,
                                       rows, G, max_rows, count);
    return hipGetLastError();
}

}  // namespace ngram
