// Backward of the hashed n-gram table: sort, dedupe, window slots and the
// signed segment reduction (gfx950).
//
// Only rows that occur in the batch receive a gradient and an optimizer step,
// and gradients are accumulated over 4 steps before the update (the
// @classiclarryd post quoted on the airebao.com item; modded-nanogpt README,
// technique list).  For one micro-step (spread mode) or one whole window
// (burst mode) this file computes, per channel and per distinct row r,
//     S[r] = sum over positions i hashed to r, in position order, of s_i dY[i]
// and adds it to the window accumulator G[slot(r)].
//
// Pipeline per call, both channels in every launch (blockIdx.y = channel):
//   1. LSD radix sort of (row, position|sign) pairs, 8-bit digits.  Each pass
//      is a per-tile LDS histogram, one digit-major scan, and a stable
//      scatter: ranks within a tile come from wavefront ballots (64-lane
//      match of the digit), the tile is reordered in LDS, then written out in
//      digit runs so global writes stay contiguous.
//   2. Segment heads; rows new to the window get the next slots in ascending
//      row order (tile counts, one scan, tile-local prefix: no atomics, so the
//      slot layout is deterministic).
//   3. Segment reduction: one wavefront per 64 sorted keys.  A lane holds 12
//      floats of a 768-wide row; each key costs three coalesced 1 KB loads of
//      dY.  A segment that ends in the chunk is written straight to G; one that
//      spills into the next chunk only is finished by the chunk where it
//      starts; longer ones (hot n-grams: thousands of keys) leave one partial
//      row per chunk, which a 16-wavefront block sums in a fixed order.
//      Every sum therefore has a fixed association and results are bitwise
//      reproducible; there are no floating-point atomics.
#include "ngram_dev.hpp"

#include "../../include/ngram.h"

namespace ngram {

namespace {

__device__ __forceinline__ uint32_t count_of(const uint32_t *n_dev, uint32_t n_host)
{
    return n_dev ? min(*n_dev, n_host) : n_host;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t o = __shfl_up(v, d);
        if (lane >= d)
            v += o;
    }
    return v;
}

// Exclusive scan over a block of NT threads; *total (if given) gets the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *s_wave, uint32_t *total)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const uint32_t inc = wave_incl_scan(v);
    if (lane == kWave - 1)
        s_wave[w] = inc;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) {
        const uint32_t x = s_wave[i];
        off += (i < w) ? x : 0u;
        tot += x;
    }
    __syncthreads();
    if (total)
        *total = tot;
    return off + inc - v;
}

// ------------------------------------------------------------ radix sort
//
// Tiles of 2048 keys (256 threads x 8).  Per pass: per-tile digit counts
// (hist[c][d][tile], digit-major), then one block per (digit, channel) turns
// its row of tile counts into exclusive tile offsets and a digit total, then
// the scatter adds the exclusive scan of the digit totals (done per block in
// LDS) to get each tile's global digit offsets.

// Key build for one tile, fused with the first pass's digit counts.  Spread:
// position i of the micro-step is hashed from the tokens.  Burst: every
// position kept in the stash, whose packed indices were hashed when kept.
// Also clears the fix-up record counts of the reduce that follows.
template <bool FROM_STASH>
__global__ __launch_bounds__(kSortThreads) void keys_tile_kernel(
    const int32_t *__restrict__ tok, const uint32_t *__restrict__ sidx, const uint32_t *__restrict__ spos,
    HashParams hp, uint32_t n_host, uint32_t *__restrict__ keys, uint32_t *__restrict__ vals, int64_t nk,
    uint32_t *__restrict__ hist, uint32_t nblk, WsHeader *__restrict__ hdr)
{
    __shared__ uint32_t h[2][kRadix];
    const int tid = threadIdx.x;
    const uint32_t b = blockIdx.x;
    const uint32_t n = FROM_STASH ? min(hdr->n_stash, n_host) : n_host;
    if (b == 0 && tid == 0) {
        hdr->n_owner[0] = 0;
        hdr->n_owner[1] = 0;
    }
    h[0][tid] = 0;
    h[1][tid] = 0;
    __syncthreads();
    const uint32_t base = b * kSortTile;
    bool bad = false;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t i = base + j * kSortThreads + tid;
        if (i < n) {
            uint32_t ib, it, pos = i;
            if (FROM_STASH) {
                ib = sidx[i];
                it = sidx[nk + i];
                pos = spos[i];
            } else {
                bad |= ngram_index(tok, i, hp, ib, it);
            }
            keys[i] = ib & 0x7FFFFFFFu;
            vals[i] = pos | (ib & 0x80000000u);
            keys[nk + i] = it & 0x7FFFFFFFu;
            vals[nk + i] = pos | (it & 0x80000000u);
            atomicAdd(&h[0][ib & (kRadix - 1)], 1u);
            atomicAdd(&h[1][it & (kRadix - 1)], 1u);
        }
    }
    if (bad)
        atomicOr(&hdr->flags, NGRAM_FLAG_BAD_TOKEN);
    __syncthreads();
    hist[((size_t)0 * kRadix + tid) * nblk + b] = h[0][tid];
    hist[((size_t)1 * kRadix + tid) * nblk + b] = h[1][tid];
}

__global__ __launch_bounds__(kSortThreads) void radix_hist_kernel(
    const uint32_t *__restrict__ keys, int64_t nk, const uint32_t *n_dev, uint32_t n_host, int shift,
    uint32_t *__restrict__ hist, uint32_t nblk)
{
    __shared__ uint32_t h[kRadix];
    const int c = blockIdx.y;
    const uint32_t b = blockIdx.x;
    const int tid = threadIdx.x;
    const uint32_t n = count_of(n_dev, n_host);
    h[tid] = 0;
    __syncthreads();
    const uint32_t *k = keys + (size_t)c * nk;
    const uint32_t base = b * kSortTile;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t i = base + j * kSortThreads + tid;
        if (i < n)
            atomicAdd(&h[(k[i] >> shift) & (kRadix - 1)], 1u);
    }
    __syncthreads();
    hist[((size_t)c * kRadix + tid) * nblk + b] = h[tid];
}

// Block (d, c): exclusive scan of digit d's tile counts in place, total to
// tot[c][d].  Each thread owns a contiguous run of tiles.
__global__ __launch_bounds__(kSortThreads) void scan_digits_kernel(uint32_t *__restrict__ hist, uint32_t nblk,
                                                                   uint32_t *__restrict__ tot)
{
    __shared__ uint32_t s_wave[kSortThreads / kWave];
    const int d = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
    uint32_t *row = hist + ((size_t)c * kRadix + d) * nblk;
    const uint32_t per = (nblk + kSortThreads - 1) / kSortThreads;
    const uint32_t lo = min(tid * per, nblk), hi = min(lo + per, nblk);
    uint32_t sum = 0;
    for (uint32_t j = lo; j < hi; ++j)
        sum += row[j];
    uint32_t total;
    uint32_t run = block_excl_scan<kSortThreads>(sum, s_wave, &total);
    for (uint32_t j = lo; j < hi; ++j) {
        const uint32_t x = row[j];
        row[j] = run;
        run += x;
    }
    if (tid == 0)
        tot[c * kRadix + d] = total;
}

// Stable scatter of one tile by the current digit.  Wave w owns tile keys
// [w*512, w*512+512), processed 64 at a time in index order.
__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(
    const uint32_t *__restrict__ kin, const uint32_t *__restrict__ vin, uint32_t *__restrict__ kout,
    uint32_t *__restrict__ vout, int64_t nk, const uint32_t *n_dev, uint32_t n_host, int shift,
    const uint32_t *__restrict__ hist, const uint32_t *__restrict__ tot, uint32_t nblk)
{
    constexpr int kPerWave = kSortTile / (kSortThreads / kWave);
    __shared__ uint32_t s_cnt[kSortThreads / kWave][kRadix];
    __shared__ uint32_t s_tile[kRadix];
    __shared__ uint32_t s_glob[kRadix];
    __shared__ uint32_t s_k[kSortTile];
    __shared__ uint32_t s_v[kSortTile];
    __shared__ uint32_t s_wave[kSortThreads / kWave];

    const int c = blockIdx.y;
    const uint32_t b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const uint32_t n = count_of(n_dev, n_host);
    const uint32_t base = b * kSortTile;
    if (base >= n)
        return;
    const uint32_t *ki = kin + (size_t)c * nk;
    const uint32_t *vi = vin + (size_t)c * nk;

    for (int r = tid; r < (kSortThreads / kWave) * kRadix; r += kSortThreads)
        (&s_cnt[0][0])[r] = 0;
    {
        const uint32_t digit_base = block_excl_scan<kSortThreads>(tot[c * kRadix + tid], s_wave, nullptr);
        s_glob[tid] = digit_base + hist[((size_t)c * kRadix + tid) * nblk + b];
    }
    __syncthreads();

    uint32_t key[kSortItems], val[kSortItems], rank[kSortItems];
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t i = base + w * kPerWave + j * kWave + lane;
        const bool ok = i < n;
        key[j] = ok ? ki[i] : 0u;
        val[j] = ok ? vi[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const bool ok = base + w * kPerWave + j * kWave + lane < n;
        const uint32_t d = (key[j] >> shift) & (kRadix - 1);
        uint64_t m = __ballot(ok);
#pragma unroll
        for (int bit = 0; bit < kRadixBits; ++bit) {
            const bool on = (d >> bit) & 1u;
            const uint64_t bb = __ballot(on);
            m &= on ? bb : ~bb;
        }
        const uint32_t before = s_cnt[w][d];
        if (ok && lane == 63 - __clzll(m))
            s_cnt[w][d] = before + (uint32_t)__popcll(m);
        rank[j] = before + (uint32_t)__popcll(m & below);
    }
    __syncthreads();
    {
        uint32_t run = 0;
#pragma unroll
        for (int ww = 0; ww < kSortThreads / kWave; ++ww) {
            const uint32_t x = s_cnt[ww][tid];
            s_cnt[ww][tid] = run;
            run += x;
        }
        s_tile[tid] = block_excl_scan<kSortThreads>(run, s_wave, nullptr);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const bool ok = base + w * kPerWave + j * kWave + lane < n;
        if (ok) {
            const uint32_t d = (key[j] >> shift) & (kRadix - 1);
            const uint32_t pos = s_tile[d] + s_cnt[w][d] + rank[j];
            s_k[pos] = key[j];
            s_v[pos] = val[j];
        }
    }
    __syncthreads();
    uint32_t *ko = kout + (size_t)c * nk;
    uint32_t *vo = vout + (size_t)c * nk;
    const uint32_t nv = min((uint32_t)kSortTile, n - base);
    for (uint32_t p = tid; p < nv; p += kSortThreads) {
        const uint32_t k = s_k[p];
        const uint32_t d = (k >> shift) & (kRadix - 1);
        const uint32_t dst = s_glob[d] + (p - s_tile[d]);
        ko[dst] = k;
        vo[dst] = s_v[p];
    }
}

// ------------------------------------------------- heads and window slots
//
// mark: every segment head looks its row up in the slot map once; a row
// already in this window records its slot, a new one the marker kNewHead.
// assign: new heads get the next free slots in ascending row order (tile
// prefix + thread prefix: no atomics, deterministic layout).

constexpr uint32_t kNewHead = 0xFFFFFFFEu;
constexpr uint32_t kDropped = 0xFFFFFFFFu;

struct SlotArgs {
    const uint32_t *rows;   // sorted keys [2][nk]
    int64_t nk;
    const uint32_t *n_dev;
    uint32_t n_host;
    SlotEntry *slot_map[2];
    uint32_t *slot_rows[2];
    uint32_t *seg_info;     // [2][nk]: at heads, slot | new << 31
    uint32_t *blk;          // [2][nblk]: new heads per tile
    uint32_t nblk;
    uint32_t wrows;
    WsHeader *hdr;
};

// Thread-contiguous items: thread t of tile b owns keys b*2048 + t*8 + [0, 8).
__global__ __launch_bounds__(kSortThreads) void mark_kernel(SlotArgs a)
{
    __shared__ uint32_t s_wave[kSortThreads / kWave];
    const int c = blockIdx.y;
    const uint32_t n = count_of(a.n_dev, a.n_host);
    const uint32_t i0 = blockIdx.x * kSortTile + threadIdx.x * kSortItems;
    const uint32_t *R = a.rows + (size_t)c * a.nk;
    const SlotEntry *sm = a.slot_map[c];
    uint32_t *info = a.seg_info + (size_t)c * a.nk;
    const uint32_t epoch = a.hdr->epoch;
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t i = i0 + j;
        if (i < n) {
            const uint32_t r = R[i];
            if (i == 0 || R[i - 1] != r) {
                const SlotEntry e = sm[r];
                const bool known = e.epoch == epoch;
                info[i] = known ? e.slot : kNewHead;
                cnt += known ? 0u : 1u;
            }
        }
    }
    uint32_t total;
    block_excl_scan<kSortThreads>(cnt, s_wave, &total);
    if (threadIdx.x == 0)
        a.blk[(size_t)c * a.nblk + blockIdx.x] = total;
}

__global__ __launch_bounds__(kSortThreads) void assign_kernel(SlotArgs a)
{
    __shared__ uint32_t s_wave[kSortThreads / kWave];
    const int c = blockIdx.y;
    const uint32_t b = blockIdx.x;
    const int tid = threadIdx.x;
    const uint32_t n = count_of(a.n_dev, a.n_host);
    const uint32_t *blk = a.blk + (size_t)c * a.nblk;
    // new heads in earlier tiles (block 0 also counts all tiles)
    const uint32_t upto = b == 0 ? a.nblk : b;
    uint32_t part = 0, part_before = 0;
    for (uint32_t k = tid; k < upto; k += kSortThreads) {
        const uint32_t x = blk[k];
        part += x;
        part_before += k < b ? x : 0u;
    }
    uint32_t before_tiles, all_tiles;
    block_excl_scan<kSortThreads>(part_before, s_wave, &before_tiles);
    block_excl_scan<kSortThreads>(part, s_wave, &all_tiles);
    const uint32_t old = a.hdr->n_slots[c];
    if (b == 0 && tid == 0) {
        uint64_t now = (uint64_t)old + all_tiles;
        if (now > a.wrows) {
            atomicOr(&a.hdr->flags, NGRAM_FLAG_WINDOW_FULL);
            now = a.wrows;
        }
        a.hdr->n_next[c] = (uint32_t)now;
    }
    const uint32_t i0 = b * kSortTile + tid * kSortItems;
    const uint32_t *R = a.rows + (size_t)c * a.nk;
    uint32_t *info = a.seg_info + (size_t)c * a.nk;
    uint32_t mask = 0, cnt = 0;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t i = i0 + j;
        if (i < n && (i == 0 || R[i - 1] != R[i]) && info[i] == kNewHead) {
            mask |= 1u << j;
            ++cnt;
        }
    }
    uint32_t slot = old + before_tiles + block_excl_scan<kSortThreads>(cnt, s_wave, nullptr);
    SlotEntry *sm = a.slot_map[c];
    const uint32_t epoch = a.hdr->epoch;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        if (mask & (1u << j)) {
            const uint32_t i = i0 + j;
            const uint32_t r = R[i];
            if (slot < a.wrows) {
                sm[r] = SlotEntry{epoch, slot};
                a.slot_rows[c][slot] = r;
                info[i] = slot | 0x80000000u;
            } else {
                info[i] = kDropped;   // window full: row dropped (flagged)
            }
            ++slot;
        }
    }
}

// ------------------------------------------------------ segment reduction

constexpr int kRedThreads = 256;
constexpr int kRedU = 4;   // dY rows in flight per wavefront

// Reduction modes: accumulate into the window, or fused with the step on a
// bf16 / fp32 table.
constexpr int kAccum = 0;
constexpr int kFuseBf16 = 2;
constexpr int kFuseF32 = 4;

struct RedArgs {
    const uint32_t *rows;   // sorted [2][nk]
    const uint32_t *vals;   // sorted [2][nk]: dY row code | neg << 31
    const uint32_t *info;   // [2][nk] at heads
    int64_t nk;
    const uint32_t *n_dev;
    uint32_t n_host;
    const float *dY;        // [positions][768], indexed by the row code
    const float *const *dy_ptrs;   // burst by reference: dY of each micro-step
    int pos_bits;           // burst by reference: row code = micro-step << pos_bits | position
    float *gacc;            // [2][wrows][768]
    uint32_t *slot_rows[2];
    int64_t wrows;
    float *partial;         // [2][nchunk][2][768]
    uint64_t *owners;       // [2][nchunk]: chunk | info << 32
    int64_t nchunk;
    WsHeader *hdr;
    FuseArgs f;             // fused modes only
};

__device__ __forceinline__ float4 add4(float4 a, float4 b)
{
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// Start of the dY row a key refers to.
__device__ __forceinline__ const float *dy_row(const RedArgs &a, uint32_t code)
{
    if (a.dy_ptrs)
        return a.dy_ptrs[code >> a.pos_bits] + (size_t)(code & ((1u << a.pos_bits) - 1u)) * kDim;
    return a.dY + (size_t)code * kDim;
}

__device__ __forceinline__ uint32_t lane_val(uint32_t v0, uint32_t v1, int j)
{
    return j < kWave ? (uint32_t)__builtin_amdgcn_readlane((int)v0, j)
                     : (uint32_t)__builtin_amdgcn_readlane((int)v1, j - kWave);
}

// Lane l of a wavefront holds elements l + 64 m (m = 0..11) of a 768-wide
// row, so every load, store and atomic of a row is twelve 256-byte (fp32) or
// 128-byte (bf16) contiguous wavefront accesses.
constexpr int kPer = kDim / kWave;   // 12

__device__ __forceinline__ void store_row(float *dst, const float (&acc)[kPer], int lane)
{
#pragma unroll
    for (int m = 0; m < kPer; ++m)
        dst[lane + m * kWave] = acc[m];
}

// Adds a micro-step's sum into its window row.  A row new to the window is
// written; an existing one gets G += S through fire-and-forget atomic adds
// (the read-modify-write happens in L2 and the wavefront does not wait for
// it).  Every window row has exactly one segment, hence exactly one writer,
// per launch, so each element sees a single addition: the result is the
// plain fp32 sum G + S and does not depend on timing.
__device__ __forceinline__ void flush_window_row(const float (&acc)[kPer], float *gacc, int64_t wrows, int c,
                                                 uint32_t info, int lane)
{
    if (info == kDropped)
        return;   // window full: row dropped (flagged when slots were assigned)
    float *g = gacc + ((size_t)c * wrows + (info & 0x7FFFFFFFu)) * kDim;
    if (info >> 31) {
        store_row(g, acc, lane);
    } else {
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            unsafeAtomicAdd(g + lane + m * kWave, acc[m]);
    }
}

// Fused flush: the row's window gradient is complete.  A row the window
// already holds adds its stored gradient first (G = G_window + S, the same
// addition the accumulate path would make) and its slot is marked stepped;
// then the row is stepped in place.
template <int MODE>
__device__ __forceinline__ void flush_fused(float (&acc)[kPer], const RedArgs &a, int c, uint32_t row,
                                            uint32_t info, int lane)
{
    if (info != kNewHead) {
        const float *g = a.gacc + ((size_t)c * a.wrows + info) * kDim + lane;
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            acc[m] = g[m * kWave] + acc[m];
        if (lane == 0)
            a.slot_rows[c][info] = row | kSlotStepped;
    }
    float w[kPer];
    if (MODE == kFuseBf16) {
        const uint16_t *wp = reinterpret_cast<const uint16_t *>(a.f.w[c]) + (size_t)row * kDim + lane;
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            w[m] = __uint_as_float((uint32_t)wp[m * kWave] << 16);
    } else {
        const float *wp = reinterpret_cast<const float *>(a.f.w[c]) + (size_t)row * kDim + lane;
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            w[m] = wp[m * kWave];
    }
    const RowState st = a.f.st[c][row];
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < kPer; ++m)
        ss += acc[m] * acc[m];
    ss = wave_sum(ss);
    float vn;
    bool order_bad;
    const float scale = step_scale(ss, st, a.f.p, vn, order_bad);
    if (MODE == kFuseBf16) {
        uint16_t *wp = reinterpret_cast<uint16_t *>(a.f.w[c]) + (size_t)row * kDim + lane;
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            wp[m * kWave] = (uint16_t)bf16_rne(w[m] - scale * acc[m]);
    } else {
        float *wp = reinterpret_cast<float *>(a.f.w[c]) + (size_t)row * kDim + lane;
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            wp[m * kWave] = w[m] - scale * acc[m];
    }
    if (lane == 0) {
        a.f.st[c][row] = RowState{vn, a.f.p.t};
        if (order_bad)
            atomicOr(&a.hdr->flags, NGRAM_FLAG_STEP_ORDER);
    }
}

// One wavefront per 64 sorted keys.  Keys are consumed in order, kRedU dY rows
// in flight at a time, whatever the segment boundaries.  A segment's sum is
// reset at its first key and flushed at its last:
//   - a segment that starts and ends here goes to the window (or, fused, is
//     completed and stepped);
//   - the first piece, if it continues a segment from the previous chunk, is
//     skipped when that chunk finishes it, else left as partial row 0;
//   - the last piece, if it spills into the next chunk, is finished here when
//     it ends within that chunk (its keys are loaded as lanes 64..127), else
//     left as partial row 1 with a fix-up record.
template <int MODE>
__global__ __launch_bounds__(kRedThreads) void seg_reduce_kernel(RedArgs a)
{
    const int c = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t chunk = (int64_t)blockIdx.x * (kRedThreads / kWave) + threadIdx.x / kWave;
    const uint32_t n = count_of(a.n_dev, a.n_host);
    if (MODE == kAccum && chunk == 0 && lane == 0)
        a.hdr->n_slots[c] = a.hdr->n_next[c];   // the slots assign_kernel handed out
    const int64_t c0 = chunk * kChunk;
    if (c0 >= n)
        return;
    const uint32_t *R = a.rows + (size_t)c * a.nk;
    const uint32_t *V = a.vals + (size_t)c * a.nk;
    const uint32_t *I = a.info + (size_t)c * a.nk;
    const int nv = (int)min<int64_t>(kChunk, (int64_t)n - c0);
    const bool valid = lane < nv;
    const uint32_t r0 = valid ? R[c0 + lane] : 0xFFFFFFFFu;
    const uint32_t v0 = valid ? V[c0 + lane] : 0u;
    uint32_t prev = __shfl_up(r0, 1);
    if (lane == 0)
        prev = c0 > 0 ? R[c0 - 1] : 0xFFFFFFFFu;
    const bool head = valid && (r0 != prev);
    const uint64_t hm = __ballot(head);
    const uint32_t i0 = head ? I[c0 + lane] : 0u;
    const uint32_t row_last = (uint32_t)__builtin_amdgcn_readlane((int)r0, nv - 1);
    const bool cont_after = nv == kChunk && c0 + kChunk < n && R[c0 + kChunk] == row_last;

    // first piece: continuation of the previous chunk's last segment?
    const bool first_cont = !(hm & 1ull);
    const int e0 = hm ? (int)__builtin_ctzll(hm) : nv;   // end of the first piece
    bool skip_first = false;
    if (first_cont) {
        const uint32_t row0 = (uint32_t)__builtin_amdgcn_readlane((int)r0, 0);
        const bool piece0_cont = (e0 == nv) && cont_after;
        const bool head_in_prev = (c0 == kChunk) || (R[c0 - kChunk - 1] != row0);
        skip_first = head_in_prev && !piece0_cont;
    }
    // last piece: starts at the highest head; spills over if cont_after
    const int la = hm ? 63 - (int)__builtin_clzll(hm) : -1;
    const bool last_spills = hm && cont_after;
    bool owner_full = false;
    uint32_t v1 = 0;
    int extra = 0;
    if (last_spills) {
        owner_full = !(c0 + 2 * kChunk < n && R[c0 + 2 * kChunk] == row_last);
        if (owner_full) {
            const int64_t i1 = c0 + kChunk + lane;
            const bool ok1 = i1 < n;
            const uint32_t r1 = ok1 ? R[i1] : 0xFFFFFFFFu;
            v1 = ok1 ? V[i1] : 0u;
            extra = __popcll(__ballot(ok1 && r1 == row_last));
        }
    }
    const int j0 = skip_first ? e0 : 0;
    const int jend = owner_full ? kChunk + extra : nv;

    float acc[kPer];
    int ps = j0;   // start key of the open segment
#pragma unroll
    for (int m = 0; m < kPer; ++m)
        acc[m] = 0.f;
    for (int j = j0; j < jend; j += kRedU) {
        float x[kRedU][kPer];
        uint32_t sg[kRedU];
#pragma unroll
        for (int u = 0; u < kRedU; ++u) {
            if (j + u < jend) {
                const uint32_t v = lane_val(v0, v1, j + u);
                sg[u] = v & 0x80000000u;
                const float *p = dy_row(a, v & 0x7FFFFFFFu) + lane;
#pragma unroll
                for (int m = 0; m < kPer; ++m)
                    x[u][m] = p[m * kWave];
            }
        }
#pragma unroll
        for (int u = 0; u < kRedU; ++u) {
            const int k = j + u;
            if (k >= jend)
                break;
            if (k < kChunk && k != j0 && ((hm >> k) & 1ull)) {
                ps = k;
#pragma unroll
                for (int m = 0; m < kPer; ++m)
                    acc[m] = 0.f;
            }
#pragma unroll
            for (int m = 0; m < kPer; ++m)
                acc[m] += __uint_as_float(__float_as_uint(x[u][m]) ^ sg[u]);
            // does the open segment end at key k?
            bool ends;
            if (k >= kChunk - 1 && owner_full)
                ends = (k == jend - 1);
            else if (k == nv - 1)
                ends = true;
            else
                ends = (k + 1 < kChunk) && ((hm >> (k + 1)) & 1ull);
            if (!ends)
                continue;
            if (ps == 0 && first_cont) {
                store_row(a.partial + (((size_t)c * a.nchunk + chunk) * 2 + 0) * kDim, acc, lane);
            } else if (ps == la && last_spills && !owner_full) {
                const uint32_t info = (uint32_t)__builtin_amdgcn_readlane((int)i0, ps);
                store_row(a.partial + (((size_t)c * a.nchunk + chunk) * 2 + 1) * kDim, acc, lane);
                if (lane == 0) {
                    const uint32_t k2 = atomicAdd(&a.hdr->n_owner[c], 1u);
                    a.owners[(size_t)c * a.nchunk + k2] = (uint64_t)chunk | ((uint64_t)info << 32);
                }
            } else {
                const uint32_t info = (uint32_t)__builtin_amdgcn_readlane((int)i0, ps);
                if (MODE == kAccum)
                    flush_window_row(acc, a.gacc, a.wrows, c, info, lane);
                else
                    flush_fused<MODE>(acc, a, c, (uint32_t)__builtin_amdgcn_readlane((int)r0, ps), info, lane);
            }
        }
    }
}

// Sums the partial rows of each segment longer than two chunks: the starting
// chunk's tail piece, then every following chunk's head piece, split into 16
// contiguous runs (one per wavefront) that are added in run order.  Then the
// row goes to the window, or (fused) is completed and stepped by the block.
constexpr int kFixThreads = 1024;
template <int MODE>
__global__ __launch_bounds__(kFixThreads) void fixup_kernel(RedArgs a)
{
    constexpr int kW = kFixThreads / kWave;
    __shared__ float4 s_part[kW][kDim / 4];
    __shared__ float s_ss[kW];
    const int c = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const uint32_t nown = a.hdr->n_owner[c];
    const uint32_t n = count_of(a.n_dev, a.n_host);
    const uint32_t *R = a.rows + (size_t)c * a.nk;
    const float4 *P = reinterpret_cast<const float4 *>(a.partial + (size_t)c * a.nchunk * 2 * kDim);
    for (uint32_t k = blockIdx.x; k < nown; k += gridDim.x) {
        const uint64_t rec = a.owners[(size_t)c * a.nchunk + k];
        const int64_t chunk = (int64_t)(uint32_t)rec;
        const uint32_t info = (uint32_t)(rec >> 32);
        const uint32_t row = R[chunk * kChunk + kChunk - 1];
        int64_t m = 0;   // following chunks that start inside the segment
        for (;;) {
            const int64_t cc = chunk + 1 + m + tid;
            const bool hit = cc * kChunk < (int64_t)n && R[cc * kChunk] == row;
            const int cnt = __syncthreads_count(hit);
            m += cnt;
            if (cnt < kFixThreads)
                break;
        }
        const int64_t np = m + 1;
        const int64_t lo = np * w / kW, hi = np * (w + 1) / kW;
        float4 acc[3] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f),
                         make_float4(0.f, 0.f, 0.f, 0.f)};
        for (int64_t p = lo; p < hi; p += kRedU) {
            float4 x[kRedU][3];
#pragma unroll
            for (int u = 0; u < kRedU; ++u) {
                if (p + u < hi) {
                    const int64_t src = p + u == 0 ? chunk * 2 + 1 : (chunk + p + u) * 2;
                    const float4 *s = P + src * (kDim / 4) + lane;
                    x[u][0] = s[0];
                    x[u][1] = s[kWave];
                    x[u][2] = s[2 * kWave];
                }
            }
#pragma unroll
            for (int u = 0; u < kRedU; ++u) {
                if (p + u < hi) {
#pragma unroll
                    for (int q = 0; q < 3; ++q)
                        acc[q] = add4(acc[q], x[u][q]);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 3; ++q)
            s_part[w][lane + q * kWave] = acc[q];
        __syncthreads();
        float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tid < kDim / 4) {
            sum = s_part[0][tid];
#pragma unroll
            for (int ww = 1; ww < kW; ++ww)
                sum = add4(sum, s_part[ww][tid]);
        }
        if (MODE == kAccum) {
            if (tid < kDim / 4 && info != kDropped) {
                float4 *g = reinterpret_cast<float4 *>(a.gacc + ((size_t)c * a.wrows + (info & 0x7FFFFFFFu)) * kDim) + tid;
                if (!(info >> 31))
                    sum = add4(*g, sum);
                *g = sum;
            }
        } else {
            // complete the row's window gradient, then step it with the block:
            // thread t < 192 owns elements 4t .. 4t+3
            if (tid < kDim / 4 && info != kNewHead)
                sum = add4(reinterpret_cast<const float4 *>(a.gacc + ((size_t)c * a.wrows + info) * kDim)[tid], sum);
            if (tid == 0 && info != kNewHead)
                a.slot_rows[c][info] = row | kSlotStepped;
            float ss = tid < kDim / 4 ? sum.x * sum.x + sum.y * sum.y + sum.z * sum.z + sum.w * sum.w : 0.f;
            ss = wave_sum(ss);
            if (lane == 0)
                s_ss[w] = ss;
            __syncthreads();
            ss = 0.f;
#pragma unroll
            for (int ww = 0; ww < kW; ++ww)
                ss += s_ss[ww];
            const RowState st = a.f.st[c][row];
            float vn;
            bool order_bad;
            const float scale = step_scale(ss, st, a.f.p, vn, order_bad);
            if (tid < kDim / 4) {
                if (MODE == kFuseBf16) {
                    uint2 *wp = reinterpret_cast<uint2 *>(a.f.w[c] + (size_t)row * kDim * 2) + tid;
                    const uint2 x = *wp;
                    *wp = make_uint2(bf16_pack(bf16_lo(x.x) - scale * sum.x, bf16_hi(x.x) - scale * sum.y),
                                     bf16_pack(bf16_lo(x.y) - scale * sum.z, bf16_hi(x.y) - scale * sum.w));
                } else {
                    float4 *wp = reinterpret_cast<float4 *>(a.f.w[c] + (size_t)row * kDim * 4) + tid;
                    const float4 x = *wp;
                    *wp = make_float4(x.x - scale * sum.x, x.y - scale * sum.y, x.z - scale * sum.z,
                                      x.w - scale * sum.w);
                }
            }
            if (tid == 0) {
                a.f.st[c][row] = RowState{vn, a.f.p.t};
                if (order_bad)
                    atomicOr(&a.hdr->flags, NGRAM_FLAG_STEP_ORDER);
            }
        }
        __syncthreads();
    }
}

}  // namespace

namespace {

hipError_t reduce_impl(const WsLayout &L, uint8_t *ws, const HashParams &hp, const int32_t *tok, int64_t T,
                       const float *dY, const FuseArgs *f, hipStream_t s)
{
    // spread: T keys known on the host; burst: the stash count on the device,
    // bounded by the stash capacity (grids cover the bound, blocks past the
    // count exit)
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + L.hdr);
    const bool burst = tok == nullptr;
    const uint32_t n_host = (uint32_t)T;
    const uint32_t *n_dev = burst ? &hdr->n_stash : nullptr;
    if (n_host == 0)
        return hipSuccess;
    const uint32_t nblk = (n_host + kSortTile - 1) / kSortTile;
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + L.hist);
    uint32_t *tot = reinterpret_cast<uint32_t *>(ws + L.tot);
    uint32_t *k0 = reinterpret_cast<uint32_t *>(ws + L.keys[0]);
    uint32_t *v0 = reinterpret_cast<uint32_t *>(ws + L.vals[0]);

    prof_begin(NGRAM_PROF_SORT, s);
    if (burst)
        keys_tile_kernel<true><<<nblk, kSortThreads, 0, s>>>(
            nullptr, reinterpret_cast<const uint32_t *>(ws + L.stash_idx),
            reinterpret_cast<const uint32_t *>(ws + L.stash_pos), hp, n_host, k0, v0, L.nk, hist, nblk, hdr);
    else
        keys_tile_kernel<false><<<nblk, kSortThreads, 0, s>>>(tok, nullptr, nullptr, hp, n_host, k0, v0, L.nk, hist,
                                                             nblk, hdr);
    int cur = 0;
    for (int p = 0; p < L.passes; ++p) {
        const int shift = p * kRadixBits;
        uint32_t *kin = reinterpret_cast<uint32_t *>(ws + L.keys[cur]);
        uint32_t *vin = reinterpret_cast<uint32_t *>(ws + L.vals[cur]);
        uint32_t *kout = reinterpret_cast<uint32_t *>(ws + L.keys[cur ^ 1]);
        uint32_t *vout = reinterpret_cast<uint32_t *>(ws + L.vals[cur ^ 1]);
        if (p > 0)
            radix_hist_kernel<<<dim3(nblk, 2), kSortThreads, 0, s>>>(kin, L.nk, n_dev, n_host, shift, hist, nblk);
        scan_digits_kernel<<<dim3(kRadix, 2), kSortThreads, 0, s>>>(hist, nblk, tot);
        radix_scatter_kernel<<<dim3(nblk, 2), kSortThreads, 0, s>>>(kin, vin, kout, vout, L.nk, n_dev, n_host,
                                                                    shift, hist, tot, nblk);
        cur ^= 1;
    }
    SlotArgs sa;
    sa.rows = reinterpret_cast<const uint32_t *>(ws + L.keys[cur]);
    sa.nk = L.nk;
    sa.n_dev = n_dev;
    sa.n_host = n_host;
    for (int c = 0; c < 2; ++c) {
        sa.slot_map[c] = reinterpret_cast<SlotEntry *>(ws + L.slot_map[c]);
        sa.slot_rows[c] = reinterpret_cast<uint32_t *>(ws + L.slot_rows[c]);
    }
    sa.seg_info = reinterpret_cast<uint32_t *>(ws + L.seg_info);
    sa.blk = reinterpret_cast<uint32_t *>(ws + L.blk);
    sa.nblk = nblk;
    sa.wrows = (uint32_t)L.wrows;
    sa.hdr = hdr;
    mark_kernel<<<dim3(nblk, 2), kSortThreads, 0, s>>>(sa);
    if (!f)   // fused: rows new to the window are stepped at once and need no slot
        assign_kernel<<<dim3(nblk, 2), kSortThreads, 0, s>>>(sa);
    prof_end(NGRAM_PROF_SORT, s);

    RedArgs ra;
    ra.rows = sa.rows;
    ra.vals = reinterpret_cast<const uint32_t *>(ws + L.vals[cur]);
    ra.info = sa.seg_info;
    ra.nk = L.nk;
    ra.n_dev = n_dev;
    ra.n_host = n_host;
    ra.dY = burst && !L.by_ref ? reinterpret_cast<const float *>(ws + L.stash_dy) : dY;
    ra.dy_ptrs = L.by_ref ? reinterpret_cast<const float *const *>(ws + L.dy_ptrs) : nullptr;
    ra.pos_bits = L.pos_bits;
    ra.gacc = reinterpret_cast<float *>(ws + L.gacc);
    ra.slot_rows[0] = sa.slot_rows[0];
    ra.slot_rows[1] = sa.slot_rows[1];
    ra.wrows = L.wrows;
    ra.partial = reinterpret_cast<float *>(ws + L.partial);
    ra.owners = reinterpret_cast<uint64_t *>(ws + L.owners);
    ra.nchunk = L.nchunk;
    ra.hdr = hdr;
    if (f)
        ra.f = *f;
    const uint32_t nchunk = (n_host + kChunk - 1) / kChunk;
    const uint32_t per_block = kRedThreads / kWave;
    const dim3 grid((nchunk + per_block - 1) / per_block, 2);
    prof_begin(NGRAM_PROF_REDUCE, s);
    if (!f) {
        seg_reduce_kernel<kAccum><<<grid, kRedThreads, 0, s>>>(ra);
        prof_end(NGRAM_PROF_REDUCE, s);
        fixup_kernel<kAccum><<<dim3(256, 2), kFixThreads, 0, s>>>(ra);
    } else if (f->dtype == NGRAM_DTYPE_BF16) {
        seg_reduce_kernel<kFuseBf16><<<grid, kRedThreads, 0, s>>>(ra);
        prof_end(NGRAM_PROF_REDUCE, s);
        fixup_kernel<kFuseBf16><<<dim3(256, 2), kFixThreads, 0, s>>>(ra);
    } else {
        seg_reduce_kernel<kFuseF32><<<grid, kRedThreads, 0, s>>>(ra);
        prof_end(NGRAM_PROF_REDUCE, s);
        fixup_kernel<kFuseF32><<<dim3(256, 2), kFixThreads, 0, s>>>(ra);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const WsLayout &L, uint8_t *ws, const HashParams &hp, const int32_t *tok, int64_t T,
                         const float *dY, hipStream_t s)
{
    return reduce_impl(L, ws, hp, tok, T, dY, nullptr, s);
}

hipError_t launch_reduce_step(const WsLayout &L, uint8_t *ws, const HashParams &hp, const int32_t *tok, int64_t T,
                              const float *dY, const FuseArgs &f, hipStream_t s)
{
    return reduce_impl(L, ws, hp, tok, T, dY, &f, s);
}

}  // namespace ngram
