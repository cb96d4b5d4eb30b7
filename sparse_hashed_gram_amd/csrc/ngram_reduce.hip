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
//   1. LSD radix sort of (row, position|sign) pairs, 9-bit digits.  Each pass
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

// ------------------------------------------------------------ radix sort
//
// Radix tiles of 256 threads x 8 keys (2,048), or x 16 (4,096) when a channel
// has at least 2^20 keys to sort.  Per pass: per-tile digit counts
// (hist[c][d][tile], digit-major), then one block per (digit, channel) turns
// its row of tile counts into exclusive tile offsets and a digit total, then
// the scatter adds the exclusive scan of the digit totals (done per block in
// LDS) to get each tile's global digit offsets.

// Key build for one tile, fused with the first pass's digit counts.  Spread:
// position i of the micro-step is hashed from the tokens.  Burst: every
// position kept in the stash, whose packed indices were hashed when kept.
// Also clears the fix-up record counts of the reduce that follows.
// NESTED: only the trigram keys are built here; each position's packed
// bigram index goes to bidx[row code], from where the bigram keys are
// gathered in trigram order once the trigram keys are sorted.
template <bool FROM_STASH, int ITEMS, bool NESTED>
__global__ __launch_bounds__(kSortThreads) void keys_tile_kernel(
    const int32_t *__restrict__ tok, const uint32_t *__restrict__ sidx, const uint32_t *__restrict__ spos,
    HashParams hp, uint32_t n_host, uint32_t *__restrict__ keys, uint32_t *__restrict__ vals, int64_t nk,
    uint32_t *__restrict__ hist, uint32_t nblk, WsHeader *__restrict__ hdr, uint32_t *__restrict__ bidx)
{
    __shared__ uint32_t h[2][kRadix];
    const int tid = threadIdx.x;
    const uint32_t b = blockIdx.x;
    const uint32_t n = FROM_STASH ? min(hdr->n_stash, n_host) : n_host;
    if (b == 0 && tid == 0) {
        hdr->n_owner[0] = 0;
        hdr->n_owner[1] = 0;
        hdr->n_trun = 0;
    }
    for (int d = tid; d < kRadix; d += kSortThreads) {
        h[0][d] = 0;
        h[1][d] = 0;
    }
    __syncthreads();
    const uint32_t base = b * radix_tile(ITEMS);
    bool bad = false;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
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
            if (NESTED) {
                bidx[pos] = ib;
            } else {
                keys[i] = ib & 0x7FFFFFFFu;
                vals[i] = pos | (ib & 0x80000000u);
                atomicAdd(&h[0][ib & (kRadix - 1)], 1u);
            }
            keys[nk + i] = it & 0x7FFFFFFFu;
            vals[nk + i] = pos | (it & 0x80000000u);
            atomicAdd(&h[1][it & (kRadix - 1)], 1u);
        }
    }
    if (bad)
        atomicOr(&hdr->flags, NGRAM_FLAG_BAD_TOKEN);
    __syncthreads();
    for (int d = tid; d < kRadix; d += kSortThreads) {
        if (!NESTED)
            hist[((size_t)0 * kRadix + d) * nblk + b] = h[0][d];
        hist[((size_t)1 * kRadix + d) * nblk + b] = h[1][d];
    }
}

// Nested sort: the bigram keys in the order of the sorted trigram keys (the
// row code of each sorted trigram payload names its position's bigram
// index), fused with the first bigram pass's digit counts.  A stable sort of
// this sequence by bigram row gives the (bigram row, trigram row, position)
// order.  The rows are also kept in this order (btro), where mark_kernel
// compares the bigram rows of consecutive trigram keys.
template <int ITEMS>
__global__ __launch_bounds__(kSortThreads) void gather_bigram_kernel(
    const uint32_t *__restrict__ vt, const uint32_t *__restrict__ bidx, const uint32_t *n_dev, uint32_t n_host,
    uint32_t *__restrict__ keys0, uint32_t *__restrict__ vals0, uint32_t *__restrict__ hist, uint32_t nblk,
    uint32_t *__restrict__ btro)
{
    __shared__ uint32_t h[kRadix];
    const int tid = threadIdx.x;
    const uint32_t b = blockIdx.x;
    const uint32_t n = count_of(n_dev, n_host);
    for (int d = tid; d < kRadix; d += kSortThreads)
        h[d] = 0;
    __syncthreads();
    const uint32_t base = b * radix_tile(ITEMS);
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t i = base + j * kSortThreads + tid;
        if (i < n) {
            const uint32_t code = vt[i] & 0x7FFFFFFFu;
            const uint32_t ib = bidx[code];
            keys0[i] = ib & 0x7FFFFFFFu;
            btro[i] = ib & 0x7FFFFFFFu;
            vals0[i] = code | (ib & 0x80000000u);
            atomicAdd(&h[ib & (kRadix - 1)], 1u);
        }
    }
    __syncthreads();
    for (int d = tid; d < kRadix; d += kSortThreads)
        hist[(size_t)d * nblk + b] = h[d];
}

template <int ITEMS>
__global__ __launch_bounds__(kSortThreads) void radix_hist_kernel(
    const uint32_t *__restrict__ keys, int64_t nk, const uint32_t *n_dev, uint32_t n_host, int shift,
    uint32_t *__restrict__ hist, uint32_t nblk, int cbase)
{
    __shared__ uint32_t h[kRadix];
    const int c = cbase + (int)blockIdx.y;
    const uint32_t b = blockIdx.x;
    const int tid = threadIdx.x;
    const uint32_t n = count_of(n_dev, n_host);
    for (int d = tid; d < kRadix; d += kSortThreads)
        h[d] = 0;
    __syncthreads();
    const uint32_t *k = keys + (size_t)c * nk;
    const uint32_t base = b * radix_tile(ITEMS);
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t i = base + j * kSortThreads + tid;
        if (i < n)
            atomicAdd(&h[(k[i] >> shift) & (kRadix - 1)], 1u);
    }
    __syncthreads();
    for (int d = tid; d < kRadix; d += kSortThreads)
        hist[((size_t)c * kRadix + d) * nblk + b] = h[d];
}

// Block (d, c): exclusive scan of digit d's tile counts in place, total to
// tot[c][d].  Each thread owns a contiguous run of tiles.
__global__ __launch_bounds__(kSortThreads) void scan_digits_kernel(uint32_t *__restrict__ hist, uint32_t nblk,
                                                                   uint32_t *__restrict__ tot, int cbase)
{
    __shared__ uint32_t s_wave[kSortThreads / kWave];
    const int d = blockIdx.x, c = cbase + (int)blockIdx.y, tid = threadIdx.x;
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

// Stable scatter of one tile of NT x ITEMS keys by the current digit.  Wave
// w owns the w-th of the tile's NT / 64 equal parts, processed 64 keys at a
// time in index order.  X3 (one channel): a third payload moves with the
// keys, xin -> xout; a null xin stands for each key's index before the pass.
template <int ITEMS, int NT, bool X3>
__global__ __launch_bounds__(NT) void radix_scatter_kernel(
    const uint32_t *__restrict__ kin, const uint32_t *__restrict__ vin, uint32_t *__restrict__ kout,
    uint32_t *__restrict__ vout, int64_t nk, const uint32_t *n_dev, uint32_t n_host, int shift,
    const uint32_t *__restrict__ hist, const uint32_t *__restrict__ tot, uint32_t nblk, int cbase,
    const uint32_t *__restrict__ xin, uint32_t *__restrict__ xout)
{
    constexpr int kTile = NT * ITEMS;
    constexpr int kW = NT / kWave;
    constexpr int kD = kRadix / NT;   // digits per thread in the per-digit loops
    static_assert(kRadix % NT == 0, "digits are split evenly over the threads");
    constexpr int kPerWave = kTile / kW;
    __shared__ uint32_t s_cnt[kW][kRadix];
    __shared__ uint32_t s_tile[kRadix];
    __shared__ uint32_t s_glob[kRadix];
    __shared__ uint32_t s_k[kTile];
    __shared__ uint32_t s_v[kTile];
    __shared__ uint32_t s_x[X3 ? kTile : 1];
    __shared__ uint32_t s_wave[kW];

    const int c = cbase + (int)blockIdx.y;
    const uint32_t b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const uint32_t n = count_of(n_dev, n_host);
    const uint32_t base = b * kTile;
    if (base >= n)
        return;
    const uint32_t *ki = kin + (size_t)c * nk;
    const uint32_t *vi = vin + (size_t)c * nk;

    for (int r = tid; r < kW * kRadix; r += NT)
        (&s_cnt[0][0])[r] = 0;
    {
        // thread t owns digits t * kD .. t * kD + kD - 1
        uint32_t v[kD], sum = 0;
#pragma unroll
        for (int j = 0; j < kD; ++j) {
            v[j] = tot[c * kRadix + tid * kD + j];
            sum += v[j];
        }
        uint32_t run = block_excl_scan<NT>(sum, s_wave, nullptr);
#pragma unroll
        for (int j = 0; j < kD; ++j) {
            const int d = tid * kD + j;
            s_glob[d] = run + hist[((size_t)c * kRadix + d) * nblk + b];
            run += v[j];
        }
    }
    __syncthreads();

    uint32_t key[ITEMS], val[ITEMS], rank[ITEMS], x3[X3 ? ITEMS : 1];
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t i = base + w * kPerWave + j * kWave + lane;
        const bool ok = i < n;
        key[j] = ok ? ki[i] : 0u;
        val[j] = ok ? vi[i] : 0u;
        if constexpr (X3)
            x3[j] = xin ? (ok ? xin[i] : 0u) : i;
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
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
        // per digit: exclusive offsets of the wavefronts' runs, then the
        // exclusive scan of the digit totals over the tile
        uint32_t dtot[kD], sum = 0;
#pragma unroll
        for (int j = 0; j < kD; ++j) {
            const int d = tid * kD + j;
            uint32_t run = 0;
#pragma unroll
            for (int ww = 0; ww < kW; ++ww) {
                const uint32_t x = s_cnt[ww][d];
                s_cnt[ww][d] = run;
                run += x;
            }
            dtot[j] = run;
            sum += run;
        }
        uint32_t run = block_excl_scan<NT>(sum, s_wave, nullptr);
#pragma unroll
        for (int j = 0; j < kD; ++j) {
            s_tile[tid * kD + j] = run;
            run += dtot[j];
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const bool ok = base + w * kPerWave + j * kWave + lane < n;
        if (ok) {
            const uint32_t d = (key[j] >> shift) & (kRadix - 1);
            const uint32_t pos = s_tile[d] + s_cnt[w][d] + rank[j];
            s_k[pos] = key[j];
            s_v[pos] = val[j];
            if constexpr (X3)
                s_x[pos] = x3[j];
        }
    }
    __syncthreads();
    uint32_t *ko = kout + (size_t)c * nk;
    uint32_t *vo = vout + (size_t)c * nk;
    const uint32_t nv = min((uint32_t)kTile, n - base);
    for (uint32_t p = tid; p < nv; p += NT) {
        const uint32_t k = s_k[p];
        const uint32_t d = (k >> shift) & (kRadix - 1);
        const uint32_t dst = s_glob[d] + (p - s_tile[d]);
        const uint32_t v = s_v[p];
        ko[dst] = k;
        vo[dst] = v;
        if constexpr (X3)
            xout[dst] = s_x[p];
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
    const uint32_t *vals;   // sorted payloads [2][nk]: dY row code | neg << 31
    int64_t nk;
    const uint32_t *n_dev;
    uint32_t n_host;
    SlotEntry *slot_map[2];
    uint32_t *slot_rows[2];
    uint32_t *seg_info;     // [2][nk]: at heads, slot | new << 31
    uint32_t *blk;          // [2][nblk]: new heads per tile
    uint32_t *kept;         // [nblk]: trigram keys the singleton split keeps, per tile
    uint32_t nblk;
    uint32_t wrows;
    WsHeader *hdr;
    bool fused;             // the reduction is fused with the step
    uint32_t *tinfo;        // singleton map: per dY row code, or (nested sort) per index in the trigram order
    uint32_t *split_rows;   // compacted trigram keys, payloads and head info
    uint32_t *split_vals;
    uint32_t *split_info;
    bool nested;            // fused + nested sort: trigram rows nested in one bigram segment
    const uint32_t *btro;   // nested: bigram row of each key in the trigram order
    uint8_t *tkept;         // nested: per sorted trigram key, kept for the trigram pass
};

// Singleton split.  A trigram row that occurs at exactly one position of the
// reduced keys has the sum s_t dY of that one position, and the bigram pass
// holds that dY row in registers anyway: it applies the row there, and the
// trigram pass only walks the other keys.  The singleton map records, per dY
// row code:
//   fused reduction (rows new to the window only): row | neg << 31, and the
//     bigram pass steps the row;
//   accumulating reduction: slot | new << 31 | neg << 30 (kDropSingle if the
//     window had no slot left), and the bigram pass stores (new) or adds the
//     signed row into that window slot;
//   kNotSingle otherwise.
constexpr uint32_t kNotSingle = 0xFFFFFFFFu;
constexpr uint32_t kDropSingle = 0x3FFFFFFFu;   // slot field of all ones: never a slot
// Nested trigram rows (fused reduction, nested sort).  The bigram keys are
// sorted by (bigram row, trigram row, position).  Every position of a
// trigram key has the same bigram key, so a trigram row whose positions all
// have one bigram row lies in one bigram segment as one contiguous run.  If
// the row is new to the window, the bigram pass sums the run from the dY
// rows it loads anyway and the trigram pass skips its keys: a run inside
// one wavefront's walk is summed and stepped there; a run that crosses the
// end of a walk (inside a bigram segment of many chunks) leaves one piece
// per walk in tpart, and the fix-up adds the pieces in order and steps the
// row.  The record is row | neg << 31, plus, for a run of several keys,
// kMultiKey, and kRunHead / kRunTail on its first / last key.  With the
// nested sort the map is indexed by the key's place in the trigram order
// (mark_kernel writes it in that order, one contiguous store per key), and
// the bigram sort carries that index along with each bigram key (tix).
constexpr uint32_t kMultiKey = 0x40000000u;
constexpr uint32_t kRunHead = 0x20000000u;
constexpr uint32_t kRunTail = 0x10000000u;
constexpr uint32_t kTrowMask = 0x0FFFFFFFu;

__device__ __forceinline__ bool is_run(uint32_t rec) { return rec != kNotSingle && (rec & kMultiKey) != 0u; }

// Inclusive running maximum over a block of NT threads; *excl (if given)
// gets the maximum over the threads before this one (-1 for thread 0).
template <int NT>
__device__ __forceinline__ int block_incl_max(int v, int *s_wave, int *excl)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(v, d);
        if (lane >= d)
            v = max(v, o);
    }
    if (lane == kWave - 1)
        s_wave[w] = v;
    __syncthreads();
    int before = -1;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i)
        before = i < w ? max(before, s_wave[i]) : before;
    __syncthreads();
    const int prev_in_wave = __shfl_up(v, 1);
    if (excl)
        *excl = max(before, lane > 0 ? prev_in_wave : -1);
    return max(before, v);
}

// A thread's kSortItems consecutive entries i0 .. i0 + kSortItems - 1 of p
// (those below n; 0 past it): two 16-byte loads when all are below n and
// p + i0 is 16-byte aligned (i0 is a multiple of kSortItems; a channel's
// arrays start at c nk, which need not be), else one load each.
__device__ __forceinline__ void load_items(const uint32_t *p, uint32_t i0, uint32_t n, uint32_t (&v)[kSortItems])
{
    static_assert(kSortItems == 8, "two 16-byte pieces");
    if (i0 + kSortItems <= n && ((uintptr_t)(p + i0) & 15u) == 0) {
        const uint4 x = *reinterpret_cast<const uint4 *>(p + i0), y = *reinterpret_cast<const uint4 *>(p + i0 + 4);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
    } else {
#pragma unroll
        for (int j = 0; j < kSortItems; ++j)
            v[j] = i0 + j < n ? p[i0 + j] : 0u;
    }
}
// The matching stores of the entries below n.
__device__ __forceinline__ void store_items(uint32_t *p, uint32_t i0, uint32_t n, const uint32_t (&v)[kSortItems])
{
    if (i0 + kSortItems <= n && ((uintptr_t)(p + i0) & 15u) == 0) {
        *reinterpret_cast<uint4 *>(p + i0) = make_uint4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<uint4 *>(p + i0 + 4) = make_uint4(v[4], v[5], v[6], v[7]);
    } else {
#pragma unroll
        for (int j = 0; j < kSortItems; ++j)
            if (i0 + j < n)
                p[i0 + j] = v[j];
    }
}

// Thread-contiguous items: thread t of tile b owns keys b*2048 + t*8 + [0, 8).
// For the trigram channel it also counts, per tile, the keys the singleton
// split keeps (split_kernel's layout).
//
// Nested sort, trigram channel: decides which trigram rows the bigram pass
// completes.  A row qualifies if its keys lie in this tile of the trigram
// order (its head here, its end here), it is new to the window, and all its
// keys have the same bigram row (compared key to key in btro).  Its
// keys get their records in the singleton map and are dropped from the
// trigram pass; every other key keeps kNotSingle and is kept.  The trigram
// order lists a row's keys by position, as the bigram order lists the run,
// so the segment's head and end are the run's first and last key.
__global__ __launch_bounds__(kSortThreads) void mark_kernel(SlotArgs a)
{
    __shared__ uint32_t s_wave[kSortThreads / kWave];
    __shared__ int s_iwave[kSortThreads / kWave];
    __shared__ uint8_t s_fail[kSortTile];
    const int c = blockIdx.y;
    const uint32_t n = count_of(a.n_dev, a.n_host);
    const uint32_t tile0 = blockIdx.x * kSortTile;
    const uint32_t i0 = tile0 + threadIdx.x * kSortItems;
    const uint32_t *R = a.rows + (size_t)c * a.nk;
    const uint32_t *V = a.vals + (size_t)c * a.nk;
    const SlotEntry *sm = a.slot_map[c];
    uint32_t *info = a.seg_info + (size_t)c * a.nk;
    const uint32_t epoch = a.hdr->epoch;
    const bool empty = a.hdr->n_slots[c] == 0;   // the window holds no row yet: no lookups
    const bool nest = a.nested && c == 1;
    uint32_t cnt = 0, kept = 0;
    uint32_t headm = 0, knownm = 0, endm = 0;    // per item bits
    // the rows of the thread's items, and of the keys just before and after
    uint32_t rq[kSortItems];
    load_items(R, i0, n, rq);
    const uint32_t r_before = i0 > 0 && i0 < n ? R[i0 - 1] : 0u;
    const uint32_t r_after = i0 + kSortItems < n ? R[i0 + kSortItems] : 0u;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t i = i0 + j;
        if (i < n) {
            const uint32_t r = rq[j];
            const bool end = i + 1 == n || (j + 1 < kSortItems ? rq[j + 1] : r_after) != r;
            endm |= end ? 1u << j : 0u;
            bool single = false;
            if (i == 0 || (j > 0 ? rq[j - 1] : r_before) != r) {
                bool known = false;
                uint32_t slot = 0;
                if (!empty) {
                    const SlotEntry e = sm[r];
                    known = e.epoch == epoch;
                    slot = e.slot;
                }
                info[i] = known ? slot : kNewHead;
                cnt += known ? 0u : 1u;
                single = end && !(a.fused && known);
                headm |= 1u << j;
                knownm |= known ? 1u << j : 0u;
            }
            kept += single ? 0u : 1u;
        }
    }
    uint32_t total;
    block_excl_scan<kSortThreads>(cnt, s_wave, &total);
    if (threadIdx.x == 0)
        a.blk[(size_t)c * a.nblk + blockIdx.x] = total;
    if (nest) {
        // the tile-local head of each item's segment (-1: the segment began
        // before this tile)
        int last = -1;
#pragma unroll
        for (int j = 0; j < kSortItems; ++j)
            if (headm & (1u << j))
                last = (int)(threadIdx.x * kSortItems + j);
        int carry;
        block_incl_max<kSortThreads>(last, s_iwave, &carry);
        for (int j = threadIdx.x; j < kSortTile; j += kSortThreads)
            s_fail[j] = 0;
        __syncthreads();
        // the payloads and bigram rows of the thread's items (the rows are
        // compared only between keys of one segment of several keys), and
        // the bigram row of the key before the first item if that item
        // continues a segment
        uint32_t vq[kSortItems], bq[kSortItems];
        uint32_t b_prev = 0;
        load_items(V, i0, n, vq);
        load_items(a.btro, i0, n, bq);
        if (i0 < n && !(headm & 1u) && carry >= 0)
            b_prev = a.btro[i0 - 1];
        int hl[kSortItems];
        int run = carry;
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const uint32_t i = i0 + j;
            if (headm & (1u << j))
                run = (int)(threadIdx.x * kSortItems + j);
            hl[j] = i < n ? run : -1;
            if (i >= n || run < 0)
                continue;
            if (headm & (1u << j)) {
                if (knownm & (1u << j))
                    s_fail[run] = 1;   // the window already holds the row
            } else if ((j == 0 ? b_prev : bq[j - 1]) != bq[j]) {
                s_fail[run] = 1;   // another bigram row than the key before
            }
            if (j == kSortItems - 1 || i + 1 == n) {
                // a segment running past the tile is not decided here
                if (i + 1 < n && i + 1 == tile0 + kSortTile && r_after == rq[j])
                    s_fail[run] = 1;
            }
        }
        __syncthreads();
        kept = 0;
        uint32_t rec[kSortItems];
        uint32_t keep[2] = {0u, 0u};   // the kept flags, a byte per item
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const uint32_t i = i0 + j;
            const bool nested = i < n && hl[j] >= 0 && !s_fail[hl[j]];
            const uint32_t v = vq[j];
            const bool hd = (headm & (1u << j)) != 0, ed = (endm & (1u << j)) != 0;
            const uint32_t run_bits = (hd && ed) ? 0u : (kMultiKey | (hd ? kRunHead : 0u) | (ed ? kRunTail : 0u));
            rec[j] = nested ? (rq[j] | (v & 0x80000000u) | run_bits) : kNotSingle;
            keep[j >> 2] |= nested ? 0u : 1u << (8 * (j & 3));
            kept += i < n && !nested ? 1u : 0u;
        }
        store_items(a.tinfo, i0, n, rec);
        if (i0 + kSortItems <= n) {   // i0 is a multiple of 8 and tkept 256-byte aligned
            *reinterpret_cast<uint2 *>(a.tkept + i0) = make_uint2(keep[0], keep[1]);
        } else {
#pragma unroll
            for (int j = 0; j < kSortItems; ++j)
                if (i0 + j < n)
                    a.tkept[i0 + j] = (uint8_t)((keep[j >> 2] >> (8 * (j & 3))) & 1u);
        }
    }
    if (c == 1) {
        block_excl_scan<kSortThreads>(kept, s_wave, &total);
        if (threadIdx.x == 0)
            a.kept[blockIdx.x] = total;
    }
}

// One table: the keys this sort covered (the split records it otherwise).
__global__ void sorted_count_kernel(WsHeader *__restrict__ hdr, const uint32_t *n_dev, uint32_t n_host)
{
    hdr->sorted_n = count_of(n_dev, n_host);
}

// Singleton split of the trigram keys, once the heads have their final info:
// writes every key's singleton-map entry and copies the keys that stay in the
// trigram pass, in order, with their head info to the split arrays;
// hdr->n_multi gets their count.
__global__ __launch_bounds__(kSortThreads) void split_kernel(SlotArgs a)
{
    __shared__ uint32_t s_wave[kSortThreads / kWave];
    constexpr int c = 1;
    const uint32_t b = blockIdx.x;
    const int tid = threadIdx.x;
    const uint32_t n = count_of(a.n_dev, a.n_host);
    const uint32_t upto = b == 0 ? a.nblk : b;
    uint32_t part = 0, part_before = 0;
    for (uint32_t k = tid; k < upto; k += kSortThreads) {
        const uint32_t x = a.kept[k];
        part += x;
        part_before += k < b ? x : 0u;
    }
    uint32_t before_tiles, all_tiles;
    block_excl_scan<kSortThreads>(part_before, s_wave, &before_tiles);
    block_excl_scan<kSortThreads>(part, s_wave, &all_tiles);
    if (b == 0 && tid == 0) {
        a.hdr->n_multi = all_tiles;
        a.hdr->sorted_n = n;   // the keys this sort covered
    }
    const uint32_t i0 = b * kSortTile + tid * kSortItems;
    const uint32_t *R = a.rows + (size_t)c * a.nk;
    const uint32_t *V = a.vals + (size_t)c * a.nk;
    const uint32_t *info = a.seg_info + (size_t)c * a.nk;
    uint32_t keep = 0, cnt = 0;
    uint32_t rq[kSortItems], vq[kSortItems];   // rows and payloads of the items
    if (a.nested) {
        // the map records and the kept flags (a byte per key) were written
        // by mark_kernel
        uint32_t k8[2] = {0u, 0u};
        if (i0 + kSortItems <= n) {   // i0 is a multiple of 8 and tkept 256-byte aligned
            const uint2 t = *reinterpret_cast<const uint2 *>(a.tkept + i0);
            k8[0] = t.x;
            k8[1] = t.y;
        } else {
#pragma unroll
            for (int j = 0; j < kSortItems; ++j)
                if (i0 + j < n)
                    k8[j >> 2] |= (uint32_t)a.tkept[i0 + j] << (8 * (j & 3));
        }
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            if ((k8[j >> 2] >> (8 * (j & 3))) & 0xFFu) {
                keep |= 1u << j;
                ++cnt;
            }
        }
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            rq[j] = 0u;
            vq[j] = 0u;
        }
    } else {
        load_items(R, i0, n, rq);
        load_items(V, i0, n, vq);
        const uint32_t r_before = i0 > 0 && i0 < n ? R[i0 - 1] : 0u;
        const uint32_t r_after = i0 + kSortItems < n ? R[i0 + kSortItems] : 0u;
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const uint32_t i = i0 + j;
            if (i < n) {
                const uint32_t r = rq[j];
                const uint32_t v = vq[j];
                uint32_t rec = kNotSingle;
                if ((i == 0 || (j > 0 ? rq[j - 1] : r_before) != r) &&
                    (i + 1 == n || (j + 1 < kSortItems ? rq[j + 1] : r_after) != r)) {
                    const uint32_t in = info[i];
                    if (a.fused) {
                        if (in == kNewHead)
                            rec = r | (v & 0x80000000u);
                    } else {
                        rec = in == kDropped ? kDropSingle : (in | ((v & 0x80000000u) >> 1));
                    }
                }
                a.tinfo[v & 0x7FFFFFFFu] = rec;
                if (rec == kNotSingle) {
                    keep |= 1u << j;
                    ++cnt;
                }
            }
        }
    }
    uint32_t o = before_tiles + block_excl_scan<kSortThreads>(cnt, s_wave, nullptr);
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        if (keep & (1u << j)) {
            const uint32_t i = i0 + j;
            a.split_rows[o] = a.nested ? R[i] : rq[j];
            a.split_vals[o] = a.nested ? V[i] : vq[j];
            a.split_info[o] = info[i];
            ++o;
        }
    }
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
    uint32_t rq[kSortItems], iq[kSortItems];   // rows and head info of the items
    load_items(R, i0, n, rq);
    load_items(info, i0, n, iq);
    const uint32_t r_before = i0 > 0 && i0 < n ? R[i0 - 1] : 0u;
    uint32_t mask = 0, cnt = 0;
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t i = i0 + j;
        if (i < n && (i == 0 || (j > 0 ? rq[j - 1] : r_before) != rq[j]) && iq[j] == kNewHead) {
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
            const uint32_t r = rq[j];
            if (slot < a.wrows) {
                sm[r] = SlotEntry{epoch, slot};
                a.slot_rows[c][slot] = r;
                iq[j] = slot | 0x80000000u;
            } else {
                iq[j] = kDropped;   // window full: row dropped (flagged)
            }
            ++slot;
        }
    }
    if (mask)   // the thread's items again, the new heads' info changed
        store_items(info, i0, n, iq);
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
    const uint32_t *rows[2];    // per channel: sorted row keys
    const uint32_t *vals[2];    // per channel: dY row code | neg << 31
    const uint32_t *info[2];    // per channel: at segment heads, slot (| new << 31) or kNewHead
    const uint32_t *n_dev[2];   // per channel: device key count (null: n_host)
    uint32_t n_host;            // key count bound (grids cover it)
    const uint8_t *dY;          // [positions][768] of the dY dtype, indexed by the row code
    const uint8_t *const *dy_ptrs;   // burst by reference: dY of each micro-step
    int pos_bits;           // row code = micro-step << pos_bits | position (31: one dY buffer)
    float *gacc;            // [2][wrows][768]
    uint32_t *slot_rows[2];
    int64_t wrows;
    float *partial;         // [2][nchunk][2][768]
    uint64_t *owners;       // [2][nchunk]: chunk | info << 32
    int64_t nchunk;
    float *gpart;           // [2][ngroup][768]: sums of groups of kGroup chunks inside one segment
    int64_t ngroup;
    WsHeader *hdr;
    const uint32_t *tinfo;  // singleton map (see SlotArgs)
    bool nested;            // the map also names nested trigram rows of several keys (kMultiKey)
    const uint32_t *tix0;   // nested: per sorted bigram key, its index in the trigram order
                            // (the singleton map's index); else the map is indexed by row code
    float *tpart;           // nested: [nchunk][2][768] pieces of runs that cross a walk's end
    uint64_t *trec;         // nested: [nchunk] such runs, chunk of the first piece | record << 32
    bool burst;             // the keys are the burst stash's: check the window is ready
    FuseArgs f;             // fused modes only
};

// Burst modes: a window is reduced only if every micro-step whose keys are
// kept has its gradients attached (else a dY row code could name gradients
// that never came) and its keys were sorted after the last of them.
// Otherwise the launch does nothing and flags the window (one thread).
__device__ __forceinline__ bool window_ready(const RedArgs &a)
{
    if (!a.burst)
        return true;
    const WsHeader *h = a.hdr;
    const bool ok = h->n_micro == h->n_keyed && h->sorted_n == h->n_stash;
    if (!ok && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        atomicOr(&a.hdr->flags, NGRAM_FLAG_WINDOW_UNREADY);
        a.hdr->dropped = 1;   // the window's step changes nothing
    }
    return ok;
}

__device__ __forceinline__ float4 add4(float4 a, float4 b)
{
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

__device__ __forceinline__ uint32_t lane_val(uint32_t v0, uint32_t v1, int j)
{
    return j < kWave ? (uint32_t)__builtin_amdgcn_readlane((int)v0, j)
                     : (uint32_t)__builtin_amdgcn_readlane((int)v1, j - kWave);
}

constexpr int kPer = kDim / kWave;   // 12 elements of a row per lane

// Which keys of its 64-key chunk a wavefront consumes, and how its first and
// last pieces are finished.  Keys are consumed in order; a segment's sum is
// reset at its first key and flushed at its last:
//   - a segment that starts and ends here is finished here;
//   - the first piece, if it continues a segment from the previous chunk, is
//     skipped when that chunk finishes it, else left as partial row 0;
//   - the last piece, if it spills into the next chunk, is finished here when
//     it ends within that chunk (its keys are loaded as lanes 64..127), else
//     left as partial row 1 with a fix-up record.
struct ChunkPlan {
    uint32_t r0, v0, i0;   // this lane's key: row, dY row code | sign, head info
    uint32_t v1;           // lanes 64..127: keys of an owned spill-over
    uint64_t hm;           // segment heads among the chunk's keys
    int nv;                // keys in the chunk
    int j0, jend;          // keys this wavefront consumes
    int la;                // first key of the last piece (-1: no head)
    bool first_cont;       // key 0 continues the previous chunk's segment
    bool last_spills;      // the last piece continues into the next chunk
    bool owner_full;       // ... and this chunk finishes it
    uint32_t row_last;
};

// False if the chunk is past the end of the keys.
__device__ __forceinline__ bool chunk_plan(const RedArgs &a, int c, int64_t chunk, uint32_t n, int lane,
                                           ChunkPlan &p)
{
    const int64_t c0 = chunk * kChunk;
    if (c0 >= n)
        return false;
    const uint32_t *R = a.rows[c];
    const uint32_t *V = a.vals[c];
    const uint32_t *I = a.info[c];
    p.nv = (int)min<int64_t>(kChunk, (int64_t)n - c0);
    const bool valid = lane < p.nv;
    p.r0 = valid ? R[c0 + lane] : 0xFFFFFFFFu;
    p.v0 = valid ? V[c0 + lane] : 0u;
    uint32_t prev = __shfl_up(p.r0, 1);
    if (lane == 0)
        prev = c0 > 0 ? R[c0 - 1] : 0xFFFFFFFFu;
    const bool head = valid && (p.r0 != prev);
    p.hm = __ballot(head);
    p.i0 = head ? I[c0 + lane] : 0u;
    p.row_last = (uint32_t)__builtin_amdgcn_readlane((int)p.r0, p.nv - 1);
    const bool cont_after = p.nv == kChunk && c0 + kChunk < n && R[c0 + kChunk] == p.row_last;

    p.first_cont = !(p.hm & 1ull);
    const int e0 = p.hm ? (int)__builtin_ctzll(p.hm) : p.nv;   // end of the first piece
    bool skip_first = false;
    if (p.first_cont) {
        const uint32_t row0 = (uint32_t)__builtin_amdgcn_readlane((int)p.r0, 0);
        const bool piece0_cont = (e0 == p.nv) && cont_after;
        const bool head_in_prev = (c0 == kChunk) || (R[c0 - kChunk - 1] != row0);
        skip_first = head_in_prev && !piece0_cont;
    }
    p.la = p.hm ? 63 - (int)__builtin_clzll(p.hm) : -1;
    p.last_spills = p.hm && cont_after;
    p.owner_full = false;
    p.v1 = 0;
    int extra = 0;
    if (p.last_spills) {
        p.owner_full = !(c0 + 2 * kChunk < n && R[c0 + 2 * kChunk] == p.row_last);
        if (p.owner_full) {
            const int64_t i1 = c0 + kChunk + lane;
            const bool ok1 = i1 < n;
            const uint32_t r1 = ok1 ? R[i1] : 0xFFFFFFFFu;
            p.v1 = ok1 ? V[i1] : 0u;
            extra = __popcll(__ballot(ok1 && r1 == p.row_last));
        }
    }
    p.j0 = skip_first ? e0 : 0;
    p.jend = p.owner_full ? kChunk + extra : p.nv;
    return true;
}

// Does the open segment end at key k?
__device__ __forceinline__ bool seg_ends(const ChunkPlan &p, int k)
{
    if (k >= kChunk - 1 && p.owner_full)
        return k == p.jend - 1;
    if (k == p.nv - 1)
        return true;
    return (k + 1 < kChunk) && ((p.hm >> (k + 1)) & 1ull);
}

// Lane m < 64 holds the base address of micro-step m's dY (burst by
// reference) or, with one dY buffer, every lane holds that buffer's address;
// a key's dY row address then needs no dependent load and no branch.
__device__ __forceinline__ uint64_t dy_lane_base(const RedArgs &a, int lane)
{
    return a.dy_ptrs ? (uint64_t)a.dy_ptrs[lane] : (uint64_t)a.dY;
}

template <int DYE>
__device__ __forceinline__ uint64_t dy_row_addr(const RedArgs &a, uint64_t lane_base, uint32_t code)
{
    const int m = (int)(code >> a.pos_bits);   // uniform across the wavefront
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lane_base, m);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(lane_base >> 32), m);
    const uint32_t pos = code & (uint32_t)((1ull << a.pos_bits) - 1u);
    return ((uint64_t)lo | ((uint64_t)hi << 32)) + (uint64_t)pos * (kDim * DYE);
}

// dY elements are loaded as raw bits (DYE bytes each) and widened to fp32 only
// where they are used, so a batch's loads stay in flight together; a bf16
// value widens exactly.
template <int DYE>
__device__ __forceinline__ float dy_f32(uint32_t raw)
{
    return DYE == 4 ? __uint_as_float(raw) : __uint_as_float(raw << 16);
}

// The chunk's per-lane values are read through readlane inside the key loop.
__device__ __forceinline__ void settle_plan(ChunkPlan &p)
{
    settle(p.r0);
    settle(p.v0);
    settle(p.i0);
    settle(p.v1);
}

// Partial row of a piece that another chunk or the fix-up finishes.
template <typename Store>
__device__ __forceinline__ void flush_partial(const RedArgs &a, const ChunkPlan &p, int c, int64_t chunk, int ps,
                                              int lane, Store store)
{
    const uint64_t base = (uint64_t)a.partial + (((uint64_t)c * a.nchunk + chunk) * 2) * (kDim * 4);
    if (ps == 0 && p.first_cont) {
        store(base);
    } else {
        const uint32_t info = (uint32_t)__builtin_amdgcn_readlane((int)p.i0, ps);
        store(base + kDim * 4);
        if (lane == 0) {
            const uint32_t k2 = atomicAdd(&a.hdr->n_owner[c], 1u);
            a.owners[(size_t)c * a.nchunk + k2] = (uint64_t)chunk | ((uint64_t)info << 32);
        }
    }
}

// Accumulating reduction (one wavefront per 64 sorted keys, kRedU dY rows in
// flight whatever the segment boundaries): each finished segment goes to its
// window row.  With the singleton split the bigram pass also writes, for
// every key it reads, the signed dY row into the window slot of that
// position's trigram row when the singleton map names one.  Lane l holds elements l + 64 m (m = 0..11), so every load,
// store and atomic of a row is twelve 256-byte contiguous wavefront accesses.
template <int DYE>
__global__ __launch_bounds__(kRedThreads) void seg_reduce_kernel(RedArgs a)
{
    const int c = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t chunk = (int64_t)blockIdx.x * (kRedThreads / kWave) + threadIdx.x / kWave;
    const uint32_t n = count_of(a.n_dev[c], a.n_host);
    if (!window_ready(a))
        return;
    if (chunk == 0 && lane == 0)
        a.hdr->n_slots[c] = a.hdr->n_next[c];   // the slots assign_kernel handed out
    ChunkPlan p;
    if (!chunk_plan(a, c, chunk, n, lane, p))
        return;
    const bool tsplit = a.tinfo != nullptr && c == 0;
    uint32_t t0 = kNotSingle, t1 = kNotSingle;   // singleton-map entries of keys lane, 64 + lane
    if (tsplit) {
        if (lane < p.nv)
            t0 = a.tinfo[p.v0 & 0x7FFFFFFFu];
        if (p.owner_full && kChunk + lane < p.jend)
            t1 = a.tinfo[p.v1 & 0x7FFFFFFFu];
    }
    uint64_t lane_base = dy_lane_base(a, lane);
    settle_plan(p);
    settle(lane_base);
    settle(t0);
    settle(t1);
    const uint64_t gacc = (uint64_t)a.gacc + (uint64_t)c * a.wrows * (kDim * 4) + 4 * lane;
    const uint64_t gacc_t = (uint64_t)a.gacc + (uint64_t)a.wrows * (kDim * 4) + 4 * lane;

    float acc[kPer];
    int ps = p.j0;   // start key of the open segment
#pragma unroll
    for (int m = 0; m < kPer; ++m)
        acc[m] = 0.f;
    for (int j = p.j0; j < p.jend; j += kRedU) {
        uint32_t x[kRedU][kPer];   // raw dY bits
        uint32_t sg[kRedU];
#pragma unroll
        for (int u = 0; u < kRedU; ++u) {
            if (j + u < p.jend) {
                const uint32_t v = lane_val(p.v0, p.v1, j + u);
                sg[u] = v & 0x80000000u;
                const uint64_t q = dy_row_addr<DYE>(a, lane_base, v & 0x7FFFFFFFu) + DYE * lane;
#pragma unroll
                for (int m = 0; m < kPer; ++m)
                    x[u][m] = DYE == 4 ? ld_global_nt<uint32_t>(q + m * kWave * 4)
                                       : (uint32_t)ld_global_nt<uint16_t>(q + m * kWave * 2);
            }
        }
#pragma unroll
        for (int u = 0; u < kRedU; ++u) {
            const int k = j + u;
            if (k >= p.jend)
                break;
            if (k < kChunk && k != p.j0 && ((p.hm >> k) & 1ull)) {
                ps = k;
#pragma unroll
                for (int m = 0; m < kPer; ++m)
                    acc[m] = 0.f;
            }
            const float sgn = sg[u] ? -1.f : 1.f;   // acc +- dY, one rounding
#pragma unroll
            for (int m = 0; m < kPer; ++m)
                acc[m] = fmaf(dy_f32<DYE>(x[u][m]), sgn, acc[m]);
            if (tsplit) {
                // this position's trigram row, if a singleton: its whole sum is
                // s_t dY, stored into a new slot or added (its one addition of
                // this launch) into an existing one
                const uint32_t tv = lane_val(t0, t1, k);
                if (tv != kNotSingle && tv != kDropSingle) {
                    const float ts = (tv & 0x40000000u) ? -1.f : 1.f;
                    const uint64_t g = gacc_t + (uint64_t)(tv & 0x3FFFFFFFu) * (kDim * 4);
                    if (tv >> 31) {
#pragma unroll
                        for (int m = 0; m < kPer; ++m)
                            st_global<float>(g + m * kWave * 4, ts * dy_f32<DYE>(x[u][m]));
                    } else {
#pragma unroll
                        for (int m = 0; m < kPer; ++m)
                            atomic_add_global(g + m * kWave * 4, ts * dy_f32<DYE>(x[u][m]));
                    }
                }
            }
            if (!seg_ends(p, k))
                continue;
            if ((ps == 0 && p.first_cont) || (ps == p.la && p.last_spills && !p.owner_full)) {
                flush_partial(a, p, c, chunk, ps, lane, [&](uint64_t dst) {
#pragma unroll
                    for (int m = 0; m < kPer; ++m)
                        st_global<float>(dst + 4 * (lane + m * kWave), acc[m]);
                });
                continue;
            }
            // A row new to the window is written; an existing one gets G += S
            // through fire-and-forget atomic adds executed in L2 (the
            // wavefront does not wait for the old row).  Every window row has
            // exactly one segment, hence one writer, per launch, so each
            // element sees a single addition and the result is the plain fp32
            // sum G + S, whatever the timing.
            const uint32_t info = (uint32_t)__builtin_amdgcn_readlane((int)p.i0, ps);
            if (info == kDropped)
                continue;   // window full: row dropped (flagged when slots were assigned)
            const uint64_t g = gacc + (uint64_t)(info & 0x7FFFFFFFu) * (kDim * 4);
            if (info >> 31) {
#pragma unroll
                for (int m = 0; m < kPer; ++m)
                    st_global<float>(g + m * kWave * 4, acc[m]);
            } else {
#pragma unroll
                for (int m = 0; m < kPer; ++m)
                    atomic_add_global(g + m * kWave * 4, acc[m]);
            }
        }
    }
}

// ----------------------------------------------- reduction fused with step
//
// The same walk over the sorted keys, but a finished segment is the row's
// complete window gradient G (plus what the window already holds for it, if
// anything): the row is stepped at once and G never goes to memory.  Here
// lane l holds elements 4l..4l+3 of each 256-wide third of a row, so a dY
// row is three 1 KB wavefront loads and a bf16 table row three 512 B ones.
// The table row and state of every segment that ends among the keys of a
// batch are loaded together with the batch's dY rows, so a short segment
// costs one memory round trip, not two.

constexpr int kQ = kDim / (4 * kWave);   // 3 float4 per lane
constexpr int kStepU = 2;   // keys per batch

template <int ELT>
struct WRow;
template <>
struct WRow<2> {   // 4 bf16
    uint2 q[kQ];
};
template <>
struct WRow<4> {   // 4 fp32
    float4 q[kQ];
};

// addr: the row's start + this lane's offset (ELT * 4 * lane).
template <int ELT>
__device__ __forceinline__ void load_wrow(WRow<ELT> &w, uint64_t addr)
{
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        if constexpr (ELT == 2)
            w.q[q] = ld_global_nt<uint2>(addr + q * kWave * 8);
        else
            w.q[q] = ld_global_nt<float4>(addr + q * kWave * 16);
    }
}

// W <- W - scale * G, rounded once to the table dtype.  bf16: the hardware's
// round-to-nearest-even pair conversion; if any lane holds a NaN the whole
// wavefront takes the bitwise rounding instead, which writes NaN as 0x7FC0.
template <int ELT>
__device__ __forceinline__ void store_stepped(const WRow<ELT> &w, const float4 (&g)[kQ], float scale, uint64_t addr)
{
    if constexpr (ELT == 2) {
        float r[kQ][4];
        bool nan = false;
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const uint2 x = w.q[q];
            r[q][0] = bf16_lo(x.x) - scale * g[q].x;
            r[q][1] = bf16_hi(x.x) - scale * g[q].y;
            r[q][2] = bf16_lo(x.y) - scale * g[q].z;
            r[q][3] = bf16_hi(x.y) - scale * g[q].w;
            nan |= __builtin_isunordered(r[q][0], r[q][1]) | __builtin_isunordered(r[q][2], r[q][3]);
        }
        if (!__any(nan)) {
#pragma unroll
            for (int q = 0; q < kQ; ++q)
                st_global_nt<uint2>(addr + q * kWave * 8,
                                 make_uint2(bf16_pack_rne(r[q][0], r[q][1]), bf16_pack_rne(r[q][2], r[q][3])));
        } else {
#pragma unroll
            for (int q = 0; q < kQ; ++q)
                st_global_nt<uint2>(addr + q * kWave * 8,
                                 make_uint2(bf16_pack(r[q][0], r[q][1]), bf16_pack(r[q][2], r[q][3])));
        }
    } else {
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const float4 x = w.q[q];
            st_global_nt<float4>(addr + q * kWave * 16, make_float4(x.x - scale * g[q].x, x.y - scale * g[q].y,
                                                                 x.z - scale * g[q].z, x.w - scale * g[q].w));
        }
    }
}

// One row's step from its complete window gradient g (sum of squares by the
// wavefront), its prefetched table row w and state st.
template <int ELT>
__device__ __forceinline__ void step_one(const float4 (&g)[kQ], const WRow<ELT> &w, RowState st, uint32_t row,
                                         uint64_t table, uint64_t state, const RedArgs &a, const StepParams &sp,
                                         bool sp_ok, int lane)
{
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
        ss += g[q].x * g[q].x + g[q].y * g[q].y + g[q].z * g[q].z + g[q].w * g[q].w;
    ss = wave_sum(ss);
    float vn;
    bool order_bad;
    const float scale = step_scale(ss, st, sp, vn, order_bad);
    if (!sp_ok)
        return;
    store_stepped<ELT>(w, g, scale, table + (uint64_t)row * (kDim * ELT));
    if (lane == 0) {
        st_global<RowState>(state + (uint64_t)row * sizeof(RowState), RowState{vn, sp.t});
        if (order_bad)
            atomicOr(&a.hdr->flags, NGRAM_FLAG_STEP_ORDER);
    }
}

// With the singleton split, the bigram pass (channel 0) also steps, for every
// key it reads, the trigram row of that key's position when tinfo marks it a
// singleton (its gradient is s_t dY of this very row of dY) or the end of a
// nested run; the trigram pass then only walks the keys the split kept.
// Four consecutive dY elements of one lane: raw bits as loaded (16 bytes of
// fp32 or 8 bytes of bf16), widened where they are used.
template <int DYE>
struct DyQuad;
template <>
struct DyQuad<4> {
    typedef uint4 type;
};
template <>
struct DyQuad<2> {
    typedef uint2 type;
};

__device__ __forceinline__ float4 dy_quad_f32(uint4 x)
{
    return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
}

__device__ __forceinline__ float4 dy_quad_f32(uint2 x)
{
    return make_float4(bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y));
}

// Three wavefronts per SIMD with two keys per batch (at most 168 VGPRs, no
// spills) keep more loads in flight per CU than two wavefronts with four keys
// per batch: 1.3 % faster with fp32 dY, 2-4 % with bf16 dY on the full table.
// fp32 tables (wider row registers; small tables only) take two wavefronts
// per SIMD, which leaves the compiler room without spilling.
template <int ELT>
constexpr int kStepWaves = ELT == 2 ? 3 : 2;
template <int ELT, int DYE>
__global__ __launch_bounds__(kRedThreads) __attribute__((amdgpu_waves_per_eu(kStepWaves<ELT>, kStepWaves<ELT>))) void seg_step_kernel(RedArgs a)
{
    // per wavefront: the running sum of the nested trigram run being walked
    // (lane l holds elements 4l..4l+3 of each third, as in registers)
    __shared__ float4 s_tacc[kRedThreads / kWave][kQ][kWave];
    const int c = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t chunk = (int64_t)blockIdx.x * (kRedThreads / kWave) + threadIdx.x / kWave;
    const uint32_t n = count_of(a.n_dev[c], a.n_host);
    if (!window_ready(a))
        return;
    ChunkPlan p;
    if (!chunk_plan(a, c, chunk, n, lane, p))
        return;
    const bool tsplit = a.tinfo != nullptr && c == 0;
    uint32_t t0 = kNotSingle, t1 = kNotSingle;   // trigram singleton of keys lane, 64 + lane
    if (tsplit) {
        const int64_t c0 = chunk * kChunk;
        if (lane < p.nv)
            t0 = a.tinfo[a.tix0 ? a.tix0[c0 + lane] : (p.v0 & 0x7FFFFFFFu)];
        if (p.owner_full && kChunk + lane < p.jend)
            t1 = a.tinfo[a.tix0 ? a.tix0[c0 + kChunk + lane] : (p.v1 & 0x7FFFFFFFu)];
    }
    // nested runs: keys j0 .. kc_end continue a run from the walk before
    // (the walk's first piece of that run, completed by the fix-up)
    int kc_end = -1;
    if (tsplit && a.nested && p.j0 < p.jend) {
        const uint32_t tj = (uint32_t)__builtin_amdgcn_readlane((int)t0, p.j0);
        if (is_run(tj) && !(tj & kRunHead)) {
            const uint64_t tails = __ballot(is_run(t0) && (t0 & kRunTail)) & (~0ull << p.j0);
            kc_end = tails ? (int)__builtin_ctzll(tails) : p.nv - 1;
        }
    }
    uint64_t lane_base = dy_lane_base(a, lane);
    settle_plan(p);
    settle(lane_base);
    settle(t0);
    settle(t1);
    const uint64_t table = (uint64_t)a.f.w[c] + (uint64_t)ELT * 4 * lane;
    const uint64_t state = (uint64_t)a.f.st[c];
    const uint64_t table_t = (uint64_t)a.f.w[1] + (uint64_t)ELT * 4 * lane;
    const uint64_t state_t = (uint64_t)a.f.st[1];
    const uint64_t gacc = (uint64_t)a.gacc + (uint64_t)c * a.wrows * (kDim * 4) + 16 * lane;
    bool sp_ok;
    const StepParams sp = step_params(a.f.p, a.f.p_dev, sp_ok);

    // keys 0..63 that end a segment stepped here (not a partial piece); an
    // owned spill-over ends at jend - 1 >= 64
    uint64_t fin = (p.hm >> 1) | (1ull << (p.nv - 1));
    if (p.first_cont && p.j0 == 0) {
        const int e0 = p.hm ? (int)__builtin_ctzll(p.hm) : p.nv;
        fin &= ~(1ull << (e0 - 1));
    }
    if (p.last_spills)
        fin &= ~(1ull << 63);   // nv == 64: finished past the chunk or left partial

    float4 acc[kQ];
    int ps = p.j0;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
        acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = p.j0; j < p.jend; j += kStepU) {
        typename DyQuad<DYE>::type x[kStepU][kQ];   // raw dY bits
        uint32_t sg[kStepU];
        WRow<ELT> w[kStepU], wt[kStepU];
        RowState st[kStepU], stt[kStepU];
        uint32_t row[kStepU], tv[kStepU];
        bool ends_here[kStepU], tlast[kStepU];
#pragma unroll
        for (int u = 0; u < kStepU; ++u) {
            const int k = j + u;
            ends_here[u] = false;
            tlast[u] = false;
            tv[u] = kNotSingle;
            if (k < p.jend) {
                const uint32_t v = lane_val(p.v0, p.v1, k);
                sg[u] = v & 0x80000000u;
                const uint64_t q = dy_row_addr<DYE>(a, lane_base, v & 0x7FFFFFFFu) + 4 * DYE * lane;
#pragma unroll
                for (int qq = 0; qq < kQ; ++qq)
                    x[u][qq] = ld_global_nt<typename DyQuad<DYE>::type>(q + qq * kWave * 4 * DYE);
                ends_here[u] = k < kChunk ? ((fin >> k) & 1ull) != 0 : (p.owner_full && k == p.jend - 1);
                if (ends_here[u]) {
                    row[u] = k < kChunk ? (uint32_t)__builtin_amdgcn_readlane((int)p.r0, k) : p.row_last;
                    load_wrow<ELT>(w[u], table + (uint64_t)row[u] * (kDim * ELT));
                    st[u] = ld_global_nt<RowState>(state + (uint64_t)row[u] * sizeof(RowState));
                }
                if (tsplit) {
                    tv[u] = lane_val(t0, t1, k);
                    if (tv[u] != kNotSingle) {
                        // the key that completes its trigram row: a singleton, or
                        // the last key of a nested run that began in this walk
                        tlast[u] = !(a.nested && (tv[u] & kMultiKey)) || (k > kc_end && (tv[u] & kRunTail));
                        if (tlast[u]) {
                            const uint32_t tr = tv[u] & (a.nested ? kTrowMask : 0x7FFFFFFFu);
                            load_wrow<ELT>(wt[u], table_t + (uint64_t)tr * (kDim * ELT));
                            stt[u] = ld_global_nt<RowState>(state_t + (uint64_t)tr * sizeof(RowState));
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kStepU; ++u) {
            const int k = j + u;
            if (k >= p.jend)
                break;
            if (k < kChunk && k != p.j0 && ((p.hm >> k) & 1ull)) {
                ps = k;
#pragma unroll
                for (int q = 0; q < kQ; ++q)
                    acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            // s dY + acc: the product by +-1 is exact, so this is acc +- dY
            // with a single rounding
            const float sgn = sg[u] ? -1.f : 1.f;
#pragma unroll
            for (int q = 0; q < kQ; ++q) {
                const float4 d = dy_quad_f32(x[u][q]);
                acc[q].x = fmaf(d.x, sgn, acc[q].x);
                acc[q].y = fmaf(d.y, sgn, acc[q].y);
                acc[q].z = fmaf(d.z, sgn, acc[q].z);
                acc[q].w = fmaf(d.w, sgn, acc[q].w);
            }
            if (tv[u] != kNotSingle) {
                // this position's trigram row is completed here: G = s_t dY for a
                // singleton; a nested run adds s_t dY of its keys in order, the
                // running sum kept in LDS between keys
                const float ts = (tv[u] & 0x80000000u) ? -1.f : 1.f;
                float4 g[kQ];
#pragma unroll
                for (int q = 0; q < kQ; ++q) {
                    const float4 d = dy_quad_f32(x[u][q]);
                    g[q] = make_float4(ts * d.x, ts * d.y, ts * d.z, ts * d.w);
                }
                const int wv = threadIdx.x / kWave;
                const bool run = a.nested && (tv[u] & kMultiKey);
                if (run && k != p.j0 && !(tv[u] & kRunHead)) {   // the key before is of the same run
#pragma unroll
                    for (int q = 0; q < kQ; ++q)
                        g[q] = add4(s_tacc[wv][q][lane], g[q]);
                }
                if (tlast[u]) {
                    step_one<ELT>(g, wt[u], stt[u], tv[u] & (a.nested ? kTrowMask : 0x7FFFFFFFu), table_t, state_t,
                                  a, sp, sp_ok, lane);
                } else if (run && (k == kc_end || k == p.jend - 1)) {
                    // a piece of a run that crosses the walk's start (slot 0) or
                    // end (slot 1); the fix-up adds the pieces and steps the row
                    const int slot = k <= kc_end ? 0 : 1;
                    const uint64_t dst = (uint64_t)a.tpart + ((uint64_t)chunk * 2 + slot) * (kDim * 4) + 16 * lane;
#pragma unroll
                    for (int q = 0; q < kQ; ++q)
                        st_global<float4>(dst + q * (kWave * 16), g[q]);
                    if (slot == 1 && lane == 0) {
                        const uint32_t k2 = atomicAdd(&a.hdr->n_trun, 1u);
                        a.trec[k2] = (uint64_t)chunk | ((uint64_t)tv[u] << 32);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < kQ; ++q)
                        s_tacc[wv][q][lane] = g[q];
                }
            }
            if (ends_here[u]) {
                const uint32_t info = (uint32_t)__builtin_amdgcn_readlane((int)p.i0, ps);
                float4 g[kQ];
#pragma unroll
                for (int q = 0; q < kQ; ++q)
                    g[q] = acc[q];
                if (info != kNewHead) {   // G = G_window + S, as the accumulating path adds it
                    const uint64_t gw = gacc + (uint64_t)info * (kDim * 4);
#pragma unroll
                    for (int q = 0; q < kQ; ++q)
                        g[q] = add4(ld_global_nt<float4>(gw + q * kWave * 16), g[q]);
                    if (lane == 0)
                        a.slot_rows[c][info] = row[u] | kSlotStepped;
                }
                step_one<ELT>(g, w[u], st[u], row[u], table, state, a, sp, sp_ok, lane);
            } else if (seg_ends(p, k)) {
                flush_partial(a, p, c, chunk, ps, lane, [&](uint64_t dst) {
#pragma unroll
                    for (int q = 0; q < kQ; ++q)
                        st_global<float4>(dst + 16 * (lane + q * kWave), acc[q]);
                });
            }
        }
    }
}

// Long segments (hot n-grams: up to thousands of chunks) leave one partial row
// per chunk.  A group of kGroup chunks that lies inside one segment -- the
// keys just before and just after the group have the same row, so every
// chunk of the group starts and ends inside that segment and its partial row
// 0 is the whole chunk -- is summed here once, in a fixed order (4 runs of 16
// chunks, then the runs in order), and the fix-up adds the group's sum
// instead of its kGroup pieces.
constexpr int kGroupThreads = 256;
__global__ __launch_bounds__(kGroupThreads) void group_sum_kernel(RedArgs a)
{
    constexpr int kW = kGroupThreads / kWave;
    constexpr int kRun = kGroup / kW;
    __shared__ float4 s_part[kW][kDim / 4];
    const int c = blockIdx.y;
    const int64_t g = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int64_t n = count_of(a.n_dev[c], a.n_host);
    const int64_t k0 = g * kGroup * kChunk;   // the group's first key
    const int64_t k1 = k0 + kGroup * kChunk;  // the first key after it
    if (g == 0 || k1 >= n)
        return;
    const uint32_t *R = a.rows[c];
    if (R[k0 - 1] != R[k1])
        return;   // not inside one segment
    const float4 *P = reinterpret_cast<const float4 *>(a.partial + (size_t)c * a.nchunk * 2 * kDim);
    float4 acc[3] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f),
                     make_float4(0.f, 0.f, 0.f, 0.f)};
    const int64_t c0 = g * kGroup + w * kRun;
    for (int i = 0; i < kRun; i += kRedU) {
        float4 x[kRedU][3];
#pragma unroll
        for (int u = 0; u < kRedU; ++u) {
            const float4 *s = P + (c0 + i + u) * 2 * (kDim / 4) + lane;   // partial row 0 of the chunk
#pragma unroll
            for (int q = 0; q < 3; ++q)
                x[u][q] = s[q * kWave];
        }
#pragma unroll
        for (int u = 0; u < kRedU; ++u)
#pragma unroll
            for (int q = 0; q < 3; ++q)
                acc[q] = add4(acc[q], x[u][q]);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
        s_part[w][lane + q * kWave] = acc[q];
    __syncthreads();
    if (tid < kDim / 4) {
        float4 sum = s_part[0][tid];
#pragma unroll
        for (int ww = 1; ww < kW; ++ww)
            sum = add4(sum, s_part[ww][tid]);
        reinterpret_cast<float4 *>(a.gpart + ((size_t)c * a.ngroup + g) * kDim)[tid] = sum;
    }
}

// Sums the partial rows of each segment longer than two chunks: the starting
// chunk's tail piece, then the following chunks' head pieces -- the sums of
// the whole groups inside the segment in place of their chunks' pieces --
// split into 8 contiguous runs (one per wavefront) that are added in run
// order.  Then the row goes to the window, or (fused) is completed and
// stepped by the block.  Most segments span 3 or 4 chunks and a record's
// time is its chain of dependent loads, so blocks of 512 threads, one record
// each at a time over twice as many blocks as with 1,024 threads, overlap more
// of the chains (the full window's fix-up 35.8 -> 26.2 us).
constexpr int kFixThreads = 512;
template <int MODE>
__global__ __launch_bounds__(kFixThreads) void fixup_kernel(RedArgs a)
{
    constexpr int kW = kFixThreads / kWave;
    __shared__ float4 s_part[kW][kDim / 4];
    __shared__ float s_ss[kW];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    // the records of both channels are shared out over all blocks of the grid
    const uint32_t blk = blockIdx.x + blockIdx.y * gridDim.x, nblk = gridDim.x * gridDim.y;
    const uint32_t nown0 = a.hdr->n_owner[0];
    const uint32_t nown_all = nown0 + (gridDim.y > 1 ? a.hdr->n_owner[1] : 0u);
    bool sp_ok = true;
    const StepParams sp = MODE == kAccum ? a.f.p : step_params(a.f.p, a.f.p_dev, sp_ok);
    for (uint32_t u = blk; u < nown_all; u += nblk) {
        const int c = u < nown0 ? 0 : 1;
        const uint32_t k = u - (c ? nown0 : 0u);
        const uint32_t n = count_of(a.n_dev[c], a.n_host);
        const uint32_t *R = a.rows[c];
        const float4 *P = reinterpret_cast<const float4 *>(a.partial + (size_t)c * a.nchunk * 2 * kDim);
        const uint64_t rec = a.owners[(size_t)c * a.nchunk + k];
        const int64_t chunk = (int64_t)(uint32_t)rec;
        const uint32_t info = (uint32_t)(rec >> 32);
        const uint32_t row = R[chunk * kChunk + kChunk - 1];
        // what the row's completion needs besides the sum, loaded first so
        // that it arrives while the pieces are found and added: the window
        // row (if the window holds the row), and (fused) the table row and
        // the row's state.  Thread t < 192 owns elements 4t .. 4t+3.
        const bool in_window = MODE == kAccum ? (info != kDropped && !(info >> 31)) : info != kNewHead;
        const uint32_t slot = MODE == kAccum ? (info & 0x7FFFFFFFu) : info;
        float4 gw = make_float4(0.f, 0.f, 0.f, 0.f);
        uint2 wb = make_uint2(0u, 0u);
        float4 wf = make_float4(0.f, 0.f, 0.f, 0.f);
        RowState st = RowState{0.f, 0};
        if (tid < kDim / 4) {
            if (in_window)
                gw = ld_global_nt<float4>((uint64_t)(a.gacc + ((size_t)c * a.wrows + slot) * kDim) + 16 * tid);
            if (MODE == kFuseBf16)
                wb = ld_global_nt<uint2>((uint64_t)(a.f.w[c] + (size_t)row * kDim * 2) + 8 * tid);
            else if (MODE == kFuseF32)
                wf = ld_global_nt<float4>((uint64_t)(a.f.w[c] + (size_t)row * kDim * 4) + 16 * tid);
        }
        if (MODE != kAccum)
            st = ld_global_nt<RowState>((uint64_t)(a.f.st[c] + row));
        // m = following chunks that start inside the segment (rows are
        // sorted, so they are consecutive): every wavefront probes the next
        // 64 chunk heads; a segment longer than that is scanned by the whole
        // block, kFixThreads heads at a time
        int64_t m = 0;
        {
            const int64_t cc = chunk + 1 + lane;
            const bool hit = cc * kChunk < (int64_t)n && R[cc * kChunk] == row;
            m = __popcll(__ballot(hit));
        }
        if (m == kWave) {
            for (;;) {
                const int64_t cc = chunk + 1 + m + tid;
                const bool hit = cc * kChunk < (int64_t)n && R[cc * kChunk] == row;
                const int cnt = __syncthreads_count(hit);
                m += cnt;
                if (cnt < kFixThreads)
                    break;
            }
        }
        // items: the owner's tail piece; the head pieces of chunks first ..
        // 64 g_lo - 1; the sums of groups g_lo .. g_hi - 1 (chunks inside
        // first .. last - 1); the head pieces of chunks 64 g_hi .. last
        const int64_t first = chunk + 1, last = chunk + m;
        const int64_t g_lo = (first + kGroup - 1) / kGroup, g_hi = last / kGroup;
        const int64_t ng = g_hi > g_lo ? g_hi - g_lo : 0;
        const int64_t n_before = ng ? g_lo * kGroup - first : m;
        const int64_t np = 1 + n_before + ng + (ng ? last - g_hi * kGroup + 1 : 0);
        const float4 *G4 = reinterpret_cast<const float4 *>(a.gpart + (size_t)c * a.ngroup * kDim);
        auto item = [&](int64_t q) -> const float4 * {
            if (q == 0)
                return P + (chunk * 2 + 1) * (kDim / 4);
            if (q <= n_before)
                return P + (first + q - 1) * 2 * (kDim / 4);
            if (q <= n_before + ng)
                return G4 + (g_lo + q - 1 - n_before) * (kDim / 4);
            return P + (g_hi * kGroup + q - 1 - n_before - ng) * 2 * (kDim / 4);
        };
        const int64_t lo = np * w / kW, hi = np * (w + 1) / kW;
        float4 acc[3] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f),
                         make_float4(0.f, 0.f, 0.f, 0.f)};
        for (int64_t p = lo; p < hi; p += kRedU) {
            float4 x[kRedU][3];
#pragma unroll
            for (int u = 0; u < kRedU; ++u) {
                if (p + u < hi) {
                    const float4 *s = item(p + u) + lane;
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
            if (in_window)
                sum = add4(gw, sum);   // G = window row + this reduction's sum
        }
        if (MODE == kAccum) {
            if (tid < kDim / 4 && info != kDropped)
                st_global<float4>((uint64_t)(a.gacc + ((size_t)c * a.wrows + slot) * kDim) + 16 * tid, sum);
        } else {
            // step the row with the block
            if (tid == 0 && in_window)
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
            float vn;
            bool order_bad;
            const float scale = step_scale(ss, st, sp, vn, order_bad);
            if (tid < kDim / 4 && sp_ok) {
                if (MODE == kFuseBf16) {
                    st_global_nt<uint2>((uint64_t)(a.f.w[c] + (size_t)row * kDim * 2) + 8 * tid,
                                        make_uint2(bf16_pack(bf16_lo(wb.x) - scale * sum.x,
                                                             bf16_hi(wb.x) - scale * sum.y),
                                                   bf16_pack(bf16_lo(wb.y) - scale * sum.z,
                                                             bf16_hi(wb.y) - scale * sum.w)));
                } else {
                    st_global_nt<float4>((uint64_t)(a.f.w[c] + (size_t)row * kDim * 4) + 16 * tid,
                                         make_float4(wf.x - scale * sum.x, wf.y - scale * sum.y,
                                                     wf.z - scale * sum.z, wf.w - scale * sum.w));
                }
            }
            if (tid == 0 && sp_ok) {
                a.f.st[c][row] = RowState{vn, sp.t};
                if (order_bad)
                    atomicOr(&a.hdr->flags, NGRAM_FLAG_STEP_ORDER);
            }
        }
        __syncthreads();
    }
    if constexpr (MODE != kAccum) {
        // Nested trigram runs that crossed the end of a walk, one per
        // wavefront of the grid: the piece in slot 1 of the run's first
        // chunk, then slot 0 of each following chunk whose first key
        // continues the run, added in order; then the row's step.
        if (a.nested) {
            constexpr int ELT = MODE == kFuseBf16 ? 2 : 4;
            const uint32_t ntr = a.hdr->n_trun;
            const int64_t n0 = count_of(a.n_dev[0], a.n_host);
            const uint64_t table_t = (uint64_t)a.f.w[1] + (uint64_t)ELT * 4 * lane;
            const uint64_t state_t = (uint64_t)a.f.st[1];
            const uint64_t P = (uint64_t)a.tpart + 16 * lane;
            for (uint32_t r = blk * kW + w; r < ntr; r += nblk * kW) {
                const uint64_t rec = a.trec[r];
                const int64_t x = (int64_t)(uint32_t)rec;
                const uint32_t tv = (uint32_t)(rec >> 32);
                const uint32_t row = tv & kTrowMask;
                WRow<ELT> wr;
                load_wrow<ELT>(wr, table_t + (uint64_t)row * (kDim * ELT));
                const RowState rst = ld_global_nt<RowState>(state_t + (uint64_t)row * sizeof(RowState));
                // m = the following chunks whose first key continues the run
                // (consecutive: the run's keys are contiguous), 64 probed at a time
                int64_t m = 0;
                for (;;) {
                    const int64_t cc = x + 1 + m + lane;
                    bool hit = false;
                    if (cc * kChunk < n0) {
                        const uint32_t t = a.tinfo[a.tix0[cc * kChunk]];
                        hit = is_run(t) && !(t & kRunHead) && ((t ^ tv) & kTrowMask) == 0;
                    }
                    const uint64_t miss = ~__ballot(hit);
                    const int lead = miss ? (int)__builtin_ctzll(miss) : kWave;
                    m += lead;
                    if (lead < kWave)
                        break;
                }
                float4 g[kQ];
#pragma unroll
                for (int q = 0; q < kQ; ++q)
                    g[q] = ld_global<float4>(P + ((uint64_t)x * 2 + 1) * (kDim * 4) + q * (kWave * 16));
                for (int64_t i = 1; i <= m; i += kRedU) {
                    float4 y[kRedU][kQ];
#pragma unroll
                    for (int u = 0; u < kRedU; ++u) {
                        if (i + u <= m) {
#pragma unroll
                            for (int q = 0; q < kQ; ++q)
                                y[u][q] = ld_global<float4>(P + (uint64_t)(x + i + u) * 2 * (kDim * 4) +
                                                            q * (kWave * 16));
                        }
                    }
#pragma unroll
                    for (int u = 0; u < kRedU; ++u) {
                        if (i + u <= m) {
#pragma unroll
                            for (int q = 0; q < kQ; ++q)
                                g[q] = add4(g[q], y[u][q]);
                        }
                    }
                }
                step_one<ELT>(g, wr, rst, row, table_t, state_t, a, sp, sp_ok, lane);
            }
        }
    }
}

}  // namespace

namespace {

// Whether a reduction of up to n_host keys per table takes the nested sort.
// Below 2^20 keys the second, serial sort (a few hundred tiles per pass at
// most) costs more than the trigram rows it completes save: one shard's
// window of 4 x 49,152 positions took 0.622 ms without it against 0.673 ms
// with it, while the full window (4 x 393,216) took 3.44 ms with it against
// 3.53 ms without, and the collision-stress window 2.75 against 3.10 ms.
constexpr uint32_t kNestMinKeys = 1u << 20;
bool nested_sort(const WsLayout &L, uint32_t n_host, bool fused)
{
    return fused && L.nested && (L.nest_always || n_host >= kNestMinKeys);
}

// The sorted arrays, the singleton split's outputs and the slot pointers of
// one reduce.  The radix sort ping-pongs between the two key/payload buffers,
// so after L.passes passes the sorted keys are in buffer passes % 2; the
// other buffer is free and holds the compacted trigram keys.
SlotArgs slot_args(const WsLayout &L, uint8_t *ws, const uint32_t *n_dev, uint32_t n_host, bool fused)
{
    const int cur = L.passes & 1;
    SlotArgs sa;
    sa.rows = reinterpret_cast<const uint32_t *>(ws + L.keys[cur]);
    sa.vals = reinterpret_cast<const uint32_t *>(ws + L.vals[cur]);
    sa.nk = L.nk;
    sa.n_dev = n_dev;
    sa.n_host = n_host;
    for (int c = 0; c < 2; ++c) {
        sa.slot_map[c] = reinterpret_cast<SlotEntry *>(ws + L.slot_map[c]);
        sa.slot_rows[c] = reinterpret_cast<uint32_t *>(ws + L.slot_rows[c]);
    }
    sa.seg_info = reinterpret_cast<uint32_t *>(ws + L.seg_info);
    sa.blk = reinterpret_cast<uint32_t *>(ws + L.blk);
    sa.nblk = (n_host + kSortTile - 1) / kSortTile;
    sa.wrows = (uint32_t)L.wrows;
    sa.hdr = reinterpret_cast<WsHeader *>(ws + L.hdr);
    uint32_t *spare_k = reinterpret_cast<uint32_t *>(ws + L.keys[cur ^ 1]);
    uint32_t *spare_v = reinterpret_cast<uint32_t *>(ws + L.vals[cur ^ 1]);
    sa.kept = reinterpret_cast<uint32_t *>(ws + L.kept);
    sa.fused = fused;
    sa.tinfo = reinterpret_cast<uint32_t *>(ws + L.tinfo);
    sa.split_rows = spare_k + L.nk;
    sa.split_vals = spare_v + L.nk;
    sa.split_info = spare_k;
    sa.nested = nested_sort(L, n_host, fused);
    sa.btro = reinterpret_cast<const uint32_t *>(ws + L.btro);
    sa.tkept = reinterpret_cast<uint8_t *>(ws + L.tkept);
    return sa;
}

// The scatter's block for the 4,096-key tiles of large sorts: 512 threads
// of 8 keys (the full window's sort group 6 us faster than 256 threads of 16).
constexpr int kScatterThreadsBig = 512, kScatterItemsBig = 8;
static_assert(kScatterThreadsBig * kScatterItemsBig == radix_tile(kRadixItemsBig), "one tile per scatter block");

// The radix passes over the channels [cbase, cbase + nch) (the first pass's
// digit counts already taken), from key buffer 0.  tix (one channel): each
// key's index before the first pass is carried along, ping-ponging between
// L.tix[0] and L.tix[1] (the last pass writes L.tix[passes & 1]).
void radix_passes(const WsLayout &L, uint8_t *ws, const uint32_t *n_dev, uint32_t n_host, bool big, uint32_t nrb,
                  int cbase, int nch, bool tix, hipStream_t s)
{
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + L.hist);
    uint32_t *tot = reinterpret_cast<uint32_t *>(ws + L.tot);
    int cur = 0;
    for (int p = 0; p < L.passes; ++p) {
        const int shift = p * kRadixBits;
        uint32_t *kin = reinterpret_cast<uint32_t *>(ws + L.keys[cur]);
        uint32_t *vin = reinterpret_cast<uint32_t *>(ws + L.vals[cur]);
        uint32_t *kout = reinterpret_cast<uint32_t *>(ws + L.keys[cur ^ 1]);
        uint32_t *vout = reinterpret_cast<uint32_t *>(ws + L.vals[cur ^ 1]);
        if (p > 0)
            (big ? radix_hist_kernel<kRadixItemsBig> : radix_hist_kernel<kRadixItemsSmall>)
                <<<dim3(nrb, nch), kSortThreads, 0, s>>>(kin, L.nk, n_dev, n_host, shift, hist, nrb, cbase);
        scan_digits_kernel<<<dim3(kRadix, nch), kSortThreads, 0, s>>>(hist, nrb, tot, cbase);
        const uint32_t *xin = p == 0 ? nullptr : reinterpret_cast<const uint32_t *>(ws + L.tix[p & 1]);
        uint32_t *xout = reinterpret_cast<uint32_t *>(ws + L.tix[(p + 1) & 1]);
        if (big && tix)
            radix_scatter_kernel<kScatterItemsBig, kScatterThreadsBig, true>
                <<<dim3(nrb, nch), kScatterThreadsBig, 0, s>>>(kin, vin, kout, vout, L.nk, n_dev, n_host, shift,
                                                               hist, tot, nrb, cbase, xin, xout);
        else if (big)
            radix_scatter_kernel<kScatterItemsBig, kScatterThreadsBig, false>
                <<<dim3(nrb, nch), kScatterThreadsBig, 0, s>>>(kin, vin, kout, vout, L.nk, n_dev, n_host, shift,
                                                               hist, tot, nrb, cbase, nullptr, nullptr);
        else if (tix)
            radix_scatter_kernel<kRadixItemsSmall, kSortThreads, true>
                <<<dim3(nrb, nch), kSortThreads, 0, s>>>(kin, vin, kout, vout, L.nk, n_dev, n_host, shift, hist,
                                                         tot, nrb, cbase, xin, xout);
        else
            radix_scatter_kernel<kRadixItemsSmall, kSortThreads, false>
                <<<dim3(nrb, nch), kSortThreads, 0, s>>>(kin, vin, kout, vout, L.nk, n_dev, n_host, shift, hist,
                                                         tot, nrb, cbase, nullptr, nullptr);
        cur ^= 1;
    }
}

// Keys, radix sort, segment heads, window slots (accumulating reduce only)
// and the singleton split.  Spread: the T keys of `tok`; burst (tok null):
// the stash, its count on the device, bounded by n_host.
void sort_part(const WsLayout &L, uint8_t *ws, const HashParams &hp, const int32_t *tok, uint32_t n_host, bool fused,
               hipStream_t s)
{
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + L.hdr);
    const bool burst = tok == nullptr;
    const uint32_t *n_dev = burst ? &hdr->n_stash : nullptr;
    const bool nested = nested_sort(L, n_host, fused);
    // (one channel per launch in the nested sort: 2,048-key tiles there were
    // slower on the full window, 0.296 against 0.286 ms for the sort group)
    const bool big = n_host >= kRadixBigKeys;
    const uint32_t tile = radix_tile(big ? kRadixItemsBig : kRadixItemsSmall);
    const uint32_t nrb = (n_host + tile - 1) / tile;   // radix tiles
    const uint32_t nblk = (n_host + kSortTile - 1) / kSortTile;     // slot / split tiles
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + L.hist);
    uint32_t *k0 = reinterpret_cast<uint32_t *>(ws + L.keys[0]);
    uint32_t *v0 = reinterpret_cast<uint32_t *>(ws + L.vals[0]);

    uint32_t *bidx = reinterpret_cast<uint32_t *>(ws + L.bidx);
    auto keys_k = nested ? (burst ? (big ? keys_tile_kernel<true, kRadixItemsBig, true>
                                         : keys_tile_kernel<true, kRadixItemsSmall, true>)
                                  : (big ? keys_tile_kernel<false, kRadixItemsBig, true>
                                         : keys_tile_kernel<false, kRadixItemsSmall, true>))
                         : (burst ? (big ? keys_tile_kernel<true, kRadixItemsBig, false>
                                         : keys_tile_kernel<true, kRadixItemsSmall, false>)
                                  : (big ? keys_tile_kernel<false, kRadixItemsBig, false>
                                         : keys_tile_kernel<false, kRadixItemsSmall, false>));
    launch_prof(NGRAM_PROF_SORT, true, false, keys_k, dim3(nrb), dim3(kSortThreads), 0, s, tok,
                burst ? reinterpret_cast<const uint32_t *>(ws + L.stash_idx) : nullptr,
                burst ? reinterpret_cast<const uint32_t *>(ws + L.stash_pos) : nullptr, hp, n_host, k0, v0, L.nk,
                hist, nrb, hdr, bidx);
    if (!nested) {
        radix_passes(L, ws, n_dev, n_host, big, nrb, 0, L.nch, false, s);
    } else {
        // the trigram keys alone, then the bigram keys in trigram order (the
        // same buffer 0 the trigram keys started from, their own half), then
        // the bigram keys by row: (bigram row, trigram row, position), each
        // carrying its index in the trigram order
        radix_passes(L, ws, n_dev, n_host, big, nrb, 1, 1, false, s);
        const uint32_t *vt = reinterpret_cast<const uint32_t *>(ws + L.vals[L.passes & 1]) + L.nk;
        (big ? gather_bigram_kernel<kRadixItemsBig> : gather_bigram_kernel<kRadixItemsSmall>)
            <<<nrb, kSortThreads, 0, s>>>(vt, bidx, n_dev, n_host, k0, v0, hist, nrb,
                                          reinterpret_cast<uint32_t *>(ws + L.btro));
        radix_passes(L, ws, n_dev, n_host, big, nrb, 0, 1, true, s);
    }
    const SlotArgs sa = slot_args(L, ws, n_dev, n_host, fused);
    // one table (token-indexed): no trigram channel, no singleton split
    launch_prof(NGRAM_PROF_SORT, false, L.nch == 1 && fused, mark_kernel, dim3(nblk, L.nch), dim3(kSortThreads),
                0, s, sa);
    if (!fused)   // fused: rows new to the window are stepped at once and need no slot
        launch_prof(NGRAM_PROF_SORT, false, L.nch == 1, assign_kernel, dim3(nblk, L.nch), dim3(kSortThreads), 0, s,
                    sa);
    if (L.nch == 2)
        launch_prof(NGRAM_PROF_SORT, false, true, split_kernel, dim3(nblk), dim3(kSortThreads), 0, s, sa);
    else
        sorted_count_kernel<<<1, 1, 0, s>>>(reinterpret_cast<WsHeader *>(ws + L.hdr), n_dev, n_host);
}

// The signed segment reduction of the sorted keys (accumulating, or fused
// with the step when f is set), then the fix-up of long segments.
hipError_t reduce_part(const WsLayout &L, uint8_t *ws, uint32_t n_host, bool burst, const void *dY,
                       const FuseArgs *f, hipStream_t s)
{
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + L.hdr);
    const uint32_t *n_dev = burst ? &hdr->n_stash : nullptr;
    const SlotArgs sa = slot_args(L, ws, n_dev, n_host, f != nullptr);
    RedArgs ra;
    for (int c = 0; c < 2; ++c) {
        ra.rows[c] = sa.rows + (size_t)c * L.nk;
        ra.vals[c] = sa.vals + (size_t)c * L.nk;
        ra.info[c] = sa.seg_info + (size_t)c * L.nk;
        ra.n_dev[c] = n_dev;
    }
    // the trigram pass walks the keys the singleton split kept
    ra.rows[1] = sa.split_rows;
    ra.vals[1] = sa.split_vals;
    ra.info[1] = sa.split_info;
    ra.n_dev[1] = &hdr->n_multi;
    ra.n_host = n_host;
    ra.tinfo = L.nch == 2 ? sa.tinfo : nullptr;
    ra.nested = sa.nested;
    ra.tix0 = sa.nested ? reinterpret_cast<const uint32_t *>(ws + L.tix[L.passes & 1]) : nullptr;
    ra.tpart = reinterpret_cast<float *>(ws + L.tpart);
    ra.trec = reinterpret_cast<uint64_t *>(ws + L.trec);
    ra.dY = burst && !L.by_ref ? ws + L.stash_dy : static_cast<const uint8_t *>(dY);
    ra.dy_ptrs = L.by_ref ? reinterpret_cast<const uint8_t *const *>(ws + L.dy_ptrs) : nullptr;
    ra.pos_bits = L.by_ref ? L.pos_bits : 31;
    ra.gacc = reinterpret_cast<float *>(ws + L.gacc);
    ra.slot_rows[0] = sa.slot_rows[0];
    ra.slot_rows[1] = sa.slot_rows[1];
    ra.wrows = L.wrows;
    ra.partial = reinterpret_cast<float *>(ws + L.partial);
    ra.owners = reinterpret_cast<uint64_t *>(ws + L.owners);
    ra.nchunk = L.nchunk;
    ra.gpart = reinterpret_cast<float *>(ws + L.gpart);
    ra.ngroup = L.ngroup;
    ra.hdr = hdr;
    ra.burst = burst;
    if (f)
        ra.f = *f;
    const uint32_t nchunk = (n_host + kChunk - 1) / kChunk;
    const uint32_t per_block = kRedThreads / kWave;
    const dim3 grid((nchunk + per_block - 1) / per_block, L.nch);
    const bool dy16 = L.dy_elt == 2;
    const dim3 ggrid((unsigned)((nchunk + kGroup - 1) / kGroup), L.nch);
    if (!f) {
        launch_prof(NGRAM_PROF_REDUCE, true, true, dy16 ? seg_reduce_kernel<2> : seg_reduce_kernel<4>, grid,
                    dim3(kRedThreads), 0, s, ra);
        group_sum_kernel<<<ggrid, kGroupThreads, 0, s>>>(ra);
        fixup_kernel<kAccum><<<dim3(512, L.nch), kFixThreads, 0, s>>>(ra);
    } else if (f->dtype == NGRAM_DTYPE_BF16) {
        launch_prof(NGRAM_PROF_REDUCE, true, true, dy16 ? seg_step_kernel<2, 2> : seg_step_kernel<2, 4>, grid,
                    dim3(kRedThreads), 0, s, ra);
        group_sum_kernel<<<ggrid, kGroupThreads, 0, s>>>(ra);
        fixup_kernel<kFuseBf16><<<dim3(512, L.nch), kFixThreads, 0, s>>>(ra);
    } else {
        launch_prof(NGRAM_PROF_REDUCE, true, true, dy16 ? seg_step_kernel<4, 2> : seg_step_kernel<4, 4>, grid,
                    dim3(kRedThreads), 0, s, ra);
        group_sum_kernel<<<ggrid, kGroupThreads, 0, s>>>(ra);
        fixup_kernel<kFuseF32><<<dim3(512, L.nch), kFixThreads, 0, s>>>(ra);
    }
    return hipGetLastError();
}

hipError_t reduce_impl(const WsLayout &L, uint8_t *ws, const HashParams &hp, const int32_t *tok, int64_t T,
                       const void *dY, const FuseArgs *f, hipStream_t s)
{
    // spread: T keys known on the host; burst: the stash count on the device,
    // bounded by the stash capacity (grids cover the bound, blocks past the
    // count exit)
    const uint32_t n_host = (uint32_t)T;
    if (n_host == 0)
        return hipSuccess;
    sort_part(L, ws, hp, tok, n_host, f != nullptr, s);
    return reduce_part(L, ws, n_host, tok == nullptr, dY, f, s);
}

}  // namespace

hipError_t launch_reduce(const WsLayout &L, uint8_t *ws, const HashParams &hp, const int32_t *tok, int64_t T,
                         const void *dY, hipStream_t s)
{
    return reduce_impl(L, ws, hp, tok, T, dY, nullptr, s);
}

hipError_t launch_reduce_step(const WsLayout &L, uint8_t *ws, const HashParams &hp, const int32_t *tok, int64_t T,
                              const void *dY, const FuseArgs &f, hipStream_t s)
{
    return reduce_impl(L, ws, hp, tok, T, dY, &f, s);
}

hipError_t launch_window_sort(const WsLayout &L, uint8_t *ws, const HashParams &hp, hipStream_t s)
{
    sort_part(L, ws, hp, nullptr, (uint32_t)L.nk, true, s);
    return hipGetLastError();
}

hipError_t launch_reduce_step_sorted(const WsLayout &L, uint8_t *ws, const FuseArgs &f, hipStream_t s)
{
    return reduce_part(L, ws, (uint32_t)L.nk, true, nullptr, &f, s);
}

}  // namespace ngram
