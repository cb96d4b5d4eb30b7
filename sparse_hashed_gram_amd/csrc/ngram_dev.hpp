// Device helpers, workspace layout and kernel launchers of libngram (gfx950).
//
// Everything here is HIP for CDNA4 only: 64-lane wavefronts, 16-byte row
// accesses, LDS tiles.  No host code of the C ABI lives here; ngram_abi.hip
// validates arguments and calls the launchers declared at the bottom.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ngram {

constexpr int kDim = 768;
constexpr int kWave = 64;

// ---------------------------------------------------------------- hashing
//
// Hashed bigram/trigram rows with a +/-1 sign (modded-nanogpt README,
// technique list).  The pages give no hash; this is the SplitMix64 finaliser
// (Steele, Lea & Flood 2014, Stafford's Mix13 multipliers) of (key ^ seed)
// advanced by the golden gamma, reduced to [0, R) by Lemire's multiply-shift
// of the upper 32 bits, with the sign in bit 0.

struct HashParams {
    uint32_t vocab;   // V; V itself encodes "no token"
    int32_t eos;
    uint32_t rows[2];
    uint64_t seed[2];
    uint32_t direct;  // one table indexed by the token id itself (no hashing, no sign)
};

__device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Packed index: row | (negative << 31).
__device__ __forceinline__ uint32_t hash_pack(uint64_t key, uint64_t seed, uint32_t R)
{
    const uint64_t z = mix64((key ^ seed) + 0x9E3779B97F4A7C15ull);
    const uint32_t hi = (uint32_t)(z >> 32);
    const uint32_t row = (uint32_t)(((uint64_t)hi * (uint64_t)R) >> 32);
    return row | ((uint32_t)z << 31);
}

// Context of position i (micro-step local) and both channels' packed
// indices.  The EoS opens its document: no n-gram reaches back across it, and
// the micro-step start has no context.  Returns true if t[i] is not a valid id.
__device__ __forceinline__ bool ngram_index(const int32_t *__restrict__ tok, int64_t i,
                                            const HashParams &hp, uint32_t &ib, uint32_t &it)
{
    const int32_t t0 = tok[i];
    if (hp.direct) {
        // a token-indexed table (value embeddings): row = the id; an id
        // outside the table takes row 0 (and is flagged: it is outside [0, V))
        ib = (uint32_t)t0 < hp.rows[0] ? (uint32_t)t0 : 0u;
        it = 0;
        return (uint32_t)t0 >= hp.vocab;
    }
    const int32_t t1 = i >= 1 ? tok[i - 1] : 0;
    const int32_t t2 = i >= 2 ? tok[i - 2] : 0;
    const uint64_t none = hp.vocab;
    const bool opens = (t0 == hp.eos);
    const uint64_t p1 = (i >= 1 && !opens) ? (uint64_t)(uint32_t)t1 : none;
    const uint64_t p2 = (i >= 2 && !opens && t1 != hp.eos) ? (uint64_t)(uint32_t)t2 : none;
    const uint64_t B = none + 1;
    const uint64_t tt = (uint64_t)(uint32_t)t0;
    const uint64_t kb = p1 * B + tt;
    const uint64_t kt = (p2 * B + p1) * B + tt;
    ib = hash_pack(kb, hp.seed[0], hp.rows[0]);
    it = hash_pack(kt, hp.seed[1], hp.rows[1]);
    return (uint32_t)t0 >= hp.vocab;
}

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest, ties to even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t bf16_pack(float lo, float hi)
{
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// The same rounding by gfx950's pair conversion (v_cvt_pk_bf16_f32); equal to
// bf16_pack except for NaN inputs, whose sign and payload it may keep.
__device__ __forceinline__ uint32_t bf16_pack_rne(float lo, float hi)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {lo, hi};
    const bf16x2 b = __builtin_convertvector(v, bf16x2);
    uint32_t u;
    __builtin_memcpy(&u, &b, 4);
    return u;
}

// ------------------------------------------------------- memory access
//
// Accesses through the global address space.  An address formed at run time
// (taken from another lane, or read from memory) would otherwise be used
// with flat instructions, and a wait for LDS results (lgkmcnt) then also has
// to drain every flat load in flight.

template <int BYTES>
struct RawWord;
template <>
struct RawWord<2> {
    typedef uint16_t type;
};
template <>
struct RawWord<4> {
    typedef uint32_t type;
};
template <>
struct RawWord<8> {
    typedef uint32_t type __attribute__((ext_vector_type(2)));
};
template <>
struct RawWord<16> {
    typedef uint32_t type __attribute__((ext_vector_type(4)));
};

template <typename T>
__device__ __forceinline__ T ld_global(uint64_t addr)
{
    typedef typename RawWord<sizeof(T)>::type W;
    const W w = *(const __attribute__((address_space(1))) W *)addr;
    T v;
    __builtin_memcpy(&v, &w, sizeof(T));
    return v;
}

template <typename T>
__device__ __forceinline__ void st_global(uint64_t addr, const T &v)
{
    typedef typename RawWord<sizeof(T)>::type W;
    W w;
    __builtin_memcpy(&w, &v, sizeof(T));
    *(__attribute__((address_space(1))) W *)addr = w;
}

// Non-temporal (streaming) forms: the access carries the nt hint, so the
// line is not kept in the caches for reuse.  For data a launch touches once:
// dY rows, window rows, table rows and row state in the reduction and the
// step, the forward's output rows.  On MI355X the hint raises random 3 KB row
// gathers from about 5.9 to 6.5 TB/s and plain streaming reads from 6.3 to
// 7.1 TB/s; the forward's table reads keep the default policy, because hot
// n-gram rows are served from the caches.
template <typename T>
__device__ __forceinline__ T ld_global_nt(uint64_t addr)
{
    typedef typename RawWord<sizeof(T)>::type W;
    const W w = __builtin_nontemporal_load((const __attribute__((address_space(1))) W *)addr);
    T v;
    __builtin_memcpy(&v, &w, sizeof(T));
    return v;
}

template <typename T>
__device__ __forceinline__ void st_global_nt(uint64_t addr, const T &v)
{
    typedef typename RawWord<sizeof(T)>::type W;
    W w;
    __builtin_memcpy(&w, &v, sizeof(T));
    __builtin_nontemporal_store(w, (__attribute__((address_space(1))) W *)addr);
}

__device__ __forceinline__ void atomic_add_global(uint64_t addr, float v)
{
    __hip_atomic_fetch_add((__attribute__((address_space(1))) float *)addr, v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Marks x as produced here.  Used on per-lane values loaded before a loop and
// read inside it through readlane: the wait for their loads then happens once,
// here, and not as a full drain of the loop's own loads at every use.
template <typename T>
__device__ __forceinline__ void settle(T &x)
{
    asm volatile("" : "+v"(x));
}

// ---------------------------------------------------------------- scans

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

// ------------------------------------------------------------ workspace
//
// One device allocation, carved by the host (WsLayout).  All mutable state
// of a window lives here so the hot calls never need a host round trip.

struct WsHeader {
    uint32_t magic;
    uint32_t flags;        // NGRAM_FLAG_* (sticky)
    uint32_t n_slots[2];   // distinct rows in the window, per channel
    uint32_t n_next[2];    // n_slots once the micro-step being reduced is in
    uint32_t n_owner[2];   // long-segment fix-up records of the current reduce
    uint32_t n_stash;      // burst mode: positions kept since the last reduce
    uint32_t epoch;        // window number; slot-map entries of other windows are stale
    uint32_t n_micro;      // burst modes: micro-steps whose gradients are attached
    uint32_t n_multi;      // fused reduction: trigram keys left after the singleton split
    uint32_t n_keyed;      // burst modes: micro-steps whose keys are kept (>= n_micro)
    uint32_t sorted_n;     // burst modes: n_stash when the keys were last sorted
    uint32_t dropped;      // the window was found unready: its step changes no row
    uint32_t n_trun;       // fused reduction: nested trigram runs left to the fix-up
    uint32_t pad[48];
};
static_assert(sizeof(WsHeader) == 256, "header is one 256-byte block");

constexpr uint32_t kMagic = 0x6E677231u;

// Window slots stay below this (the singleton map keeps two flag bits above a slot).
constexpr int64_t kMaxWindowRows = (int64_t(1) << 30) - 1;

// Row -> window slot map entry.  A row is in the current window iff its
// epoch equals the header's; ending a window just advances the epoch, so the
// sparse step never has to clear entries.
struct SlotEntry {
    uint32_t epoch;
    uint32_t slot;
};

// Burst modes: where a kept micro-step's positions start in the stash, and
// how many it has.
struct MicroStep {
    uint32_t base;
    uint32_t T;
};
constexpr int kMaxMicro = 64;   // accum_steps is at most this

// Per-row optimizer state, as the caller stores it (ngram_row_state).
struct RowState {
    float v;
    int32_t t_last;
};

// Sort tiles: 256 threads x 8 keys.
constexpr int kSortThreads = 256;
constexpr int kSortItems = 8;
constexpr int kSortTile = kSortThreads * kSortItems;
#ifndef NGRAM_RADIX_BITS
#define NGRAM_RADIX_BITS 9
#endif
constexpr int kRadixBits = NGRAM_RADIX_BITS;   // 26-bit rows of the full table: 3 passes
constexpr int kRadix = 1 << kRadixBits;
constexpr int kDpt = kRadix / kSortThreads;    // digits per thread in the per-digit loops
static_assert(kRadix % kSortThreads == 0, "digits are split evenly over the threads");
// Radix tiles (key build, digit counts, scatter): 256 threads x ITEMS keys.
// A larger tile gives the scatter longer runs of each digit to write, but
// fewer blocks: 16 keys per thread when a channel has at least 1M keys to
// sort (the full burst window's sort: 0.217 -> 0.191 ms), else 8 (a spread
// micro-step or a shard window would leave CUs idle).
constexpr int kRadixItemsBig = 16, kRadixItemsSmall = 8;
constexpr uint32_t kRadixBigKeys = 1u << 20;
__host__ __device__ constexpr int radix_tile(int items) { return kSortThreads * items; }

// Segment-reduce chunks: one wavefront per 64 sorted keys.
constexpr int kChunk = 64;
// Chunks per group in the fix-up of long segments.
constexpr int kGroup = 64;

struct WsLayout {
    uint64_t hdr;
    uint64_t slot_map[2];   // SlotEntry [rows[c]]: {window epoch, slot} of each row
    uint64_t slot_rows[2];  // uint32 [wrows]: row of each slot
    uint64_t gacc;          // fp32 [2][wrows][768]: window gradient
    uint64_t keys[2];       // uint32 [2][nk]: sort key buffers A/B (row)
    uint64_t vals[2];       // uint32 [2][nk]: sort payload A/B (position | neg << 31)
    uint64_t seg_info;      // uint32 [2][nk]: slot | new << 31 at segment heads
    uint64_t hist;          // uint32 [2][kRadix][nrblk]: per-tile digit counts, then offsets
    uint64_t tot;           // uint32 [2][256]: digit totals of a pass
    uint64_t blk;           // uint32 [2][nblk]
    uint64_t kept;          // uint32 [nblk]: trigram keys kept per sort tile by the singleton split
    uint64_t partial;       // fp32 [2][nchunk][2][768]
    uint64_t owners;        // uint64 [2][nchunk]
    uint64_t gpart;         // fp32 [2][ngroup][768]: sums of 64-chunk groups inside one segment
    uint64_t tinfo;         // uint32 [code_cap]: per dY row code (nested sort: per index in
                            // the trigram order), its trigram row's record when the bigram
                            // pass completes that row (see the singleton split and the nested
                            // trigram rows), else kNotSingle
    uint64_t tix[2];        // uint32 [nk] each (nested sort): the bigram keys' indices in the
                            // trigram order, carried through the bigram passes
    uint64_t bidx;          // uint32 [code_cap]: per dY row code, its packed bigram index
                            // (nested sort: the bigram keys are gathered in trigram order)
    uint64_t btro;          // uint32 [nk] (nested sort): the bigram row of each key in the
                            // trigram order, as gathered for the bigram sort
    uint64_t tpart;         // fp32 [nchunk][2][768] (nested sort): pieces of nested trigram
                            // runs that cross the end of a chunk's walk (slot 0: the piece
                            // at the walk's start, slot 1: the piece at its end)
    uint64_t trec;          // uint64 [nchunk] (nested sort): chunk | record << 32 of each run
                            // whose first piece is in slot 1 of that chunk
    uint64_t tkept;         // uint8 [nk]: per trigram-sorted key, kept for the trigram pass
    uint64_t stash_idx;     // uint32 [2][nk] (burst): packed indices of kept positions
    uint64_t stash_pos;     // uint32 [nk] (burst): dY row code of each kept position
    uint64_t stash_dy;      // dY dtype [nk][768] (burst, copying): the kept dY rows
    uint64_t dy_ptrs;       // const void * [64] (burst by reference): dY of each micro-step
    uint64_t mstep;         // MicroStep [64] (burst modes)
    uint64_t tbits[2];      // uint32 [ceil(rows[c] / 32)]: touched-row bits (ngram_touched_rows)
    uint64_t tblk;          // uint32 [ceil(words / 8192)]: set bits per block of words
    uint64_t total;

    int64_t rows[2];
    int64_t wrows;          // window capacity per channel
    int64_t nk;             // keys per channel one reduce can hold
    int64_t nblk;           // sort tiles for nk keys
    int64_t nrblk;          // radix tiles for nk keys
    int64_t nchunk;         // 64-key chunks for nk keys
    int64_t ngroup;         // groups of 64 chunks
    int passes;             // radix passes (kRadixBits each)
    bool burst;             // micro-steps are kept and reduced at step time
    bool by_ref;            // ... and their dY is read where the caller keeps it
    int pos_bits;           // by_ref: dY row code = micro-step << pos_bits | position
    int dy_elt;             // bytes per dY element: 4 (fp32) or 2 (bf16)
    int64_t code_cap;       // dY row codes are below this
    int accum;              // micro-steps per window
    int nch;                // tables: 2 (bigram, trigram), or 1 (token-indexed)
    bool nested;            // fused reductions of at least 2^20 keys sort the bigram keys
                            // by (bigram row, trigram row) and complete nested trigram
                            // rows in the bigram pass (two tables, rows[1] <= 2^28)
    bool nest_always;       // ... and so do smaller ones (NGRAM_OPT_NEST_ALWAYS)
    bool one_shot;          // a whole burst window reduced and stepped in one call on an
                            // empty window: no slot maps, slot rows or window
                            // accumulator (their offsets name no memory and are
                            // never dereferenced on that path)
};

// -------------------------------------------------------------- row step
//
// The lazy row-wise step (Adam with beta1 = 0, one second moment per row,
// beta2 applied for every optimizer step the row missed): given the row's
// window gradient G (its sum of squares sum_g2) and its state, returns the
// factor lr / (sqrt(v') + eps) that multiplies G, and v' itself.

struct StepParams {
    int32_t t;
    float lr;
    float beta2;
    float eps;
};

// beta2^k by square-and-multiply in fp64 (relative error below k * 2^-52).
__device__ __forceinline__ double pow_steps(double b, int32_t k)
{
    double r = 1.0;
    while (k > 0) {
        if (k & 1)
            r *= b;
        b *= b;
        k >>= 1;
    }
    return r;
}

// Sum over the 64 lanes, the same bits in every lane: butterflies inside each
// row of 16 lanes through DPP (xor 1, xor 2, half-row mirror, row mirror),
// then the four row sums read as scalars and added in a fixed order.  No LDS
// traffic, so it does not wait on outstanding memory operations.
__device__ __forceinline__ float wave_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));   // row_half_mirror
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));   // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (r0 + r1) + (r2 + r3);
}

// order_bad: t does not exceed t_last (the row then decays by beta2^0).
__device__ __forceinline__ float step_scale(float sum_g2, RowState s, const StepParams &p, float &vn,
                                            bool &order_bad)
{
    int32_t k = p.t - s.t_last;
    order_bad = k < 1;
    if (k < 1)
        k = 0;
    const double decay = pow_steps((double)p.beta2, k);
    vn = (float)(decay * (double)s.v + (1.0 - (double)p.beta2) * ((double)sum_g2 * (1.0 / kDim)));
    return p.lr / (sqrtf(vn) + p.eps);
}

// The step parameters a kernel uses: the call's own, or (p_dev set) those in
// device memory, read when the kernel runs, so that a replayed HIP graph picks
// up new values.  ok is false if device-read values are out of range (t < 1,
// beta2 outside [0, 1), eps not positive and finite, lr not finite); the
// kernels then write no table row and no row state.
__device__ __forceinline__ StepParams step_params(const StepParams &p, const StepParams *p_dev, bool &ok)
{
    if (!p_dev) {
        ok = true;
        return p;
    }
    const StepParams q = *p_dev;
    ok = q.t >= 1 && __builtin_isfinite(q.lr) && q.beta2 >= 0.f && q.beta2 < 1.f && q.eps > 0.f &&
         __builtin_isfinite(q.eps);
    return q;
}

// Tables and state the fused reduce + step writes.
struct FuseArgs {
    uint8_t *w[2];
    RowState *st[2];
    StepParams p;
    const StepParams *p_dev;   // if set, the parameters are read from here
    int dtype;
};

// Slot rows whose step already ran inside the fused reduction carry this bit.
constexpr uint32_t kSlotStepped = 0x80000000u;

// ------------------------------------------------------------- profiling
// Optional event pairs per kernel group (ngram_profile_events); thread-local.
// The group's first kernel carries the start event and its last kernel the
// stop event through hipExtLaunchKernelGGL, which takes them from that
// dispatch's own start and end timestamps: no marker packet enters the
// stream, so measuring adds no idle time between kernels.

struct ProfSlot {
    hipEvent_t start;
    hipEvent_t stop;
};
constexpr int kProfGroups = 5;
extern thread_local ProfSlot g_prof[kProfGroups];

// Launches kernel<<<grid, block, shmem, s>>>(args...); `first` / `last` mark
// it as the first / last kernel of `group` for the events above.
template <typename... KArgs, typename... Args>
inline void launch_prof(int group, bool first, bool last, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                        uint32_t shmem, hipStream_t s, Args... args)
{
    hipEvent_t a = first ? g_prof[group].start : nullptr;
    hipEvent_t b = last ? g_prof[group].stop : nullptr;
    if (a || b)
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, a, b, 0u, static_cast<KArgs>(args)...);
    else
        kernel<<<grid, block, shmem, s>>>(static_cast<KArgs>(args)...);
}

// ---------------------------------------------------------------- launchers
// Implemented in the .hip files of this directory; all enqueue on `s`.

hipError_t launch_init(const WsLayout &L, uint8_t *ws, hipStream_t s);
hipError_t launch_hash(const HashParams &hp, const int32_t *tok, int64_t T, uint32_t *idx,
                       uint32_t *flags, hipStream_t s);
hipError_t launch_fwd(int dtype, bool out_f32, const HashParams &hp, const void *wb, const void *wt,
                      const int32_t *tok, int64_t T, void *out, uint32_t *flags, hipStream_t s);

// Burst: keep one micro-step (packed indices + dY rows) in the stash.
hipError_t launch_stash(const WsLayout &L, uint8_t *ws, const HashParams &hp,
                        const int32_t *tok, const void *dY, int64_t T, hipStream_t s);
// Burst: keep one micro-step's keys only (its gradients come later).
hipError_t launch_keys(const WsLayout &L, uint8_t *ws, const HashParams &hp, const int32_t *tok, int64_t T,
                       hipStream_t s);
// Burst: sort the kept keys for the fused reduction (keys, radix sort, heads,
// singleton split); sets sorted_n.
hipError_t launch_window_sort(const WsLayout &L, uint8_t *ws, const HashParams &hp, hipStream_t s);
// Burst: the fused reduction + step of a window sorted by launch_window_sort.
hipError_t launch_reduce_step_sorted(const WsLayout &L, uint8_t *ws, const FuseArgs &f, hipStream_t s);

// Build the sort keys of both channels (spread: hashed from `tok`, T of them;
// burst: from every kept stash position, a device count bounded by nk), sort
// them by row, find segments, assign window slots and reduce the signed dY
// rows into the window.
hipError_t launch_reduce(const WsLayout &L, uint8_t *ws, const HashParams &hp, const int32_t *tok,
                         int64_t T, const void *dY, hipStream_t s);
// The same reduction fused with the sparse step: each row's gradient of the
// window is completed (with what the window already holds for it) and the
// row is stepped at once; rows only the window holds are left for
// launch_step, which skips the stepped ones.
hipError_t launch_reduce_step(const WsLayout &L, uint8_t *ws, const HashParams &hp, const int32_t *tok,
                              int64_t T, const void *dY, const FuseArgs &f, hipStream_t s);

// Burst: mark the stash empty after a reduce.
hipError_t launch_stash_clear(const WsLayout &L, uint8_t *ws, hipStream_t s);

hipError_t launch_step(const WsLayout &L, uint8_t *ws, const FuseArgs &f, hipStream_t s);

hipError_t launch_flags_clear(uint8_t *ws, const WsLayout &L, hipStream_t s);
// ORs the workspace's sticky flags into the device word `out`.
hipError_t launch_flags_export(const WsLayout &L, const uint8_t *ws, uint32_t *out, hipStream_t s);

hipError_t launch_export(const WsLayout &L, const uint8_t *ws, int channel, uint32_t *rows,
                         float *G, uint32_t max_rows, uint32_t *count, hipStream_t s);

// The window's distinct rows of channel c in ascending order (ngram_touched_rows).
hipError_t launch_touched(const WsLayout &L, uint8_t *ws, int c, int32_t *rows, uint64_t max_rows, int64_t *count,
                          hipStream_t s);
// Writes a count of 0 (a channel with no table).
hipError_t launch_touched_none(int64_t *count, hipStream_t s);

}  // namespace ngram
