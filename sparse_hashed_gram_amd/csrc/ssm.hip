// Sampled-softmax training loss on gfx950 (the method and readings are in
// include/ssm.h): the candidate set, then three bf16 contractions on the
// matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation) with the softmax
// work fused into their epilogues:
//
//   forward   z = X W_S^T per 128 x 128 tile -> per-tile (max, sum exp) of
//             each position, the target's logit, and z itself (fp32, kept
//             in the workspace); a per-position pass folds the tiles into
//             lse and the loss.
//   backward  a streaming pass over the stored z -> dz = g (exp(z - lse) -
//             onehot), bf16, row-major; dX = dz W_S; dW[S] += dz^T X.
//
// Every contraction is C[m][n] = sum_k A[m][k] B[n][k]; B is k-contiguous in
// memory (the backward's transposed X and W_S are written first), A too
// except in dW, where A = dz^T is read k-major straight from dz through the
// LDS transpose read.  One kernel template serves all three: four wavefronts
// per block, each owning WM x WN matrix-core tiles of 32 x 32, and a
// pipelined main loop with direct global -> LDS loads.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ssm.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 768;
constexpr int kLdt = 64 + 4;    // fp32 per column of the forward's epilogue tile (16-byte rows, conflict-free)
constexpr int kLdb = 128 + 16;  // bf16 per row of the dz epilogue's row-major tile (paired 4-byte writes conflict-free)
constexpr int kTile = 128;      // T and C are padded to multiples of this
// Per contraction: the k-step BK, the number NS of pipelined stages (two
// blocks per CU), and the block tile, four wavefronts of WM x WN matrix-core
// tiles of 32 x 32.  Chosen by measurement on MI355X (49,152 positions x
// 10,240 candidates x 768).
constexpr int kFwdWN = 3, kFwdBK = 64, kFwdS = 2;            // forward, 128 x 64 WN
constexpr int kDxWM = 2, kDxWN = 3, kDxBK = 64, kDxS = 2;    // dX, 128 x 192
constexpr int kDwBK = 64, kDwS = 2;                          // dW, 128 x 192 or 128 x 128 by round fill
constexpr int kMaxSplit = 4;                                 // dW: most parts of k

constexpr uint32_t kMagic = 0x53534d31u;
constexpr uint64_t kAlign = 256;

struct Hdr {
    uint32_t magic;
    uint32_t flags;        // sticky SSM_FLAG_*
    uint32_t void_batch;   // nonzero: the last candidate set is void
    uint32_t n_present;    // distinct targets of the last candidate set
    int32_t z_T;           // T of the logits the last forward stored; -1: none for this candidate set
    uint32_t pad[59];
};
static_assert(sizeof(Hdr) == 256, "header is 256 bytes");

struct Layout {
    int64_t Tp, Cp;   // padded maxima
    uint64_t hdr, rank, cnt, blk, absent, zt, part, xt, wst, dz, zb, dwp, total;
};

inline int64_t rup(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

Layout layout(const ssm_config *c)
{
    Layout L{};
    L.Tp = rup(c->max_tokens, kTile);
    L.Cp = rup(c->candidates, kTile);
    uint64_t o = 0;
    auto take = [&](uint64_t bytes) {
        uint64_t at = o;
        o += (bytes + kAlign - 1) / kAlign * kAlign;
        return at;
    };
    L.hdr = take(sizeof(Hdr));
    L.rank = take(4ull * c->vocab);
    L.cnt = take(4ull * c->vocab);
    {
        const uint64_t nbs = (c->vocab + 1023) / 1024;   // blocks of the candidate ranking
        L.blk = take(4ull * 2 * nbs);
        L.absent = take(4ull * 32 * nbs);
    }
    L.zt = take(4ull * L.Tp);
    L.part = take(8ull * L.Tp * (L.Cp / kTile));
    L.xt = take(2ull * kD * L.Tp);
    L.wst = take(2ull * kD * L.Cp);
    L.dz = take(2ull * L.Tp * L.Cp);
    L.zb = take(2ull * L.Tp * L.Cp);
    L.dwp = take(4ull * kMaxSplit * L.Cp * kD);
    L.total = o;
    return L;
}

// ------------------------------------------------------------ candidate set

__global__ void init_kernel(Hdr *h)
{
    if (threadIdx.x == 0) {
        h->magic = kMagic;
        h->flags = 0;
        h->void_batch = 0;
        h->n_present = 0;
        h->z_T = -1;
    }
}

__global__ void flags_clear_kernel(Hdr *h)
{
    if (threadIdx.x == 0)
        h->flags = 0;
}

__global__ void cand_clear_kernel(int32_t *rank, int32_t *cnt, int32_t V, Hdr *h)
{
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v < V) {
        rank[v] = 0;
        cnt[v] = 0;
    }
    if (v == 0) {
        h->void_batch = 0;
        h->z_T = -1;   // a new candidate set: no stored logits belong to it yet
    }
}

// rank[] holds the presence mark (1) until the select kernel ranks it.
__global__ void cand_mark_kernel(const int32_t *tgt, int64_t T, const int32_t *perm, int32_t V,
                                 int32_t *rank, int32_t *cnt, Hdr *h)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < T) {
        const int32_t y = tgt[i];
        if ((uint32_t)y < (uint32_t)V) {
            rank[y] = 1;
        } else {
            atomicOr(&h->flags, SSM_FLAG_BAD_TARGET);
            atomicOr(&h->void_batch, 1u);
        }
    }
    if (i < V) {
        const int32_t p = perm[i];
        if ((uint32_t)p < (uint32_t)V) {
            atomicAdd(&cnt[p], 1);
        } else {
            atomicOr(&h->flags, SSM_FLAG_BAD_PERM);
            atomicOr(&h->void_batch, 1u);
        }
    }
}

// The candidate order, over blocks of 1,024 ids (and of 1,024 places of the
// permutation): present ids ascending into cand[0, n), then absent ids in
// permutation order into cand[n, C).  Both are ranks of 0/1 flags:
// cand_count_kernel counts each block's flags (and keeps the absent flags
// of its permutation places as bits), cand_rank_kernel adds the counts of
// the blocks before its own and ranks its flags by wavefront ballots.
constexpr int kSelBlock = 1024;
constexpr int kSelWaves = kSelBlock / 64;

__device__ inline int32_t rank_in_wave(uint64_t m)
{
    const int lane = threadIdx.x & 63;
    return __popcll(m & ((1ull << lane) - 1ull));
}

// rank[] still holds the presence marks (0 / 1) here.  Also prefills cand
// (in range whatever follows) and flags a permutation in which some id does
// not occur exactly once.
__global__ __launch_bounds__(kSelBlock) void cand_count_kernel(const int32_t *perm, int32_t V, int32_t C,
                                                                const int32_t *rank, const int32_t *cnt,
                                                                int32_t *cand, int32_t *blk, uint32_t *absent,
                                                                int32_t nbs, Hdr *h)
{
    __shared__ int32_t s_c[2][kSelWaves];
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int32_t b = blockIdx.x;
    for (int64_t c = (int64_t)b * kSelBlock + t; c < C; c += (int64_t)gridDim.x * kSelBlock)
        cand[c] = 0;
    const int32_t v = b * kSelBlock + t;
    const bool pres = v < V && rank[v] != 0;
    if (v < V && cnt[v] != 1) {
        atomicOr(&h->flags, SSM_FLAG_BAD_PERM);
        atomicOr(&h->void_batch, 1u);
    }
    const int32_t p = v < V ? perm[v] : -1;
    const bool ab = (uint32_t)p < (uint32_t)V && rank[p] == 0;
    const uint64_t mp = __ballot(pres), ma = __ballot(ab);
    if (lane == 0) {
        s_c[0][w] = __popcll(mp);
        s_c[1][w] = __popcll(ma);
        absent[(int64_t)b * 2 * kSelWaves + 2 * w] = (uint32_t)ma;
        absent[(int64_t)b * 2 * kSelWaves + 2 * w + 1] = (uint32_t)(ma >> 32);
    }
    __syncthreads();
    if (t < 2) {
        int32_t sum = 0;
        for (int k = 0; k < kSelWaves; ++k)
            sum += s_c[t][k];
        blk[(int64_t)t * nbs + b] = sum;
    }
}

__global__ __launch_bounds__(kSelBlock) void cand_rank_kernel(const int32_t *perm, int32_t V, int32_t C,
                                                               int32_t *rank, int32_t *cand, const int32_t *blk,
                                                               const uint32_t *absent, int32_t nbs, Hdr *h)
{
    __shared__ int32_t s_red[4][kSelWaves];
    __shared__ int32_t s_w[2][kSelWaves];
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int32_t b = blockIdx.x;
    // counts of the blocks before this one, and of all blocks
    int32_t pre0 = 0, pre1 = 0, tot0 = 0, tot1 = 0;
    for (int32_t k = t; k < nbs; k += kSelBlock) {
        const int32_t c0 = blk[k], c1 = blk[(int64_t)nbs + k];
        tot0 += c0;
        tot1 += c1;
        pre0 += k < b ? c0 : 0;
        pre1 += k < b ? c1 : 0;
    }
    int32_t r4[4] = {pre0, pre1, tot0, tot1};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1)
            r4[q] += __shfl_xor(r4[q], d, 64);
        if (lane == 0)
            s_red[q][w] = r4[q];
    }
    const int32_t v = b * kSelBlock + t;
    const bool pres = v < V && rank[v] != 0;
    const uint64_t mp = __ballot(pres);
    const uint64_t ma = (uint64_t)absent[(int64_t)b * 2 * kSelWaves + 2 * w] |
                        ((uint64_t)absent[(int64_t)b * 2 * kSelWaves + 2 * w + 1] << 32);
    const bool ab = (ma >> lane) & 1ull;
    if (lane == 0) {
        s_w[0][w] = __popcll(mp);
        s_w[1][w] = __popcll(ma);
    }
    __syncthreads();
    int32_t base[4] = {0, 0, 0, 0}, woff0 = 0, woff1 = 0;
#pragma unroll
    for (int k = 0; k < kSelWaves; ++k) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            base[q] += s_red[q][k];
        woff0 += k < w ? s_w[0][k] : 0;
        woff1 += k < w ? s_w[1][k] : 0;
    }
    const int32_t n = base[2];   // present ids in all
    if (v < V) {
        const int32_t r = base[0] + woff0 + rank_in_wave(mp);
        rank[v] = pres ? r : -1;
        if (pres && r < C)
            cand[r] = v;
        const int32_t pos = base[1] + woff1 + rank_in_wave(ma);
        if (ab && n + pos < C)
            cand[n + pos] = perm[v];
    }
    if (b == 0 && t == 0) {
        h->n_present = (uint32_t)n;
        if (n > C) {
            atomicOr(&h->flags, SSM_FLAG_OVERFLOW);
            atomicOr(&h->void_batch, 1u);
        }
    }
}

__global__ void cand_slot_kernel(const int32_t *tgt, int64_t T, int32_t V, int32_t C,
                                 const int32_t *rank, int32_t *slot)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T)
        return;
    const int32_t y = tgt[i];
    int32_t s = 0;
    if ((uint32_t)y < (uint32_t)V) {
        const int32_t r = rank[y];
        s = (r >= 0 && r < C) ? r : 0;
    }
    slot[i] = s;
}

// --------------------------------------------------------- the contraction

// Row i of an operand: base + row * ld, with row = idx[i] for a gathered
// operand.  Rows at or past n read row n - 1 (their results are masked).
struct Rows {
    const uint16_t *base;
    int64_t ld;            // elements between rows
    const int32_t *idx;    // gather ids, or nullptr
    int32_t n;             // rows that exist (>= 1)
    int32_t V;             // gather ids must be below V
};

__device__ inline const uint16_t *row_ptr(const Rows &r, int64_t i, uint32_t *flags)
{
    int64_t j = i < r.n ? i : r.n - 1;
    if (r.idx) {
        int32_t v = r.idx[j];
        if ((uint32_t)v >= (uint32_t)r.V) {
            atomicOr(flags, SSM_FLAG_BAD_CAND);
            v = 0;
        }
        j = v;
    }
    return r.base + j * r.ld;
}

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Direct global -> LDS load (global_load_lds_dwordx4): lane l of a wavefront
// lands its 16 bytes at LDS base + 16 l (probed on the GPU), so one load
// fills a contiguous 1 KB block; the LDS base must be wavefront-uniform.
__device__ inline void lds_load16(const uint16_t *g, uint8_t *lds)
{
    __builtin_amdgcn_global_load_lds((const void *)g, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// Position of acc[mb][nb][e] in the block tile (32 x 32 matrix-core layout:
// lane l holds column l % 32 and rows 8 (e / 4) + 4 (l / 32) + e % 4).
template <int WM>
__device__ inline int tile_row(int mb, int e)
{
    const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) >> 1;
    return wm * WM * 32 + mb * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
template <int WN>
__device__ inline int tile_col(int nb)
{
    const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
    return wn * WN * 32 + nb * 32 + (lane & 31);
}

__device__ inline uint16_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Block -> output tile.  The hardware hands consecutive workgroups to the 8
// XCDs in turn; each XCD is given a contiguous range of tiles instead, walked
// in groups of 8 M-tiles (all N-tiles of a group before the next group), so
// the blocks resident on one XCD share their A and B tiles in its L2 and the
// last-level cache sees each operand tile while its users still run.
constexpr uint32_t kXcds = 8, kGroupM = 8;

__host__ __device__ inline uint32_t grid_blocks(uint32_t nM, uint32_t nN)
{
    return kXcds * ((nM * nN + kXcds - 1) / kXcds);
}

__device__ inline bool tile_of(uint32_t nM, uint32_t nN, uint32_t &mt, uint32_t &nt)
{
    const uint32_t total = nM * nN, per = (total + kXcds - 1) / kXcds;
    const uint32_t tile = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (tile >= total)
        return false;
    const uint32_t span = kGroupM * nN, g = tile / span, first = g * kGroupM;
    const uint32_t gm = nM - first < kGroupM ? nM - first : kGroupM;
    const uint32_t r = tile - g * span;
    mt = first + r % gm;
    nt = r / gm;
    return true;
}

// Pipelined form of the main loop: block tile (64 WM) x (64 WN), four
// wavefronts of (32 WM) x (32 WN) (WM, WN > 2 let each operand fragment read
// from LDS feed more matrix-core ops).  Direct global -> LDS loads into S
// stages of BK; all S start filling at once, S - 1 stay in flight while one is
// read, and one barrier per k-step both publishes the stage that landed and
// frees the one read last.
// Rows are stored unpadded, BK / 8 chunks of 16 bytes each, chunk c of row r
// at position c ^ ((r >> SH) & (CH - 1)), so the lanes of one ds_read_b128
// (consecutive rows, one chunk) spread over the banks (the PMC bank-conflict
// counter reads 0); each lane fetches the source chunk that belongs at its
// position.  The next sub-step's fragments are read while the current one's
// products run.
template <int WM, int WN, int BK, int S>
struct WideTile {
    static constexpr int BM = 64 * WM, BN = 64 * WN;
    static constexpr int CH = BK / 8, RB = CH * 16, RPI = 1024 / RB;
    static constexpr int SH = CH == 8 ? 1 : (CH == 4 ? 2 : 3);
    static constexpr int LA = BM / (4 * RPI), LB = BN / (4 * RPI);   // loads per thread per stage
    static constexpr uint32_t STAGE = (uint32_t)(BM + BN) * RB;
    static constexpr uint32_t SMEM = S * STAGE;
    static_assert(BM % (4 * RPI) == 0 && BN % (4 * RPI) == 0, "whole loads per wavefront");
    static_assert(S >= 2 && (S - 2) * (LA + LB) < 64, "outstanding loads fit the counter");
};

// s_waitcnt that waits for this wavefront's vector-memory count to drop to N
// and leaves the other counters alone (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Block barrier with no memory fence.  A fence would make the compiler wait
// for every outstanding LDS-bound load (they count as vector-memory ops), which
// defeats the stages; the caller waits for exactly the loads it needs, this
// waits for the wavefront's LDS reads, and the empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ inline void barrier_nofence()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt left alone
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// TA: A is stored k-major (A[m][k] at A.base[k A.ld + m], rows of A.base are
// k); the stage then holds BK rows of BM m-values (row r's 16-byte chunk c at
// position c ^ 4 (r & 3)) and the fragments come from gfx950's LDS transpose
// read, ds_read_b64_tr_b16: within each 16 lanes, lane i receives element
// i % 4 of the 8-byte chunks addressed by lanes 4 j + i / 4, j = 0..3 (probed
// on the GPU), so with lane p addressing row k0 + p / 4, column c0 + 4 (p % 4)
// lane i gets rows k0 .. k0 + 3 of column c0 + i.
template <int WM, int WN, int BK, int S, bool TA = false>
__device__ inline void mainloop_wide(const Rows &A, const Rows &B, int64_t K, int64_t m0, int64_t n0,
                                     uint8_t *sm, f32x16 (&acc)[WM][WN], uint32_t *flags)
{
    using WT = WideTile<WM, WN, BK, S>;
    constexpr int CH = WT::CH, RB = WT::RB, RPI = WT::RPI, SH = WT::SH, LA = WT::LA, LB = WT::LB;
    constexpr int RBA = TA ? 2 * WT::BM : RB;       // bytes per LDS row of A
    constexpr int RPIA = 1024 / RBA;                 // A rows one wavefront load covers
    static_assert(!TA || WM == 2, "k-major A: 128 m-values per row (16 chunks)");
    static_assert(!TA || BK / (4 * RPIA) == LA, "same loads per stage either way");
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int lrow = lane / CH, lpos = lane % CH;
    // load j of wavefront w fills rows (4 j + w) RPI .. + RPI of its operand
    const uint16_t *pa[LA], *pb[LB];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        if constexpr (TA) {
            const int r = (4 * j + w) * RPIA + lane / 16, pos = lane % 16;   // k row, chunk position
            pa[j] = A.base + r * A.ld + m0 + 8 * (pos ^ (4 * (r & 3)));
        } else {
            const int r = (4 * j + w) * RPI + lrow;
            pa[j] = row_ptr(A, m0 + r, flags) + 8 * (lpos ^ ((r >> SH) & (CH - 1)));
        }
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        const int r = (4 * j + w) * RPI + lrow;
        pb[j] = row_ptr(B, n0 + r, flags) + 8 * (lpos ^ ((r >> SH) & (CH - 1)));
    }
    const int64_t ka = TA ? A.ld : 1;   // elements per step of k in A
    auto issue = [&](int stage, int64_t k0) {
        uint8_t *ab = sm + stage * WT::STAGE, *bb = ab + WT::BM * RB;
#pragma unroll
        for (int j = 0; j < LA; ++j)
            lds_load16(pa[j] + k0 * ka, ab + (4 * j + w) * RPIA * RBA);
#pragma unroll
        for (int j = 0; j < LB; ++j)
            lds_load16(pb[j] + k0, bb + (4 * j + w) * RPI * RB);
    };
#pragma unroll
    for (int mb = 0; mb < WM; ++mb)
#pragma unroll
        for (int nb = 0; nb < WN; ++nb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[mb][nb][e] = 0.f;
    const int64_t nk = K / BK;
    constexpr int KK = BK / 16, L = LA + LB;
    static_assert(KK % 2 == 0, "fragment buffers alternate within a stage");
    // every buffer starts filling at once; buffer kt % S is refilled with
    // stage kt + S as soon as all wavefronts have read stage kt
#pragma unroll
    for (int st = 0; st < S; ++st)
        if (st < nk)
            issue(st, st * BK);
    // rows of one fragment start at a multiple of 32, so every fragment of a
    // lane has the same swizzle
    const int ar = wm * WM * 32 + (lane & 31), br = wn * WN * 32 + (lane & 31), kq = lane >> 5;
    const int sa = (ar >> SH) & (CH - 1), sb = (br >> SH) & (CH - 1);
    // k-major A: lane p = lane % 16 of group G = lane / 16 addresses row
    // 16 kk + 8 (G / 2) + 4 h + p / 4 and column wm 64 + 32 mb + 16 (G % 2) +
    // 4 (p % 4); the column's chunk has bit 2 = mb, so the swizzle is an XOR
    const int tp = lane & 15, tg = lane >> 4;
    const int ta_row = (8 * (tg >> 1) + (tp >> 2)) * RBA + 8 * (tp & 1);
    const int ta_chunk = (8 * wm + 2 * (tg & 1) + ((tp >> 1) & 1)) ^ (4 * (tp >> 2));
    bf16x8 fa[2][WM], fb[2][WN];
    // reads in the order the products use them: A fragment 0, the B
    // fragments, then the other A fragments
    auto rd = [&](int stage, int kk, bf16x8 (&a)[WM], bf16x8 (&b)[WN]) {
        const uint8_t *ab = sm + stage * WT::STAGE, *bb = ab + WT::BM * RB;
        const int c = 2 * kk + kq;
        auto rda = [&](int mb) {
            if constexpr (TA) {
                const uint8_t *q = ab + ta_row + 16 * kk * RBA + 16 * (ta_chunk ^ (4 * mb));
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)q);
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(q + 4 * RBA));
                a[mb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            } else {
                a[mb] = *(const bf16x8 *)(ab + (ar + 32 * mb) * RB + 16 * (c ^ sa));
            }
        };
        rda(0);
#pragma unroll
        for (int nb = 0; nb < WN; ++nb)
            b[nb] = *(const bf16x8 *)(bb + (br + 32 * nb) * RB + 16 * (c ^ sb));
#pragma unroll
        for (int mb = 1; mb < WM; ++mb)
            rda(mb);
    };
    auto mm = [&](int mb0, int mb1, const bf16x8 (&a)[WM], const bf16x8 (&b)[WN]) {
#pragma unroll
        for (int mb = mb0; mb < mb1; ++mb)
#pragma unroll
            for (int nb = 0; nb < WN; ++nb)
                acc[mb][nb] = mfma(a[mb], b[nb], acc[mb][nb]);
    };
    // one phase: the reads of the next fragments interleaved with the
    // products of the current ones (read, product, read, ... then the rest of
    // the products), fenced off from the phases around it
    auto phase = [&](bool more, int stage, int kk, const bf16x8 (&a)[WM], const bf16x8 (&b)[WN],
                     bf16x8 (&na)[WM], bf16x8 (&nb)[WN]) {
        __builtin_amdgcn_sched_barrier(0);
        if (more)
            rd(stage, kk, na, nb);
        mm(0, WM, a, b);
        if (more) {
            constexpr int NR = (TA ? 2 : 1) * WM + WN, NM = WM * WN, NP = NR < NM ? NR : NM;
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix-core op
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
            }
            if constexpr (NM > NP)
                __builtin_amdgcn_sched_group_barrier(0x008, NM - NP, 0);
            if constexpr (NR > NP)
                __builtin_amdgcn_sched_group_barrier(0x100, NR - NP, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    if (nk >= S)
        wait_vmcnt<(S - 1) * L>();
    else
        wait_vmcnt<0>();
    barrier_nofence();
    rd(0, 0, fa[0], fb[0]);
    int cur = 0;
    constexpr int last = (KK - 1) & 1;
    // all but the last sub-step of a k-step; fragments of its sub-step 0 are
    // in fa[0], fb[0]
    auto inner = [&]() {
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk)
            phase(true, cur, kk + 1, fa[kk & 1], fb[kk & 1], fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
    };
    for (int64_t kt = 0; kt + 1 < nk; ++kt) {
        inner();
        if (kt + S - 1 < nk)
            wait_vmcnt<(S - 2) * L>();   // stage kt + 1 has landed; later ones may still fly
        else
            wait_vmcnt<0>();
        barrier_nofence();               // ... for every wavefront, which are all done with stage kt
        if (kt + S < nk)
            issue(cur, (kt + S) * BK);
        cur = cur + 1 == S ? 0 : cur + 1;
        phase(true, cur, 0, fa[last], fb[last], fa[0], fb[0]);
    }
    inner();
    phase(false, cur, 0, fa[last], fb[last], fa[0], fb[0]);
    __syncthreads();   // LDS free for whatever follows
}

enum { EPI_FWD = 0, EPI_DZ = 1, EPI_DX = 2, EPI_DW = 3 };

struct GemmArgs {
    Rows A, B;
    int64_t K;
    int64_t T;             // positions
    int32_t C;             // candidates
    int32_t V;
    const int32_t *slot;   // [T]
    const int32_t *cand;   // [C]
    const float *lse;      // [T]
    const float *g;        // [T]
    float *zt;             // forward: target logits [T]
    float2 *part;          // forward: per-tile (max, sum exp) [column tiles][T]
    uint16_t *zb;          // forward -> dz: fp16 exp(z - M) per logit, fragment-major (below)
    uint16_t *dz;          // [Tq][Cp] bf16
    int64_t Tq, Cp;
    uint32_t tiles_m, tiles_n;   // output tiles
    float *out;            // dX [T][768] or dW [V][768]
    int32_t ksplit;        // dW: parts of k, each a block of its own (1: add into dW directly)
    float *dwp;            // dW parts [ksplit][Cp][768] when ksplit > 1
    Hdr *h;
};

constexpr uint32_t cmax(uint32_t x, uint32_t y) { return x > y ? x : y; }

// What the forward keeps of each logit z for the dz kernel: q = exp(z - M)
// in fp16 (round to nearest), M the largest logit of its row among the
// candidates of its forward column tile (the tile's per-row maximum, kept in
// part).  q lies in (0, 1], where fp16 holds it to 2^-11 relative (2^-25
// absolute below 2^-14); dz then needs only exp(M - lse) per row and tile.
// Buffer, fragment-major: the 32 x 32 matrix-core tile of rows 32 R .. and
// columns 32 Cb .. is 2 KB at 16-byte unit (R Cp/32 + Cb) 128, holding the
// accumulators as a wavefront has them: entries 8 h .. 8 h + 7 of lane l in
// unit h 64 + l.  So any block tiling can store or reload its fragments, each
// access a contiguous 1 KB per wavefront.
__device__ inline u32x4 *q_frag(const GemmArgs &a, int64_t row0, int64_t col0)
{
    return reinterpret_cast<u32x4 *>(a.zb) + ((row0 >> 5) * (a.Cp >> 5) + (col0 >> 5)) * 128 + (threadIdx.x & 63);
}
__device__ inline uint32_t pack_f16(float lo, float hi)
{
    const _Float16 l = (_Float16)lo, h = (_Float16)hi;   // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}
__device__ inline float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ inline float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// q of the block tile's accumulators; s_M: each row's M, indexed by the row
// in the tile.
template <int WM, int WN>
__device__ inline void store_q(const GemmArgs &a, int64_t m0, int64_t n0, const f32x16 (&acc)[WM][WN],
                               const float *s_M)
{
    const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
        float mr[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 m4 = *(const float4 *)(s_M + tile_row<WM>(mb, 4 * g));   // 4 consecutive rows
            mr[4 * g] = m4.x;
            mr[4 * g + 1] = m4.y;
            mr[4 * g + 2] = m4.z;
            mr[4 * g + 3] = m4.w;
        }
#pragma unroll
        for (int nb = 0; nb < WN; ++nb) {
            const int64_t col0 = n0 + wn * WN * 32 + nb * 32;
            if (col0 >= a.Cp)
                continue;   // past the padded candidates (wavefront-uniform)
            uint32_t v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = pack_f16(__expf(acc[mb][nb][2 * e] - mr[2 * e]), __expf(acc[mb][nb][2 * e + 1] - mr[2 * e + 1]));
            u32x4 *zb = q_frag(a, m0 + wm * WM * 32 + mb * 32, col0);
            __builtin_nontemporal_store(u32x4{v[0], v[1], v[2], v[3]}, zb);
            __builtin_nontemporal_store(u32x4{v[4], v[5], v[6], v[7]}, zb + 64);
        }
    }
}

// dz from what the forward stored, one 128 x 128 tile per block:
// dz = g (q exp(M - lse) - onehot) rounded to bf16 (q exp(M - lse) is
// exp(z - lse)), written row-major [Tq][Cp].  The tile's columns lie in at
// most two column tiles of the forward (kFwdCols wide; a 32-column fragment
// in one), whose M per row comes from part.  Values that the last forward
// did not store for this candidate set and T give zeros and
// SSM_FLAG_NO_LOGITS.
constexpr int kFwdCols = 64 * kFwdWN;
static_assert(kFwdCols % 32 == 0 && kFwdCols >= 128, "a fragment in one forward tile, a dz tile in two");
__global__ __launch_bounds__(256) void dz_kernel(GemmArgs a)
{
    __shared__ __align__(16) uint8_t smem[128 * kLdb * 2 + 5 * 128 * 4];
    uint32_t mt, nt;
    // N-tiles fastest: consecutive blocks write neighbouring 256-byte pieces
    // of the same dz rows (measured faster than M-tiles fastest or grouped)
    if (blockIdx.x >= a.tiles_m * a.tiles_n)
        return;
    mt = blockIdx.x / a.tiles_n;
    nt = blockIdx.x % a.tiles_n;
    const int64_t m0 = (int64_t)mt * 128, n0 = (int64_t)nt * 128;
    const int t = threadIdx.x;
    f32x16 acc[2][2];
    {
        const int w = t >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const u32x4 *zb = q_frag(a, m0 + wm * 64 + mb * 32, n0 + wn * 64 + nb * 32);
                const u32x4 lo = __builtin_nontemporal_load(zb), hi = __builtin_nontemporal_load(zb + 64);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[mb][nb][2 * e] = f16_lo(lo[e]);
                    acc[mb][nb][2 * e + 1] = f16_hi(lo[e]);
                    acc[mb][nb][8 + 2 * e] = f16_lo(hi[e]);
                    acc[mb][nb][8 + 2 * e + 1] = f16_hi(hi[e]);
                }
            }
    }
    const bool have = a.h->z_T == (int32_t)a.T;
    if (!have && blockIdx.x == 0 && t == 0)
        atomicOr(&a.h->flags, SSM_FLAG_NO_LOGITS);
    uint16_t *bt = reinterpret_cast<uint16_t *>(smem);   // [128][kLdb] bf16
    float *s_f = reinterpret_cast<float *>(smem + 128 * kLdb * 2);   // [2][128]: exp(M - lse)
    float *s_g = s_f + 2 * 128;
    int32_t *s_y = reinterpret_cast<int32_t *>(s_g + 128);
    const int64_t ft0 = n0 / kFwdCols;   // the first forward column tile of this tile
    {
        // thread t: row t % 128 of forward tile ft0 + t / 128 (the second
        // only where the tile reaches into it)
        const int r = t & 127, k = t >> 7;
        const int64_t i = m0 + r;
        const bool ok = have && i < a.T && a.h->void_batch == 0;
        const bool in = k == 0 || (ft0 + 1) * kFwdCols < n0 + 128;
        float f = 0.f;
        if (ok && in)
            f = __expf(a.part[(ft0 + k) * a.T + i].x - a.lse[i]);
        s_f[k * 128 + r] = f;
        if (k == 0) {
            s_g[r] = ok ? a.g[i] : 0.f;
            s_y[r] = ok ? a.slot[i] : -1;
        }
    }
    __syncthreads();
    // dz of the tile as bf16, packed in registers (a lane holds 4
    // consecutive rows of one column per group of 4 accumulator entries),
    // then written through LDS so it leaves as whole 256-byte rows
    uint32_t hp[2][2][4][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int r4 = tile_row<2>(mb, 4 * g);   // 4 consecutive rows, 16-byte aligned
            const float4 g4 = *(const float4 *)(s_g + r4);
            const int4 y4 = *(const int4 *)(s_y + r4);
            const float gr[4] = {g4.x, g4.y, g4.z, g4.w};
            const int yr[4] = {y4.x, y4.y, y4.z, y4.w};
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int cc = tile_col<2>(nb);
                const int c = (int)n0 + cc;        // candidates < 2^31
                const bool col_ok = c < a.C;
                // the fragment's forward tile (wavefront-uniform)
                const int k = (int)((n0 + (cc & ~31)) / kFwdCols - ft0);
                const float4 f4 = *(const float4 *)(s_f + k * 128 + r4);
                const float fr[4] = {f4.x, f4.y, f4.z, f4.w};
                uint16_t h[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // padding rows and columns, and a void batch, give 0
                    // (masked, not branched around: no divergence)
                    const float p = acc[mb][nb][4 * g + j] * fr[j];
                    const float dv = gr[j] * (p - (yr[j] == c ? 1.f : 0.f));
                    const uint32_t keep = col_ok && gr[j] != 0.f ? 0xffffffffu : 0u;
                    const float d = __uint_as_float(__float_as_uint(dv) & keep);
                    h[j] = bf16_rne(d);
                }
                hp[mb][nb][g][0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
                hp[mb][nb][g][1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
            }
        }
    // row-major tile: lanes l and l ^ 1 hold adjacent columns, so they swap
    // halves and each writes two rows of a column pair (4-byte writes):
    // even lanes rows r4, r4 + 1 of columns cc, cc + 1, odd lanes rows
    // r4 + 2, r4 + 3 of columns cc - 1, cc
    const int odd = t & 1;
    uint16_t *bp = bt + odd * (2 * kLdb - 1);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint32_t x = hp[mb][nb][g][0], y = hp[mb][nb][g][1];   // rows r4, r4 + 1 | r4 + 2, r4 + 3
                const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? x : y), 0xB1, 0xF, 0xF, false);
                const uint32_t lo = odd ? o : x, hi = odd ? y : o;   // left and right column
                uint16_t *q = bp + tile_row<2>(mb, 4 * g) * kLdb + tile_col<2>(nb);
                *(uint32_t *)q = (lo & 0xffffu) | (hi << 16);
                *(uint32_t *)(q + kLdb) = (lo >> 16) | (hi & 0xffff0000u);
            }
    __syncthreads();
    // row-major: 16 chunks of 16 B per row
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int rr = (t >> 4) + 16 * p, q = t & 15;
        const u32x4 v = *(const u32x4 *)(bt + rr * kLdb + q * 8);
        __builtin_nontemporal_store(v, (u32x4 *)(a.dz + (m0 + rr) * a.Cp + n0 + q * 8));
    }
}


template <int EPI, int WM, int WN, int BK, int NS>
constexpr uint32_t smem_bytes()
{
    constexpr uint32_t main = WideTile<WM, WN, BK, NS>::SMEM;
    return EPI == EPI_FWD ? cmax(main, 64 * WN * kLdt * 4 + 4 * 64 * 8 + 64 * WM * 4) : main;
}

// One contraction C[m][n] = sum_k A[m][k] B[n][k] per block tile (the
// pipelined loop, NS stages), then the epilogue EPI.  The forward's softmax
// epilogue takes 128 x 128 tiles.
template <int EPI, int WM, int WN, int BK, int NS>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a)
{
    static_assert(EPI == EPI_FWD || EPI == EPI_DX || EPI == EPI_DW, "contraction epilogues");
    static_assert(EPI != EPI_FWD || WM == 2, "the forward's epilogue takes 128-row tiles");
    static_assert(NS >= 2, "pipelined loop");
    constexpr int BM = 64 * WM, BN = 64 * WN;
    __shared__ __align__(16) uint8_t smem[smem_bytes<EPI, WM, WN, BK, NS>()];
    uint32_t mt, nt;
    // dW with k split: part p of k is M-tile row p of a taller grid, so the
    // blocks of one group share their k range (and the rows of X^T they read)
    const uint32_t parts = EPI == EPI_DW ? (uint32_t)a.ksplit : 1u;
    if (!tile_of(a.tiles_m * parts, a.tiles_n, mt, nt))
        return;   // the whole block: no barrier is reached
    Rows A = a.A, B = a.B;
    int64_t K = a.K;
    uint32_t part = 0;
    if constexpr (EPI == EPI_DW) {
        part = mt / a.tiles_m;
        mt -= part * a.tiles_m;
        const int64_t nk = a.K / BK, k0 = (int64_t)part * nk / parts * BK, k1 = (int64_t)(part + 1) * nk / parts * BK;
        A.base += k0 * A.ld;   // k-major: rows of A are k
        B.base += k0;
        K = k1 - k0;
    }
    const int64_t m0 = (int64_t)mt * BM, n0 = (int64_t)nt * BN;
    f32x16 acc[WM][WN];
    mainloop_wide<WM, WN, BK, NS, EPI == EPI_DW>(A, B, K, m0, n0, smem, acc, &a.h->flags);
    const int t = threadIdx.x;

    if constexpr (EPI == EPI_FWD) {
        // two halves of 64 rows.  The half's two wavefronts store their
        // accumulators to LDS column-major (a lane's 4 consecutive rows of
        // one column are one 16-byte store); wavefront q then folds columns
        // q CW .. (q + 1) CW of every row of the half, a row per lane (reads
        // of consecutive rows), and the four quarters meet in LDS
        constexpr int CW = BN / 4;
        float *tile = reinterpret_cast<float *>(smem);                      // [BN][kLdt]
        float2 *pq = reinterpret_cast<float2 *>(smem + BN * kLdt * 4);      // [4][64]
        float *s_M = reinterpret_cast<float *>(pq + 4 * 64);                // [BM]: each row's M
        const int w = t >> 6, r = t & 63, q = w, wm = w >> 1;
        const int64_t c0 = n0 + CW * q;
        const int64_t left = (int64_t)a.C - c0;
        const int nv = __builtin_amdgcn_readfirstlane(left <= 0 ? 0 : (left >= CW ? CW : (int)left));
        const float *zc = tile + CW * q * kLdt + r;   // column q CW + k at zc[k kLdt]
        for (int h = 0; h < 2; ++h) {
            if (wm == h) {
#pragma unroll
                for (int mb = 0; mb < WM; ++mb)
#pragma unroll
                    for (int nb = 0; nb < WN; ++nb)
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            *(float4 *)(tile + tile_col<WN>(nb) * kLdt + tile_row<WM>(mb, 4 * g) - 64 * h) =
                                make_float4(acc[mb][nb][4 * g], acc[mb][nb][4 * g + 1], acc[mb][nb][4 * g + 2],
                                            acc[mb][nb][4 * g + 3]);
            }
            __syncthreads();
            const int64_t i = m0 + 64 * h + r;
            float m = -INFINITY, s = 0.f;
            if (nv == CW) {
                float v[CW];
#pragma unroll
                for (int k = 0; k < CW; ++k)
                    v[k] = zc[k * kLdt];
#pragma unroll
                for (int k = 0; k < CW; ++k)
                    m = fmaxf(m, v[k]);
#pragma unroll
                for (int k = 0; k < CW; ++k)
                    s += __expf(v[k] - m);
            } else if (nv > 0) {
                for (int k = 0; k < nv; ++k)
                    m = fmaxf(m, zc[k * kLdt]);
                for (int k = 0; k < nv; ++k)
                    s += __expf(zc[k * kLdt] - m);
            }
            if (i < a.T) {
                const int64_t y = a.slot[i];
                if (y >= c0 && y < c0 + nv)
                    a.zt[i] = zc[(y - c0) * kLdt];
            }
            pq[q * 64 + r] = make_float2(m, s);
            __syncthreads();
            if (q == 0) {
                float M = -INFINITY;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    M = fmaxf(M, pq[k * 64 + r].x);
                s_M[64 * h + r] = M;
                if (i < a.T) {
                    float S = 0.f;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float2 o = pq[k * 64 + r];
                        if (o.y > 0.f)
                            S += o.y * __expf(o.x - M);
                    }
                    a.part[(int64_t)nt * a.T + i] = make_float2(M, S);
                }
            }
            __syncthreads();
        }
        // q = exp(z - M) for the dz kernel, fragment by fragment (each store:
        // 64 lanes x 16 bytes, contiguous; non-temporal: 2 T C bytes would
        // otherwise push the operands out of the caches)
        store_q<WM, WN>(a, m0, n0, acc, s_M);
    } else if constexpr (EPI == EPI_DX) {
#pragma unroll
        for (int mb = 0; mb < WM; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t i = m0 + tile_row<WM>(mb, e);
                if (i < a.T) {
#pragma unroll
                    for (int nb = 0; nb < WN; ++nb)
                        a.out[i * kD + n0 + tile_col<WN>(nb)] = acc[mb][nb][e];
                }
            }
    } else if (parts > 1) {   // EPI_DW, one part of k: plain stores, summed by dw_reduce_kernel
        float *dwp = a.dwp + (int64_t)part * a.Cp * kD;
#pragma unroll
        for (int mb = 0; mb < WM; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t c = m0 + tile_row<WM>(mb, e);
#pragma unroll
                for (int nb = 0; nb < WN; ++nb)
                    dwp[c * kD + n0 + tile_col<WN>(nb)] = acc[mb][nb][e];
            }
    } else {   // EPI_DW
#pragma unroll
        for (int mb = 0; mb < WM; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t c = m0 + tile_row<WM>(mb, e);
                if (c < a.C) {
                    const int32_t v = a.cand[c];
                    if ((uint32_t)v < (uint32_t)a.V) {
#pragma unroll
                        for (int nb = 0; nb < WN; ++nb) {
                            float *o = a.out + (int64_t)v * kD + n0 + tile_col<WN>(nb);
                            *o += acc[mb][nb][e];
                        }
                    }
                }
            }
    }
}

// dW[cand[c]] += the parts of k in order (part 0 first): deterministic.
__global__ void dw_reduce_kernel(const float *dwp, int parts, int64_t Cp, const int32_t *cand, int32_t C,
                                 int32_t V, float *dW)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // float4 of [C][768]
    if (i >= (int64_t)C * (kD / 4))
        return;
    const int64_t c = i / (kD / 4), q = i % (kD / 4);
    const int32_t v = cand[c];
    if ((uint32_t)v >= (uint32_t)V)
        return;
    const float4 *p = reinterpret_cast<const float4 *>(dwp) + c * (kD / 4) + q;
    float4 s = p[0];
    for (int k = 1; k < parts; ++k) {
        const float4 x = p[k * Cp * (kD / 4)];
        s.x += x.x;
        s.y += x.y;
        s.z += x.z;
        s.w += x.w;
    }
    float4 *o = reinterpret_cast<float4 *>(dW + (int64_t)v * kD) + q;
    float4 d = *o;
    d.x += s.x;
    d.y += s.y;
    d.z += s.z;
    d.w += s.w;
    *o = d;
}

// Folds the per-tile sums of each position: lse = M + log sum_t s_t e^(m_t - M).
// (Tile 0 has a finite maximum, its first column being a candidate; a later
// tile wholly past C is (-inf, 0) and adds exp(-inf) * 0 = 0.)
// Four adjacent lanes per position: lane q folds column tiles q, q + 4, ...
// (one pass, rescaling the running sum whenever the running maximum grows),
// then the four partial (max, sum) pairs meet by shuffles in a fixed order.
constexpr int kLseLanes = 4;
__global__ void lse_kernel(const float2 *part, int64_t T, int nct, const int32_t *slot, int32_t C,
                           const float *zt, float *loss, float *lse, Hdr *h)
{
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t i = g / kLseLanes;
    const int q = (int)(g % kLseLanes);
    float M = -INFINITY, S = 0.f;
    if (i < T) {
        for (int c = q; c < nct; c += kLseLanes) {
            const float2 p = part[(int64_t)c * T + i];
            if (p.y == 0.f)
                continue;   // a column tile wholly past C: (-inf, 0)
            if (p.x > M) {
                S = S * expf(M - p.x) + p.y;
                M = p.x;
            } else {
                S += p.y * expf(p.x - M);
            }
        }
    }
#pragma unroll
    for (int d = 1; d < kLseLanes; d <<= 1) {
        const float Mo = __shfl_xor(M, d, 64), So = __shfl_xor(S, d, 64);
        // the lower lane's pair first, so both lanes compute the same bits
        const bool low = (q & d) == 0;
        const float Ma = low ? M : Mo, Sa = low ? S : So, Mb = low ? Mo : M, Sb = low ? So : S;
        const float Mn = fmaxf(Ma, Mb);
        S = (Sa != 0.f ? Sa * expf(Ma - Mn) : 0.f) + (Sb != 0.f ? Sb * expf(Mb - Mn) : 0.f);
        M = Mn;
    }
    if (i >= T || q != 0)
        return;
    const float l = M + logf(S);
    const int32_t y = slot[i];
    const bool ok = (uint32_t)y < (uint32_t)C;
    if (!ok)
        atomicOr(&h->flags, SSM_FLAG_BAD_SLOT);
    const bool bad = h->void_batch != 0;
    lse[i] = bad ? NAN : l;
    loss[i] = (bad || !ok) ? NAN : l - zt[i];
    if (i == 0)
        h->z_T = (int32_t)T;   // the forward's logits (stored before this kernel) are T's
}

// dst[d][j] = element d of source row j for j < n, 0 for n <= j < (grid.x * 64);
// dst is [768][ldd] bf16.
__global__ __launch_bounds__(256) void transpose_kernel(Rows src, int64_t n, uint16_t *dst, int64_t ldd,
                                                        uint32_t *flags)
{
    __shared__ __align__(16) uint16_t s[64][72];
    const int t = threadIdx.x;
    const int64_t j0 = (int64_t)blockIdx.x * 64;
    const int d0 = blockIdx.y * 64;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = (t >> 3) + 32 * p, q = t & 7;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (j0 + r < n)
            v = *(const u32x4 *)(row_ptr(src, j0 + r, flags) + d0 + q * 8);
        *(u32x4 *)&s[r][q * 8] = v;
    }
    __syncthreads();
    const int d = t >> 2, rb = (t & 3) * 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            wv[e] = (uint32_t)s[rb + 8 * h + 2 * e][d] | ((uint32_t)s[rb + 8 * h + 2 * e + 1][d] << 16);
        *(u32x4 *)(dst + (int64_t)(d0 + d) * ldd + j0 + rb + 8 * h) = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
}

// ------------------------------------------------------------------ launch

struct ProfPair {
    hipEvent_t start, stop;
};
thread_local ProfPair g_prof[SSM_PROF_GROUPS];

template <typename... KArgs, typename... Args>
void launch(int group, bool first, bool last, void (*kernel)(KArgs...), dim3 grid, dim3 block,
            hipStream_t s, Args... args)
{
    hipEvent_t a = first ? g_prof[group].start : nullptr;
    hipEvent_t b = last ? g_prof[group].stop : nullptr;
    if (a || b)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, a, b, 0u, static_cast<KArgs>(args)...);
    else
        kernel<<<grid, block, 0, s>>>(static_cast<KArgs>(args)...);
}

int check_cfg(const ssm_config *c)
{
    if (!c)
        return SSM_ENULL;
    if (c->dim != kD || c->vocab < 1 || c->candidates < 1 || c->candidates > c->vocab ||
        c->reserved != 0 || c->max_tokens < 1 || c->max_tokens > (1 << 24))
        return SSM_ECONFIG;
    return SSM_OK;
}

bool aligned(const void *p, uint64_t a) { return ((uintptr_t)p % a) == 0; }

constexpr uint32_t kCUs = 256;   // MI355X compute units

// Share of the resident slots busy over all rounds of a launch of nb blocks.
double round_fill(uint32_t nb, uint32_t slots)
{
    const uint32_t rounds = (nb + slots - 1) / slots;
    return rounds ? (double)nb / ((double)rounds * slots) : 1.0;
}

int done(hipError_t e) { return e == hipSuccess ? SSM_OK : SSM_EHIP; }

uint32_t blocks(int64_t n, int b) { return (uint32_t)((n + b - 1) / b); }

}   // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char *ssm_status_string(int status)
{
    switch (status) {
    case SSM_OK: return "ok";
    case SSM_ENULL: return "a required pointer is NULL";
    case SSM_EALIGN: return "a pointer is misaligned";
    case SSM_ECONFIG: return "invalid config";
    case SSM_ESIZE: return "size out of range";
    case SSM_EARG: return "argument out of range";
    case SSM_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int ssm_workspace_bytes(const ssm_config *cfg, uint64_t *bytes)
{
    const int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (!bytes)
        return SSM_ENULL;
    *bytes = layout(cfg).total;
    return SSM_OK;
}

int ssm_workspace_init(const ssm_config *cfg, void *ws, uint64_t ws_bytes, void *stream)
{
    const int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (!ws)
        return SSM_ENULL;
    if (!aligned(ws, kAlign))
        return SSM_EALIGN;
    const Layout L = layout(cfg);
    if (ws_bytes < L.total)
        return SSM_ESIZE;
    hipStream_t s = (hipStream_t)stream;
    init_kernel<<<1, 64, 0, s>>>(reinterpret_cast<Hdr *>((uint8_t *)ws + L.hdr));
    return done(hipGetLastError());
}

int ssm_candidates(const ssm_config *cfg, void *ws, const int32_t *targets, int64_t T,
                   const int32_t *perm, int32_t *cand, int32_t *slot, void *stream)
{
    const int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (!ws || !targets || !perm || !cand || !slot)
        return SSM_ENULL;
    if (!aligned(ws, kAlign))
        return SSM_EALIGN;
    if (T < 0 || T > cfg->max_tokens)
        return SSM_ESIZE;
    if (T == 0)
        return SSM_OK;
    const Layout L = layout(cfg);
    uint8_t *w = (uint8_t *)ws;
    Hdr *h = reinterpret_cast<Hdr *>(w + L.hdr);
    int32_t *rank = reinterpret_cast<int32_t *>(w + L.rank);
    int32_t *cnt = reinterpret_cast<int32_t *>(w + L.cnt);
    const int32_t V = cfg->vocab, C = cfg->candidates;
    hipStream_t s = (hipStream_t)stream;
    launch(SSM_PROF_CAND, true, false, cand_clear_kernel, dim3(blocks(V, 256)), dim3(256), s, rank, cnt, V, h);
    launch(SSM_PROF_CAND, false, false, cand_mark_kernel, dim3(blocks(T > V ? T : V, 256)), dim3(256), s,
           targets, T, perm, V, rank, cnt, h);
    const int32_t nbs = (int32_t)blocks(V, kSelBlock);
    int32_t *blk = reinterpret_cast<int32_t *>(w + L.blk);
    uint32_t *absent = reinterpret_cast<uint32_t *>(w + L.absent);
    launch(SSM_PROF_CAND, false, false, cand_count_kernel, dim3(nbs), dim3(kSelBlock), s, perm, V, C,
           (const int32_t *)rank, (const int32_t *)cnt, cand, blk, absent, nbs, h);
    launch(SSM_PROF_CAND, false, false, cand_rank_kernel, dim3(nbs), dim3(kSelBlock), s, perm, V, C, rank, cand,
           (const int32_t *)blk, (const uint32_t *)absent, nbs, h);
    launch(SSM_PROF_CAND, false, true, cand_slot_kernel, dim3(blocks(T, 256)), dim3(256), s, targets, T, V,
           C, (const int32_t *)rank, slot);
    return done(hipGetLastError());
}

static int check_loss_args(const ssm_config *cfg, void *ws, const void *X, const void *W,
                           const int32_t *cand, const int32_t *slot, int64_t T)
{
    const int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (!ws || !X || !W || !cand || !slot)
        return SSM_ENULL;
    if (!aligned(ws, kAlign) || !aligned(X, 16) || !aligned(W, 16))
        return SSM_EALIGN;
    if (T < 0 || T > cfg->max_tokens)
        return SSM_ESIZE;
    return SSM_OK;
}

int ssm_loss_fwd(const ssm_config *cfg, void *ws, const void *X, const void *W, const int32_t *cand,
                 const int32_t *slot, int64_t T, float *loss, float *lse, void *stream)
{
    int rc = check_loss_args(cfg, ws, X, W, cand, slot, T);
    if (rc)
        return rc;
    if (!loss || !lse)
        return SSM_ENULL;
    if (T == 0)
        return SSM_OK;
    const Layout L = layout(cfg);
    uint8_t *w = (uint8_t *)ws;
    Hdr *h = reinterpret_cast<Hdr *>(w + L.hdr);
    const int32_t V = cfg->vocab, C = cfg->candidates;
    const int64_t Tq = rup(T, kTile);
    const int nct = (int)blocks(L.Cp, 64 * kFwdWN);   // column tiles of the forward
    GemmArgs a{};
    a.A = Rows{(const uint16_t *)X, kD, nullptr, (int32_t)T, V};
    a.B = Rows{(const uint16_t *)W, kD, cand, C, V};
    a.K = kD;
    a.T = T;
    a.C = C;
    a.V = V;
    a.slot = slot;
    a.cand = cand;
    a.zt = reinterpret_cast<float *>(w + L.zt);
    a.part = reinterpret_cast<float2 *>(w + L.part);
    a.zb = reinterpret_cast<uint16_t *>(w + L.zb);
    a.Tq = Tq;
    a.Cp = L.Cp;
    a.h = h;
    hipStream_t s = (hipStream_t)stream;
    a.tiles_m = blocks(Tq, 128);
    a.tiles_n = (uint32_t)nct;
    launch(SSM_PROF_FWD, true, true, gemm_kernel<EPI_FWD, 2, kFwdWN, kFwdBK, kFwdS>, dim3(grid_blocks(a.tiles_m, a.tiles_n)),
           dim3(256), s, a);
    launch(SSM_PROF_LSE, true, true, lse_kernel, dim3(blocks(T * kLseLanes, 256)), dim3(256), s,
           (const float2 *)a.part, T, nct, slot, C, (const float *)a.zt, loss, lse, h);
    return done(hipGetLastError());
}

int ssm_loss_bwd(const ssm_config *cfg, void *ws, const void *X, const void *W, const int32_t *cand,
                 const int32_t *slot, const float *lse, const float *dloss, int64_t T, float *dX,
                 float *dW, void *stream)
{
    int rc = check_loss_args(cfg, ws, X, W, cand, slot, T);
    if (rc)
        return rc;
    if (!lse || !dloss || !dX || !dW)
        return SSM_ENULL;
    if (!aligned(dX, 16) || !aligned(dW, 16))
        return SSM_EALIGN;
    if (T == 0)
        return SSM_OK;
    const Layout L = layout(cfg);
    uint8_t *w = (uint8_t *)ws;
    Hdr *h = reinterpret_cast<Hdr *>(w + L.hdr);
    const int32_t V = cfg->vocab, C = cfg->candidates;
    const int64_t Tq = rup(T, kTile), Cp = L.Cp;
    uint16_t *xt = reinterpret_cast<uint16_t *>(w + L.xt);
    uint16_t *wst = reinterpret_cast<uint16_t *>(w + L.wst);
    uint16_t *dz = reinterpret_cast<uint16_t *>(w + L.dz);
    hipStream_t s = (hipStream_t)stream;

    const Rows xr{(const uint16_t *)X, kD, nullptr, (int32_t)T, V};
    const Rows wr{(const uint16_t *)W, kD, cand, C, V};
    launch(SSM_PROF_TRANS, true, false, transpose_kernel, dim3(blocks(Tq, 64), kD / 64), dim3(256), s, xr, T,
           xt, Tq, &h->flags);
    launch(SSM_PROF_TRANS, false, true, transpose_kernel, dim3(blocks(Cp, 64), kD / 64), dim3(256), s, wr,
           (int64_t)C, wst, Cp, &h->flags);

    GemmArgs a{};
    a.T = T;
    a.C = C;
    a.V = V;
    a.slot = slot;
    a.cand = cand;
    a.lse = lse;
    a.g = dloss;
    a.dz = dz;
    a.zb = reinterpret_cast<uint16_t *>(w + L.zb);
    a.part = reinterpret_cast<float2 *>(w + L.part);
    a.Tq = Tq;
    a.Cp = Cp;
    a.h = h;

    a.tiles_m = blocks(Tq, 128);
    a.tiles_n = blocks(Cp, 128);
    launch(SSM_PROF_DZ, true, true, dz_kernel, dim3(grid_blocks(a.tiles_m, a.tiles_n)), dim3(256), s, a);

    a.A = Rows{dz, Cp, nullptr, (int32_t)Tq, V};
    a.B = Rows{wst, Cp, nullptr, kD, V};
    a.K = Cp;
    a.out = dX;
    a.tiles_m = blocks(Tq, 64 * kDxWM);
    a.tiles_n = kD / (64 * kDxWN);
    launch(SSM_PROF_DX, true, true, gemm_kernel<EPI_DX, kDxWM, kDxWN, kDxBK, kDxS>,
           dim3(grid_blocks(a.tiles_m, a.tiles_n)), dim3(256), s, a);

    a.A = Rows{dz, Cp, nullptr, (int32_t)Tq, V};   // k-major: rows of dz are positions
    a.B = Rows{xt, Tq, nullptr, kD, V};
    a.K = Tq;
    a.out = dW;
    a.tiles_m = blocks(Cp, 128);
    a.dwp = reinterpret_cast<float *>(w + L.dwp);
    // dW's blocks are few and long (k = T), so the last round of resident
    // blocks (two per CU) decides much of its time.  Choose the tile and the
    // number of parts of k by modelled time: 128 x 192 tiles do about 1.25x
    // the work per unit time of 128 x 128 ones (measured at equal fill), a
    // split costs its reduction (about 3 %), and the rounds' fill is known.
    int wn = 2, split = 1;
    double best = 0.0;
    const int64_t nk = Tq / kDwBK;
    for (int cwn = 2; cwn <= 3; ++cwn)
        for (int p = 1; p <= kMaxSplit && p <= nk; ++p) {
            const uint32_t nb = a.tiles_m * (uint32_t)(kD / (64 * cwn)) * (uint32_t)p;
            const double score = (cwn == 3 ? 1.25 : 1.0) * round_fill(nb, 2 * kCUs) * (p > 1 ? 0.97 : 1.0);
            if (score > best + 1e-9) {
                best = score;
                wn = cwn;
                split = p;
            }
        }
    a.ksplit = split;
    a.tiles_n = kD / (64 * wn);
    const dim3 grid(grid_blocks(a.tiles_m * (uint32_t)split, a.tiles_n));
    if (wn == 3)
        launch(SSM_PROF_DW, true, split == 1, gemm_kernel<EPI_DW, 2, 3, kDwBK, kDwS>, grid, dim3(256), s, a);
    else
        launch(SSM_PROF_DW, true, split == 1, gemm_kernel<EPI_DW, 2, 2, kDwBK, kDwS>, grid, dim3(256), s, a);
    if (split > 1)
        launch(SSM_PROF_DW, false, true, dw_reduce_kernel, dim3(blocks((int64_t)C * (kD / 4), 256)), dim3(256), s,
               (const float *)a.dwp, split, Cp, cand, C, V, dW);
    return done(hipGetLastError());
}

int ssm_device_status(const ssm_config *cfg, const void *ws, uint32_t *flags, int clear, void *stream)
{
    const int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (!ws || !flags)
        return SSM_ENULL;
    if (!aligned(ws, kAlign))
        return SSM_EALIGN;
    const Layout L = layout(cfg);
    hipStream_t s = (hipStream_t)stream;
    const Hdr *h = reinterpret_cast<const Hdr *>((const uint8_t *)ws + L.hdr);
    if (hipStreamSynchronize(s) != hipSuccess)
        return SSM_EHIP;
    if (hipMemcpy(flags, &h->flags, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
        return SSM_EHIP;
    if (clear) {
        flags_clear_kernel<<<1, 64, 0, s>>>(const_cast<Hdr *>(h));
        if (hipGetLastError() != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
            return SSM_EHIP;
    }
    return SSM_OK;
}

int ssm_profile_events(int group, void *start_event, void *stop_event)
{
    if (group < 0 || group >= SSM_PROF_GROUPS)
        return SSM_EARG;
    g_prof[group].start = (hipEvent_t)start_event;
    g_prof[group].stop = (hipEvent_t)stop_event;
    return SSM_OK;
}

}   // extern "C"
