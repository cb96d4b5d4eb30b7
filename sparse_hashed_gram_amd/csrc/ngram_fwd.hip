// Hash, forward gather-sum, and the burst-mode stash (gfx950).
//
// Forward (modded-nanogpt README, technique list: hashed bigram + trigram
// table with sign trick): out[i] = s_b W_b[r_b(i)] + s_t W_t[r_t(i)].
// A 768-wide row is 96 (bf16) or 192 (fp32) 16-byte chunks.  A block owns 64
// consecutive positions: 64 threads hash them into LDS, then all 256 threads
// sweep the 64 x chunks grid so that consecutive lanes read consecutive
// 16-byte pieces of a row (coalesced 1.5 KB / 3 KB row reads) and write the
// output rows contiguously.  Each thread keeps several chunks' loads in
// flight before it consumes any of them.
#include "ngram_dev.hpp"

#include "../../include/ngram.h"

namespace ngram {

namespace {

constexpr int kFwdTok = 64;
constexpr int kFwdThreads = 256;

__device__ __forceinline__ uint4 add_bf16x8(uint4 a, uint4 b)
{
    uint4 r;
    r.x = bf16_pack(bf16_lo(a.x) + bf16_lo(b.x), bf16_hi(a.x) + bf16_hi(b.x));
    r.y = bf16_pack(bf16_lo(a.y) + bf16_lo(b.y), bf16_hi(a.y) + bf16_hi(b.y));
    r.z = bf16_pack(bf16_lo(a.z) + bf16_lo(b.z), bf16_hi(a.z) + bf16_hi(b.z));
    r.w = bf16_pack(bf16_lo(a.w) + bf16_lo(b.w), bf16_hi(a.w) + bf16_hi(b.w));
    return r;
}

__device__ __forceinline__ uint4 add_f32x4(uint4 a, uint4 b)
{
    uint4 r;
    r.x = __float_as_uint(__uint_as_float(a.x) + __uint_as_float(b.x));
    r.y = __float_as_uint(__uint_as_float(a.y) + __uint_as_float(b.y));
    r.z = __float_as_uint(__uint_as_float(a.z) + __uint_as_float(b.z));
    r.w = __float_as_uint(__uint_as_float(a.w) + __uint_as_float(b.w));
    return r;
}

// Negation is a sign-bit flip of every element: exact for both dtypes.
__device__ __forceinline__ uint4 flip(uint4 a, uint32_t m)
{
    return make_uint4(a.x ^ m, a.y ^ m, a.z ^ m, a.w ^ m);
}

// The exact fp32 sum of two signed bf16 quads, as two float quads (the
// forward's fp32 output of a bf16 table: the sum, not rounded again).
__device__ __forceinline__ void add_bf16x8_f32(uint4 a, uint4 b, uint4 &lo, uint4 &hi)
{
    lo.x = __float_as_uint(bf16_lo(a.x) + bf16_lo(b.x));
    lo.y = __float_as_uint(bf16_hi(a.x) + bf16_hi(b.x));
    lo.z = __float_as_uint(bf16_lo(a.y) + bf16_lo(b.y));
    lo.w = __float_as_uint(bf16_hi(a.y) + bf16_hi(b.y));
    hi.x = __float_as_uint(bf16_lo(a.z) + bf16_lo(b.z));
    hi.y = __float_as_uint(bf16_hi(a.z) + bf16_hi(b.z));
    hi.z = __float_as_uint(bf16_lo(a.w) + bf16_lo(b.w));
    hi.w = __float_as_uint(bf16_hi(a.w) + bf16_hi(b.w));
}

// ELT: table element bytes; OUT_F32: fp32 output for a bf16 table (else the
// output has the table's dtype); DIRECT: one token-indexed table, the output
// is its row as stored (no second row, no sign).
template <int ELT, bool OUT_F32 = false, bool DIRECT = false>
__global__ __launch_bounds__(kFwdThreads) void fwd_kernel(const int32_t *__restrict__ tok, int64_t T,
                                                          HashParams hp,
                                                          const uint8_t *__restrict__ wb,
                                                          const uint8_t *__restrict__ wt,
                                                          uint8_t *__restrict__ out,
                                                          uint32_t *__restrict__ flags)
{
    constexpr int kRowBytes = kDim * ELT;
    constexpr int kCpr = kRowBytes / 16;                  // 16-byte chunks per row
    constexpr int kIter = kFwdTok * kCpr / kFwdThreads;   // 24 (bf16) or 48 (fp32)
    constexpr int kU = 4;                                 // chunks in flight per thread
    constexpr uint32_t kSign = ELT == 2 ? 0x80008000u : 0x80000000u;
    static_assert(kIter % kU == 0, "unroll must divide the sweep");

    __shared__ uint32_t s_idx[2][kFwdTok];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kFwdTok;
    if (tid < kFwdTok) {
        uint32_t ib = 0, it = 0;
        const int64_t i = t0 + tid;
        if (i < T) {
            if (ngram_index(tok, i, hp, ib, it) && flags)
                atomicOr(flags, NGRAM_FLAG_BAD_TOKEN);
        }
        s_idx[0][tid] = ib;
        s_idx[1][tid] = it;
    }
    __syncthreads();
    const int ntok = (int)min<int64_t>(kFwdTok, T - t0);
    constexpr int kOutRowBytes = OUT_F32 ? kDim * 4 : kRowBytes;
    uint4 *orow = reinterpret_cast<uint4 *>(out + (size_t)t0 * kOutRowBytes);

#pragma unroll
    for (int g = 0; g < kIter; g += kU) {
        uint4 a[kU], b[kU];
        int e[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            e[u] = tid + (g + u) * kFwdThreads;
            const int lt = e[u] / kCpr;
            const int c = e[u] - lt * kCpr;
            if (lt < ntok) {
                const uint32_t ib = s_idx[0][lt], it = s_idx[1][lt];
                const uint4 *pb = reinterpret_cast<const uint4 *>(wb + (size_t)(ib & 0x7FFFFFFFu) * kRowBytes) + c;
                const uint4 *pt = reinterpret_cast<const uint4 *>(wt + (size_t)(it & 0x7FFFFFFFu) * kRowBytes) + c;
                a[u] = flip(*pb, (ib >> 31) ? kSign : 0u);
                if (!DIRECT)
                    b[u] = flip(*pt, (it >> 31) ? kSign : 0u);
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int lt = e[u] / kCpr;
            if (lt < ntok) {   // output rows are written once: streaming stores
                if constexpr (OUT_F32 && ELT == 2) {
                    // chunk c of a bf16 row holds elements 8c..8c+7: fp32 pieces 2c, 2c+1
                    uint4 lo, hi;
                    // x + (-0) = x for every x, signed zeros and NaN included:
                    // the direct row widens exactly
                    add_bf16x8_f32(a[u], DIRECT ? make_uint4(0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u) : b[u],
                                   lo, hi);
                    const int c = e[u] - lt * kCpr;
                    uint4 *o = orow + (size_t)lt * (kOutRowBytes / 16) + 2 * c;
                    st_global_nt<uint4>((uint64_t)o, lo);
                    st_global_nt<uint4>((uint64_t)(o + 1), hi);
                } else {
                    st_global_nt<uint4>((uint64_t)(orow + e[u]),
                                        DIRECT ? a[u] : ELT == 2 ? add_bf16x8(a[u], b[u]) : add_f32x4(a[u], b[u]));
                }
            }
        }
    }
}

__global__ void hash_kernel(const int32_t *__restrict__ tok, int64_t T, HashParams hp,
                            uint32_t *__restrict__ idx, uint32_t *__restrict__ flags)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T)
        return;
    uint32_t ib, it;
    if (ngram_index(tok, i, hp, ib, it) && flags)
        atomicOr(flags, NGRAM_FLAG_BAD_TOKEN);
    idx[i] = ib;
    idx[T + i] = it;
}

// Burst modes: keep the packed indices of one micro-step at the end of the
// stash, with each position's dY row code: the stash position itself when the
// dY rows are copied next to it (copying burst), or micro-step << pos_bits |
// position when dY stays where the caller keeps it (burst by reference).
// A micro-step's keys may have been kept ahead (KEYS_ONLY launch, from its
// tokens alone); its backward then only attaches the gradients: the address
// (by reference) or a copy of the dY rows (copying burst) at the positions
// its keys took.
// One block per 256 positions: each thread hashes one; when copying, the
// block then copies its 256 dY rows in 16-byte pieces (row_bytes = 768 x the
// dY element size).  stash_advance_kernel then moves the counts forward.
constexpr int kStashTok = 256;
template <bool BY_REF, bool KEYS_ONLY>
__global__ __launch_bounds__(256) void stash_kernel(const int32_t *__restrict__ tok, const uint8_t *__restrict__ dY,
                                                    int64_t T, HashParams hp, uint32_t *__restrict__ sidx,
                                                    uint32_t *__restrict__ spos, uint8_t *__restrict__ sdy,
                                                    int row_bytes, int64_t nk, int pos_bits, int accum,
                                                    const MicroStep *__restrict__ mstep, WsHeader *__restrict__ hdr)
{
    const uint32_t mk = hdr->n_keyed;
    const uint32_t m = KEYS_ONLY ? mk : hdr->n_micro;
    const bool ahead = !KEYS_ONLY && m < mk;   // keys kept ahead: attach the gradients only
    uint32_t base;
    if (ahead) {
        const MicroStep ms = mstep[m];
        if (ms.T != (uint32_t)T)
            return;   // flagged by stash_advance_kernel
        base = ms.base;
    } else {
        base = hdr->n_stash;
        if ((int64_t)base + T > nk || (int)m >= accum)
            return;   // flagged by stash_advance_kernel
    }
    const int64_t t0 = (int64_t)blockIdx.x * kStashTok;
    const int tid = threadIdx.x;
    if (!ahead && t0 + tid < T) {
        const int64_t i = t0 + tid;
        uint32_t ib, it;
        if (ngram_index(tok, i, hp, ib, it))
            atomicOr(&hdr->flags, NGRAM_FLAG_BAD_TOKEN);
        sidx[base + i] = ib;
        sidx[nk + base + i] = it;
        spos[base + i] = BY_REF ? (m << pos_bits) | (uint32_t)i : base + (uint32_t)i;
    }
    if (!BY_REF && !KEYS_ONLY) {
        const int ntok = (int)min<int64_t>(kStashTok, T - t0);
        const uint4 *src = reinterpret_cast<const uint4 *>(dY + (size_t)t0 * row_bytes);
        uint4 *dst = reinterpret_cast<uint4 *>(sdy + ((size_t)base + t0) * row_bytes);
        for (int e = tid; e < ntok * (row_bytes / 16); e += 256)
            st_global_nt<uint4>((uint64_t)(dst + e), ld_global_nt<uint4>((uint64_t)(src + e)));
    }
}

// The counts after a stash_kernel launch (one thread; also the whole job
// when T = 0).  KEYS_ONLY: the micro-step's keys are kept, its gradients are
// still to come.
template <bool KEYS_ONLY>
__global__ void stash_advance_kernel(int64_t T, int64_t nk, int accum, const uint8_t *dY,
                                     const uint8_t **__restrict__ dy_ptrs, MicroStep *__restrict__ mstep,
                                     WsHeader *__restrict__ hdr)
{
    const uint32_t mk = hdr->n_keyed;
    const uint32_t m = KEYS_ONLY ? mk : hdr->n_micro;
    if (!KEYS_ONLY && m < mk) {   // attach to keys kept ahead
        if (mstep[m].T != (uint32_t)T) {
            atomicOr(&hdr->flags, NGRAM_FLAG_KEYS_MISMATCH);
            return;
        }
        if (dy_ptrs)
            dy_ptrs[m] = dY;
        hdr->n_micro = m + 1;
        return;
    }
    const uint32_t base = hdr->n_stash;
    if ((int64_t)base + T > nk || (int)m >= accum) {
        atomicOr(&hdr->flags, NGRAM_FLAG_STASH_FULL);
        return;
    }
    mstep[m] = MicroStep{base, (uint32_t)T};
    hdr->n_stash = base + (uint32_t)T;
    hdr->n_keyed = m + 1;
    if (!KEYS_ONLY) {
        if (dy_ptrs)
            dy_ptrs[m] = dY;
        hdr->n_micro = m + 1;
    }
}

__global__ void stash_clear_kernel(WsHeader *__restrict__ hdr)
{
    hdr->n_stash = 0;
    hdr->n_micro = 0;
    hdr->n_keyed = 0;
    hdr->sorted_n = 0;
}

__global__ void flags_clear_kernel(WsHeader *__restrict__ hdr) { hdr->flags = 0; }

__global__ void flags_export_kernel(const WsHeader *__restrict__ hdr, uint32_t *__restrict__ out)
{
    *out |= hdr->flags;
}

__global__ void fill_u32_kernel(uint32_t *__restrict__ p, uint64_t n, uint32_t v)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

unsigned grid_for(int64_t n, int per)
{
    return (unsigned)((n + per - 1) / per);
}

}  // namespace

hipError_t launch_init(const WsLayout &L, uint8_t *ws, hipStream_t s)
{
    // header: zero everything, then the magic word and window epoch 1; slot
    // map entries start at epoch 0, i.e. in no window
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + L.hdr);
    fill_u32_kernel<<<1, 64, 0, s>>>(reinterpret_cast<uint32_t *>(hdr), sizeof(WsHeader) / 4, 0u);
    fill_u32_kernel<<<1, 1, 0, s>>>(&hdr->magic, 1, kMagic);
    fill_u32_kernel<<<1, 1, 0, s>>>(&hdr->epoch, 1, 1u);
    if (L.one_shot)
        return hipGetLastError();   // no slot maps
    for (int c = 0; c < 2; ++c)
        fill_u32_kernel<<<2048, 256, 0, s>>>(reinterpret_cast<uint32_t *>(ws + L.slot_map[c]),
                                             2 * (uint64_t)L.rows[c], 0u);
    return hipGetLastError();
}

hipError_t launch_hash(const HashParams &hp, const int32_t *tok, int64_t T, uint32_t *idx,
                       uint32_t *flags, hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    hash_kernel<<<grid_for(T, 256), 256, 0, s>>>(tok, T, hp, idx, flags);
    return hipGetLastError();
}

hipError_t launch_fwd(int dtype, bool out_f32, const HashParams &hp, const void *wb, const void *wt,
                      const int32_t *tok, int64_t T, void *out, uint32_t *flags, hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    const unsigned g = grid_for(T, kFwdTok);
    auto k = dtype == NGRAM_DTYPE_BF16 ? (out_f32 ? fwd_kernel<2, true> : fwd_kernel<2>) : fwd_kernel<4>;
    if (hp.direct)
        k = dtype == NGRAM_DTYPE_BF16 ? (out_f32 ? fwd_kernel<2, true, true> : fwd_kernel<2, false, true>)
                                      : fwd_kernel<4, false, true>;
    launch_prof(NGRAM_PROF_FWD, true, true, k, dim3(g),
                dim3(kFwdThreads), 0, s, tok, T, hp, wb, wt, out, flags);
    return hipGetLastError();
}

hipError_t launch_stash(const WsLayout &L, uint8_t *ws, const HashParams &hp, const int32_t *tok,
                        const void *dY, int64_t T, hipStream_t s)
{
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + L.hdr);
    uint32_t *sidx = reinterpret_cast<uint32_t *>(ws + L.stash_idx);
    uint32_t *spos = reinterpret_cast<uint32_t *>(ws + L.stash_pos);
    MicroStep *mstep = reinterpret_cast<MicroStep *>(ws + L.mstep);
    const uint8_t **dy_ptrs = L.by_ref ? reinterpret_cast<const uint8_t **>(ws + L.dy_ptrs) : nullptr;
    if (T > 0)
        launch_prof(NGRAM_PROF_STASH, true, false, L.by_ref ? stash_kernel<true, false> : stash_kernel<false, false>,
                    dim3(grid_for(T, kStashTok)), dim3(256), 0, s, tok, dY, T, hp, sidx, spos,
                    L.by_ref ? nullptr : ws + L.stash_dy, L.dy_elt * kDim, L.nk, L.pos_bits, L.accum, mstep, hdr);
    launch_prof(NGRAM_PROF_STASH, T == 0, true, stash_advance_kernel<false>, dim3(1), dim3(1), 0, s, T, L.nk,
                L.accum, dY, dy_ptrs, mstep, hdr);
    return hipGetLastError();
}

hipError_t launch_keys(const WsLayout &L, uint8_t *ws, const HashParams &hp, const int32_t *tok, int64_t T,
                       hipStream_t s)
{
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + L.hdr);
    uint32_t *sidx = reinterpret_cast<uint32_t *>(ws + L.stash_idx);
    uint32_t *spos = reinterpret_cast<uint32_t *>(ws + L.stash_pos);
    MicroStep *mstep = reinterpret_cast<MicroStep *>(ws + L.mstep);
    if (T > 0)
        launch_prof(NGRAM_PROF_STASH, true, false, L.by_ref ? stash_kernel<true, true> : stash_kernel<false, true>,
                    dim3(grid_for(T, kStashTok)), dim3(256), 0, s, tok, nullptr, T, hp, sidx, spos, nullptr,
                    L.dy_elt * kDim, L.nk, L.pos_bits, L.accum, mstep, hdr);
    launch_prof(NGRAM_PROF_STASH, T == 0, true, stash_advance_kernel<true>, dim3(1), dim3(1), 0, s, T, L.nk,
                L.accum, nullptr, nullptr, mstep, hdr);
    return hipGetLastError();
}

hipError_t launch_stash_clear(const WsLayout &L, uint8_t *ws, hipStream_t s)
{
    stash_clear_kernel<<<1, 1, 0, s>>>(reinterpret_cast<WsHeader *>(ws + L.hdr));
    return hipGetLastError();
}

hipError_t launch_flags_clear(uint8_t *ws, const WsLayout &L, hipStream_t s)
{
    flags_clear_kernel<<<1, 1, 0, s>>>(reinterpret_cast<WsHeader *>(ws + L.hdr));
    return hipGetLastError();
}

hipError_t launch_flags_export(const WsLayout &L, const uint8_t *ws, uint32_t *out, hipStream_t s)
{
    flags_export_kernel<<<1, 1, 0, s>>>(reinterpret_cast<const WsHeader *>(ws + L.hdr), out);
    return hipGetLastError();
}

}  // namespace ngram
