// C ABI of libngram: argument checks, workspace layout, launches.
//
// Host code only.  Every entry point validates its arguments before touching
// the HIP runtime, so a rejected call enqueues nothing.  The hot calls never
// allocate, free or synchronise: device-side counts (distinct rows, kept
// positions) stay in the workspace header and kernels read them, with grids
// sized from host-known bounds.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/ngram.h"
#include "ngram_dev.hpp"

using namespace ngram;

namespace ngram {
thread_local ProfSlot g_prof[kProfGroups] = {};
}

static_assert(sizeof(ngram_config) == 80, "ngram_config layout (the Python binding mirrors it)");

namespace {

constexpr uint64_t kAlign = 256;

uint64_t up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int check_cfg(const ngram_config *c)
{
    if (!c)
        return NGRAM_ENULL;
    if (c->vocab < 1 || c->vocab > (1 << 30))
        return NGRAM_ECONFIG;
    if (c->eos_id < 0 || c->eos_id >= c->vocab)
        return NGRAM_ECONFIG;
    if (c->dim != kDim)
        return NGRAM_ECONFIG;
    if (c->dtype != NGRAM_DTYPE_F32 && c->dtype != NGRAM_DTYPE_BF16)
        return NGRAM_ECONFIG;
    for (int k = 0; k < 2; ++k)
        if (c->rows[k] < 1 || c->rows[k] > INT32_MAX)
            return NGRAM_ECONFIG;
    if (c->max_tokens < 1 || c->max_tokens > (int64_t(1) << 28))
        return NGRAM_ECONFIG;
    if (c->accum_steps < 1 || c->accum_steps > 64)
        return NGRAM_ECONFIG;
    if (c->mode != NGRAM_MODE_SPREAD && c->mode != NGRAM_MODE_BURST && c->mode != NGRAM_MODE_BURST_REF)
        return NGRAM_ECONFIG;
    if (c->mode != NGRAM_MODE_SPREAD && (int64_t)c->accum_steps * c->max_tokens > (int64_t(1) << 30))
        return NGRAM_ECONFIG;
    if (c->mode == NGRAM_MODE_BURST_REF && c->max_tokens > (int64_t(1) << 25))
        return NGRAM_ECONFIG;
    if (c->window_rows < 0)
        return NGRAM_ECONFIG;
    if (c->dy_dtype != NGRAM_DTYPE_F32 && c->dy_dtype != NGRAM_DTYPE_BF16)
        return NGRAM_ECONFIG;
    if ((c->options & ~(NGRAM_OPT_PRESORT | NGRAM_OPT_OUT_F32 | NGRAM_OPT_DIRECT | NGRAM_OPT_NEST_ALWAYS)) != 0)
        return NGRAM_ECONFIG;
    if ((c->options & NGRAM_OPT_DIRECT) && c->rows[0] < c->vocab)
        return NGRAM_ECONFIG;   // every token id needs its row
    if ((c->options & NGRAM_OPT_PRESORT) && c->mode == NGRAM_MODE_SPREAD)
        return NGRAM_ECONFIG;
    {   // window slots must fit 30 bits (the singleton map packs new and sign bits above them)
        const int64_t window_keys = (int64_t)c->accum_steps * c->max_tokens;
        const int64_t rmax = c->rows[0] > c->rows[1] ? c->rows[0] : c->rows[1];
        const int64_t wrows = c->window_rows > 0 ? c->window_rows : (window_keys < rmax ? window_keys : rmax);
        if (wrows >= kMaxWindowRows)
            return NGRAM_ECONFIG;
    }
    return NGRAM_OK;
}

// one_shot: the layout of a whole burst window reduced and stepped in one
// call on an empty window (ngram_window_step_noalloc): the slot maps, slot
// rows and window accumulator, which only rows of an earlier reduce of the
// window would use, take no memory.
WsLayout layout(const ngram_config *c, bool one_shot = false)
{
    WsLayout L;
    memset(&L, 0, sizeof(L));
    L.one_shot = one_shot;
    L.burst = c->mode != NGRAM_MODE_SPREAD;
    L.by_ref = c->mode == NGRAM_MODE_BURST_REF;
    L.accum = c->accum_steps;
    L.nch = (c->options & NGRAM_OPT_DIRECT) ? 1 : 2;
    L.dy_elt = c->dy_dtype == NGRAM_DTYPE_BF16 ? 2 : 4;
    L.pos_bits = 0;
    while ((int64_t(1) << L.pos_bits) < c->max_tokens)
        ++L.pos_bits;
    L.rows[0] = c->rows[0];
    L.rows[1] = c->rows[1];
    const int64_t window_keys = (int64_t)c->accum_steps * c->max_tokens;
    const int64_t rmax = c->rows[0] > c->rows[1] ? c->rows[0] : c->rows[1];
    L.wrows = c->window_rows > 0 ? c->window_rows : (window_keys < rmax ? window_keys : rmax);
    L.nk = L.burst ? window_keys : c->max_tokens;
    L.nblk = (L.nk + kSortTile - 1) / kSortTile;
    L.nrblk = (L.nk + radix_tile(kRadixItemsSmall) - 1) / radix_tile(kRadixItemsSmall);   // the most radix tiles
    L.nchunk = (L.nk + kChunk - 1) / kChunk;
    int bits = 0;
    while (bits < 31 && ((int64_t(1) << bits) < rmax))
        ++bits;
    L.passes = bits == 0 ? 1 : (bits + kRadixBits - 1) / kRadixBits;

    uint64_t o = 0;
    L.hdr = o;
    o = up(o + sizeof(WsHeader));
    for (int k = 0; k < 2; ++k) {
        L.slot_map[k] = o;
        o = up(o + (one_shot ? 0 : sizeof(SlotEntry) * (uint64_t)c->rows[k]));
    }
    for (int k = 0; k < 2; ++k) {
        L.slot_rows[k] = o;
        o = up(o + (one_shot ? 0 : 4ull * (uint64_t)L.wrows));
    }
    L.gacc = o;
    o = up(o + (one_shot ? 0 : 4ull * 2 * (uint64_t)L.wrows * kDim));
    for (int k = 0; k < 2; ++k) {
        L.keys[k] = o;
        o = up(o + 4ull * 2 * (uint64_t)L.nk);
        L.vals[k] = o;
        o = up(o + 4ull * 2 * (uint64_t)L.nk);
    }
    L.seg_info = o;
    o = up(o + 4ull * 2 * (uint64_t)L.nk);
    L.hist = o;
    o = up(o + 4ull * 2 * kRadix * (uint64_t)L.nrblk);
    L.tot = o;
    o = up(o + 4ull * 2 * kRadix);
    L.blk = o;
    o = up(o + 4ull * 2 * (uint64_t)L.nblk);
    L.kept = o;
    o = up(o + 4ull * (uint64_t)L.nblk);
    L.partial = o;
    o = up(o + 4ull * 2 * (uint64_t)L.nchunk * 2 * kDim);
    L.owners = o;
    o = up(o + 8ull * 2 * (uint64_t)L.nchunk);
    L.ngroup = (L.nchunk + kGroup - 1) / kGroup;
    L.gpart = o;
    o = up(o + 4ull * 2 * (uint64_t)L.ngroup * kDim);
    L.code_cap = L.by_ref ? ((int64_t)L.accum << L.pos_bits) : L.nk;
    L.tinfo = o;
    o = up(o + 4ull * (uint64_t)L.code_cap);
    // nested trigram records keep four flag bits above the row
    L.nested = L.nch == 2 && c->rows[1] <= (int64_t(1) << 28);
    L.nest_always = (c->options & NGRAM_OPT_NEST_ALWAYS) != 0;
    L.bidx = o;
    o = up(o + (L.nested ? 4ull * (uint64_t)L.code_cap : 0));
    L.btro = o;
    o = up(o + (L.nested ? 4ull * (uint64_t)L.nk : 0));
    for (int k = 0; k < 2; ++k) {
        L.tix[k] = o;
        o = up(o + (L.nested ? 4ull * (uint64_t)L.nk : 0));
    }
    L.tpart = o;
    o = up(o + (L.nested ? 4ull * (uint64_t)L.nchunk * 2 * kDim : 0));
    L.trec = o;
    o = up(o + (L.nested ? 8ull * (uint64_t)L.nchunk : 0));
    L.tkept = o;
    o = up(o + (L.nested ? (uint64_t)L.nk : 0));
    if (L.burst) {
        L.stash_idx = o;
        o = up(o + 4ull * 2 * (uint64_t)L.nk);
        L.stash_pos = o;
        o = up(o + 4ull * (uint64_t)L.nk);
        L.mstep = o;
        o = up(o + sizeof(MicroStep) * kMaxMicro);
        if (L.by_ref) {
            L.dy_ptrs = o;
            o = up(o + 8ull * kMaxMicro);
        } else {
            L.stash_dy = o;
            o = up(o + (uint64_t)L.dy_elt * (uint64_t)L.nk * kDim);
        }
    }
    // ngram_touched_rows: a bit per table row and the set bits per block of
    // 8,192 words (none in the one-call window's layout)
    uint64_t tw_max = 0;
    for (int k = 0; k < 2; ++k) {
        const uint64_t words = one_shot ? 0 : ((uint64_t)c->rows[k] + 31) / 32;
        L.tbits[k] = o;
        o = up(o + 4 * words);
        tw_max = words > tw_max ? words : tw_max;
    }
    L.tblk = o;
    o = up(o + 4 * ((tw_max + 8191) / 8192));
    L.total = o;
    return L;
}

HashParams hash_params(const ngram_config *c)
{
    HashParams hp;
    hp.vocab = (uint32_t)c->vocab;
    hp.eos = c->eos_id;
    hp.rows[0] = (uint32_t)c->rows[0];
    hp.rows[1] = (uint32_t)c->rows[1];
    hp.seed[0] = c->seed[0];
    hp.seed[1] = c->seed[1];
    hp.direct = (c->options & NGRAM_OPT_DIRECT) ? 1u : 0u;
    return hp;
}

int hip_status(hipError_t e) { return e == hipSuccess ? NGRAM_OK : NGRAM_EHIP; }

int check_tokens(const ngram_config *c, const int32_t *tok, int64_t T)
{
    if (T < 0 || T > c->max_tokens)
        return NGRAM_ESIZE;
    if (T > 0 && !tok)
        return NGRAM_ENULL;
    if (!aligned(tok, 4))
        return NGRAM_EALIGN;
    return NGRAM_OK;
}

uint32_t *flags_of(void *ws) { return ws ? &reinterpret_cast<WsHeader *>(ws)->flags : nullptr; }

}  // namespace

extern "C" {

int ngram_abi_version(void) { return NGRAM_ABI_VERSION; }

const char *ngram_status_string(int s)
{
    switch (s) {
    case NGRAM_OK: return "ok";
    case NGRAM_ENULL: return "a required pointer is NULL";
    case NGRAM_EALIGN: return "a pointer is not aligned as required";
    case NGRAM_ECONFIG: return "invalid ngram_config";
    case NGRAM_ESIZE: return "a size is out of range";
    case NGRAM_EARG: return "a scalar argument is out of range";
    case NGRAM_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int ngram_config_check(const ngram_config *cfg) { return check_cfg(cfg); }

int ngram_workspace_bytes(const ngram_config *cfg, uint64_t *bytes)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (!bytes)
        return NGRAM_ENULL;
    *bytes = layout(cfg).total;
    return NGRAM_OK;
}

int ngram_workspace_init(const ngram_config *cfg, void *ws, uint64_t ws_bytes, void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (!ws)
        return NGRAM_ENULL;
    if (!aligned(ws, kAlign))
        return NGRAM_EALIGN;
    const WsLayout L = layout(cfg);
    if (ws_bytes < L.total)
        return NGRAM_ESIZE;
    return hip_status(launch_init(L, (uint8_t *)ws, (hipStream_t)stream));
}

int ngram_hash(const ngram_config *cfg, const int32_t *tokens, int64_t T, uint32_t *idx, void *ws,
               void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if ((rc = check_tokens(cfg, tokens, T)))
        return rc;
    if (T > 0 && !idx)
        return NGRAM_ENULL;
    if (!aligned(idx, 4) || !aligned(ws, kAlign))
        return NGRAM_EALIGN;
    return hip_status(launch_hash(hash_params(cfg), tokens, T, idx, flags_of(ws), (hipStream_t)stream));
}

int ngram_embed_fwd(const ngram_config *cfg, const void *W_b, const void *W_t, const int32_t *tokens,
                    int64_t T, void *out, void *ws, void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if ((rc = check_tokens(cfg, tokens, T)))
        return rc;
    const bool direct = (cfg->options & NGRAM_OPT_DIRECT) != 0;   // W_t is not used then
    if (!W_b || (!W_t && !direct) || (T > 0 && !out))
        return NGRAM_ENULL;
    if (!aligned(W_b, 16) || !aligned(W_t, 16) || !aligned(out, 16) || !aligned(ws, kAlign))
        return NGRAM_EALIGN;
    return hip_status(launch_fwd(cfg->dtype, (cfg->options & NGRAM_OPT_OUT_F32) != 0, hash_params(cfg), W_b, W_t,
                                 tokens, T, out, flags_of(ws),
                                 (hipStream_t)stream));
}

int ngram_embed_bwd_accum(const ngram_config *cfg, void *ws, const int32_t *tokens, const void *dY,
                          int64_t T, void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if ((rc = check_tokens(cfg, tokens, T)))
        return rc;
    if (!ws || (T > 0 && !dY))
        return NGRAM_ENULL;
    if (!aligned(ws, kAlign) || !aligned(dY, 16))
        return NGRAM_EALIGN;
    const WsLayout L = layout(cfg);
    uint8_t *w = (uint8_t *)ws;
    hipStream_t s = (hipStream_t)stream;
    const HashParams hp = hash_params(cfg);
    if (L.burst)
        return hip_status(launch_stash(L, w, hp, tokens, dY, T, s));
    if (T == 0)
        return NGRAM_OK;
    return hip_status(launch_reduce(L, w, hp, tokens, T, dY, s));
}

int ngram_window_reduce(const ngram_config *cfg, void *ws, void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (!ws)
        return NGRAM_ENULL;
    if (!aligned(ws, kAlign))
        return NGRAM_EALIGN;
    const WsLayout L = layout(cfg);
    if (!L.burst)
        return NGRAM_OK;
    uint8_t *w = (uint8_t *)ws;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_reduce(L, w, hash_params(cfg), nullptr, L.nk, nullptr, s);
    if (e == hipSuccess)
        e = launch_stash_clear(L, w, s);
    return hip_status(e);
}

namespace {

int check_step_ptrs(const ngram_config *cfg, void *ws, void *W_b, void *W_t, ngram_row_state *state_b,
                    ngram_row_state *state_t)
{
    const bool direct = (cfg->options & NGRAM_OPT_DIRECT) != 0;   // the second table is not used then
    if (!ws || !W_b || !state_b || (!direct && (!W_t || !state_t)))
        return NGRAM_ENULL;
    if (!aligned(ws, kAlign) || !aligned(W_b, 16) || !aligned(W_t, 16) || !aligned(state_b, 8) ||
        !aligned(state_t, 8))
        return NGRAM_EALIGN;
    return NGRAM_OK;
}

int check_step_scalars(int32_t t, float lr, float beta2, float eps)
{
    if (t < 1 || !isfinite(lr) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f) || !isfinite(eps))
        return NGRAM_EARG;
    return NGRAM_OK;
}

int check_params_ptr(const ngram_step_params *params)
{
    if (!params)
        return NGRAM_ENULL;
    if (!aligned(params, 16))
        return NGRAM_EALIGN;
    return NGRAM_OK;
}

FuseArgs fuse_args(const ngram_config *cfg, void *W_b, void *W_t, ngram_row_state *state_b,
                   ngram_row_state *state_t, int32_t t, float lr, float beta2, float eps,
                   const ngram_step_params *params)
{
    static_assert(sizeof(ngram_step_params) == sizeof(StepParams), "step parameter layout");
    FuseArgs f;
    f.w[0] = (uint8_t *)W_b;
    f.w[1] = (uint8_t *)W_t;
    f.st[0] = reinterpret_cast<RowState *>(state_b);
    f.st[1] = reinterpret_cast<RowState *>(state_t);
    f.p = StepParams{t, lr, beta2, eps};
    f.p_dev = reinterpret_cast<const StepParams *>(params);
    f.dtype = cfg->dtype;
    return f;
}

// Burst mode: reduce the kept micro-steps fused with the step (sorting them
// first unless the caller sorts each window: NGRAM_OPT_PRESORT), then step
// the rows the window held from an earlier explicit reduce (if any) and end
// the window (which also empties the stash).
int burst_step(const ngram_config *cfg, const WsLayout &L, uint8_t *w, const FuseArgs &f, hipStream_t s)
{
    hipError_t e = (cfg->options & NGRAM_OPT_PRESORT)
                       ? launch_reduce_step_sorted(L, w, f, s)
                       : launch_reduce_step(L, w, hash_params(cfg), nullptr, L.nk, nullptr, f, s);
    if (e == hipSuccess)
        e = launch_step(L, w, f, s);
    return hip_status(e);
}

int sparse_step_impl(const ngram_config *cfg, void *ws, const FuseArgs &f, hipStream_t s)
{
    const WsLayout L = layout(cfg);
    uint8_t *w = (uint8_t *)ws;
    if (L.burst)
        return burst_step(cfg, L, w, f, s);
    return hip_status(launch_step(L, w, f, s));
}

int bwd_step_impl(const ngram_config *cfg, void *ws, const int32_t *tokens, const void *dY, int64_t T,
                  const FuseArgs &f, hipStream_t s)
{
    const WsLayout L = layout(cfg);
    uint8_t *w = (uint8_t *)ws;
    const HashParams hp = hash_params(cfg);
    if (L.burst) {
        hipError_t e = launch_stash(L, w, hp, tokens, dY, T, s);
        if (e != hipSuccess)
            return NGRAM_EHIP;
        return burst_step(cfg, L, w, f, s);
    }
    hipError_t e = hipSuccess;
    if (T > 0)
        e = launch_reduce_step(L, w, hp, tokens, T, dY, f, s);
    if (e == hipSuccess)
        e = launch_step(L, w, f, s);
    return hip_status(e);
}

int check_bwd_inputs(const ngram_config *cfg, const int32_t *tokens, const void *dY, int64_t T)
{
    int rc = check_tokens(cfg, tokens, T);
    if (rc)
        return rc;
    if (T > 0 && !dY)
        return NGRAM_ENULL;
    if (!aligned(dY, 16))
        return NGRAM_EALIGN;
    return NGRAM_OK;
}

}  // namespace

int ngram_sparse_step(const ngram_config *cfg, void *ws, void *W_b, void *W_t, ngram_row_state *state_b,
                      ngram_row_state *state_t, int32_t t, float lr, float beta2, float eps, void *stream)
{
    static_assert(sizeof(ngram_row_state) == sizeof(RowState), "row state layout");
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if ((rc = check_step_ptrs(cfg, ws, W_b, W_t, state_b, state_t)) || (rc = check_step_scalars(t, lr, beta2, eps)))
        return rc;
    return sparse_step_impl(cfg, ws, fuse_args(cfg, W_b, W_t, state_b, state_t, t, lr, beta2, eps, nullptr),
                            (hipStream_t)stream);
}

int ngram_sparse_step_dev(const ngram_config *cfg, void *ws, void *W_b, void *W_t, ngram_row_state *state_b,
                          ngram_row_state *state_t, const ngram_step_params *params, void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if ((rc = check_step_ptrs(cfg, ws, W_b, W_t, state_b, state_t)) || (rc = check_params_ptr(params)))
        return rc;
    return sparse_step_impl(cfg, ws, fuse_args(cfg, W_b, W_t, state_b, state_t, 0, 0.f, 0.f, 0.f, params),
                            (hipStream_t)stream);
}

int ngram_embed_bwd_step(const ngram_config *cfg, void *ws, const int32_t *tokens, const void *dY, int64_t T,
                         void *W_b, void *W_t, ngram_row_state *state_b, ngram_row_state *state_t, int32_t t,
                         float lr, float beta2, float eps, void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if ((rc = check_bwd_inputs(cfg, tokens, dY, T)))
        return rc;
    if ((rc = check_step_ptrs(cfg, ws, W_b, W_t, state_b, state_t)) || (rc = check_step_scalars(t, lr, beta2, eps)))
        return rc;
    return bwd_step_impl(cfg, ws, tokens, dY, T,
                         fuse_args(cfg, W_b, W_t, state_b, state_t, t, lr, beta2, eps, nullptr),
                         (hipStream_t)stream);
}

int ngram_embed_bwd_step_dev(const ngram_config *cfg, void *ws, const int32_t *tokens, const void *dY, int64_t T,
                             void *W_b, void *W_t, ngram_row_state *state_b, ngram_row_state *state_t,
                             const ngram_step_params *params, void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if ((rc = check_bwd_inputs(cfg, tokens, dY, T)))
        return rc;
    if ((rc = check_step_ptrs(cfg, ws, W_b, W_t, state_b, state_t)) || (rc = check_params_ptr(params)))
        return rc;
    return bwd_step_impl(cfg, ws, tokens, dY, T,
                         fuse_args(cfg, W_b, W_t, state_b, state_t, 0, 0.f, 0.f, 0.f, params),
                         (hipStream_t)stream);
}

int ngram_window_keys(const ngram_config *cfg, void *ws, const int32_t *tokens, int64_t T, void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if ((rc = check_tokens(cfg, tokens, T)))
        return rc;
    if (!ws)
        return NGRAM_ENULL;
    if (!aligned(ws, kAlign))
        return NGRAM_EALIGN;
    const WsLayout L = layout(cfg);
    if (!L.burst)
        return NGRAM_OK;   // spread mode reduces each micro-step with its gradients
    return hip_status(launch_keys(L, (uint8_t *)ws, hash_params(cfg), tokens, T, (hipStream_t)stream));
}

int ngram_window_sort(const ngram_config *cfg, void *ws, void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (!ws)
        return NGRAM_ENULL;
    if (!aligned(ws, kAlign))
        return NGRAM_EALIGN;
    const WsLayout L = layout(cfg);
    if (!L.burst)
        return NGRAM_OK;
    return hip_status(launch_window_sort(L, (uint8_t *)ws, hash_params(cfg), (hipStream_t)stream));
}

int ngram_window_export(const ngram_config *cfg, const void *ws, int channel, uint32_t *rows, float *G,
                        int64_t max_rows, uint32_t *count, void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (!ws || !rows || !count)
        return NGRAM_ENULL;
    if (channel != 0 && channel != 1)
        return NGRAM_EARG;
    if (max_rows < 0 || max_rows > INT32_MAX)
        return NGRAM_ESIZE;
    if (!aligned(ws, kAlign) || !aligned(rows, 4) || !aligned(G, 16) || !aligned(count, 4))
        return NGRAM_EALIGN;
    const WsLayout L = layout(cfg);
    return hip_status(launch_export(L, (const uint8_t *)ws, channel, rows, G, (uint32_t)max_rows, count,
                                    (hipStream_t)stream));
}

}  // extern "C"

// ------------------------------------------------ allocation-free window step
//
// For callers that cannot allocate device memory: the workspace of one whole
// window lives in `scratch`, a fixed array in this library's device code.
// Each GPU holds its own copy of the array at its own address; host code
// never uses the array's name except to ask for that address
// (hipGetSymbolAddress, once per device, kept in g_scratch).

namespace {

constexpr uint64_t kScratchBytes = 32ull << 20;
constexpr int64_t kNoallocMaxPositions = 65536;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
uint8_t *g_scratch[kMaxDevices];

// The device address of `scratch` on the current device, looked up on the
// first call there; nullptr if HIP fails.
uint8_t *scratch_ptr()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        g_scratch[dev] = static_cast<uint8_t *>(p);
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" {

int ngram_window_step_noalloc(const ngram_config *cfg, const int32_t *tokens, const void *dY, int64_t T,
                              int32_t n_micro, void *W_b, void *W_t, ngram_row_state *state_b,
                              ngram_row_state *state_t, int32_t t, float lr, float beta2, float eps, uint32_t *flags,
                              void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (T < 0 || n_micro < 1 || n_micro > kMaxMicro)
        return NGRAM_ESIZE;
    if ((int64_t)n_micro * T > kNoallocMaxPositions)
        return NGRAM_ESIZE;
    if (T > 0 && (!tokens || !dY))
        return NGRAM_ENULL;
    if (!aligned(tokens, 4) || !aligned(dY, 16))
        return NGRAM_EALIGN;
    const bool direct = (cfg->options & NGRAM_OPT_DIRECT) != 0;
    if (!W_b || !state_b || (!direct && (!W_t || !state_t)))
        return NGRAM_ENULL;
    if (!aligned(W_b, 16) || !aligned(W_t, 16) || !aligned(state_b, 8) || !aligned(state_t, 8) ||
        !aligned(flags, 4))
        return NGRAM_EALIGN;
    if ((rc = check_step_scalars(t, lr, beta2, eps)))
        return rc;
    if (T == 0)
        return NGRAM_OK;   // an empty window touches no row
    // the window as its own burst-by-reference configuration: n_micro
    // micro-steps of T positions, reduced fused with the step
    ngram_config c = *cfg;
    c.mode = NGRAM_MODE_BURST_REF;
    c.accum_steps = n_micro;
    c.max_tokens = T;
    c.window_rows = 0;
    c.options &= ~NGRAM_OPT_PRESORT;
    if ((rc = check_cfg(&c)))
        return rc;
    const WsLayout L = layout(&c, true);
    if (L.total > kScratchBytes)
        return NGRAM_ESIZE;
    uint8_t *ws = scratch_ptr();
    if (!ws)
        return NGRAM_EHIP;
    hipStream_t s = (hipStream_t)stream;
    const HashParams hp = hash_params(&c);
    const size_t dy_row = (size_t)L.dy_elt * kDim;
    hipError_t e = launch_init(L, ws, s);
    for (int m = 0; m < n_micro && e == hipSuccess; ++m)
        e = launch_stash(L, ws, hp, tokens + (size_t)m * T, static_cast<const uint8_t *>(dY) + (size_t)m * T * dy_row,
                         T, s);
    if (e != hipSuccess)
        return NGRAM_EHIP;
    rc = burst_step(&c, L, ws, fuse_args(&c, W_b, W_t, state_b, state_t, t, lr, beta2, eps, nullptr), s);
    if (rc == NGRAM_OK && flags)
        rc = hip_status(launch_flags_export(L, ws, flags, s));
    return rc;
}

int ngram_touched_rows(const ngram_config *cfg, void *ws, int channel, int32_t *rows, int64_t max_rows,
                       int64_t *count, void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (!ws || !count || (max_rows > 0 && !rows))
        return NGRAM_ENULL;
    if (channel != 0 && channel != 1)
        return NGRAM_EARG;
    if (max_rows < 0)
        return NGRAM_ESIZE;
    if (!aligned(ws, kAlign) || !aligned(rows, 4) || !aligned(count, 8))
        return NGRAM_EALIGN;
    const WsLayout L = layout(cfg);
    if (channel >= L.nch)   // a token-indexed table has no second channel: no rows
        return hip_status(launch_touched_none(count, (hipStream_t)stream));
    return hip_status(launch_touched(L, (uint8_t *)ws, channel, rows, (uint64_t)max_rows, count,
                                     (hipStream_t)stream));
}

int ngram_profile_events(int group, void *start_event, void *stop_event)
{
    if (group < 0 || group >= kProfGroups)
        return NGRAM_EARG;
    g_prof[group].start = (hipEvent_t)start_event;
    g_prof[group].stop = (hipEvent_t)stop_event;
    return NGRAM_OK;
}

int ngram_device_status(const ngram_config *cfg, const void *ws, uint32_t *flags, int clear, void *stream)
{
    int rc = check_cfg(cfg);
    if (rc)
        return rc;
    if (!ws || !flags)
        return NGRAM_ENULL;
    if (!aligned(ws, kAlign))
        return NGRAM_EALIGN;
    const WsLayout L = layout(cfg);
    hipStream_t s = (hipStream_t)stream;
    const WsHeader *hdr = reinterpret_cast<const WsHeader *>((const uint8_t *)ws + L.hdr);
    if (hipStreamSynchronize(s) != hipSuccess)
        return NGRAM_EHIP;
    if (hipMemcpy(flags, &hdr->flags, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
        return NGRAM_EHIP;
    if (clear) {
        if (launch_flags_clear((uint8_t *)ws, L, s) != hipSuccess)
            return NGRAM_EHIP;
        if (hipStreamSynchronize(s) != hipSuccess)
            return NGRAM_EHIP;
    }
    return NGRAM_OK;
}

}  // extern "C"
