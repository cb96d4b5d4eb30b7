// Host model of the indexing of the fused reduction + step (seg_step_kernel,
// group_sum_kernel and fixup_kernel in ngram_reduce.hip), for bounds checks on
// the CPU.  TEST INFRASTRUCTURE.
//
// Each 64-key chunk is planned and walked as the kernel's wavefront does,
// with the wavefront's 64 lanes as arrays and its ballots, readlanes and
// lane shuffles as loops.  Every address the kernel forms -- sorted keys,
// payloads and head info, the singleton map, dY rows (micro-step base +
// position), table rows and row state of both channels, window rows and
// slot rows, partial rows, fix-up records, group sums, nested trigram run
// pieces and their records -- is checked against the extent of its buffer
// before it would be used.  The model also checks what the indexing is for:
// every key is walked by exactly one wavefront, every segment is completed
// exactly once (in its chunk, by the owner of a one-chunk spill-over, or by
// the fix-up), every partial row, group sum and run piece the fix-up reads
// was written, every trigram row the bigram pass completes is stepped once,
// and every key of such a row is in exactly one completed sum.
//
// Build: g++ -O2 -std=c++17 -shared -fPIC seg_step_index.cpp (the test does).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

namespace {

constexpr int kWave = 64;
constexpr int kChunk = 64;
constexpr int kGroup = 64;
constexpr int kFixThreads = 512;
constexpr uint32_t kNewHead = 0xFFFFFFFEu;
constexpr uint32_t kNotSingle = 0xFFFFFFFFu;
constexpr uint32_t kMultiKey = 0x40000000u;
constexpr uint32_t kRunHead = 0x20000000u;
constexpr uint32_t kRunTail = 0x10000000u;
constexpr uint32_t kTrowMask = 0x0FFFFFFFu;

bool is_run(uint32_t t) { return t != kNotSingle && (t & kMultiKey) != 0; }

struct Ctx {
    // inputs
    int64_t n;              // keys of this channel
    const uint32_t *R, *V, *I;
    int64_t nk;             // capacity of the sorted arrays (R, V, I extents)
    const uint32_t *tinfo;  // singleton map (bigram pass only), code_cap entries
    int64_t code_cap;
    const uint32_t *tix;    // nested sort: per sorted key, the map's index (trigram order);
                            // null: the map is indexed by the key's row code
    int pos_bits;           // dY row code = micro-step << pos_bits | position
    int n_micro;            // micro-steps whose dY addresses are attached
    const int64_t *Tm;      // positions of each micro-step
    int64_t rows_c, rows_t; // rows of this channel's table and of the trigram table
    int64_t wrows;          // window slots
    int64_t nchunk, ngroup; // extents of the partial rows / fix-up records, group sums
    int step_u;             // keys per batch
    bool nested;            // the singleton map also names nested runs of several keys
    // results
    std::vector<int> walked;        // per key: wavefronts that walked it
    std::vector<int> completed;     // per key at a segment head: completions of the segment
    std::vector<int> tstepped;      // per dY row code: trigram rows stepped at this key
    std::vector<int> tsum;          // per dY row code: completed trigram sums holding this key
    std::vector<int> partial_w;     // [nchunk][2]: partial rows written
    std::vector<uint64_t> owners;   // fix-up records
    std::vector<int> tpart_w;       // [nchunk][2]: nested run pieces written
    std::vector<int64_t> tpart_lo, tpart_hi;   // [nchunk][2]: the piece's first and last key
    std::vector<uint64_t> trec;     // nested run records
    int64_t violations = 0;
    char first[256] = {0};
    int64_t accesses = 0;
};

void bad(Ctx &x, const char *what, int64_t idx, int64_t ext, int64_t chunk)
{
    if (x.violations++ == 0)
        snprintf(x.first, sizeof(x.first), "%s index %lld outside [0, %lld) in chunk %lld", what, (long long)idx,
                 (long long)ext, (long long)chunk);
}

bool in(Ctx &x, const char *what, int64_t idx, int64_t ext, int64_t chunk)
{
    ++x.accesses;
    if (idx < 0 || idx >= ext) {
        bad(x, what, idx, ext, chunk);
        return false;
    }
    return true;
}

uint32_t getR(Ctx &x, int64_t i, int64_t chunk)
{
    return in(x, "sorted row", i, x.nk, chunk) && in(x, "sorted row (count)", i, x.n, chunk) ? x.R[i] : 0u;
}

// The singleton-map record of sorted key i (payload v), as the kernel reads
// it: through tix in the nested sort, else by row code.
uint32_t rec_of(Ctx &x, int64_t i, uint32_t v, int64_t chunk)
{
    int64_t m = v & 0x7FFFFFFFu;
    if (x.tix) {
        if (!in(x, "tix", i, x.nk, chunk) || !in(x, "tix (count)", i, x.n, chunk))
            return kNotSingle;
        m = x.tix[i];
    }
    return in(x, "singleton map", m, x.code_cap, chunk) ? x.tinfo[m] : kNotSingle;
}

struct Plan {
    uint32_t r0[kWave], v0[kWave], i0[kWave], v1[kWave];
    uint64_t hm;
    int nv, j0, jend, la;
    bool first_cont, last_spills, owner_full;
    uint32_t row_last;
};

int ctz64(uint64_t m) { return __builtin_ctzll(m); }
int clz64(uint64_t m) { return __builtin_clzll(m); }

bool plan(Ctx &x, int64_t chunk, Plan &p)
{
    const int64_t c0 = chunk * kChunk;
    if (c0 >= x.n)
        return false;
    p.nv = (int)(x.n - c0 < kChunk ? x.n - c0 : kChunk);
    bool head[kWave];
    p.hm = 0;
    for (int l = 0; l < kWave; ++l) {
        const bool valid = l < p.nv;
        p.r0[l] = valid ? getR(x, c0 + l, chunk) : 0xFFFFFFFFu;
        p.v0[l] = valid && in(x, "sorted payload", c0 + l, x.nk, chunk) ? x.V[c0 + l] : 0u;
    }
    for (int l = 0; l < kWave; ++l) {
        uint32_t prev = l > 0 ? p.r0[l - 1] : (c0 > 0 ? getR(x, c0 - 1, chunk) : 0xFFFFFFFFu);
        head[l] = l < p.nv && p.r0[l] != prev;
        if (head[l])
            p.hm |= 1ull << l;
    }
    for (int l = 0; l < kWave; ++l)
        p.i0[l] = head[l] && in(x, "head info", c0 + l, x.nk, chunk) ? x.I[c0 + l] : 0u;
    p.row_last = p.r0[p.nv - 1];
    const bool cont_after = p.nv == kChunk && c0 + kChunk < x.n && getR(x, c0 + kChunk, chunk) == p.row_last;
    p.first_cont = !(p.hm & 1ull);
    const int e0 = p.hm ? ctz64(p.hm) : p.nv;
    bool skip_first = false;
    if (p.first_cont) {
        const uint32_t row0 = p.r0[0];
        const bool piece0_cont = (e0 == p.nv) && cont_after;
        const bool head_in_prev = (c0 == kChunk) || (getR(x, c0 - kChunk - 1, chunk) != row0);
        skip_first = head_in_prev && !piece0_cont;
    }
    p.la = p.hm ? 63 - clz64(p.hm) : -1;
    p.last_spills = p.hm && cont_after;
    p.owner_full = false;
    int extra = 0;
    for (int l = 0; l < kWave; ++l)
        p.v1[l] = 0;
    if (p.last_spills) {
        p.owner_full = !(c0 + 2 * kChunk < x.n && getR(x, c0 + 2 * kChunk, chunk) == p.row_last);
        if (p.owner_full) {
            for (int l = 0; l < kWave; ++l) {
                const int64_t i1 = c0 + kChunk + l;
                const bool ok1 = i1 < x.n;
                const uint32_t r1 = ok1 ? getR(x, i1, chunk) : 0xFFFFFFFFu;
                p.v1[l] = ok1 && in(x, "spill payload", i1, x.nk, chunk) ? x.V[i1] : 0u;
                extra += (ok1 && r1 == p.row_last) ? 1 : 0;
            }
        }
    }
    p.j0 = skip_first ? e0 : 0;
    p.jend = p.owner_full ? kChunk + extra : p.nv;
    return true;
}

bool seg_ends(const Plan &p, int k)
{
    if (k >= kChunk - 1 && p.owner_full)
        return k == p.jend - 1;
    if (k == p.nv - 1)
        return true;
    return (k + 1 < kChunk) && ((p.hm >> (k + 1)) & 1ull);
}

// The readlane of lane j (< 128) of the pair (v0: lanes 0..63, v1: 64..127).
uint32_t lane_val(Ctx &x, const uint32_t *v0, const uint32_t *v1, int j, int64_t chunk)
{
    if (j < 0 || j >= 2 * kWave) {
        bad(x, "readlane", j, 2 * kWave, chunk);
        return 0;
    }
    return j < kWave ? v0[j] : v1[j - kWave];
}

// The address checks of one dY row (by reference: the micro-step's own buffer).
void dy_row(Ctx &x, uint32_t code, int64_t chunk)
{
    const int64_t m = (int64_t)(code >> x.pos_bits);
    const int64_t pos = code & (uint32_t)((1ull << x.pos_bits) - 1u);
    if (in(x, "dY micro-step (readlane of the dY base lanes)", m, kWave, chunk) &&
        in(x, "dY micro-step attached", m, x.n_micro, chunk))
        in(x, "dY position", pos, x.Tm[m], chunk);
}

void walk_chunk(Ctx &x, int64_t chunk, bool tsplit)
{
    Plan p;
    if (!plan(x, chunk, p))
        return;
    const int64_t c0 = chunk * kChunk;
    uint32_t t0[kWave], t1[kWave];
    for (int l = 0; l < kWave; ++l) {
        t0[l] = t1[l] = kNotSingle;
        if (tsplit) {
            if (l < p.nv)
                t0[l] = rec_of(x, c0 + l, p.v0[l], chunk);
            if (p.owner_full && kChunk + l < p.jend)
                t1[l] = rec_of(x, c0 + kChunk + l, p.v1[l], chunk);
        }
    }
    uint64_t fin = (p.hm >> 1) | (1ull << (p.nv - 1));
    if (p.first_cont && p.j0 == 0) {
        const int e0 = p.hm ? ctz64(p.hm) : p.nv;
        fin &= ~(1ull << (e0 - 1));
    }
    if (p.last_spills)
        fin &= ~(1ull << 63);
    // nested runs: keys j0 .. kc_end continue a run from the walk before
    int kc_end = -1;
    if (tsplit && x.nested && p.j0 < p.jend) {
        uint32_t tj = 0;
        if (in(x, "readlane of the walk's first record", p.j0, kWave, chunk))
            tj = t0[p.j0];
        if (is_run(tj) && !(tj & kRunHead)) {
            uint64_t tails = 0;
            for (int l = 0; l < kWave; ++l)
                if (is_run(t0[l]) && (t0[l] & kRunTail))
                    tails |= 1ull << l;
            tails &= ~0ull << p.j0;
            kc_end = tails ? ctz64(tails) : p.nv - 1;
        }
    }
    int64_t piece_lo = -1;   // first key of the run piece being summed
    int ps = p.j0;
    for (int j = p.j0; j < p.jend; j += x.step_u) {
        for (int u = 0; u < x.step_u; ++u) {
            const int k = j + u;
            if (k >= p.jend)
                break;
            const uint32_t v = lane_val(x, p.v0, p.v1, k, chunk);
            dy_row(x, v & 0x7FFFFFFFu, chunk);
            const int64_t key = c0 + k;   // keys past the chunk are the next chunk's (owned spill-over)
            if (in(x, "walked key", key, x.n, chunk))
                x.walked[key] += 1;
            const bool ends_here = k < kChunk ? ((fin >> k) & 1ull) != 0 : (p.owner_full && k == p.jend - 1);
            if (k < kChunk && k != p.j0 && ((p.hm >> k) & 1ull))
                ps = k;
            if (tsplit) {
                const uint32_t tv = lane_val(x, t0, t1, k, chunk);
                if (tv != kNotSingle) {
                    const bool run = x.nested && (tv & kMultiKey);
                    const bool tlast = !run || (k > kc_end && (tv & kRunTail));
                    const int64_t key = c0 + k;
                    if (run && k != p.j0 && !(tv & kRunHead)) {
                        // adds the running sum: the key before must be of the same run
                        const uint32_t pv = lane_val(x, t0, t1, k - 1, chunk);
                        if (!is_run(pv) || ((pv ^ tv) & kTrowMask) != 0 || piece_lo < 0)
                            bad(x, "nested run continuing another record (key)", key, x.n, chunk);
                    } else {
                        piece_lo = key;
                    }
                    if (tlast) {
                        const uint32_t tr = tv & (x.nested ? kTrowMask : 0x7FFFFFFFu);
                        in(x, "trigram table row (completed in the bigram pass)", tr, x.rows_t, chunk);
                        if (run) {
                            // the run began in this walk: its first key carries kRunHead
                            const uint32_t hv = rec_of(x, piece_lo, x.V[piece_lo], chunk);
                            if (!(hv & kRunHead))
                                bad(x, "nested run completed without its first key (key)", key, x.n, chunk);
                        }
                        if (in(x, "trigram step count", v & 0x7FFFFFFFu, x.code_cap, chunk))
                            x.tstepped[v & 0x7FFFFFFFu] += 1;
                        for (int64_t i = piece_lo; i <= key; ++i)
                            if (in(x, "summed key", i, x.n, chunk))
                                x.tsum[x.V[i] & 0x7FFFFFFFu] += 1;
                        piece_lo = -1;
                    } else if (run && (k == kc_end || k == p.jend - 1)) {
                        const int slot = k <= kc_end ? 0 : 1;
                        if (slot == 0 && piece_lo != c0 + p.j0)
                            bad(x, "run piece of slot 0 not at the walk's start (key)", key, x.n, chunk);
                        if (in(x, "run piece", chunk, x.nchunk, chunk)) {
                            x.tpart_w[2 * chunk + slot] += 1;
                            x.tpart_lo[2 * chunk + slot] = piece_lo;
                            x.tpart_hi[2 * chunk + slot] = key;
                        }
                        if (slot == 1 && in(x, "run record", (int64_t)x.trec.size(), x.nchunk, chunk))
                            x.trec.push_back((uint64_t)chunk | ((uint64_t)tv << 32));
                        piece_lo = -1;
                    } else if (run) {
                        // the piece goes on: the next key walked is of the same run
                        const uint32_t nx = k + 1 < p.jend ? lane_val(x, t0, t1, k + 1, chunk) : kNotSingle;
                        if (!is_run(nx) || ((nx ^ tv) & kTrowMask) != 0 || (nx & kRunHead))
                            bad(x, "nested run piece left open (key)", key, x.n, chunk);
                    }
                }
            }
            if (ends_here) {
                const uint32_t row = k < kChunk ? lane_val(x, p.r0, p.r0, k, chunk) : p.row_last;
                in(x, "table row", row, x.rows_c, chunk);
                const uint32_t info = lane_val(x, p.i0, p.i0, ps, chunk);
                if (info != kNewHead)
                    in(x, "window slot", info, x.wrows, chunk);
                const int64_t head = c0 + ps;
                if (in(x, "segment head", head, x.n, chunk))
                    x.completed[head] += 1;
            } else if (seg_ends(p, k)) {
                // flush_partial
                if (ps == 0 && p.first_cont) {
                    if (in(x, "partial row", chunk, x.nchunk, chunk))
                        x.partial_w[2 * chunk] += 1;
                } else {
                    const uint32_t info = lane_val(x, p.i0, p.i0, ps, chunk);
                    if (in(x, "partial row", chunk, x.nchunk, chunk))
                        x.partial_w[2 * chunk + 1] += 1;
                    if (in(x, "fix-up record", (int64_t)x.owners.size(), x.nchunk, chunk))
                        x.owners.push_back((uint64_t)chunk | ((uint64_t)info << 32));
                }
            }
        }
    }
}

// group_sum_kernel: which groups of 64 chunks get a sum (partial rows 0 of
// all their chunks read).
void group_sums(Ctx &x, std::vector<int> &gw)
{
    const int64_t ng = (x.n > 0) ? ((x.n + kChunk - 1) / kChunk + kGroup - 1) / kGroup : 0;
    for (int64_t g = 0; g < ng; ++g) {
        const int64_t k0 = g * kGroup * kChunk, k1 = k0 + kGroup * kChunk;
        if (g == 0 || k1 >= x.n)
            continue;
        if (getR(x, k0 - 1, -1) != getR(x, k1, -1))
            continue;
        for (int64_t c = g * kGroup; c < (g + 1) * kGroup; ++c)
            if (in(x, "group member partial", c, x.nchunk, -1) && x.partial_w[2 * c] != 1)
                bad(x, "group sum of an unwritten partial row (chunk)", c, x.nchunk, -1);
        if (in(x, "group sum", g, x.ngroup, -1))
            gw[g] = 1;
    }
}

void fixup(Ctx &x, const std::vector<int> &gw)
{
    for (size_t k = 0; k < x.owners.size(); ++k) {
        const int64_t chunk = (int64_t)(uint32_t)x.owners[k];
        const uint32_t info = (uint32_t)(x.owners[k] >> 32);
        const uint32_t row = getR(x, chunk * kChunk + kChunk - 1, chunk);
        if (info != kNewHead)
            in(x, "fix-up window slot", info, x.wrows, chunk);
        in(x, "fix-up table row", row, x.rows_c, chunk);
        int64_t m = 0;
        for (int l = 0; l < kWave; ++l) {
            const int64_t cc = chunk + 1 + l;
            m += (cc * kChunk < x.n && getR(x, cc * kChunk, chunk) == row) ? 1 : 0;
        }
        if (m == kWave) {
            for (;;) {
                int cnt = 0;
                for (int t = 0; t < kFixThreads; ++t) {
                    const int64_t cc = chunk + 1 + m + t;
                    cnt += (cc * kChunk < x.n && getR(x, cc * kChunk, chunk) == row) ? 1 : 0;
                }
                m += cnt;
                if (cnt < kFixThreads)
                    break;
            }
        }
        const int64_t first = chunk + 1, last = chunk + m;
        const int64_t g_lo = (first + kGroup - 1) / kGroup, g_hi = last / kGroup;
        const int64_t ng = g_hi > g_lo ? g_hi - g_lo : 0;
        const int64_t n_before = ng ? g_lo * kGroup - first : m;
        const int64_t np = 1 + n_before + ng + (ng ? last - g_hi * kGroup + 1 : 0);
        // the owner's tail piece, then the items in order
        if (in(x, "fix-up tail piece", chunk, x.nchunk, chunk) && x.partial_w[2 * chunk + 1] != 1)
            bad(x, "fix-up of an unwritten tail piece (chunk)", chunk, x.nchunk, chunk);
        for (int64_t q = 1; q < np; ++q) {
            if (q <= n_before || q > n_before + ng) {
                const int64_t c = q <= n_before ? first + q - 1 : g_hi * kGroup + q - 1 - n_before - ng;
                if (in(x, "fix-up head piece", c, x.nchunk, chunk) && x.partial_w[2 * c] != 1)
                    bad(x, "fix-up of an unwritten head piece (chunk)", c, x.nchunk, chunk);
            } else {
                const int64_t g = g_lo + q - 1 - n_before;
                if (in(x, "fix-up group sum", g, x.ngroup, chunk) && gw[g] != 1)
                    bad(x, "fix-up of an unwritten group sum (group)", g, x.ngroup, chunk);
            }
        }
        // the segment's head: the last head of the owner chunk
        int64_t h = chunk * kChunk + kChunk - 1;
        while (h > chunk * kChunk && x.R[h - 1] == row)
            --h;
        x.completed[h] += 1;
    }
}

// The fix-up of nested trigram runs that crossed a walk's end: slot 1 of the
// record's chunk, then slot 0 of each following chunk whose first key
// continues the run (probed 64 chunks at a time, as the wavefront does).
void trun_fixup(Ctx &x, int64_t n0, const uint32_t *V0)
{
    for (size_t r = 0; r < x.trec.size(); ++r) {
        const int64_t c = (int64_t)(uint32_t)x.trec[r];
        const uint32_t tv = (uint32_t)(x.trec[r] >> 32);
        in(x, "run fix-up trigram row", tv & kTrowMask, x.rows_t, c);
        int64_t m = 0;
        for (;;) {
            int lead = kWave;
            for (int l = 0; l < kWave; ++l) {
                const int64_t cc = c + 1 + m + l;
                bool hit = false;
                if (cc * kChunk < n0) {
                    const uint32_t t = rec_of(x, cc * kChunk, V0[cc * kChunk], c);
                    hit = is_run(t) && !(t & kRunHead) && ((t ^ tv) & kTrowMask) == 0;
                }
                if (!hit) {
                    lead = l;
                    break;
                }
            }
            m += lead;
            if (lead < kWave)
                break;
        }
        if (!in(x, "run fix-up first piece", c, x.nchunk, c) || x.tpart_w[2 * c + 1] != 1) {
            bad(x, "run fix-up of an unwritten first piece (chunk)", c, x.nchunk, c);
            continue;
        }
        int64_t lo = x.tpart_lo[2 * c + 1], hi = x.tpart_hi[2 * c + 1];
        bool ok = (rec_of(x, lo, x.V[lo], c) & kRunHead) != 0;
        for (int64_t i = 1; i <= m; ++i) {
            const int64_t cc = c + i;
            if (!in(x, "run fix-up piece", cc, x.nchunk, c) || x.tpart_w[2 * cc] != 1) {
                bad(x, "run fix-up of an unwritten piece (chunk)", cc, x.nchunk, c);
                ok = false;
                break;
            }
            ok = ok && x.tpart_lo[2 * cc] == hi + 1;   // the pieces follow each other
            hi = x.tpart_hi[2 * cc];
        }
        if (!ok || !(rec_of(x, hi, x.V[hi], c) & kRunTail)) {
            bad(x, "run fix-up pieces not one whole run (chunk)", c, x.nchunk, c);
            continue;
        }
        x.tstepped[x.V[hi] & 0x7FFFFFFFu] += 1;
        for (int64_t i = lo; i <= hi; ++i)
            x.tsum[x.V[i] & 0x7FFFFFFFu] += 1;
    }
}

}  // namespace

extern "C" {

// Returns the number of violations; `msg` (256 bytes) gets the first.  Fills
// walked[n], completed[n] (at segment heads), tstepped[code_cap] and
// tsum[code_cap]; n_trec gets the number of nested run records.
int64_t model_channel(int64_t n, const uint32_t *R, const uint32_t *V, const uint32_t *I, int64_t nk,
                      const uint32_t *tinfo, int64_t code_cap, const uint32_t *tix, int pos_bits, int n_micro,
                      const int64_t *Tm,
                      int64_t rows_c, int64_t rows_t, int64_t wrows, int64_t nchunk, int64_t ngroup, int step_u,
                      int nested, int32_t *walked, int32_t *completed, int32_t *tstepped, int32_t *tsum,
                      int64_t *n_trec, int64_t *accesses, char *msg)
{
    Ctx x;
    x.nested = nested != 0;
    x.n = n; x.R = R; x.V = V; x.I = I; x.nk = nk; x.tinfo = tinfo; x.code_cap = code_cap; x.tix = tix;
    x.pos_bits = pos_bits; x.n_micro = n_micro; x.Tm = Tm; x.rows_c = rows_c; x.rows_t = rows_t;
    x.wrows = wrows; x.nchunk = nchunk; x.ngroup = ngroup; x.step_u = step_u;
    x.walked.assign(n, 0);
    x.completed.assign(n, 0);
    x.tstepped.assign(code_cap, 0);
    x.tsum.assign(code_cap, 0);
    x.partial_w.assign(2 * nchunk, 0);
    x.tpart_w.assign(2 * nchunk, 0);
    x.tpart_lo.assign(2 * nchunk, -1);
    x.tpart_hi.assign(2 * nchunk, -1);
    const int64_t chunks = (n + kChunk - 1) / kChunk;
    for (int64_t ch = 0; ch < chunks; ++ch)
        walk_chunk(x, ch, tinfo != nullptr);
    std::vector<int> gw(ngroup > 0 ? ngroup : 1, 0);
    group_sums(x, gw);
    fixup(x, gw);
    trun_fixup(x, n, V);
    for (int64_t i = 0; i < n; ++i) {
        walked[i] = x.walked[i];
        completed[i] = x.completed[i];
    }
    for (int64_t i = 0; i < code_cap; ++i) {
        tstepped[i] = x.tstepped[i];
        tsum[i] = x.tsum[i];
    }
    *accesses = x.accesses;
    *n_trec = (int64_t)x.trec.size();
    memcpy(msg, x.first, sizeof(x.first));
    return x.violations;
}

}  // extern "C"
