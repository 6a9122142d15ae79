// sd_topk.hip -- exact top-k of long rows, the top-k chain decision, and the
// DDTree best-first tree build.
//
// Page "大模型投机解码：Medusa、MTP、EAGLE、DFlash、DDTree 与 DSpark"
// (chzhyang.github.io): §1 (probability truncation must be folded into both p
// and q; accept test, first rejection, residual correction, extra token) and
// §5 DDTree (score Q(u) = prod q_i(u_i) of the displayed equation, prefixes
// chosen best-first with a heap under a node budget, numbered as chosen, each
// node seeing itself and its ancestors).
//
// k_topk_rows: one workgroup per row streams the row once. Each element whose
// key (value desc, id asc, NaN never kept) beats the workgroup's current k-th
// best key is appended to an LDS candidate buffer; when the buffer overflows it
// is sorted (bitonic, LDS) and cut back to k, which raises the threshold. The
// result is exact for any arrival order, because an element is dropped only
// when k kept elements already beat it.
//
// k_topk_short: rows of up to 32768 fp32 marginals (the tree's) are held in
// the registers of one workgroup, which bounds the top W from its threads'
// maxima and ranks the few tokens above the bound.
//
// k_tree_walk_topk_rows: the DDTree walk under a sampling target with top-k
// truncation, one workgroup per sequence taking the exact top-k of each row
// it visits (in registers when the row fits, else streamed as above).
#include "sd_device.hpp"
#include "sd_internal.hpp"

#include <math.h>

namespace sd {

namespace {


struct TopEntry {
    int32_t idx;
    float x;
};

// Order-preserving 32-bit image of a non-NaN float; -0 and +0 map together.
__device__ __forceinline__ uint32_t ordered_bits(float x) {
    if (x == 0.f) x = 0.f;
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}
// Larger key = better: higher value, then lower id.
__device__ __forceinline__ unsigned long long make_key(float x, int idx) {
    return ((unsigned long long)ordered_bits(x) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)idx);
}

__device__ __forceinline__ int pow2_at_least(int n) {
    int p = 2;
    while (p < n) p <<= 1;
    return p;
}

// Row task -> row pointer. Chain: task = ((b * slots) + s) * 2 + side, side 0 =
// target row s (s <= k_b), side 1 = draft row s (s < k_b). Tree: task = b*K + d.
template <class E>
__device__ const typename E::raw* topk_row(const typename E::raw* tgt, const typename E::raw* dft,
                                           const int32_t* cu, int K_max, int V, int task,
                                           bool chain) {
    if (!chain) return tgt + (int64_t)task * V;
    const int side = task & 1;
    const int rest = task >> 1;
    const int slots = K_max + 1;
    const int s = rest % slots;
    const int b = rest / slots;
    int d0, k;
    seq_range(cu, b, K_max, d0, k);
    if (side == 0) return (s <= k) ? tgt + ((int64_t)d0 + b + s) * V : nullptr;
    return (s < k) ? dft + ((int64_t)d0 + s) * V : nullptr;
}

constexpr int kTopkSample = 8;           // vectors per thread held in registers for the threshold
#ifndef SD_TOPK_U
#define SD_TOPK_U 4
#endif
constexpr int kTopkU = SD_TOPK_U;        // vectors per thread per main-pass step (as many more in flight)
constexpr int kWaveCap = 512;            // per-wave candidate buffer (64-bit keys)
constexpr int kTopkPhaseSplit = 2;       // slots streamed before the first decision
constexpr size_t kTopkPhaseMinElems = size_t(1) << 24;   // smaller windows: one phase
constexpr int kQueue = kTopkSample * kWave;   // per-wave queue of vector indices that may hold a candidate
static_assert(kQueue >= kWave * kTopkU, "one offer step must fit an empty queue");

// 16-byte vector `gvi` of a row as raw element bits; elements past the row
// (or past gvend) read as an all-ones NaN, which no test keeps.
template <class E, bool VEC>
__device__ __forceinline__ uint4 topk_raw(const typename E::raw* row, int V, int gvend, int gvi) {
    if (VEC) {
        if (gvi < gvend) return load16(row, gvi);
        return make_uint4(0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu);
    }
    constexpr int EV = E::kVec;
    uint32_t wd[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
    const int j0 = gvi * EV;
    if (gvi < gvend) {
        if (EV == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j0 + e < V) wd[e] = __float_as_uint(E::at(row, j0 + e));
        } else {
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const uint32_t h = (j0 + e < V) ? (__float_as_uint(E::at(row, j0 + e)) >> 16) : 0xffffu;
                wd[e / 2] = (e & 1) ? ((wd[e / 2] & 0xffffu) | (h << 16)) : ((wd[e / 2] & 0xffff0000u) | h);
            }
        }
    }
    return make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

// Element e of a raw vector as a float.
template <class E>
__device__ __forceinline__ float raw_elem(const uint4& v, int e) {
    if (E::kVec == 4) {
        const uint32_t w = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
        return __uint_as_float(w);
    }
    const int q = e >> 1;
    const uint32_t w = q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

typedef short short2_t __attribute__((ext_vector_type(2)));

// Whether some element of v may reach t > 0 (t16 / t32: the threshold's bits).
// For t > 0 a signed-integer compare of the raw bits orders the elements
// correctly: negatives (sign bit set) compare below, NaN compares high and is
// weeded out later by the float test. bf16 uses packed 16-bit maxima.
template <class E>
__device__ __forceinline__ bool vec_may_reach(const uint4& v, int32_t tbits) {
    if (E::kVec == 4) {
        const int32_t m = max(max((int32_t)v.x, (int32_t)v.y), max((int32_t)v.z, (int32_t)v.w));
        return m >= tbits;
    }
    const short2_t a = __builtin_bit_cast(short2_t, v.x), b = __builtin_bit_cast(short2_t, v.y);
    const short2_t c = __builtin_bit_cast(short2_t, v.z), d = __builtin_bit_cast(short2_t, v.w);
    const short2_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                                 __builtin_elementwise_max(c, d));
    return max((int32_t)m.x, (int32_t)m.y) >= tbits;
}

// Whether some element of v reaches t (any t; NaN never does).
template <class E>
__device__ __forceinline__ bool vec_reaches(const uint4& v, float t) {
    float f[E::kVec];
    E::unpack(v, f);
    bool r = false;
#pragma unroll
    for (int e = 0; e < E::kVec; ++e) r = r || (f[e] >= t);
    return r;
}

// A wave's running top-k: `cnt` keys in its LDS buffer, every kept key beats
// `thr` (whose value part is `tf`); `seen` counts every key ever appended.
// Uniform across the wave's lanes.
struct WaveTop {
    int cnt;
    int seen;
    unsigned long long thr;
    float tf;
};

// Sorts the wave's buffer, keeps its best topk and raises the threshold to
// the topk-th key (which topk real tokens reach). Out of line: it runs rarely.
__device__ __noinline__ WaveTop wave_compact(unsigned long long* wb, WaveTop st, int topk) {
    const int lane = threadIdx.x & (kWave - 1);
    const int n = st.cnt;
    const int np2 = pow2_at_least(n < 2 ? 2 : n);
    for (int i = n + lane; i < np2; i += kWave) wb[i] = 0ull;
    wave_sort_desc(wb, np2);
    if (n >= topk) {
        st.cnt = topk;
        st.thr = wb[topk - 1];
        st.tf = from_ordered((uint32_t)((st.thr + 1ull) >> 32));
    }
    return st;
}

// Per-wave state of the row pass: the running top-k, a queue of the 16-byte
// vector indices that may hold a candidate, and the threshold's raw bits for
// the integer pre-check.
struct Offer {
    WaveTop st;
    int qn;
    int32_t tbits;
    int32_t* qi;
    unsigned long long* wb;
};

template <class E>
__device__ __forceinline__ int32_t threshold_bits(float tf) {
    const uint32_t u = __float_as_uint(tf);
    return E::kVec == 4 ? (int32_t)u : (int32_t)(u >> 16);
}

// Processes the queue, one vector per lane per round: the vector is read
// again (queued vectors are a few per cent of the row) and each element whose
// key beats the threshold is appended, one element per lane per step, slots
// from a wave ballot. Before a step could overflow the buffer, and whenever it
// holds 2*topk keys, the buffer is compacted, which raises the threshold.
template <class E, bool VEC>
__device__ __forceinline__ void wave_drain(Offer& o, const typename E::raw* row, int V, int gvend,
                                           int topk) {
    constexpr int EV = E::kVec;
    const int lane = threadIdx.x & (kWave - 1);
    const int trigger = min(2 * topk, kWaveCap - kWave);
    wave_lds_sync();
    for (int base = 0; base < o.qn; base += kWave) {
        const bool live = base + lane < o.qn;
        const int vi = live ? o.qi[base + lane] : gvend;
        const uint4 v = topk_raw<E, VEC>(row, V, gvend, vi);
        uint32_t mask = 0u;
#pragma unroll
        for (int e = 0; e < EV; ++e) mask |= (raw_elem<E>(v, e) >= o.st.tf) ? (1u << e) : 0u;
        while (true) {
            const bool has = mask != 0u;
            if (__ballot(has) == 0ull) break;
            if (o.st.cnt >= trigger) o.st = wave_compact(o.wb, o.st, topk);
            unsigned long long key = 0ull;
            if (has) {
                const int e = __builtin_ctz(mask);
                mask &= mask - 1u;
                key = make_key(raw_elem<E>(v, e), vi * EV + e);
            }
            const bool take = has && key > o.st.thr;
            const unsigned long long bal = __ballot(take);
            if (take) {
                const int off = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                o.wb[o.st.cnt + off] = key;
            }
            o.st.cnt += __popcll(bal);
            o.st.seen += __popcll(bal);
        }
    }
    wave_lds_sync();                 // the queue is rewritten after this
    o.qn = 0;
    o.tbits = threshold_bits<E>(o.st.tf);
}

// Offers N raw vectors per lane (16-byte indices vi0 + u * kBlock): a
// pre-check against the wave's threshold, then ballots; the vectors that may
// hold a candidate are queued (their indices), after draining the queue if it
// could overflow. POS: the threshold is positive, so the integer pre-check on
// the raw bits applies.
template <class E, bool VEC, bool POS, int N, bool DRAIN = true>
__device__ __forceinline__ void offer_vecs(Offer& o, const uint4 (&v)[N], int vi0,
                                           const typename E::raw* row, int V, int gvend, int topk) {
    bool may[N];
    unsigned long long bal[N];
    int n = 0;
#pragma unroll
    for (int u = 0; u < N; ++u) {
        may[u] = POS ? vec_may_reach<E>(v[u], o.tbits) : vec_reaches<E>(v[u], o.st.tf);
        bal[u] = __ballot(may[u]);
        n += __popcll(bal[u]);
    }
    if (n == 0) return;
    if (DRAIN && o.qn + n > kQueue) wave_drain<E, VEC>(o, row, V, gvend, topk);
#pragma unroll
    for (int u = 0; u < N; ++u) {
        if (may[u]) {
            const int slot = o.qn + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[u] >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bal[u], 0u));
            o.qi[slot] = vi0 + u * kBlock;
        }
        o.qn += __popcll(bal[u]);
    }
}

// Streams vectors [v_start, gvend) of the row through offer_vecs, kTopkU
// vectors per thread per step with the next step's loads in flight. Whole
// steps load without bounds checks; one checked step takes the ragged end.
template <class E, bool VEC, bool POS>
__device__ __forceinline__ void offer_range(Offer& o, const typename E::raw* row, int V, int gvend,
                                            int v_start, int topk, const uint4 (&pre)[kTopkU],
                                            bool have_pre) {
    constexpr int kStep = kBlock * kTopkU;
    const int tid = threadIdx.x;
    const int nsteps = VEC ? (gvend - v_start) / kStep : 0;
    const int full_end = v_start + nsteps * kStep;
    pipelined_steps<kTopkU>(
        nsteps,
        [&](uint4 (&buf)[kTopkU], int st) {
            if (st == 0 && have_pre) {       // the first step, loaded by the caller
#pragma unroll
                for (int u = 0; u < kTopkU; ++u) buf[u] = pre[u];
                return;
            }
#pragma unroll
            for (int u = 0; u < kTopkU; ++u) buf[u] = load16(row, v_start + st * kStep + u * kBlock + tid);
        },
        [&](const uint4 (&buf)[kTopkU], int st) {
            offer_vecs<E, VEC, POS, kTopkU>(o, buf, v_start + st * kStep + tid, row, V, gvend, topk);
        });
    for (int v0 = full_end; v0 < gvend; v0 += kStep) {
        uint4 cur[kTopkU];
#pragma unroll
        for (int u = 0; u < kTopkU; ++u) cur[u] = topk_raw<E, VEC>(row, V, gvend, v0 + u * kBlock + tid);
        offer_vecs<E, VEC, POS, kTopkU>(o, cur, v0 + tid, row, V, gvend, topk);
    }
    if (o.qn > 0) wave_drain<E, VEC>(o, row, V, gvend, topk);
}

// One pass over the row from threshold t: with SAMPLE, the held sample first
// and then vectors from the end of the sample on (the first whole step of
// them already loaded into pre when have_pre); else the whole row. Leaves
// each wave's best min(cnt, topk) keys sorted at the front of its buffer.
template <class E, bool VEC, bool POS, bool SAMPLE>
__device__ __forceinline__ WaveTop row_pass(const typename E::raw* row, int V, int gvend, float t,
                                            const uint4 (&hs)[kTopkSample], int32_t* qi,
                                            unsigned long long* wb, int topk,
                                            const uint4 (&pre)[kTopkU], bool have_pre) {
    Offer o;
    o.st.cnt = 0;
    o.st.seen = 0;
    o.st.thr = t == -INFINITY ? 0ull : ((unsigned long long)ordered_bits(t) << 32) - 1ull;
    o.st.tf = t;
    o.qn = 0;
    o.tbits = threshold_bits<E>(t);
    o.qi = qi;
    o.wb = wb;
    int v_start = 0;
    if (SAMPLE) {
        // the whole sample fits the empty queue: no drain while it is held
        offer_vecs<E, VEC, POS, kTopkSample, false>(o, hs, threadIdx.x, row, V, gvend, topk);
        v_start = kTopkSample * kBlock;
    }
    offer_range<E, VEC, POS>(o, row, V, gvend, v_start, topk, pre, SAMPLE && have_pre);
    return wave_compact(wb, o.st, topk);
}

// Softmax statistics of a kept list and p(y) of one token (fp64).
struct RowTop {
    int32_t count;      // kept entries
    int32_t valid;      // finite maximum and a finite positive sum
    double m;           // max of x / T over the kept set
    double S;           // sum of exp(x / T - m)
    double py;          // p(y) of the position's draft token (0 if not kept)
};

// Rank (from 0) of the sample maximum taken as the first threshold guess:
// about twice the number of the row's top-k expected among the sampled
// tokens, plus 4; the topk-th maximum (always a valid bound) when the sample
// covers the row.
__device__ __forceinline__ int guess_rank(int topk, int sampled, int V) {
    if (sampled >= V) return topk - 1;
    const int j = (int)ceilf(2.0f * (float)topk * (float)sampled / (float)V) + 4;
    return min(j, topk) - 1;
}

// LDS of one workgroup's exact top-k of one row.
struct TopkSmem {
    unsigned long long wbuf[kWavesPerBlock][kWaveCap];
    int32_t qi[kWavesPerBlock][kQueue];
    uint32_t smax[kWavesPerBlock][kWave];
    int wcnt[kWavesPerBlock];
    int wseen[kWavesPerBlock];
    double red[kWavesPerBlock];
};

// The j-th largest (j >= 1) of the 256 order-preserving keys smax[4][64]
// (0 = none; 0 if fewer than j are nonzero), the same in every wave: each lane
// holds four keys and the value is built from the top bit down, one ballot
// count per candidate. The maxima of bf16 rows are bf16 values, whose keys
// end in 16 zero bits (value >= +0) or 16 one bits (below it), so their top
// 16 bits decide and the rest follows from the sign.
template <class E>
__device__ __forceinline__ uint32_t rank_value(const uint32_t (&smax)[kWavesPerBlock][kWave], int lane,
                                               int j) {
    constexpr int kLowBit = E::kVec == 8 ? 16 : 0;
    uint32_t km[kWavesPerBlock];
#pragma unroll
    for (int o = 0; o < kWavesPerBlock; ++o) km[o] = smax[o][lane];
    uint32_t g = 0u;
#pragma unroll 4
    for (int bit = 31; bit >= kLowBit; --bit) {
        const uint32_t c = g | (1u << bit);
        int n = 0;
#pragma unroll
        for (int o = 0; o < kWavesPerBlock; ++o) n += __popcll(__ballot(km[o] >= c));
        if (n >= j) g = c;
    }
    if (kLowBit != 0 && g != 0u && !(g & 0x80000000u)) g |= (1u << kLowBit) - 1u;
    return g;
}

// What row_topk leaves besides the list: the kept count and, with stats, the
// fp64 softmax statistics over the kept set at temperature T (m = max x/T,
// S = sum exp(x/T - m), ey = the term of token y, 0 if y is not kept).
struct KeptStats {
    int kept;
    double m;
    double S;
    double ey;
};

// The exact top-k of one row by one workgroup, in key order (value desc, then
// lower id first), written as TopEntry to L[0 .. kept) (global memory or LDS);
// uniform results in every thread.
//  1. Every thread holds kTopkSample vectors of the row's start and takes
//     their maximum. Ranked among the 256 maxima (distinct tokens), the
//     topk-th is a guaranteed bound (at least topk tokens reach it) and a
//     higher one is a guess; both come from ballot bisections over all 256
//     maxima in every wave.
//  2. With the guess as threshold, each wave streams its share of the row.
//     A vector whose largest element may reach the threshold is queued; full
//     queues are processed one vector per lane, appending each element that
//     beats the wave's running k-th key to its LDS buffer, which is compacted
//     (sorted, cut to topk) as it fills, raising the threshold.
//  3. If fewer than topk tokens reached the guess, it was too high: the row is
//     streamed again from the guaranteed bound (rare; the result is exact
//     either way, since a token is dropped only when topk tokens beat it).
//  4. The waves' sorted lists are merged by rank (binary search in the other
//     lists) and the first topk written.
template <class E, bool VEC>
__device__ __forceinline__ KeptStats row_topk(const typename E::raw* __restrict__ row, int V, int topk,
                                              double T, int y, bool stats, TopEntry* L, TopkSmem& sm) {
    constexpr int EV = E::kVec;
    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int gvend = (V + EV - 1) / EV;
    // 1. thresholds from the held sample
    uint4 hs[kTopkSample];
    if (VEC && kTopkSample * kBlock <= gvend) {      // the usual case: no bounds checks
#pragma unroll
        for (int i = 0; i < kTopkSample; ++i) hs[i] = load16(row, i * kBlock + tid);
    } else {
#pragma unroll
        for (int i = 0; i < kTopkSample; ++i) hs[i] = topk_raw<E, VEC>(row, V, gvend, i * kBlock + tid);
    }
    // the streaming pass's first whole step, issued now so that its loads
    // overlap the ranking of the thresholds below (bf16 rows: measured
    // faster despite the extra spill; fp32 keeps its registers)
    constexpr int kStep = kBlock * kTopkU;
    const bool have_pre = VEC && EV == 8 && gvend - kTopkSample * kBlock >= kStep;
    uint4 pre[kTopkU];
    if (have_pre) {
#pragma unroll
        for (int u = 0; u < kTopkU; ++u) pre[u] = load16(row, kTopkSample * kBlock + u * kBlock + tid);
    } else {
#pragma unroll
        for (int u = 0; u < kTopkU; ++u) pre[u] = make_uint4(0u, 0u, 0u, 0u);
    }
    float m = NAN;                   // fmaxf skips NaN; stays NaN only if all are
#pragma unroll
    for (int i = 0; i < kTopkSample; ++i) {
        float f[EV];
        E::unpack(hs[i], f);
#pragma unroll
        for (int e = 0; e < EV; ++e) m = fmaxf(m, f[e]);
    }
    // Opaque to the optimiser: the unpacked sample is not kept alive (in
    // registers) until the sample is offered.
#pragma unroll
    for (int i = 0; i < kTopkSample; ++i)
        asm volatile("" : "+v"(hs[i].x), "+v"(hs[i].y), "+v"(hs[i].z), "+v"(hs[i].w));
    const bool any = m == m;
    // The value at rank jg (the guess) among the 256 maxima (value desc; NaN
    // not ranked), and on a retry the one at rank topk - 1 (reached by topk
    // sampled tokens: a guaranteed bound): after one exchange through LDS
    // every wave holds all 256 maxima as order-preserving bits (0 = none),
    // four per lane, and builds the value bit by bit from the top with
    // ballots -- the largest r that at least j maxima reach is the j-th
    // largest. Every wave computes the same value, so no second barrier is
    // needed.
    const int jg = guess_rank(topk, min(V, kTopkSample * kBlock * EV), V);
    const uint32_t mb = any ? ordered_bits(m) : 0u;
    sm.smax[w][lane] = mb;
    __syncthreads();
    const uint32_t gb = rank_value<E>(sm.smax, lane, jg + 1);
    // 2. the pass from the guess
    const float tg = gb == 0u ? -INFINITY : from_ordered(gb);
    WaveTop st = tg > 0.f ? row_pass<E, VEC, true, true>(row, V, gvend, tg, hs, sm.qi[w], sm.wbuf[w], topk,
                                                         pre, have_pre)
                          : row_pass<E, VEC, false, true>(row, V, gvend, tg, hs, sm.qi[w], sm.wbuf[w], topk,
                                                          pre, have_pre);
    if (lane == 0) {
        sm.wcnt[w] = st.cnt;
        sm.wseen[w] = st.seen;
    }
    __syncthreads();
    int seen = 0;
    for (int i = 0; i < kWavesPerBlock; ++i) seen += sm.wseen[i];
    // 3. exact unless fewer than topk tokens reached a guess above the bound
    if (seen < topk && tg != -INFINITY && jg + 1 < topk) {
        const uint32_t sb = rank_value<E>(sm.smax, lane, topk);    // the same in every wave
        const float ts = sb == 0u ? -INFINITY : from_ordered(sb);
        if (tg != ts) {
            __syncthreads();
            st = ts > 0.f ? row_pass<E, VEC, true, false>(row, V, gvend, ts, hs, sm.qi[w], sm.wbuf[w], topk,
                                                          pre, false)
                          : row_pass<E, VEC, false, false>(row, V, gvend, ts, hs, sm.qi[w], sm.wbuf[w], topk,
                                                           pre, false);
            if (lane == 0) sm.wcnt[w] = st.cnt;
            __syncthreads();
        }
    }
    // 4. merge the waves' lists by rank
    int total = 0;
    float xmax = -INFINITY;
    bool have = false;
    for (int i = 0; i < kWavesPerBlock; ++i) {
        const int c = sm.wcnt[i];
        total += c;
        if (c > 0) {
            const float x0 = from_ordered((uint32_t)(sm.wbuf[i][0] >> 32));
            xmax = have ? fmaxf(xmax, x0) : x0;
            have = true;
        }
    }
    KeptStats ks;
    ks.kept = total < topk ? total : topk;
    ks.m = have ? (double)xmax / T : 0.0;
    double sum = 0.0, ey = 0.0;
    const int own = sm.wcnt[w];
    for (int i = lane; i < own; i += kWave) {
        const unsigned long long key = sm.wbuf[w][i];
        int rank = i;
#pragma unroll
        for (int o2 = 0; o2 < kWavesPerBlock; ++o2)
            if (o2 != w) rank += count_above(sm.wbuf[o2], sm.wcnt[o2], key);
        if (rank < topk) {
            TopEntry te;
            te.idx = (int32_t)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
            te.x = from_ordered((uint32_t)(key >> 32));
            L[rank] = te;
            if (stats) {
                const double e = exp((double)te.x / T - ks.m);
                sum += e;
                if (te.idx == y) ey = e;
            }
        }
    }
    if (stats) {
        sum = block_sum(sum, sm.red);
        ey = block_sum(ey, sm.red);  // at most one thread holds y
    }
    ks.S = sum;
    ks.ey = ey;
    return ks;
}

// One workgroup per row task: row_topk's list written to the task's slot;
// for the rows of a chain also the row's softmax statistics over the kept set
// and p(y) of the position's draft token (fp64).
template <class E, bool VEC>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_topk_rows(const typename E::raw* __restrict__ tgt,
                                                      const typename E::raw* __restrict__ dft,
                                                      const int32_t* __restrict__ cu, int K_max,
                                                      int V, int topk, int chain,
                                                      const int32_t* __restrict__ tok, float temperature,
                                                      TopEntry* __restrict__ lists,
                                                      int32_t* __restrict__ counts,
                                                      RowTop* __restrict__ rowtop, int slot_lo,
                                                      int slot_span,
                                                      const int32_t* __restrict__ live,
                                                      int32_t* __restrict__ live_n) {
    __shared__ TopkSmem sm;
    // chain: block -> (sequence, slot in [slot_lo, slot_lo + slot_span), side);
    // the row's task number keeps the layout of the whole window. Group g's
    // 2 * slot_span rows take its blocks rotated by g: consecutive blocks go
    // to the XCDs in turn, so each kind of row (the bonus row's empty draft
    // side, a late slot) is spread over all of them instead of always landing
    // on the same XCD. In the second phase group g is the g-th sequence still
    // undecided (count and entry loaded together), so that the live
    // workgroups are the first ones dispatched and spread evenly over the CUs.
    int task = blockIdx.x;
    if (chain) {
        const int n = 2 * slot_span;
        const int g = (int)blockIdx.x / n;
        int b = g;
        if (live != nullptr) {
            const int cnt = *live_n, e = live[g];
            if (g >= cnt) return;
            b = e;
        } else if (live_n != nullptr && blockIdx.x == 0 && threadIdx.x == 0) {
            *live_n = 0;             // the first phase: the second phase's list starts empty
        }
        const int j = ((int)blockIdx.x - g * n + n - g % n) % n;
        task = ((b * (K_max + 1) + slot_lo + (j >> 1)) << 1) | (j & 1);
    }
    const typename E::raw* row = topk_row<E>(tgt, dft, cu, K_max, V, task, chain != 0);
    if (row == nullptr) return;
    const int tid = threadIdx.x;
    const bool stats = rowtop != nullptr;
    int y = -1;
    if (stats && chain) {            // task = ((b * (K_max + 1) + s) * 2 + side)
        const int rest = task >> 1;
        const int s = rest % (K_max + 1);
        int d0, k;
        seq_range(cu, rest / (K_max + 1), K_max, d0, k);
        if (s < k) y = tok[d0 + s];
    }
    TopEntry* L = lists + (int64_t)task * topk;
    const KeptStats ks = row_topk<E, VEC>(row, V, topk, (double)temperature, y, stats, L, sm);
    for (int i = ks.kept + tid; i < topk; i += kBlock) {
        TopEntry te;
        te.idx = -1;
        te.x = -INFINITY;
        L[i] = te;
    }
    if (tid == 0) counts[task] = ks.kept;
    if (stats && tid == 0) {
        RowTop r;
        r.count = ks.kept;
        r.m = ks.m;
        r.S = ks.S;
        r.valid = (ks.kept > 0 && isfinite(ks.m) && isfinite(ks.S) && ks.S > 0.0) ? 1 : 0;
        r.py = (r.valid && y >= 0 && y < V) ? ks.ey / ks.S : 0.0;
        rowtop[task] = r;
    }
}

// ---------------------------------------------------------------------------
// Chain decision over top-k lists (fp64 throughout; the lists are tiny).
// ---------------------------------------------------------------------------
// Inverse CDF in token-id order over the kept entries of target list P (at
// most kMaxTopk): weight p_j - q_j clamped at 0 (q_j from list D when it keeps
// j) when `residual`, otherwise p_j. One wave; its LDS scratch is wbuf/ibuf.
__device__ int list_inverse_cdf(const TopEntry* P, const RowTop& sp, const TopEntry* D,
                                const RowTop& sq, bool residual, double T, double u, double* wbuf,
                                int* ibuf, TopEntry* pl, TopEntry* dl, double* R_out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int np = sp.count;
    const int nd = (residual && sq.valid) ? sq.count : 0;
    // copies padded to a multiple of 8 with ids no search matches (pl: above
    // every id, dl: -1), so the searches below read 8 entries per wait
    const int np8 = (np + 7) & ~7, nd8 = (nd + 7) & ~7;
    for (int i = lane; i < np8; i += kWave) {
        TopEntry e = {0x7fffffff, 0.f};
        if (i < np) e = P[i];
        pl[i] = e;
    }
    for (int i = lane; i < nd8; i += kWave) {
        TopEntry e = {-1, 0.f};
        if (i < nd) e = D[i];
        dl[i] = e;
    }
    wave_lds_sync();
    for (int i = lane; i < np; i += kWave) {
        const int id = pl[i].idx;
        double wgt = exp((double)pl[i].x / T - sp.m) / sp.S;
        if (residual) {
            // q_j from the draft list (ids are distinct within a list); the
            // search first, then one exp, so the wave never runs an exp per
            // list entry
            int jm = -1;
            for (int j = 0; j < nd8; j += 8) {
                int d8[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) d8[q] = dl[j + q].idx;
#pragma unroll
                for (int q = 0; q < 8; ++q) jm = (d8[q] == id) ? j + q : jm;
            }
            const double q = jm >= 0 ? exp((double)dl[jm].x / T - sq.m) / sq.S : 0.0;
            wgt = wgt - q;
            if (!(wgt > 0.0)) wgt = 0.0;
        }
        int rank = 0;
        for (int j = 0; j < np8; j += 8) {
            int p8[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) p8[q] = pl[j + q].idx;
#pragma unroll
            for (int q = 0; q < 8; ++q) rank += (p8[q] < id) ? 1 : 0;
        }
        wbuf[rank] = wgt;
        ibuf[rank] = id;
    }
    wave_lds_sync();
    // inverse CDF over the id-sorted weights: lane l holds entries 4l .. 4l+3
    // (np <= 256); lane sums, a wave prefix sum, then the first entry whose
    // running mass exceeds u * R (else the last entry with positive mass)
    double w4[4];
    double ls = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 4 * lane + e;
        w4[e] = i < np ? wbuf[i] : 0.0;
        ls += w4[e];
    }
    const double before = wave_excl_scan(ls);
    const double R = __shfl(before + ls, kWave - 1, kWave);
    const double target = u * R;
    int hit = -1, last = -1;
    double C = before;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        C += w4[e];
        if (w4[e] > 0.0) {
            last = 4 * lane + e;
            if (hit < 0 && C > target) hit = 4 * lane + e;
        }
    }
    const unsigned long long hb = __ballot(hit >= 0);
    int at;
    if (hb) {
        at = __shfl(hit, __ffsll(hb) - 1, kWave);
    } else {
        at = last;
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) at = max(at, __shfl_xor(at, o, kWave));
    }
    const int pick = at >= 0 ? ibuf[at] : -1;
    wave_lds_sync();
    *R_out = R;
    return pick;
}

// One wave per sequence: accept bits from the rows' p(y) and q(y) (computed by
// the row pass), A (ballot), and the final token from the decision row's lists.
__device__ __forceinline__ RowTop shfl_rowtop(const RowTop& r, int src) {
    RowTop o;
    o.count = __shfl(r.count, src, kWave);
    o.valid = __shfl(r.valid, src, kWave);
    o.m = __shfl(r.m, src, kWave);
    o.S = __shfl(r.S, src, kWave);
    o.py = __shfl(r.py, src, kWave);
    return o;
}

#ifndef SD_TOPK_DECIDE_SEQS
#define SD_TOPK_DECIDE_SEQS 1
#endif
constexpr int kDecideSeqs = SD_TOPK_DECIDE_SEQS;     // sequences (waves) per workgroup

__global__ __launch_bounds__(kDecideSeqs * kWave) void k_chain_topk_decide(
    const TopEntry* __restrict__ lists, const RowTop* __restrict__ rowtop,
    const int32_t* __restrict__ tok, const float* __restrict__ uni, const int32_t* __restrict__ cu,
    int B, int K_max, int V, int topk, float temperature, int32_t* __restrict__ A_out,
    int32_t* __restrict__ next_out, float* __restrict__ probs_out, float* __restrict__ R_out,
    int32_t* __restrict__ status_out, const int32_t* __restrict__ cap,
    int32_t* __restrict__ A_full_out, int hi, int32_t* __restrict__ state, int phase,
    int32_t* __restrict__ live, int32_t* __restrict__ live_n) {
    __shared__ double wbuf_all[kDecideSeqs][kMaxTopk];
    __shared__ int ibuf_all[kDecideSeqs][kMaxTopk];
    __shared__ TopEntry pl_all[kDecideSeqs][kMaxTopk];
    __shared__ TopEntry dl_all[kDecideSeqs][kMaxTopk];
    const int w = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int b = blockIdx.x * kDecideSeqs + w;
    if (b >= B) return;
    if (phase > 0 && state[b] != phase) return;        // decided in an earlier phase
    const int slots = K_max + 1;
    const double T = (double)temperature;
    auto task_of = [&](int s, int side) { return (((int64_t)b * slots + s) * 2 + side); };
    // lane s reads the statistics of slot s's rows (every slot streamed so
    // far); these loads do not wait for cu
    const int ns = slots < hi ? slots : hi;
    RowTop rp{0, 0, 0.0, 0.0, 0.0}, rq{0, 0, 0.0, 0.0, 0.0};
    if (lane < ns) {
        rp = rowtop[task_of(lane, 0)];
        if (lane < K_max) rq = rowtop[task_of(lane, 1)];
    }
    int d0, k;
    seq_range(cu, b, K_max, d0, k);
    const int kk = k < hi ? k : hi;                     // positions whose rows are ready
    bool acc = true;
    int st = 0;
    if (lane < kk) {
        const int y = tok[d0 + lane];
        const bool yok = (y >= 0 && y < V);
        const double py = yok ? rp.py : 0.0, qy = yok ? rq.py : 0.0;
        const double u = (double)uni[d0 + b + lane];
        acc = rp.valid && rq.valid && yok && py > 0.0 && u * qy <= py;
        st = (yok ? 0 : 1) | ((rp.valid && rq.valid) ? 0 : 2);
        if (probs_out) {
            probs_out[2 * (int64_t)(d0 + lane)] = (float)py;
            probs_out[2 * (int64_t)(d0 + lane) + 1] = (float)qy;
        }
    }
    const unsigned long long rej = __ballot(!acc);
    // state[b]: p + 1 while undecided after phase p, -(p + 1) once decided in it
    if (rej == 0ull && k >= hi) {                       // every position so far passed: next phase
        if (lane == 0) {
            state[b] = phase + 1;
            live[atomicAdd(live_n, 1)] = b;                 // streamed in the next phase (any order)
        }
        return;
    }
    if (state != nullptr && lane == 0) state[b] = -(phase + 1);
    const int A_full = rej ? (__ffsll(rej) - 1) : k;
    const int kc = committed_len(cap, b, k);
    const int A = A_full < kc ? A_full : kc;
    int status = (lane < kc && lane <= A) ? st : 0;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) status |= __shfl_xor(status, o, kWave);
    const double uf = (double)uni[d0 + b + kc];
    int next = -1;
    double R = 0.0;
    double* wbuf = wbuf_all[w];
    int* ibuf = ibuf_all[w];
    TopEntry* pl = pl_all[w];
    TopEntry* dl = dl_all[w];
    if (A < kc) {
        const RowTop sp = shfl_rowtop(rp, A);
        const RowTop sq = shfl_rowtop(rq, A);
        if (sp.valid) {
            next = list_inverse_cdf(lists + task_of(A, 0) * topk, sp, lists + task_of(A, 1) * topk, sq,
                                    true, T, uf, wbuf, ibuf, pl, dl, &R);
            if (!(R > 0.0)) {
                double unused;
                next = list_inverse_cdf(lists + task_of(A, 0) * topk, sp, nullptr, sq, false, T, uf,
                                        wbuf, ibuf, pl, dl, &unused);
            }
        }
    } else {
        // the extra-token row: slot kc (past the lanes only in a 64-position window)
        const RowTop sp = kc < kWave ? shfl_rowtop(rp, kc) : rowtop[task_of(kc, 0)];
        if (sp.valid) {
            double unused;
            next = list_inverse_cdf(lists + task_of(kc, 0) * topk, sp, nullptr, sp, false, T, uf, wbuf,
                                    ibuf, pl, dl, &unused);
        } else {
            status |= 2;
        }
        R = 0.0;
    }
    if (lane == 0) {
        A_out[b] = A;
        if (A_full_out) A_full_out[b] = A_full;
        next_out[b] = next;
        if (R_out) R_out[b] = (float)R;
        if (status_out) status_out[b] = status;
    }
}

// ---------------------------------------------------------------------------
// DDTree walk under a sampling target with top-k truncation [SD §5 DDTree,
// SD §1]: one workgroup per sequence, reading only the rows on its walk. At
// each node the workgroup takes the exact top-k of the node's row (the list
// in LDS); wave 0 forms the softmax over the kept set, draws the target's
// token from it (token-id order, the node's uniform) and moves to the child
// that carries it. Wave 0 holds the node table, one node per lane.
//
// A row of at most kTileVecs 16-byte vectors is held in registers and its
// top-k taken there (tile_topk); longer rows, and the rare tile whose bound
// admits too many candidates, are streamed by row_topk.
// ---------------------------------------------------------------------------
constexpr int kTileVecs = 16;                   // 16-byte vectors per thread
constexpr int kTileSeg = 128;                   // candidates per wave (LDS segment)
static_assert(kTileVecs <= 32 && kTileSeg % 8 == 0, "vector mask bits; 8-key reads");

// Vector k of v for a lane-varying k (a select chain, no indexed registers).
__device__ __forceinline__ uint4 pick_vec(const uint4 (&v)[kTileVecs], int k) {
    uint4 x = v[0];
#pragma unroll
    for (int i = 1; i < kTileVecs; ++i) {
        const bool t = k == i;
        x.x = t ? v[i].x : x.x;
        x.y = t ? v[i].y : x.y;
        x.z = t ? v[i].z : x.z;
        x.w = t ? v[i].w : x.w;
    }
    return x;
}

// Exact top-k of a row held as v[i] = vector i * kBlock + tid: every token
// below the bound is beaten by topk others, so the tokens at or above it
// contain the top-k. Each wave gathers its candidates into its LDS segment,
// working through the vectors that may hold one (lowest first, one per lane
// per round) and their passing elements (one per lane per step, slots from a
// ballot); the candidates are then ranked by counting (keys are distinct).
// Writes lst[0 .. kept) in key order and returns kept, or returns -1 having
// written nothing when a wave finds more than kTileSeg candidates.
template <class E>
__device__ __forceinline__ int tile_topk(const uint4 (&v)[kTileVecs], int topk, TopEntry* lst,
                                         unsigned long long* cbuf, int* s_rank, uint32_t* s_bound,
                                         int* s_wcnt) {
    constexpr int EV = E::kVec;
    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = tid & (kWave - 1);
    // 1. each vector's and each thread's maximum (NaN skipped; a thread with
    //    none holds key 0)
    float vmax[kTileVecs];
    float m = NAN;
#pragma unroll
    for (int i = 0; i < kTileVecs; ++i) {
        vmax[i] = NAN;
#pragma unroll
        for (int e = 0; e < EV; ++e) vmax[i] = fmaxf(vmax[i], raw_elem<E>(v[i], e));
        m = fmaxf(m, vmax[i]);
    }
    const uint32_t mk = m == m ? ordered_bits(m) : 0u;
    // 2. in each wave the j-th largest maximum (j = ceil(topk / waves)) is
    //    reached by j of its tokens; the smallest over the waves by topk
    //    tokens. 0 (a wave with fewer than j values) admits every token. A
    //    bf16 key's value lives in its top 16 bits: the bound keeps those and
    //    admits exactly the tokens of that bf16 value and above.
    constexpr int kLo = EV == 8 ? 16 : 0;
    const uint32_t tw = wave_jth_largest<kLo>(mk, (topk + kWavesPerBlock - 1) / kWavesPerBlock);
    if (lane == 0) s_bound[w] = tw;
    __syncthreads();
    uint32_t tb = s_bound[0];
#pragma unroll
    for (int o = 1; o < kWavesPerBlock; ++o) tb = min(tb, s_bound[o]);
    // (a bound kept to 16 bits below -inf's key decodes to a NaN: every value
    // reaches -inf, so -inf is the bound then)
    float tf = tb == 0u ? -INFINITY : from_ordered(tb);
    if (tf != tf) tf = -INFINITY;
    // 3. the candidates x >= tf (NaN never), in the vectors whose maximum
    //    reaches the bound
    uint32_t vm = 0u;
#pragma unroll
    for (int i = 0; i < kTileVecs; ++i) vm |= vmax[i] >= tf ? (1u << i) : 0u;
    unsigned long long* seg = cbuf + w * kTileSeg;
    int cnt = 0;                     // wave-uniform
    while (__ballot(vm != 0u)) {
        const int i = vm != 0u ? __builtin_ctz(vm) : 0;
        const uint4 x = pick_vec(v, i);
        uint32_t em = 0u;
        if (vm != 0u) {
#pragma unroll
            for (int e = 0; e < EV; ++e) em |= raw_elem<E>(x, e) >= tf ? (1u << e) : 0u;
        }
        vm &= vm - 1u;
        while (true) {
            const bool has = em != 0u;
            const unsigned long long bal = __ballot(has);
            if (bal == 0ull) break;
            if (has) {
                const int e = __builtin_ctz(em);
                em &= em - 1u;
                const int slot = cnt + (int)__builtin_amdgcn_mbcnt_hi(
                                           (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                if (slot < kTileSeg) seg[slot] = make_key(raw_elem<E>(x, e), (i * kBlock + tid) * EV + e);
            }
            cnt += __popcll(bal);
        }
    }
    // pad the segment to a multiple of 8 with keys that beat nothing
    if (cnt <= kTileSeg)
        for (int a = cnt + lane; a < ((cnt + 7) & ~7); a += kWave) seg[a] = 0ull;
    if (lane == 0) s_wcnt[w] = cnt;
    for (int a = tid; a < kWavesPerBlock * kTileSeg; a += kBlock) s_rank[a] = 0;
    __syncthreads();
    static_assert(kWavesPerBlock == 4, "four wave segments");
    const int wc0 = s_wcnt[0], wc1 = s_wcnt[1], wc2 = s_wcnt[2], wc3 = s_wcnt[3];
    const int C = wc0 + wc1 + wc2 + wc3;
    if (wc0 > kTileSeg || wc1 > kTileSeg || wc2 > kTileSeg || wc3 > kTileSeg) return -1;
    // 4. rank by counting: one (candidate, segment) pair per thread and
    //    round, 8 keys per read, the partial counts summed in LDS
    for (int p = tid; p < kWavesPerBlock * C; p += kBlock) {
        const int c = p / kWavesPerBlock;
        const int o = p % kWavesPerBlock;
        // candidate c -> slot a of its segment
        const int a = c < wc0                   ? c
                      : c < wc0 + wc1             ? kTileSeg + (c - wc0)
                      : c < wc0 + wc1 + wc2       ? 2 * kTileSeg + (c - wc0 - wc1)
                                                  : 3 * kTileSeg + (c - wc0 - wc1 - wc2);
        const unsigned long long key = cbuf[a];
        const unsigned long long* so = cbuf + o * kTileSeg;
        const int n8 = ((o == 0 ? wc0 : o == 1 ? wc1 : o == 2 ? wc2 : wc3) + 7) & ~7;
        int part = 0;
        for (int j = 0; j < n8; j += 8) {
            unsigned long long k8[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) k8[q] = so[j + q];
#pragma unroll
            for (int q = 0; q < 8; ++q) part += k8[q] > key ? 1 : 0;
        }
        if (part > 0) atomicAdd(&s_rank[a], part);
    }
    __syncthreads();
    for (int a = tid; a < kWavesPerBlock * kTileSeg; a += kBlock) {
        const int rank = s_rank[a];
        const int sa = a / kTileSeg;
        if (a % kTileSeg < (sa == 0 ? wc0 : sa == 1 ? wc1 : sa == 2 ? wc2 : wc3) && rank < topk) {
            const unsigned long long key = cbuf[a];
            TopEntry te;
            te.idx = (int32_t)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
            te.x = from_ordered((uint32_t)(key >> 32));
            lst[rank] = te;
        }
    }
    __syncthreads();
    return C < topk ? C : topk;
}

// row_topk's list without statistics, out of line: the walk's tile path keeps
// its registers to itself.
template <class E, bool VEC>
__device__ __noinline__ int row_topk_list(const typename E::raw* row, int V, int topk, TopEntry* lst,
                                          TopkSmem* sm) {
    const int kept = row_topk<E, VEC>(row, V, topk, 1.0, -1, false, lst, *sm).kept;
    __syncthreads();
    return kept;
}

template <class E, bool VEC>
__global__ __launch_bounds__(kBlock) void k_tree_walk_topk_rows(
    const typename E::raw* __restrict__ target, const int32_t* __restrict__ node_token,
    const int32_t* __restrict__ node_parent, const int32_t* __restrict__ n_nodes,
    const float* __restrict__ uniforms, int B, int N, int V, int topk, float temperature,
    int32_t* __restrict__ path, int32_t* __restrict__ A_out, int32_t* __restrict__ next_out,
    int32_t* __restrict__ status_out) {
    __shared__ TopkSmem sm;
    __shared__ unsigned long long cbuf[kWavesPerBlock * kTileSeg];
    __shared__ int s_rank[kWavesPerBlock * kTileSeg];
    __shared__ TopEntry lst[kMaxTopk];
    __shared__ TopEntry pl[kMaxTopk];
    __shared__ double cw[kMaxTopk];
    __shared__ int ci[kMaxTopk];
    __shared__ uint32_t s_bound[kWavesPerBlock];
    __shared__ int s_wcnt[kWavesPerBlock];
    __shared__ int s_pick[3];
    constexpr int EV = E::kVec;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const bool w0 = tid < kWave;
    const int gvend = (V + EV - 1) / EV;
    const bool in_tile = gvend <= kTileVecs * kBlock;
    int nn = n_nodes[b];
    nn = nn < 1 ? 1 : (nn > N ? N : nn);
    const int my_tok = (w0 && lane < nn) ? node_token[(int64_t)b * N + lane] : -1;
    const int my_par = (w0 && lane < nn) ? node_parent[(int64_t)b * N + lane] : -2;
    for (int i = tid; i < N; i += kBlock) path[(int64_t)b * N + i] = -1;
    const double T = (double)temperature;
    int node = 0, len = 0, next = -1, status = 0;
    for (int step = 0; step < N; ++step) {
        const int64_t r = (int64_t)b * N + node;
        const typename E::raw* row = target + r * V;
        int kept = -1;
        if (in_tile) {
            uint4 v[kTileVecs];
#pragma unroll
            for (int i = 0; i < kTileVecs; ++i) v[i] = topk_raw<E, VEC>(row, V, gvend, i * kBlock + tid);
            kept = tile_topk<E>(v, topk, lst, cbuf, s_rank, s_bound, s_wcnt);
        }
        if (kept < 0) kept = row_topk_list<E, VEC>(row, V, topk, lst, &sm);   // uniform
        if (w0) {
            // softmax over the kept set (fp64), then the draw and the child
            const double m = kept > 0 ? (double)lst[0].x / T : 0.0;
            double S = 0.0;
            for (int i = lane; i < kept; i += kWave) S += exp((double)lst[i].x / T - m);
            S = wave_sum(S);
            const bool valid = kept > 0 && isfinite(m) && isfinite(S) && S > 0.0;
            int g = -1;
            unsigned long long h = 0ull;
            if (valid) {
                RowTop sp;
                sp.count = kept;
                sp.valid = 1;
                sp.m = m;
                sp.S = S;
                sp.py = 0.0;
                double unused;
                g = list_inverse_cdf(lst, sp, nullptr, sp, false, T, (double)uniforms[r], cw, ci, pl, pl,
                                     &unused);
                h = __ballot(g >= 0 && lane >= 1 && lane < nn && my_par == node && my_tok == g);
            }
            if (lane == 0) {
                s_pick[0] = valid ? 1 : 0;
                s_pick[1] = g;
                s_pick[2] = h ? __ffsll(h) - 1 : -1;
            }
        }
        // the next write of s_pick, lst or the row scratch follows the next
        // row's first barrier, after every thread has read this step's pick
        __syncthreads();
        const int valid = s_pick[0], g = s_pick[1], child = s_pick[2];
        if (!valid) {
            status |= 2;
            next = -1;
            break;
        }
        if (child < 0) {
            next = g;
            break;
        }
        if (tid == 0) path[(int64_t)b * N + len] = child;
        ++len;
        node = child;
    }
    if (tid == 0) {
        A_out[b] = len;
        next_out[b] = next;
        if (status_out) status_out[b] = status;
    }
}

// ---------------------------------------------------------------------------
// DDTree best-first build: one 256-thread workgroup per sequence. The tree is
// the first N-1 prefixes in the pop order below; build_by_threshold finds them
// directly in the common case, and otherwise wave 0 pops them one by one.
// The frontier of the pop loop holds, for the
// nodes popped so far, the first child and the next sibling not yet taken,
// kept sorted best first under (Q desc, depth asc, rank tuple lexicographically
// asc), one prefix per lane (lane 0 the best). A pop reads lane 0; its child
// and its sibling are placed by two wave ballots (how many frontier entries
// beat each), and one lane permutation removes the head and opens their
// slots. The rank tuple is packed 6 bits per depth, big end first, in two
// 64-bit words, so equal-depth tuples compare as integers. The frontier never
// needs more than 64 entries: after n pops it holds at most n + 1.
// ---------------------------------------------------------------------------
struct Prefix {
    float Q;
    int meta;                   // depth | parent << 5 | rank << 11 (rank at the last depth)
    unsigned long long w0, w1;  // rank tuple
};

__device__ __forceinline__ int meta_depth(int m) { return m & 31; }
__device__ __forceinline__ int meta_parent(int m) { return (m >> 5) & 63; }
__device__ __forceinline__ int meta_rank(int m) { return (m >> 11) & 63; }
__device__ __forceinline__ int make_meta(int depth, int parent, int rank) {
    return depth | (parent << 5) | (rank << 11);
}

// a before b in the pop order (distinct prefixes never compare equal);
// bitwise logic, so a wave evaluates it without branches
__device__ __forceinline__ bool prefix_before(const Prefix& a, const Prefix& b) {
    const int da = meta_depth(a.meta), db = meta_depth(b.meta);
    const bool w_less = (a.w0 < b.w0) | ((a.w0 == b.w0) & (a.w1 < b.w1));
    return (a.Q > b.Q) | ((a.Q == b.Q) & ((da < db) | ((da == db) & w_less)));
}

__device__ __forceinline__ void set_rank(Prefix& f, int pos, int r) {
    const bool lo = pos < 10;
    const int sh = 54 - 6 * (lo ? pos : pos - 10);
    const unsigned long long w = lo ? f.w0 : f.w1;
    const unsigned long long v = (w & ~(0x3full << sh)) | ((unsigned long long)r << sh);
    f.w0 = lo ? v : f.w0;
    f.w1 = lo ? f.w1 : v;
}

__device__ __forceinline__ unsigned long long readlane64(unsigned long long v, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
    return ((unsigned long long)hi << 32) | lo;
}

// DPP lane shifts of a 32-bit value across the whole wave: from the next lane
// (lane 63 keeps its own) and from the previous lane (lane 0 keeps its own).
__device__ __forceinline__ uint32_t from_next_lane(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x130, 0xf, 0xf, false);   // wave_shl:1
}
__device__ __forceinline__ uint32_t from_prev_lane(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x138, 0xf, 0xf, false);   // wave_shr:1
}
// v from lane+1 (nb == 0), this lane (nb == 1) or lane-1 (nb == 2)
__device__ __forceinline__ uint32_t shift_pick(uint32_t v, int nb) {
    const uint32_t up = from_next_lane(v), down = from_prev_lane(v);
    return nb == 0 ? up : (nb == 1 ? v : down);
}
__device__ __forceinline__ unsigned long long shift_pick64(unsigned long long v, int nb) {
    return ((unsigned long long)shift_pick((uint32_t)(v >> 32), nb) << 32) | shift_pick((uint32_t)v, nb);
}

// The same tree by threshold, for the common case. With at least N-1 entries
// in the depth-1 list, beta = the (N-1)-th of them is a lower bound on the
// score of the (N-1)-th prefix (the N-1 depth-1 prefixes all reach it), so the
// tree lies inside C = {prefixes with Q >= beta}. C is prefix-closed (a
// child's score never exceeds its parent's), so it is enumerated level by
// level: each member's children at the next depth are a prefix of that
// depth's list, found by a binary search over the fp32 products. The members
// are ranked by counting under the pop order, and the first N-1 are the tree
// (every prefix before a tree node is itself in C). Returns false, having
// written nothing, when the list is shorter or C exceeds kBuildCap; the pop
// loop then builds the tree.
// The pop order of the threshold path's members as one 64-bit key, larger
// first: score (non-negative, so its bits order it once a -0 product counts
// as +0), then lower depth, then lower slot. Within a depth the members are enumerated in rank-tuple order (the
// children of a level by parent slot, then by their own rank), so slot order
// there is the tuple order.
__device__ __forceinline__ unsigned long long pop_key(float Q, int depth, int slot) {
    return ((unsigned long long)(Q == 0.f ? 0u : __float_as_uint(Q)) << 32) |
           ((unsigned long long)(31 - depth) << 16) |
           (unsigned long long)(0xffff - slot);
}

constexpr int kBuildThreads = 256;
constexpr int kBuildCap = 256;
constexpr int kBuildWaves = kBuildThreads / kWave;
static_assert(kBuildCap <= kBuildThreads, "one parent per thread when a level is expanded");

__device__ __forceinline__ int cinfo(int depth, int rank, int parent_plus1) {
    return depth | (rank << 5) | (parent_plus1 << 11);
}

__device__ bool build_by_threshold(const float (*qv)[64], const int (*tv)[64], const int* s_cnt, int K,
                                   int N, int32_t* __restrict__ tok_out, int32_t* __restrict__ par_out,
                                   int32_t* __restrict__ dep_out, float* __restrict__ score_out,
                                   unsigned long long* __restrict__ anc_out, int32_t* __restrict__ nn_out) {
    __shared__ float cQ[kBuildCap];
    __shared__ int cInfo[kBuildCap];            // depth | rank << 5 | (parent candidate + 1) << 11
    __shared__ unsigned long long cK[kBuildCap];  // pop-order key, larger first
    __shared__ int cRank[kBuildCap];
    __shared__ int sOff[kBuildCap + 1];
    __shared__ int wsum[kBuildWaves];
    __shared__ int nTok[kWave], nPar[kWave], nDep[kWave];
    __shared__ float nScore[kWave];
    __shared__ unsigned long long nAnc[kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    if (K < 1 || s_cnt[0] < N - 1) return false;
    const float beta = qv[0][N - 2];
    if (!(beta > 0.0f)) return false;
    // depth 1: ranks 0 .. N-2
    if (tid < N - 1) {
        cQ[tid] = 1.0f * qv[0][tid];
        cInfo[tid] = cinfo(1, tid, 0);
        cK[tid] = pop_key(cQ[tid], 1, tid);
    }
    int nc = N - 1, lo = 0, hi = N - 1, maxd = 1;
    for (int d = 1; d < K; ++d) {               // members at depth d get children at depth d+1
        __syncthreads();
        const int nd = s_cnt[d];
        const int i = lo + tid;
        int c = 0;
        if (i < hi && nd > 0) {
            const float Qi = cQ[i];
            int a = 0, z = nd;
            while (a < z) {
                const int mid = (a + z) >> 1;
                if (Qi * qv[d][mid] >= beta) a = mid + 1;
                else z = mid;
            }
            c = a;
        }
        // block scan of the child counts (members lo.. one per thread)
        const int ws = wave_incl_scan_int(c);
        if (lane == kWave - 1) wsum[w] = ws;
        __syncthreads();
        int total = 0, excl = ws - c;
#pragma unroll
        for (int k = 0; k < kBuildWaves; ++k) {
            excl += k < w ? wsum[k] : 0;
            total += wsum[k];
        }
        if (total == 0) break;
        if (nc + total > kBuildCap) return false;
        if (i < hi) sOff[tid] = excl;
        if (tid == 0) sOff[hi - lo] = total;
        __syncthreads();
        // child slot j: its parent p is the last with sOff[p] <= j
        for (int j = tid; j < total; j += kBuildThreads) {
            int a = 0, z = hi - lo;
            while (z - a > 1) {
                const int mid = (a + z) >> 1;
                if (sOff[mid] <= j) a = mid;
                else z = mid;
            }
            const int ip = lo + a, sr = j - sOff[a], slot = nc + j;
            const float Qc = cQ[ip] * qv[d][sr];
            cQ[slot] = Qc;
            cInfo[slot] = cinfo(d + 1, sr, ip + 1);
            cK[slot] = pop_key(Qc, d + 1, slot);
        }
        lo = nc;
        hi = nc + total;
        nc += total;
        maxd = d + 1;
    }
    // pad to a multiple of 8 with keys after every member, so the counting
    // below reads 8 keys per wait
    const int nc8 = (nc + 7) & ~7;
    if (tid >= nc && tid < nc8) cK[tid] = 0ull;
    __syncthreads();
    // ranks by counting under the pop order
    for (int i = tid; i < nc; i += kBuildThreads) {
        const unsigned long long me = cK[i];
        int r = 0;
        for (int j = 0; j < nc8; j += 8) {
            unsigned long long k8[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) k8[q] = cK[j + q];
#pragma unroll
            for (int q = 0; q < 8; ++q) r += k8[q] > me ? 1 : 0;
        }
        cRank[i] = r;
    }
    __syncthreads();
    // the first N-1 become nodes 1 .. N-1 in that order
    for (int i = tid; i < nc; i += kBuildThreads) {
        const int r = cRank[i];
        if (r < N - 1) {
            const int info = cInfo[i];
            const int d = info & 31, sr = (info >> 5) & 63, pc = (info >> 11) - 1;
            const int id = r + 1;
            nTok[id] = tv[d - 1][sr];
            nDep[id] = d;
            nScore[id] = cQ[i];
            nPar[id] = pc < 0 ? 0 : cRank[pc] + 1;
        }
    }
    if (tid == 0) {
        nTok[0] = -1;
        nPar[0] = -1;
        nDep[0] = 0;
        nScore[0] = 1.0f;
        nAnc[0] = 1ull;
    }
    __syncthreads();
    // ancestor masks, one depth at a time (a parent sits one depth up)
    for (int d = 1; d <= maxd; ++d) {
        if (tid >= 1 && tid < N && nDep[tid] == d) nAnc[tid] = nAnc[nPar[tid]] | (1ull << tid);
        __syncthreads();
    }
    if (tid < N) {
        tok_out[tid] = nTok[tid];
        par_out[tid] = nPar[tid];
        dep_out[tid] = nDep[tid];
        score_out[tid] = nScore[tid];
        anc_out[tid] = nAnc[tid];
    }
    if (tid == 0) *nn_out = N;
    return true;
}

__global__ __launch_bounds__(kBuildThreads) void k_tree_build(
    const TopEntry* __restrict__ lists, const int32_t* __restrict__ counts, int K, int N, int W,
    int32_t* __restrict__ node_token, int32_t* __restrict__ node_parent,
    int32_t* __restrict__ node_depth, float* __restrict__ node_score,
    unsigned long long* __restrict__ node_anc, int32_t* __restrict__ n_nodes) {
    __shared__ float qv[kMaxTreeK][64];
    __shared__ int tv[kMaxTreeK][64];
    __shared__ int s_cnt[kMaxTreeK];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;        // (the pop loop runs on wave 0: lane < 64)
    // all loads first (one memory latency), then the LDS copies
    TopEntry e[kMaxTreeK];
#pragma unroll
    for (int d = 0; d < kMaxTreeK; ++d)
        if (d < K && lane < W) e[d] = lists[((int64_t)b * K + d) * W + lane];
    // lane d: the depth-d list's length and best probability (read by readlane)
    const int cnt_d = lane < K ? counts[(int64_t)b * K + lane] : 0;
#pragma unroll
    for (int d = 0; d < kMaxTreeK; ++d)
        if (d < K && lane < W) {
            qv[d][lane] = e[d].x;
            tv[d][lane] = e[d].idx;
        }
    if (lane < kMaxTreeK) s_cnt[lane] = cnt_d;
    __syncthreads();
    if (build_by_threshold(qv, tv, s_cnt, K, N, node_token + (int64_t)b * N,
                           node_parent + (int64_t)b * N, node_depth + (int64_t)b * N,
                           node_score + (int64_t)b * N, node_anc + (int64_t)b * N, n_nodes + b))
        return;
    if (lane >= kWave) return;
    const float q0_d = lane < K ? qv[lane][0] : 0.f;
    // lane n: node n's outputs (node 0 is the root)
    int my_tok = -1, my_par = -1, my_dep = 0;
    float my_score = lane == 0 ? 1.0f : 0.f;
    unsigned long long my_anc = lane == 0 ? 1ull : 0ull;
    Prefix f;                        // this lane's frontier entry (valid below cnt)
    f.Q = 0.f;
    f.meta = 0;
    f.w0 = 0ull;
    f.w1 = 0ull;
    int cnt = 0;
    if (K > 0 && __builtin_amdgcn_readlane(cnt_d, 0) > 0) {
        if (lane == 0) {
            f.Q = 1.0f * q0_d;
            f.meta = make_meta(1, 0, 0);
        }
        cnt = 1;
    }
    int n = 1;
    for (; n < N && cnt > 0; ++n) {
        // The head (lane 0) is node n. Wave-uniform values live in scalar
        // registers; the per-lane work is selects and compares, no branches.
        Prefix X;
        X.Q = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f.Q), 0));
        X.meta = __builtin_amdgcn_readlane(f.meta, 0);
        X.w0 = readlane64(f.w0, 0);
        X.w1 = readlane64(f.w1, 0);
        const int m = meta_depth(X.meta), par = meta_parent(X.meta), rk = meta_rank(X.meta);
        const unsigned long long anc = readlane64(my_anc, par) | (1ull << n);
        const float par_score = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_score), par));
        const int cnt_sib = __builtin_amdgcn_readlane(cnt_d, m - 1);
        const bool hasS = rk + 1 < cnt_sib;
        // (both LDS reads stay inside the list rows: rk + 1 <= 63)
        const float q_sib = qv[m - 1][rk + 1 < 64 ? rk + 1 : 63];
        const int tok_n = tv[m - 1][rk];
        const int mc = m < K ? m : 0;
        const bool hasC = m < K && __builtin_amdgcn_readlane(cnt_d, mc) > 0;
        const float q_child = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, q0_d), mc));
        const bool me = lane == n;
        my_tok = me ? tok_n : my_tok;
        my_par = me ? par : my_par;
        my_dep = me ? m : my_dep;
        my_score = me ? X.Q : my_score;
        my_anc = me ? anc : my_anc;
        // its first child and its next sibling
        Prefix C, S = X;
        C.Q = X.Q * q_child;
        C.meta = make_meta(m + 1, n, 0);         // rank 0 at depth m: its tuple slot is already 0
        C.w0 = X.w0;
        C.w1 = X.w1;
        S.Q = par_score * q_sib;
        S.meta = make_meta(m, par, rk + 1);
        set_rank(S, m - 1, rk + 1);
        // places among the rest of the frontier (lanes 1 .. cnt-1)
        const bool rest = lane >= 1 && lane < cnt;
        const int pc = __popcll(__ballot(hasC & rest & prefix_before(f, C)));
        const int ps = __popcll(__ballot(hasS & rest & prefix_before(f, S)));
        const bool s_first = hasC && hasS && prefix_before(S, C);
        const int fC = hasC ? pc + (s_first ? 1 : 0) : -1;
        const int fS = hasS ? ps + ((hasC && !s_first) ? 1 : 0) : -1;
        // lane j takes C, S, or the entry that lands on j: from lane j+1 when
        // neither was placed before j, lane j after one, lane j-1 after both
        const int nb = (((fC >= 0) & (fC < lane)) ? 1 : 0) + (((fS >= 0) & (fS < lane)) ? 1 : 0);
        const bool tc = lane == fC, ts = lane == fS;
        const float gQ = __builtin_bit_cast(float, shift_pick(__builtin_bit_cast(uint32_t, f.Q), nb));
        const int gm = (int)shift_pick((uint32_t)f.meta, nb);
        const unsigned long long g0 = shift_pick64(f.w0, nb), g1 = shift_pick64(f.w1, nb);
        f.Q = tc ? C.Q : (ts ? S.Q : gQ);
        f.meta = tc ? C.meta : (ts ? S.meta : gm);
        f.w0 = tc ? C.w0 : (ts ? S.w0 : g0);
        f.w1 = tc ? C.w1 : (ts ? S.w1 : g1);
        cnt = min(kWave, cnt - 1 + (hasC ? 1 : 0) + (hasS ? 1 : 0));
    }
    const int64_t o0 = (int64_t)b * N;
    if (lane < N) {
        node_token[o0 + lane] = my_tok;
        node_parent[o0 + lane] = my_par;
        node_depth[o0 + lane] = my_dep;
        node_score[o0 + lane] = my_score;
        node_anc[o0 + lane] = my_anc;
    }
    if (lane == 0) n_nodes[b] = n;
}

// ---------------------------------------------------------------------------
// Exact top-W of a short row held in registers (the tree's per-depth marginal
// rows): one 512-thread workgroup per row, 16 vectors per thread, in the key
// order above (value desc, id asc; NaN never kept).
//  1. Every thread loads its vectors (all in flight together) and takes its
//     largest value.
//  2. Each wave's 8th-largest thread maximum, rounded down to 16 key bits
//     (a ballot bisection), is reached by at least 8 of the wave's tokens, so
//     the smallest of them over the 8 waves (t) is reached by at least 64 > W
//     tokens: every token of the top W has a value >= t.
//  3. The tokens with a value >= t (about a hundred on a row of
//     probabilities) go to LDS as keys in one pass, placed by an LDS counter;
//     each key takes its rank by counting the larger keys (8 per LDS wait),
//     and the first W are written in rank order.
//  4. Should more than kShortCap tokens reach t (mass ties), a key bound is
//     found by bisection over the key space, reached by at least W and at
//     most kShortCap keys (keys are distinct, so such a bound exists).
// The passes compare plain values; 64-bit keys are formed for candidates only.
// ---------------------------------------------------------------------------
constexpr int kShortThreads = 512;
constexpr int kShortVecs = 16;                  // 16-byte vectors per thread
constexpr int kShortWaves = kShortThreads / kWave;
constexpr int kShortRth = 8;                    // kShortRth * kShortWaves > W
constexpr int kShortCap = 512;                  // candidates ranked by counting
static_assert(kShortRth * kShortWaves >= 64, "the bound must be reached by W <= 63 tokens");

template <class E, bool VEC>
__global__ __launch_bounds__(kShortThreads) void k_topk_short(const typename E::raw* __restrict__ rows,
                                                              int V, int W,
                                                              TopEntry* __restrict__ lists,
                                                              int32_t* __restrict__ counts) {
    __shared__ unsigned long long cand[kShortCap];
    __shared__ uint32_t wkey[kShortWaves];
    __shared__ int wsum[kShortWaves];
    __shared__ int s_total;
    constexpr int EV = E::kVec;
    const int task = blockIdx.x;
    const typename E::raw* row = rows + (int64_t)task * V;
    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int gvend = (V + EV - 1) / EV;
    uint4 v[kShortVecs];
#pragma unroll
    for (int i = 0; i < kShortVecs; ++i) v[i] = topk_raw<E, VEC>(row, V, gvend, i * kShortThreads + tid);
    // Each pass reads the raw data and a token base that are opaque to the
    // optimiser, so that no per-token value is kept alive across passes.
    int jb = tid * EV;
    auto fresh = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kShortVecs; ++i)
            asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
        asm volatile("" : "+v"(jb));
    };
    // block sum of per-thread counts (every thread gets it) and, in *excl,
    // the sum over the threads before this one
    auto block_count = [&](int c, int* excl) __attribute__((always_inline)) -> int {
        const int ws = wave_incl_scan_int(c);
        __syncthreads();             // wsum is reused
        if (lane == kWave - 1) wsum[w] = ws;
        __syncthreads();
        int tot = 0, before = ws - c;
#pragma unroll
        for (int i = 0; i < kShortWaves; ++i) {
            before += i < w ? wsum[i] : 0;
            tot += wsum[i];
        }
        *excl = before;
        return tot;
    };
    // number of this thread's keys >= k (k > 0), for the bisection; it reads
    // the row again, one vector at a time (the rare path keeps no second copy
    // of the row in registers)
    auto count_key_ge = [&](unsigned long long k) __attribute__((always_inline)) -> int {
        int c = 0;
#pragma unroll 1
        for (int i = 0; i < kShortVecs; ++i) {
            const int gvi = i * kShortThreads + tid;
            const uint4 u = topk_raw<E, VEC>(row, V, gvend, gvi);
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const float x = raw_elem<E>(u, e);
                c += (x == x && make_key(x, gvi * EV + e) >= k) ? 1 : 0;
            }
        }
        return c;
    };
    // 1. each vector's and the thread's largest value (fmaxf skips NaN; NaN
    // only if all are)
    float vmax[kShortVecs];
    float m = NAN;
#pragma unroll
    for (int i = 0; i < kShortVecs; ++i) {
        vmax[i] = NAN;
#pragma unroll
        for (int e = 0; e < EV; ++e) vmax[i] = fmaxf(vmax[i], raw_elem<E>(v[i], e));
        m = fmaxf(m, vmax[i]);
    }
    // 2. each wave's kShortRth-th largest thread maximum as order-preserving
    // bits, kept to its top 16 bits (rounded down: still reached by at least
    // kShortRth of the wave's maxima; 0: fewer than kShortRth kept)
    const uint32_t rth = wave_jth_largest<16>((m == m) ? ordered_bits(m) : 0u, kShortRth);
    if (lane == 0) wkey[w] = rth;
    if (tid == 0) s_total = 0;
    __syncthreads();
    uint32_t tb = wkey[0];
#pragma unroll
    for (int i = 1; i < kShortWaves; ++i) tb = min(tb, wkey[i]);
    // a wave without kShortRth kept maxima: every kept token competes (and a
    // bound kept to 16 bits below -inf's key, which decodes to a NaN, is -inf)
    float t = tb == 0u ? -INFINITY : from_ordered(tb);
    if (t != t) t = -INFINITY;
    // 3. the candidates (value >= t) to LDS in one pass, placed by an LDS
    // counter (their order does not matter: ranks come from the keys); the
    // count tells whether they fit. Only the vectors whose maximum reaches t
    // are visited, one per lane per round (lowest first), and their passing
    // elements one per lane per step, the wave's slots from one atomic.
    {
        fresh();
        uint32_t vm = 0u;
#pragma unroll
        for (int i = 0; i < kShortVecs; ++i) vm |= vmax[i] >= t ? (1u << i) : 0u;
        while (__ballot(vm != 0u)) {
            const int i = vm != 0u ? __builtin_ctz(vm) : 0;
            uint4 x = v[0];
#pragma unroll
            for (int k = 1; k < kShortVecs; ++k) {
                const bool sel = i == k;
                x.x = sel ? v[k].x : x.x;
                x.y = sel ? v[k].y : x.y;
                x.z = sel ? v[k].z : x.z;
                x.w = sel ? v[k].w : x.w;
            }
            uint32_t em = 0u;
            if (vm != 0u) {
#pragma unroll
                for (int e = 0; e < EV; ++e) em |= raw_elem<E>(x, e) >= t ? (1u << e) : 0u;
            }
            vm &= vm - 1u;
            while (true) {
                const bool has = em != 0u;
                const unsigned long long bal = __ballot(has);
                if (bal == 0ull) break;
                int base = 0;
                if (lane == 0) base = atomicAdd(&s_total, (int)__popcll(bal));
                base = __shfl(base, 0, kWave);
                if (has) {
                    const int e = __builtin_ctz(em);
                    em &= em - 1u;
                    const int at = base + (int)__builtin_amdgcn_mbcnt_hi(
                                              (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                    if (at < kShortCap) cand[at] = make_key(raw_elem<E>(x, e), jb + i * kShortThreads * EV + e);
                }
            }
        }
    }
    __syncthreads();
    int total = s_total;
    if (total > kShortCap) {
        unsigned long long kb = 0ull;
        // 4. mass ties: bisection over keys for a bound reached by W ..
        // kShortCap keys; lo is reached by more than kShortCap keys, hi by none
        // (the key of t's value at token 0 is not below any key of value >= t)
        unsigned long long lo = make_key(t, 0) & 0xffffffff00000000ull;
        unsigned long long hi = 0xffffffffffffffffull;
        // Halving a 64-bit interval: at most 64 rounds. The interval never
        // narrows to one key (one key separates counts that differ by at most
        // one, and kShortCap >= W), so a bound is found before that.
        for (int it = 0; it < 64; ++it) {
            const unsigned long long mid = lo + ((hi - lo) >> 1);
            int unused;
            const int n = block_count(count_key_ge(mid), &unused);
            if (n > kShortCap) {
                lo = mid;
            } else if (n >= W) {
                kb = mid;
                break;
            } else {
                hi = mid;
            }
        }
        // the candidates again, by key (between W and kShortCap of them)
        __syncthreads();
        if (tid == 0) s_total = 0;
        __syncthreads();
        fresh();
#pragma unroll
        for (int i = 0; i < kShortVecs; ++i) {
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const float x = raw_elem<E>(v[i], e);
                if (x >= t) {
                    const unsigned long long k = make_key(x, jb + i * kShortThreads * EV + e);
                    if (k >= kb) {
                        const int at = atomicAdd(&s_total, 1);
                        if (at < kShortCap) cand[at] = k;
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        total = s_total;
    }
    total = total < kShortCap ? total : kShortCap;
    TopEntry* L = lists + (int64_t)task * W;
    auto put = [&](unsigned long long k, int rank) __attribute__((always_inline)) {
        if (rank < W) {
            TopEntry te;
            te.idx = (int32_t)(0xffffffffu - (uint32_t)(k & 0xffffffffull));
            te.x = from_ordered((uint32_t)(k >> 32));
            L[rank] = te;
        }
    };
    // keys past the candidates read as 0, which no key beats: the counts
    // below read 8 keys per LDS wait
    const int padded = (total + 31) & ~31;
    for (int i = total + tid; i < padded; i += kShortThreads) cand[i] = 0ull;
    __syncthreads();
    auto count_above8 = [&](int j, unsigned long long k) __attribute__((always_inline)) -> int {
        unsigned long long c8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) c8[q] = cand[j + q];
        int r = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) r += c8[q] > k ? 1 : 0;
        return r;
    };
    if (total <= kShortThreads / 4) {
        // four threads (a DPP quad) count the larger keys in a quarter of the
        // 8-key blocks each
        const int ci = tid >> 2, part = tid & 3;
        const unsigned long long k = ci < total ? cand[ci] : ~0ull;
        int r = 0;
        for (int j = part * 8; j < padded; j += 32) r += count_above8(j, k);
        r += __builtin_amdgcn_update_dpp(0, r, 0xb1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
        r += __builtin_amdgcn_update_dpp(0, r, 0x4e, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
        if (ci < total && part == 0) put(k, r);
    } else {
        for (int ci = tid; ci < total; ci += kShortThreads) {
            const unsigned long long k = cand[ci];
            int rank = 0;
            for (int j = 0; j < padded; j += 8) rank += count_above8(j, k);
            put(k, rank);
        }
    }
    const int kept = total < W ? total : W;
    for (int i = kept + tid; i < W; i += kShortThreads) {
        TopEntry te;
        te.idx = -1;
        te.x = -INFINITY;
        L[i] = te;
    }
    if (tid == 0) counts[task] = kept;
}

}  // namespace

struct TopkLayout {
    TopEntry* lists;
    int32_t* counts;
    RowTop* rowtop;
    int32_t* live;      // sequences undecided after the first phase, then their count
};

// Carves the workspace: per row task its kept list, count and statistics,
// then `n_state` int32 (the per-sequence phase state). Returns the state
// buffer; *bytes, if given, receives the total size.
static int32_t* topk_layout(void* ws, size_t tasks, int topk, TopkLayout* L, size_t n_state,
                            size_t* bytes = nullptr) {
    Carve cv;
    const size_t o_lists = cv.take(tasks * topk * sizeof(TopEntry));
    const size_t o_counts = cv.take(tasks * sizeof(int32_t));
    const size_t o_rowtop = cv.take(tasks * sizeof(RowTop));
    const size_t o_state = cv.take(n_state * sizeof(int32_t));
    const size_t o_live = cv.take((n_state + 1) * sizeof(int32_t));
    if (bytes) *bytes = cv.off;
    if (L == nullptr) return nullptr;
    char* w = static_cast<char*>(ws);
    L->lists = reinterpret_cast<TopEntry*>(w + o_lists);
    L->counts = reinterpret_cast<int32_t*>(w + o_counts);
    L->rowtop = reinterpret_cast<RowTop*>(w + o_rowtop);
    L->live = reinterpret_cast<int32_t*>(w + o_live);
    return reinterpret_cast<int32_t*>(w + o_state);
}

size_t chain_topk_ws_bytes(int B, int K_max, int V, int top_k) {
    (void)V;
    size_t n = 0;
    topk_layout(nullptr, (size_t)B * (K_max + 1) * 2, top_k, nullptr, (size_t)B, &n);
    return n;
}

size_t tree_build_ws_bytes(int B, int K, int V, int N) {
    const int W = (N - 1) < V ? (N - 1) : V;
    size_t n = 0;
    topk_layout(nullptr, (size_t)B * K, W, nullptr, 0, &n);
    return n;
}

template <class E, bool VEC>
static hipError_t chain_topk_impl(const ChainArgs& a) {
    const size_t tasks = (size_t)a.B * (a.K_max + 1) * 2;
    TopkLayout L;
    int32_t* phase_state = topk_layout(a.ws, tasks, a.top_k, &L, (size_t)a.B);
    using raw = typename E::raw;
    // Positions in two phases, as in the full-vocabulary path: slots 0-1 of
    // every sequence, then the rest only where both first drafts passed.
    const bool phased = a.probs_out == nullptr && a.cap == nullptr && a.accepted_full == nullptr &&
                        kTopkPhaseSplit < a.K_max + 1 &&
                        (size_t)a.B * (a.K_max + 1) * a.V >= kTopkPhaseMinElems;
    const int bounds[3] = {0, phased ? kTopkPhaseSplit : a.K_max + 1, a.K_max + 1};
    const int n_phases = phased ? 2 : 1;
    int32_t* state = phased ? phase_state : nullptr;
    const unsigned seq_blocks = (unsigned)((a.B + kDecideSeqs - 1) / kDecideSeqs);
    for (int ph = 0; ph < n_phases; ++ph) {
        const int lo = bounds[ph], hi = bounds[ph + 1];
        const unsigned grid = (unsigned)((size_t)a.B * (hi - lo) * 2);
        int32_t* live_n = L.live + a.B;
        if (ph == 0)
            PassTimer::launch(k_topk_rows<E, VEC>, dim3(grid), dim3(kBlock), a.stream,
                              static_cast<const raw*>(a.target), static_cast<const raw*>(a.draft),
                              a.cu, a.K_max, a.V, a.top_k, 1, a.tokens, a.temperature, L.lists,
                              L.counts, L.rowtop, lo, hi - lo, (const int32_t*)nullptr,
                              phased ? live_n : nullptr);
        else
            hipLaunchKernelGGL((k_topk_rows<E, VEC>), dim3(grid), dim3(kBlock), 0, a.stream,
                               static_cast<const raw*>(a.target), static_cast<const raw*>(a.draft),
                               a.cu, a.K_max, a.V, a.top_k, 1, a.tokens, a.temperature, L.lists,
                               L.counts, L.rowtop, lo, hi - lo, (const int32_t*)L.live, live_n);
        hipLaunchKernelGGL(k_chain_topk_decide, dim3(seq_blocks), dim3(kDecideSeqs * kWave), 0, a.stream, L.lists,
                           L.rowtop, a.tokens, a.uniforms, a.cu, a.B, a.K_max, a.V, a.top_k,
                           a.temperature, a.accepted_len, a.next_token, a.probs_out,
                           a.resid_mass_out, a.seq_status, a.cap, a.accepted_full, hi, state, ph, L.live,
                           live_n);
    }
    return hipGetLastError();
}

hipError_t launch_chain_topk(const ChainArgs& a) {
    if (a.dtype == 1) {
        if (a.V % Bf16::kVec == 0) return chain_topk_impl<Bf16, true>(a);
        return chain_topk_impl<Bf16, false>(a);
    }
    if (a.V % F32::kVec == 0) return chain_topk_impl<F32, true>(a);
    return chain_topk_impl<F32, false>(a);
}

template <class E, bool VEC>
static void walk_topk_rows(const void* target, const int32_t* tok, const int32_t* par,
                           const int32_t* n_nodes, const float* uniforms, int B, int N, int V,
                           float temperature, int top_k, int32_t* path, int32_t* accepted_len,
                           int32_t* next_token, int32_t* seq_status, hipStream_t stream) {
    PassTimer::launch(k_tree_walk_topk_rows<E, VEC>, dim3((unsigned)B), dim3(kBlock), stream,
                      static_cast<const typename E::raw*>(target), tok, par, n_nodes, uniforms, B, N, V,
                      top_k, temperature, path, accepted_len, next_token, seq_status);
}

hipError_t launch_tree_walk_topk(const void* target, int dtype, const int32_t* tok, const int32_t* par,
                                 const int32_t* n_nodes, const float* uniforms, int B, int N, int V,
                                 float temperature, int top_k, int32_t* path, int32_t* accepted_len,
                                 int32_t* next_token, int32_t* seq_status, hipStream_t stream) {
    if (dtype == 1) {
        if (V % Bf16::kVec == 0)
            walk_topk_rows<Bf16, true>(target, tok, par, n_nodes, uniforms, B, N, V, temperature, top_k, path,
                                       accepted_len, next_token, seq_status, stream);
        else
            walk_topk_rows<Bf16, false>(target, tok, par, n_nodes, uniforms, B, N, V, temperature, top_k, path,
                                        accepted_len, next_token, seq_status, stream);
    } else {
        if (V % F32::kVec == 0)
            walk_topk_rows<F32, true>(target, tok, par, n_nodes, uniforms, B, N, V, temperature, top_k, path,
                                      accepted_len, next_token, seq_status, stream);
        else
            walk_topk_rows<F32, false>(target, tok, par, n_nodes, uniforms, B, N, V, temperature, top_k, path,
                                       accepted_len, next_token, seq_status, stream);
    }
    return hipGetLastError();
}

hipError_t launch_tree_build(const float* marg, int B, int K, int V, int N, int32_t* tok,
                             int32_t* par, int32_t* dep, float* score, uint64_t* anc,
                             int32_t* n_nodes, void* ws, hipStream_t stream) {
    const int W = (N - 1) < V ? (N - 1) : V;
    const size_t tasks = (size_t)B * K;
    TopkLayout L;
    topk_layout(ws, tasks, W, &L, 0);
    if (tasks > 0 && V <= kShortThreads * kShortVecs * F32::kVec) {
        if (V % F32::kVec == 0)
            PassTimer::launch(k_topk_short<F32, true>, dim3((unsigned)tasks), dim3(kShortThreads), stream,
                              marg, V, W, L.lists, L.counts);
        else
            PassTimer::launch(k_topk_short<F32, false>, dim3((unsigned)tasks), dim3(kShortThreads), stream,
                              marg, V, W, L.lists, L.counts);
    } else if (tasks > 0) {
        if (V % F32::kVec == 0)
            PassTimer::launch(k_topk_rows<F32, true>, dim3((unsigned)tasks), dim3(kBlock), stream, marg,
                              marg, nullptr, 0, V, W, 0, nullptr, 1.0f, L.lists, L.counts, nullptr, 0,
                              1, (const int32_t*)nullptr, (int32_t*)nullptr);
        else
            PassTimer::launch(k_topk_rows<F32, false>, dim3((unsigned)tasks), dim3(kBlock), stream, marg,
                              marg, nullptr, 0, V, W, 0, nullptr, 1.0f, L.lists, L.counts, nullptr, 0,
                              1, (const int32_t*)nullptr, (int32_t*)nullptr);
    } else {
        PassTimer::mark_before(stream);
        PassTimer::mark_after(stream);
    }
    hipLaunchKernelGGL(k_tree_build, dim3(B), dim3(kBuildThreads), 0, stream, L.lists, L.counts, K, N, W, tok,
                       par, dep, score, reinterpret_cast<unsigned long long*>(anc), n_nodes);
    return hipGetLastError();
}

}  // namespace sd
