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

// Sorts buf[0..n) descending (bitonic network, n a power of two <= kCap). All
// kBlock threads call it.
__device__ void bitonic_desc(unsigned long long* buf, int n) {
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < n / 2; i += kBlock) {
                const int lo = 2 * stride * (i / stride) + (i % stride);
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const unsigned long long a = buf[lo], b = buf[hi];
                if ((a < b) == desc) {
                    buf[lo] = b;
                    buf[hi] = a;
                }
            }
            __syncthreads();
        }
    }
}

__device__ __forceinline__ int pow2_at_least(int n) {
    int p = 2;
    while (p < n) p <<= 1;
    return p;
}

// Sorts the first n keys of buf descending (entries n.. must be zero-filled up
// to the next power of two). All threads call it.
__device__ void sort_candidates(unsigned long long* buf, int n) {
    bitonic_desc(buf, pow2_at_least(n < 2 ? 2 : n));
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
constexpr int kTopkU = 4;                // vectors per thread per main-pass step (as many more in flight)
constexpr int kWaveCap = 512;            // per-wave candidate buffer (64-bit keys)

template <class E, bool VEC>
__device__ __forceinline__ void topk_load(const typename E::raw* row, int V, int nvec, int vi,
                                          float (&f)[E::kVec]) {
    constexpr int EV = E::kVec;
    if (VEC) {
        if (vi < nvec) {
            E::unpack(load16(row, vi), f);
        } else {
#pragma unroll
            for (int e = 0; e < EV; ++e) f[e] = NAN;
        }
    } else {
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            const int j = vi * EV + e;
            f[e] = (vi < nvec && j < V) ? E::at(row, j) : NAN;
        }
    }
}

// Orders the wave's LDS traffic: every lane's earlier LDS writes are visible
// to every lane's later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bitonic sort (descending) of a[0..n) by one wave, n a power of two.
__device__ void wave_sort_desc(unsigned long long* a, int n) {
    const int lane = threadIdx.x & (kWave - 1);
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            wave_lds_sync();
            for (int i = lane; i < n / 2; i += kWave) {
                const int lo = 2 * stride * (i / stride) + (i % stride);
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const unsigned long long x = a[lo], y = a[hi];
                if ((x < y) == desc) {
                    a[lo] = y;
                    a[hi] = x;
                }
            }
        }
    }
    wave_lds_sync();
}

// A wave's running top-k: `cnt` keys in its LDS buffer, every kept key beats
// `thr` (whose value part is `tf`). Uniform across the wave's lanes.
struct WaveTop {
    int cnt;
    unsigned long long thr;
    float tf;
};

// Sorts the wave's buffer, keeps its best topk and raises the threshold to
// the topk-th key (which topk real tokens reach). Out of line: it runs rarely
// and keeps the per-token loop of the caller small enough to unroll.
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

// Offers one vector per lane (values f, 16-byte vector index vi): tokens whose
// key beats the wave's threshold are appended to its buffer; slots come from a
// wave ballot (no atomics). A float pre-check and wave-wide ballots skip the
// 64-bit key work for token slots no lane needs.
template <int EV>
__device__ __forceinline__ void wave_offer(const float (&f)[EV], int vi, unsigned long long* wb,
                                           WaveTop& st, int topk) {
    float vm = f[0];
#pragma unroll
    for (int e = 1; e < EV; ++e) vm = fmaxf(vm, f[e]);
    if (__ballot(vm >= st.tf) == 0ull) return;        // NaN and sub-threshold vectors
#pragma unroll
    for (int e = 0; e < EV; ++e) {
        const float x = f[e];
        const bool pass = x >= st.tf;
        if (__ballot(pass) == 0ull) continue;
        const unsigned long long key = pass ? make_key(x, vi * EV + e) : 0ull;
        bool take = pass && key > st.thr;
        unsigned long long bal = __ballot(take);
        if (bal == 0ull) continue;
        if (st.cnt + __popcll(bal) > kWaveCap) {
            st = wave_compact(wb, st, topk);
            take = take && key > st.thr;
            bal = __ballot(take);
        }
        if (take) {
            const int off = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            wb[st.cnt + off] = key;
        }
        st.cnt += __popcll(bal);
        if (st.cnt >= kWaveCap / 2) st = wave_compact(wb, st, topk);   // keep the threshold tight
    }
}

// Reads 16-byte vector `gvi` (index within the row) of tokens [.., end) into f;
// NaN past the end.
template <class E, bool VEC>
__device__ __forceinline__ void topk_load_range(const typename E::raw* row, int end, int gvend,
                                                int gvi, float (&f)[E::kVec]) {
    constexpr int EV = E::kVec;
    if (VEC) {
        if (gvi < gvend) {
            E::unpack(load16(row, gvi), f);
        } else {
#pragma unroll
            for (int e = 0; e < EV; ++e) f[e] = NAN;
        }
    } else {
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            const int j = gvi * EV + e;
            f[e] = (gvi < gvend && j < end) ? E::at(row, j) : NAN;
        }
    }
}

// Softmax statistics of a kept list and p(y) of one token (fp64).
struct RowTop {
    int32_t count;      // kept entries
    int32_t valid;      // finite maximum and a finite positive sum
    double m;           // max of x / T over the kept set
    double S;           // sum of exp(x / T - m)
    double py;          // p(y) of the position's draft token (0 if not kept)
};

// One workgroup per row task: the exact top-k of the row, in key order (value
// desc, then lower id first), written as TopEntry; for the rows of a chain
// also the row's softmax statistics over the kept set and p(y) of the
// position's draft token (fp64).
//  1. Every thread holds kTopkSample vectors of the row's start in registers
//     and takes their maximum. The topk-th largest of these 256 maxima (distinct
//     tokens) is reached by at least topk tokens, so no token below it can be
//     in the top-k: it is every wave's starting threshold.
//  2. Each wave offers its held vectors and then its share of the rest of the
//     row (streamed, next step in flight) to its own LDS buffer; when the
//     buffer is half full the wave sorts it, keeps its best topk and raises its
//     threshold. No workgroup barrier.
//  3. The waves' lists are merged (sorted together) and the first topk written.
template <class E, bool VEC>
__global__ __launch_bounds__(kBlock) void k_topk_rows(const typename E::raw* __restrict__ tgt,
                                                      const typename E::raw* __restrict__ dft,
                                                      const int32_t* __restrict__ cu, int K_max,
                                                      int V, int topk, int chain,
                                                      const int32_t* __restrict__ tok, float temperature,
                                                      TopEntry* __restrict__ lists,
                                                      int32_t* __restrict__ counts,
                                                      RowTop* __restrict__ rowtop) {
    __shared__ unsigned long long wbuf[kWavesPerBlock][kWaveCap];
    __shared__ unsigned long long mbuf[kWavesPerBlock * kMaxTopk];
    __shared__ float lmax[kBlock];
    __shared__ int wcnt[kWavesPerBlock];
    __shared__ unsigned long long thr0;
    constexpr int EV = E::kVec;
    const int task = blockIdx.x;
    const typename E::raw* row = topk_row<E>(tgt, dft, cu, K_max, V, task, chain != 0);
    if (row == nullptr) return;
    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int end = V;
    const int vb = 0;
    const int gvend = (V + EV - 1) / EV;
    const uint4 nanv = make_uint4(0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu);
    // 1. starting threshold from the held sample (kept packed)
    uint4 hs[kTopkSample];
#pragma unroll
    for (int i = 0; i < kTopkSample; ++i) {
        const int gvi = vb + i * kBlock + tid;
        if (VEC) {
            hs[i] = gvi < gvend ? load16(row, gvi) : nanv;
        } else {
            float f[EV];
            topk_load_range<E, VEC>(row, end, gvend, gvi, f);
            uint32_t wd[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
            if (EV == 4) {
#pragma unroll
                for (int e = 0; e < 4 && e < EV; ++e) wd[e] = __float_as_uint(f[e]);
            } else {
#pragma unroll
                for (int e = 0; e < EV; e += 2)
                    wd[e / 2] = (__float_as_uint(f[e]) >> 16) | (__float_as_uint(f[e + 1]) & 0xffff0000u);
            }
            hs[i] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        }
    }
    float m = -INFINITY;
    bool any = false;
#pragma unroll
    for (int i = 0; i < kTopkSample; ++i) {
        float f[EV];
        E::unpack(hs[i], f);
#pragma unroll
        for (int e = 0; e < EV; ++e)
            if (f[e] == f[e]) {
                m = any ? fmaxf(m, f[e]) : f[e];
                any = true;
            }
    }
    lmax[tid] = any ? m : NAN;
    if (tid == 0) thr0 = 0ull;     // keeps every non-NaN token unless raised below
    __syncthreads();
    if (any) {
        int rank = 0;
        for (int j = 0; j < kBlock; ++j) {
            const float o = lmax[j];
            rank += (o > m) || (o == m && j < tid);
        }
        if (rank == topk - 1) {
            const float t = (m == 0.f) ? 0.f : m;
            thr0 = ((unsigned long long)ordered_bits(t) << 32) - 1ull;   // every x >= t passes
        }
    }
    __syncthreads();
    WaveTop st;
    st.cnt = 0;
    st.thr = thr0;
    st.tf = st.thr == 0ull ? -INFINITY : from_ordered((uint32_t)((st.thr + 1ull) >> 32));
    unsigned long long* wb = wbuf[w];
    // 2. offer the held sample, then stream the rest of the row
#pragma unroll
    for (int i = 0; i < kTopkSample; ++i) {
        float f[EV];
        E::unpack(hs[i], f);
        wave_offer<EV>(f, vb + i * kBlock + tid, wb, st, topk);
    }
    const int v_start = vb + kTopkSample * kBlock;
    if (VEC) {
        uint4 cur[kTopkU], nxt[kTopkU];
#pragma unroll
        for (int u = 0; u < kTopkU; ++u) {
            const int gvi = v_start + u * kBlock + tid;
            cur[u] = gvi < gvend ? load16(row, gvi) : nanv;
        }
        for (int v0 = v_start; v0 < gvend; v0 += kBlock * kTopkU) {
            const int vn = v0 + kBlock * kTopkU;
#pragma unroll
            for (int u = 0; u < kTopkU; ++u) {
                const int gvi = vn + u * kBlock + tid;
                nxt[u] = gvi < gvend ? load16(row, gvi) : nanv;
            }
#pragma unroll
            for (int u = 0; u < kTopkU; ++u) {
                float f[EV];
                E::unpack(cur[u], f);
                wave_offer<EV>(f, v0 + u * kBlock + tid, wb, st, topk);
            }
#pragma unroll
            for (int u = 0; u < kTopkU; ++u) cur[u] = nxt[u];
        }
    } else {
        for (int v0 = v_start; v0 < gvend; v0 += kBlock * kTopkU) {
            float f[kTopkU][EV];
#pragma unroll
            for (int u = 0; u < kTopkU; ++u) topk_load_range<E, VEC>(row, end, gvend, v0 + u * kBlock + tid, f[u]);
#pragma unroll
            for (int u = 0; u < kTopkU; ++u) wave_offer<EV>(f[u], v0 + u * kBlock + tid, wb, st, topk);
        }
    }
    st = wave_compact(wb, st, topk);         // each wave: its best min(cnt, topk), sorted
    if (lane == 0) wcnt[w] = st.cnt;
    __syncthreads();
    // 3. merge the waves' lists
    int off = 0, total = 0;
    for (int i = 0; i < kWavesPerBlock; ++i) {
        if (i < w) off += wcnt[i];
        total += wcnt[i];
    }
    unsigned long long* mb = mbuf;
    for (int j = lane; j < st.cnt; j += kWave) mb[off + j] = wb[j];
    const int np2 = pow2_at_least(total < 2 ? 2 : total);
    for (int i = total + tid; i < np2; i += kBlock) mb[i] = 0ull;
    __syncthreads();
    bitonic_desc(mb, np2);
    const int kept = total < topk ? total : topk;
    TopEntry* L = lists + (int64_t)task * topk;
    for (int i = tid; i < topk; i += kBlock) {
        TopEntry te;
        if (i < kept) {
            const unsigned long long key = mb[i];
            te.idx = (int32_t)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
            te.x = from_ordered((uint32_t)(key >> 32));
        } else {
            te.idx = -1;
            te.x = -INFINITY;
        }
        L[i] = te;
    }
    if (tid == 0) counts[task] = kept;
    if (rowtop == nullptr || w != 0) return;
    // softmax statistics of the kept set and p(y) (wave 0, fp64)
    int y = -1;                      // task = ((b * (K_max + 1) + s) * 2 + side)
    {
        const int rest = task >> 1;
        const int s = rest % (K_max + 1);
        int d0, k;
        seq_range(cu, rest / (K_max + 1), K_max, d0, k);
        if (s < k) y = tok[d0 + s];
    }
    const double T = (double)temperature;
    RowTop r;
    r.count = kept;
    r.m = kept > 0 ? (double)from_ordered((uint32_t)(mb[0] >> 32)) / T : 0.0;
    double sum = 0.0, ey = 0.0;
    for (int i = lane; i < kept; i += kWave) {
        const unsigned long long key = mb[i];
        const double e = exp((double)from_ordered((uint32_t)(key >> 32)) / T - r.m);
        sum += e;
        if ((int32_t)(0xffffffffu - (uint32_t)(key & 0xffffffffull)) == y) ey = e;
    }
    sum = wave_sum(sum);
    ey = wave_sum(ey);               // at most one lane holds y
    r.S = sum;
    r.valid = (kept > 0 && isfinite(r.m) && isfinite(sum) && sum > 0.0) ? 1 : 0;
    r.py = (r.valid && y >= 0 && y < V) ? ey / sum : 0.0;
    if (lane == 0) rowtop[task] = r;
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
    for (int i = lane; i < np; i += kWave) pl[i] = P[i];
    for (int i = lane; i < nd; i += kWave) dl[i] = D[i];
    wave_lds_sync();
    for (int i = lane; i < np; i += kWave) {
        const int id = pl[i].idx;
        double wgt = exp((double)pl[i].x / T - sp.m) / sp.S;
        if (residual) {
            double q = 0.0;
            for (int j = 0; j < nd; ++j)
                if (dl[j].idx == id) q = exp((double)dl[j].x / T - sq.m) / sq.S;
            wgt = wgt - q;
            if (!(wgt > 0.0)) wgt = 0.0;
        }
        int rank = 0;
        for (int j = 0; j < np; ++j) rank += (pl[j].idx < id);
        wbuf[rank] = wgt;
        ibuf[rank] = id;
    }
    wave_lds_sync();
    int pick = -1;
    double R = 0.0;
    if (lane == 0) {
        for (int i = 0; i < np; ++i) R += wbuf[i];
        const double target = u * R;
        double C = 0.0;
        int last = -1;
        for (int i = 0; i < np; ++i) {
            C += wbuf[i];
            if (wbuf[i] > 0.0) last = ibuf[i];
            if (C > target && wbuf[i] > 0.0) {
                pick = ibuf[i];
                break;
            }
        }
        if (pick < 0) pick = last;
    }
    wave_lds_sync();
    *R_out = __shfl(R, 0, kWave);
    return __shfl(pick, 0, kWave);
}

// One wave per sequence: accept bits from the rows' p(y) and q(y) (computed by
// the row pass), A (ballot), and the final token from the decision row's lists.
__global__ __launch_bounds__(kBlock) void k_chain_topk_decide(
    const TopEntry* __restrict__ lists, const RowTop* __restrict__ rowtop,
    const int32_t* __restrict__ tok, const float* __restrict__ uni, const int32_t* __restrict__ cu,
    int B, int K_max, int V, int topk, float temperature, int32_t* __restrict__ A_out,
    int32_t* __restrict__ next_out, float* __restrict__ probs_out, float* __restrict__ R_out,
    int32_t* __restrict__ status_out) {
    __shared__ double wbuf_all[kWavesPerBlock][kMaxTopk];
    __shared__ int ibuf_all[kWavesPerBlock][kMaxTopk];
    __shared__ TopEntry pl_all[kWavesPerBlock][kMaxTopk];
    __shared__ TopEntry dl_all[kWavesPerBlock][kMaxTopk];
    const int w = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int b = blockIdx.x * kWavesPerBlock + w;
    if (b >= B) return;
    const int slots = K_max + 1;
    int d0, k;
    seq_range(cu, b, K_max, d0, k);
    const double T = (double)temperature;
    auto task_of = [&](int s, int side) { return (((int64_t)b * slots + s) * 2 + side); };
    bool acc = true;
    int st = 0;
    if (lane < k) {
        const RowTop rp = rowtop[task_of(lane, 0)];
        const RowTop rq = rowtop[task_of(lane, 1)];
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
    const int A = rej ? (__ffsll(rej) - 1) : k;
    int status = (lane < k && lane <= A) ? st : 0;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) status |= __shfl_xor(status, o, kWave);
    const double uf = (double)uni[d0 + b + k];
    int next = -1;
    double R = 0.0;
    double* wbuf = wbuf_all[w];
    int* ibuf = ibuf_all[w];
    TopEntry* pl = pl_all[w];
    TopEntry* dl = dl_all[w];
    if (A < k) {
        const RowTop sp = rowtop[task_of(A, 0)];
        const RowTop sq = rowtop[task_of(A, 1)];
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
        const RowTop sp = rowtop[task_of(k, 0)];
        if (sp.valid) {
            double unused;
            next = list_inverse_cdf(lists + task_of(k, 0) * topk, sp, nullptr, sp, false, T, uf, wbuf,
                                    ibuf, pl, dl, &unused);
        } else {
            status |= 2;
        }
        R = 0.0;
    }
    if (lane == 0) {
        A_out[b] = A;
        next_out[b] = next;
        if (R_out) R_out[b] = (float)R;
        if (status_out) status_out[b] = status;
    }
}

// ---------------------------------------------------------------------------
// DDTree best-first build: one wave per sequence. The frontier (at most 64
// prefixes, one per lane) holds, for every popped node, its first child and
// its next sibling; a pop is a wave argmax under (Q desc, depth asc, rank tuple
// lexicographically asc). The rank tuple is packed 6 bits per depth, big-end
// first, in two 64-bit words, so equal-depth tuples compare as integers.
// ---------------------------------------------------------------------------
struct Front {
    float Q;
    int depth;
    unsigned long long w0, w1;
    int parent;
    int rank;        // rank at the last depth
    int valid;
};

__device__ __forceinline__ bool front_better(const Front& a, const Front& b) {
    if (!a.valid) return false;
    if (!b.valid) return true;
    if (a.Q != b.Q) return a.Q > b.Q;
    if (a.depth != b.depth) return a.depth < b.depth;
    if (a.w0 != b.w0) return a.w0 < b.w0;
    return a.w1 < b.w1;
}

__device__ __forceinline__ void set_rank(Front& f, int pos, int r) {
    if (pos < 10) {
        const int sh = 54 - 6 * pos;
        f.w0 = (f.w0 & ~(0x3full << sh)) | ((unsigned long long)r << sh);
    } else {
        const int sh = 54 - 6 * (pos - 10);
        f.w1 = (f.w1 & ~(0x3full << sh)) | ((unsigned long long)r << sh);
    }
}

__device__ Front shfl_front(const Front& f, int src) {
    Front r;
    r.Q = __shfl(f.Q, src, kWave);
    r.depth = __shfl(f.depth, src, kWave);
    r.w0 = __shfl(f.w0, src, kWave);
    r.w1 = __shfl(f.w1, src, kWave);
    r.parent = __shfl(f.parent, src, kWave);
    r.rank = __shfl(f.rank, src, kWave);
    r.valid = __shfl(f.valid, src, kWave);
    return r;
}

__global__ __launch_bounds__(kWave) void k_tree_build(
    const TopEntry* __restrict__ lists, const int32_t* __restrict__ counts, int K, int N, int W,
    int32_t* __restrict__ node_token, int32_t* __restrict__ node_parent,
    int32_t* __restrict__ node_depth, float* __restrict__ node_score,
    unsigned long long* __restrict__ node_anc, int32_t* __restrict__ n_nodes) {
    __shared__ float qv[kMaxTreeK][64];
    __shared__ int tv[kMaxTreeK][64];
    __shared__ int cntv[kMaxTreeK];
    __shared__ float nscore[64];
    __shared__ unsigned long long nanc[64];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    for (int d = 0; d < K; ++d) {
        const TopEntry* L = lists + ((int64_t)b * K + d) * W;
        if (lane < W) {
            qv[d][lane] = L[lane].x;
            tv[d][lane] = L[lane].idx;
        }
        if (lane == 0) cntv[d] = counts[(int64_t)b * K + d];
    }
    __shared__ int otok[64], opar[64], odep[64];
    if (lane < 64) {
        otok[lane] = -1;
        opar[lane] = -1;
        odep[lane] = 0;
        nscore[lane] = 0.f;
        nanc[lane] = 0ull;
    }
    __syncthreads();
    if (lane == 0) {
        nscore[0] = 1.0f;
        nanc[0] = 1ull;
    }
    Front f;
    f.valid = 0;
    f.Q = 0.f;
    f.depth = 0;
    f.w0 = 0ull;
    f.w1 = 0ull;
    f.parent = -1;
    f.rank = 0;
    if (lane == 0 && K > 0 && cntv[0] > 0) {
        f.valid = 1;
        f.Q = 1.0f * qv[0][0];
        f.depth = 1;
        f.parent = 0;
        f.rank = 0;
    }
    __syncthreads();
    int n = 1;
    while (n < N) {
        // wave argmax
        Front best = f;
        int best_lane = lane;
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) {
            const Front other = shfl_front(best, lane ^ o);
            const int ol = __shfl_xor(best_lane, o, kWave);
            if (front_better(other, best)) {
                best = other;
                best_lane = ol;
            }
        }
        // every lane now holds the same winner
        if (!best.valid) break;
        const int m = best.depth;
        const int tokn = tv[m - 1][best.rank];
        const int par = best.parent;
        const unsigned long long anc = nanc[par] | (1ull << n);
        if (lane == 0) {
            otok[n] = tokn;
            opar[n] = par;
            odep[n] = m;
            nscore[n] = best.Q;
            nanc[n] = anc;
        }
        __syncthreads();
        // the winner's slot becomes the first child of node n
        if (lane == best_lane) {
            if (m < K && cntv[m] > 0) {
                f.Q = best.Q * qv[m][0];
                f.depth = m + 1;
                set_rank(f, m, 0);
                f.parent = n;
                f.rank = 0;
                f.valid = 1;
            } else {
                f.valid = 0;
            }
        }
        // the next sibling goes to the lowest free lane
        if (best.rank + 1 < cntv[m - 1]) {
            const unsigned long long freem = __ballot(!f.valid);
            const int dst = __ffsll(freem) - 1;
            if (lane == dst) {
                f = best;
                f.Q = nscore[par] * qv[m - 1][best.rank + 1];
                set_rank(f, m - 1, best.rank + 1);
                f.rank = best.rank + 1;
                f.valid = 1;
            }
        }
        ++n;
    }
    __syncthreads();
    const int64_t o0 = (int64_t)b * N;
    if (lane < N) {
        node_token[o0 + lane] = otok[lane];
        node_parent[o0 + lane] = opar[lane];
        node_depth[o0 + lane] = odep[lane];
        node_score[o0 + lane] = nscore[lane];
        node_anc[o0 + lane] = nanc[lane];
    }
    if (lane == 0) n_nodes[b] = n;
}

}  // namespace

struct TopkLayout {
    TopEntry* lists;
    int32_t* counts;
    RowTop* rowtop;
};

static size_t topk_layout(void* ws, size_t tasks, int topk, TopkLayout* L) {
    Carve cv;
    const size_t o_lists = cv.take(tasks * topk * sizeof(TopEntry));
    const size_t o_counts = cv.take(tasks * sizeof(int32_t));
    const size_t o_rowtop = cv.take(tasks * sizeof(RowTop));
    if (L) {
        char* w = static_cast<char*>(ws);
        L->lists = reinterpret_cast<TopEntry*>(w + o_lists);
        L->counts = reinterpret_cast<int32_t*>(w + o_counts);
        L->rowtop = reinterpret_cast<RowTop*>(w + o_rowtop);
    }
    return cv.off;
}

size_t chain_topk_ws_bytes(int B, int K_max, int V, int top_k) {
    (void)V;
    return topk_layout(nullptr, (size_t)B * (K_max + 1) * 2, top_k, nullptr);
}

size_t tree_build_ws_bytes(int B, int K, int V, int N) {
    const int W = (N - 1) < V ? (N - 1) : V;
    return topk_layout(nullptr, (size_t)B * K, W, nullptr);
}

template <class E, bool VEC>
static hipError_t chain_topk_impl(const ChainArgs& a) {
    const size_t tasks = (size_t)a.B * (a.K_max + 1) * 2;
    TopkLayout L;
    topk_layout(a.ws, tasks, a.top_k, &L);
    using raw = typename E::raw;
    PassTimer::mark_before(a.stream);
    hipLaunchKernelGGL((k_topk_rows<E, VEC>), dim3((unsigned)tasks), dim3(kBlock), 0, a.stream,
                       static_cast<const raw*>(a.target), static_cast<const raw*>(a.draft), a.cu,
                       a.K_max, a.V, a.top_k, 1, a.tokens, a.temperature, L.lists, L.counts, L.rowtop);
    PassTimer::mark_after(a.stream);
    hipLaunchKernelGGL(k_chain_topk_decide, dim3((unsigned)((a.B + kWavesPerBlock - 1) / kWavesPerBlock)),
                       dim3(kBlock), 0, a.stream, L.lists, L.rowtop, a.tokens, a.uniforms, a.cu, a.B,
                       a.K_max, a.V, a.top_k, a.temperature, a.accepted_len, a.next_token, a.probs_out,
                       a.resid_mass_out, a.seq_status);
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

hipError_t launch_tree_build(const float* marg, int B, int K, int V, int N, int32_t* tok,
                             int32_t* par, int32_t* dep, float* score, uint64_t* anc,
                             int32_t* n_nodes, void* ws, hipStream_t stream) {
    const int W = (N - 1) < V ? (N - 1) : V;
    const size_t tasks = (size_t)B * K;
    TopkLayout L;
    topk_layout(ws, tasks, W, &L);
    PassTimer::mark_before(stream);
    if (tasks > 0) {
        if (V % F32::kVec == 0)
            hipLaunchKernelGGL((k_topk_rows<F32, true>), dim3((unsigned)tasks), dim3(kBlock), 0, stream,
                               marg, marg, nullptr, 0, V, W, 0, nullptr, 1.0f, L.lists, L.counts, nullptr);
        else
            hipLaunchKernelGGL((k_topk_rows<F32, false>), dim3((unsigned)tasks), dim3(kBlock), 0, stream,
                               marg, marg, nullptr, 0, V, W, 0, nullptr, 1.0f, L.lists, L.counts, nullptr);
    }
    PassTimer::mark_after(stream);
    hipLaunchKernelGGL(k_tree_build, dim3(B), dim3(kWave), 0, stream, L.lists, L.counts, K, N, W, tok,
                       par, dep, score, reinterpret_cast<unsigned long long*>(anc), n_nodes);
    return hipGetLastError();
}

}  // namespace sd
