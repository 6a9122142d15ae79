// sd_rerank.hip -- EAGLE-2-style choice of the verification tree.
//
// Page "大模型投机解码：Medusa、MTP、EAGLE、DFlash、DDTree 与 DSpark"
// (chzhyang.github.io), §4 EAGLE-2: candidates are expanded along paths of high
// cumulative confidence, then re-ranked, and the final verification tree is
// chosen from them (its depth and width follow the context).
//
// Input per sequence: an expanded candidate tree in topological order
// (candidate 0 the root, every other candidate's parent an earlier one) with
// each candidate's token and conditional draft probability. Its cumulative
// confidence is the fp32 product of the conditional probabilities along its
// path, root first. The tree keeps the root plus the N-1 best candidates by
// (confidence desc, depth asc, candidate index asc); a child never beats its
// parent under that order, so the kept set is closed under taking parents.
// Nodes are numbered in that order, with the outputs of the DDTree build.
//
// One workgroup per sequence: confidences formed level by level in LDS, one
// barrier per level (a level stamp per candidate tells a finished parent from
// one formed in the same round); then the N-1 best keys by a bound from the
// waves' best keys and ranking by counting of the few keys that reach it
// (heavy ties: each wave sorts its keys and the four lists merge by rank);
// then one thread per kept node.
#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {

namespace {

constexpr int kMaxCand = 1024;
constexpr int kCandPerThread = kMaxCand / kBlock;
constexpr int kSelCap = 256;     // candidates the threshold path ranks by counting

__device__ __forceinline__ uint32_t conf_bits(float x) {
    // x in [0, 1] (a -0 probability gives -0): its bits order it once -0
    // counts as +0 (no other negatives, no NaN)
    return x == 0.f ? 0u : __float_as_uint(x);
}

__global__ __launch_bounds__(kBlock) void k_rerank_tree(
    const int32_t* __restrict__ cand_parent, const int32_t* __restrict__ cand_token,
    const float* __restrict__ cand_prob, const int32_t* __restrict__ n_cand, int M, int N,
    int32_t* __restrict__ node_token, int32_t* __restrict__ node_parent,
    int32_t* __restrict__ node_depth, float* __restrict__ node_score,
    unsigned long long* __restrict__ node_anc, int32_t* __restrict__ node_cand,
    int32_t* __restrict__ n_nodes) {
    __shared__ float score[kMaxCand];
    __shared__ int par[kMaxCand];
    __shared__ int lvl[kMaxCand];            // depth once the confidence is known, else -1
    __shared__ int s_more[3];                // round l sets slot l % 3 when it formed a candidate
    __shared__ unsigned long long wkeys[kWavesPerBlock][kWave * kCandPerThread];
    __shared__ unsigned long long top[64];
    __shared__ int node_of[kMaxCand];
    __shared__ int tok_s[kMaxCand];
    __shared__ unsigned long long sel[kSelCap];
    __shared__ uint32_t s_bound[kWavesPerBlock];
    __shared__ int s_sel;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    int nc = n_cand[b];
    nc = nc < 0 ? 0 : (nc > M ? M : nc);
    const int64_t o = (int64_t)b * M;
    // 1. candidates: a bad parent or probability leaves a candidate (and its
    //    subtree) out
    //    (each thread's own parent, state, confidence and depth stay in
    //    registers; the LDS copies serve the children)
    float prob[kCandPerThread], my_sc[kCandPerThread];
    int my_par[kCandPerThread], my_dep[kCandPerThread];
    bool my_rdy[kCandPerThread];
#pragma unroll
    for (int j = 0; j < kCandPerThread; ++j) {
        const int i = j * kBlock + tid;
        int p = -1, t = -1;
        float q = 0.f;
        if (i < nc) t = cand_token[o + i];   // read now: the outputs need the kept ones
        if (i < nc && i > 0) {
            p = cand_parent[o + i];
            q = cand_prob[o + i];
        }
        const bool ok = i > 0 && i < nc && p >= 0 && p < i && q >= 0.f && q <= 1.f;
        my_par[j] = ok ? p : -1;
        prob[j] = q;
        my_rdy[j] = i == 0 && nc > 0;
        my_sc[j] = (i == 0) ? 1.0f : 0.f;
        my_dep[j] = 0;
        par[i] = my_par[j];
        lvl[i] = my_rdy[j] ? 0 : -1;
        score[i] = my_sc[j];
        node_of[i] = (i == 0) ? 0 : -1;
        tok_s[i] = t;
    }
    if (tid < 3) s_more[tid] = 0;
    __syncthreads();
    // 2. confidences level by level, root first: in round l a candidate
    //    whose parent was formed in an earlier round takes its parent's
    //    confidence times its own probability and depth l. A parent formed in
    //    this round reads as -1 or l, never below l, so one barrier per round
    //    keeps every read on values finished before it. Round l clears slot
    //    (l + 1) % 3 for the next round while slot (l - 1) % 3 may still be
    //    read after the previous barrier.
    bool more = true;
    for (int l = 1; more; ++l) {
        bool any = false;
        if (tid == 0) s_more[(l + 1) % 3] = 0;
#pragma unroll
        for (int j = 0; j < kCandPerThread; ++j) {
            const int p = my_par[j];
            if (!my_rdy[j] && p >= 0) {
                const int lp = lvl[p];
                if (lp >= 0 && lp < l) {
                    const int i = j * kBlock + tid;
                    my_sc[j] = score[p] * prob[j];
                    my_dep[j] = l;
                    my_rdy[j] = true;
                    score[i] = my_sc[j];
                    lvl[i] = l;
                    any = true;
                }
            }
        }
        if (any) s_more[l % 3] = 1;
        __syncthreads();
        more = s_more[l % 3] != 0;
    }
    // 3. keys: (confidence desc, depth asc, index asc); 0 = not a candidate.
    const int w = tid / kWave, lane = tid & (kWave - 1);
    const int kept_max = N - 1;
    unsigned long long key[kCandPerThread];
    unsigned long long kmax = 0ull;
#pragma unroll
    for (int j = 0; j < kCandPerThread; ++j) {
        const int i = j * kBlock + tid;
        key[j] = (i > 0 && my_rdy[j]) ? ((unsigned long long)conf_bits(my_sc[j]) << 32) |
                                            ((unsigned long long)(0xffff - my_dep[j]) << 16) |
                                            (unsigned long long)(0xffff - i)
                                      : 0ull;
        kmax = key[j] > kmax ? key[j] : kmax;
    }
    if (tid < 64) top[tid] = 0ull;
    // Threshold path: in each wave the ceil((N-1)/4)-th largest confidence
    // among its threads' best keys is reached by that many keys, so the
    // smallest of the four waves' values is reached by N-1 keys, and no key
    // below it is kept. The keys at or above it are ranked by counting. With
    // 0 (too few confidences above zero) every key competes.
    const uint32_t tw = wave_jth_largest<0>((uint32_t)(kmax >> 32), (kept_max + kWavesPerBlock - 1) / kWavesPerBlock);
    if (lane == 0) s_bound[w] = tw;
    if (tid == 0) s_sel = 0;
    __syncthreads();
    uint32_t tb = s_bound[0];
#pragma unroll
    for (int i = 1; i < kWavesPerBlock; ++i) tb = min(tb, s_bound[i]);
#pragma unroll
    for (int j = 0; j < kCandPerThread; ++j) {
        if (key[j] != 0ull && (uint32_t)(key[j] >> 32) >= tb) {
            const int at = atomicAdd(&s_sel, 1);
            if (at < kSelCap) sel[at] = key[j];
        }
    }
    __syncthreads();
    const int C = s_sel;
    if (C <= kSelCap) {
        // pad to a multiple of 8 with keys that beat nothing
        const int C8 = (C + 7) & ~7;
        if (tid >= C && tid < C8) sel[tid] = 0ull;
        __syncthreads();
        if (tid < C) {
            const unsigned long long k = sel[tid];
            int rank = 0;
            for (int j = 0; j < C8; j += 8) {
                unsigned long long k8[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) k8[q] = sel[j + q];
#pragma unroll
                for (int q = 0; q < 8; ++q) rank += k8[q] > k ? 1 : 0;
            }
            if (rank < kept_max) top[rank] = k;
        }
        __syncthreads();
    } else {
        // Too many keys reach the bound (ties): each wave sorts its own
        // candidates' keys; a key among the first N-1 of its wave's list
        // takes its rank from its place there plus, by binary search, the
        // keys above it in the other waves' first N-1.
        unsigned long long* wk = wkeys[w];
#pragma unroll
        for (int j = 0; j < kCandPerThread; ++j) wk[lane * kCandPerThread + j] = key[j];
        wave_sort_desc(wk, kWave * kCandPerThread);
        __syncthreads();
        for (int p = lane; p < kept_max; p += kWave) {
            const unsigned long long k = wk[p];
            if (k != 0ull) {
                int rank = p;
                for (int o2 = 0; o2 < kWavesPerBlock; ++o2)
                    if (o2 != w) rank += count_above(wkeys[o2], kept_max, k);
                if (rank < kept_max) top[rank] = k;
            }
        }
        __syncthreads();
    }
    // 4. the first N-1 keys are the kept nodes, numbered in order
    if (tid < kept_max && top[tid] != 0ull) node_of[0xffff - (int)(top[tid] & 0xffffull)] = tid + 1;
    __syncthreads();
    const int64_t on = (int64_t)b * N;
    if (tid < N) {
        int tok = -1, pn = -1, dep = 0, cand = 0;
        float sc = 1.0f;
        unsigned long long anc = 1ull;
        if (tid > 0) {
            const unsigned long long key = top[tid - 1];
            if (key != 0ull) {
                cand = 0xffff - (int)(key & 0xffffull);
                tok = tok_s[cand];
                pn = node_of[par[cand]];
                dep = lvl[cand];
                sc = score[cand];
                anc = 1ull << tid;
                for (int c = par[cand]; c > 0; c = par[c]) anc |= 1ull << node_of[c];
                anc |= 1ull;                                   // the root
            } else {
                cand = -1;
                sc = 0.f;
                anc = 0ull;
            }
        }
        node_token[on + tid] = tok;
        node_parent[on + tid] = pn;
        node_depth[on + tid] = dep;
        node_score[on + tid] = sc;
        node_anc[on + tid] = anc;
        if (node_cand) node_cand[on + tid] = cand;
    }
    if (tid < kWave) {               // the kept keys fill top[0 .. k): count them
        const unsigned long long kb = __ballot(tid < kept_max && top[tid] != 0ull);
        if (tid == 0) n_nodes[b] = 1 + __popcll(kb);
    }
}

// EAGLE-2 expansion step (same page, §4 EAGLE-2: branches are expanded along
// high cumulative confidence). One workgroup per sequence: wave 0 lists the
// expanded nodes in slot order (a ballot gives each its rank), every thread
// appends children, C per expanded node, with confidence fl32(parent
// confidence x probability) (-1 when the probability is not in [0, 1]); the
// next nodes to expand are the W best new candidates by (confidence desc,
// index asc), ranked by counting over 64-bit keys in LDS.
constexpr int kMaxExpandW = 64;

__global__ __launch_bounds__(kBlock) void k_expand_tree(
    int32_t* __restrict__ cand_parent, int32_t* __restrict__ cand_token, float* __restrict__ cand_prob,
    float* __restrict__ cand_conf, int32_t* __restrict__ n_cand, const int32_t* expand_in,
    int32_t* expand_out, const int32_t* __restrict__ child_token,
    const float* __restrict__ child_prob, int M, int W, int C) {
    __shared__ int s_node[kMaxExpandW];        // the r-th expanded node, in slot order
    __shared__ int s_slot[kMaxExpandW];        // its slot
    __shared__ float s_pconf[kMaxExpandW];     // its confidence
    __shared__ unsigned long long keys[kMaxCand];
    __shared__ int s_n0, s_nexp;
    __shared__ int s_cnt[kWavesPerBlock];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t o = (int64_t)b * M;
    // 1. the nodes expanded by this call (expand_in is read before any write
    //    to expand_out, so the two may be one array)
    if (tid < kWave) {
        int n0 = n_cand[b];
        n0 = n0 < 0 ? 0 : (n0 > M ? M : n0);
        const bool root = n0 == 0;
        int id = -1;
        float pc = 0.f;
        if (tid < W) {
            if (root) {
                id = tid == 0 ? 0 : -1;
                pc = 1.0f;
            } else if (expand_in != nullptr) {
                id = expand_in[(int64_t)b * W + tid];
                if (id >= 0 && id < n0) {
                    pc = cand_conf[o + id];
                    if (!(pc >= 0.f)) id = -1;
                } else {
                    id = -1;
                }
            }
        }
        if (root && tid == 0) {                 // the tree starts at its root
            cand_parent[o] = -1;
            cand_token[o] = -1;
            cand_prob[o] = 1.0f;
            cand_conf[o] = 1.0f;
        }
        const unsigned long long m = __ballot(id >= 0);
        const int r = __popcll(m & ((1ull << tid) - 1ull));
        if (id >= 0) {
            s_node[r] = id;
            s_slot[r] = tid;
            s_pconf[r] = pc;
        }
        if (tid == 0) {
            s_n0 = root ? 1 : n0;
            s_nexp = __popcll(m);
        }
    }
    __syncthreads();
    const int n0 = s_n0;
    const int room = M - n0;
    const int nnew = min(s_nexp * C, room);
    // 2. the children of the expanded nodes, appended in slot order
    for (int j = tid; j < nnew; j += kBlock) {
        const int r = j / C, c = j - (j / C) * C;
        const int64_t src = ((int64_t)b * W + s_slot[r]) * C + c;
        const float q = child_prob[src];
        const float cf = (q >= 0.f && q <= 1.f) ? s_pconf[r] * q : -1.0f;
        const int i = n0 + j;
        cand_parent[o + i] = s_node[r];
        cand_token[o + i] = child_token[src];
        cand_prob[o + i] = q;
        cand_conf[o + i] = cf;
        // (confidence desc, index asc) as one key; +0 and -0 order alike; 0 = unusable
        const uint32_t cb = conf_bits(cf);
        keys[j] = cf >= 0.f ? (((unsigned long long)cb << 32) | (0xffffffffu - (uint32_t)i)) : 0ull;
    }
    __syncthreads();
    // 3. the W best new candidates: rank = number of larger keys (keys are distinct)
    int usable = 0;
    for (int j = tid; j < nnew; j += kBlock) {
        const unsigned long long k = keys[j];
        if (k == 0ull) continue;
        ++usable;
        int rank = 0;
        for (int i = 0; i < nnew; ++i) rank += keys[i] > k ? 1 : 0;
        if (rank < W) expand_out[(int64_t)b * W + rank] = n0 + j;
    }
    // the usable count over the block; the slots past it get -1
    int cnt = usable;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, kWave);
    if ((tid & (kWave - 1)) == 0) s_cnt[tid / kWave] = cnt;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) total += s_cnt[w];
    if (tid < W && tid >= total) expand_out[(int64_t)b * W + tid] = -1;
    if (tid == 0) n_cand[b] = n0 + nnew;
}

}  // namespace

hipError_t launch_expand_tree(int32_t* cand_parent, int32_t* cand_token, float* cand_prob,
                              float* cand_conf, int32_t* n_cand, const int32_t* expand_in,
                              int32_t* expand_out, const int32_t* child_token, const float* child_prob,
                              int B, int M, int W, int C, hipStream_t stream) {
    hipLaunchKernelGGL(k_expand_tree, dim3(B), dim3(kBlock), 0, stream, cand_parent, cand_token,
                       cand_prob, cand_conf, n_cand, expand_in, expand_out, child_token, child_prob, M,
                       W, C);
    return hipGetLastError();
}

hipError_t launch_rerank_tree(const int32_t* cand_parent, const int32_t* cand_token,
                              const float* cand_prob, const int32_t* n_cand, int B, int M, int N,
                              int32_t* tok, int32_t* par, int32_t* dep, float* score, uint64_t* anc,
                              int32_t* node_cand, int32_t* n_nodes, hipStream_t stream) {
    PassTimer::launch(k_rerank_tree, dim3(B), dim3(kBlock), stream, cand_parent, cand_token,
                      cand_prob, n_cand, M, N, tok, par, dep, score,
                      reinterpret_cast<unsigned long long*>(anc), node_cand, n_nodes);
    return hipGetLastError();
}

}  // namespace sd
